"""Plain, slow CPU oracle for the Muon-style optimizer step (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product (the HIP library and its Python binding) never does,
and this module imports nothing from the product.

What it computes, with the passages it follows:
  * Momentum: a moving average of the gradient is kept per weight matrix
    (page "きみはNanoGPT speedrunを知っているか？", prednext.com, section
    "Muonとは"; the neo-ai.one article on the Muon author, section
    "Muonが登場", calls it SGD-momentum).
  * Approximate orthogonalisation of that momentum by Newton-Schulz iteration,
    pushing its singular values towards one (same two sections).  The
    iteration used is the odd polynomial X <- aX + (bA + cA^2)X with A = XX^T,
    after Frobenius normalisation, on the wide orientation of the matrix
    (tall matrices are transposed so that A is the small Gram matrix).
  * Parameter update with the orthogonalised matrix (section "Muonとは"), with
    decoupled weight decay, optionally masked element-wise by sign agreement
    with a slow momentum (page "Training NanoGPT in 39.9 Seconds",
    seosoyoung.eiaserinnys.me digest, section "ANVIL II와 가중치 평균",
    first paragraph: fast and slow momentum, six polynomial-map steps,
    cautious weight decay chosen by agreement with the slow momentum).
  * EMA weight average theta_bar_t = beta*theta_bar_{t-1} + (1-beta)*theta_t
    (same section, its displayed equation) and the final readout blend of
    35 % final weights and 65 % average (same section, paragraph after it).
  * Weighted running mean of the weights as an alternative average: stochastic
    weight averaging (equal weights) and weighted checkpoint averaging, both
    named in the results table of the Slowrun page without a formula; read as
    E_n = sum_k w_k W_k / sum_k w_k, kept as E <- (S/(S+w)) E + (w/(S+w)) W.

Precision: the orthogonalisation and the parameter update are computed in
float64.  The stored optimizer state (momentum, slow momentum, EMA) is fp32
and must match the GPU bit for bit, so those recurrences are also provided in
an explicit fp32 operation order: every product and every sum rounded to fp32,
no fused multiply-add: m = fl(fl(beta*m) + fl((1-beta)*g)), where (1-beta)
itself is computed in fp32.

Readings where the pages are silent (each is listed in the design notes):
  * coefficients (a, b, c) per iteration are inputs;
  * eps = 1e-7 is added to the Frobenius norm;
  * momentum is the EMA form M <- beta*M + (1-beta)*G with M_0 = 0;
    Nesterov (off by default) uses U = beta*M_t + (1-beta)*G;
  * weight decay is decoupled and lr-scaled, W <- W - lr*wd*mask*W - lr*O,
    on W_{t-1}; the mask is [W_{t-1} * S_t > 0] (zero in either: no decay);
  * the fast momentum is the one orthogonalised; the slow one is only used
    for the mask;
  * the EMA is set to W_t at its first averaged step;
  * fp32 -> bf16 conversion is round-to-nearest-even.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

F32 = np.float32


# ----------------------------------------------------------------------------
# bfloat16 rounding, written from the format's definition: 8 significant bits
# (1 implicit + 7 stored), the same exponent range as fp32, ties to even.
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (returned as float64).

    Direct rounding from the float64 value (no intermediate fp32 step).
    NaN stays NaN; values beyond the largest finite bfloat16 (with ties going
    to infinity as in round-to-nearest-even) become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                    # xf = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)                # below 2**-126 the spacing is fixed
    scale = np.ldexp(1.0, 8 - e)           # 8 significant bits
    q = np.rint(xf * scale) / scale        # np.rint rounds half to even
    big = np.abs(q) > 3.3895313892515355e38   # largest finite bf16
    q[big] = np.sign(q[big]) * np.inf
    out[fin] = q
    return out


def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (returned as float32), ties to even.

    Same result as round_to_bf16 for float32 inputs (checked by the pins);
    works on the bit pattern: keep the top 16 bits, adding half of the
    dropped part rounded to even.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)).view(F32)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = np.nan
    return r


# ----------------------------------------------------------------------------
# Newton-Schulz style orthogonalisation (float64)
def ns_poly_scalar(x: float, coeffs: np.ndarray) -> float:
    """The scalar map x -> p_K(...p_1(x)) with p_j(x) = a_j x + b_j x^3 + c_j x^5."""
    for a, b, c in np.asarray(coeffs, dtype=np.float64).reshape(-1, 3):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def orthogonalize(U: np.ndarray, coeffs: np.ndarray, eps: float = 1e-7) -> np.ndarray:
    """Approximately orthogonalise one matrix (float64 throughout).

    Steps: take the wide orientation (transpose when rows > cols), divide by
    (Frobenius norm + eps), run one iteration X <- aX + (bA + cA^2)X with
    A = X X^T for each coefficient row (a, b, c), transpose back.
    """
    X = np.array(U, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.copy()
    X = X / (np.sqrt(np.sum(X * X)) + eps)
    for a, b, c in np.asarray(coeffs, dtype=np.float64).reshape(-1, 3):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T.copy() if tall else X


# ----------------------------------------------------------------------------
# fp32 recurrences in the fixed operation order (bit-exact state)
def ema_f32(prev: np.ndarray, new: np.ndarray, beta: float) -> np.ndarray:
    """fl(fl(beta*prev) + fl((1-beta)*new)), all in fp32, no fused ops."""
    b = F32(beta)
    ob = F32(1.0) - b
    p = np.asarray(prev, dtype=F32)
    n = np.asarray(new, dtype=F32)
    return (b * p).astype(F32) + (ob * n).astype(F32)


def running_mean_coeffs(weight_sum: float, w: float):
    """Weighted running mean E <- b*E + ob*W with b = S/(S+w), ob = w/(S+w),
    computed in double and rounded to fp32 (S: weights averaged so far).
    Equal weights give the running arithmetic mean (stochastic weight
    averaging); the Slowrun page's results table names both it and weighted
    checkpoint averaging without giving a formula."""
    tot = float(weight_sum) + float(w)
    return F32(float(weight_sum) / tot), F32(float(w) / tot)


def average_f32(prev: np.ndarray, new: np.ndarray, b, ob) -> np.ndarray:
    """fl(fl(b*prev) + fl(ob*new)) in fp32 with given fp32 coefficients."""
    p = np.asarray(prev, dtype=F32)
    n = np.asarray(new, dtype=F32)
    return ((F32(b) * p).astype(F32) + (F32(ob) * n).astype(F32)).astype(F32)


def momentum_f32(M: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """Momentum as a moving average of the gradient, fp32 operation order."""
    return ema_f32(M, G, beta)


def nesterov_f32(M_new: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    return ema_f32(M_new, G, beta)


def cautious_mask(W: np.ndarray, S: np.ndarray) -> np.ndarray:
    """1 where W and S are both strictly positive or both strictly negative."""
    W = np.asarray(W)
    S = np.asarray(S)
    return ((W > 0) & (S > 0)) | ((W < 0) & (S < 0))


def update_f64(W: np.ndarray, O: np.ndarray, lr: float, wd: float,
               mask: Optional[np.ndarray] = None) -> np.ndarray:
    """W - lr*wd*mask*W - lr*O in float64 (mask None means decay everywhere)."""
    W = np.asarray(W, dtype=np.float64)
    m = 1.0 if mask is None else np.asarray(mask, dtype=np.float64)
    return W - lr * wd * m * W - lr * np.asarray(O, dtype=np.float64)


def update_f32(W: np.ndarray, O: np.ndarray, lr: float, wd: float,
               mask: Optional[np.ndarray] = None) -> np.ndarray:
    """The same update in the fp32 operation order fl(fl(w - fl(d*w)) - fl(lr*o)),
    d = fl(lr*wd) where the mask is set and 0 elsewhere.  Used to check the
    arithmetic of the update on identical inputs."""
    w = np.asarray(W, dtype=F32)
    o = np.asarray(O, dtype=F32)
    lrwd = F32(lr) * F32(wd)
    d = np.full(w.shape, lrwd, dtype=F32) if mask is None else \
        np.where(np.asarray(mask, dtype=bool), lrwd, F32(0.0)).astype(F32)
    t = (w - (d * w).astype(F32)).astype(F32)
    return (t - (F32(lr) * o).astype(F32)).astype(F32)


def blend_f32(W: np.ndarray, E: np.ndarray, w_final: float) -> np.ndarray:
    """Readout blend w_final*W + (1-w_final)*E in the fp32 operation order."""
    wf = F32(w_final)
    owf = F32(1.0) - wf
    return ((wf * np.asarray(W, F32)).astype(F32) +
            (owf * np.asarray(E, F32)).astype(F32)).astype(F32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a result to the storage type ("bf16", "f32" or "f64")."""
    if dtype == "bf16":
        if np.asarray(x).dtype == F32:
            return round_f32_to_bf16(x).astype(np.float64)
        return round_to_bf16(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    return np.asarray(x, dtype=np.float64).astype(F32).astype(np.float64)


# ----------------------------------------------------------------------------
class OracleState:
    """Optimizer state: fp32 buffers per matrix plus integer counters."""

    def __init__(self, shapes: Sequence, beta_slow: float = -1.0,
                 beta_ema: float = -1.0, ema_start: int = 1, avg_mode: str = "ema"):
        self.mom = [np.zeros(s, dtype=F32) for s in shapes]
        self.slow = [np.zeros(s, dtype=F32) for s in shapes] if beta_slow >= 0 else None
        self.ema = [np.zeros(s, dtype=F32) for s in shapes] if beta_ema >= 0 else None
        self.beta_slow = beta_slow
        self.beta_ema = beta_ema
        self.ema_start = ema_start
        self.step = 0
        self.ema_count = 0
        self.avg_mode = avg_mode      # "ema" or "weighted"
        self.avg_sum = 0.0            # weights averaged so far ("weighted")


def muon_step(params: List[np.ndarray], grads: List[np.ndarray], st: OracleState,
              coeffs: np.ndarray, lr: float, wd: float, beta: float,
              param_dtype: str = "bf16", eps: float = 1e-7, nesterov: bool = False,
              cautious: bool = False, keep: bool = True,
              avg_weight: float = 1.0) -> Dict[str, list]:
    """One optimizer step over a list of matrices.

    params: stored parameter values (float64 arrays holding bf16/fp32 values);
    grads: gradient values (exact fp32 values of the stored gradients).
    Returns the new parameters (rounded to param_dtype) and, when keep is set,
    the orthogonalised updates and masks.  The state is updated in place.
    """
    st.step += 1
    ema_on = st.ema is not None and st.step >= st.ema_start
    first_ema = ema_on and st.ema_count == 0
    weighted = ema_on and st.avg_mode == "weighted"
    if weighted:
        s0 = 0.0 if first_ema else st.avg_sum
        avg_b, avg_ob = running_mean_coeffs(s0, avg_weight)
    new_params, outs, masks = [], [], []
    for i, (W, G) in enumerate(zip(params, grads)):
        G32 = np.asarray(G, dtype=F32)
        st.mom[i] = momentum_f32(st.mom[i], G32, beta)
        if st.slow is not None:
            st.slow[i] = momentum_f32(st.slow[i], G32, st.beta_slow)
        U = nesterov_f32(st.mom[i], G32, beta) if nesterov else st.mom[i]
        O = orthogonalize(U.astype(np.float64), coeffs, eps)
        mask = cautious_mask(W, st.slow[i]) if cautious else None
        Wn = store(update_f64(W, O, lr, wd, mask), param_dtype)
        if ema_on:
            if first_ema:
                st.ema[i] = Wn.astype(F32)
            elif weighted:
                st.ema[i] = average_f32(st.ema[i], Wn, avg_b, avg_ob)
            else:
                st.ema[i] = ema_f32(st.ema[i], Wn, st.beta_ema)
        new_params.append(Wn)
        if keep:
            outs.append(O)
            masks.append(mask)
    if ema_on:
        st.ema_count += 1
    if weighted:
        st.avg_sum = s0 + avg_weight
    return {"params": new_params, "O": outs, "mask": masks}


def ns_flops_dense(m: int, n: int, steps: int, quintic: bool = True) -> float:
    """Flops of the plain (non-symmetric) float64 iteration on an m x n matrix."""
    m, n = min(m, n), max(m, n)
    return steps * (4.0 * m * m * n + (2.0 * m ** 3 if quintic else 0.0))


def singular_values(X: np.ndarray) -> np.ndarray:
    return np.linalg.svd(np.asarray(X, dtype=np.float64), compute_uv=False)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = math.sqrt(float(np.sum(b * b)))
    return math.sqrt(float(np.sum((a - b) ** 2))) / (den if den > 0 else 1.0)
