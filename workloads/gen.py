"""Seeded synthetic inputs for the Muon-style optimizer step.

This module is shared by the tests, the benchmark and the scripts that write
stored expected values.  It holds no arithmetic of the optimizer step itself:
only matrix-set shapes, hyperparameter tables and seeded random draws.

Gradient recipe (one matrix, shape r x c):
  * P (r x 8) and Q (c x 8) are the orthonormal factors of QR decompositions of
    iid N(0,1) draws; E is an iid N(0,1) r x c draw; draw order is P, Q, E.
  * G = 10 * P @ Q.T + 0.1 * E  -- a rank-8 component with singular values 10
    plus iid noise of standard deviation 0.1 (the small single-matrix case).
  * For the model-shaped matrix sets G is rescaled to an entry RMS of 1e-3
    (the "N(0, 1e-3)" gradient scale) and rounded to bfloat16.
Random streams: numpy ``default_rng([seed, step, matrix_index])`` for
gradients and ``default_rng([seed, 2**20, matrix_index])`` for initial
parameters, which are 0.02 * N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

PARAM_STREAM = 2 ** 20
RANK = 8


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.

    A storage conversion for inputs (data preparation), not part of the step.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def lowrank_noise(rows: int, cols: int, rng: np.random.Generator,
                  top: float = 10.0, noise: float = 0.1) -> np.ndarray:
    """Rank-8 (singular values ``top``) plus iid noise (std ``noise``), fp64."""
    k = min(RANK, rows, cols)
    p, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    q, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    e = rng.standard_normal((rows, cols))
    return top * (p @ q.T) + noise * e


def grad_matrix(rows: int, cols: int, seed: int, step: int, index: int,
                rms: float | None = None) -> np.ndarray:
    """One gradient matrix (fp64); rescaled to entry RMS ``rms`` if given."""
    g = lowrank_noise(rows, cols, np.random.default_rng([seed, step, index]))
    if rms is not None:
        g *= rms / np.sqrt(np.mean(g * g))
    return g


def param_matrix(rows: int, cols: int, seed: int, index: int,
                 std: float = 0.02) -> np.ndarray:
    """One initial parameter matrix (fp64), std * N(0, 1)."""
    rng = np.random.default_rng([seed, PARAM_STREAM, index])
    return std * rng.standard_normal((rows, cols))


def uniform_matrix(rows: int, cols: int, seed: int, step: int, index: int,
                   lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """iid uniform entries; used for edge-case tests (signs of W and S)."""
    rng = np.random.default_rng([seed, step, index, 7])
    return rng.uniform(lo, hi, size=(rows, cols))


# --------------------------------------------------------------------------
# Coefficient tables for the odd-polynomial iteration X <- aX + (bA + cA^2)X.
# cubic: p(x) = 1.5x - 0.5x^3 (Newton-Schulz for the polar factor).
# quintic: p(x) = (15x - 10x^3 + 3x^5) / 8, the next member of that family
# (p(1) = 1, p'(1) = p''(1) = 0).
CUBIC = (1.5, -0.5, 0.0)
QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


def coeff_table(kind: str, steps: int) -> np.ndarray:
    base = {"cubic": CUBIC, "quintic": QUINTIC}[kind]
    return np.array([base] * steps, dtype=np.float64).reshape(steps, 3)


# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MatrixSet:
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    dtype: str            # "bf16" or "f32" for params and grads
    steps: int            # Newton-Schulz iterations
    coeffs: str           # coefficient table kind
    lr: float = 0.02
    wd: float = 0.0
    beta: float = 0.95
    beta_slow: float = -1.0
    beta_ema: float = -1.0
    ema_start: int = 1
    cautious: bool = False
    grad_rms: float | None = 1e-3
    n_opt_steps: int = 1

    @property
    def numel(self) -> int:
        return sum(r * c for r, c in self.shapes)


def gpt124m_shapes() -> List[Tuple[int, int]]:
    d, f = 768, 3072
    out = []
    for _ in range(12):
        out += [(d, d)] * 4 + [(d, f), (f, d)]
    return out


def gpt2p7b_shapes() -> List[Tuple[int, int]]:
    d, f = 2560, 10240
    out = []
    for _ in range(32):
        out += [(d, d)] * 4 + [(d, f), (f, d)]
    return out


def moe_share_shapes() -> List[Tuple[int, int]]:
    out = []
    for _ in range(64):
        out += [(2048, 1408), (1408, 2048)]
    for _ in range(24):
        out += [(2048, 2048)] * 4
    return out


SETS = {
    # one fp32 256x512 gradient, one step
    "single_256x512": MatrixSet("single_256x512", ((256, 512),), "f32", 5,
                                "quintic", grad_rms=None),
    # 124M GPT-2 matrix set, plain Muon step
    "gpt124m": MatrixSet("gpt124m", tuple(gpt124m_shapes()), "bf16", 5,
                         "quintic"),
    # same set with fast/slow momentum, 6 map steps, cautious WD, EMA
    "gpt124m_anvil": MatrixSet("gpt124m_anvil", tuple(gpt124m_shapes()),
                               "bf16", 6, "quintic", wd=0.1, beta=0.9,
                               beta_slow=0.99, beta_ema=0.99, ema_start=1,
                               cautious=True, n_opt_steps=10),
    # 2.7B transformer matrix set, WD 1.6
    "gpt2p7b": MatrixSet("gpt2p7b", tuple(gpt2p7b_shapes()), "bf16", 5,
                         "quintic", wd=1.6),
    # MoE one-GPU share: 128 expert matrices + 96 attention matrices
    "moe_share": MatrixSet("moe_share", tuple(moe_share_shapes()), "bf16", 5,
                           "quintic"),
}


def ns_flops(shapes: Sequence[Tuple[int, int]], steps: int,
             cubic: bool = False) -> Tuple[float, float]:
    """(symmetric, dense-equivalent) flop counts of the iterations.

    Per iteration on effective shape m x n (m <= n): Gram m(m+1)n, square
    m^2(m+1) (absent for the cubic), apply 2m^2 n.  Dense: 4m^2 n + 2m^3.
    """
    sym = dense = 0.0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        sym += m * (m + 1) * n + 2.0 * m * m * n + (0 if cubic else m * m * (m + 1))
        dense += 4.0 * m * m * n + (0 if cubic else 2.0 * m ** 3)
    return sym * steps, dense * steps


def make_inputs(ms: MatrixSet, seed: int = 0, step: int = 0,
                indices: Sequence[int] | None = None):
    """Host inputs for a set: list of (grad, param) arrays in storage dtype.

    bf16 sets return uint16 bit patterns; f32 sets return float32 arrays.
    """
    idx = range(len(ms.shapes)) if indices is None else indices
    out = []
    for i in idx:
        r, c = ms.shapes[i]
        g = grad_matrix(r, c, seed, step, i, ms.grad_rms)
        w = param_matrix(r, c, seed, i)
        if ms.dtype == "bf16":
            out.append((bf16_bits_from_f32(g.astype(np.float32)),
                        bf16_bits_from_f32(w.astype(np.float32))))
        else:
            out.append((g.astype(np.float32), w.astype(np.float32)))
    return out


def torch_grad_matrix(rows: int, cols: int, seed: int, step: int, index: int, device,
                      rms: float | None = 1e-3, dtype=None):
    """Device-side variant of grad_matrix for large sets: the rank-8 factors
    come from numpy (same streams as grad_matrix), the iid noise from a torch
    generator seeded with (seed, step, index).  Returns a device tensor."""
    import torch
    rng = np.random.default_rng([seed, step, index])
    k = min(RANK, rows, cols)
    p, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    q, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    gtr = torch.Generator(device=device)
    gtr.manual_seed((seed * 1_000_003 + step) * 1_000_003 + index)
    e = torch.randn((rows, cols), generator=gtr, device=device, dtype=torch.float32)
    pt = torch.from_numpy((10.0 * p).astype(np.float32)).to(device)
    qt = torch.from_numpy(q.astype(np.float32)).to(device)
    g = torch.addmm(e.mul_(0.1), pt, qt.T)
    if rms is not None:
        g.mul_(rms / g.square().mean().sqrt())
    return g if dtype is None else g.to(dtype)


def torch_param_matrix(rows: int, cols: int, seed: int, index: int, device, std: float = 0.02,
                       dtype=None):
    import torch
    gtr = torch.Generator(device=device)
    gtr.manual_seed((seed * 1_000_003 + PARAM_STREAM) * 1_000_003 + index)
    w = torch.randn((rows, cols), generator=gtr, device=device, dtype=torch.float32).mul_(std)
    return w if dtype is None else w.to(dtype)


# ---------------------------------------------------------------------------
# AdamW inputs: the parameters that are not weight matrices of the blocks.
ADAMW_STREAM = 2 ** 21


def gpt124m_adamw_sizes() -> List[int]:
    """Element counts of the 124M GPT-2 parameters left to AdamW: token and
    position embeddings, then per layer LayerNorm 1 gain and bias, Q, K, V and
    output-projection biases, LayerNorm 2 gain and bias, MLP up and down
    biases; then the final LayerNorm gain and bias."""
    vocab, ctx, c, layers = 50257, 1024, 768, 12
    sizes = [vocab * c, ctx * c]
    for _ in range(layers):
        sizes += [c, c, c, c, c, c, c, c, 4 * c, c]
    return sizes + [c, c]


def flat_param(n: int, seed: int, index: int, std: float = 0.02) -> np.ndarray:
    """fp32 draw of std * N(0,1) from default_rng([seed, 2**21, index])."""
    rng = np.random.default_rng([seed, ADAMW_STREAM, index])
    return (std * rng.standard_normal(n)).astype(np.float32)


def flat_grad(n: int, seed: int, step: int, index: int, rms: float = 1e-3) -> np.ndarray:
    """fp32 gradient draw rms * N(0,1) from default_rng([seed, 2**21 + 1 + step, index])."""
    rng = np.random.default_rng([seed, ADAMW_STREAM + 1 + step, index])
    return (rms * rng.standard_normal(n)).astype(np.float32)


def flat_moments(n: int, seed: int, index: int, rms: float = 1e-3):
    """A non-trivial AdamW state: m ~ rms*N(0,1), v = (rms*N(0,1))^2, both fp32."""
    rng = np.random.default_rng([seed, ADAMW_STREAM - 1, index])
    m = (rms * rng.standard_normal(n)).astype(np.float32)
    v = np.square(rms * rng.standard_normal(n)).astype(np.float32)
    return m, v


def torch_flat(x: np.ndarray, device, dtype):
    """fp32 host array -> device tensor of `dtype` (bf16 rounded to nearest even)."""
    import torch
    if dtype == torch.bfloat16:
        bits = bf16_bits_from_f32(x).view(np.int16)
        return torch.from_numpy(bits.copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
