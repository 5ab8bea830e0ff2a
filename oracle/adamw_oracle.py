"""Plain, slow CPU oracle for the AdamW step of the parameters that are not
weight matrices (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product (the HIP library and its Python binding) never does,
and this module imports nothing from the product.

What it computes: the pages recommend AdamW for every parameter that is not a
matrix, since orthogonalisation only applies to matrix-shaped layers (page
"きみはNanoGPT speedrunを知っているか？", prednext.com, section "Muonとは").
They give no formula or hyperparameters, so this is the textbook method:
Adam's moving averages of the gradient and of its square, each divided by its
bias (1 - beta^t), with weight decay decoupled from the gradient.

Readings where the pages are silent (each is listed in the design notes):
  * m_0 = v_0 = 0; t counts the steps of this parameter set from 1;
  * decay is decoupled and lr-scaled and acts on p_{t-1}:
        p_t = p_{t-1} - lr*wd*p_{t-1} - lr * mhat / (sqrt(vhat) + eps),
        mhat = m_t / (1 - beta1^t),  vhat = v_t / (1 - beta2^t);
    eps is added after the square root;
  * the stored moments are fp32 and follow a fixed fp32 operation order with
    every product and sum rounded on its own (no fused multiply-add):
        m = fl(fl(b1*m) + fl(ob1*g)),  v = fl(fl(b2*v) + fl(ob2*fl(g*g))),
    with b = fp32(beta) and ob = fl(1 - b) computed in fp32;
  * bf16 parameters are stored round-to-nearest-even.

Precision: the moments in the fp32 order above (so that a device
implementation can match them bit for bit); the parameter update in float64
from those fp32 moments.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from oracle.muon_oracle import store

F32 = np.float32


def adamw_moments_f32(m: np.ndarray, v: np.ndarray, g: np.ndarray, beta1: float,
                      beta2: float) -> Tuple[np.ndarray, np.ndarray]:
    """First and second moment averages in the fixed fp32 operation order."""
    b1, b2 = F32(beta1), F32(beta2)
    ob1, ob2 = F32(1.0) - b1, F32(1.0) - b2
    g = np.asarray(g, dtype=F32)
    m = np.asarray(m, dtype=F32)
    v = np.asarray(v, dtype=F32)
    m_new = ((b1 * m).astype(F32) + (ob1 * g).astype(F32)).astype(F32)
    gg = (g * g).astype(F32)
    v_new = ((b2 * v).astype(F32) + (ob2 * gg).astype(F32)).astype(F32)
    return m_new, v_new


def adamw_update_f64(p: np.ndarray, m: np.ndarray, v: np.ndarray, t: int, lr: float,
                     beta1: float, beta2: float, eps: float, wd: float) -> np.ndarray:
    """p - lr*wd*p - lr * mhat / (sqrt(vhat) + eps) in float64, where the
    moments are the stored fp32 values and the bias terms use the fp32 betas."""
    b1 = float(F32(beta1))
    b2 = float(F32(beta2))
    c1 = 1.0 - b1 ** t
    c2 = 1.0 - b2 ** t
    p = np.asarray(p, dtype=np.float64)
    mhat = np.asarray(m, dtype=np.float64) / c1
    vhat = np.asarray(v, dtype=np.float64) / c2
    return p - lr * wd * p - lr * mhat / (np.sqrt(vhat) + eps)


class AdamWState:
    """fp32 moments per tensor plus the step counter."""

    def __init__(self, sizes: Sequence[int]):
        self.m = [np.zeros(int(n), dtype=F32) for n in sizes]
        self.v = [np.zeros(int(n), dtype=F32) for n in sizes]
        self.step = 0


def adamw_step(params: List[np.ndarray], grads: List[np.ndarray], st: AdamWState, lr: float,
               beta1: float, beta2: float, eps: float, wd: float,
               param_dtype: str = "bf16") -> List[np.ndarray]:
    """One step over a list of flat tensors; returns the new parameters rounded
    to param_dtype ("bf16" or "f32"); the moments are updated in place."""
    st.step += 1
    out = []
    for i, (p, g) in enumerate(zip(params, grads)):
        st.m[i], st.v[i] = adamw_moments_f32(st.m[i], st.v[i], g, beta1, beta2)
        pn = adamw_update_f64(p, st.m[i], st.v[i], st.step, lr, beta1, beta2, eps, wd)
        out.append(store(pn, param_dtype))
    return out


def adamw_update_bound(p: np.ndarray, m: np.ndarray, v: np.ndarray, t: int, lr: float,
                       beta1: float, beta2: float, eps: float, wd: float) -> np.ndarray:
    """Scale of the terms of the update, for fp32 tolerances:
    |p| + lr*wd*|p| + lr*|mhat|/(sqrt(vhat) + eps)."""
    b1 = float(F32(beta1))
    b2 = float(F32(beta2))
    p = np.abs(np.asarray(p, dtype=np.float64))
    mhat = np.abs(np.asarray(m, dtype=np.float64)) / (1.0 - b1 ** t)
    vhat = np.asarray(v, dtype=np.float64) / (1.0 - b2 ** t)
    return p + lr * abs(wd) * p + lr * mhat / (np.sqrt(vhat) + eps)


def adamw_bytes_per_element(param_bytes: int, grad_bytes: int) -> int:
    """Algorithmic HBM bytes per element: p read+write, g read, m and v fp32
    read+write."""
    return 2 * param_bytes + grad_bytes + 16


def bias_terms(t: int, beta1: float, beta2: float) -> Tuple[float, float]:
    """(1 - beta1^t, 1 - beta2^t) with the fp32 betas, in float64."""
    return 1.0 - float(F32(beta1)) ** t, 1.0 - float(F32(beta2)) ** t


__all__ = ["adamw_moments_f32", "adamw_update_f64", "AdamWState", "adamw_step",
           "adamw_update_bound", "adamw_bytes_per_element", "bias_terms"]
