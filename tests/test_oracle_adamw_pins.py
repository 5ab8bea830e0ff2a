"""Pins for the AdamW oracle: checks against the method's closed forms, a
hand-worked step, an independent scalar fp32 emulation and a library
implementation of the same textbook method -- none of them reuse the oracle's
code path.  Each is chosen so that a plausible slip (a dropped bias
correction, eps inside the square root, a wrong decay sign or factor, a fused
or reordered fp32 operation) fails at least one test."""
import os
import struct

import numpy as np
import pytest

from oracle import adamw_oracle as ada

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _run(p0, grads, lr, b1, b2, eps, wd):
    st = ada.AdamWState([p0.size])
    p = p0.astype(np.float64)
    for g in grads:
        p = ada.adamw_step([p], [g], st, lr, b1, b2, eps, wd, param_dtype="f64")[0]
    return p, st


def test_hand_worked_steps():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "adamw_hand.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        p0, g, lr, wd, b1, b2, eps, p1 = map(float, r)
        p, _ = _run(np.array([p0]), [np.array([g], dtype=np.float32)], lr, b1, b2, eps, wd)
        assert abs(p[0] - p1) <= 1e-15 * max(1.0, abs(p1)), (r, p[0])


def test_constant_gradient_closed_form():
    """m0 = v0 = 0 and a constant gradient: mhat = g and vhat = g^2 at every
    step (up to the fp32 rounding of the stored moments), so
    p_t = (1 - lr*wd) p_{t-1} - lr * g / (|g| + eps)."""
    rng = np.random.default_rng(3)
    n, lr, b1, b2, eps, wd = 257, 1e-2, 0.9, 0.999, 1e-8, 0.1
    p0 = rng.normal(0, 1, n)
    g = (rng.uniform(1e-3, 1e-1, n) * rng.choice([-1, 1], n)).astype(np.float32)
    p, _ = _run(p0, [g] * 6, lr, b1, b2, eps, wd)
    ref = p0.copy()
    gd = g.astype(np.float64)
    for _ in range(6):
        ref = (1 - lr * wd) * ref - lr * gd / (np.abs(gd) + eps)
    np.testing.assert_allclose(p, ref, rtol=0, atol=6 * lr * 1e-6)


def test_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(4)
    p0 = rng.normal(0, 1, 100)
    lr, wd = 0.03, 0.2
    p, st = _run(p0, [np.zeros(100, np.float32)] * 5, lr, 0.9, 0.99, 1e-8, wd)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) ** 5, rtol=1e-14, atol=0)
    assert not st.m[0].any() and not st.v[0].any()


def test_matches_library_adamw_in_float64():
    """torch.optim.AdamW implements the same textbook update; run it in
    float64 on the CPU.  The oracle keeps fp32 moments, so the two differ by
    the moments' fp32 rounding only."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    n, lr, b1, b2, eps, wd = 300, 3e-3, 0.9, 0.95, 1e-8, 0.05
    p0 = rng.normal(0, 1, n)
    grads = [rng.normal(0, 1e-2, n).astype(np.float32) for _ in range(5)]
    p, _ = _run(p0, grads, lr, b1, b2, eps, wd)
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    # the fp32 betas, as the oracle and the device use them
    opt = torch.optim.AdamW([tp], lr=lr, betas=(float(np.float32(b1)), float(np.float32(b2))),
                            eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        tp.grad = torch.tensor(g.astype(np.float64))
        opt.step()
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=0, atol=5 * lr * 1e-5)


def test_moments_follow_the_fp32_operation_order():
    """Independent scalar emulation: each product and sum rounded to fp32
    through struct packing (products of two fp32 values are exact in double).
    A single-rounding (fused) variant must differ somewhere, which shows that
    this pin sees the operation order."""
    rng = np.random.default_rng(6)
    n = 400
    m = rng.normal(0, 1e-2, n).astype(np.float32)
    v = rng.uniform(0, 1e-4, n).astype(np.float32)
    g = rng.normal(0, 1e-2, n).astype(np.float32)
    b1, b2 = 0.9, 0.999
    mo, vo = ada.adamw_moments_f32(m, v, g, b1, b2)
    f1, f2 = _f32(b1), _f32(b2)
    o1, o2 = _f32(1.0 - f1), _f32(1.0 - f2)
    fused_differs = 0
    for i in range(n):
        mi = _f32(_f32(f1 * float(m[i])) + _f32(o1 * float(g[i])))
        gg = _f32(float(g[i]) * float(g[i]))
        vi = _f32(_f32(f2 * float(v[i])) + _f32(o2 * gg))
        assert mo[i] == np.float32(mi), i
        assert vo[i] == np.float32(vi), i
        fused = _f32(f2 * float(v[i]) + o2 * float(g[i]) * float(g[i]))
        fused_differs += fused != vi
    assert fused_differs > 0


def test_bias_correction_is_applied():
    """First step: mhat = g exactly, so a unit gradient with eps = 0 moves
    every parameter by exactly lr (a missing 1/(1 - beta1) would move it by
    lr*(1 - beta1)/sqrt(1 - beta2))."""
    p, _ = _run(np.zeros(4), [np.ones(4, np.float32)], 0.25, 0.9, 0.999, 0.0, 0.0)
    np.testing.assert_allclose(p, -0.25 * np.ones(4), rtol=0, atol=1e-15)
