"""The plain update inside the last APPLY launch (bf16 parameters, 256-wide
tiles): W must be bit for bit what the separate finish kernel writes (a twin
optimizer with diagnostic outputs takes that path) and equal to the oracle's
fp32 update of the same O; calls that do not qualify keep the finish kernel."""
import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import muon_oracle as orc
from tests.gpu_helpers import announce, dev_bf16, host
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()
    monkeypatch.setenv("MUON_TILE", "256")


# square, wide, tall; 1408 ends inside a tile, 200 and 72 are below one tile
SHAPES = [(768, 768), (512, 1280), (1280, 512), (1408, 2048), (200, 72), (72, 200)]


def _inputs(shapes, seed):
    ws = [gen.bf16_bits_from_f32(gen.param_matrix(r, c, seed, i).astype(np.float32))
          for i, (r, c) in enumerate(shapes)]

    def grads(t):
        return [dev_bf16(gen.bf16_bits_from_f32(
                    gen.grad_matrix(r, c, seed, t, i, 1e-3).astype(np.float32)))
                for i, (r, c) in enumerate(shapes)]
    return ws, grads


def _step_count(opt, grads, phase="finish"):
    """Take one step; return how many launches of `phase` it made."""
    mo.probe_arm(phase, 16)
    opt.step(grads)
    torch.cuda.synchronize()
    n = len(mo.probe_read(16))
    mo.probe_disarm()
    return n


_step_count_finish = _step_count


@pytest.mark.parametrize("coeffs,steps,wd", [("quintic", 5, 0.1), ("cubic", 5, 0.0),
                                             ("quintic", 1, 1.6)])
def test_fused_update_equals_finish_kernel(coeffs, steps, wd):
    announce(f"fused update vs finish kernel: {coeffs} K={steps} wd={wd}")
    ws, grads = _inputs(SHAPES, 7)
    pa = [dev_bf16(w) for w in ws]
    pb = [dev_bf16(w) for w in ws]
    kw = dict(lr=0.02, wd=wd, beta=0.95, steps=steps, coeffs=coeffs)
    a = mo.Muon(pa, diagnostics=True, **kw)   # separate finish kernel
    b = mo.Muon(pb, **kw)                      # update in the last APPLY launch
    for t in range(3):
        g = grads(t)
        w_prev = [host(p).astype(np.float64) for p in pa]
        assert _step_count_finish(a, g) == 1
        assert _step_count_finish(b, g) == 0
        for i, shape in enumerate(SHAPES):
            np.testing.assert_array_equal(host(pb[i]), host(pa[i]),
                                          err_msg=f"step {t} W[{i}] {shape}")
            np.testing.assert_array_equal(host(b.mom[i]), host(a.mom[i]))
            want = orc.store(orc.update_f32(w_prev[i], host(a.update[i]), 0.02, wd), "bf16")
            np.testing.assert_array_equal(host(pb[i]).astype(np.float64), want,
                                          err_msg=f"step {t} W[{i}] {shape} vs oracle update")


def test_strided_parameter_views():
    """Parameters that are column slices of wider buffers (row pitch a multiple
    of 8, 16-byte aligned base): the fused path writes inside the slices only."""
    announce("fused update on strided views")
    shapes = [(768, 1024), (1024, 768)]
    ws, grads = _inputs(shapes, 8)
    bufs, views, twins = [], [], []
    for (r, c), w in zip(shapes, ws):
        big = torch.full((r, c + 24), 3.0, dtype=torch.bfloat16, device="cuda")
        v = big[:, 8:8 + c]
        v.copy_(dev_bf16(w))
        bufs.append(big)
        views.append(v)
        twins.append(dev_bf16(w))
    before = [host(b).copy() for b in bufs]
    a = mo.Muon(twins, lr=0.02, wd=0.1, diagnostics=True)
    b = mo.Muon(views, lr=0.02, wd=0.1)
    g = grads(0)
    assert _step_count_finish(a, g) == 1
    assert _step_count_finish(b, g) == 0
    for i in range(len(shapes)):
        np.testing.assert_array_equal(host(views[i]), host(twins[i]))
        after = host(bufs[i])
        c = shapes[i][1]
        np.testing.assert_array_equal(after[:, :8], before[i][:, :8])
        np.testing.assert_array_equal(after[:, 8 + c:], before[i][:, 8 + c:])


def test_calls_that_do_not_qualify_keep_the_finish_kernel():
    announce("fused update: fallbacks")
    # a column count that is not a multiple of 8
    ws, grads = _inputs([(768, 768), (200, 333)], 9)
    opt = mo.Muon([dev_bf16(w) for w in ws], lr=0.02)
    assert _step_count_finish(opt, grads(0)) == 1
    # cautious decay and the weight average
    ws, grads = _inputs([(768, 768)], 10)
    opt = mo.Muon([dev_bf16(w) for w in ws], lr=0.02, wd=0.1, beta_slow=0.99, cautious=True)
    assert _step_count_finish(opt, grads(0)) == 1
    opt = mo.Muon([dev_bf16(w) for w in ws], lr=0.02, beta_ema=0.99, ema_start=1)
    assert _step_count_finish(opt, grads(0)) == 1
    # fp32 parameters
    opt = mo.Muon([torch.zeros((768, 768), device="cuda")], lr=0.02)
    assert _step_count_finish(opt, [torch.ones((768, 768), device="cuda")]) == 1


def test_graph_replays_of_a_fused_step():
    announce("fused update: graph replays")
    ws, grads = _inputs(SHAPES[:4], 11)
    pa = [dev_bf16(w) for w in ws]
    pb = [dev_bf16(w) for w in ws]
    a = mo.Muon(pa, lr=0.02, wd=0.1, diagnostics=True)
    b = mo.Muon(pb, lr=0.02, wd=0.1)
    static = [torch.empty_like(x) for x in grads(0)]
    for s, x in zip(static, grads(0)):
        s.copy_(x)
    gr = b.graph(static)
    for t in range(3):
        g = grads(t)
        for s, x in zip(static, g):
            s.copy_(x)
        gr.replay()
        a.step(g)
        torch.cuda.synchronize()
        for i in range(len(pa)):
            np.testing.assert_array_equal(host(pb[i]), host(pa[i]), err_msg=f"replay {t} W[{i}]")


def test_launch_phases_of_a_fused_step():
    """Five iterations: a fused step has four plain APPLY launches and one that
    carries the update; an unfused step has five and a finish launch."""
    announce("fused update: launch phases")
    ws, grads = _inputs(SHAPES[:2], 12)
    a = mo.Muon([dev_bf16(w) for w in ws], lr=0.02, diagnostics=True)
    b = mo.Muon([dev_bf16(w) for w in ws], lr=0.02)
    g = grads(0)
    assert (_step_count(a, g, "apply"), _step_count(a, g, "apply_update")) == (5, 0)
    assert (_step_count(b, g, "apply"), _step_count(b, g, "apply_update")) == (4, 1)


def test_nan_gradient_stays_in_its_matrix():
    """A NaN in one gradient reaches only that matrix's parameters, as with the
    finish kernel (NaN compares equal to NaN here)."""
    announce("fused update: NaN confinement")
    ws, grads = _inputs(SHAPES[:4], 13)
    pa = [dev_bf16(w) for w in ws]
    pb = [dev_bf16(w) for w in ws]
    a = mo.Muon(pa, lr=0.02, wd=0.1, diagnostics=True)
    b = mo.Muon(pb, lr=0.02, wd=0.1)
    g = grads(0)
    g[2][5, 7] = float("nan")
    assert _step_count(a, g) == 1
    assert _step_count(b, g) == 0
    for i in range(len(pa)):
        wa, wb = host(pa[i]), host(pb[i])
        np.testing.assert_array_equal(wb, wa)
        if i == 2:
            assert np.isnan(wb).all()
        else:
            assert np.isfinite(wb).all()
