"""GPU parity: the HIP path against the fp64 CPU oracle, through the C ABI."""
import os

import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import muon_oracle as orc
from tests.gpu_helpers import (TOL_BF16, TOL_F32, TOL_SIGMA, announce, dev_bf16, dev_f32, host,
                               sigma_dev)
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


@pytest.fixture
def tile(request):
    """Force a Newton-Schulz tile edge for the duration of a test."""
    old = os.environ.get("MUON_TILE")
    val = getattr(request, "param", None)
    if val:
        os.environ["MUON_TILE"] = str(val)
    yield val
    if old is None:
        os.environ.pop("MUON_TILE", None)
    else:
        os.environ["MUON_TILE"] = old


def _table(kind, k):
    return gen.coeff_table(kind, k)


def _ortho(us, kind, k, ns, out_dtype=torch.float32, eps=1e-7):
    ins = [dev_f32(u) if u.dtype == np.float32 else dev_bf16(u) for u in us]
    outs = [torch.empty(t.shape, dtype=out_dtype, device="cuda") for t in ins]
    mo.orthogonalize(ins, outs, coeffs=_table(kind, k), steps=k, ns_dtype=ns, eps=eps)
    torch.cuda.synchronize()
    return [host(o) for o in outs]


# ------------------------------------------------------------ orthogonalize
@pytest.mark.parametrize("kind", ["cubic", "quintic"])
@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_single_matrix_256x512(kind, ns, tol):
    announce(f"orthogonalize 256x512 {kind} {ns}")
    G = gen.grad_matrix(256, 512, 0, 0, 0).astype(np.float32)
    (O,) = _ortho([G], kind, 5, ns)
    ref = orc.orthogonalize(G.astype(np.float64), _table(kind, 5))
    assert orc.rel_fro(O, ref) <= tol
    assert sigma_dev(O, ref) <= TOL_SIGMA


# ten effective shapes: more than one grouped launch set per phase (at most
# eight groups per launch)
RAGGED = [(200, 333), (333, 200), (7, 11), (11, 7), (1, 5), (5, 1), (300, 300), (64, 1000),
          (1000, 70), (200, 333), (129, 65), (40, 90), (91, 41), (17, 257)]


@pytest.mark.parametrize("tile", [64, 128, 256], indirect=True)
@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_ragged_mixed_shapes(tile, ns, tol):
    announce(f"orthogonalize ragged tile={tile} {ns}")
    us = [gen.grad_matrix(r, c, 1, 0, i).astype(np.float32) for i, (r, c) in enumerate(RAGGED)]
    outs = _ortho(us, "quintic", 5, ns)
    for u, o in zip(us, outs):
        ref = orc.orthogonalize(u.astype(np.float64), _table("quintic", 5))
        # a 1-row or 1-column matrix has one singular value; bf16 rounding of a
        # near-unit vector stays well inside the tolerance
        assert orc.rel_fro(o, ref) <= tol, u.shape
        assert sigma_dev(o, ref) <= TOL_SIGMA, u.shape


@pytest.mark.parametrize("tile", [128, 256], indirect=True)
@pytest.mark.parametrize("ns,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_mixed_coefficient_table(tile, ns, tol):
    """A different polynomial per iteration: quintic, cubic (no A^2 term), a
    purely linear step (b = c = 0: the product term vanishes) and quintic
    again, on mixed shapes."""
    announce(f"orthogonalize mixed coefficient table tile={tile} {ns}")
    table = np.array([gen.QUINTIC, gen.CUBIC, (1.25, 0.0, 0.0), gen.QUINTIC, gen.CUBIC],
                     dtype=np.float64)
    shapes = [(300, 520), (520, 300), (256, 256), (100, 700)]
    us = [gen.grad_matrix(r, c, 5, 0, i).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    ins = [dev_f32(u) for u in us]
    outs = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in ins]
    mo.orthogonalize(ins, outs, coeffs=table, steps=len(table), ns_dtype=ns)
    torch.cuda.synchronize()
    for u, o in zip(us, outs):
        ref = orc.orthogonalize(u.astype(np.float64), table)
        assert orc.rel_fro(host(o), ref) <= tol, u.shape
        assert sigma_dev(host(o), ref) <= TOL_SIGMA, u.shape


# small matrices in at most eight effective-shape groups: 64-wide tiles, all
# iterations in one launch when MUON_NS_SINGLE_LAUNCH=1
SINGLE = [(256, 512), (512, 256), (200, 333), (129, 65), (17, 257), (300, 300), (64, 1000),
          (8, 8)]
# 64-wide tiles forced: up to 960 tiles per product, so most blocks take
# several tiles of a product in turn
MANY = [(512, 512)] * 12 + [(256, 768)] * 4


@pytest.mark.parametrize("kind,shapes,force", [("quintic", SINGLE, None), ("cubic", SINGLE, None),
                                               ("mixed", SINGLE, None), ("quintic", MANY, "64")])
def test_single_launch_matches_separate_launches(kind, shapes, force, monkeypatch):
    """The one-launch path computes every tile with the code of the separate
    launches, so O must be the same bit for bit; a product that read another
    block's output before the barrier made it visible would differ.  Twenty
    calls in a row on one workspace (the counters reset themselves) all
    match, and O matches the oracle."""
    announce(f"single launch vs one launch per product, {kind}, {len(shapes)} matrices")
    if force:
        monkeypatch.setenv("MUON_TILE", force)
    table = (np.array([gen.QUINTIC, gen.CUBIC, (1.25, 0.0, 0.0), gen.QUINTIC, gen.CUBIC])
             if kind == "mixed" else _table(kind, 5))
    assert mo.plan_info(shapes, len(table), table)["launches_per_step"] > 3
    us = [gen.grad_matrix(r, c, 3, 0, i).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    ins = [dev_f32(u) for u in us]

    def run():
        outs = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in ins]
        mo.orthogonalize(ins, outs, coeffs=table, steps=len(table), ns_dtype="bf16")
        torch.cuda.synchronize()
        return outs

    want = run()
    monkeypatch.setenv("MUON_NS_SINGLE_LAUNCH", "1")
    info = mo.plan_info(shapes, len(table), table)
    assert info["launches_per_step"] == 3 and info["tile"] == 64
    for rep in range(20 if force is None else 5):
        got = run()
        for o, w, sh in zip(got, want, shapes):
            assert torch.equal(o, w), (rep, sh)
    for u, o in zip(us, want):
        ref = orc.orthogonalize(u.astype(np.float64), table)
        assert orc.rel_fro(host(o), ref) <= TOL_BF16, u.shape
        assert sigma_dev(host(o), ref) <= TOL_SIGMA, u.shape


def test_single_launch_step_twins(monkeypatch):
    """Optimizer steps through the one-launch path and through separate
    launches on identical buffers stay bitwise equal over five steps."""
    announce("single launch: optimizer twins over five steps")
    shapes = SINGLE[:4]
    gs, ws = _make(shapes, "bf16")
    pa = [_dev(w) for w in ws]
    pb = [p.clone() for p in pa]
    a = mo.Muon(pa, lr=0.02, wd=0.1, beta=0.95, steps=5)
    b = mo.Muon(pb, lr=0.02, wd=0.1, beta=0.95, steps=5)
    for t in range(5):
        grads = [_dev(gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 1, t, i, 1e-3).astype(np.float32)))
                 for i, (r, c) in enumerate(shapes)]
        monkeypatch.setenv("MUON_NS_SINGLE_LAUNCH", "1")
        a.step(grads)
        monkeypatch.delenv("MUON_NS_SINGLE_LAUNCH")
        b.step(grads)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(pa[i], pb[i]), (t, shapes[i])


def test_single_launch_failure_is_never_silent(monkeypatch):
    """A block that gives up waiting at a grid barrier (forced from the host
    with a zero poll limit, so no wait hangs) marks the step failed and every
    O comes out NaN; the next call, with the normal limit, is correct again."""
    announce("single launch: forced barrier failure")
    shapes = SINGLE[:3]
    us = [gen.grad_matrix(r, c, 4, 0, i).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    ins = [dev_f32(u) for u in us]
    outs = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in ins]
    monkeypatch.setenv("MUON_NS_SINGLE_LAUNCH", "1")
    monkeypatch.setenv("MUON_NS_SPIN_LIMIT", "0")
    mo.orthogonalize(ins, outs, coeffs=_table("quintic", 5), steps=5, ns_dtype="bf16")
    torch.cuda.synchronize()
    for o in outs:
        assert bool(torch.isnan(o).all())
    monkeypatch.delenv("MUON_NS_SPIN_LIMIT")
    mo.orthogonalize(ins, outs, coeffs=_table("quintic", 5), steps=5, ns_dtype="bf16")
    torch.cuda.synchronize()
    for u, o in zip(us, outs):
        ref = orc.orthogonalize(u.astype(np.float64), _table("quintic", 5))
        assert orc.rel_fro(host(o), ref) <= TOL_BF16, u.shape


@pytest.mark.parametrize("tile", [256], indirect=True)
def test_tiny_coefficient_ratios_run_unfolded(tile):
    """The 256-wide bf16 products fold the term bA (or aX) into their
    accumulators as (b/c)A (or (a/b)X).  Rows where that ratio would overflow
    fp32 -- c tiny or subnormal, a cubic row with tiny b -- must give the
    oracle's result (the library then adds the term at the store), and the
    step keeps its separate finish kernel."""
    announce(f"orthogonalize tiny coefficient ratios tile={tile}")
    rows = [gen.QUINTIC, (1.875, -1.25, 1e-30), (1.5, 1e-38, 0.0), gen.QUINTIC,
            (1.5, -0.5, 1e-40)]
    # the library takes fp32 coefficients: the oracle gets the same values
    table = np.array(rows, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        assert np.float32(1e-40) != 0 and np.isinf(np.float32(-1.25) / np.float32(1e-40))
    shapes = [(768, 3072), (3072, 768), (300, 520), (256, 256)]
    us = [gen.grad_matrix(r, c, 6, 0, i).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    ins = [dev_f32(u) for u in us]
    outs = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in ins]
    mo.orthogonalize(ins, outs, coeffs=table, steps=len(table), ns_dtype="bf16")
    torch.cuda.synchronize()
    for u, o in zip(us, outs):
        O = host(o)
        assert np.all(np.isfinite(O)), u.shape
        ref = orc.orthogonalize(u.astype(np.float64), table)
        assert orc.rel_fro(O, ref) <= TOL_BF16, u.shape
        assert sigma_dev(O, ref) <= TOL_SIGMA, u.shape
    info = mo.plan_info(shapes, len(table), table)
    assert info["tile"] == 256
    # prepare, four rows with a polynomial launch, one without, and a separate
    # finish launch (the update cannot run in the last product's epilogue)
    assert info["launches_per_step"] == 2 + 4 * 3 + 2
    # a full step with this table against the oracle's fp32 update of the same O
    gs, ws = _make([(768, 3072), (512, 256)], "bf16")
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, lr=0.02, wd=0.1, beta=0.95, steps=len(table), coeffs=table,
                  diagnostics=False)
    twin = [p.clone() for p in params]
    opt_t = mo.Muon(twin, lr=0.02, wd=0.1, beta=0.95, steps=len(table), coeffs=table,
                    diagnostics=True)
    grads = [_dev(g) for g in gs]
    opt.step(grads)
    opt_t.step(grads)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        O = host(opt_t.update[i])
        assert np.all(np.isfinite(O))
        want = orc.store(orc.update_f32(_val(w), O, 0.02, 0.1), "bf16").astype(np.float32)
        np.testing.assert_array_equal(host(opt_t.params[i]), want)
        assert torch.equal(params[i], twin[i])


def test_bf16_inputs_and_outputs():
    announce("orthogonalize bf16 in/out")
    shapes = [(96, 160), (160, 96), (128, 128)]
    us = [gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 2, 0, i).astype(np.float32) * 1e-3)
          for i, (r, c) in enumerate(shapes)]
    outs = _ortho(us, "quintic", 6, "bf16", out_dtype=torch.bfloat16)
    for u, o in zip(us, outs):
        ref = orc.orthogonalize(gen.f32_from_bf16_bits(u).astype(np.float64), _table("quintic", 6))
        assert orc.rel_fro(o, ref) <= TOL_BF16
        assert sigma_dev(o, ref) <= TOL_SIGMA


@pytest.mark.parametrize("ns,tol", [("f32", 1e-6), ("bf16", 5e-3)])
def test_zero_steps_is_normalisation(ns, tol):
    announce(f"orthogonalize steps=0 {ns}")
    us = [gen.grad_matrix(r, c, 3, 0, i).astype(np.float32) for i, (r, c) in
          enumerate([(40, 72), (72, 40)])]
    outs = _ortho(us, "quintic", 0, ns)
    for u, o in zip(us, outs):
        ref = u.astype(np.float64) / (np.linalg.norm(u.astype(np.float64)) + 1e-7)
        assert orc.rel_fro(o, ref) <= tol
        assert sigma_dev(o, ref) <= TOL_SIGMA


def test_cubic_converges_to_polar_factor():
    announce("orthogonalize cubic polar")
    rng = np.random.default_rng(11)
    P, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    Q, _ = np.linalg.qr(rng.standard_normal((96, 64)))
    U = (P @ np.diag(np.linspace(1.0, 3.0, 64)) @ Q.T).astype(np.float32)
    (O,) = _ortho([U], "cubic", 16, "f32")
    Pu, _, Qt = np.linalg.svd(U.astype(np.float64), full_matrices=False)
    assert np.linalg.norm(O - Pu @ Qt) / np.sqrt(64) < 1e-4


def test_zero_matrix_gives_zero():
    announce("orthogonalize zero")
    (O,) = _ortho([np.zeros((33, 70), np.float32)], "quintic", 5, "bf16")
    assert np.all(O == 0)


# ------------------------------------------------------------ full step
def _make(shapes, dtype, seed=0, rms=1e-3):
    gs, ws = [], []
    for i, (r, c) in enumerate(shapes):
        g = gen.grad_matrix(r, c, seed, 0, i, rms).astype(np.float32)
        w = gen.param_matrix(r, c, seed, i).astype(np.float32)
        if dtype == "bf16":
            gs.append(gen.bf16_bits_from_f32(g))
            ws.append(gen.bf16_bits_from_f32(w))
        else:
            gs.append(g)
            ws.append(w)
    return gs, ws


def _dev(a):
    return dev_bf16(a) if a.dtype == np.uint16 else dev_f32(a)


def _val(a):
    return gen.f32_from_bf16_bits(a) if a.dtype == np.uint16 else a


@pytest.mark.parametrize("dtype,ns", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_step_matches_oracle(dtype, ns):
    announce(f"step {dtype} ns={ns}")
    shapes = [(256, 512), (512, 256), (200, 333), (64, 64)]
    gs, ws = _make(shapes, dtype, rms=None if dtype == "f32" else 1e-3)
    params = [_dev(w) for w in ws]
    grads = [_dev(g) for g in gs]
    lr, wd, beta = 0.02, 0.1, 0.95
    opt = mo.Muon(params, lr=lr, wd=wd, beta=beta, steps=5, coeffs="quintic", ns_dtype=ns,
                  diagnostics=True)
    opt.step(grads)
    torch.cuda.synchronize()
    st = orc.OracleState(shapes)
    w0 = [_val(w).astype(np.float64) for w in ws]
    # the C ABI takes lr and wd as fp32 numbers: the oracle gets the same values
    lr32, wd32 = float(np.float32(lr)), float(np.float32(wd))
    ref = orc.muon_step(w0, [_val(g) for g in gs], st, _table("quintic", 5), lr32, wd32, beta,
                        param_dtype=dtype)
    tol = TOL_F32 if ns == "f32" else TOL_BF16
    for i in range(len(shapes)):
        np.testing.assert_array_equal(host(opt.mom[i]), st.mom[i])
        O = host(opt.update[i])
        assert orc.rel_fro(O, ref["O"][i]) <= tol, shapes[i]
        assert sigma_dev(O, ref["O"][i]) <= TOL_SIGMA
        want = orc.store(orc.update_f32(w0[i], O, lr, wd), dtype)
        np.testing.assert_array_equal(host(params[i]).astype(np.float64), want)
        assert np.all(host(opt.mask[i]) == 1)
        # free-running: on top of lr times the deviation of O, the device's
        # three fp32 operations round at the scale of their operands (W_{t-1}
        # and lr*O, which matters where they nearly cancel) and both sides
        # round once to the storage type (half a unit each, so one unit of the
        # larger result between them)
        w = host(params[i]).astype(np.float64)
        wr = ref["params"][i]
        res = np.maximum(np.abs(w), np.abs(wr)).astype(np.float32)
        ops = np.maximum(np.abs(w0[i]), np.abs(lr32 * O)).astype(np.float32)
        unit = np.spacing(res).astype(np.float64) * (2 ** 16 if dtype == "bf16" else 1)
        ulp = unit + 4 * np.spacing(ops).astype(np.float64)
        dev = np.abs(O - ref["O"][i])
        excess = np.abs(w - wr) - (ulp + lr32 * dev)
        assert np.all(excess <= 1e-12), (shapes[i], float(excess.max()))
    assert opt.step_count == 1


@pytest.mark.parametrize("pdt,gdt", [("bf16", "f32"), ("f32", "bf16")])
def test_step_with_mixed_parameter_and_gradient_types(pdt, gdt):
    """bf16 weights with fp32 gradients (accumulated in fp32) and the
    reverse: the momentum takes the gradient's values exactly, O is within the
    bf16-path tolerance of the oracle and W is exactly the oracle's fp32
    update of the GPU's own O, stored in the weight's type."""
    announce(f"step params {pdt}, grads {gdt}")
    shapes = [(256, 512), (512, 256), (200, 333)]
    gf = [gen.grad_matrix(r, c, 6, 0, i, 1e-3).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    wf = [gen.param_matrix(r, c, 6, i).astype(np.float32) for i, (r, c) in enumerate(shapes)]
    gs = [gen.bf16_bits_from_f32(g) if gdt == "bf16" else g for g in gf]
    ws = [gen.bf16_bits_from_f32(w) if pdt == "bf16" else w for w in wf]
    params = [_dev(w) for w in ws]
    grads = [_dev(g) for g in gs]
    lr, wd, beta = 0.02, 0.1, 0.95
    opt = mo.Muon(params, lr=lr, wd=wd, beta=beta, steps=5, coeffs="quintic", diagnostics=True)
    opt.step(grads)
    torch.cuda.synchronize()
    lr32, wd32 = float(np.float32(lr)), float(np.float32(wd))
    for i in range(len(shapes)):
        G = _val(gs[i])
        M = orc.momentum_f32(np.zeros(shapes[i], np.float32), G, beta)
        np.testing.assert_array_equal(host(opt.mom[i]), M)
        O = host(opt.update[i])
        ref = orc.orthogonalize(M.astype(np.float64), _table("quintic", 5))
        assert orc.rel_fro(O, ref) <= TOL_BF16, shapes[i]
        assert sigma_dev(O, ref) <= TOL_SIGMA, shapes[i]
        want = orc.store(orc.update_f32(_val(ws[i]), O, lr32, wd32), pdt)
        np.testing.assert_array_equal(host(params[i]).astype(np.float64), want)


def test_anvil_ten_steps_state_forced():
    """Fast/slow momentum, six map steps, cautious decay, EMA: at every step the
    oracle starts from the GPU's stored state and must agree exactly on the
    state, the mask and the update arithmetic, and within tolerance on O."""
    announce("anvil 10 steps")
    shapes = [(128, 256), (256, 128), (96, 96), (100, 37)]
    _, ws = _make(shapes, "bf16")
    params = [_dev(w) for w in ws]
    lr, wd, beta, bs, be = 0.02, 0.1, 0.9, 0.99, 0.99
    opt = mo.Muon(params, lr=lr, wd=wd, beta=beta, steps=6, coeffs="quintic", beta_slow=bs,
                  beta_ema=be, ema_start=1, cautious=True, diagnostics=True)
    coeffs = _table("quintic", 6)
    M = [np.zeros(s, np.float32) for s in shapes]
    S = [np.zeros(s, np.float32) for s in shapes]
    E = [np.zeros(s, np.float32) for s in shapes]
    W = [_val(w) for w in ws]
    for t in range(1, 11):
        gs = [gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 0, t, i, 1e-3).astype(np.float32))
              for i, (r, c) in enumerate(shapes)]
        opt.step([_dev(g) for g in gs])
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            g = _val(gs[i])
            M[i] = orc.momentum_f32(M[i], g, beta)
            S[i] = orc.momentum_f32(S[i], g, bs)
            np.testing.assert_array_equal(host(opt.mom[i]), M[i])
            np.testing.assert_array_equal(host(opt.mom_slow[i]), S[i])
            mask = orc.cautious_mask(W[i], S[i])
            np.testing.assert_array_equal(host(opt.mask[i]).astype(bool), mask)
            O = host(opt.update[i])
            ref = orc.orthogonalize(M[i].astype(np.float64), coeffs)
            assert orc.rel_fro(O, ref) <= TOL_BF16
            assert sigma_dev(O, ref) <= TOL_SIGMA
            Wn = orc.store(orc.update_f32(W[i], O, lr, wd, mask), "bf16").astype(np.float32)
            np.testing.assert_array_equal(host(params[i]), Wn)
            E[i] = Wn.copy() if t == 1 else orc.ema_f32(E[i], Wn, be)
            np.testing.assert_array_equal(host(opt.ema[i]), E[i])
            W[i] = host(params[i])
        assert opt.step_count == t and opt.ema_count == t


def test_weighted_average_state_forced():
    """Weighted running mean of the weights (SWA with unit weights, weighted
    checkpoint averaging otherwise) from step 2 on, weights changing per step:
    the average must equal the oracle's recurrence on the GPU's own weights,
    bit for bit, and the weight sum must follow."""
    announce("weighted average 6 steps")
    shapes = [(128, 256), (256, 128), (100, 37)]
    _, ws = _make(shapes, "bf16")
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, lr=0.02, wd=0.1, beta=0.9, steps=5, coeffs="quintic",
                  beta_ema=0.0, ema_start=2, avg="weighted")
    weights = [9.0, 1.0, 2.0, 0.5, 3.0, 1.0]    # the first is outside the window
    E = [None] * len(shapes)
    s = 0.0
    for t, wt in enumerate(weights, start=1):
        gs = [gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 0, t, i, 1e-3).astype(np.float32))
              for i, (r, c) in enumerate(shapes)]
        opt.avg_weight = wt
        opt.step([_dev(g) for g in gs])
        torch.cuda.synchronize()
        if t < 2:
            assert opt.ema_count == 0
            continue
        b, ob = orc.running_mean_coeffs(s, wt)
        for i in range(len(shapes)):
            Wn = host(params[i])
            E[i] = Wn.copy() if t == 2 else orc.average_f32(E[i], Wn, b, ob)
            np.testing.assert_array_equal(host(opt.ema[i]), E[i], err_msg=f"step {t}")
        s += wt
        assert opt.ema_count == t - 1 and opt.state.avg_weight_sum == s
    with pytest.raises(ValueError):
        opt.graph([_dev(g) for g in gs])


def test_blend():
    announce("blend")
    shapes = [(64, 96), (96, 64)]
    _, ws = _make(shapes, "bf16")
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, steps=5, beta_ema=0.9, ema_start=1)
    for t in range(3):
        opt.step([_dev(gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 0, t, i, 1e-3)
                                              .astype(np.float32))) for i, (r, c) in enumerate(shapes)])
    outs = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt.blend(outs, 0.35)
    outs_b = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    opt.blend(outs_b, 0.35)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        want = orc.blend_f32(host(params[i]), host(opt.ema[i]), 0.35)
        np.testing.assert_array_equal(host(outs[i]), want)
        np.testing.assert_array_equal(host(outs_b[i]), orc.store(want, "bf16").astype(np.float32))


def test_nesterov():
    announce("nesterov")
    shapes = [(96, 160)]
    gs, ws = _make(shapes, "bf16")
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, lr=0.02, beta=0.95, steps=5, nesterov=True, diagnostics=True)
    opt.step([_dev(g) for g in gs])
    torch.cuda.synchronize()
    g = _val(gs[0])
    M = orc.momentum_f32(np.zeros(shapes[0], np.float32), g, 0.95)
    U = orc.nesterov_f32(M, g, 0.95)
    ref = orc.orthogonalize(U.astype(np.float64), _table("quintic", 5))
    np.testing.assert_array_equal(host(opt.mom[0]), M)
    assert orc.rel_fro(host(opt.update[0]), ref) <= TOL_BF16
    assert sigma_dev(host(opt.update[0]), ref) <= TOL_SIGMA


def test_zero_gradient_pure_decay():
    announce("zero gradient")
    shapes = [(48, 80), (80, 48)]
    _, ws = _make(shapes, "f32")
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, lr=0.02, wd=1.6, steps=5, diagnostics=True)
    W = [w.copy() for w in ws]
    for _ in range(3):
        opt.step([torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes])
        W = [orc.update_f32(w, np.zeros_like(w), 0.02, 1.6) for w in W]
    torch.cuda.synchronize()
    for i in range(2):
        assert np.all(host(opt.update[i]) == 0)
        np.testing.assert_array_equal(host(params[i]), W[i])


def test_nan_stays_in_its_matrix():
    announce("nan confinement")
    shapes = [(64, 96), (96, 64), (64, 96)]
    gs, ws = _make(shapes, "bf16")
    g0 = gen.f32_from_bf16_bits(gs[0]).copy()
    g0[3, 5] = np.nan
    gs[0] = gen.bf16_bits_from_f32(g0)
    params = [_dev(w) for w in ws]
    opt = mo.Muon(params, steps=5)
    opt.step([_dev(g) for g in gs])
    torch.cuda.synchronize()
    assert np.isnan(host(params[0])).all()
    assert np.isfinite(host(params[1])).all() and np.isfinite(host(params[2])).all()


def test_deterministic_and_resumable():
    announce("determinism and resume")
    shapes = [(128, 200), (200, 128), (64, 64)]
    _, ws = _make(shapes, "bf16")

    def grads(t):
        return [_dev(gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 5, t, i, 1e-3)
                                            .astype(np.float32))) for i, (r, c) in enumerate(shapes)]

    def run(n0, n1, resume_from=None):
        params = [_dev(w) for w in ws]
        opt = mo.Muon(params, lr=0.02, wd=0.1, beta=0.9, steps=6, beta_slow=0.99,
                      beta_ema=0.99, cautious=True)
        if resume_from is not None:
            sd, pw = resume_from
            opt.load_state_dict(sd)
            for p, w in zip(params, pw):
                p.copy_(w)
        for t in range(n0, n1):
            opt.step(grads(t))
        torch.cuda.synchronize()
        return opt, params

    a, pa = run(0, 10)
    b, pb = run(0, 10)
    for x, y in zip(pa, pb):
        assert torch.equal(x, y)
    h, ph = run(0, 5)
    r, pr = run(5, 10, resume_from=(h.state_dict(), [p.clone() for p in ph]))
    for x, y in zip(pa, pr):
        assert torch.equal(x, y)
    for x, y in zip(a.ema, r.ema):
        assert torch.equal(x, y)
    assert r.step_count == 10 and r.ema_count == 10


def test_workspace_reallocated_at_the_same_address():
    """Free every buffer of a step and allocate the same configuration again:
    the allocator tends to hand out the same addresses, so the per-call
    descriptor table must be sent again rather than assumed to be resident."""
    announce("step after freeing and reallocating identical buffers")
    shapes = [(300, 520), (520, 300), (256, 256)]

    def one_round():
        dev = torch.device("cuda")
        p = [gen.torch_param_matrix(r, c, 4, i, dev, dtype=torch.bfloat16)
             for i, (r, c) in enumerate(shapes)]
        g = [gen.torch_grad_matrix(r, c, 4, 0, i, dev, rms=1e-3, dtype=torch.bfloat16)
             for i, (r, c) in enumerate(shapes)]
        opt = mo.Muon(p, lr=0.02, wd=0.01, steps=5)
        opt.step(g)
        torch.cuda.synchronize()
        out = [host(t) for t in p] + [host(m) for m in opt.mom]
        del opt, p, g
        torch.cuda.empty_cache()
        return out

    first = one_round()
    for _ in range(2):
        again = one_round()
        for a, b in zip(first, again):
            assert np.all(np.isfinite(b))
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("tile,ns", [(64, "bf16"), (128, "bf16"), (256, "bf16"), (128, "f32")],
                         indirect=["tile"])
def test_twin_optimizers_stay_bitwise_equal(tile, ns):
    """Several optimizers stepped in turn on identical buffers must agree bit
    for bit after every step: the products have a fixed summation order, so
    any difference means a kernel read LDS or memory that another wave was
    still changing (block timing differs from launch to launch)."""
    announce(f"twin optimizers, tile {tile}, {ns} operands")
    shapes = [(768, 3072), (3072, 768), (768, 768), (200, 333), (333, 200), (64, 1000)]
    dev = torch.device("cuda")
    base = [gen.torch_param_matrix(r, c, 11, i, dev, dtype=torch.bfloat16)
            for i, (r, c) in enumerate(shapes)]
    twins = 6
    params = [[p.clone() for p in base] for _ in range(twins)]
    opts = [mo.Muon(p, lr=0.02, wd=0.1, beta=0.9, steps=5, ns_dtype=ns, diagnostics=True)
            for p in params]
    for t in range(8):
        g = [gen.torch_grad_matrix(r, c, 11, t, i, dev, rms=1e-3, dtype=torch.bfloat16)
             for i, (r, c) in enumerate(shapes)]
        for o in opts:
            o.step(g)
        torch.cuda.synchronize()
        for k in range(1, twins):
            for i in range(len(shapes)):
                assert torch.equal(opts[0].update[i], opts[k].update[i]), (t, k, i)
                assert torch.equal(params[0][i], params[k][i]), (t, k, i)
                assert torch.equal(opts[0].mom[i], opts[k].mom[i]), (t, k, i)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_views_match_oracle(dtype):
    """Parameters and gradients that are column windows of wider buffers:
    row pitch larger than the width, odd pitches and bases that break 16-byte
    alignment (the elementwise kernels' scalar paths), tall and wide.  The
    step must match the oracle and leave the rest of each buffer untouched."""
    announce(f"strided views {dtype}")
    shapes = [(200, 333), (333, 200), (64, 130)]
    pitches = [1001, 257, 136]
    gs, ws = _make(shapes, dtype, rms=None if dtype == "f32" else 1e-3)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sentinel = 7.0
    bufs, params, grads = [], [], []
    for (r, c), ld, g, w in zip(shapes, pitches, gs, ws):
        pb = torch.full((r, ld), sentinel, dtype=tdt, device="cuda")
        gb = torch.full((r, ld + 5), sentinel, dtype=tdt, device="cuda")
        pv, gv = pb[:, 3:3 + c], gb[:, 1:1 + c]
        pv.copy_(_dev(w))
        gv.copy_(_dev(g))
        bufs.append((pb, gb, 3, 1))
        params.append(pv)
        grads.append(gv)
    lr, wd, beta = 0.02, 0.1, 0.95
    opt = mo.Muon(params, lr=lr, wd=wd, beta=beta, steps=5, coeffs="quintic", diagnostics=True)
    opt.step(grads)
    torch.cuda.synchronize()
    st = orc.OracleState(shapes)
    w0 = [_val(w).astype(np.float64) for w in ws]
    lr32, wd32 = float(np.float32(lr)), float(np.float32(wd))
    ref = orc.muon_step(w0, [_val(g) for g in gs], st, _table("quintic", 5), lr32, wd32, beta,
                        param_dtype=dtype)
    for i, (r, c) in enumerate(shapes):
        np.testing.assert_array_equal(host(opt.mom[i]), st.mom[i])
        O = host(opt.update[i])
        assert orc.rel_fro(O, ref["O"][i]) <= TOL_BF16, shapes[i]
        assert sigma_dev(O, ref["O"][i]) <= TOL_SIGMA, shapes[i]
        want = orc.store(orc.update_f32(w0[i], O, lr, wd), dtype)
        np.testing.assert_array_equal(host(params[i]).astype(np.float64), want)
        pb, gb, po, go = bufs[i]
        hp, hg = host(pb), host(gb)
        hp[:, po:po + c] = sentinel
        hg[:, go:go + c] = sentinel
        assert np.all(hp == sentinel) and np.all(hg == sentinel), shapes[i]
