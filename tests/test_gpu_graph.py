"""Graph capture of the whole optimizer step: every replay against an eager
twin optimizer on identical buffers, bit for bit (same kernels, same inputs,
deterministic reductions), with eager device work and synchronisation
between replays."""
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from tests.gpu_helpers import announce
from workloads import gen

pytestmark = pytest.mark.gpu

SHAPES = [(768, 3072), (3072, 768), (768, 768), (200, 333), (333, 200), (64, 1000)]
# small enough for 64-wide tiles: all iterations in one launch on request
SMALL = [(256, 512), (512, 256), (200, 333), (64, 64)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


def _params(seed, shapes=SHAPES):
    dev = torch.device("cuda")
    return [gen.torch_param_matrix(r, c, seed, i, dev, dtype=torch.bfloat16)
            for i, (r, c) in enumerate(shapes)]


def _grads(seed, step, shapes=SHAPES):
    dev = torch.device("cuda")
    return [gen.torch_grad_matrix(r, c, seed, step, i, dev, rms=1e-3, dtype=torch.bfloat16)
            for i, (r, c) in enumerate(shapes)]


def _eager_work():
    x = torch.randn(512, 512, device="cuda")
    y = (x @ x).sum()
    torch.cuda.synchronize()
    return float(y)


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def _run(kw, eager_first, replays, shapes=SHAPES):
    pa = _params(7, shapes)
    pb = [p.clone() for p in pa]
    A = mo.Muon(pa, **kw)
    B = mo.Muon(pb, **kw)
    static = [torch.empty_like(g) for g in _grads(7, 0, shapes)]
    t = 0
    for _ in range(eager_first):
        g = _grads(7, t, shapes)
        A.step(g)
        B.step(g)
        t += 1
    graph = B.graph(static)
    for _ in range(replays):
        g = _grads(7, t, shapes)
        for dst, src in zip(static, g):
            dst.copy_(src)
        A.step(g)
        _eager_work()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(pa, pb), t
        assert _same(A.mom, B.mom), t
        if A.mom_slow is not None:
            assert _same(A.mom_slow, B.mom_slow), t
        if A.ema is not None:
            assert _same(A.ema, B.ema), t
        assert (A.step_count, A.ema_count) == (B.step_count, B.ema_count)
        t += 1


def test_graph_replays_match_eager_plain():
    announce("graph: plain Muon, six replays")
    _run(dict(lr=0.02, wd=0.01, beta=0.95, steps=5), eager_first=0, replays=6)


def test_graph_replays_match_eager_anvil_ema():
    announce("graph: fast/slow momentum, cautious decay, weight average")
    kw = dict(lr=0.02, wd=0.1, beta=0.9, steps=6, beta_slow=0.99, cautious=True,
              beta_ema=0.99, ema_start=1)
    _run(kw, eager_first=2, replays=5)


def test_graph_replays_match_eager_single_launch(monkeypatch):
    """A small set whose iterations run in one launch with grid barriers: the
    barrier counters reset themselves at the end of every replay."""
    announce("graph: small set, all iterations in one launch, eight replays")
    monkeypatch.setenv("MUON_NS_SINGLE_LAUNCH", "1")
    assert mo.plan_info(SMALL, 5)["launches_per_step"] == 3
    _run(dict(lr=0.02, wd=0.01, beta=0.95, steps=5), eager_first=1, replays=8, shapes=SMALL)


def test_graph_refused_before_average_starts():
    announce("graph: capture refused before the weight average starts")
    p = _params(8)
    opt = mo.Muon(p, beta_ema=0.99, ema_start=3)
    with pytest.raises(ValueError):
        opt.graph(_grads(8, 0))
    assert opt.step_count == 0


def test_c_abi_refuses_capture_of_weighted_average_steps():
    """The weighted average's coefficients change every step; muon_step
    itself (not only the Python wrapper) refuses to be captured for such a
    step, enqueues nothing and leaves the counters alone."""
    announce("graph: C ABI refuses capture with the weighted average")
    p = _params(9)
    opt = mo.Muon(p, beta_ema=0.0, ema_start=1, avg="weighted")
    g = _grads(9, 0)
    opt.step(g)
    torch.cuda.synchronize()
    opt.step_prepare(g)
    torch.cuda.synchronize()
    before = [x.clone() for x in p]
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(mo._lib.MuonError) as err:
        with torch.cuda.graph(graph):
            code = opt.lib.muon_step(opt._pmats, opt._grad_mats(g), opt.state, opt._coeffs_c,
                                     opt.steps, opt.lr, opt.wd, opt.beta,
                                     torch.cuda.current_stream().cuda_stream)
            mo._lib.check(code, "muon_step")
    assert err.value.code == mo._lib.CODES["MUON_E_CAPTURE"]
    torch.cuda.synchronize()
    assert opt.step_count == 1 and opt.ema_count == 1
    assert all(torch.equal(a, b) for a, b in zip(before, p))


def test_graph_replays_survive_blends_and_eager_calls_on_the_workspace():
    """Between replays: a readout blend, an eager step on other gradient
    buffers and an orthogonalisation through the same workspace.  Those calls
    send their own descriptor tables; the replayed step must still read the
    one muon_step_prepare sent (a separate region of the workspace) and stay
    bit for bit equal to an eager twin that makes the same calls."""
    announce("graph: replays with blends and eager calls in between")
    kw = dict(lr=0.02, wd=0.1, beta=0.9, steps=5, beta_ema=0.99, ema_start=1)
    pa = _params(12)
    pb = [p.clone() for p in pa]
    A = mo.Muon(pa, **kw)
    B = mo.Muon(pb, **kw)
    static = [torch.empty_like(g) for g in _grads(12, 0)]
    g = _grads(12, 0)
    A.step(g)
    B.step(g)
    graph = B.graph(static)
    for t in range(1, 5):
        g = _grads(12, t)
        for dst, src in zip(static, g):
            dst.copy_(src)
        A.step(g)
        graph.replay()
        torch.cuda.synchronize()
        assert _same(pa, pb), t
        assert _same(A.mom, B.mom) and _same(A.ema, B.ema), t
        assert (A.step_count, A.ema_count) == (B.step_count, B.ema_count), t
        # calls that send other tables into the same workspaces
        oa = [torch.empty(p.shape, dtype=torch.float32, device="cuda") for p in pa]
        ob = [torch.empty_like(x) for x in oa]
        A.blend(oa, 0.35)
        B.blend(ob, 0.35)
        torch.cuda.synchronize()
        assert _same(oa, ob), t
        if t % 2:
            other = _grads(13, t)
            A.step(other)
            B.step(other)
        ins = _grads(14, t)
        ua = [torch.empty(p.shape, dtype=torch.float32, device="cuda") for p in pa]
        ub = [torch.empty_like(x) for x in ua]
        mo.orthogonalize(ins, ua, steps=5, workspace=A.workspace)
        mo.orthogonalize(ins, ub, steps=5, workspace=B.workspace)
        torch.cuda.synchronize()
        assert _same(ua, ub), t
        assert _same(pa, pb), t
