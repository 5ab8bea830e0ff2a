"""The allocation-free step (muon_step_noalloc: the library's static per-GPU
scratch instead of a caller workspace) against muon_step, through the C ABI:
two calls in a row on different matrix sets, the second smaller, must give
the same parameters and state bit for bit; a set whose workspace exceeds the
scratch is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from tests.gpu_helpers import announce
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


def _sets(shapes, seed):
    dev = torch.device("cuda")
    p = [gen.torch_param_matrix(r, c, seed, i, dev, dtype=torch.bfloat16)
         for i, (r, c) in enumerate(shapes)]
    return p


def _grads(shapes, seed, t):
    dev = torch.device("cuda")
    return [gen.torch_grad_matrix(r, c, seed, t, i, dev, rms=1e-3, dtype=torch.bfloat16)
            for i, (r, c) in enumerate(shapes)]


def _noalloc_step(opt, grads):
    return opt.lib.muon_step_noalloc(opt._pmats, opt._grad_mats(grads), opt.state, opt._coeffs_c,
                                     opt.steps, opt.lr, opt.wd, opt.beta,
                                     torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("kw", [dict(lr=0.02, wd=0.1, beta=0.95, steps=5),
                                dict(lr=0.02, wd=0.1, beta=0.9, steps=6, beta_slow=0.99,
                                     cautious=True, beta_ema=0.99, ema_start=1)])
def test_noalloc_matches_muon_step_two_calls_second_smaller(kw):
    announce(f"no-alloc step vs muon_step {sorted(kw)}")
    for shapes, seed in (([(768, 3072), (3072, 768), (768, 768), (200, 333)], 21),
                         ([(96, 160), (64, 64)], 22)):
        need = mo.workspace_bytes(shapes)
        assert 0 < need <= mo._lib.NOALLOC_SCRATCH_BYTES, need
        pa = _sets(shapes, seed)
        pb = [p.clone() for p in pa]
        A = mo.Muon(pa, **kw)
        B = mo.Muon(pb, **kw)
        # the allocation-free entry point ignores the state's workspace
        B.state.workspace = None
        B.state.workspace_bytes = 0
        for t in range(2):
            g = _grads(shapes, seed, t)
            A.step(g)
            mo._lib.check(_noalloc_step(B, g), "muon_step_noalloc")
            torch.cuda.synchronize()
            for i in range(len(shapes)):
                assert torch.equal(pa[i], pb[i]), (shapes[i], t)
                assert torch.equal(A.mom[i], B.mom[i]), (shapes[i], t)
                if A.mom_slow is not None:
                    assert torch.equal(A.mom_slow[i], B.mom_slow[i]), (shapes[i], t)
                if A.ema is not None:
                    assert torch.equal(A.ema[i], B.ema[i]), (shapes[i], t)
            assert (A.step_count, A.ema_count) == (B.step_count, B.ema_count)


def test_noalloc_refuses_sets_beyond_the_scratch():
    announce("no-alloc step refuses a set larger than its scratch")
    shapes = [(3072, 3072), (3072, 3072)]
    assert mo.workspace_bytes(shapes) > mo._lib.NOALLOC_SCRATCH_BYTES
    p = _sets(shapes, 23)
    before = [x.clone() for x in p]
    opt = mo.Muon(p, lr=0.02, wd=0.1, steps=5)
    code = _noalloc_step(opt, _grads(shapes, 23, 0))
    torch.cuda.synchronize()
    assert code == mo._lib.CODES["MUON_E_WORKSPACE"]
    assert opt.step_count == 0
    assert all(torch.equal(a, b) for a, b in zip(before, p))
    assert all(not m.any() for m in opt.mom)
