"""GPU parity at the full sizes of the model-shaped matrix sets, in the launch
configuration the benchmark times (default tile and wave choice).

Every matrix is checked exactly where the result is exact (momentum, slow
momentum, EMA, masks, the update arithmetic given the GPU's own O, counters);
the orthogonalised update O is compared with the fp64 oracle on sampled
matrices, which the oracle can afford one by one."""
import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import muon_oracle as orc
from tests.gpu_helpers import TOL_BF16, TOL_SIGMA, announce, host, sigma_dev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_o(O, M, coeffs, shape):
    ref = orc.orthogonalize(M.astype(np.float64), coeffs)
    err = orc.rel_fro(O, ref)
    assert err <= TOL_BF16, (shape, err)
    assert sigma_dev(O, ref) <= TOL_SIGMA, shape


def test_gpt124m_one_step_full_size():
    announce("full size: gpt124m one step")
    ms = gen.SETS["gpt124m"]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    inputs = gen.make_inputs(ms, seed=0)
    params = [_dev_bits(w) for _, w in inputs]
    grads = [_dev_bits(g) for g, _ in inputs]
    opt = mo.Muon(params, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  diagnostics=True)
    assert mo.plan_info(shapes, ms.steps, coeffs)["tile"] == 256
    opt.step(grads)
    torch.cuda.synchronize()
    lr32 = float(np.float32(ms.lr))
    sample = {0, 4, 5, 70, 71}
    for i, (g, w) in enumerate(inputs):
        G = gen.f32_from_bf16_bits(g)
        M = orc.momentum_f32(np.zeros(shapes[i], np.float32), G, ms.beta)
        np.testing.assert_array_equal(host(opt.mom[i]), M)
        O = host(opt.update[i])
        W0 = gen.f32_from_bf16_bits(w)
        want = orc.store(orc.update_f32(W0, O, lr32, ms.wd), "bf16").astype(np.float32)
        np.testing.assert_array_equal(host(params[i]), want)
        if i in sample:
            _check_o(O, M, coeffs, shapes[i])
    assert opt.step_count == 1


def test_gpt124m_anvil_ten_steps_full_size():
    """Fast (0.9) and slow (0.99) momentum, six map steps, cautious wd 0.1, EMA
    0.99 from step 1, ten steps with fresh gradients; state-forced checks on
    all 72 matrices at every step."""
    announce("full size: gpt124m ANVIL ten steps")
    ms = gen.SETS["gpt124m_anvil"]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    params = [gen.bf16_bits_from_f32(gen.param_matrix(r, c, 0, i).astype(np.float32))
              for i, (r, c) in enumerate(shapes)]
    pdev = [_dev_bits(w) for w in params]
    opt = mo.Muon(pdev, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  beta_slow=ms.beta_slow, beta_ema=ms.beta_ema, ema_start=ms.ema_start,
                  cautious=True, diagnostics=True)
    lr32, wd32 = float(np.float32(ms.lr)), float(np.float32(ms.wd))
    M = [np.zeros(s, np.float32) for s in shapes]
    S = [np.zeros(s, np.float32) for s in shapes]
    E = [None] * len(shapes)
    W = [gen.f32_from_bf16_bits(w) for w in params]
    dev = torch.device("cuda")
    for t in range(1, ms.n_opt_steps + 1):
        gdev = [gen.torch_grad_matrix(r, c, 0, t, i, dev, rms=1e-3, dtype=torch.bfloat16)
                for i, (r, c) in enumerate(shapes)]
        opt.step(gdev)
        torch.cuda.synchronize()
        for i, s in enumerate(shapes):
            G = gen.f32_from_bf16_bits(_bits(gdev[i]))
            M[i] = orc.momentum_f32(M[i], G, ms.beta)
            S[i] = orc.momentum_f32(S[i], G, ms.beta_slow)
            np.testing.assert_array_equal(host(opt.mom[i]), M[i])
            np.testing.assert_array_equal(host(opt.mom_slow[i]), S[i])
            mask = orc.cautious_mask(W[i], S[i])
            np.testing.assert_array_equal(host(opt.mask[i]).astype(bool), mask)
            O = host(opt.update[i])
            Wn = orc.store(orc.update_f32(W[i], O, lr32, wd32, mask), "bf16").astype(np.float32)
            np.testing.assert_array_equal(host(pdev[i]), Wn)
            E[i] = Wn.copy() if t == 1 else orc.ema_f32(E[i], Wn, ms.beta_ema)
            np.testing.assert_array_equal(host(opt.ema[i]), E[i])
            if (t, i) in {(1, 0), (1, 4), (10, 5), (10, 71)}:
                _check_o(O, M[i], coeffs, s)
            W[i] = Wn
        assert opt.step_count == t and opt.ema_count == t
        del gdev


@pytest.mark.parametrize("name,sample", [("gpt2p7b", (0, 5)), ("moe_share", (0, 1, 130))])
def test_large_sets_one_step_sampled(name, sample):
    announce(f"full size: {name} one step (sampled checks)")
    ms = gen.SETS[name]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    dev = torch.device("cuda")
    params = [gen.torch_param_matrix(r, c, 0, i, dev, dtype=torch.bfloat16)
              for i, (r, c) in enumerate(shapes)]
    w0 = {i: gen.f32_from_bf16_bits(_bits(params[i])) for i in sample}
    grads = [gen.torch_grad_matrix(r, c, 0, 0, i, dev, rms=1e-3, dtype=torch.bfloat16)
             for i, (r, c) in enumerate(shapes)]
    opt = mo.Muon(params, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  diagnostics=True)
    opt.step(grads)
    torch.cuda.synchronize()
    lr32, wd32 = float(np.float32(ms.lr)), float(np.float32(ms.wd))
    for i in sample:
        G = gen.f32_from_bf16_bits(_bits(grads[i]))
        M = orc.momentum_f32(np.zeros(shapes[i], np.float32), G, ms.beta)
        np.testing.assert_array_equal(host(opt.mom[i]), M)
        O = host(opt.update[i])
        want = orc.store(orc.update_f32(w0[i], O, lr32, wd32), "bf16").astype(np.float32)
        np.testing.assert_array_equal(host(params[i]), want)
        _check_o(O, M, coeffs, shapes[i])
    # every matrix: O is finite and nonzero, and its squared Frobenius norm
    # (the sum of m squared singular values, each mapped into [0, 1] by the
    # convergent quintic) is at most m up to the bf16 tolerance
    for i, s in enumerate(shapes):
        o = opt.update[i]
        assert bool(torch.isfinite(o).all())
        fro2 = float(o.double().square().sum())
        assert 0.0 < fro2 <= min(s) * (1 + 2 * TOL_BF16), (i, s, fro2 / min(s))


@pytest.mark.parametrize("name", ["gpt124m", "gpt2p7b", "moe_share"])
def test_bench_configuration_matches_finish_kernel(name):
    """The configuration the benchmark times: no diagnostic outputs, so the
    plain update runs in the last APPLY launch.  Every parameter matrix must be
    bit for bit what a twin with diagnostic outputs (separate finish kernel,
    checked against the oracle above) writes."""
    announce(f"full size: {name} bench configuration vs finish kernel")
    ms = gen.SETS[name]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    dev = torch.device("cuda")
    pa = [gen.torch_param_matrix(r, c, 0, i, dev, dtype=torch.bfloat16)
          for i, (r, c) in enumerate(shapes)]
    pb = [p.clone() for p in pa]
    grads = [gen.torch_grad_matrix(r, c, 0, 0, i, dev, rms=1e-3, dtype=torch.bfloat16)
             for i, (r, c) in enumerate(shapes)]
    kw = dict(lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs)
    a = mo.Muon(pa, diagnostics=True, **kw)
    b = mo.Muon(pb, **kw)
    for t in range(2):
        a.step(grads)
        mo.probe_arm("finish", 4)
        b.step(grads)
        torch.cuda.synchronize()
        assert len(mo.probe_read(4)) == 0, "the benchmark configuration launched a finish kernel"
        mo.probe_disarm()
        for i in range(len(shapes)):
            assert torch.equal(pb[i], pa[i]), (t, i, shapes[i])
            assert torch.equal(b.mom[i], a.mom[i]), (t, i, shapes[i])
