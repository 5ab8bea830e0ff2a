"""GPU parity at the full sizes of the model-shaped matrix sets, in the launch
configuration the benchmark times (default tile and wave choice).

Every matrix is checked exactly where the result is exact (momentum, slow
momentum, EMA, masks, the update arithmetic given the GPU's own O, counters).
The orthogonalised update O is compared with the fp64 oracle (relative
Frobenius error and singular values) on every matrix of the 124M set (one
plain step; the first and last of ten ANVIL steps) and, on the 2.7B and MoE
sets, on one matrix per effective-shape group and residue of its slot modulo
eight (the grouped launches deal slot j of every group to XCD j mod 8)."""
import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import muon_oracle as orc
from tests.gpu_helpers import TOL_BF16, TOL_F32, TOL_SIGMA, announce, host, sigma_dev
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


def _check_o(O, M, coeffs, shape, tol=TOL_BF16):
    ref = orc.orthogonalize(M.astype(np.float64), coeffs)
    err = orc.rel_fro(O, ref)
    assert err <= tol, (shape, err)
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
    for i, (g, w) in enumerate(inputs):
        G = gen.f32_from_bf16_bits(g)
        M = orc.momentum_f32(np.zeros(shapes[i], np.float32), G, ms.beta)
        np.testing.assert_array_equal(host(opt.mom[i]), M)
        O = host(opt.update[i])
        W0 = gen.f32_from_bf16_bits(w)
        want = orc.store(orc.update_f32(W0, O, lr32, ms.wd), "bf16").astype(np.float32)
        np.testing.assert_array_equal(host(params[i]), want)
        _check_o(O, M, coeffs, shapes[i])
    assert opt.step_count == 1


def test_gpt124m_fp32_iterations_full_size():
    """The fp32 Newton-Schulz path (fp32 MFMA, 128-wide tiles) on the whole
    124M set: O of every matrix within the fp32 tolerance of the oracle."""
    announce("full size: gpt124m one step, fp32 iterations")
    ms = gen.SETS["gpt124m"]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    inputs = gen.make_inputs(ms, seed=2)
    params = [_dev_bits(w) for _, w in inputs]
    grads = [_dev_bits(g) for g, _ in inputs]
    opt = mo.Muon(params, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  ns_dtype="f32", diagnostics=True)
    assert mo.plan_info(shapes, ms.steps, coeffs, ns_dtype="f32")["tile"] == 128
    opt.step(grads)
    torch.cuda.synchronize()
    for i, (g, _) in enumerate(inputs):
        M = orc.momentum_f32(np.zeros(shapes[i], np.float32), gen.f32_from_bf16_bits(g), ms.beta)
        np.testing.assert_array_equal(host(opt.mom[i]), M)
        _check_o(host(opt.update[i]), M, coeffs, shapes[i], tol=TOL_F32)


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
            if t in (1, ms.n_opt_steps):
                _check_o(O, M[i], coeffs, s)
            W[i] = Wn
        assert opt.step_count == t and opt.ema_count == t
        del gdev


def _group_residue_sample(shapes, group):
    """Matrix indices: for the effective-shape group `group` (its rank among
    the groups in order of first appearance), the first slot of each residue
    modulo eight."""
    eff = [(min(r, c), max(r, c)) for r, c in shapes]
    keys = list(dict.fromkeys(eff))
    members = [i for i, k in enumerate(eff) if k == keys[group]]
    return members[:8]


@pytest.mark.parametrize("name,group", [("gpt2p7b", 0), ("gpt2p7b", 1), ("moe_share", 0),
                                        ("moe_share", 1)])
def test_large_sets_one_step_per_group_and_residue(name, group):
    ms = gen.SETS[name]
    shapes = list(ms.shapes)
    sample = _group_residue_sample(shapes, group)
    assert len(sample) == 8
    announce(f"full size: {name} one step, O checked on matrices {sample}")
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
    # every matrix: the first momentum is fl((1 - beta) G) and the update
    # fl(fl(W - fl(fl(lr wd) W)) - fl(lr O)) rounded to bf16, each operation a
    # separate correctly rounded torch kernel in fp32; O is finite and nonzero,
    # and its squared Frobenius norm (the sum of m squared singular values,
    # each mapped into [0, 1] by the convergent quintic) is at most m up to
    # the bf16 tolerance
    ob = torch.tensor(np.float32(1.0) - np.float32(ms.beta), device=dev)
    lr_t = torch.tensor(np.float32(ms.lr), device=dev)
    lrwd_t = torch.tensor(np.float32(ms.lr) * np.float32(ms.wd), device=dev)
    for i, s in enumerate(shapes):
        assert torch.equal(opt.mom[i], ob * grads[i].float()), (i, s)
        o = opt.update[i]
        w_prev = gen.torch_param_matrix(*s, 0, i, dev, dtype=torch.bfloat16).float()
        want = ((w_prev - lrwd_t * w_prev) - lr_t * o).to(torch.bfloat16)
        assert torch.equal(params[i], want), (i, s)
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


def test_gpt124m_anvil_free_running_one_layer():
    """Free-running comparison of the ANVIL-style step (page "Training
    NanoGPT in 39.9 Seconds", section "ANVIL II와 가중치 평균"): the GPU and
    the oracle each step their own weights for ten steps on one layer of the
    124M set.  The momenta do not depend on the weights and must agree bit for
    bit; O agrees within the bf16 tolerance at every step; the weights drift
    apart by at most what the O deviations and one bf16 rounding per step
    allow, and the count of weight elements by distance in bf16 units and of
    flipped decay-mask elements is printed per step."""
    announce("full size: gpt124m ANVIL free-running, one layer, ten steps")
    ms = gen.SETS["gpt124m_anvil"]
    shapes = list(ms.shapes)[:6]
    assert sorted(shapes) == sorted([(768, 768)] * 4 + [(768, 3072), (3072, 768)])
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    w_bits = [gen.bf16_bits_from_f32(gen.param_matrix(r, c, 0, i).astype(np.float32))
              for i, (r, c) in enumerate(shapes)]
    pdev = [_dev_bits(w) for w in w_bits]
    opt = mo.Muon(pdev, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  beta_slow=ms.beta_slow, beta_ema=ms.beta_ema, ema_start=ms.ema_start,
                  cautious=True, diagnostics=True)
    lr32, wd32 = float(np.float32(ms.lr)), float(np.float32(ms.wd))
    st = orc.OracleState(shapes, beta_slow=ms.beta_slow, beta_ema=ms.beta_ema,
                         ema_start=ms.ema_start)
    W_orc = [gen.f32_from_bf16_bits(w).astype(np.float64) for w in w_bits]
    bound = [np.zeros(s) for s in shapes]       # elementwise bound on |W_gpu - W_orc|
    emax = [np.zeros(s) for s in shapes]
    for t in range(1, ms.n_opt_steps + 1):
        g_bits = [gen.bf16_bits_from_f32(gen.grad_matrix(r, c, 0, t, i, 1e-3).astype(np.float32))
                  for i, (r, c) in enumerate(shapes)]
        opt.step([_dev_bits(g) for g in g_bits])
        torch.cuda.synchronize()
        ref = orc.muon_step(W_orc, [gen.f32_from_bf16_bits(g) for g in g_bits], st, coeffs,
                            lr32, wd32, ms.beta, param_dtype="bf16", cautious=True)
        hist = np.zeros(4, dtype=np.int64)
        flips = 0
        for i, s in enumerate(shapes):
            np.testing.assert_array_equal(host(opt.mom[i]), st.mom[i])
            np.testing.assert_array_equal(host(opt.mom_slow[i]), st.slow[i])
            O = host(opt.update[i])
            assert orc.rel_fro(O, ref["O"][i]) <= TOL_BF16, (t, s)
            assert sigma_dev(O, ref["O"][i]) <= TOL_SIGMA, (t, s)
            w_prev = np.maximum(np.abs(W_orc[i]), np.abs(W_orc[i]) + bound[i])
            w_gpu = host(pdev[i]).astype(np.float64)
            w_orc = ref["params"][i]
            # |dW_t| <= |dW_{t-1}| (1 + lr wd) + lr |dO_t| + one bf16 unit of the
            # larger weight (each side rounds once; a flipped mask only occurs
            # where the weights differ in sign, i.e. |W| <= |dW|, and changes
            # the decay term by lr wd |W|)
            # (the fp32 operations round at the scale of the previous weight)
            big = np.maximum.reduce([np.abs(w_gpu), np.abs(w_orc), w_prev]).astype(np.float32)
            ulp = np.spacing(big).astype(np.float64) * 2 ** 16
            bound[i] = bound[i] * (1 + lr32 * wd32) + lr32 * np.abs(O - ref["O"][i]) + ulp
            dw = np.abs(w_gpu - w_orc)
            assert np.all(dw <= bound[i] * (1 + 1e-6) + 1e-30), (t, s, float((dw - bound[i]).max()))
            units = np.minimum(np.rint(dw / np.maximum(ulp, 1e-45)), 3).astype(np.int64)
            hist += np.bincount(units.ravel(), minlength=4)[:4]
            flips += int(np.sum(host(opt.mask[i]).astype(bool) != ref["mask"][i]))
            # the averages are convex combinations of the weights (fp32 rounding
            # aside), so they differ by at most the largest weight deviation so far
            emax[i] = np.maximum(emax[i], dw)
            de = np.abs(host(opt.ema[i]).astype(np.float64) - st.ema[i].astype(np.float64))
            assert np.all(de <= emax[i] + 1e-5 * np.abs(st.ema[i]) + 1e-30), (t, s)
            W_orc[i] = w_orc
        n = int(hist.sum())
        print(f"step {t}: W elements by bf16 units apart (0, 1, 2, >=3): {hist.tolist()} of {n}; "
              f"mask flips {flips}", flush=True)
    assert opt.step_count == ms.n_opt_steps and opt.ema_count == ms.n_opt_steps
