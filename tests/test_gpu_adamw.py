"""GPU parity of the AdamW entry point (muon_adamw_step) against the CPU
oracle: moments bit for bit, parameters within one rounding of the stored
type, state forced from the device at every step."""
import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import adamw_oracle as ada
from oracle import muon_oracle as orc
from tests.gpu_helpers import announce, host
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def _check_params(p_dev, p_prev, m, v, t, hp, dtype, where):
    lr, b1, b2, eps, wd = hp
    ref = ada.adamw_update_f64(p_prev, m, v, t, lr, b1, b2, eps, wd)
    got = host(p_dev).astype(np.float64)
    # fp32 arithmetic error of the device, relative to the size of the terms
    # (p and lr*u nearly cancel for some elements, so it is absolute)
    f32_err = 16 * 2.0 ** -24 * ada.adamw_update_bound(p_prev, m, v, t, lr, b1, b2, eps, wd)
    if dtype == torch.bfloat16:
        # plus one rounding to bf16 on either side
        exp = orc.store(ref, "bf16")
        bad = np.abs(got - exp) > _bf16_ulp(ref) * 1.0001 + f32_err
    else:
        bad = np.abs(got - ref) > f32_err
    assert not bad.any(), (where, int(bad.sum()), np.flatnonzero(bad)[:5])


def _make(sizes, pdts, gdts, seed, state=False, unaligned=()):
    dev = torch.device("cuda")
    params, keep = [], []
    for i, (n, dt) in enumerate(zip(sizes, pdts)):
        t = gen.torch_flat(gen.flat_param(n, seed, i, std=0.5), dev, dt)
        if i in unaligned:
            # one element into a larger buffer: 4- or 2-byte aligned, not 16
            big = torch.empty(n + 8, dtype=dt, device=dev)
            big[1:1 + n].copy_(t)
            keep.append(big)
            t = big[1:1 + n]
        params.append(t)
    opt = mo.AdamW(params, lr=1e-2, betas=(0.9, 0.95), eps=1e-8, wd=0.1)
    if state:
        for i, n in enumerate(sizes):
            m, v = gen.flat_moments(n, seed, i)
            opt.m[i].copy_(torch.from_numpy(m))
            opt.v[i].copy_(torch.from_numpy(v))
    grads = lambda t: [gen.torch_flat(gen.flat_grad(n, seed, t, i), dev, dt)  # noqa: E731
                       for i, (n, dt) in enumerate(zip(sizes, gdts))]
    return opt, params, grads, keep


def _step_and_check(opt, params, g, hp, pdts, tag):
    p_prev = [host(p).astype(np.float64) for p in params]
    m_prev = [host(x) for x in opt.m]
    v_prev = [host(x) for x in opt.v]
    g_host = [host(x) for x in g]
    opt.step(g)
    torch.cuda.synchronize()
    t = opt.step_count
    for i in range(len(params)):
        m_o, v_o = ada.adamw_moments_f32(m_prev[i], v_prev[i], g_host[i], hp[1], hp[2])
        np.testing.assert_array_equal(host(opt.m[i]), m_o, err_msg=f"{tag} m[{i}]")
        np.testing.assert_array_equal(host(opt.v[i]), v_o, err_msg=f"{tag} v[{i}]")
        _check_params(params[i], p_prev[i], m_o, v_o, t, hp, pdts[i], f"{tag} p[{i}]")


HP = (1e-2, 0.9, 0.95, 1e-8, 0.1)


def test_ragged_tensor_list_four_steps():
    """Sizes around the 4096-element chunk, an empty tensor, mixed element
    types and two buffers that are not 16-byte aligned."""
    announce("adamw ragged list, 4 steps")
    bf, f32 = torch.bfloat16, torch.float32
    sizes = [1, 7, 4095, 4096, 4097, 10000, 2309, 0, 50001, 8]
    pdts = [bf, f32, bf, bf, f32, bf, f32, bf, bf, f32]
    gdts = [f32, bf, bf, f32, f32, bf, bf, f32, bf, f32]
    opt, params, grads, _keep = _make(sizes, pdts, gdts, seed=1, unaligned=(4, 6))
    for t in range(4):
        _step_and_check(opt, params, grads(t), HP, pdts, f"step {t + 1}")
    assert opt.step_count == 4


def test_late_step_from_a_nontrivial_state():
    """Bias terms at a large step count, moments not starting from zero."""
    announce("adamw step 1000 from a seeded state")
    bf = torch.bfloat16
    sizes = [3000, 12345]
    opt, params, grads, _ = _make(sizes, [bf, bf], [bf, bf], seed=2, state=True)
    opt.state.step = 999
    _step_and_check(opt, params, grads(0), HP, [bf, bf], "step 1000")


def test_zero_gradient_and_nan_confinement():
    announce("adamw zero gradient, NaN confined to its elements")
    f32 = torch.float32
    sizes = [5000, 5000]
    opt, params, grads, _ = _make(sizes, [f32, f32], [f32, f32], seed=3)
    g = [torch.zeros(5000, device="cuda"), grads(0)[1]]
    _step_and_check(opt, params, g, HP, [f32, f32], "zero grad")
    p1 = host(params[1]).copy()
    g = [torch.zeros(5000, device="cuda"), torch.zeros(5000, device="cuda")]
    g[0][17] = float("nan")
    opt.step(g)
    torch.cuda.synchronize()
    p0 = host(params[0])
    assert np.isnan(p0[17]) and np.isfinite(np.delete(p0, 17)).all()
    assert np.isfinite(host(params[1])).all() and not np.array_equal(host(params[1]), p1)


def test_full_size_gpt124m_non_matrix_parameters():
    """The 124M model's embeddings, LayerNorm and bias vectors (124 tensors,
    39.5M elements), bf16, from a seeded state at step 50: every element."""
    announce("adamw gpt124m non-matrix set, full size")
    bf = torch.bfloat16
    sizes = gen.gpt124m_adamw_sizes()
    n = len(sizes)
    opt, params, grads, _ = _make(sizes, [bf] * n, [bf] * n, seed=4, state=True)
    opt.state.step = 49
    _step_and_check(opt, params, grads(0), HP, [bf] * n, "gpt124m step 50")


def test_repeatable_bit_for_bit():
    announce("adamw twins agree bit for bit")
    bf = torch.bfloat16
    sizes = [70000, 4096 * 3 + 5]
    a, pa, grads, _ = _make(sizes, [bf, bf], [bf, bf], seed=5)
    b, pb, _, _ = _make(sizes, [bf, bf], [bf, bf], seed=5)
    for t in range(3):
        g = grads(t)
        a.step(g)
        b.step(g)
    torch.cuda.synchronize()
    for x, y in zip(pa + a.m + a.v, pb + b.m + b.v):
        assert torch.equal(x, y)


def test_capture_is_refused():
    """The bias terms change every step: a captured AdamW step would replay
    stale ones, so the call refuses capture and leaves everything as it was."""
    announce("adamw refuses graph capture")
    bf = torch.bfloat16
    opt, params, grads, _ = _make([5000], [bf], [bf], seed=6)
    g = grads(0)
    opt.step(g)
    torch.cuda.synchronize()
    before = [host(x).copy() for x in params + opt.m + opt.v]
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(mo._lib.MuonError) as err:
        with torch.cuda.graph(graph):
            opt.step(g)
    assert err.value.code == mo._lib.CODES["MUON_E_CAPTURE"]
    torch.cuda.synchronize()
    assert opt.step_count == 1
    for a, b in zip(before, [host(x) for x in params + opt.m + opt.v]):
        np.testing.assert_array_equal(a, b)
    opt.step(g)                       # eager steps still work afterwards
    torch.cuda.synchronize()
    assert opt.step_count == 2


def test_tensor_beyond_int32_elements():
    """One bf16 tensor of 2^31 + 4099 elements (64-bit element indices, a
    ragged last chunk): moments bit for bit and parameters within tolerance
    on sampled elements, including the last ones."""
    announce("adamw 2^31 + 4099 elements")
    n = 2 ** 31 + 4099
    dev = torch.device("cuda")
    gtr = torch.Generator(device=dev)
    gtr.manual_seed(31)
    p = torch.randn(n, generator=gtr, device=dev, dtype=torch.float32).mul_(0.5).to(torch.bfloat16)
    g = torch.randn(n, generator=gtr, device=dev, dtype=torch.float32).mul_(1e-3).to(torch.bfloat16)
    opt = mo.AdamW([p], lr=1e-2, betas=(0.9, 0.95), eps=1e-8, wd=0.1)
    idx = torch.cat([torch.randint(0, n, (20000,), generator=gtr, device=dev),
                     torch.arange(n - 5000, n, device=dev),
                     torch.arange(2 ** 31 - 64, 2 ** 31 + 64, device=dev)])
    p0 = host(p[idx]).astype(np.float64)
    gs = host(g[idx])
    opt.step([g])
    torch.cuda.synchronize()
    m_o, v_o = ada.adamw_moments_f32(np.zeros(len(gs), np.float32), np.zeros(len(gs), np.float32),
                                     gs, HP[1], HP[2])
    np.testing.assert_array_equal(host(opt.m[0][idx]), m_o)
    np.testing.assert_array_equal(host(opt.v[0][idx]), v_o)
    _check_params(p[idx], p0, m_o, v_o, 1, HP, torch.bfloat16, "p")
