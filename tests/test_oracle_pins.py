"""Pins for the CPU oracle: checks against facts fixed by the pages and by the
mathematics, independent of the oracle's own code path.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a missing normalisation, a fused or
reordered fp32 operation) fails at least one test.
"""
import math
import os
import struct

import numpy as np
import pytest

from oracle import muon_oracle as orc
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SETS = {
    "cubic": np.array([gen.CUBIC]),
    "quintic": np.array([gen.QUINTIC]),
    # not convergent, exercises every coefficient with an unusual sign mix
    "odd": np.array([(2.0, -1.3, 0.4)]),
}


def _table(kind, k):
    return np.repeat(SETS[kind], k, axis=0)


def _closed_form(U, coeffs, eps):
    """O = P diag(p_K..p_1(sigma_i / (||U||_F + eps))) Q^T from the SVD."""
    P, s, Qt = np.linalg.svd(U, full_matrices=False)
    x = s / (np.linalg.norm(U) + eps)
    px = np.array([orc.ns_poly_scalar(v, coeffs) for v in x])
    return (P * px) @ Qt


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_known_values():
    one = 1.0
    cases = {
        one + 2 ** -8: 1.0,                       # tie -> even (1.0)
        one + 3 * 2 ** -8: one + 2 ** -6,         # tie -> even (1 + 2^-6)
        one + 2 ** -8 + 2 ** -30: one + 2 ** -7,  # just above the tie
        -(one + 3 * 2 ** -8): -(one + 2 ** -6),
        0.0: 0.0,
        2.0 ** -133: 2.0 ** -133,                 # smallest bf16 subnormal
        1.5 * 2.0 ** -133: 2.0 ** -132,           # subnormal tie -> even
        3.3895313892515355e38: 3.3895313892515355e38,
        3.4e38: math.inf,
    }
    for x, want in cases.items():
        got = float(orc.round_to_bf16(np.array([x]))[0])
        assert got == want, (x, got, want)
    assert np.isnan(orc.round_to_bf16(np.array([np.nan]))[0])


def test_bf16_fast_path_matches_definition():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-40, 40, 300000))).astype(np.float32)
    x[:4] = [np.float32(1 + 2 ** -8), np.float32(1 + 3 * 2 ** -8), np.float32(-0.0), np.float32(3.4e38)]
    np.testing.assert_array_equal(orc.round_f32_to_bf16(x).astype(np.float64),
                                  orc.round_to_bf16(x.astype(np.float64)))


def test_bf16_matches_bit_rounding_on_fp32_inputs():
    # An independent implementation (integer rounding of fp32 bit patterns)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    bits = gen.bf16_bits_from_f32(x)
    want = gen.f32_from_bf16_bits(bits).astype(np.float64)
    got = orc.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# -------------------------------------------------------- NS vs closed forms
@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32), (1, 7), (9, 1)])
@pytest.mark.parametrize("kind", ["cubic", "quintic", "odd"])
@pytest.mark.parametrize("k", [1, 5, 6])
def test_ns_matches_svd_closed_form(shape, kind, k):
    rng = np.random.default_rng([3, shape[0], shape[1], k])
    U = rng.standard_normal(shape) * 1e-3
    coeffs = _table(kind, k)
    O = orc.orthogonalize(U, coeffs, eps=1e-7)
    ref = _closed_form(U, coeffs, 1e-7)
    assert orc.rel_fro(O, ref) < 1e-10


def test_ns_closed_form_on_the_single_matrix_case():
    # the 256 x 512 low-rank + noise gradient, seed 0
    G = gen.grad_matrix(256, 512, 0, 0, 0)
    for kind in ("cubic", "quintic"):
        coeffs = _table(kind, 5)
        O = orc.orthogonalize(G, coeffs)
        assert orc.rel_fro(O, _closed_form(G, coeffs, 1e-7)) < 1e-11


def test_eps_enters_as_added_to_the_norm():
    # a matrix whose norm is comparable to eps makes eps visible
    rng = np.random.default_rng(5)
    U = rng.standard_normal((6, 9))
    U *= 2e-7 / np.linalg.norm(U)
    coeffs = _table("quintic", 3)
    O = orc.orthogonalize(U, coeffs, eps=1e-7)
    np.testing.assert_allclose(O, _closed_form(U, coeffs, 1e-7), rtol=1e-10, atol=1e-14)
    assert orc.rel_fro(O, _closed_form(U, coeffs, 0.0)) > 1e-2


def test_polar_factor_limit():
    # cubic and quintic Newton-Schulz converge to the polar factor P Q^T
    rng = np.random.default_rng(11)
    P, _ = np.linalg.qr(rng.standard_normal((4, 4)))
    Q, _ = np.linalg.qr(rng.standard_normal((6, 4)))
    U = P @ np.diag([4.0, 3.0, 2.0, 1.0]) @ Q.T        # condition number 4
    polar = P @ Q.T
    assert np.linalg.norm(orc.orthogonalize(U, _table("cubic", 12)) - polar) < 1e-12
    assert np.linalg.norm(orc.orthogonalize(U, _table("quintic", 8)) - polar) < 1e-12
    assert np.linalg.norm(orc.orthogonalize(U.T, _table("quintic", 8)) - polar.T) < 1e-12


@pytest.mark.parametrize("kind", ["cubic", "quintic"])
def test_singular_values_move_toward_one(kind):
    for k in (1, 5, 6):
        coeffs = _table(kind, k)
        for x in np.linspace(1e-4, 1.0, 2001):
            assert abs(orc.ns_poly_scalar(x, coeffs) - 1) <= abs(x - 1) + 1e-15
    G = gen.grad_matrix(64, 96, 0, 0, 1)
    s_in = orc.singular_values(G) / (np.linalg.norm(G) + 1e-7)
    s_out = orc.singular_values(orc.orthogonalize(G, _table(kind, 5)))
    assert np.all(np.abs(s_out - 1) <= np.abs(s_in - 1) + 1e-12)


def test_rank_deficient_keeps_zero_singular_values():
    rng = np.random.default_rng(2)
    U = rng.standard_normal((8, 3)) @ rng.standard_normal((3, 12))
    s = orc.singular_values(orc.orthogonalize(U, _table("quintic", 6)))
    assert np.all(s[3:] < 1e-12) and np.all(s[:3] > 0.1)


# ------------------------------------------------------------------ invariances
def test_transpose_invariance_exact():
    U = gen.grad_matrix(20, 36, 0, 0, 2)
    c = _table("quintic", 5)
    np.testing.assert_array_equal(orc.orthogonalize(U.T, c), orc.orthogonalize(U, c).T)


def test_scale_invariance():
    U = gen.grad_matrix(20, 36, 0, 0, 3)
    c = _table("quintic", 5)
    a = orc.orthogonalize(U, c, eps=0.0)
    b = orc.orthogonalize(U * 37.5, c, eps=0.0)
    assert orc.rel_fro(b, a) < 1e-13


def test_orthogonal_equivariance():
    rng = np.random.default_rng(9)
    U = rng.standard_normal((10, 14))
    Q1, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    Q2, _ = np.linalg.qr(rng.standard_normal((14, 14)))
    c = _table("odd", 4)
    lhs = orc.orthogonalize(Q1 @ U @ Q2, c)
    rhs = Q1 @ orc.orthogonalize(U, c) @ Q2
    assert orc.rel_fro(lhs, rhs) < 1e-12


def test_diagonal_input_gives_scalar_map():
    d = np.array([3.0, -2.0, 0.5, 1e-3])
    U = np.zeros((4, 7))
    U[np.arange(4), np.arange(4)] = d
    c = _table("quintic", 5)
    O = orc.orthogonalize(U, c, eps=0.0)
    want = np.zeros_like(U)
    want[np.arange(4), np.arange(4)] = [orc.ns_poly_scalar(v, c) for v in d / np.linalg.norm(d)]
    np.testing.assert_allclose(O, want, rtol=1e-13, atol=1e-15)


def test_rank_one():
    rng = np.random.default_rng(4)
    u, v = rng.standard_normal(9), rng.standard_normal(5)
    c = _table("cubic", 5)
    O = orc.orthogonalize(np.outer(u, v), c, eps=1e-7)
    sig = np.linalg.norm(u) * np.linalg.norm(v)
    want = orc.ns_poly_scalar(sig / (sig + 1e-7), c) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    np.testing.assert_allclose(O, want, rtol=1e-12, atol=1e-15)


def test_one_by_one_brute_force():
    for g in (2.5, -0.75):
        c = _table("quintic", 6)
        want = orc.ns_poly_scalar(g / (abs(g) + 1e-7), c)
        assert abs(orc.orthogonalize(np.array([[g]]), c)[0, 0] - want) < 1e-15


# ------------------------------------------------------------------ golden files
def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = [float(t) for t in v.split()]
    return vals


def test_golden_hand_worked_2x3():
    g = _read_golden("ns_hand_2x3.txt")
    U = np.array(g["U"]).reshape(2, 3)
    for kind in ("cubic", "quintic"):
        O = orc.orthogonalize(U, np.array([g["coeffs_" + kind]]), eps=0.0)
        np.testing.assert_allclose(O.ravel(), g["O_" + kind], rtol=0, atol=1e-15)
        O = orc.orthogonalize(U.T, np.array([g["coeffs_" + kind]]), eps=0.0)
        np.testing.assert_allclose(O.T.ravel(), g["O_" + kind], rtol=0, atol=1e-15)


def test_golden_hand_worked_state():
    g = _read_golden("state_hand.txt")
    m = orc.momentum_f32(np.array(g["m0"], np.float32), np.array(g["g"], np.float32), g["beta"][0])
    np.testing.assert_array_equal(m, np.array(g["m1"], np.float32))
    W = np.array(g["W"])
    S = np.array(g["S"])
    np.testing.assert_array_equal(orc.cautious_mask(W, S), np.array(g["mask"]) > 0)
    u = orc.nesterov_f32(m, np.array(g["g"], np.float32), g["beta"][0])
    np.testing.assert_array_equal(u, np.array(g["nesterov_u"], np.float32))
    args = (np.array(g["w0"]), np.array(g["o"]), g["lr"][0], g["wd"][0], np.array(g["upd_mask"]) > 0)
    np.testing.assert_array_equal(orc.update_f32(*args), np.array(g["w1"], np.float32))
    np.testing.assert_array_equal(orc.update_f64(*args), np.array(g["w1"]))


# ------------------------------------------------------------ fp32 state order
def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def test_fp32_operation_order_matches_scalar_emulation():
    # fl(fl(b*m) + fl((1-b)*g)) with every operation rounded to fp32
    rng = np.random.default_rng(7)
    m = (rng.standard_normal(4000) * 1e-3).astype(np.float32)
    g = (rng.standard_normal(4000) * 1e-2).astype(np.float32)
    for beta in (0.95, 0.9, 0.99):
        b = _f32(beta)
        ob = _f32(1.0 - b)
        want = np.array([_f32(_f32(b * float(mi)) + _f32(ob * float(gi))) for mi, gi in zip(m, g)],
                        dtype=np.float32)
        np.testing.assert_array_equal(orc.momentum_f32(m, g, beta), want)
    # and it differs from a fused multiply-add somewhere on this data
    fused = np.array([_f32(_f32(b * float(mi)) + ob * float(gi)) for mi, gi in zip(m, g)], np.float32)
    assert np.any(fused != orc.momentum_f32(m, g, 0.99))


def test_update_f32_matches_scalar_emulation():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal(500) * 0.02).astype(np.float32)
    o = (rng.standard_normal(500) * 0.03).astype(np.float32)
    mk = rng.random(500) < 0.5
    lr, wd = 0.02, 0.1
    d1 = _f32(_f32(lr) * _f32(wd))
    want = []
    for wi, oi, mi in zip(w, o, mk):
        d = d1 if mi else 0.0
        t = _f32(float(wi) - _f32(d * float(wi)))
        want.append(_f32(t - _f32(_f32(lr) * float(oi))))
    np.testing.assert_array_equal(orc.update_f32(w, o, lr, wd, mk), np.array(want, np.float32))


def test_update_f32_within_fp32_rounding_of_the_exact_update():
    # every operation of the fp32 order rounds once (relative 2^-24), so the
    # result lies within a few fp32 units of the operands' scale of the exact
    # value; a dropped or mis-scaled term would be off by lr*wd*|w| or lr*|o|
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(4000) * 0.02).astype(np.float32)
    o = (rng.standard_normal(4000) * 0.03).astype(np.float32)
    mk = rng.random(4000) < 0.5
    for lr, wd in ((0.02, 0.1), (0.02, 1.6), (0.003, 0.0)):
        lr32, wd32 = _f32(lr), _f32(wd)
        exact = orc.update_f64(w, o, lr32, wd32, mk)
        got = orc.update_f32(w, o, lr32, wd32, mk).astype(np.float64)
        scale = np.abs(w) + lr32 * wd32 * np.abs(w) + lr32 * np.abs(o)
        assert np.all(np.abs(got - exact) <= 4 * 2.0 ** -24 * scale)
        assert np.max(np.abs(got - exact) / scale) > 0      # the fp32 order does round


def test_nesterov_constant_gradient_closed_form():
    # with M_0 = 0 and a constant gradient, M_t = (1 - beta^t) G, so the
    # look-ahead beta M_t + (1 - beta) G is (1 - beta^(t+1)) G
    G = (np.random.default_rng(4).standard_normal((5, 6))).astype(np.float32)
    M = np.zeros_like(G)
    beta = 0.95
    for t in range(1, 41):
        M = orc.momentum_f32(M, G, beta)
        U = orc.nesterov_f32(M, G, beta)
        np.testing.assert_allclose(U, (1 - beta ** (t + 1)) * G.astype(np.float64),
                                   rtol=2e-6 * (t + 1), atol=1e-7)


def test_nesterov_step_orthogonalises_the_look_ahead():
    # two steps with independent gradients: M_2 = beta (1-beta) G1 + (1-beta) G2,
    # and the step orthogonalises beta M_2 + (1-beta) G2
    #   = beta^2 (1-beta) G1 + (1 - beta^2) G2
    # (not M_2 itself, whose G1:G2 mix is beta : 1 instead of beta^2 : (1+beta))
    shape = (7, 11)
    G1 = gen.grad_matrix(*shape, 3, 1, 0).astype(np.float32).astype(np.float64)
    G2 = gen.grad_matrix(*shape, 3, 2, 0).astype(np.float32).astype(np.float64)
    beta, c = 0.8, _table("quintic", 5)
    for nesterov in (True, False):
        st = orc.OracleState([shape])
        W = [np.zeros(shape)]
        orc.muon_step(W, [G1], st, c, 0.02, 0.0, beta, param_dtype="f64", nesterov=nesterov)
        out = orc.muon_step(W, [G2], st, c, 0.02, 0.0, beta, param_dtype="f64", nesterov=nesterov)
        U = (beta ** 2 * (1 - beta) * G1 + (1 - beta ** 2) * G2 if nesterov
             else beta * (1 - beta) * G1 + (1 - beta) * G2)
        other = (beta * (1 - beta) * G1 + (1 - beta) * G2 if nesterov
                 else beta ** 2 * (1 - beta) * G1 + (1 - beta ** 2) * G2)
        want = _closed_form(U, c, 1e-7)
        # fp32 state rounding of M and U: relative ~1e-7
        assert orc.rel_fro(out["O"][0], want) < 1e-5
        assert orc.rel_fro(out["O"][0], _closed_form(other, c, 1e-7)) > 1e-2


# -------------------------------------------------- recurrence closed forms
def test_momentum_constant_gradient_closed_form():
    G = (np.random.default_rng(3).standard_normal((5, 6))).astype(np.float32)
    M = np.zeros_like(G)
    beta = 0.95
    for t in range(1, 41):
        M = orc.momentum_f32(M, G, beta)
        np.testing.assert_allclose(M, (1 - beta ** t) * G.astype(np.float64), rtol=2e-6 * t, atol=1e-7)


def test_ema_closed_form():
    rng = np.random.default_rng(6)
    Ws = [rng.standard_normal((3, 4)).astype(np.float32) for _ in range(12)]
    beta = 0.9
    E = Ws[0].copy()                   # set to W at the first averaged step
    for W in Ws[1:]:
        E = orc.ema_f32(E, W, beta)
    T = len(Ws) - 1
    want = beta ** T * Ws[0].astype(np.float64)
    for t in range(1, T + 1):
        want = want + (1 - beta) * beta ** (T - t) * Ws[t].astype(np.float64)
    np.testing.assert_allclose(E, want, rtol=1e-5, atol=1e-6)


def test_blend_is_the_stated_mix():
    W = np.array([1.0, -2.0, 0.5], np.float32)
    E = np.array([0.0, 2.0, 0.25], np.float32)
    np.testing.assert_allclose(orc.blend_f32(W, E, 0.35), 0.35 * W + 0.65 * E, rtol=1e-6)


# ---------------------------------------------------- whole-step special cases
def test_zero_gradient_gives_pure_decay():
    shapes = [(6, 9), (9, 6)]
    st = orc.OracleState(shapes)
    W0 = [np.random.default_rng(i).standard_normal(s) for i, s in enumerate(shapes)]
    W = [w.copy() for w in W0]
    lr, wd = 0.02, 1.6
    for t in range(1, 6):
        out = orc.muon_step(W, [np.zeros(s) for s in shapes], st, _table("quintic", 5),
                            lr, wd, 0.95, param_dtype="f64")
        W = out["params"]
        assert all(np.all(o == 0) for o in out["O"])
        for w, w0 in zip(W, W0):
            np.testing.assert_allclose(w, (1 - lr * wd) ** t * w0, rtol=1e-13)
    assert st.step == 5


def test_cautious_with_zero_slow_momentum_never_decays():
    shapes = [(5, 7)]
    st = orc.OracleState(shapes, beta_slow=0.99)
    W = [np.random.default_rng(0).standard_normal(shapes[0])]
    out = orc.muon_step(W, [np.zeros(shapes[0])], st, _table("quintic", 6), 0.02, 0.1, 0.9,
                        param_dtype="f64", cautious=True)
    np.testing.assert_array_equal(out["params"][0], W[0])
    assert not out["mask"][0].any()


def test_cautious_decay_only_where_signs_agree():
    shapes = [(4, 4)]
    st = orc.OracleState(shapes, beta_slow=0.5)
    W = [np.array([[1.0, -1.0, 1.0, -1.0]] * 4)]
    G = np.array([[1.0, -1.0, -1.0, 1.0]] * 4)
    st.mom[0] = np.zeros((4, 4), np.float32)
    # tiny lr on the orthogonalised part isolates the decay: use steps with c such
    # that O = 0 is not possible; instead compare with lr*O removed explicitly
    out = orc.muon_step(W, [G], st, _table("quintic", 1), 0.01, 0.5, 0.9,
                        param_dtype="f64", cautious=True)
    mask = out["mask"][0]
    np.testing.assert_array_equal(mask, np.array([[True, True, False, False]] * 4))
    decay_part = out["params"][0] + 0.01 * out["O"][0] - W[0]
    np.testing.assert_allclose(decay_part, -0.01 * 0.5 * W[0] * mask, atol=1e-15)


def test_steps_zero_is_normalised_momentum():
    G = gen.grad_matrix(7, 11, 0, 0, 0)
    st = orc.OracleState([G.shape])
    W = [np.zeros(G.shape)]
    out = orc.muon_step(W, [G.astype(np.float32)], st, np.zeros((0, 3)), 0.02, 0.0, 0.9,
                        param_dtype="f64")
    M = (np.float32(1) - np.float32(0.9)) * G.astype(np.float32)
    U = M.astype(np.float64)
    np.testing.assert_allclose(out["params"][0], -0.02 * U / (np.linalg.norm(U) + 1e-7), rtol=1e-14)


def test_nan_is_confined_to_its_matrix():
    shapes = [(4, 6), (6, 4)]
    st = orc.OracleState(shapes)
    G = [gen.grad_matrix(4, 6, 0, 0, 0), gen.grad_matrix(6, 4, 0, 0, 1)]
    G[0][1, 2] = np.nan
    out = orc.muon_step([np.zeros(s) for s in shapes], G, st, _table("quintic", 5), 0.02, 0.0,
                        0.95, param_dtype="f64")
    assert np.isnan(out["params"][0]).all()
    assert np.isfinite(out["params"][1]).all()


def test_ema_counters():
    shapes = [(3, 5)]
    st = orc.OracleState(shapes, beta_ema=0.9, ema_start=3)
    W = [np.random.default_rng(1).standard_normal(shapes[0])]
    for t in range(1, 6):
        out = orc.muon_step(W, [gen.grad_matrix(3, 5, 0, t, 0)], st, _table("cubic", 2),
                            0.02, 0.0, 0.95, param_dtype="f64")
        if t == 3:
            np.testing.assert_array_equal(st.ema[0], out["params"][0].astype(np.float32))
        W = out["params"]
        assert st.step == t and st.ema_count == max(0, t - 2)


def test_mask_uses_slow_not_fast_momentum():
    # Two steps, G2 = -0.7 G1: the fast momentum (beta 0.5) flips sign, the
    # slow one (beta 0.99) does not, so the mask follows the slow momentum.
    shapes = [(3, 4)]
    st = orc.OracleState(shapes, beta_slow=0.99)
    G1 = np.abs(gen.grad_matrix(3, 4, 0, 0, 0)) + 0.1
    W = [np.ones(shapes[0])]
    c = _table("quintic", 1)
    out = orc.muon_step(W, [G1], st, c, 0.01, 0.1, 0.5, param_dtype="f64", cautious=True)
    out = orc.muon_step(out["params"], [-0.7 * G1], st, c, 0.01, 0.1, 0.5, param_dtype="f64",
                        cautious=True)
    assert np.all(st.mom[0] < 0) and np.all(st.slow[0] > 0)
    assert out["mask"][0].all()


# ---------------------------------------------------------------- weighted averages
def _averaged(ws, weights):
    """Run the oracle's running-mean recurrence over a sequence of fp32 arrays."""
    e, s = None, 0.0
    for w, wt in zip(ws, weights):
        if e is None:
            e, s = np.asarray(w, np.float32).copy(), float(wt)
            continue
        b, ob = orc.running_mean_coeffs(s, wt)
        e = orc.average_f32(e, w, b, ob)
        s += wt
    return e


def test_equal_weights_give_the_arithmetic_mean():
    """Stochastic weight averaging: the running form must reproduce the plain
    mean of the averaged weights (up to fp32 rounding per step)."""
    rng = np.random.default_rng(21)
    ws = [rng.normal(0, 0.02, 500).astype(np.float32) for _ in range(9)]
    e = _averaged(ws, [1.0] * 9)
    ref = np.mean(np.array(ws, dtype=np.float64), axis=0)
    np.testing.assert_allclose(e, ref, rtol=0, atol=9 * 2.0 ** -23 * 0.1)


def test_weights_give_the_weighted_mean():
    rng = np.random.default_rng(22)
    wts = [0.5, 2.0, 1.0, 3.0, 0.25, 4.0]
    ws = [rng.normal(0, 1, 300).astype(np.float32) for _ in wts]
    e = _averaged(ws, wts)
    ref = np.tensordot(np.array(wts), np.array(ws, dtype=np.float64), axes=1) / sum(wts)
    np.testing.assert_allclose(e, ref, rtol=0, atol=len(wts) * 2.0 ** -22 * 4)
    # a weighted mean differs from the plain mean here: the weights matter
    assert np.max(np.abs(ref - np.mean(np.array(ws, np.float64), axis=0))) > 0.1


def test_zero_weight_leaves_the_average_unchanged():
    rng = np.random.default_rng(23)
    a, b = (rng.normal(0, 1, 64).astype(np.float32) for _ in range(2))
    e = _averaged([a, b], [1.0, 0.0])
    np.testing.assert_array_equal(e, a)


def test_oracle_step_wires_the_weighted_average():
    """Through muon_step: with steps whose parameters are known, the state's
    average equals the weighted mean of the stored parameters."""
    rng = np.random.default_rng(24)
    shape = (16, 24)
    st = orc.OracleState([shape], beta_ema=0.0, ema_start=2, avg_mode="weighted")
    W = orc.store(rng.normal(0, 0.02, shape), "bf16")
    coeffs = np.repeat(np.array([gen.QUINTIC]), 5, axis=0)
    hist, wts = [], [0.0, 1.0, 3.0, 0.5]   # the first step is outside the window
    for t, wt in enumerate(wts):
        G = rng.normal(0, 1e-3, shape).astype(np.float32)
        W = orc.muon_step([W], [G], st, coeffs, 0.02, 0.1, 0.9, avg_weight=wt)["params"][0]
        if t >= 1:
            hist.append(W)
    ref = np.tensordot(np.array(wts[1:]), np.array(hist), axes=1) / sum(wts[1:])
    np.testing.assert_allclose(st.ema[0], ref, rtol=0, atol=4 * 2.0 ** -23 * 0.1)
    assert st.ema_count == 3 and st.avg_sum == sum(wts[1:])
