"""Host-only checks of the C ABI: the library loads, exports every function
declared in include/muon.h, agrees with the header on struct layout, and
rejects bad arguments before touching the GPU (no kernel is launched here)."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from orthogonalising_matrix_optimizer_amd import _lib
from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from orthogonalising_matrix_optimizer_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_\w+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert "muon_step" in names and "muon_orthogonalize" in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (muon_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_c_compiler():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "muon.h"
#define O(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("muon_mat %zu\nmuon_options %zu\nmuon_state %zu\n", sizeof(muon_mat),
         sizeof(muon_options), sizeof(muon_state));
  O(muon_mat, ptr); O(muon_mat, rows); O(muon_mat, cols); O(muon_mat, ld); O(muon_mat, dtype);
  O(muon_options, beta_slow); O(muon_options, beta_ema); O(muon_options, eps);
  O(muon_options, nesterov); O(muon_options, ema_start); O(muon_options, cautious);
  O(muon_options, ns_dtype); O(muon_options, avg_mode);
  O(muon_state, n); O(muon_state, mom); O(muon_state, mom_slow); O(muon_state, ema);
  O(muon_state, mask_out); O(muon_state, update_out); O(muon_state, workspace);
  O(muon_state, workspace_bytes); O(muon_state, step); O(muon_state, ema_count);
  O(muon_state, opt); O(muon_state, avg_weight); O(muon_state, avg_weight_sum);
  printf("muon_vec %zu\nmuon_adamw_hparams %zu\nmuon_adamw_state %zu\n", sizeof(muon_vec),
         sizeof(muon_adamw_hparams), sizeof(muon_adamw_state));
  O(muon_vec, ptr); O(muon_vec, numel); O(muon_vec, dtype);
  O(muon_adamw_hparams, lr); O(muon_adamw_hparams, beta1); O(muon_adamw_hparams, beta2);
  O(muon_adamw_hparams, eps); O(muon_adamw_hparams, wd);
  O(muon_adamw_state, n); O(muon_adamw_state, m); O(muon_adamw_state, v);
  O(muon_adamw_state, workspace); O(muon_adamw_state, workspace_bytes);
  O(muon_adamw_state, step);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.split() for l in lines if l.strip())
    ct = {"muon_mat": _lib.MuonMat, "muon_options": _lib.MuonOptions, "muon_state": _lib.MuonState,
          "muon_vec": _lib.MuonVec, "muon_adamw_hparams": _lib.AdamWHparams,
          "muon_adamw_state": _lib.AdamWState}
    for k, v in got.items():
        if "." in k:
            s, f = k.split(".")
            assert getattr(ct[s], f).offset == int(v), k
        else:
            assert ctypes.sizeof(ct[k]) == int(v), k


def test_status_strings(lib):
    for code in _lib.STATUS:
        assert lib.muon_status_str(code)
    assert lib.muon_status_str(0) == b"ok"


# ---------------------------------------------------------------- validation
BASE = 0x7f0000000000   # fake device addresses: validation fails before any use


def _setup(lib, shapes, dtype=_lib.MUON_BF16, ws_bytes=None, **opt_kw):
    n = len(shapes)
    addr = [BASE]

    def take(nbytes):
        a = addr[0]
        addr[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return a

    es = 2 if dtype == _lib.MUON_BF16 else 4
    params = _lib.mat_array((take(r * c * es), r, c, c, dtype) for r, c in shapes)
    grads = _lib.mat_array((take(r * c * es), r, c, c, dtype) for r, c in shapes)
    mom = _lib.ptr_array(take(r * c * 4) for r, c in shapes)
    opt = _lib.default_options()
    for k, v in opt_kw.items():
        setattr(opt, k, v)
    need = lib.muon_workspace_bytes(params, n, opt, 5)
    st = _lib.MuonState()
    st.n = n
    st.mom = ctypes.cast(mom, ctypes.POINTER(ctypes.c_void_p))
    st.workspace = take(need)
    st.workspace_bytes = need if ws_bytes is None else ws_bytes
    st.opt = opt
    keep = [params, grads, mom]
    return params, grads, st, keep


def _coeffs(k=5):
    return _lib.float_array(np.array([gen.QUINTIC] * k).ravel())


def _step(lib, params, grads, st, coeffs=None, steps=5, lr=0.02, wd=0.0, beta=0.95):
    return lib.muon_step(params, grads, st if st is not None else None,
                         coeffs if coeffs is not None else _coeffs(steps), steps, lr, wd, beta,
                         None)


E = _lib.CODES


def test_rejects_bad_scalars(lib):
    p, g, st, keep = _setup(lib, [(8, 16), (16, 8)])
    assert lib.muon_step(p, g, None, _coeffs(), 5, 0.02, 0.0, 0.95, None) == E["MUON_E_NULL"]
    assert _step(lib, p, g, st, steps=17, coeffs=_coeffs(17)) == E["MUON_E_COEFFS"]
    assert lib.muon_step(p, g, st, _coeffs(), -1, 0.02, 0.0, 0.95, None) == E["MUON_E_COEFFS"]
    bad = _lib.float_array([1.0, float("nan"), 0.0] * 5)
    assert _step(lib, p, g, st, coeffs=bad) == E["MUON_E_COEFFS"]
    assert lib.muon_step(p, g, st, None, 5, 0.02, 0.0, 0.95, None) == E["MUON_E_NULL"]
    assert _step(lib, p, g, st, lr=float("inf")) == E["MUON_E_HPARAM"]
    assert _step(lib, p, g, st, wd=float("nan")) == E["MUON_E_HPARAM"]
    assert _step(lib, p, g, st, beta=1.0) == E["MUON_E_HPARAM"]
    assert _step(lib, p, g, st, beta=-0.1) == E["MUON_E_HPARAM"]
    assert st.step == 0 and st.ema_count == 0


def test_rejects_bad_options(lib):
    p, g, st, keep = _setup(lib, [(8, 16)])
    for field, val, code in [("eps", float("nan"), "MUON_E_HPARAM"), ("eps", -1.0, "MUON_E_HPARAM"),
                             ("ns_dtype", 7, "MUON_E_DTYPE"), ("beta_slow", 1.0, "MUON_E_HPARAM"),
                             ("beta_ema", 2.0, "MUON_E_HPARAM"), ("cautious", 1, "MUON_E_HPARAM"),
                             ("nesterov", 3, "MUON_E_HPARAM")]:
        o = _lib.default_options()
        setattr(o, field, val)
        st.opt = o
        assert _step(lib, p, g, st) == E[code], field
    assert st.step == 0


def test_rejects_bad_matrices(lib):
    p, g, st, keep = _setup(lib, [(8, 16), (16, 8)])
    good = (p[1].ptr, p[1].rows, p[1].cols, p[1].ld, p[1].dtype)
    for (r, c, ld, dt, code) in [(0, 8, 8, 0, "MUON_E_SHAPE"), (16, 8, 4, 0, "MUON_E_SHAPE"),
                                 (16, 8, 8, 5, "MUON_E_DTYPE")]:
        p[1] = _lib.MuonMat(good[0], r, c, ld, dt, 0)
        assert _step(lib, p, g, st) == E[code]
    p[1] = _lib.MuonMat(good[0] + 1, 16, 8, 8, _lib.MUON_BF16, 0)
    assert _step(lib, p, g, st) == E["MUON_E_ALIGN"]
    p[1] = _lib.MuonMat(None, 16, 8, 8, _lib.MUON_BF16, 0)
    assert _step(lib, p, g, st) == E["MUON_E_NULL"]
    p[1] = _lib.MuonMat(*good, 0)
    g[1] = _lib.MuonMat(g[1].ptr, 8, 16, 16, _lib.MUON_BF16, 0)
    assert _step(lib, p, g, st) == E["MUON_E_SHAPE"]
    assert st.step == 0


def test_rejects_missing_state(lib):
    p, g, st, keep = _setup(lib, [(8, 16)], beta_slow=0.99)
    assert _step(lib, p, g, st) == E["MUON_E_STATE"]        # slow momentum missing
    p, g, st, keep = _setup(lib, [(8, 16)], beta_ema=0.99)
    assert _step(lib, p, g, st) == E["MUON_E_STATE"]        # average missing
    p, g, st, keep = _setup(lib, [(8, 16)])
    st.mom = None
    assert _step(lib, p, g, st) == E["MUON_E_NULL"]


def test_step_prepare_validates_like_step(lib):
    """muon_step_prepare runs muon_step's validation (errors before any HIP
    call) and never touches the counters."""
    p, g, st, keep = _setup(lib, [(8, 16), (16, 8)])
    need = st.workspace_bytes
    st.workspace_bytes = need - 1
    assert lib.muon_step_prepare(p, g, st, None) == E["MUON_E_WORKSPACE"]
    st.workspace_bytes = need
    g0 = g[0]
    g[0] = _lib.MuonMat(p[0].ptr + 64, g0.rows, g0.cols, g0.ld, g0.dtype, 0)
    assert lib.muon_step_prepare(p, g, st, None) == E["MUON_E_ALIAS"]
    g[0] = g0
    p2, g2, st2, keep2 = _setup(lib, [(8, 16)], beta_slow=0.99)
    assert lib.muon_step_prepare(p2, g2, st2, None) == E["MUON_E_STATE"]
    st.n = 0
    assert lib.muon_step_prepare(p, g, st, None) == 0
    assert st.step == 0 and st.ema_count == 0
    assert lib.muon_step_prepare(p, g, None, None) == E["MUON_E_NULL"]


def test_rejects_workspace_and_aliasing(lib):
    p, g, st, keep = _setup(lib, [(8, 16), (16, 8)])
    need = st.workspace_bytes
    st.workspace_bytes = need - 1
    assert _step(lib, p, g, st) == E["MUON_E_WORKSPACE"]
    st.workspace_bytes = need
    ws = st.workspace
    st.workspace = None
    assert _step(lib, p, g, st) == E["MUON_E_WORKSPACE"]
    st.workspace = ws + 16
    assert _step(lib, p, g, st) == E["MUON_E_ALIGN"]
    st.workspace = ws
    g0 = g[0]
    g[0] = _lib.MuonMat(p[0].ptr + 64, g0.rows, g0.cols, g0.ld, g0.dtype, 0)   # overlaps params[0]
    assert _step(lib, p, g, st) == E["MUON_E_ALIAS"]
    g[0] = g0
    st.mom[1] = p[1].ptr                                                      # momentum over params
    assert _step(lib, p, g, st) == E["MUON_E_ALIAS"]
    st.mom[1] = ws + 1024                                                     # momentum in workspace
    assert _step(lib, p, g, st) == E["MUON_E_ALIAS"]
    assert st.step == 0 and st.ema_count == 0


def test_empty_step_only_advances_counters(lib):
    st = _lib.MuonState()
    st.n = 0
    st.opt = _lib.default_options()
    st.opt.beta_ema = 0.9
    st.opt.ema_start = 2
    for t in range(1, 4):
        assert lib.muon_step(None, None, st, _coeffs(), 5, 0.02, 0.0, 0.95, None) == 0
        assert st.step == t and st.ema_count == max(0, t - 1)


def test_orthogonalize_and_blend_validation(lib):
    p, g, st, keep = _setup(lib, [(8, 16), (16, 8)])
    opt = _lib.default_options()
    need = lib.muon_workspace_bytes(p, 2, opt, 5)
    assert lib.muon_orthogonalize(p, g, 2, _coeffs(), 5, opt, st.workspace, need - 256, None) == \
        E["MUON_E_WORKSPACE"]
    g[1] = _lib.MuonMat(g[1].ptr, 8, 16, 16, _lib.MUON_BF16, 0)
    assert lib.muon_orthogonalize(p, g, 2, _coeffs(), 5, opt, st.workspace, need, None) == \
        E["MUON_E_SHAPE"]
    assert lib.muon_orthogonalize(p, p, 1, _coeffs(), 5, opt, st.workspace, need, None) == \
        E["MUON_E_ALIAS"]
    assert lib.muon_orthogonalize(p, g, 0, _coeffs(), 5, opt, st.workspace, need, None) == 0
    assert lib.muon_ema_blend(p, p, st, 0.35, None) == E["MUON_E_STATE"]
    assert lib.muon_ema_blend(p, p, st, 1.5, None) == E["MUON_E_HPARAM"]
    assert lib.muon_probe_arm(9, 4) == E["MUON_E_HPARAM"]
    assert lib.muon_probe_arm(8, 4) == E["MUON_E_HPARAM"]
    # phase 6 (the APPLY launch that carries the update) is a phase; arming it
    # creates HIP events, which fails without a GPU
    assert lib.muon_probe_arm(6, 4) != E["MUON_E_HPARAM"]
    lib.muon_probe_disarm()
    assert lib.muon_probe_arm(1, 0) == E["MUON_E_HPARAM"]


# ---------------------------------------------------------------- planning
def _plan(lib, shapes, steps=5, coeffs=None, ns=_lib.MUON_BF16, cautious=0, beta_ema=-1.0,
          pdt=_lib.MUON_BF16):
    mats = _lib.mat_array((0, r, c, c, pdt) for r, c in shapes)
    opt = _lib.default_options()
    opt.ns_dtype = ns
    opt.cautious = cautious
    opt.beta_ema = beta_ema
    ng, lps = ctypes.c_int32(), ctypes.c_int32()
    tiles = (ctypes.c_int32 * 16)()
    c = _lib.float_array(np.array(coeffs if coeffs is not None else [gen.QUINTIC] * steps).ravel())
    assert lib.muon_plan_info(mats, len(shapes), opt, steps, c, ctypes.byref(ng), tiles, 16,
                              ctypes.byref(lps)) == 0
    return ng.value, tiles[0], lps.value, lib.muon_workspace_bytes(mats, len(shapes), opt, steps)


def test_plan_groups_and_launches(lib):
    shapes = gen.gpt124m_shapes()
    ng, ts, lps, ws = _plan(lib, shapes)
    assert ng == 2 and ts == 256
    # prepare, 5 x (gram, poly, apply); the plain update of bf16 matrices with
    # shapes in multiples of 8 runs in the last APPLY launch
    assert lps == 1 + 5 * 3
    assert _plan(lib, shapes, coeffs=[gen.CUBIC] * 5)[2] == 1 + 5 * 2
    # a separate finish launch: cautious decay, the average, fp32 parameters, a
    # shape that is not a multiple of 8
    assert _plan(lib, shapes, cautious=1)[2] == 2 + 5 * 3
    assert _plan(lib, shapes, beta_ema=0.99)[2] == 2 + 5 * 3
    assert _plan(lib, shapes, pdt=_lib.MUON_F32)[2] == 2 + 5 * 3
    assert _plan(lib, shapes + [(200, 333)])[2] == 2 + 5 * 3
    # iterate ping-pong + Gram + polynomial buffers for 48 (768,768) and 24 (768,3072)
    floor = 2 * (48 * (2 * 768 * 768 + 2 * 768 * 768) + 24 * (2 * 768 * 3072 + 2 * 768 * 768))
    assert floor <= ws <= floor * 1.01
    assert ws % 256 == 0
    ng, ts, lps, ws32 = _plan(lib, [(256, 512)], ns=_lib.MUON_F32)
    assert ng == 1 and ts == 64            # one small matrix: smallest tiles
    assert lps == 2 + 5 * 3                # fp32 operands: one launch per product
    assert ws32 >= 4 * (2 * 256 * 512 + 2 * 256 * 256)
    assert _plan(lib, gen.moe_share_shapes())[0] == 2
    assert _plan(lib, [(5, 3), (3, 5), (7, 7)])[0] == 2


def test_small_problems_can_run_the_iterations_in_one_launch(lib, monkeypatch):
    # default: one launch per product
    ng, ts, lps, _ = _plan(lib, [(256, 512)])
    assert ts == 64 and lps == 2 + 5 * 3
    assert _plan(lib, [(256, 512)], coeffs=[gen.CUBIC] * 5)[2] == 2 + 5 * 2
    # on request (read at every call), 64-wide tiles with bf16 operands:
    # prepare, one launch for all products, finish (the plain update needs
    # 256-wide tiles to run in an epilogue)
    monkeypatch.setenv("MUON_NS_SINGLE_LAUNCH", "1")
    assert _plan(lib, [(256, 512)])[2] == 3
    assert _plan(lib, [(256, 512)], coeffs=[gen.CUBIC] * 5)[2] == 3
    assert _plan(lib, [(256, 512)], steps=16)[2] == 3
    assert _plan(lib, [(256, 512)], ns=_lib.MUON_F32)[2] == 2 + 5 * 3
    # more than 1024 tiles in a product: separate launches
    monkeypatch.setenv("MUON_TILE", "64")
    many = [(512, 512)] * 40                # 40 x 36 = 1440 GRAM tiles of 64
    assert _plan(lib, many)[1] == 64
    assert _plan(lib, many)[2] == 2 + 5 * 3


def test_workspace_bytes_rejects_bad_shapes(lib):
    mats = _lib.mat_array([(0, 0, 5, 5, 0)])
    assert lib.muon_workspace_bytes(mats, 1, None, 5) == 0
    assert lib.muon_workspace_bytes(None, -1, None, 5) == 0


# ---------------------------------------------------------------- AdamW
def _adamw_case(n_elems=(10, 0, 4096)):
    """Fake device addresses (never dereferenced: every case below fails
    validation, or has n == 0)."""
    base = 1 << 40
    specs_p, specs_g, ms, vs = [], [], [], []
    off = 0
    for ne in n_elems:
        sz = max(ne, 1) * 4
        specs_p.append((base + off if ne else 0, ne, _lib.MUON_BF16)); off += 2 * sz + 256
        specs_g.append((base + off if ne else 0, ne, _lib.MUON_F32)); off += 2 * sz + 256
        ms.append(base + off if ne else 0); off += 2 * sz + 256
        vs.append(base + off if ne else 0); off += 2 * sz + 256
    return specs_p, specs_g, ms, vs, (base + off + 4096 + 255) // 256 * 256


def _adamw_call(lib, specs_p, specs_g, ms, vs, ws, ws_bytes=None, hp=None, n=None):
    P = _lib.vec_array(specs_p)
    G = _lib.vec_array(specs_g)
    mp, vp = _lib.ptr_array(ms), _lib.ptr_array(vs)
    st = _lib.AdamWState(len(specs_p) if n is None else n, 0,
                         ctypes.cast(mp, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(vp, ctypes.POINTER(ctypes.c_void_p)), ws,
                         lib.muon_adamw_workspace_bytes(len(specs_p)) if ws_bytes is None
                         else ws_bytes, 5)
    hp = hp or _lib.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0)
    code = lib.muon_adamw_step(P, G, st, hp, None)
    return code, st


def test_adamw_workspace_bytes(lib):
    assert lib.muon_adamw_workspace_bytes(-1) == 0
    assert lib.muon_adamw_workspace_bytes(0) > 0
    assert lib.muon_adamw_workspace_bytes(100) >= 100 * 48 + 101 * 8


def test_adamw_rejects_bad_arguments(lib):
    E = _lib.CODES
    p, g, m, v, ws = _adamw_case()
    HP = _lib.AdamWHparams
    for hp in [HP(float("nan"), 0.9, 0.999, 1e-8, 0, 0), HP(1e-3, 1.0, 0.999, 1e-8, 0, 0),
               HP(1e-3, 0.9, -0.1, 1e-8, 0, 0), HP(1e-3, 0.9, 0.999, -1e-8, 0, 0),
               HP(1e-3, 0.9, 0.999, 1e-8, float("inf"), 0)]:
        code, st = _adamw_call(lib, p, g, m, v, ws, hp=hp)
        assert code == E["MUON_E_HPARAM"] and st.step == 5
    bad = [list(x) for x in g]
    bad[2][1] = 4095                                            # numel mismatch
    assert _adamw_call(lib, p, [tuple(x) for x in bad], m, v, ws)[0] == E["MUON_E_SHAPE"]
    bad = [list(x) for x in p]
    bad[0][2] = 7                                               # unknown dtype
    assert _adamw_call(lib, [tuple(x) for x in bad], g, m, v, ws)[0] == E["MUON_E_DTYPE"]
    bad = [list(x) for x in p]
    bad[0][0] += 1                                              # odd bf16 address
    assert _adamw_call(lib, [tuple(x) for x in bad], g, m, v, ws)[0] == E["MUON_E_ALIGN"]
    mm = list(m)
    mm[2] = 0                                                   # missing moment buffer
    assert _adamw_call(lib, p, g, mm, v, ws)[0] == E["MUON_E_NULL"]
    vv = list(v)
    vv[0] = m[0]                                                # v aliases m
    assert _adamw_call(lib, p, g, m, vv, ws)[0] == E["MUON_E_ALIAS"]
    assert _adamw_call(lib, p, g, m, v, ws, ws_bytes=16)[0] == E["MUON_E_WORKSPACE"]
    assert _adamw_call(lib, p, g, m, v, 0)[0] == E["MUON_E_WORKSPACE"]
    assert _adamw_call(lib, p, g, m, v, ws + 64)[0] == E["MUON_E_ALIGN"]
    assert _adamw_call(lib, p, g, m, v, p[0][0])[0] == E["MUON_E_ALIAS"]


def test_adamw_empty_call_only_advances_the_counter(lib):
    st = _lib.AdamWState(0, 0, None, None, None, 0, 0)
    hp = _lib.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 0)
    for t in range(1, 4):
        assert lib.muon_adamw_step(None, None, st, hp, None) == 0
        assert st.step == t


def test_weighted_average_validation(lib):
    """Weights of the weighted running mean: negative, non-finite, or a zero
    first weight are rejected before any device work; with n == 0 the weight
    sum still advances with the average's step count."""
    E = _lib.CODES
    st = _lib.MuonState()
    st.n = 0
    st.opt = _lib.default_options()
    st.opt.beta_ema = 0.0
    st.opt.avg_mode = _lib.MUON_AVG_WEIGHTED
    for bad in (-1.0, float("nan"), float("inf"), 0.0):
        st.avg_weight = bad
        assert lib.muon_step(None, None, st, _coeffs(), 5, 0.02, 0.0, 0.95, None) == \
            E["MUON_E_HPARAM"]
        assert st.step == 0 and st.ema_count == 0
    for t, w in enumerate([2.0, 0.0, 0.5], start=1):
        st.avg_weight = w
        assert lib.muon_step(None, None, st, _coeffs(), 5, 0.02, 0.0, 0.95, None) == 0
        assert st.step == t and st.ema_count == t
    assert st.avg_weight_sum == 2.5
    st.opt.avg_mode = 7
    assert lib.muon_step(None, None, st, _coeffs(), 5, 0.02, 0.0, 0.95, None) == \
        E["MUON_E_HPARAM"]


def test_rejects_matrices_beyond_32_bit_offsets(lib):
    """The GEMMs address one matrix's padded iterate with 32-bit offsets: a
    bf16 60000 x 60000 matrix (about 7.2 GB padded) is rejected, one of
    30000 x 60000 (3.6 GB) is planned."""
    big = _lib.mat_array([(0, 60000, 60000, 60000, _lib.MUON_BF16)])
    ok = _lib.mat_array([(0, 30000, 60000, 60000, _lib.MUON_BF16)])
    opt = _lib.default_options()
    assert lib.muon_workspace_bytes(big, 1, opt, 5) == 0
    assert lib.muon_workspace_bytes(ok, 1, opt, 5) > 3 * 2 ** 30
    opt.ns_dtype = _lib.MUON_F32
    assert lib.muon_workspace_bytes(ok, 1, opt, 5) == 0


def _layout(lib, shapes, ns=_lib.MUON_BF16):
    mats = _lib.mat_array((0, r, c, c, _lib.MUON_BF16) for r, c in shapes)
    opt = _lib.default_options()
    opt.ns_dtype = ns
    vals = [ctypes.c_size_t() for _ in range(4)]
    assert lib.muon_workspace_layout(mats, len(shapes), opt, *[ctypes.byref(v) for v in vals]) == 0
    return [v.value for v in vals] + [lib.muon_workspace_bytes(mats, len(shapes), opt, 5)]


@pytest.mark.parametrize("shapes", [gen.gpt124m_shapes(), [(256, 512)], [(5, 3), (3, 5), (7, 7)],
                                    gen.moe_share_shapes()])
def test_table_regions_are_disjoint(lib, shapes):
    """Uncaptured calls (step, orthogonalise, blend) write the eager table
    region; captured steps read the capture region, which only
    muon_step_prepare writes: the two must not overlap each other or the
    iterate buffers."""
    eager, capture, tab, buffers, total = _layout(lib, shapes)
    n = len(shapes)
    assert tab >= n * 120                         # descriptors of every matrix fit
    lo, hi = sorted([eager, capture])
    assert lo + tab <= hi and hi + tab <= buffers <= total
    assert eager % 256 == 0 and capture % 256 == 0 and buffers % 256 == 0


def test_layout_rejects_bad_arguments(lib):
    v = [ctypes.c_size_t() for _ in range(4)]
    r = [ctypes.byref(x) for x in v]
    mats = _lib.mat_array([(0, 0, 4, 4, _lib.MUON_BF16)])
    assert lib.muon_workspace_layout(mats, 1, None, *r) == E["MUON_E_SHAPE"]
    assert lib.muon_workspace_layout(None, 1, None, *r) == E["MUON_E_NULL"]
    mats = _lib.mat_array([(0, 4, 4, 4, _lib.MUON_BF16)])
    assert lib.muon_workspace_layout(mats, 1, None, None, *r[1:]) == E["MUON_E_NULL"]


def test_state_advance_follows_the_step_rules(lib):
    st = _lib.MuonState()
    st.opt = _lib.default_options()
    st.step = 7
    assert lib.muon_state_advance(ctypes.byref(st), 3) == 0
    assert st.step == 10 and st.ema_count == 0
    assert lib.muon_state_advance(ctypes.byref(st), -1) == E["MUON_E_HPARAM"]
    assert lib.muon_state_advance(None, 1) == E["MUON_E_NULL"]
    # exponential average started at step 5: each replay folds into it
    st.opt.beta_ema = 0.99
    st.opt.ema_start = 5
    st.ema_count = 6
    assert lib.muon_state_advance(ctypes.byref(st), 2) == 0
    assert st.step == 12 and st.ema_count == 8
    # an average that has not started could not have been captured
    st.ema_count = 0
    st.step = 1
    assert lib.muon_state_advance(ctypes.byref(st), 1) == E["MUON_E_CAPTURE"]
    assert st.step == 1 and st.ema_count == 0
    # neither could a weighted running mean
    st.ema_count = 3
    st.step = 9
    st.opt.avg_mode = _lib.MUON_AVG_WEIGHTED
    assert lib.muon_state_advance(ctypes.byref(st), 1) == E["MUON_E_CAPTURE"]
    assert st.step == 9 and st.ema_count == 3
    st.opt.avg_mode = 7
    assert lib.muon_state_advance(ctypes.byref(st), 1) == E["MUON_E_HPARAM"]
