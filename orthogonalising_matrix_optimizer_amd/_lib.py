"""ctypes view of include/muon.h.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint8, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
# MUON_LIB_PATH selects another build of the same library (the host-sanitised
# build of the C ABI used by the CPU tests); the default is the in-tree build
LIB_PATH = os.environ.get("MUON_LIB_PATH") or os.path.join(PKG, "libmuon_mi355x.so")

MUON_BF16, MUON_F32 = 0, 1
MUON_AVG_EMA, MUON_AVG_WEIGHTED = 0, 1
STATUS = {
    0: "MUON_OK", 1: "MUON_E_NULL", 2: "MUON_E_SHAPE", 3: "MUON_E_DTYPE",
    4: "MUON_E_COEFFS", 5: "MUON_E_HPARAM", 6: "MUON_E_WORKSPACE",
    7: "MUON_E_ALIAS", 8: "MUON_E_ALIGN", 9: "MUON_E_HIP", 10: "MUON_E_STATE",
    11: "MUON_E_CAPTURE",
}
CODES = {v: k for k, v in STATUS.items()}
PHASES = {"prepare": 0, "gram": 1, "poly": 2, "apply": 3, "finish": 4, "adamw": 5,
          "apply_update": 6, "ns_single": 7}
MAX_STEPS = 16
NOALLOC_SCRATCH_BYTES = 64 << 20


class MuonMat(ctypes.Structure):
    _fields_ = [("ptr", c_void_p), ("rows", c_int64), ("cols", c_int64), ("ld", c_int64),
                ("dtype", c_int32), ("_pad", c_int32)]


class MuonOptions(ctypes.Structure):
    _fields_ = [("beta_slow", c_float), ("beta_ema", c_float), ("eps", c_float),
                ("nesterov", c_int32), ("ema_start", c_int64), ("cautious", c_int32),
                ("ns_dtype", c_int32), ("avg_mode", c_int32), ("_pad", c_int32)]


class MuonState(ctypes.Structure):
    _fields_ = [("n", c_int32), ("_pad", c_int32),
                ("mom", POINTER(c_void_p)), ("mom_slow", POINTER(c_void_p)),
                ("ema", POINTER(c_void_p)), ("mask_out", POINTER(c_void_p)),
                ("update_out", POINTER(c_void_p)),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("step", c_int64), ("ema_count", c_int64), ("opt", MuonOptions),
                ("avg_weight", c_float), ("_pad2", c_int32), ("avg_weight_sum", ctypes.c_double)]


class MuonVec(ctypes.Structure):
    _fields_ = [("ptr", c_void_p), ("numel", c_int64), ("dtype", c_int32), ("_pad", c_int32)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("wd", c_float), ("_pad", c_int32)]


class AdamWState(ctypes.Structure):
    _fields_ = [("n", c_int32), ("_pad", c_int32), ("m", POINTER(c_void_p)),
                ("v", POINTER(c_void_p)), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("step", c_int64)]


class MuonError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({code})")
        self.code = code


_LIB = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m orthogonalising_matrix_optimizer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    lib.muon_default_options.argtypes = [P(MuonOptions)]
    lib.muon_default_options.restype = None
    lib.muon_workspace_bytes.argtypes = [P(MuonMat), c_int32, P(MuonOptions), c_int32]
    lib.muon_workspace_bytes.restype = c_size_t
    lib.muon_step.argtypes = [P(MuonMat), P(MuonMat), P(MuonState), P(c_float), c_int32,
                              c_float, c_float, c_float, c_void_p]
    lib.muon_step.restype = c_int32
    lib.muon_step_prepare.argtypes = [P(MuonMat), P(MuonMat), P(MuonState), c_void_p]
    lib.muon_step_prepare.restype = c_int32
    lib.muon_orthogonalize.argtypes = [P(MuonMat), P(MuonMat), c_int32, P(c_float), c_int32,
                                       P(MuonOptions), c_void_p, c_size_t, c_void_p]
    lib.muon_orthogonalize.restype = c_int32
    lib.muon_ema_blend.argtypes = [P(MuonMat), P(MuonMat), P(MuonState), c_float, c_void_p]
    lib.muon_ema_blend.restype = c_int32
    lib.muon_status_str.argtypes = [c_int32]
    lib.muon_status_str.restype = ctypes.c_char_p
    lib.muon_probe_arm.argtypes = [c_int32, c_int32]
    lib.muon_probe_arm.restype = c_int32
    lib.muon_probe_read.argtypes = [P(c_float), c_int32, P(c_int32)]
    lib.muon_probe_read.restype = c_int32
    lib.muon_probe_disarm.argtypes = []
    lib.muon_probe_disarm.restype = c_int32
    lib.muon_plan_info.argtypes = [P(MuonMat), c_int32, P(MuonOptions), c_int32, P(c_float),
                                   P(c_int32), P(c_int32), c_int32, P(c_int32)]
    lib.muon_plan_info.restype = c_int32
    lib.muon_step_noalloc.argtypes = [P(MuonMat), P(MuonMat), P(MuonState), P(c_float), c_int32,
                                      c_float, c_float, c_float, c_void_p]
    lib.muon_step_noalloc.restype = c_int32
    lib.muon_state_advance.argtypes = [P(MuonState), c_int32]
    lib.muon_state_advance.restype = c_int32
    lib.muon_workspace_layout.argtypes = [P(MuonMat), c_int32, P(MuonOptions), P(c_size_t),
                                          P(c_size_t), P(c_size_t), P(c_size_t)]
    lib.muon_workspace_layout.restype = c_int32
    lib.muon_adamw_workspace_bytes.argtypes = [c_int32]
    lib.muon_adamw_workspace_bytes.restype = c_size_t
    lib.muon_adamw_step.argtypes = [P(MuonVec), P(MuonVec), P(AdamWState), P(AdamWHparams),
                                    c_void_p]
    lib.muon_adamw_step.restype = c_int32
    _LIB = lib
    return lib


def check(code: int, where: str) -> None:
    if code != 0:
        raise MuonError(code, where)


def default_options() -> MuonOptions:
    o = MuonOptions()
    load().muon_default_options(ctypes.byref(o))
    return o


def mat_array(specs) -> ctypes.Array:
    """specs: iterable of (ptr, rows, cols, ld, dtype)."""
    specs = list(specs)
    arr = (MuonMat * max(1, len(specs)))()
    for i, (p, r, c, ld, dt) in enumerate(specs):
        arr[i] = MuonMat(c_void_p(p), r, c, ld, dt, 0)
    return arr


def ptr_array(ptrs):
    ptrs = list(ptrs)
    arr = (c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = c_void_p(p) if p else None
    return arr


def float_array(vals):
    vals = [float(v) for v in vals]
    return (c_float * max(1, len(vals)))(*vals)


def vec_array(specs) -> ctypes.Array:
    """specs: iterable of (ptr, numel, dtype)."""
    specs = list(specs)
    arr = (MuonVec * max(1, len(specs)))()
    for i, (p, ne, dt) in enumerate(specs):
        arr[i] = MuonVec(c_void_p(p) if p else None, ne, dt, 0)
    return arr


_ = c_uint8
