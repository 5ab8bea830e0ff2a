"""Torch-facing wrapper of the C ABI: owns device buffers, marshals pointers.

Every step of the computation runs in the HIP library; this module only
allocates state and workspace tensors, builds the pointer tables and passes
them, together with the current HIP stream, to the C entry points.  It
raises if the library has not been built or the tensors are not on a GPU.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Union

import numpy as np
import torch

from . import _lib

# Coefficient rows (a, b, c) of the map x -> a x + b x^3 + c x^5.
CUBIC = (1.5, -0.5, 0.0)                       # Newton-Schulz for the polar factor
QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)  # next member of that family

_DT = {torch.bfloat16: _lib.MUON_BF16, torch.float32: _lib.MUON_F32}
_NSDT = {"bf16": _lib.MUON_BF16, "f32": _lib.MUON_F32}


def coeff_rows(coeffs: Union[str, Sequence], steps: int) -> np.ndarray:
    if isinstance(coeffs, str):
        base = {"cubic": CUBIC, "quintic": QUINTIC}[coeffs]
        return np.array([base] * steps, dtype=np.float32).reshape(steps, 3)
    c = np.asarray(coeffs, dtype=np.float32).reshape(-1, 3)
    if c.shape[0] != steps:
        raise ValueError(f"coefficient table has {c.shape[0]} rows, steps={steps}")
    return c


def _mat(t: torch.Tensor):
    if t.dim() != 2:
        raise ValueError("matrices must be 2-D")
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return (t.data_ptr(), t.shape[0], t.shape[1], max(ld, t.shape[1]), _DT[t.dtype])


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(shapes: Sequence, ns_dtype: str = "bf16") -> int:
    lib = _lib.load()
    mats = _lib.mat_array((0, r, c, c, _lib.MUON_BF16) for r, c in shapes)
    opt = _lib.default_options()
    opt.ns_dtype = _NSDT[ns_dtype]
    return int(lib.muon_workspace_bytes(mats, len(shapes), opt, 0))


def orthogonalize(inputs: List[torch.Tensor], outputs: List[torch.Tensor],
                  coeffs: Union[str, Sequence] = "quintic", steps: int = 5,
                  ns_dtype: str = "bf16", eps: float = 1e-7,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """outputs[i] <- Newton-Schulz orthogonalisation of inputs[i] (in the library)."""
    lib = _lib.load()
    n = len(inputs)
    ins = _lib.mat_array(_mat(t) for t in inputs)
    outs = _lib.mat_array(_mat(t) for t in outputs)
    opt = _lib.default_options()
    opt.ns_dtype = _NSDT[ns_dtype]
    opt.eps = eps
    need = int(lib.muon_workspace_bytes(ins, n, opt, steps))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=inputs[0].device)
    c = coeff_rows(coeffs, steps)
    code = lib.muon_orthogonalize(ins, outs, n, _lib.float_array(c.ravel()), steps, opt,
                                  workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(code, "muon_orthogonalize")
    return workspace


class Muon:
    """Muon-style optimizer over a list of 2-D parameter tensors.

    Options follow include/muon.h: momentum `beta`, optional slow momentum
    `beta_slow` with `cautious` weight decay, optional weight average
    `beta_ema` from step `ema_start`, Nesterov look-ahead, bf16 or fp32
    Newton-Schulz operands.  `diagnostics` allocates per-matrix buffers that
    receive the applied mask and update O on every step.
    """

    def __init__(self, params: List[torch.Tensor], lr: float = 0.02, wd: float = 0.0,
                 beta: float = 0.95, steps: int = 5,
                 coeffs: Union[str, Sequence] = "quintic",
                 beta_slow: Optional[float] = None, beta_ema: Optional[float] = None,
                 ema_start: int = 1, cautious: bool = False, nesterov: bool = False,
                 ns_dtype: str = "bf16", eps: float = 1e-7, diagnostics: bool = False,
                 avg: str = "ema"):
        self.lib = _lib.load()
        self.params = list(params)
        self.lr, self.wd, self.beta, self.steps = float(lr), float(wd), float(beta), int(steps)
        self.coeffs = coeff_rows(coeffs, self.steps)
        self._coeffs_c = _lib.float_array(self.coeffs.ravel())
        dev = self.params[0].device if self.params else torch.device("cuda")
        f32 = dict(dtype=torch.float32, device=dev)
        self.mom = [torch.zeros(p.shape, **f32) for p in self.params]
        self.mom_slow = [torch.zeros(p.shape, **f32) for p in self.params] if beta_slow is not None else None
        self.ema = [torch.zeros(p.shape, **f32) for p in self.params] if beta_ema is not None else None
        self.mask = [torch.zeros(p.shape, dtype=torch.uint8, device=dev) for p in self.params] \
            if diagnostics else None
        self.update = [torch.zeros(p.shape, **f32) for p in self.params] if diagnostics else None
        self.opt = _lib.default_options()
        self.opt.beta_slow = -1.0 if beta_slow is None else float(beta_slow)
        self.opt.beta_ema = -1.0 if beta_ema is None else float(beta_ema)
        self.opt.eps = float(eps)
        self.opt.ema_start = int(ema_start)
        self.opt.cautious = int(bool(cautious))
        self.opt.nesterov = int(bool(nesterov))
        self.opt.ns_dtype = _NSDT[ns_dtype]
        self.opt.avg_mode = {"ema": _lib.MUON_AVG_EMA, "weighted": _lib.MUON_AVG_WEIGHTED}[avg]
        self._pmats = _lib.mat_array(_mat(p) for p in self.params)
        need = int(self.lib.muon_workspace_bytes(self._pmats, len(self.params), self.opt,
                                                 self.steps))
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.state = _lib.MuonState()
        self.state.n = len(self.params)
        self.state.avg_weight = 1.0
        self._keep = []
        self._bind_state()
        self._gkey = None
        self._gmats = None

    def _bind_state(self):
        st = self.state
        keep = []

        def arr(ts):
            if ts is None:
                return None
            a = _lib.ptr_array(t.data_ptr() for t in ts)
            keep.append(a)
            return ctypes_cast(a)

        st.mom = arr(self.mom)
        st.mom_slow = arr(self.mom_slow)
        st.ema = arr(self.ema)
        st.mask_out = arr(self.mask)
        st.update_out = arr(self.update)
        st.workspace = self.workspace.data_ptr()
        st.workspace_bytes = self.workspace.numel()
        st.opt = self.opt
        self._keep = keep

    @property
    def step_count(self) -> int:
        return int(self.state.step)

    @property
    def ema_count(self) -> int:
        return int(self.state.ema_count)

    @property
    def avg_weight(self) -> float:
        """Weight of the next averaged step (avg="weighted"; 1 = plain SWA)."""
        return float(self.state.avg_weight)

    @avg_weight.setter
    def avg_weight(self, w: float) -> None:
        self.state.avg_weight = float(w)

    def _grad_mats(self, grads: List[torch.Tensor]):
        key = tuple((g.data_ptr(), g.stride(0), g.dtype) for g in grads)
        if key != self._gkey:
            self._gmats = _lib.mat_array(_mat(g) for g in grads)
            self._gkey = key
        return self._gmats

    def step_prepare(self, grads: List[torch.Tensor]) -> None:
        """Make the device descriptor table for these gradient buffers resident
        (no launch, counters unchanged), so a step with them can be captured."""
        code = self.lib.muon_step_prepare(self._pmats, self._grad_mats(grads), self.state,
                                          _stream())
        _lib.check(code, "muon_step_prepare")

    def graph(self, grads: List[torch.Tensor], lr: Optional[float] = None,
              wd: Optional[float] = None) -> "StepGraph":
        """Capture one step on `grads` as a device graph; see StepGraph."""
        return StepGraph(self, grads, lr, wd)

    def step(self, grads: List[torch.Tensor], lr: Optional[float] = None,
             wd: Optional[float] = None) -> None:
        self._grad_mats(grads)
        code = self.lib.muon_step(self._pmats, self._gmats, self.state, self._coeffs_c,
                                  self.steps, self.lr if lr is None else lr,
                                  self.wd if wd is None else wd, self.beta, _stream())
        _lib.check(code, "muon_step")

    def blend(self, outputs: List[torch.Tensor], w_final: float = 0.35) -> None:
        outs = _lib.mat_array(_mat(t) for t in outputs)
        code = self.lib.muon_ema_blend(outs, self._pmats, self.state, w_final, _stream())
        _lib.check(code, "muon_ema_blend")

    # ---------------------------------------------------------- checkpointing
    def state_dict(self) -> Dict:
        return {
            "step": self.step_count, "ema_count": self.ema_count,
            "avg_weight_sum": float(self.state.avg_weight_sum),
            "mom": [m.clone() for m in self.mom],
            "mom_slow": None if self.mom_slow is None else [m.clone() for m in self.mom_slow],
            "ema": None if self.ema is None else [m.clone() for m in self.ema],
        }

    def load_state_dict(self, sd: Dict) -> None:
        for dst, src in zip(self.mom, sd["mom"]):
            dst.copy_(src)
        if self.mom_slow is not None:
            for dst, src in zip(self.mom_slow, sd["mom_slow"]):
                dst.copy_(src)
        if self.ema is not None:
            for dst, src in zip(self.ema, sd["ema"]):
                dst.copy_(src)
        self.state.step = int(sd["step"])
        self.state.ema_count = int(sd["ema_count"])
        self.state.avg_weight_sum = float(sd.get("avg_weight_sum", 0.0))


class StepGraph:
    """One optimizer step captured as a device graph and replayed.

    The first replay performs the captured step; every replay repeats it on the
    same buffers (parameters, the gradient tensors given at capture, state,
    workspace) with the captured lr, wd, beta, coefficients and weight-average
    flags.  Write new gradients into the captured gradient tensors before a
    replay.  Host counters advance per replay as for an eager step (through
    the library's muon_state_advance).  Eager steps, orthogonalisations and
    blends on the same optimizer between replays are allowed; capturing
    another graph on it replaces the table this one replays with.  Capture is
    refused for a step whose weight-average flags would not repeat (the average
    not yet started, or starting at this step): take eager steps first.
    """

    def __init__(self, opt: Muon, grads: List[torch.Tensor], lr: Optional[float] = None,
                 wd: Optional[float] = None):
        o = opt.opt
        st = opt.state
        if o.beta_ema >= 0.0 and o.avg_mode == _lib.MUON_AVG_WEIGHTED:
            raise ValueError("the weighted average changes its coefficients every step; "
                             "a replay would repeat the captured ones")
        if o.beta_ema >= 0.0:
            if st.step + 1 < o.ema_start or st.ema_count == 0:
                raise ValueError("capture after the weight average has started "
                                 "(its first step re-initialises it)")
        self.opt = opt
        self.grads = list(grads)
        opt.step_prepare(self.grads)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            opt.step(self.grads, lr, wd)
        # the capturing call advanced the counters for the step the first
        # replay performs
        self._pending = True

    def replay(self) -> None:
        self.g.replay()
        if self._pending:
            self._pending = False
            return
        _lib.check(self.opt.lib.muon_state_advance(self.opt.state, 1), "muon_state_advance")


def _vec(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("AdamW tensors must be contiguous")
    return (t.data_ptr() if t.numel() else 0, t.numel(), _DT[t.dtype])


class AdamW:
    """AdamW over a list of contiguous tensors (the parameters that are not
    weight matrices), one grouped launch per step; see include/muon.h.

    State: fp32 first and second moments per tensor and the step counter."""

    def __init__(self, params: List[torch.Tensor], lr: float = 1e-3,
                 betas: Sequence[float] = (0.9, 0.999), eps: float = 1e-8, wd: float = 0.0):
        self.lib = _lib.load()
        self.params = list(params)
        dev = self.params[0].device if self.params else torch.device("cuda")
        self.hp = _lib.AdamWHparams(float(lr), float(betas[0]), float(betas[1]), float(eps),
                                    float(wd), 0)
        self.m = [torch.zeros(p.numel(), dtype=torch.float32, device=dev) for p in self.params]
        self.v = [torch.zeros(p.numel(), dtype=torch.float32, device=dev) for p in self.params]
        n = len(self.params)
        self.workspace = torch.empty(int(self.lib.muon_adamw_workspace_bytes(n)),
                                     dtype=torch.uint8, device=dev)
        self._pvecs = _lib.vec_array(_vec(p) for p in self.params)
        self._mp = _lib.ptr_array(t.data_ptr() if t.numel() else 0 for t in self.m)
        self._vp = _lib.ptr_array(t.data_ptr() if t.numel() else 0 for t in self.v)
        self.state = _lib.AdamWState(n, 0, ctypes_cast(self._mp), ctypes_cast(self._vp),
                                     self.workspace.data_ptr(), self.workspace.numel(), 0)
        self._gkey = None
        self._gvecs = None

    @property
    def step_count(self) -> int:
        return int(self.state.step)

    def step(self, grads: List[torch.Tensor], lr: Optional[float] = None) -> None:
        key = tuple((g.data_ptr(), g.dtype, g.numel()) for g in grads)
        if key != self._gkey:
            self._gvecs = _lib.vec_array(_vec(g) for g in grads)
            self._gkey = key
        hp = self.hp
        if lr is not None:
            hp = _lib.AdamWHparams(float(lr), hp.beta1, hp.beta2, hp.eps, hp.wd, 0)
        code = self.lib.muon_adamw_step(self._pvecs, self._gvecs, self.state, hp, _stream())
        _lib.check(code, "muon_adamw_step")

    def state_dict(self) -> Dict:
        return {"step": self.step_count, "m": [t.clone() for t in self.m],
                "v": [t.clone() for t in self.v]}

    def load_state_dict(self, sd: Dict) -> None:
        for dst, src in zip(self.m, sd["m"]):
            dst.copy_(src)
        for dst, src in zip(self.v, sd["v"]):
            dst.copy_(src)
        self.state.step = int(sd["step"])


def ctypes_cast(a):
    import ctypes
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))


def probe_arm(phase: str, capacity: int) -> None:
    _lib.check(_lib.load().muon_probe_arm(_lib.PHASES[phase], capacity), "muon_probe_arm")


def probe_read(capacity: int) -> List[float]:
    import ctypes
    buf = (ctypes.c_float * capacity)()
    cnt = ctypes.c_int32(0)
    _lib.check(_lib.load().muon_probe_read(buf, capacity, ctypes.byref(cnt)), "muon_probe_read")
    return [buf[i] for i in range(cnt.value)]


def probe_disarm() -> None:
    _lib.check(_lib.load().muon_probe_disarm(), "muon_probe_disarm")


def plan_info(shapes: Sequence, steps: int, coeffs: Union[str, Sequence] = "quintic",
              ns_dtype: str = "bf16"):
    import ctypes
    lib = _lib.load()
    mats = _lib.mat_array((0, r, c, c, _lib.MUON_BF16) for r, c in shapes)
    opt = _lib.default_options()
    opt.ns_dtype = _NSDT[ns_dtype]
    c = coeff_rows(coeffs, steps)
    ng = ctypes.c_int32(0)
    tiles = (ctypes.c_int32 * 64)()
    lps = ctypes.c_int32(0)
    _lib.check(lib.muon_plan_info(mats, len(shapes), opt, steps, _lib.float_array(c.ravel()),
                                  ctypes.byref(ng), tiles, 64, ctypes.byref(lps)), "muon_plan_info")
    return {"groups": ng.value, "tile": tiles[0] if ng.value else 0, "launches_per_step": lps.value}
