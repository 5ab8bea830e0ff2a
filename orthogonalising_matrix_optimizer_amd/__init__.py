"""MI355X (gfx950) Muon-style optimizer step: HIP kernels behind a C ABI.

`libmuon_mi355x.so` (built from csrc/ by `build.py`) does all the work; this
package only marshals torch tensors to its entry points.
"""
from . import _lib
from .optimizer import (CUBIC, QUINTIC, AdamW, Muon, StepGraph, coeff_rows, orthogonalize, plan_info,
                        probe_arm, probe_disarm, probe_read, workspace_bytes)

__all__ = ["Muon", "AdamW", "StepGraph", "orthogonalize", "workspace_bytes", "plan_info", "probe_arm",
           "probe_read", "probe_disarm", "coeff_rows", "CUBIC", "QUINTIC", "_lib"]
