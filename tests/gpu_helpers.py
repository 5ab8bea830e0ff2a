"""Shared helpers of the GPU tests (device transfer, tolerances)."""
import numpy as np
import torch

from workloads import gen

# Tolerances: relative Frobenius error of O against the fp64 oracle, and the
# largest deviation of its singular values.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_SIGMA = 1e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy as float32 (bf16 values widened exactly)."""
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return gen.f32_from_bf16_bits(bits)
    return t.float().cpu().numpy()


def sigma_dev(a: np.ndarray, b: np.ndarray) -> float:
    sa = np.linalg.svd(np.asarray(a, np.float64), compute_uv=False)
    sb = np.linalg.svd(np.asarray(b, np.float64), compute_uv=False)
    return float(np.max(np.abs(sa - sb)))


def announce(msg: str) -> None:
    print(msg, flush=True)
