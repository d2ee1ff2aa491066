"""Helpers shared by the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

FP32_TOL = 1e-5      # relative L-inf, float32 I/O
BF16_TOL = 2e-2      # relative L-inf, bf16 I/O with float32 state


def rel_linf(got, ref):
    """max |got - ref| / max |ref| in float64 (0 when both are all-zero)."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = ref.detach().double().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.max(np.abs(r)) if r.size else 0.0
    num = np.max(np.abs(g - r)) if r.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def dev(a, dtype=torch.float32):
    """numpy (float32 values, bf16-representable when dtype is bf16) -> device."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=dtype).contiguous()


def host(t):
    return t.detach().double().cpu().numpy()


def tol(dtype):
    return BF16_TOL if dtype == torch.bfloat16 else FP32_TOL
