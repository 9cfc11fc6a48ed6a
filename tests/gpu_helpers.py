"""Helpers shared by the GPU parity tests: host↔device copies and checks."""
import numpy as np
import torch

from rotated_top_activation_amd import workloads as wl


def dev(a, dtype):
    return wl.to_torch(a, dtype, "cuda")


def host(t) -> np.ndarray:
    """A device tensor's exact values as float64 (or int64 for integers)."""
    t = t.detach().cpu()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy().astype(np.int64)
    return t.to(torch.float64).numpy() if t.dtype == torch.bfloat16 else t.numpy().astype(np.float64)


def host_f32(t) -> np.ndarray:
    return t.detach().cpu().to(torch.float32).numpy()


def guarded(shape, dtype, pad=64, fill=1234.5):
    """An output tensor inside a buffer with canary padding on both sides.
    Returns (view, checker)."""
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    view = buf[pad:pad + n].view(*shape)

    def intact():
        b = buf.cpu()
        return bool((b[:pad] == fill).all() and (b[pad + n:] == fill).all())
    return view, intact


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |a| (float64)."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(np.where(a == 0, 1e-38, a))
    return np.ldexp(1.0, np.maximum(e - 8, -133))
