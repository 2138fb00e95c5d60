"""Shared helpers for the GPU tests (upload of seeded inputs, comparisons)."""
import numpy as np
import torch

DEV = "cuda:0"


def bf16_to_device(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bf16 tensor on the GPU (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_to_device(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close_rows(got, want, atol, rtol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    both_nan = np.isnan(got) & np.isnan(want)
    # outputs are fp32: their own rounding (2^-24 relative) is always allowed
    with np.errstate(invalid="ignore"):
        tol = atol + (rtol + 2.0 ** -24) * np.abs(want)
        ok = both_inf | both_nan | (np.abs(got - want) <= tol)
    if not ok.all():
        bad = np.flatnonzero(~ok)[:8]
        raise AssertionError(f"{what}: {(~ok).sum()} rows off; first {bad.tolist()}: "
                             f"got {got[bad].tolist()} want {want[bad].tolist()}")


def bits_equal(a, b) -> bool:
    """Bitwise equality of two tensors (NaNs with equal payloads compare equal)."""
    import torch
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    if a.dtype in (torch.float32, torch.int32):
        return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    return torch.equal(a, b)
