"""Helpers for the GPU tests: host <-> device marshalling and the tolerance gate."""
from __future__ import annotations

import numpy as np

# Gate for the bf16 output against the fp64 oracle, per element
#   |out - ref| <= ATOL_REL * max(1, |ref|)
# and over the whole output  ||out - ref||_F / ||ref||_F <= FRO_REL.
# Rounding the fp32 accumulator to bf16 alone contributes up to 2^-9 |ref|
# per element (~1.1e-3 RMS relative); fp32 accumulation adds ~1e-6.
ATOL_REL = 1e-2
FRO_REL = 4e-3


def torch_dev():
    import torch
    return torch.device("cuda:0")


def bf16_to_torch(a_u16: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).to(device)


def u32_to_torch(a_u32: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u32).view(np.int32)).to(device)


def i32_to_torch(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def torch_bf16_to_u16(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def torch_to_u32(t) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def bf16_u16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_gate(out_f64: np.ndarray, ref: np.ndarray, what: str = ""):
    """Raise AssertionError (with the worst offenders) unless the gate holds."""
    assert out_f64.shape == ref.shape, (out_f64.shape, ref.shape)
    assert np.isfinite(out_f64).all(), f"{what}: non-finite output"
    err = np.abs(out_f64 - ref)
    lim = ATOL_REL * np.maximum(1.0, np.abs(ref))
    bad = err > lim
    if bad.any():
        i = np.argsort((err / lim).ravel())[::-1][:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements over the gate; "
                             f"worst (flat idx, out, ref): "
                             f"{[(int(k), float(out_f64.ravel()[k]), float(ref.ravel()[k])) for k in i]}")
    den = np.linalg.norm(ref)
    if den > 0:
        fro = np.linalg.norm(out_f64 - ref) / den
        assert fro <= FRO_REL, f"{what}: relative Frobenius error {fro:.3e} > {FRO_REL}"
