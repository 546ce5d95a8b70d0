"""Expert-routed affine-quantised matmul (gather_qmm) for AMD Instinct MI355X.

A thin ctypes binding over ``libmq.so`` (C ABI in ``include/mq.h``).  The
functions carry the C names and only marshal arguments: they take torch
tensors on the GPU, allocate outputs and workspaces with torch on the
current stream, and pass raw device pointers plus the current HIP stream to
the library.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  If ``libmq.so`` has not been built, importing works but
the first call raises ``RuntimeError``.

Shapes:
    x            bf16 [T, Ax, M, K]          (Ax in {1, A})
    wq           uint32 (int32 storage) [E, N, K*bits/32]   transpose=True
                                            [E, K, N*bits/32]   transpose=False
    scales/biases bf16 [E, N, K/group_size] / [E, K, N/group_size]
    rhs_indices  int32 [T, A]
    out          bf16 [T, A, M, N]
A stored expert weight is always quantised along its last axis; transpose
selects whether it is applied transposed (x @ w_hat^T, the forward product)
or as stored (x @ w_hat, the backward product's orientation).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "MQError", "lib_path", "load", "mq_status_str", "mq_quantize", "mq_route_workspace",
    "mq_route", "mq_gather_qmm_workspace", "mq_gather_qmm", "mq_gather_route",
    "mq_gather_sums", "mq_gather_qmm_routed", "mq_qmm_workspace", "mq_qmm", "WsLayout",
    "mq_gather_mm_workspace", "mq_gather_mm",
    "mq_gather_qmm_glu", "ACT_SILU", "ACT_GELU", "mq_quantize_mx", "mq_gather_qmm_mx",
    "mq_quantize_nv", "mq_gather_qmm_nv", "mq_gather_qmm_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmq.so"
_lib = None

MQ_OK, MQ_ERR_INVALID, MQ_ERR_UNSUPPORTED, MQ_ERR_WORKSPACE, MQ_ERR_HIP = range(5)

# size of the library's own per-GPU scratch (MQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


class MQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mq_status_str(status)}")


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t)
                for n in ("offsets", "perm", "error", "tiles", "sums", "part", "total")]


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load libmq.so (once).  Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m quantized_moe_grouped_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_size_t
    lib.mq_status_str.restype = ctypes.c_char_p
    lib.mq_status_str.argtypes = [I]
    lib.mq_quantize.restype = I
    lib.mq_quantize.argtypes = [P, I64, I64, I, I, P, P, P, P]
    lib.mq_route_workspace.restype = I
    lib.mq_route_workspace.argtypes = [I64, I32, ctypes.POINTER(SZ)]
    lib.mq_route.restype = I
    lib.mq_route.argtypes = [P, I64, I32, I, P, P, P, SZ, P]
    lib.mq_gather_qmm_workspace.restype = I
    lib.mq_gather_qmm_workspace.argtypes = [I64, I64, I64, I64, I64, I32, I, I, ctypes.POINTER(WsLayout)]
    lib.mq_gather_qmm.restype = I
    lib.mq_gather_qmm.argtypes = [P, I64, I64, I64, I64, P, P, P, I32, I64, P, I64,
                                  I, I, I, I, P, P, SZ, P]
    lib.mq_gather_route.restype = I
    lib.mq_gather_route.argtypes = [P, I64, I64, I64, I32, P, SZ, P]
    lib.mq_gather_sums.restype = I
    lib.mq_gather_sums.argtypes = [P, I64, I64, I64, I64, I64, I32, I, P, SZ, P]
    lib.mq_gather_qmm_routed.restype = I
    lib.mq_gather_qmm_routed.argtypes = [P, I64, I64, I64, I64, P, P, P, I32, I64, I64,
                                         I, I, I, P, P, SZ, P]
    lib.mq_qmm_workspace.restype = I
    lib.mq_qmm_workspace.argtypes = [I64, I64, I, ctypes.POINTER(SZ)]
    lib.mq_qmm.restype = I
    lib.mq_qmm.argtypes = [P, I64, I64, P, P, P, I64, I, I, I, P, P, SZ, P]
    lib.mq_gather_qmm_glu.restype = I
    lib.mq_gather_qmm_glu.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, I32, I64, P, I64,
                                      I, I, I, I, I, P, P, SZ, P]
    lib.mq_gather_mm_workspace.restype = I
    lib.mq_gather_mm_workspace.argtypes = [I64, I64, I64, I64, I64, I32, ctypes.POINTER(WsLayout)]
    lib.mq_gather_mm.restype = I
    lib.mq_gather_mm.argtypes = [P, I64, I64, I64, I64, P, I32, I64, P, I64, I, I, P, P, SZ, P]
    lib.mq_quantize_mx.restype = I
    lib.mq_quantize_mx.argtypes = [P, I64, I64, I, P, P, P]
    lib.mq_gather_qmm_mx.restype = I
    lib.mq_gather_qmm_mx.argtypes = [P, I64, I64, I64, I64, P, P, I32, I64, P, I64, I, I, I, P,
                                     P, SZ, P]
    lib.mq_quantize_nv.restype = I
    lib.mq_quantize_nv.argtypes = [P, I64, I64, I64, P, P, P, P]
    lib.mq_gather_qmm_nv.restype = I
    lib.mq_gather_qmm_nv.argtypes = [P, I64, I64, I64, I64, P, P, P, I32, I64, P, I64, I, I, P,
                                     P, SZ, P]
    lib.mq_gather_qmm_noalloc.restype = I
    lib.mq_gather_qmm_noalloc.argtypes = [P, I64, I64, I64, I64, P, P, P, I32, I64, P, I64,
                                          I, I, I, I, P, P]
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != MQ_OK:
        raise MQError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, dtype, name):
    import torch
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def mq_status_str(status: int) -> str:
    return load().mq_status_str(status).decode()


def mq_quantize(w, group_size: int = 64, bits: int = 4):
    """Affine-quantise ``w`` (bf16 [..., K]) along its last axis.

    Returns (wq int32 [..., K*bits/32] holding the uint32 words, scales bf16
    [..., K/gs], biases bf16 [..., K/gs])."""
    import torch
    lib = load()
    _need(w, torch.bfloat16, "w")
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    lead = tuple(w.shape[:-1])
    wq = torch.empty(lead + (K * bits // 32,), dtype=torch.int32, device=w.device)
    sc = torch.empty(lead + (K // group_size if group_size else 0,), dtype=torch.bfloat16, device=w.device)
    bs = torch.empty_like(sc)
    _check(lib.mq_quantize(_ptr(w), rows, K, group_size, bits, _ptr(wq), _ptr(sc), _ptr(bs),
                           _stream(w.device)), "mq_quantize")
    return wq, sc, bs


def mq_route_workspace(n: int, E: int) -> int:
    b = ctypes.c_size_t(0)
    _check(load().mq_route_workspace(n, E, ctypes.byref(b)), "mq_route_workspace")
    return b.value


def mq_route(idx, E: int, sorted_indices: bool = False):
    """Stable grouping of flat pair indices by expert: returns (perm int32 [n],
    offsets int32 [E+1])."""
    import torch
    lib = load()
    _need(idx, torch.int32, "idx")
    n = idx.numel()
    perm = torch.empty(n, dtype=torch.int32, device=idx.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=idx.device)
    wsb = mq_route_workspace(n, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device=idx.device) if wsb else None
    _check(lib.mq_route(_ptr(idx), n, E, int(sorted_indices), _ptr(perm), offsets.data_ptr(),
                        _ptr(ws), wsb, _stream(idx.device)), "mq_route")
    return perm, offsets


def _weight_dims(wq, scales, biases, K, group_size, bits, transpose):
    """(E, N) of a quantised stack applied to x with K features."""
    E = wq.shape[0]
    if transpose:
        N = wq.shape[-2]
        ok = wq.shape[-1] * 32 == K * bits and scales.shape[-2:] == (N, K // group_size)
    else:
        N = wq.shape[-1] * 32 // bits
        ok = wq.shape[-2] == K and scales.shape[-2:] == (K, N // group_size)
    if not ok or biases.shape != scales.shape or scales.shape[0] != E:
        raise ValueError("quantised weight shapes do not match x")
    return E, N


def mq_gather_qmm_workspace(T, A, M, K, N, E, group_size=64, bits=4) -> WsLayout:
    L = WsLayout()
    _check(load().mq_gather_qmm_workspace(T, A, M, K, N, E, group_size, bits, ctypes.byref(L)),
           "mq_gather_qmm_workspace")
    return L


def mq_gather_qmm(x, wq, scales, biases, rhs_indices, transpose: bool = True,
                  group_size: int = 64, bits: int = 4, sorted_indices: bool = False,
                  out=None, workspace=None, return_workspace: bool = False):
    """out[t,a,m,:] = x[t, a*(Ax>1), m, :] @ w_hat[rhs_indices[t,a]]^T (bf16)."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(rhs_indices, torch.int32, "rhs_indices")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.bfloat16, "scales")
    _need(biases, torch.bfloat16, "biases")
    if x.dim() != 4 or rhs_indices.dim() != 2 or wq.dim() != 3:
        raise ValueError("x must be [T, Ax, M, K], rhs_indices [T, A], wq 3-d")
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    if rhs_indices.shape[0] != T:
        raise ValueError("rhs_indices must have T rows")
    E, N = _weight_dims(wq, scales, biases, K, group_size, bits, transpose)
    L = mq_gather_qmm_workspace(T, A, M, K, N, E, group_size, bits)
    if out is None:
        out = torch.empty((T, A, M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, A, M, N):
            raise ValueError("out must be [T, A, M, N]")
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=x.device)
    _check(lib.mq_gather_qmm(_ptr(x), T, Ax, M, K, _ptr(wq), _ptr(scales), _ptr(biases), E, N,
                             _ptr(rhs_indices), A, int(transpose), group_size, bits,
                             int(sorted_indices), _ptr(out), workspace.data_ptr(),
                             workspace.numel(), _stream(x.device)), "mq_gather_qmm")
    if return_workspace:
        return out, workspace, L
    return out


def mq_gather_qmm_noalloc(x, wq, scales, biases, rhs_indices, out, transpose: bool = True,
                          group_size: int = 64, bits: int = 4, sorted_indices: bool = False):
    """mq_gather_qmm on the library's own per-GPU scratch: no workspace, and
    nothing is allocated (``out`` is the caller's)."""
    import torch
    lib = load()
    for t, dt, name in ((x, torch.bfloat16, "x"), (rhs_indices, torch.int32, "rhs_indices"),
                        (wq, torch.int32, "wq"), (scales, torch.bfloat16, "scales"),
                        (biases, torch.bfloat16, "biases"), (out, torch.bfloat16, "out")):
        _need(t, dt, name)
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    E, N = _weight_dims(wq, scales, biases, K, group_size, bits, transpose)
    if tuple(out.shape) != (T, A, M, N):
        raise ValueError("out must be [T, A, M, N]")
    _check(lib.mq_gather_qmm_noalloc(_ptr(x), T, Ax, M, K, _ptr(wq), _ptr(scales), _ptr(biases),
                                     E, N, _ptr(rhs_indices), A, int(transpose), group_size, bits,
                                     int(sorted_indices), _ptr(out), _stream(x.device)),
           "mq_gather_qmm_noalloc")
    return out


ACT_SILU, ACT_GELU = 1, 2


def mq_gather_qmm_glu(x, gate, up, rhs_indices, act: int = ACT_SILU, transpose: bool = True,
                      group_size: int = 64, bits: int = 4, sorted_indices: bool = False,
                      out=None, workspace=None, return_workspace: bool = False):
    """h[t,a,m,:] = act(x_r @ w_gate[e]^T) * (x_r @ w_up[e]^T), e = rhs_indices[t,a],
    x_r = x[t, a*(Ax>1), m]; gate and up are (wq, scales, biases) triples of
    [E, F, K] quantised stacks; act ACT_SILU or ACT_GELU (bf16 out [T, A, M, F])."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(rhs_indices, torch.int32, "rhs_indices")
    for name, (wq, sc, bs) in (("gate", gate), ("up", up)):
        _need(wq, torch.int32, f"{name} wq")
        _need(sc, torch.bfloat16, f"{name} scales")
        _need(bs, torch.bfloat16, f"{name} biases")
    if x.dim() != 4 or rhs_indices.dim() != 2:
        raise ValueError("x must be [T, Ax, M, K], rhs_indices [T, A]")
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    if rhs_indices.shape[0] != T:
        raise ValueError("rhs_indices must have T rows")
    E, F = gate[0].shape[0], gate[0].shape[1]
    for wq, sc, bs in (gate, up):
        if (wq.dim() != 3 or tuple(wq.shape) != (E, F, K * bits // 32)
                or tuple(sc.shape) != (E, F, K // group_size) or sc.shape != bs.shape):
            raise ValueError("gate and up must be quantised [E, F, K] stacks matching x")
    L = mq_gather_qmm_workspace(T, A, M, K, F, E, group_size, bits)
    if out is None:
        out = torch.empty((T, A, M, F), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, A, M, F):
            raise ValueError("out must be [T, A, M, F]")
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=x.device)
    _check(lib.mq_gather_qmm_glu(_ptr(x), T, Ax, M, K, _ptr(gate[0]), _ptr(gate[1]), _ptr(gate[2]),
                                 _ptr(up[0]), _ptr(up[1]), _ptr(up[2]), E, F, _ptr(rhs_indices),
                                 A, int(transpose), group_size, bits, int(sorted_indices), int(act),
                                 _ptr(out), workspace.data_ptr(), workspace.numel(),
                                 _stream(x.device)), "mq_gather_qmm_glu")
    if return_workspace:
        return out, workspace, L
    return out


def mq_gather_mm_workspace(T, A, M, K, N, E) -> WsLayout:
    L = WsLayout()
    _check(load().mq_gather_mm_workspace(T, A, M, K, N, E, ctypes.byref(L)),
           "mq_gather_mm_workspace")
    return L


def mq_gather_mm(x, w, rhs_indices, transpose: bool = True, sorted_indices: bool = False,
                 out=None, workspace=None, return_workspace: bool = False):
    """out[t,a,m,:] = x[t, a*(Ax>1), m, :] @ w[rhs_indices[t,a]]^T with a bf16
    expert stack w [E, N, K] (bf16 out)."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(w, torch.bfloat16, "w")
    _need(rhs_indices, torch.int32, "rhs_indices")
    if x.dim() != 4 or rhs_indices.dim() != 2 or w.dim() != 3:
        raise ValueError("x must be [T, Ax, M, K], rhs_indices [T, A], w [E, N, K]")
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    if rhs_indices.shape[0] != T:
        raise ValueError("rhs_indices must have T rows")
    E, N = w.shape[0], w.shape[1]
    if w.shape[2] != K:
        raise ValueError("w must be [E, N, K] with x's K")
    L = mq_gather_mm_workspace(T, A, M, K, N, E)
    if out is None:
        out = torch.empty((T, A, M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, A, M, N):
            raise ValueError("out must be [T, A, M, N]")
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=x.device)
    _check(lib.mq_gather_mm(_ptr(x), T, Ax, M, K, _ptr(w), E, N, _ptr(rhs_indices), A,
                            int(transpose), int(sorted_indices), _ptr(out),
                            workspace.data_ptr(), workspace.numel(), _stream(x.device)),
           "mq_gather_mm")
    if return_workspace:
        return out, workspace, L
    return out


def mq_quantize_mx(w, bits: int = 4):
    """MX-quantise ``w`` (bf16 [..., K], K % 32 == 0) along its last axis:
    MXFP4 (bits 4, E2M1 codes) or MXFP8 (bits 8, E4M3 codes).

    Returns (wq int32 [..., K*bits/32] holding the uint32 words, scales uint8
    [..., K/32] holding the E8M0 exponents)."""
    import torch
    lib = load()
    _need(w, torch.bfloat16, "w")
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    lead = tuple(w.shape[:-1])
    wq = torch.empty(lead + (K * bits // 32,), dtype=torch.int32, device=w.device)
    sc = torch.empty(lead + (K // 32,), dtype=torch.uint8, device=w.device)
    _check(lib.mq_quantize_mx(_ptr(w), rows, K, bits, _ptr(wq), _ptr(sc), _stream(w.device)),
           "mq_quantize_mx")
    return wq, sc


def mq_gather_qmm_mx(x, wq, scales, rhs_indices, transpose: bool = True,
                     sorted_indices: bool = False, out=None, workspace=None,
                     return_workspace: bool = False, bits: int = 4):
    """out[t,a,m,:] = x[t, a*(Ax>1), m, :] @ w_hat[rhs_indices[t,a]]^T with an
    MX expert stack (wq int32 [E, N, K*bits/32], scales uint8 [E, N, K/32];
    bits 4 = MXFP4, 8 = MXFP8)."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.uint8, "scales")
    _need(rhs_indices, torch.int32, "rhs_indices")
    if x.dim() != 4 or rhs_indices.dim() != 2 or wq.dim() != 3 or scales.dim() != 3:
        raise ValueError("x must be [T, Ax, M, K], rhs_indices [T, A], wq [E, N, K/8], "
                         "scales [E, N, K/32]")
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    if rhs_indices.shape[0] != T:
        raise ValueError("rhs_indices must have T rows")
    E, N = wq.shape[0], wq.shape[1]
    if wq.shape[2] * (32 // bits) != K or tuple(scales.shape) != (E, N, K // 32):
        raise ValueError("wq / scales do not match x's K")
    L = mq_gather_mm_workspace(T, A, M, K, N, E)
    if out is None:
        out = torch.empty((T, A, M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, A, M, N):
            raise ValueError("out must be [T, A, M, N]")
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=x.device)
    _check(lib.mq_gather_qmm_mx(_ptr(x), T, Ax, M, K, _ptr(wq), _ptr(scales), E, N,
                                _ptr(rhs_indices), A, int(transpose), bits, int(sorted_indices),
                                _ptr(out), workspace.data_ptr(), workspace.numel(),
                                _stream(x.device)), "mq_gather_qmm_mx")
    if return_workspace:
        return out, workspace, L
    return out


def mq_quantize_nv(w):
    """NVFP4-quantise a bf16 stack ``w`` [tensors, rows, K] (K % 16 == 0).

    Returns (wq int32 [tensors, rows, K/8], scales uint8 [tensors, rows, K/16]
    (E4M3 block scales), gscale float32 [tensors])."""
    import torch
    lib = load()
    _need(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [tensors, rows, K]")
    Tn, R, K = w.shape
    wq = torch.empty((Tn, R, K // 8), dtype=torch.int32, device=w.device)
    sc = torch.empty((Tn, R, K // 16), dtype=torch.uint8, device=w.device)
    g = torch.empty((Tn,), dtype=torch.float32, device=w.device)
    _check(lib.mq_quantize_nv(_ptr(w), Tn, R, K, _ptr(wq), _ptr(sc), _ptr(g), _stream(w.device)),
           "mq_quantize_nv")
    return wq, sc, g


def mq_gather_qmm_nv(x, wq, scales, gscale, rhs_indices, transpose: bool = True,
                     sorted_indices: bool = False, out=None, workspace=None,
                     return_workspace: bool = False):
    """out[t,a,m,:] = x[t, a*(Ax>1), m, :] @ w_hat[rhs_indices[t,a]]^T with an
    NVFP4 expert stack (wq int32 [E, N, K/8], scales uint8 [E, N, K/16],
    gscale float32 [E])."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.uint8, "scales")
    _need(gscale, torch.float32, "gscale")
    _need(rhs_indices, torch.int32, "rhs_indices")
    if x.dim() != 4 or rhs_indices.dim() != 2 or wq.dim() != 3 or scales.dim() != 3:
        raise ValueError("x must be [T, Ax, M, K], rhs_indices [T, A], wq [E, N, K/8], "
                         "scales [E, N, K/16]")
    T, Ax, M, K = x.shape
    A = rhs_indices.shape[1]
    if rhs_indices.shape[0] != T:
        raise ValueError("rhs_indices must have T rows")
    E, N = wq.shape[0], wq.shape[1]
    if wq.shape[2] * 8 != K or tuple(scales.shape) != (E, N, K // 16) or gscale.numel() != E:
        raise ValueError("wq / scales / gscale do not match x's K and the expert count")
    L = mq_gather_mm_workspace(T, A, M, K, N, E)
    if out is None:
        out = torch.empty((T, A, M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, A, M, N):
            raise ValueError("out must be [T, A, M, N]")
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=x.device)
    _check(lib.mq_gather_qmm_nv(_ptr(x), T, Ax, M, K, _ptr(wq), _ptr(scales), _ptr(gscale), E, N,
                                _ptr(rhs_indices), A, int(transpose), int(sorted_indices),
                                _ptr(out), workspace.data_ptr(), workspace.numel(),
                                _stream(x.device)), "mq_gather_qmm_nv")
    if return_workspace:
        return out, workspace, L
    return out


def mq_gather_route(rhs_indices, E: int, M: int = 1, workspace=None, K: int = 64,
                    group_size: int = 64):
    """Route rhs_indices [T, A] into a workspace (returned) for later
    ``mq_gather_qmm_routed`` calls that share this routing.  A workspace
    allocated here is sized for those calls' K and group size."""
    import torch
    lib = load()
    _need(rhs_indices, torch.int32, "rhs_indices")
    T, A = rhs_indices.shape
    L = mq_gather_qmm_workspace(T, A, M, K, 0, E, group_size, 4)
    if workspace is None:
        workspace = torch.empty(L.total, dtype=torch.uint8, device=rhs_indices.device)
    _check(lib.mq_gather_route(_ptr(rhs_indices), T, A, M, E, workspace.data_ptr(),
                               workspace.numel(), _stream(rhs_indices.device)), "mq_gather_route")
    return workspace


def mq_gather_sums(x, A: int, E: int, workspace, group_size: int = 64):
    """Per-group row sums of x [T, Ax, M, K] into ``workspace`` for later
    ``mq_gather_qmm_routed`` calls on this x."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    T, Ax, M, K = x.shape
    _check(lib.mq_gather_sums(_ptr(x), T, Ax, A, M, K, E, group_size, workspace.data_ptr(),
                              workspace.numel(), _stream(x.device)), "mq_gather_sums")
    return workspace


def mq_gather_qmm_routed(x, wq, scales, biases, A: int, workspace, transpose: bool = True,
                         group_size: int = 64, bits: int = 4, out=None):
    """The matmul half of mq_gather_qmm, using the routing and the row sums of
    x held in ``workspace`` (from mq_gather_route and mq_gather_sums)."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.bfloat16, "scales")
    _need(biases, torch.bfloat16, "biases")
    T, Ax, M, K = x.shape
    E, N = _weight_dims(wq, scales, biases, K, group_size, bits, transpose)
    if out is None:
        out = torch.empty((T, A, M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib.mq_gather_qmm_routed(_ptr(x), T, Ax, M, K, _ptr(wq), _ptr(scales), _ptr(biases),
                                    E, N, A, int(transpose), group_size, bits, _ptr(out),
                                    workspace.data_ptr(), workspace.numel(),
                                    _stream(x.device)), "mq_gather_qmm_routed")
    return out


def mq_qmm_workspace(M: int, K: int, group_size: int = 64) -> int:
    b = ctypes.c_size_t(0)
    _check(load().mq_qmm_workspace(M, K, group_size, ctypes.byref(b)), "mq_qmm_workspace")
    return b.value


def mq_qmm(x, wq, scales, biases, transpose: bool = True, group_size: int = 64,
           bits: int = 4, out=None, workspace=None):
    """Dense quantised matmul: out = x @ w_hat^T (x bf16 [M, K], wq [N, K*bits/32])
    or, with transpose=False, x @ w_hat (wq [K, N*bits/32])."""
    import torch
    lib = load()
    _need(x, torch.bfloat16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.bfloat16, "scales")
    _need(biases, torch.bfloat16, "biases")
    if x.dim() != 2 or wq.dim() != 2:
        raise ValueError("x must be [M, K] and wq 2-d")
    M, K = x.shape
    _, N = _weight_dims(wq[None], scales[None], biases[None], K, group_size, bits, transpose)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(mq_qmm_workspace(M, K, group_size), 1), dtype=torch.uint8,
                                device=x.device)
    _check(lib.mq_qmm(_ptr(x), M, K, _ptr(wq), _ptr(scales), _ptr(biases), N, int(transpose),
                      group_size, bits, _ptr(out), workspace.data_ptr(), workspace.numel(),
                      _stream(x.device)), "mq_qmm")
    return out
