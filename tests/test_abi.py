"""The C ABI on the CPU: libmq.so loads, exports what include/mq.h declares,
and rejects bad arguments before touching HIP (no compute call is made; the
pointers passed are never dereferenced because validation fails first)."""
import ctypes
import os
import re

import pytest

import quantized_moe_grouped_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")
PROBE_HEADER = os.path.join(ROOT, "include", "mq_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(mq.lib_path()), "libmq_probe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(mq.lib_path()),
                                reason="libmq.so not built (run __graft_entry__.build())")

FAKE = 0x1000   # a 16-byte aligned non-null address; never dereferenced in these tests


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|mq_status)\s+(mq_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("mq_quantize", "mq_route", "mq_route_workspace", "mq_gather_qmm",
              "mq_gather_qmm_workspace", "mq_gather_route", "mq_gather_sums", "mq_gather_qmm_routed",
              "mq_qmm_workspace", "mq_qmm", "mq_status_str",
              "mq_gather_mm_workspace", "mq_gather_mm", "mq_gather_qmm_glu", "mq_quantize_mx",
              "mq_gather_qmm_mx", "mq_quantize_nv", "mq_gather_qmm_nv", "mq_gather_qmm_noalloc"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = mq.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    assert "#define MQ_NOALLOC_SCRATCH_BYTES (16u << 20)" in src
    assert mq.NOALLOC_SCRATCH_BYTES == 16 << 20


def _noalloc(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, wq=FAKE, scales=FAKE, biases=FAKE, E=4, N=32,
             idx=FAKE, A=2, transpose=1, gs=64, bits=4, sorted_indices=0, out=FAKE, stream=None)
    a.update(kw)
    return mq.load().mq_gather_qmm_noalloc(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["wq"],
                                           a["scales"], a["biases"], a["E"], a["N"], a["idx"],
                                           a["A"], a["transpose"], a["gs"], a["bits"],
                                           a["sorted_indices"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    # more workspace than the 16 MiB scratch: 65536 pairs with x rows of 4096
    # (row sums alone 65536 * 3 * 64 * 2 bytes = 24 MiB)
    (dict(T=8192, A=8, Ax=8, K=4096), mq.MQ_ERR_WORKSPACE),
    (dict(bits=3), mq.MQ_ERR_UNSUPPORTED),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(x=None), mq.MQ_ERR_INVALID),
    (dict(out=FAKE + 8), mq.MQ_ERR_INVALID),
    (dict(E=0), mq.MQ_ERR_INVALID),
])
def test_noalloc_rejects_before_any_hip_call(kw, status):
    assert _noalloc(**kw) == status


def test_status_strings():
    assert mq.mq_status_str(0) == "MQ_OK"
    assert mq.mq_status_str(2) == "MQ_ERR_UNSUPPORTED"
    assert mq.mq_status_str(99) == "MQ_ERR_UNKNOWN"


def _gather(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, wq=FAKE, scales=FAKE, biases=FAKE, E=4, N=32,
             idx=FAKE, A=2, transpose=1, gs=64, bits=4, sorted_indices=0, out=FAKE,
             ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return mq.load().mq_gather_qmm(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["wq"], a["scales"],
                                   a["biases"], a["E"], a["N"], a["idx"], a["A"], a["transpose"],
                                   a["gs"], a["bits"], a["sorted_indices"], a["out"], a["ws"],
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bits=3), mq.MQ_ERR_UNSUPPORTED),
    (dict(bits=2), mq.MQ_ERR_UNSUPPORTED),
    (dict(gs=128), mq.MQ_ERR_UNSUPPORTED),
    (dict(gs=16), mq.MQ_ERR_UNSUPPORTED),
    (dict(transpose=2), mq.MQ_ERR_INVALID),
    (dict(transpose=0, N=48), mq.MQ_ERR_INVALID),       # N % group_size (groups along N)
    (dict(transpose=0, K=96, gs=32), mq.MQ_ERR_UNSUPPORTED),   # K % 64
    (dict(K=96, gs=64), mq.MQ_ERR_INVALID),          # K % group_size
    (dict(K=96, gs=32), mq.MQ_ERR_UNSUPPORTED),      # K % 64 (GEMM chunk)
    (dict(K=0), mq.MQ_ERR_INVALID),
    (dict(E=0), mq.MQ_ERR_INVALID),
    (dict(E=4096), mq.MQ_ERR_UNSUPPORTED),
    (dict(T=-1), mq.MQ_ERR_INVALID),
    (dict(A=0), mq.MQ_ERR_INVALID),
    (dict(M=0), mq.MQ_ERR_INVALID),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(x=None), mq.MQ_ERR_INVALID),
    (dict(idx=None), mq.MQ_ERR_INVALID),
    (dict(out=None), mq.MQ_ERR_INVALID),
    (dict(wq=None), mq.MQ_ERR_INVALID),
    (dict(scales=None), mq.MQ_ERR_INVALID),
    (dict(x=FAKE + 2), mq.MQ_ERR_INVALID),           # misaligned
    (dict(ws=None), mq.MQ_ERR_WORKSPACE),
    (dict(ws_bytes=16), mq.MQ_ERR_WORKSPACE),
    # a few rows per expert (the small-M path) and more than 1024 groups per row
    (dict(T=4, A=2, E=64, K=1025 * 64, gs=64), mq.MQ_ERR_UNSUPPORTED),
])
def test_gather_rejects_before_any_hip_call(kw, status):
    assert _gather(**kw) == status


def test_workspace_query_and_layout():
    L = mq.mq_gather_qmm_workspace(2048, 8, 1, 2048, 768, 64, 64, 4)
    assert L.offsets == 0
    for f in ("perm", "error", "tiles", "sums", "part", "total"):
        assert getattr(L, f) % 256 == 0
    assert L.perm >= 65 * 4 and L.error >= L.perm + 16384 * 4
    assert L.sums > L.tiles
    # row sums: 3 bf16 parts x 32 groups for each of the T*A*M rows
    assert L.total >= L.sums + 16384 * 3 * 32 * 2
    # the routing regions do not depend on K: a workspace routed once serves
    # projections of any K
    L2 = mq.mq_gather_qmm_workspace(2048, 8, 1, 512, 2048, 64, 64, 4)
    assert (L2.offsets, L2.perm, L2.error, L2.tiles, L2.sums) == \
        (L.offsets, L.perm, L.error, L.tiles, L.sums)
    # one correction window (K = 2048 in groups of 64): no piece slots
    assert L.part == L.total
    # short workspace by one byte is refused
    assert _gather(T=2048, A=8, Ax=8, K=2048, N=768, E=64, ws_bytes=L.total - 1) == mq.MQ_ERR_WORKSPACE
    with pytest.raises(mq.MQError):
        mq.mq_gather_qmm_workspace(4, 2, 1, 100, 8, 4, 64, 4)


def test_workspace_piece_slots():
    """Tail tiles split along K need slots of 64 KiB after the row sums: one
    tail tile per expert, ceil(N / 192) column tiles, min(8, windows) pieces,
    at most 1024 slots.  They are optional: everything before `part` is
    required, the rest is used as far as it is there."""
    slot = 65536
    # K = 8192 (4 windows of 32 groups of 64), N = 4096, 4 experts
    L0 = mq.mq_gather_qmm_workspace(512, 2, 1, 8192, 4096, 4, 64, 4)
    assert L0.part % 256 == 0 and L0.part >= L0.sums + 1024 * 3 * 128 * 2
    assert L0.total - L0.part == 4 * 22 * 4 * slot
    # Mixtral-shaped down projection: K = 14336 (7 windows), N = 4096, 8
    # experts: 8 * 22 * 7 slots, capped at 1024
    L = mq.mq_gather_qmm_workspace(2048, 2, 1, 14336, 4096, 8, 64, 4)
    assert L.total - L.part == 1024 * slot
    # groups of 32: windows of 1024; two windows at K = 2048
    L3 = mq.mq_gather_qmm_workspace(2048, 8, 1, 2048, 768, 64, 32, 4)
    assert L3.total - L3.part == 64 * 4 * 2 * slot
    # short runs (tiles of fewer than 64 rows have no tail tiles): none
    L4 = mq.mq_gather_qmm_workspace(256, 8, 1, 4096, 768, 256, 64, 4)
    assert L4.total == L4.part
    # the required part: one byte short is refused (a workspace of exactly
    # `part` bytes runs unsplit: tests/test_gpu_fullsize.py)
    kw = dict(T=2048, A=2, Ax=1, K=14336, N=4096, E=8)
    assert _gather(**kw, ws_bytes=L.part - 1) == mq.MQ_ERR_WORKSPACE


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 64, 64, 3, FAKE, FAKE, FAKE, None), mq.MQ_ERR_UNSUPPORTED),
    ((FAKE, 4, 100, 64, 4, FAKE, FAKE, FAKE, None), mq.MQ_ERR_INVALID),
    ((FAKE, -1, 64, 64, 4, FAKE, FAKE, FAKE, None), mq.MQ_ERR_INVALID),
    ((None, 4, 64, 64, 4, FAKE, FAKE, FAKE, None), mq.MQ_ERR_INVALID),
    ((FAKE, 0, 64, 64, 4, None, None, None, None), mq.MQ_OK),     # nothing to do
])
def test_quantize_rejects(args, status):
    assert mq.load().mq_quantize(*args) == status


def test_route_rejects():
    lib = mq.load()
    b = ctypes.c_size_t(0)
    assert lib.mq_route_workspace(100, 8, ctypes.byref(b)) == mq.MQ_OK and b.value > 0
    assert lib.mq_route(FAKE, 100, 0, 0, FAKE, FAKE, FAKE, b.value, None) == mq.MQ_ERR_INVALID
    assert lib.mq_route(FAKE, 100, 8, 0, FAKE, FAKE, FAKE, 4, None) == mq.MQ_ERR_WORKSPACE
    assert lib.mq_route(None, 100, 8, 0, FAKE, FAKE, FAKE, b.value, None) == mq.MQ_ERR_INVALID
    assert lib.mq_route(FAKE, 100, 4096, 0, FAKE, FAKE, FAKE, b.value, None) == mq.MQ_ERR_UNSUPPORTED


def test_qmm_rejects():
    lib = mq.load()
    W = 1 << 16
    assert lib.mq_qmm(FAKE, 4, 128, FAKE, FAKE, FAKE, 64, 2, 64, 4, FAKE, FAKE, W, None) == mq.MQ_ERR_INVALID
    assert lib.mq_qmm(FAKE, 4, 128, FAKE, FAKE, FAKE, 48, 0, 64, 4, FAKE, FAKE, W, None) == mq.MQ_ERR_INVALID
    assert lib.mq_qmm(FAKE, 4, 128, FAKE, FAKE, FAKE, 64, 1, 64, 5, FAKE, FAKE, W, None) == mq.MQ_ERR_UNSUPPORTED
    assert lib.mq_qmm(None, 4, 128, FAKE, FAKE, FAKE, 64, 1, 64, 4, FAKE, FAKE, W, None) == mq.MQ_ERR_INVALID
    assert lib.mq_qmm(FAKE, 0, 128, FAKE, FAKE, FAKE, 64, 1, 64, 4, FAKE, None, 0, None) == mq.MQ_OK
    # the tiled path (M > 16) needs the row-sum workspace
    need = mq.mq_qmm_workspace(64, 128, 64)
    assert need == 64 * 3 * 32 * 2
    assert lib.mq_qmm(FAKE, 64, 128, FAKE, FAKE, FAKE, 64, 1, 64, 4, FAKE, None, 0, None) == mq.MQ_ERR_WORKSPACE
    assert lib.mq_qmm(FAKE, 64, 128, FAKE, FAKE, FAKE, 64, 1, 64, 4, FAKE, FAKE, need - 1, None) == mq.MQ_ERR_WORKSPACE


def _probe_lib():
    lib = ctypes.CDLL(PROBE_LIB)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mq_probe_stream.restype = ctypes.c_int
    lib.mq_probe_stream.argtypes = [P, I64, P, I32, P]
    lib.mq_probe_mfma.restype = ctypes.c_int
    lib.mq_probe_mfma.argtypes = [I32, P, I32, P]
    return lib


def test_probe_library_is_separate_and_exports_its_header():
    probe_names = declared_functions(PROBE_HEADER)
    assert probe_names == ["mq_probe_mfma", "mq_probe_stream"]
    lib = _probe_lib()
    for name in probe_names:
        assert hasattr(lib, name), name
        assert name not in declared_functions()
        assert not hasattr(mq.load(), name), f"{name} is in the product library"


def test_probes_reject():
    lib = _probe_lib()
    INVALID = mq.MQ_ERR_INVALID
    assert lib.mq_probe_stream(None, 1024, FAKE, 8, None) == INVALID
    assert lib.mq_probe_stream(FAKE, 1000, FAKE, 8, None) == INVALID     # not a multiple of 16
    assert lib.mq_probe_stream(FAKE + 8, 1024, FAKE, 8, None) == INVALID  # misaligned
    assert lib.mq_probe_stream(FAKE, 1024, FAKE, 0, None) == INVALID
    assert lib.mq_probe_mfma(0, FAKE, 8, None) == INVALID
    assert lib.mq_probe_mfma(4, None, 8, None) == INVALID
    assert lib.mq_probe_mfma(4, FAKE, 0, None) == INVALID


def _gather_mm(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, w=FAKE, E=4, N=32, idx=FAKE, A=2, transpose=1,
             sorted_indices=0, out=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return mq.load().mq_gather_mm(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["w"], a["E"],
                                  a["N"], a["idx"], a["A"], a["transpose"], a["sorted_indices"],
                                  a["out"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(transpose=0), mq.MQ_ERR_UNSUPPORTED),
    (dict(K=96), mq.MQ_ERR_UNSUPPORTED),              # K % 64
    (dict(K=0), mq.MQ_ERR_INVALID),
    (dict(E=0), mq.MQ_ERR_INVALID),
    (dict(E=4096), mq.MQ_ERR_UNSUPPORTED),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(T=-1), mq.MQ_ERR_INVALID),
    (dict(w=None), mq.MQ_ERR_INVALID),
    (dict(idx=None), mq.MQ_ERR_INVALID),
    (dict(x=FAKE + 2), mq.MQ_ERR_INVALID),            # misaligned
    (dict(w=FAKE + 8), mq.MQ_ERR_INVALID),
    (dict(ws=None), mq.MQ_ERR_WORKSPACE),
    (dict(ws_bytes=16), mq.MQ_ERR_WORKSPACE),
    (dict(N=1 << 20, K=1 << 11), mq.MQ_ERR_UNSUPPORTED),   # one expert's weight > 2 GiB
])
def test_gather_mm_rejects_before_any_hip_call(kw, status):
    assert _gather_mm(**kw) == status


def test_gather_mm_workspace_is_routing_only():
    L = mq.mq_gather_mm_workspace(2048, 8, 1, 2048, 768, 64)
    Q = mq.mq_gather_qmm_workspace(2048, 8, 1, 2048, 768, 64)
    assert L.sums == L.total
    assert (L.offsets, L.perm, L.error, L.tiles) == (Q.offsets, Q.perm, Q.error, Q.tiles)
    assert L.total < Q.total


def _glu(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, wg=FAKE, sg=FAKE, bg=FAKE, wu=FAKE, su=FAKE, bu=FAKE,
             E=4, F=32, idx=FAKE, A=2, transpose=1, gs=64, bits=4, sorted_indices=0, act=1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return mq.load().mq_gather_qmm_glu(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["wg"], a["sg"],
                                       a["bg"], a["wu"], a["su"], a["bu"], a["E"], a["F"], a["idx"],
                                       a["A"], a["transpose"], a["gs"], a["bits"],
                                       a["sorted_indices"], a["act"], a["out"], a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(act=0), mq.MQ_ERR_UNSUPPORTED),
    (dict(act=3), mq.MQ_ERR_UNSUPPORTED),
    (dict(bits=3), mq.MQ_ERR_UNSUPPORTED),
    (dict(transpose=0, F=64), mq.MQ_ERR_UNSUPPORTED),   # the fused gate/up is forward only
    (dict(transpose=2), mq.MQ_ERR_INVALID),
    (dict(K=100), mq.MQ_ERR_INVALID),
    (dict(wu=None), mq.MQ_ERR_INVALID),
    (dict(su=None), mq.MQ_ERR_INVALID),
    (dict(bg=None), mq.MQ_ERR_INVALID),
    (dict(wu=FAKE + 4), mq.MQ_ERR_INVALID),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(ws_bytes=8), mq.MQ_ERR_WORKSPACE),
])
def test_gather_qmm_glu_rejects_before_any_hip_call(kw, status):
    assert _glu(**kw) == status


def _gather_mx(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, wq=FAKE, sc=FAKE, E=4, N=32, idx=FAKE, A=2,
             transpose=1, bits=4, sorted_indices=0, out=FAKE, ws=FAKE, ws_bytes=1 << 20,
             stream=None)
    a.update(kw)
    return mq.load().mq_gather_qmm_mx(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["wq"], a["sc"],
                                      a["E"], a["N"], a["idx"], a["A"], a["transpose"], a["bits"],
                                      a["sorted_indices"], a["out"], a["ws"], a["ws_bytes"],
                                      a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(transpose=0), mq.MQ_ERR_UNSUPPORTED),
    (dict(bits=6), mq.MQ_ERR_UNSUPPORTED),
    (dict(bits=8, transpose=0), mq.MQ_ERR_UNSUPPORTED),
    (dict(K=96), mq.MQ_ERR_UNSUPPORTED),              # K % 64 (GEMM chunk)
    (dict(K=0), mq.MQ_ERR_INVALID),
    (dict(E=0), mq.MQ_ERR_INVALID),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(wq=None), mq.MQ_ERR_INVALID),
    (dict(wq=None, bits=8), mq.MQ_ERR_INVALID),
    (dict(sc=None), mq.MQ_ERR_INVALID),
    (dict(idx=None), mq.MQ_ERR_INVALID),
    (dict(out=None), mq.MQ_ERR_INVALID),
    (dict(wq=FAKE + 4), mq.MQ_ERR_INVALID),           # misaligned
    (dict(out=FAKE + 2), mq.MQ_ERR_INVALID),
    (dict(ws=None), mq.MQ_ERR_WORKSPACE),
    (dict(ws_bytes=16), mq.MQ_ERR_WORKSPACE),
])
def test_gather_qmm_mx_rejects_before_any_hip_call(kw, status):
    assert _gather_mx(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 48, 4, FAKE, FAKE), mq.MQ_ERR_INVALID),      # cols % 32
    ((FAKE, -1, 64, 4, FAKE, FAKE), mq.MQ_ERR_INVALID),
    ((FAKE, 4, 0, 8, FAKE, FAKE), mq.MQ_ERR_INVALID),
    ((None, 4, 64, 4, FAKE, FAKE), mq.MQ_ERR_INVALID),
    ((FAKE, 4, 64, 8, FAKE, None), mq.MQ_ERR_INVALID),
    ((FAKE + 2, 4, 64, 4, FAKE, FAKE), mq.MQ_ERR_INVALID),  # misaligned
    ((FAKE, 4, 1 << 31, 4, FAKE, FAKE), mq.MQ_ERR_UNSUPPORTED),
    ((FAKE, 4, 64, 6, FAKE, FAKE), mq.MQ_ERR_UNSUPPORTED),  # bits
    ((None, 0, 64, 8, None, None), mq.MQ_OK),               # empty: nothing to do
])
def test_quantize_mx_rejects(args, status):
    assert mq.load().mq_quantize_mx(*args, None) == status


def _gather_nv(**kw):
    a = dict(x=FAKE, T=4, Ax=2, M=1, K=128, wq=FAKE, sc=FAKE, g=FAKE, E=4, N=32, idx=FAKE, A=2,
             transpose=1, sorted_indices=0, out=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return mq.load().mq_gather_qmm_nv(a["x"], a["T"], a["Ax"], a["M"], a["K"], a["wq"], a["sc"],
                                      a["g"], a["E"], a["N"], a["idx"], a["A"], a["transpose"],
                                      a["sorted_indices"], a["out"], a["ws"], a["ws_bytes"],
                                      a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(transpose=0), mq.MQ_ERR_UNSUPPORTED),
    (dict(K=96), mq.MQ_ERR_UNSUPPORTED),              # K % 64 (GEMM chunk)
    (dict(g=None), mq.MQ_ERR_INVALID),
    (dict(g=FAKE + 2), mq.MQ_ERR_INVALID),            # misaligned
    (dict(wq=None), mq.MQ_ERR_INVALID),
    (dict(sc=None), mq.MQ_ERR_INVALID),
    (dict(Ax=3), mq.MQ_ERR_INVALID),
    (dict(ws_bytes=16), mq.MQ_ERR_WORKSPACE),
])
def test_gather_qmm_nv_rejects_before_any_hip_call(kw, status):
    assert _gather_nv(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 2, 4, 24, FAKE, FAKE, FAKE), mq.MQ_ERR_INVALID),     # cols % 16
    ((FAKE, -1, 4, 64, FAKE, FAKE, FAKE), mq.MQ_ERR_INVALID),
    ((FAKE, 2, 4, 64, FAKE, FAKE, None), mq.MQ_ERR_INVALID),
    ((FAKE, 2, 4, 64, FAKE + 4, FAKE, FAKE), mq.MQ_ERR_INVALID),  # misaligned wq
    ((FAKE, 2, 4, 1 << 31, FAKE, FAKE, FAKE), mq.MQ_ERR_UNSUPPORTED),
    ((None, 0, 4, 64, None, None, None), mq.MQ_OK),               # empty
])
def test_quantize_nv_rejects(args, status):
    assert mq.load().mq_quantize_nv(*args, None) == status
