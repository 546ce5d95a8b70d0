"""Every compiled kernel instance is dispatched, and its output checked.

With MQ_LOG=1 each kernel launch writes "[mq-dispatch] kernel<p0,p1,...>"
to stderr, naming the template instance it launched.  Each test below drives
one kernel family through the public calls, on small seeded shapes, until
every instance its launch table compiles has run (tile heights via
MQ_FORCE_BM, tile widths via MQ_FORCE_COLS, the small-M kernel's waves,
column blocks and column split via MQ_SMALL_WAVES / MQ_SMALL_COLS /
MQ_SMALL_COLSPLIT), checks each result against the oracle (bit-exact for
codes and routing, the tolerance gate for products), and then compares the
instances seen with the full list.  The lists are written out here from the
launch tables: an instance that no call reaches, or a launch of one that is
not listed, fails the test.
"""
import itertools
import re

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (bf16_to_torch, bf16_u16_to_f64, check_gate, i32_to_torch,
                      torch_bf16_to_u16, torch_to_u32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_LINE = re.compile(r"^\[mq-dispatch\] (\w+)<([-\d,]*)>$")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_grouped_amd as mq
    mq.load()                       # fail loudly if the library is missing
    return torch.device("cuda:0")


def _mq():
    import quantized_moe_grouped_amd as mq
    return mq


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def dispatched(text):
    """The set of (kernel, params) named by the dispatch lines in `text`."""
    seen = set()
    for line in text.splitlines():
        m = _LINE.match(line.strip())
        if m:
            seen.add((m.group(1), tuple(int(v) for v in m.group(2).split(",") if v)))
    return seen


def check_instances(capfd, kernel, expected):
    seen = {p for k, p in dispatched(capfd.readouterr().err) if k == kernel}
    missing = sorted(expected - seen)
    unknown = sorted(seen - expected)
    assert not missing, f"{kernel}: instances never dispatched: {missing}"
    assert not unknown, f"{kernel}: dispatched instances not in the launch table: {unknown}"


@pytest.fixture
def logged(monkeypatch):
    monkeypatch.setenv("MQ_LOG", "1")
    return monkeypatch


def _env(mp, **kv):
    """Set (value) or clear (None) each of the test hooks."""
    for k, v in kv.items():
        if v is None:
            mp.delenv(k, raising=False)
        else:
            mp.setenv(k, str(v))


def _out(t):
    return bf16_u16_to_f64(torch_bf16_to_u16(t))


# --- the tiled GEMM: BM x bits x group size x GLU with four column blocks per
# wave (NW = 2 waves for 16-row tiles, else 4), and three column blocks for
# 64/128-row tiles of 4-bit codes in groups of 64 (not fused gate/up) ---------

GEMM_INSTANCES = {(bm, bits, gs, 2 if bm == 16 else 4, glu, 4)
                  for bm, bits, gs, glu in itertools.product((16, 32, 64, 128), (4, 8), (32, 64), (0, 1))}
GEMM_INSTANCES |= {(64, 4, 64, 4, 0, 3), (128, 4, 64, 4, 0, 3)}


def test_every_gemm_instance(dev, logged, capfd):
    mq = _mq()
    for bm, bits, gs in itertools.product((16, 32, 64, 128), (4, 8), (32, 64)):
        case = workloads.gather_case("cov-gemm", 64, 2, 4, 256, 200, seed=bm + bits + gs)
        up = workloads.gather_case("cov-gemm-up", 64, 2, 4, 256, 200, seed=bm + bits + gs + 1).w
        owq = oracle.quantize(case.w, gs, bits)
        ref = oracle.gather_qmm(case.x, *owq, case.idx, gs, bits)
        x, idx = bf16_to_torch(case.x, dev), i32_to_torch(case.idx, dev)
        gate = mq.mq_quantize(bf16_to_torch(case.w, dev), gs, bits)
        widths = ("3", "4") if bm >= 64 and bits == 4 and gs == 64 else ("4",)
        for cols in widths:
            _env(logged, MQ_FORCE_BM=bm, MQ_FORCE_COLS=cols)
            _say(f"gather_gemm BM={bm} bits={bits} gs={gs} col blocks={cols}")
            out = mq.mq_gather_qmm(x, *gate, idx, True, gs, bits, False)
            torch.cuda.synchronize()
            check_gate(_out(out), ref, f"gemm BM={bm} bits={bits} gs={gs} cols={cols}")
        _env(logged, MQ_FORCE_BM=bm, MQ_FORCE_COLS=None)
        _say(f"gather_gemm GLU BM={bm} bits={bits} gs={gs}")
        upq = mq.mq_quantize(bf16_to_torch(up, dev), gs, bits)
        out = mq.mq_gather_qmm_glu(x, gate, upq, idx, 1, True, gs, bits, False)
        torch.cuda.synchronize()
        check_gate(_out(out), oracle.gather_qmm_glu(case.x, owq, oracle.quantize(up, gs, bits),
                                                    case.idx, gs, bits, 1),
                   f"glu BM={bm} bits={bits} gs={gs}")
    check_instances(capfd, "gather_gemm", GEMM_INSTANCES)


# --- the untransposed product: BM x bits ---------------------------------------

NN_INSTANCES = set(itertools.product((16, 32, 64, 128), (4, 8)))


def test_every_nn_instance(dev, logged, capfd):
    mq = _mq()
    for bits, gs in ((4, 64), (8, 32)):
        case = workloads.gather_case("cov-nn", 96, 2, 4, 192, 256, seed=bits)
        w = np.ascontiguousarray(case.w.transpose(0, 2, 1))           # [E, K=192, N=256]
        ref = oracle.gather_qmm(case.x, *oracle.quantize(w, gs, bits), case.idx, gs, bits,
                                transpose=False)
        wq = mq.mq_quantize(bf16_to_torch(w, dev), gs, bits)
        for bm in (16, 32, 64, 128):
            _env(logged, MQ_FORCE_BM=bm)
            _say(f"gather_nn BM={bm} bits={bits}")
            out = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), *wq, i32_to_torch(case.idx, dev),
                                   False, gs, bits, False)
            torch.cuda.synchronize()
            check_gate(_out(out), ref, f"nn BM={bm} bits={bits}")
    check_instances(capfd, "gather_nn", NN_INSTANCES)


# --- the bf16 routed product: BM (NW = 2 waves for 16-row tiles, else 4) -------

MM_INSTANCES = {(16, 2), (32, 4), (64, 4), (128, 4)}


def test_every_mm_instance(dev, logged, capfd):
    mq = _mq()
    case = workloads.gather_case("cov-mm", 96, 2, 4, 192, 200, seed=5)
    ref = oracle.gather_mm(case.x, case.w, case.idx)
    for bm in (16, 32, 64, 128):
        _env(logged, MQ_FORCE_BM=bm)
        _say(f"gather_mm BM={bm}")
        out = mq.mq_gather_mm(bf16_to_torch(case.x, dev), bf16_to_torch(case.w, dev),
                              i32_to_torch(case.idx, dev), True, False)
        torch.cuda.synchronize()
        check_gate(_out(out), ref, f"mm BM={bm}")
    check_instances(capfd, "gather_mm", MM_INSTANCES)


# --- the microscaled products: BM x {MXFP4, MXFP8, NVFP4} x {wide scale loads
# (K % 128 == 0), one scale per load} ------------------------------------------

MX_INSTANCES = {(bm, 2 if bm == 16 else 4, bits, wide, nv)
                for bm in (16, 32, 64, 128)
                for bits, nv in ((4, 0), (8, 0), (4, 1))
                for wide in (0, 1)}


def test_every_mx_instance(dev, logged, capfd):
    mq = _mq()
    elem = {4: "e2m1", 8: "e4m3"}
    for K in (320, 512):                 # a half pair of blocks at the end; whole pairs
        case = workloads.gather_case("cov-mx", 96, 2, 4, K, 200, seed=K)
        x, idx = bf16_to_torch(case.x, dev), i32_to_torch(case.idx, dev)
        for bits in (4, 8):
            wq, sc = mq.mq_quantize_mx(bf16_to_torch(case.w, dev), bits)
            owq, osc = oracle.quantize_mx(case.w, elem[bits])
            assert np.array_equal(torch_to_u32(wq), owq) and np.array_equal(sc.cpu().numpy(), osc)
            ref = oracle.gather_qmm_mx(case.x, owq, osc, case.idx, elem[bits])
            for bm in (16, 32, 64, 128):
                _env(logged, MQ_FORCE_BM=bm)
                _say(f"gather_mx K={K} bits={bits} BM={bm}")
                out = mq.mq_gather_qmm_mx(x, wq, sc, idx, True, False, bits=bits)
                torch.cuda.synchronize()
                check_gate(_out(out), ref, f"mx K={K} bits={bits} BM={bm}")
        wq, sc, g = mq.mq_quantize_nv(bf16_to_torch(case.w, dev))
        owq, osc, og = oracle.quantize_nv(case.w)
        assert np.array_equal(torch_to_u32(wq), owq) and np.array_equal(sc.cpu().numpy(), osc)
        ref = oracle.gather_qmm_nv(case.x, owq, osc, og, case.idx)
        for bm in (16, 32, 64, 128):
            _env(logged, MQ_FORCE_BM=bm)
            _say(f"gather_nv K={K} BM={bm}")
            out = mq.mq_gather_qmm_nv(x, wq, sc, g, idx, True, False)
            torch.cuda.synchronize()
            check_gate(_out(out), ref, f"nv K={K} BM={bm}")
    check_instances(capfd, "gather_mx", MX_INSTANCES)


# --- the small-M kernel: bits x group size x column blocks per wave (two for
# 4-bit codes only) x rows per tile (1, 2, 4, 8; the routing folded in: 4, 8)
# x {column split (4 waves), 4/8/16 waves over K}, plus the large scale block
# (K / group_size > 256; one column block, 4 or 8 waves, routing not folded).
# Parameters: <BITS, GS, waves, NT, TR, scale block bytes, column split, folded>

SCALE_BLOCK = {1: 8192, 2: 4096}
SPLIT_BLOCK = 8192          # the column split's blocks, one or two column blocks per wave
LARGE_BLOCK = 32768


def small_m_instances():
    out = set()
    for bits, gs in itertools.product((4, 8), (32, 64)):
        for nt in ((1, 2) if bits == 4 else (1,)):
            scb = SCALE_BLOCK[nt]
            for fr, trs in ((0, (1, 2, 4, 8)), (1, (4, 8))):
                for tr in trs:
                    out.add((bits, gs, 4, nt, tr, SPLIT_BLOCK, 1, fr))
                    for kw in (4, 8, 16):
                        out.add((bits, gs, kw, nt, tr, scb, 0, fr))
                    if nt == 1 and not fr:
                        for kw in (4, 8):
                            out.add((bits, gs, kw, nt, tr, LARGE_BLOCK, 0, 0))
    return out


SMALL_M_INSTANCES = small_m_instances()
assert len(SMALL_M_INSTANCES) == 176


def _steps_k(bits, gs, steps):
    """K giving `steps` steps of the small-M kernel (128 columns of K per
    step for 4-bit codes in groups of 64, else 64)."""
    return steps * (128 if bits == 4 and gs == 64 else 64)


def _dense_small(mq, dev, M, K, N, gs, bits, seed, what):
    x, w = workloads.small_m_dense(M, N, K, seed=seed)
    wq = mq.mq_quantize(bf16_to_torch(w, dev), gs, bits)
    out = mq.mq_qmm(bf16_to_torch(x, dev), *wq, True, gs, bits)
    torch.cuda.synchronize()
    check_gate(_out(out), oracle.qmm(x, *oracle.quantize(w, gs, bits), gs, bits), what)


def _routed_small(mq, dev, T, E, K, N, gs, bits, seed, what):
    # top-2: 4 tokens over E = 16 (0.5 rows per expert) give 4-row tiles,
    # 12 tokens over E = 4 (6 rows) 8-row ones
    case = workloads.gather_case("cov-small", T, 2, E, K, N, seed=seed)
    wq = mq.mq_quantize(bf16_to_torch(case.w, dev), gs, bits)
    out = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), *wq, i32_to_torch(case.idx, dev), True,
                           gs, bits, False)
    torch.cuda.synchronize()
    check_gate(_out(out), oracle.gather_qmm(case.x, *oracle.quantize(case.w, gs, bits), case.idx,
                                            gs, bits), what)


@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (8, 32), (8, 64)])
def test_every_small_m_instance(dev, logged, capfd, bits, gs):
    mq = _mq()
    N = 80                                  # ragged for every column block width
    K_cs = 256                              # short rows: the column split fits
    K_kw = _steps_k(bits, gs, 32)           # 2 steps for each of 16 waves
    K_large = 288 * gs                      # 288 groups: the large scale block
    _env(logged, MQ_SMALL_M=1, MQ_FUSE_ROUTE=None)
    for nt in ((1, 2) if bits == 4 else (1,)):
        for split, kws in ((1, (4,)), (0, (4, 8, 16))):
            for kw in kws:
                _env(logged, MQ_SMALL_COLS=nt, MQ_SMALL_WAVES=kw, MQ_SMALL_COLSPLIT=split)
                K = K_cs if split else K_kw
                tag = f"bits={bits} gs={gs} NT={nt} waves={kw} split={split} K={K}"
                for M in (1, 2, 4, 8):
                    _say(f"small_m dense M={M} {tag}")
                    _dense_small(mq, dev, M, K, N, gs, bits, M + kw, f"dense M={M} {tag}")
                for T, E in ((4, 16), (12, 4)):
                    _say(f"small_m routed (folded) T={T} E={E} {tag}")
                    _routed_small(mq, dev, T, E, K, N, gs, bits, E + kw, f"routed E={E} {tag}")
    # the large scale block: one column block, no column split, 4 or 8 waves
    for kw in (4, 8):
        _env(logged, MQ_SMALL_COLS=1, MQ_SMALL_WAVES=kw, MQ_SMALL_COLSPLIT=0)
        for M in (1, 2, 4, 8):
            tag = f"large scale block bits={bits} gs={gs} waves={kw} K={K_large} M={M}"
            _say(f"small_m {tag}")
            _dense_small(mq, dev, M, K_large, N, gs, bits, M + 7 * kw, tag)
    expected = {p for p in SMALL_M_INSTANCES if p[0] == bits and p[1] == gs}
    check_instances(capfd, "small_m", expected)


# --- quantisers and routing ---------------------------------------------------

def test_every_quantizer_instance(dev, logged, capfd):
    mq = _mq()
    rng = np.random.default_rng(17)
    w = workloads.bf16_bits_from_f32(rng.standard_normal((3, 64, 256)).astype(np.float32))
    wt = bf16_to_torch(w, dev)
    for bits, gs in ((4, 64), (8, 32)):
        _say(f"quantize bits={bits} gs={gs}")
        got = mq.mq_quantize(wt, gs, bits)
        torch.cuda.synchronize()
        want = oracle.quantize(w, gs, bits)
        assert np.array_equal(torch_to_u32(got[0]), want[0])
        assert np.array_equal(torch_bf16_to_u16(got[1]), want[1])
        assert np.array_equal(torch_bf16_to_u16(got[2]), want[2])
    for bits, elem in ((4, "e2m1"), (8, "e4m3")):
        _say(f"quantize_mx bits={bits}")
        wq, sc = mq.mq_quantize_mx(wt, bits)
        torch.cuda.synchronize()
        owq, osc = oracle.quantize_mx(w, elem)
        assert np.array_equal(torch_to_u32(wq), owq) and np.array_equal(sc.cpu().numpy(), osc)
    _say("quantize_nv")
    wq, sc, g = mq.mq_quantize_nv(wt)
    torch.cuda.synchronize()
    owq, osc, og = oracle.quantize_nv(w)
    assert np.array_equal(torch_to_u32(wq), owq) and np.array_equal(sc.cpu().numpy(), osc)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
    seen = dispatched(capfd.readouterr().err)
    assert {(k, p) for k, p in seen if k in ("quantize", "quantize_mx", "nv_gscale", "nv_quant")} == {
        ("quantize", (4,)), ("quantize", (8,)), ("quantize_mx", (4,)), ("quantize_mx", (8,)),
        ("nv_gscale", ()), ("nv_quant", ())}


def test_every_route_instance(dev, logged, capfd):
    """One routing workgroup counts its own chunk; more than one take a
    counting launch first.  Up to 256 experts the scatter keeps 257 bins in
    LDS, beyond that 2049."""
    mq = _mq()
    for n_tok, E in ((100, 64), (700, 64), (100, 300), (700, 1500)):
        rng = np.random.default_rng(n_tok + E)
        idx = rng.integers(0, E, size=(n_tok, 2), dtype=np.int32)
        _say(f"route pairs={idx.size} E={E}")
        perm, offsets = mq.mq_route(i32_to_torch(idx.reshape(-1), dev), E)
        torch.cuda.synchronize()
        _, ooff, operm = oracle.route(idx, E)
        assert np.array_equal(offsets.cpu().numpy(), ooff)
        assert np.array_equal(perm.cpu().numpy(), operm)
    seen = dispatched(capfd.readouterr().err)
    assert {(k, p) for k, p in seen if k.startswith("route_")} == {
        ("route_count", ()), ("route_scatter", (257,)), ("route_scatter", (2049,))}
