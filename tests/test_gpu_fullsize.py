"""GPU parity at full size, element by element over the whole output.

The reference for a routed product is built per expert: the rows routed to
expert e are multiplied by expert e's dequantised weight with ``oracle.qmm``
(pinned against ``oracle.gather_qmm`` by the all-indices-equal check), then
scattered back to their (token, slot) positions with ``oracle.route``.  That
is the oracle's own arithmetic, one fp64 product per expert instead of one
per pair, so the whole output of the pages' prefill microbenchmark and of the
Mixtral-shaped projections can be checked.

Also here: the tiled GEMM beyond one correction window (K > 32 groups) for
the plain projection at every tile height, and a decode step whose rows are
too long for the small-M kernel to route in LDS.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_torch, bf16_u16_to_f64, check_gate, i32_to_torch, torch_bf16_to_u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def reference_by_expert(case, owq, os_, ob, gs, bits, transpose=True):
    """fp64 [T*A*M, N]: every routed row times its expert's dequantised weight
    (oracle.qmm per expert), placed at its pair's output rows."""
    T, A, M, K = case.T, case.A, case.M, case.K
    counts, offsets, perm = oracle.route(case.idx, case.E)
    x = case.x
    N = owq.shape[1] if transpose else owq.shape[2] * (32 // bits)
    ref = np.empty((T * A * M, N), dtype=np.float64)
    for e in range(case.E):
        pairs = perm[offsets[e]:offsets[e + 1]]
        if pairs.size == 0:
            continue
        t, a = pairs // A, pairs % A
        xa = a if case.Ax == A else np.zeros_like(a)
        rows = x[t, xa].reshape(-1, K)                             # [pairs * M, K]
        y = oracle.qmm(rows, owq[e], os_[e], ob[e], gs, bits, transpose=transpose)
        dst = (pairs[:, None] * M + np.arange(M)[None, :]).reshape(-1)
        ref[dst] = y
    return ref


def gpu_gather(case, dev, gs, bits, weights=None):
    mq = _mq()
    if weights is None:
        weights = mq.mq_quantize(bf16_to_torch(case.w, dev), gs, bits)
    out = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), *weights, i32_to_torch(case.idx, dev),
                           True, gs, bits, False)
    torch.cuda.synchronize()
    return bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, out.shape[-1])


def test_prefill_gather_full_output(dev):
    """The pages' microbenchmark (T=2048, top-8 of 64 experts, K=2048,
    N=768, 4-bit gs64) in the launch configuration bench.py times: every one
    of the 12,582,912 outputs against the oracle."""
    case = workloads.prefill_microbench(0)
    _say("prefill gather_qmm, full output")
    out = gpu_gather(case, dev, 64, 4)
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    check_gate(out, reference_by_expert(case, owq, os_, ob, 64, 4), "prefill full output")


def test_prefill_dense_control_full_output(dev):
    """The equal-FLOPs dense control x [16384, 2048] x one quantised
    [768, 2048], whole output."""
    x, w = workloads.prefill_dense_control(0)
    _say("dense control, full output")
    mq = _mq()
    wq, s, b = mq.mq_quantize(bf16_to_torch(w, dev), 64, 4)
    out = mq.mq_qmm(bf16_to_torch(x, dev), wq, s, b, True, 64, 4)
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(w, 64, 4)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle.qmm(x, owq, os_, ob, 64, 4),
               "dense control full output")


@pytest.mark.parametrize("proj", ["up", "down"])
def test_mixtral_projection_full_output(dev, proj):
    """The Mixtral-shaped projections (E=8, top-2, T=2048, Zipf(1.2) routing,
    W ~ N(0, 0.02)): up K=4096 -> N=14336 and down K=14336 -> N=4096 (the
    latter walks 7 correction windows), whole output."""
    case = workloads.mixtral_ffn(0, 1.2, proj)
    _say(f"Mixtral-shaped {proj} projection, full output")
    out = gpu_gather(case, dev, 64, 4)
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    check_gate(out, reference_by_expert(case, owq, os_, ob, 64, 4), f"mixtral {proj}")


# K beyond one window of 32 groups on the tiled GEMM (the small-M path is
# switched off: 16 rows per expert would otherwise take it).
LONG_K = [(4096, 4, 64), (14336, 4, 64), (2048, 8, 32), (4096, 8, 32)]


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
@pytest.mark.parametrize("K,bits,gs", LONG_K, ids=[f"K{k}-{b}bit-gs{g}" for k, b, g in LONG_K])
def test_tiled_gemm_many_windows(dev, bm, K, bits, gs, monkeypatch):
    monkeypatch.setenv("MQ_SMALL_M", "0")
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case = workloads.gather_case("long-k", 40, 2, 5, K, 96, seed=61, bits=bits, group_size=gs)
    _say(f"tiled GEMM K={K} bits={bits} gs={gs} BM={bm}")
    out = gpu_gather(case, dev, gs, bits)
    owq, os_, ob = oracle.quantize(case.w, gs, bits)
    ref = oracle.gather_qmm(case.x, owq, os_, ob, case.idx, gs, bits).reshape(-1, case.N)
    check_gate(out, ref, f"K={K} bits={bits} gs={gs} BM={bm}")


@pytest.mark.parametrize("gs", [32, 64])
def test_decode_long_rows_route_separately(dev, gs):
    """A top-8 decode step over 128 experts at K = 14336: K / group_size is
    past what the small-M kernel can route in LDS, so the routing takes its
    own launch and the small-M kernel reads it."""
    case = workloads.gather_case("decode-long-k", 4, 8, 128, 14336, 96, seed=62, group_size=gs)
    _say(f"decode K=14336 gs={gs}")
    out = gpu_gather(case, dev, gs, 4)
    owq, os_, ob = oracle.quantize(case.w, gs, 4)
    ref = oracle.gather_qmm(case.x, owq, os_, ob, case.idx, gs, 4).reshape(-1, case.N)
    check_gate(out, ref, f"decode K=14336 gs={gs}")


# Tiles of 64 or 128 rows with three or four 16-column blocks per wave (192
# or 256 columns), on ragged N and on segments whose last tile fills 1, 2,
# 3..4 and 5..8 of its row blocks, with tail tiles (a segment's last rows, up
# to half a tile, in a tile of 32 or 64 rows) off and forced on.  4-bit codes
# in groups of 64, the format that has both widths.
TILE_SHAPES = [
    # name, T, A, E, K, N, routing
    ("ragged-N-200", 150, 4, 5, 256, 200, "uniform"),
    ("N-100", 120, 2, 3, 128, 100, "uniform"),
    ("N-8", 96, 2, 2, 192, 8, "uniform"),
    ("N-576-zipf", 200, 4, 6, 320, 576, "zipf"),
    ("N-1000-long-K", 64, 4, 4, 2560, 1000, "uniform"),
]


@pytest.mark.parametrize("tails", ["0", "1"])
@pytest.mark.parametrize("cols", ["3", "4"])
@pytest.mark.parametrize("bm", ["64", "128"])
@pytest.mark.parametrize("name,T,A,E,K,N,routing", TILE_SHAPES, ids=[t[0] for t in TILE_SHAPES])
def test_tile_widths_and_partial_tiles(dev, name, T, A, E, K, N, routing, bm, cols, tails,
                                       monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    monkeypatch.setenv("MQ_FORCE_COLS", cols)
    monkeypatch.setenv("MQ_TAIL_TILES", tails)
    case = workloads.gather_case(name, T, A, E, K, N, seed=63, routing=routing, zipf_s=2.0)
    counts = np.bincount(case.idx.reshape(-1), minlength=E)
    _say(f"tile widths {name} BM={bm} col blocks={cols} tails={tails} rows per expert {counts.tolist()}")
    out = gpu_gather(case, dev, 64, 4)
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    ref = oracle.gather_qmm(case.x, owq, os_, ob, case.idx, 64, 4).reshape(-1, N)
    check_gate(out, ref, f"{name} BM={bm} cols={cols} tails={tails}")


@pytest.mark.parametrize("tails", ["0", "1"])
@pytest.mark.parametrize("cols", ["3", "4"])
@pytest.mark.parametrize("M", [70, 130, 300, 400])
def test_dense_tile_widths(dev, M, cols, tails, monkeypatch):
    """The dense product (one weight, identity rows) on both tile widths, with
    a last tile of 6, 2, 44 and 16 rows (tail tiles off and forced on)."""
    monkeypatch.setenv("MQ_FORCE_COLS", cols)
    monkeypatch.setenv("MQ_TAIL_TILES", tails)
    x, w = workloads.small_m_dense(M, 392, 512, seed=M)
    mq = _mq()
    wq, s, b = mq.mq_quantize(bf16_to_torch(w, dev), 64, 4)
    out = mq.mq_qmm(bf16_to_torch(x, dev), wq, s, b, True, 64, 4)
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(w, 64, 4)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle.qmm(x, owq, os_, ob, 64, 4),
               f"dense M={M} cols={cols} tails={tails}")


@pytest.mark.parametrize("group", ["0", "1", "4", "8"])
def test_column_tile_groups(dev, group, monkeypatch):
    """The tile order in groups of column tiles (the last group partial: 9
    column tiles of 256) and with tail tiles forced on: the whole output
    against the oracle, identical bits for every grouping."""
    monkeypatch.setenv("MQ_COL_GROUP", group)
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    case = workloads.gather_case("col-groups", 300, 2, 6, 256, 2304, seed=64, routing="zipf", zipf_s=1.5)
    _say(f"column tile groups of {group}")
    out = gpu_gather(case, dev, 64, 4)
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    ref = oracle.gather_qmm(case.x, owq, os_, ob, case.idx, 64, 4).reshape(-1, case.N)
    check_gate(out, ref, f"column tile groups of {group}")
    monkeypatch.setenv("MQ_COL_GROUP", "0")
    assert np.array_equal(out, gpu_gather(case, dev, 64, 4))
