"""GPU parity: the HIP path (through the C ABI) against the oracle, element by
element on the same seeded inputs.

Integer and byte results (codes, scales, biases, permutation, offsets, error
word) must be bit-exact; bf16 outputs must pass the gate in ``gpu_util``.
"""
import os
import zlib

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (bf16_to_torch, bf16_u16_to_f64, check_gate, i32_to_torch, torch_bf16_to_u16,
                      torch_to_u32, u32_to_torch)

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


def gpu_quantize(w_u16, gs, bits, dev):
    wq, s, b = _mq().mq_quantize(bf16_to_torch(w_u16, dev), gs, bits)
    return wq, s, b


def run_gather(case, dev, gs=None, bits=None, weights=None, sorted_hint=None, ret_ws=False):
    gs = gs or case.group_size
    bits = bits or case.bits
    if weights is None:
        weights = gpu_quantize(case.w, gs, bits, dev)
    wq, s, b = weights
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    hint = case.sorted_indices if sorted_hint is None else sorted_hint
    res = _mq().mq_gather_qmm(x, wq, s, b, idx, True, gs, bits, hint, return_workspace=ret_ws)
    torch.cuda.synchronize()
    return res


def oracle_gather(case, gs=None, bits=None):
    gs = gs or case.group_size
    bits = bits or case.bits
    wq, s, b = oracle.quantize(case.w, gs, bits)
    return oracle.gather_qmm(case.x, wq, s, b, case.idx, gs, bits)


# --- quantize -----------------------------------------------------------------------

def _special_weights():
    rng = np.random.default_rng(5)
    w = workloads.bf16_bits_from_f32(rng.standard_normal((6, 256)).astype(np.float32))
    w[0, :64] = workloads.bf16_bits_from_f32(np.float32(1.5))           # constant group
    w[1, :32] = 0x8000                                                  # -0.0 group
    w[1, 32:64] = 0
    w[2, 64:128] = workloads.bf16_bits_from_f32(np.linspace(-1e30, 1e30, 64).astype(np.float32))
    w[3, :] = workloads.bf16_bits_from_f32(rng.standard_normal(256).astype(np.float32) * 1e-30)
    return w


@pytest.mark.parametrize("name,shape,std,gs,bits", [
    ("tiny-4b-gs64", (8, 128, 256), 1.0, 64, 4),
    ("tiny-4b-gs32", (8, 128, 256), 1.0, 32, 4),
    ("tiny-8b-gs64", (8, 128, 256), 1.0, 64, 8),
    ("tiny-8b-gs32", (8, 128, 256), 1.0, 32, 8),
    ("small-std-4b", (4, 96, 512), 0.02, 64, 4),
    ("prefill-experts", (64, 768, 2048), 1.0, 64, 4),
])
def test_quantize_bit_exact(dev, name, shape, std, gs, bits):
    _say(f"quantize {name} {shape} gs={gs} bits={bits}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = workloads.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    owq, os_, ob = oracle.quantize(w, gs, bits)
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(torch_bf16_to_u16(s), os_)
    assert np.array_equal(torch_bf16_to_u16(b), ob)


@pytest.mark.parametrize("gs,bits", [(32, 4), (64, 8)])
def test_quantize_special_values(dev, gs, bits):
    w = _special_weights()
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    owq, os_, ob = oracle.quantize(w, gs, bits)
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(torch_bf16_to_u16(s), os_)
    assert np.array_equal(torch_bf16_to_u16(b), ob)


# --- route ---------------------------------------------------------------------------

# Pairs are routed in chunks of 1024: one chunk ("tiny", "E1") is counted by
# its routing workgroup, more by a count launch ("prefill" is exactly 16
# chunks, "17-chunks" one pair more).
ROUTE_CASES = ["tiny", "prefill", "balanced-E256", "zipf", "one-expert", "sorted", "empty",
               "many-blocks", "17-chunks", "E1", "E2048"]


def _route_input(name):
    """Index arrays only (drawn lazily: collection stays cheap)."""
    rng = np.random.default_rng(11)
    if name == "tiny":
        return workloads.tiny_moe(0).idx, 8
    if name == "prefill":
        return np.random.default_rng(np.random.SeedSequence(0).spawn(4)[3]).integers(
            0, 64, (2048, 8)).astype(np.int32), 64
    if name == "balanced-E256":
        return workloads.gather_case("r", 512, 8, 256, 64, 8, 0, routing="balanced").idx, 256
    if name == "zipf":
        return workloads.gather_case("z", 2048, 2, 8, 64, 8, 0, routing="zipf").idx, 8
    if name == "one-expert":
        return np.full((300, 4), 3, np.int32), 5
    if name == "sorted":
        return np.sort(rng.integers(0, 32, 5000)).astype(np.int32).reshape(-1, 1), 32
    if name == "empty":
        return np.zeros((0, 8), np.int32), 16
    if name == "many-blocks":
        return rng.integers(0, 128, (9000, 8)).astype(np.int32), 128
    if name == "17-chunks":
        return rng.integers(0, 37, 16385).astype(np.int32).reshape(-1, 1), 37
    if name == "E1":
        return np.zeros((77, 3), np.int32), 1
    if name == "E2048":
        return rng.integers(0, 2048, (3000, 2)).astype(np.int32), 2048
    raise KeyError(name)


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_bit_exact(dev, name):
    idx, E = _route_input(name)
    _say(f"route {name} n={idx.size} E={E}")
    perm, offsets = _mq().mq_route(i32_to_torch(idx.reshape(-1), dev), E)
    torch.cuda.synchronize()
    _, ooff, operm = oracle.route(idx, E)
    assert np.array_equal(offsets.cpu().numpy(), ooff)
    assert np.array_equal(perm.cpu().numpy(), operm)


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
@pytest.mark.parametrize("T,A,E,M,routing", [(300, 4, 16, 1, "zipf"), (150, 2, 9, 3, "uniform"),
                                             (40, 8, 300, 1, "uniform"), (1, 1, 5, 1, "uniform")])
def test_tile_tables(dev, bm, T, A, E, M, routing, monkeypatch):
    """The routing's three tile tables (ceil(r/h), floor(r/h) + [r % h > t],
    [0 < r % h <= t] prefixes over the experts' rows r, t = h/2 for h >= 64)
    match the oracle's segment counts exactly."""
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case = workloads.gather_case("tile-tables", T, A, E, 64, 64, seed=T + E, routing=routing, zipf_s=1.5)
    ws = _mq().mq_gather_route(i32_to_torch(case.idx, dev), E, M)
    torch.cuda.synchronize()
    L = _mq().mq_gather_qmm_workspace(T, A, M, 64, 0, E, 64, 4)
    h = int(ws[L.error + 4:L.error + 8].view(torch.int32).item())
    assert h == int(bm)
    tabs = ws[L.tiles:L.tiles + 4 * 3 * (E + 1)].view(torch.int32).cpu().numpy().reshape(3, E + 1)
    counts, _, _ = oracle.route(case.idx, E)
    r = counts.astype(np.int64) * M
    t = h // 2 if h >= 64 else 0
    rest = r % h
    want = [-(-r // h), r // h + (rest > t), (rest > 0) & (rest <= t)]
    for k in range(3):
        assert np.array_equal(tabs[k], np.concatenate([[0], np.cumsum(want[k])])), k


def test_route_out_of_range_goes_last(dev):
    idx = np.array([3, 9, 0, -1, 3, 2, 7, 1], np.int32)       # E = 4: 9, -1, 7 are out of range
    perm, offsets = _mq().mq_route(i32_to_torch(idx, dev), 4)
    torch.cuda.synchronize()
    valid = np.where((idx >= 0) & (idx < 4))[0]
    _, ooff, operm = oracle.route(idx[valid], 4)
    off = offsets.cpu().numpy()
    p = perm.cpu().numpy()
    assert np.array_equal(off, ooff)
    assert np.array_equal(p[:off[4]], valid[operm])
    assert list(p[off[4]:]) == [1, 3, 6]


def test_route_any_workspace_content_and_reuse(dev):
    """Routing is bit-exact whatever the workspace held before the first call
    (zeros, all ones, ascending words) and on calls in a row with one
    workspace and different n (one chunk of 1024 pairs and several)."""
    mq = _mq()
    lib = mq.load()
    rng = np.random.default_rng(23)
    E = 48
    sizes = (20000, 3000, 64 * 1024, 1025)
    wsb = max(mq.mq_route_workspace(n, E) for n in sizes)
    fills = [torch.zeros(wsb, dtype=torch.uint8),
             torch.full((wsb,), 0xFF, dtype=torch.uint8),
             torch.arange(wsb // 4, dtype=torch.int32).view(torch.uint8)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    for f, fill in enumerate(fills):
        ws = fill.to(dev)
        for n in sizes:
            idx = rng.integers(0, E, n).astype(np.int32)
            _say(f"route workspace fill {f} n={n} E={E}")
            it = i32_to_torch(idx, dev)
            perm = torch.empty(n, dtype=torch.int32, device=dev)
            off = torch.empty(E + 1, dtype=torch.int32, device=dev)
            st = lib.mq_route(it.data_ptr(), n, E, 0, perm.data_ptr(), off.data_ptr(),
                              ws.data_ptr(), wsb, stream)
            assert st == mq.MQ_OK, mq.mq_status_str(st)
            torch.cuda.synchronize()
            _, ooff, operm = oracle.route(idx, E)
            assert np.array_equal(off.cpu().numpy(), ooff), (f, n)
            assert np.array_equal(perm.cpu().numpy(), operm), (f, n)


# --- gather_qmm ------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 32), (8, 64), (8, 32)])
def test_gather_tiny(dev, seed, bits, gs):
    case = workloads.tiny_moe(seed)
    _say(f"gather tiny seed={seed} bits={bits} gs={gs}")
    out = run_gather(case, dev, gs, bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case, gs, bits), "tiny")


@pytest.mark.parametrize("seed", [0, 1])
def test_gather_tiny_presorted(dev, seed):
    case = workloads.tiny_moe(seed)
    sc, order = workloads.presort(case)
    _say(f"gather tiny presorted seed={seed}")
    weights = gpu_quantize(case.w, 64, 4, dev)
    out_s = torch_bf16_to_u16(run_gather(sc, dev, weights=weights))
    out_u = torch_bf16_to_u16(run_gather(case, dev, weights=weights))
    check_gate(bf16_u16_to_f64(out_s), oracle_gather(sc), "presorted")
    # the pre-sorted problem is the unsorted one permuted: identical bits
    assert np.array_equal(out_s.reshape(-1, case.N), out_u.reshape(-1, case.N)[order])
    # the hint does not change the result
    out_h = torch_bf16_to_u16(run_gather(sc, dev, weights=weights, sorted_hint=False))
    assert np.array_equal(out_h, out_s)


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
def test_gather_every_tile_height(dev, bm, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case = workloads.gather_case("bm", 200, 4, 6, 256, 192, seed=4)
    _say(f"gather forced BM={bm}")
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case), f"BM={bm}")


GATHER_SHAPES = [
    # name, T, A, E, K, N, kwargs
    ("M2-broadcast", 24, 3, 5, 128, 64, dict(M=2, Ax=1)),
    ("M3", 17, 2, 4, 192, 96, dict(M=3)),
    ("N-ragged-200", 40, 2, 4, 256, 200, {}),
    ("N-odd-100", 40, 2, 4, 128, 100, {}),
    ("N-tiny-8", 40, 2, 4, 128, 8, {}),
    ("E1", 50, 2, 1, 128, 128, {}),
    ("K64-single-chunk", 60, 2, 3, 64, 128, {}),
    ("K4096", 8, 2, 3, 4096, 64, {}),
    ("one-hot-expert", 64, 1, 1, 256, 256, {}),
    ("zipf-skewed", 128, 2, 8, 256, 128, dict(routing="zipf", zipf_s=2.5)),
    ("many-experts-short-runs", 64, 8, 256, 128, 64, dict(routing="balanced")),
]


@pytest.mark.parametrize("name,T,A,E,K,N,kw", GATHER_SHAPES, ids=[g[0] for g in GATHER_SHAPES])
def test_gather_shapes(dev, name, T, A, E, K, N, kw):
    case = workloads.gather_case(name, T, A, E, K, N, seed=7, **kw)
    _say(f"gather {name}")
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case), name)


# The correction window holds 32 groups.  A K whose group count is a
# multiple of 8 but not of 32 ends in a partial window read with 16-byte loads
# (the lanes past the last group read zeros); any other group count takes
# the per-group loads.  Every tile height, 4-bit gs64 and 8-bit gs32.
PARTIAL_WINDOWS = [
    # K, bits, group size (groups: 8, 24, 24, 5)
    (512, 4, 64), (1536, 4, 64), (768, 8, 32), (320, 4, 64),
]


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
@pytest.mark.parametrize("K,bits,gs", PARTIAL_WINDOWS, ids=[f"K{k}-{b}bit-gs{g}" for k, b, g in PARTIAL_WINDOWS])
def test_gather_partial_correction_window(dev, bm, K, bits, gs, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case = workloads.gather_case("partial-window", 96, 4, 5, K, 160, seed=29, bits=bits,
                                 group_size=gs)
    _say(f"gather partial window K={K} bits={bits} gs={gs} BM={bm}")
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case),
               f"K={K} bits={bits} gs={gs} BM={bm}")


def test_gather_empty_experts_and_empty_batch(dev):
    case = workloads.gather_case("sparse", 30, 2, 16, 128, 64, seed=8)
    case.idx = (case.idx % 3) * 5                          # only experts 0, 5, 10 used
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case), "sparse")
    empty = workloads.gather_case("empty", 0, 2, 4, 128, 64, seed=8)
    out = run_gather(empty, dev)
    assert tuple(out.shape) == (0, 2, 1, 64)


def test_gather_out_of_range_rows_zero(dev):
    case = workloads.gather_case("oob", 20, 2, 4, 128, 64, seed=9)
    bad = case.idx.copy()
    bad[3, 1] = 4
    bad[7, 0] = -2
    bad[19, 1] = 1000
    case.idx = bad
    out, ws, L = run_gather(case, dev, ret_ws=True)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, case.N)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    err = ws[L.error:L.error + 4].view(torch.int32).item()
    assert err == int((~ok).sum())
    good = workloads.GatherCase("oob-ok", case.x.reshape(40, 1, 1, 128)[ok], case.w,
                                flat[ok].reshape(-1, 1).astype(np.int32), 4)
    check_gate(o[ok].reshape(-1, 1, 1, case.N), oracle_gather(good), "valid rows")


def test_gather_deterministic(dev):
    case = workloads.gather_case("det", 300, 4, 16, 512, 256, seed=10)
    weights = gpu_quantize(case.w, 64, 4, dev)
    a = torch_bf16_to_u16(run_gather(case, dev, weights=weights))
    b = torch_bf16_to_u16(run_gather(case, dev, weights=weights))
    assert np.array_equal(a, b)


def test_gather_all_equal_matches_qmm(dev, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", "64")
    case = workloads.gather_case("eq", 96, 2, 3, 256, 128, seed=12)
    weights = gpu_quantize(case.w, 64, 4, dev)
    for e in range(3):
        case.idx = np.full_like(case.idx, e)
        g = torch_bf16_to_u16(run_gather(case, dev, weights=weights)).reshape(-1, case.N)
        wq, s, b = weights
        d = _mq().mq_qmm(bf16_to_torch(case.x.reshape(-1, case.K), dev), wq[e], s[e], b[e], True, 64, 4)
        torch.cuda.synchronize()
        assert np.array_equal(g, torch_bf16_to_u16(d))


# --- full-size prefill shape: sampled outputs + exact routing -------------------------

@pytest.fixture(scope="module")
def prefill(dev):
    _say("prefill: drawing inputs and quantising on both sides")
    case = workloads.prefill_microbench(0)
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    weights = gpu_quantize(case.w, 64, 4, dev)
    torch.cuda.synchronize()
    return case, (owq, os_, ob), weights


def _samples(case, rng, n_rand=3000, full_pairs=6):
    P = case.T * case.A
    pairs = list(rng.integers(0, P, n_rand))
    cols = list(rng.integers(0, case.N, n_rand))
    for p in rng.integers(0, P, full_pairs):
        pairs += [int(p)] * case.N
        cols += list(range(case.N))
    return np.array(pairs), np.array(cols)


def test_prefill_quantize_exact(prefill):
    case, (owq, os_, ob), (wq, s, b) = prefill
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(torch_bf16_to_u16(s), os_)
    assert np.array_equal(torch_bf16_to_u16(b), ob)


def test_prefill_routing_exact(prefill, dev):
    """The routing a full-size call used, read back from its workspace, is the
    oracle's bit for bit (the whole output is checked in test_gpu_fullsize)."""
    case, (owq, os_, ob), weights = prefill
    _say("prefill gather_qmm (full size), routing read back")
    out, ws, L = run_gather(case, dev, weights=weights, ret_ws=True)
    o = torch_bf16_to_u16(out).reshape(-1, case.N)
    assert np.isfinite(bf16_u16_to_f64(o)).all()
    _, ooff, operm = oracle.route(case.idx, case.E)
    off = ws[L.offsets:L.offsets + 4 * (case.E + 1)].view(torch.int32).cpu().numpy()
    perm = ws[L.perm:L.perm + 4 * case.idx.size].view(torch.int32).cpu().numpy()
    assert np.array_equal(off, ooff) and np.array_equal(perm, operm)
    assert ws[L.error:L.error + 4].view(torch.int32).item() == 0


def test_prefill_presorted_equals_unsorted(prefill, dev):
    case, _, weights = prefill
    sc, order = workloads.presort(case)
    a = torch_bf16_to_u16(run_gather(case, dev, weights=weights)).reshape(-1, case.N)
    b = torch_bf16_to_u16(run_gather(sc, dev, weights=weights)).reshape(-1, case.N)
    assert np.array_equal(b, a[order])


# --- dense qmm -------------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 3, 8, 16, 100, 300])
@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 32)])
def test_qmm_small(dev, M, bits, gs):
    x, w = workloads.small_m_dense(M, 384, 512, seed=M)
    _say(f"qmm M={M} bits={bits} gs={gs}")
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    out = _mq().mq_qmm(bf16_to_torch(x, dev), wq, s, b, True, gs, bits)
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(w, gs, bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle.qmm(x, owq, os_, ob, gs, bits), f"qmm M={M}")


# --- small-M path (batched decode) ---------------------------------------------------

@pytest.mark.parametrize("B,N,K,bits,gs", [
    (1, 14336, 4096, 4, 64), (8, 14336, 4096, 4, 64), (4, 4096, 14336, 4, 64),
    (8, 4096, 14336, 8, 32), (2, 14336, 4096, 8, 32), (3, 200, 512, 4, 32), (16, 96, 256, 8, 64),
    # K = 64 mod 128 (the last 128-k step is half past K), K = 64, odd row counts,
    # two row tiles (M = 12), 8-bit groups of 64
    (5, 200, 320, 4, 64), (2, 48, 64, 4, 64), (12, 96, 192, 4, 64), (7, 130, 448, 8, 64),
    # K / group_size odd: the last 128-k step is half past K
    (3, 97, 320, 4, 64),
    # long rows: the 32 KB scale block (K / group_size = 320, and 1024 at the limit)
    (2, 64, 20480, 4, 64), (1, 32, 32768, 4, 32), (3, 48, 16384, 8, 64),
    # tiles of 1, 2 and 4 rows for every code format
    (1, 64, 256, 8, 64), (3, 96, 384, 8, 64), (1, 80, 256, 4, 32), (2, 48, 128, 4, 32),
    (2, 64, 512, 8, 32), (4, 32, 1024, 4, 64),
])
def test_qmm_small_m_decode_shapes(dev, B, N, K, bits, gs):
    x, w = workloads.small_m_dense(B, N, K, seed=B)
    _say(f"small-M qmm B={B} N={N} K={K} bits={bits} gs={gs}")
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    out = _mq().mq_qmm(bf16_to_torch(x, dev), wq, s, b, True, gs, bits)
    torch.cuda.synchronize()
    o = bf16_u16_to_f64(torch_bf16_to_u16(out))
    owq, os_, ob = oracle.quantize(w, gs, bits)
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 300)), [N - 1]]))
    ref = oracle.qmm(x, owq[cols], os_[cols], ob[cols], gs, bits)
    check_gate(o[:, cols], ref, f"small-M B={B} N={N} K={K}")


# Where every wave of the split of K has one round of steps, each copies its
# own groups' scales and biases instead of the workgroup staging the block's
# rows behind a barrier.  Same products, same order of additions: the output
# is bit-identical with the staged block (MQ_SMALL_OWN=0), and within the gate.
@pytest.mark.parametrize("B,N,K,bits,gs,waves", [
    (1, 14336, 4096, 4, 64, None), (8, 14336, 4096, 4, 64, None), (3, 200, 2048, 4, 64, "16"),
    (2, 96, 1024, 4, 32, "8"), (5, 160, 2048, 8, 32, "8"), (1, 80, 1152, 4, 64, "8"),
])
def test_small_m_own_scale_slices(dev, B, N, K, bits, gs, waves, monkeypatch):
    x, w = workloads.small_m_dense(B, N, K, seed=B + 3)
    _say(f"small-M own scale slices B={B} N={N} K={K} bits={bits} gs={gs} waves={waves}")
    if waves:
        monkeypatch.setenv("MQ_SMALL_WAVES", waves)
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    xt = bf16_to_torch(x, dev)
    own = _mq().mq_qmm(xt, wq, s, b, True, gs, bits)
    monkeypatch.setenv("MQ_SMALL_OWN", "0")
    staged = _mq().mq_qmm(xt, wq, s, b, True, gs, bits)
    torch.cuda.synchronize()
    assert torch.equal(own.view(torch.int16), staged.view(torch.int16))
    owq, os_, ob = oracle.quantize(w, gs, bits)
    cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 300)), [N - 1]]))
    ref = oracle.qmm(x, owq[cols], os_[cols], ob[cols], gs, bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(own))[:, cols], ref, f"own slices B={B} N={N} K={K}")


@pytest.mark.parametrize("name,T,A,E,K,N,kw", [
    ("moe-decode", 4, 8, 128, 2048, 768, {}),
    ("short-runs-M2", 40, 4, 32, 256, 128, dict(M=2, Ax=1)),
    ("ragged-N", 30, 2, 8, 512, 200, {}),
    ("8bit-gs32", 24, 4, 16, 256, 64, {}),
    ("ragged-K", 16, 4, 8, 320, 96, {}),
    ("odd-groups", 16, 4, 8, 320, 97, {}),
    # skewed routing over many experts: 4-row tiles, several for the busiest expert
    ("zipf-tiles-of-4", 16, 2, 64, 256, 64, dict(routing="zipf")),
])
def test_gather_small_m_path(dev, name, T, A, E, K, N, kw, monkeypatch):
    monkeypatch.setenv("MQ_SMALL_M", "1")
    bits, gs = (8, 32) if "8bit" in name else (4, 64)
    case = workloads.gather_case(name, T, A, E, K, N, seed=13, bits=bits, group_size=gs, **kw)
    _say(f"gather small-M path {name}")
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case), name)


def test_gather_small_m_matches_gemm_path(dev, monkeypatch):
    case = workloads.gather_case("paths", 64, 4, 16, 512, 256, seed=14)
    weights = gpu_quantize(case.w, 64, 4, dev)
    monkeypatch.setenv("MQ_SMALL_M", "1")
    a = bf16_u16_to_f64(torch_bf16_to_u16(run_gather(case, dev, weights=weights)))
    monkeypatch.setenv("MQ_SMALL_M", "0")
    b = bf16_u16_to_f64(torch_bf16_to_u16(run_gather(case, dev, weights=weights)))
    check_gate(a, b, "small-M vs GEMM path")
    check_gate(a, oracle_gather(case), "small-M vs oracle")


@pytest.mark.parametrize("B,N,K,bits,gs", [
    (4, 200, 512, 4, 64), (8, 130, 256, 8, 64), (3, 1000, 448, 4, 32), (1, 64, 64, 4, 64),
    (6, 520, 320, 8, 32), (8, 2048, 512, 4, 64),
])
def test_small_m_column_split_matches_k_split(dev, B, N, K, bits, gs, monkeypatch):
    """Short rows: the column split (each wave walks all of K for its own
    columns) against the K split and the oracle."""
    x, w = workloads.small_m_dense(B, N, K, seed=B + 40)
    _say(f"small-M column split B={B} N={N} K={K} bits={bits} gs={gs}")
    wq, s, b = gpu_quantize(w, gs, bits, dev)
    xt = bf16_to_torch(x, dev)
    outs = {}
    for cs in ("1", "0"):
        monkeypatch.setenv("MQ_SMALL_COLSPLIT", cs)
        outs[cs] = bf16_u16_to_f64(torch_bf16_to_u16(_mq().mq_qmm(xt, wq, s, b, True, gs, bits)))
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(w, gs, bits)
    ref = oracle.qmm(x, owq, os_, ob, gs, bits)
    check_gate(outs["1"], ref, "column split")
    check_gate(outs["0"], ref, "K split")


@pytest.mark.parametrize("name,T,A,E,K,N", [
    ("down-like-r4", 32, 8, 64, 512, 1024), ("down-like-r8", 64, 8, 64, 512, 640),
    ("short-K-ragged-N", 20, 4, 16, 256, 200),
])
def test_gather_small_m_column_split(dev, name, T, A, E, K, N, monkeypatch):
    monkeypatch.setenv("MQ_SMALL_M", "1")
    monkeypatch.setenv("MQ_SMALL_COLSPLIT", "1")
    case = workloads.gather_case(name, T, A, E, K, N, seed=41, routing="balanced")
    _say(f"gather small-M column split {name}")
    out = run_gather(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_gather(case), name)


@pytest.mark.parametrize("name,T,A,E,K,N,bad", [
    ("moe-decode", 4, 8, 128, 2048, 768, 0), ("decode-out-of-range", 4, 8, 64, 512, 200, 3),
    ("many-experts", 16, 8, 1000, 256, 96, 0), ("256-pairs", 32, 8, 256, 256, 64, 2),
    ("batched-decode-512-pairs", 64, 8, 128, 2048, 768, 0),
    ("512-pairs-out-of-range", 64, 8, 300, 256, 96, 3), ("500-pairs", 125, 4, 256, 512, 64, 1),
])
def test_gather_fused_routing_matches_separate(dev, name, T, A, E, K, N, bad, monkeypatch):
    """A decode-sized routing done inside the small-M kernel gives the same
    output bits and leaves the same routing in the workspace (offsets, perm,
    tile table, error word) as the separate routing launch."""
    case = workloads.gather_case(name, T, A, E, K, N, seed=43)
    if bad:
        flat = case.idx.reshape(-1).copy()
        flat[np.random.default_rng(1).choice(flat.size, bad, replace=False)] = [E, -1, E + 7][:bad]
        case.idx = flat.reshape(case.idx.shape)
    _say(f"fused routing {name}")
    weights = gpu_quantize(case.w, 64, 4, dev)
    res = {}
    for fuse in ("1", "0"):
        if fuse == "0":
            monkeypatch.setenv("MQ_FUSE_ROUTE", "0")
        out, ws, L = run_gather(case, dev, weights=weights, ret_ws=True)
        n = T * A
        res[fuse] = (torch_bf16_to_u16(out),
                     ws[L.offsets:L.offsets + 4 * (E + 1)].view(torch.int32).cpu().numpy(),
                     ws[L.perm:L.perm + 4 * n].view(torch.int32).cpu().numpy(),
                     ws[L.tiles:L.tiles + 4 * (E + 1)].view(torch.int32).cpu().numpy(),
                     ws[L.error:L.error + 8].view(torch.int32).cpu().numpy())
    for a, b, what in zip(res["1"], res["0"], ("out", "offsets", "perm", "tiles", "error")):
        assert np.array_equal(a, b), what
    flat = case.idx.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    assert res["1"][4][0] == int((~ok).sum())
    o = bf16_u16_to_f64(res["1"][0]).reshape(-1, N)
    assert (o[~ok] == 0).all()
    good = workloads.GatherCase(name, case.x.reshape(T * A, 1, 1, K)[ok], case.w,
                                flat[ok].reshape(-1, 1).astype(np.int32), E)
    check_gate(o[ok].reshape(-1, 1, 1, N), oracle_gather(good), name)


def test_gather_fused_routing_serves_routed_calls(dev):
    """The routing a fused call leaves in the workspace serves
    mq_gather_qmm_routed (same bits as the fused call)."""
    mq = _mq()
    case = workloads.moe_decode(3)
    wq, s, b = gpu_quantize(case.w, 64, 4, dev)
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    L = mq.mq_gather_qmm_workspace(case.T, case.A, 1, case.K, case.N, case.E, 64, 4)
    ws = torch.empty(L.total, dtype=torch.uint8, device=dev)
    a = mq.mq_gather_qmm(x, wq, s, b, idx, workspace=ws)
    r = mq.mq_gather_qmm_routed(x, wq, s, b, case.A, ws)
    torch.cuda.synchronize()
    assert np.array_equal(torch_bf16_to_u16(a), torch_bf16_to_u16(r))


# --- gate and up in one pass with the gated activation --------------------------------------

def _glu_case(name, T, A, E, K, F, seed, **kw):
    """x, routing and the gate weight from one draw, the up weight from another"""
    case = workloads.gather_case(name, T, A, E, K, F, seed=seed, **kw)
    up = workloads.gather_case(name + "-up", T, A, E, K, F, seed=seed + 1000, **kw).w
    return case, up


def run_glu(case, up_w, act, dev, ret_ws=False):
    gs, bits = case.group_size, case.bits
    gate = gpu_quantize(case.w, gs, bits, dev)
    up = gpu_quantize(up_w, gs, bits, dev)
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    res = _mq().mq_gather_qmm_glu(x, gate, up, idx, act, True, gs, bits, case.sorted_indices,
                                  return_workspace=ret_ws)
    torch.cuda.synchronize()
    return res


def oracle_glu(case, up_w, act):
    gs, bits = case.group_size, case.bits
    return oracle.gather_qmm_glu(case.x, oracle.quantize(case.w, gs, bits),
                                 oracle.quantize(up_w, gs, bits), case.idx, gs, bits, act)


GLU_SHAPES = [
    # name, T, A, E, K, F, kwargs
    ("glu-basic", 64, 4, 6, 256, 192, {}),
    ("glu-broadcast-M2", 24, 3, 5, 128, 64, dict(M=2, Ax=1)),
    ("glu-F-ragged-200", 40, 2, 4, 256, 200, {}),
    ("glu-F-odd-100", 40, 2, 4, 128, 100, {}),
    ("glu-K64", 60, 2, 3, 64, 96, {}),
    ("glu-short-runs", 64, 4, 64, 256, 128, dict(routing="balanced")),
    ("glu-8bit-gs32", 48, 4, 4, 256, 160, dict(bits=8, group_size=32)),
]


@pytest.mark.parametrize("act", [1, 2], ids=["silu", "gelu"])
@pytest.mark.parametrize("name,T,A,E,K,F,kw", GLU_SHAPES, ids=[g[0] for g in GLU_SHAPES])
def test_gather_qmm_glu_shapes(dev, name, T, A, E, K, F, kw, act):
    case, up = _glu_case(name, T, A, E, K, F, 31, **kw)
    _say(f"gather_qmm_glu {name} act={act}")
    out = run_glu(case, up, act, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_glu(case, up, act), f"{name} act={act}")


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
def test_gather_qmm_glu_every_tile_height(dev, bm, monkeypatch):
    """K = 2048 with the FFN weight scale of the Mixtral-shaped config (W ~
    N(0, 0.02)): gate and up products of O(1).  (With N(0, 1) weights both are
    ~sqrt(K) = 45 and their fp32 accumulation errors, ~1e-3 each, multiply
    into absolute errors of a few 1e-2 on outputs near zero, over the gate's
    absolute floor of 1e-2 although every factor is within it.)"""
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case, up = _glu_case("glu-bm", 150, 4, 5, 2048, 200, 37, w_std=0.02)
    for act in (1, 2):
        _say(f"gather_qmm_glu forced BM={bm} act={act}")
        out = run_glu(case, up, act, dev)
        check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_glu(case, up, act),
                   f"glu BM={bm} act={act}")


@pytest.mark.parametrize("act", [1, 2])
def test_gather_qmm_glu_unit_weights_k2048(dev, act):
    """K = 2048 with W ~ N(0, 1): gate and up products of ~45 whose product
    is checked under the unchanged gate, absolute floor 1e-2 included.  The
    4-bit codes enter the MFMA as 16 + q, so the per-group fp32 sums cancel
    little and each projection's error stays well below 1e-2 / 45."""
    case, up = _glu_case("glu-unit", 150, 4, 5, 2048, 200, 38, w_std=1.0)
    _say(f"gather_qmm_glu K=2048 W~N(0,1) act={act}")
    out = run_glu(case, up, act, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_glu(case, up, act),
               f"glu K=2048 unit weights act={act}")


def test_gather_qmm_glu_out_of_range_rows_zero(dev):
    case, up = _glu_case("glu-oob", 20, 2, 4, 128, 64, 41)
    bad = case.idx.copy()
    bad[5, 1] = 9
    bad[13, 0] = -1
    case.idx = bad
    out, ws, L = run_glu(case, up, 1, dev, ret_ws=True)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, case.N)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    assert ws[L.error:L.error + 4].view(torch.int32).item() == int((~ok).sum())
    good = workloads.GatherCase("glu-ok", case.x.reshape(40, 1, 1, 128)[ok], case.w,
                                flat[ok].reshape(-1, 1).astype(np.int32), 4)
    check_gate(o[ok].reshape(-1, 1, 1, case.N), oracle_glu(good, up, 1), "glu valid rows")


def test_gather_qmm_glu_mixtral_sampled(dev):
    """Mixtral-shaped gate and up (K=4096 -> F=14336, E=8, top-2, Zipf 1.2
    routing), full size, sampled against the oracle's per-output dot products."""
    g = workloads.mixtral_ffn(0, 1.2, "up")
    T, A, E, K, F = g.T, g.A, g.E, g.K, g.N
    up_w = workloads.gather_case("mixtral-up2", 8, 1, E, K, F, seed=77, w_std=0.02).w
    _say("gather_qmm_glu Mixtral shape (full size), sampled")
    out = run_glu(g, up_w, 1, dev)
    o = torch_bf16_to_u16(out).reshape(-1, F)
    # quantisation is per weight row: the oracle quantises only 64 sampled
    # columns of each expert, and the samples use those columns
    rng = np.random.default_rng(3)
    colset = np.sort(rng.choice(F, 64, replace=False))
    pairs = rng.integers(0, T * A, 1200)
    sub = rng.integers(0, 64, 1200)
    gq = oracle.quantize(np.ascontiguousarray(g.w[:, colset]), 64, 4)
    uq = oracle.quantize(np.ascontiguousarray(up_w[:, colset]), 64, 4)
    gr = oracle.gather_qmm_rows(g.x, *gq, g.idx, 64, 4, pairs, sub)
    ur = oracle.gather_qmm_rows(g.x, *uq, g.idx, 64, 4, pairs, sub)
    check_gate(bf16_u16_to_f64(o[pairs, colset[sub]]), oracle.glu_act(gr, 1) * ur,
               "glu Mixtral sampled")


# --- the unquantised gather (bf16 weights) ---------------------------------------------

def run_gather_mm(case, dev, ret_ws=False):
    x = bf16_to_torch(case.x, dev)
    w = bf16_to_torch(case.w, dev)
    idx = i32_to_torch(case.idx, dev)
    res = _mq().mq_gather_mm(x, w, idx, True, case.sorted_indices, return_workspace=ret_ws)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name,T,A,E,K,N,kw", GATHER_SHAPES, ids=[g[0] for g in GATHER_SHAPES])
def test_gather_mm_shapes(dev, name, T, A, E, K, N, kw):
    case = workloads.gather_case(name, T, A, E, K, N, seed=17, **kw)
    _say(f"gather_mm {name}")
    out = run_gather_mm(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
               oracle.gather_mm(case.x, case.w, case.idx), f"gather_mm {name}")


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
def test_gather_mm_every_tile_height(dev, bm, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case = workloads.gather_case("mm-bm", 150, 4, 5, 320, 200, seed=19)
    _say(f"gather_mm forced BM={bm}")
    out = run_gather_mm(case, dev)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
               oracle.gather_mm(case.x, case.w, case.idx), f"gather_mm BM={bm}")


def test_gather_mm_out_of_range_rows_zero(dev):
    case = workloads.gather_case("mm-oob", 20, 2, 4, 128, 64, seed=23)
    bad = case.idx.copy()
    bad[2, 0] = 4
    bad[11, 1] = -7
    case.idx = bad
    out, ws, L = run_gather_mm(case, dev, ret_ws=True)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, case.N)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    assert ws[L.error:L.error + 4].view(torch.int32).item() == int((~ok).sum())
    good_x = case.x.reshape(40, 1, 1, 128)[ok]
    ref = oracle.gather_mm(good_x, case.w, flat[ok].reshape(-1, 1).astype(np.int32))
    check_gate(o[ok].reshape(-1, 1, 1, case.N), ref, "gather_mm valid rows")


def test_gather_mm_prefill_sampled(prefill, dev):
    case = prefill[0]
    _say("prefill gather_mm (bf16 weights, full size), sampled parity")
    out, ws, L = run_gather_mm(case, dev, ret_ws=True)
    o = torch_bf16_to_u16(out).reshape(-1, case.N)
    _, ooff, operm = oracle.route(case.idx, case.E)
    perm = ws[L.perm:L.perm + 4 * case.idx.size].view(torch.int32).cpu().numpy()
    assert np.array_equal(perm, operm)
    pairs, cols = _samples(case, np.random.default_rng(5))
    ref = oracle.gather_mm_rows(case.x, case.w, case.idx, pairs, cols)
    check_gate(bf16_u16_to_f64(o[pairs, cols]), ref, "prefill gather_mm sampled")


def test_gather_mm_deterministic_and_presorted(dev):
    case = workloads.gather_case("mm-det", 64, 4, 8, 256, 128, seed=29)
    a = torch_bf16_to_u16(run_gather_mm(case, dev))
    b = torch_bf16_to_u16(run_gather_mm(case, dev))
    assert np.array_equal(a, b)
    # the pairs sorted by expert (stable), with the sorted hint: the same rows
    order = np.argsort(case.idx.reshape(-1), kind="stable")
    sc = workloads.GatherCase("mm-sorted", case.x.reshape(-1, 1, 1, 256)[order], case.w,
                              case.idx.reshape(-1)[order].reshape(-1, 1).astype(np.int32), 8)
    sc.sorted_indices = True
    s = torch_bf16_to_u16(run_gather_mm(sc, dev))
    assert np.array_equal(s.reshape(-1, 128), a.reshape(-1, 128)[order])


# --- one routing, several projections (routing reuse) -----------------------------------

@pytest.mark.parametrize("rows", [4, 16, 64, 128])
def test_routed_up_then_down_shares_one_routing(dev, rows):
    """The up projection (K=2048 -> 512) and the down projection (512 -> 2048)
    of the short-run workload reuse one routing (mq_gather_route); each
    projection's x gets its row sums (mq_gather_sums).  Results equal the
    full mq_gather_qmm calls bit for bit, and sampled outputs pass the gate
    against the oracle (the down projection's oracle input is the GPU's up
    output, so each product is checked on its own)."""
    mq = _mq()
    case = workloads.short_run_sweep(rows, seed=21)
    T, A, E = case.T, case.A, case.E
    _say(f"routed up/down: {rows} rows per expert, T={T}")
    wu = gpu_quantize(case.w, 64, 4, dev)
    wd = gpu_quantize(case.w_down, 64, 4, dev)
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    Lu = mq.mq_gather_qmm_workspace(T, A, 1, 2048, 512, E, 64, 4)
    Ld = mq.mq_gather_qmm_workspace(T, A, 1, 512, 2048, E, 64, 4)
    ws = torch.empty(max(Lu.total, Ld.total), dtype=torch.uint8, device=dev)
    mq.mq_gather_route(idx, E, 1, workspace=ws)
    mq.mq_gather_sums(x, A, E, ws)
    h = mq.mq_gather_qmm_routed(x, *wu, A, ws)
    mq.mq_gather_sums(h, A, E, ws)
    y = mq.mq_gather_qmm_routed(h, *wd, A, ws)
    h_full = mq.mq_gather_qmm(x, *wu, idx)
    y_full = mq.mq_gather_qmm(h_full, *wd, idx)
    torch.cuda.synchronize()
    hu, yu = torch_bf16_to_u16(h), torch_bf16_to_u16(y)
    assert np.array_equal(hu, torch_bf16_to_u16(h_full))
    assert np.array_equal(yu, torch_bf16_to_u16(y_full))
    rng = np.random.default_rng(rows)
    owu = oracle.quantize(case.w, 64, 4)
    owd = oracle.quantize(case.w_down, 64, 4)
    for name, xin, (oq, os_, ob), res, N in (("up", case.x, owu, hu, 512),
                                             ("down", hu, owd, yu, 2048)):
        pairs = rng.integers(0, T * A, 1500)
        cols = rng.integers(0, N, 1500)
        ref = oracle.gather_qmm_rows(xin, oq, os_, ob, case.idx, 64, 4, pairs, cols)
        check_gate(bf16_u16_to_f64(res.reshape(-1, N)[pairs, cols]), ref, f"routed {name} r={rows}")


# --- calibration probes -------------------------------------------------------------------

def test_probes_run(dev):
    """The calibration probes (libmq_probe.so, called through its C ABI) run
    and their sinks hold the values their definition fixes."""
    import ctypes
    mq = _mq()
    path = os.path.join(os.path.dirname(mq.lib_path()), "libmq_probe.so")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mq_probe_stream.restype = ctypes.c_int
    lib.mq_probe_stream.argtypes = [P, I64, P, I32, P]
    lib.mq_probe_mfma.restype = ctypes.c_int
    lib.mq_probe_mfma.argtypes = [I32, P, I32, P]
    stream = torch.cuda.current_stream().cuda_stream
    buf = torch.arange(1 << 20, dtype=torch.int32, device=dev)          # 4 MB
    sink = torch.zeros(16 * 256, dtype=torch.int32, device=dev)
    assert lib.mq_probe_stream(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), 16, stream) == 0
    fsink = torch.zeros(2 * 256, dtype=torch.float32, device=dev)
    assert lib.mq_probe_mfma(3, fsink.data_ptr(), 2, stream) == 0
    torch.cuda.synchronize()
    # the XOR over all lanes' words is the XOR of the whole buffer
    words = sink.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(words) == np.bitwise_xor.reduce(np.arange(1 << 20, dtype=np.uint32))
    out = fsink.cpu().numpy()
    assert np.isfinite(out).all() and (out > 0).any()


# --- MX modes: MXFP4 (E2M1 codes) and MXFP8 (E4M3 codes), E8M0 block exponents ---------

ELEM = {4: "e2m1", 8: "e4m3"}
MX_BITS = [4, 8]


def gpu_quantize_mx(w_u16, dev, bits=4):
    return _mq().mq_quantize_mx(bf16_to_torch(w_u16, dev), bits)


def _mx_special_weights():
    """Ties on every E2M1 rounding midpoint at three scales, values past 6 X,
    bf16 subnormals, an all-zero block, a -0 block, a 1e30 block and a
    block spanning 60 binades."""
    rng = np.random.default_rng(31)
    w = rng.standard_normal((8, 256)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    w[0, :32] = np.tile(mids, 4) * np.repeat(np.array([1, -1, 1, -1], np.float32), 8)
    w[0, 32:64] = w[0, :32] * np.float32(2.0 ** -9)
    w[0, 64:96] = w[0, :32] * np.float32(2.0 ** 40)
    w[1, :32] = np.array([4.0, 7.0, 6.5, 7.9, -7.5, 5.5, -5.01] + [0.3] * 25, np.float32)
    w[1, 32:64] = np.array([256.0, 448.0, 464.0, 470.0, 480.0, 500.0, 511.0, -464.0, 1.0625,
                            1.1875, 2.0 ** -10, 3 * 2.0 ** -11] + [0.7] * 20, np.float32)
    w[2, :32] = 0.0
    w[2, 32:64] = -0.0
    w[2, 64:96] = rng.integers(-100, 100, 32).astype(np.float32) * np.float32(2.0 ** -133)
    w[3, :32] = rng.standard_normal(32).astype(np.float32) * np.float32(1e30)
    w[3, 32:64] = (rng.standard_normal(32) * 2.0 ** rng.integers(-30, 30, 32)).astype(np.float32)
    w[4, :] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-36)
    return workloads.bf16_bits_from_f32(w)


@pytest.mark.parametrize("bits", MX_BITS)
@pytest.mark.parametrize("name,shape,std", [
    ("tiny", (8, 128, 256), 1.0),
    ("small-std", (4, 96, 512), 0.02),
    ("prefill-experts", (64, 768, 2048), 1.0),
])
def test_quantize_mx_bit_exact(dev, name, shape, std, bits):
    _say(f"quantize_mx {name} {shape} bits={bits}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = workloads.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    if name == "prefill-experts":
        w = w[:, :96]            # the oracle's share: every expert, 96 rows each
    wq, sc = gpu_quantize_mx(w, dev, bits)
    owq, osc = oracle.quantize_mx(w, ELEM[bits])
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(sc.cpu().numpy(), osc)


@pytest.mark.parametrize("bits", MX_BITS)
def test_quantize_mx_special_values(dev, bits):
    w = _mx_special_weights()
    wq, sc = gpu_quantize_mx(w, dev, bits)
    owq, osc = oracle.quantize_mx(w, ELEM[bits])
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(sc.cpu().numpy(), osc)


def run_gather_mx(case, dev, weights=None, ret_ws=False, bits=4):
    if weights is None:
        weights = gpu_quantize_mx(case.w, dev, bits)
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    res = _mq().mq_gather_qmm_mx(x, *weights, idx, True, case.sorted_indices,
                                 return_workspace=ret_ws, bits=bits)
    torch.cuda.synchronize()
    return res


def _mx_case(case, dev, bits=4):
    """Quantise on both sides; the codes must agree before the products are
    compared."""
    weights = gpu_quantize_mx(case.w, dev, bits)
    owq, osc = oracle.quantize_mx(case.w, ELEM[bits])
    assert np.array_equal(torch_to_u32(weights[0]), owq)
    assert np.array_equal(weights[1].cpu().numpy(), osc)
    return weights, (owq, osc)


@pytest.mark.parametrize("bits", MX_BITS)
@pytest.mark.parametrize("name,T,A,E,K,N,kw", GATHER_SHAPES, ids=[g[0] for g in GATHER_SHAPES])
def test_gather_mx_shapes(dev, name, T, A, E, K, N, kw, bits):
    case = workloads.gather_case(name, T, A, E, K, N, seed=37, **kw)
    _say(f"gather_qmm_mx {name} bits={bits}")
    weights, (owq, osc) = _mx_case(case, dev, bits)
    out = run_gather_mx(case, dev, weights, bits=bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
               oracle.gather_qmm_mx(case.x, owq, osc, case.idx, ELEM[bits]),
               f"gather_qmm_mx {name} bits={bits}")


@pytest.mark.parametrize("bits", MX_BITS)
@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
def test_gather_mx_every_tile_height(dev, bm, bits, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    for K in (320, 512):              # a half pair at the end, and whole pairs (4-byte scales)
        case = workloads.gather_case("mx-bm", 150, 4, 5, K, 200, seed=41)
        _say(f"gather_qmm_mx forced BM={bm} K={K} bits={bits}")
        weights, (owq, osc) = _mx_case(case, dev, bits)
        out = run_gather_mx(case, dev, weights, bits=bits)
        check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
                   oracle.gather_qmm_mx(case.x, owq, osc, case.idx, ELEM[bits]),
                   f"gather_qmm_mx BM={bm} K={K} bits={bits}")


def test_gather_mx_decodes_every_code_and_exponent_exactly(dev):
    """x rows are unit vectors e_k, so each output is one decoded weight:
    random codes under every exponent of the exact range 2..252 must come
    back bit for bit (the weight is a bf16 value; one product, no rounding)."""
    E, N, K = 3, 128, 256
    rng = np.random.default_rng(43)
    wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = rng.integers(2, 253, size=(E, N, K // 32)).astype(np.uint8)
    sc[0, :, :] = np.arange(2, 2 + N * K // 32).reshape(N, K // 32) % 251 + 2
    ks = rng.integers(0, K, 64)
    x = np.zeros((64, 1, 1, K), np.float32)
    x[np.arange(64), 0, 0, ks] = 1.0
    idx = rng.integers(0, E, (64, 1)).astype(np.int32)
    out = _mq().mq_gather_qmm_mx(bf16_to_torch(workloads.bf16_bits_from_f32(x), dev),
                                 u32_to_torch(wq, dev).view(torch.int32),
                                 torch.from_numpy(sc).to(dev), i32_to_torch(idx, dev))
    got = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(64, N)
    W = oracle.dequantize_mx(wq, sc)
    assert np.array_equal(got, W[idx[:, 0], :, ks])


def test_gather_mx8_decodes_every_code_and_exponent_exactly(dev):
    """The MXFP8 counterpart: every finite E4M3 code under exponents 10..246
    (where a scaled E4M3 value is a normal, finite bf16) comes back bit for
    bit through unit-vector x rows."""
    E, N, K = 3, 128, 256
    rng = np.random.default_rng(44)
    byte = rng.integers(0, 256, size=(E, N, K))
    byte[(byte & 0x7F) == 0x7F] = 0x26
    byte[0, :, :] = np.arange(N * K).reshape(N, K) % 254
    byte[0][(byte[0] & 0x7F) == 0x7F] = 0x01
    wq = np.zeros((E, N, K // 4), np.uint32)
    for j in range(4):
        wq |= byte[..., j::4].astype(np.uint32) << np.uint32(8 * j)
    sc = rng.integers(10, 247, size=(E, N, K // 32)).astype(np.uint8)
    sc[1, :, :] = np.arange(N * K // 32).reshape(N, K // 32) % 237 + 10
    ks = rng.integers(0, K, 64)
    x = np.zeros((64, 1, 1, K), np.float32)
    x[np.arange(64), 0, 0, ks] = 1.0
    idx = rng.integers(0, E, (64, 1)).astype(np.int32)
    out = _mq().mq_gather_qmm_mx(bf16_to_torch(workloads.bf16_bits_from_f32(x), dev),
                                 u32_to_torch(wq, dev), torch.from_numpy(sc).to(dev),
                                 i32_to_torch(idx, dev), bits=8)
    got = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(64, N)
    W = oracle.dequantize_mx(wq, sc, "e4m3")
    assert np.array_equal(got, W[idx[:, 0], :, ks])


@pytest.mark.parametrize("bits", MX_BITS)
def test_gather_mx_out_of_range_rows_zero(dev, bits):
    case = workloads.gather_case("mx-oob", 20, 2, 4, 128, 64, seed=47)
    bad = case.idx.copy()
    bad[3, 1] = 4
    bad[9, 0] = -2
    case.idx = bad
    weights, (owq, osc) = _mx_case(case, dev, bits)
    out, ws, L = run_gather_mx(case, dev, weights, ret_ws=True, bits=bits)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, case.N)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    assert ws[L.error:L.error + 4].view(torch.int32).item() == int((~ok).sum())
    good_x = case.x.reshape(40, 1, 1, 128)[ok]
    ref = oracle.gather_qmm_mx(good_x, owq, osc, flat[ok].reshape(-1, 1).astype(np.int32),
                               ELEM[bits])
    check_gate(o[ok].reshape(-1, 1, 1, case.N), ref, "gather_qmm_mx valid rows")


@pytest.mark.parametrize("bits", MX_BITS)
def test_gather_mx_prefill_sampled(prefill, dev, bits):
    """The full prefill shape (T=2048, top-8 of 64, K=2048, N=768) on the
    device's quantisation; the oracle quantises the sampled weight rows
    itself, and those rows' codes must match the device's first."""
    case = prefill[0]
    _say(f"prefill gather_qmm_mx (full size), sampled parity, bits={bits}")
    wq, sc = gpu_quantize_mx(case.w, dev, bits)
    out, ws, L = run_gather_mx(case, dev, (wq, sc), ret_ws=True, bits=bits)
    o = torch_bf16_to_u16(out).reshape(-1, case.N)
    assert np.isfinite(bf16_u16_to_f64(o)).all()
    pairs, cols = _samples(case, np.random.default_rng(53), n_rand=1500, full_pairs=3)
    experts = case.idx.reshape(-1)[pairs]
    rows = np.unique(np.stack([experts, cols], 1), axis=0)
    owq_r, osc_r = oracle.quantize_mx(case.w[rows[:, 0], rows[:, 1]], ELEM[bits])
    gwq, gsc = torch_to_u32(wq), sc.cpu().numpy()
    assert np.array_equal(gwq[rows[:, 0], rows[:, 1]], owq_r)
    assert np.array_equal(gsc[rows[:, 0], rows[:, 1]], osc_r)
    # the oracle's codes for the sampled rows, scattered into an otherwise
    # empty stack (only those rows are read)
    owq = np.zeros(gwq.shape, np.uint32)
    osc = np.zeros(gsc.shape, np.uint8)
    owq[rows[:, 0], rows[:, 1]] = owq_r
    osc[rows[:, 0], rows[:, 1]] = osc_r
    ref = oracle.gather_qmm_mx_rows(case.x, owq, osc, case.idx, pairs, cols, ELEM[bits])
    check_gate(bf16_u16_to_f64(o[pairs, cols]), ref, "prefill gather_qmm_mx sampled")


@pytest.mark.parametrize("bits", MX_BITS)
def test_gather_mx_deterministic_and_presorted(dev, bits):
    case = workloads.gather_case("mx-det", 64, 4, 8, 256, 128, seed=59)
    weights = gpu_quantize_mx(case.w, dev, bits)
    a = torch_bf16_to_u16(run_gather_mx(case, dev, weights, bits=bits))
    b = torch_bf16_to_u16(run_gather_mx(case, dev, weights, bits=bits))
    assert np.array_equal(a, b)
    order = np.argsort(case.idx.reshape(-1), kind="stable")
    sc = workloads.GatherCase("mx-sorted", case.x.reshape(-1, 1, 1, 256)[order], case.w,
                              case.idx.reshape(-1)[order].reshape(-1, 1).astype(np.int32), 8)
    sc.sorted_indices = True
    s = torch_bf16_to_u16(run_gather_mx(sc, dev, weights, bits=bits))
    assert np.array_equal(s.reshape(-1, 128), a.reshape(-1, 128)[order])


# --- NVFP4 (E2M1 codes, E4M3 scale per 16 weights, fp32 scale per expert) ----------------

def gpu_quantize_nv(w_u16, dev):
    return _mq().mq_quantize_nv(bf16_to_torch(w_u16, dev))


def _nv_check_codes(weights, w_u16):
    owq, osc, og = oracle.quantize_nv(w_u16)
    wq, sc, g = weights
    assert np.array_equal(torch_to_u32(wq), owq)
    assert np.array_equal(sc.cpu().numpy(), osc)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
    return owq, osc, og


@pytest.mark.parametrize("name,shape,std", [
    ("tiny", (8, 128, 256), 1.0),
    ("small-std", (4, 96, 512), 0.02),
    ("wide-experts", (3, 64, 4096), 3.0),
])
def test_quantize_nv_bit_exact(dev, name, shape, std):
    _say(f"quantize_nv {name} {shape}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = workloads.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    _nv_check_codes(gpu_quantize_nv(w, dev), w)


def test_quantize_nv_special_values(dev):
    """Ties, a block far below its tensor's largest, zero blocks, -0, bf16
    subnormals and an all-zero tensor."""
    rng = np.random.default_rng(61)
    w = rng.standard_normal((3, 8, 64)).astype(np.float32)
    w[0, 1, :16] *= np.float32(1e-4)
    w[0, 2, 16:32] = 0.0
    w[0, 2, 32:48] = -0.0
    w[0, 3, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2, np.float32)
    w[1] *= np.float32(2.0 ** -100)
    w[1, 0, :16] = rng.integers(-60, 60, 16).astype(np.float32) * np.float32(2.0 ** -133)
    w[2] = 0.0
    wb = workloads.bf16_bits_from_f32(w)
    _nv_check_codes(gpu_quantize_nv(wb, dev), wb)


def run_gather_nv(case, dev, weights, ret_ws=False):
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    res = _mq().mq_gather_qmm_nv(x, *weights, idx, True, case.sorted_indices,
                                 return_workspace=ret_ws)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name,T,A,E,K,N,kw", GATHER_SHAPES, ids=[g[0] for g in GATHER_SHAPES])
def test_gather_nv_shapes(dev, name, T, A, E, K, N, kw):
    case = workloads.gather_case(name, T, A, E, K, N, seed=67, **kw)
    _say(f"gather_qmm_nv {name}")
    weights = gpu_quantize_nv(case.w, dev)
    owq, osc, og = _nv_check_codes(weights, case.w)
    out = run_gather_nv(case, dev, weights)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
               oracle.gather_qmm_nv(case.x, owq, osc, og, case.idx), f"gather_qmm_nv {name}")


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
def test_gather_nv_every_tile_height(dev, bm, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    for K in (320, 512):
        case = workloads.gather_case("nv-bm", 150, 4, 5, K, 200, seed=71)
        _say(f"gather_qmm_nv forced BM={bm} K={K}")
        weights = gpu_quantize_nv(case.w, dev)
        owq, osc, og = _nv_check_codes(weights, case.w)
        out = run_gather_nv(case, dev, weights)
        check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
                   oracle.gather_qmm_nv(case.x, owq, osc, og, case.idx), f"gather_qmm_nv BM={bm} K={K}")


def test_gather_nv_decodes_every_code_and_scale_exactly(dev):
    """With g = 1 and unit-vector x rows each output is one e2m1 * e4m3
    product, a bf16 value: every code under every finite block scale comes
    back bit for bit."""
    E, N, K = 3, 128, 256
    rng = np.random.default_rng(73)
    wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = (np.arange(E * N * K // 16).reshape(E, N, K // 16) % 127).astype(np.uint8)
    g = np.ones(E, np.float32)
    ks = rng.integers(0, K, 64)
    x = np.zeros((64, 1, 1, K), np.float32)
    x[np.arange(64), 0, 0, ks] = 1.0
    idx = rng.integers(0, E, (64, 1)).astype(np.int32)
    out = _mq().mq_gather_qmm_nv(bf16_to_torch(workloads.bf16_bits_from_f32(x), dev),
                                 u32_to_torch(wq, dev), torch.from_numpy(sc).to(dev),
                                 torch.from_numpy(g).to(dev), i32_to_torch(idx, dev))
    got = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(64, N)
    W = oracle.dequantize_nv(wq, sc, g)
    ref = W[idx[:, 0], :, ks]
    bad = np.argwhere(got != ref)
    detail = [(int(t), int(n), int(idx[t, 0]), int(ks[t]), hex(int(wq[idx[t, 0], n, ks[t] // 8])),
               int(sc[idx[t, 0], n, ks[t] // 16]), float(got[t, n]), float(ref[t, n]))
              for t, n in bad[:8]]
    assert len(bad) == 0, f"{len(bad)} mismatches (row, col, expert, k, word, scale code, got, ref): {detail}"


def test_gather_nv_out_of_range_rows_zero(dev):
    case = workloads.gather_case("nv-oob", 20, 2, 4, 128, 64, seed=79)
    bad = case.idx.copy()
    bad[5, 1] = 4
    bad[13, 0] = -3
    case.idx = bad
    weights = gpu_quantize_nv(case.w, dev)
    owq, osc, og = _nv_check_codes(weights, case.w)
    out, ws, L = run_gather_nv(case, dev, weights, ret_ws=True)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, case.N)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    assert ws[L.error:L.error + 4].view(torch.int32).item() == int((~ok).sum())
    good_x = case.x.reshape(40, 1, 1, 128)[ok]
    ref = oracle.gather_qmm_nv(good_x, owq, osc, og, flat[ok].reshape(-1, 1).astype(np.int32))
    check_gate(o[ok].reshape(-1, 1, 1, case.N), ref, "gather_qmm_nv valid rows")


def test_gather_nv_prefill_sampled(prefill, dev):
    """The full prefill shape on the device's quantisation.  The oracle
    quantises, per expert, the sampled weight rows plus the row holding the
    expert's largest |w| (which fixes the tensor scale), repeated to a common
    row count; those rows' codes, scales and tensor scales must match the
    device's before the sampled outputs are compared."""
    case = prefill[0]
    _say("prefill gather_qmm_nv (full size), sampled parity")
    wq, sc, g = gpu_quantize_nv(case.w, dev)
    out, ws, L = run_gather_nv(case, dev, (wq, sc, g), ret_ws=True)
    o = torch_bf16_to_u16(out).reshape(-1, case.N)
    assert np.isfinite(bf16_u16_to_f64(o)).all()
    pairs, cols = _samples(case, np.random.default_rng(83), n_rand=2000, full_pairs=0)
    experts = case.idx.reshape(-1)[pairs]
    absw = case.w & np.uint16(0x7FFF)
    top = absw.reshape(case.E, -1).argmax(axis=1) // case.K
    per = [sorted(set(cols[experts == e].tolist()) | {int(top[e])}) for e in range(case.E)]
    R = max(len(p) for p in per)
    rows = np.array([p + [p[0]] * (R - len(p)) for p in per])          # [E, R]
    sub = case.w[np.arange(case.E)[:, None], rows]                     # [E, R, K]
    owq_s, osc_s, og = oracle.quantize_nv(sub)
    gwq, gsc = torch_to_u32(wq), sc.cpu().numpy()
    assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
    assert np.array_equal(gwq[np.arange(case.E)[:, None], rows], owq_s)
    assert np.array_equal(gsc[np.arange(case.E)[:, None], rows], osc_s)
    owq = np.zeros(gwq.shape, np.uint32)
    osc = np.zeros(gsc.shape, np.uint8)
    owq[np.arange(case.E)[:, None], rows] = owq_s
    osc[np.arange(case.E)[:, None], rows] = osc_s
    ref = oracle.gather_qmm_nv_rows(case.x, owq, osc, og, case.idx, pairs, cols)
    check_gate(bf16_u16_to_f64(o[pairs, cols]), ref, "prefill gather_qmm_nv sampled")


def test_gather_nv_deterministic_and_presorted(dev):
    case = workloads.gather_case("nv-det", 64, 4, 8, 256, 128, seed=89)
    weights = gpu_quantize_nv(case.w, dev)
    a = torch_bf16_to_u16(run_gather_nv(case, dev, weights))
    b = torch_bf16_to_u16(run_gather_nv(case, dev, weights))
    assert np.array_equal(a, b)
    order = np.argsort(case.idx.reshape(-1), kind="stable")
    sc = workloads.GatherCase("nv-sorted", case.x.reshape(-1, 1, 1, 256)[order], case.w,
                              case.idx.reshape(-1)[order].reshape(-1, 1).astype(np.int32), 8)
    sc.sorted_indices = True
    s = torch_bf16_to_u16(run_gather_nv(sc, dev, weights))
    assert np.array_equal(s.reshape(-1, 128), a.reshape(-1, 128)[order])


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_fp_modes_mixtral_up_sampled(dev, mode):
    """The Mixtral-shaped up projection (E=8, top-2, T=2048, K=4096 -> N=14336,
    Zipf(1.2) routing, W ~ N(0, 0.02)) in each fp mode, full size, quantised on
    the device.  Quantisation is per weight row (NVFP4: plus the expert's
    tensor scale), so the oracle quantises 64 sampled columns of each expert
    (NVFP4: with the row holding the expert's largest |w|) and the sampled
    outputs use those columns; the device's codes for them must match first."""
    case = workloads.mixtral_ffn(0, 1.2, "up")
    E, K, N = case.E, case.K, case.N
    _say(f"{mode} Mixtral up (full size), sampled")
    rng = np.random.default_rng(97)
    colset = np.sort(rng.choice(N, 64, replace=False))
    pairs = rng.integers(0, case.T * case.A, 1200)
    sub = rng.integers(0, 64, 1200)
    x = bf16_to_torch(case.x, dev)
    idx = i32_to_torch(case.idx, dev)
    if mode == "nvfp4":
        wq, sc, g = gpu_quantize_nv(case.w, dev)
        out = _mq().mq_gather_qmm_nv(x, wq, sc, g, idx)
        top = (case.w & np.uint16(0x7FFF)).reshape(E, -1).argmax(axis=1) // K
        rows = np.concatenate([np.tile(colset, (E, 1)), top[:, None]], axis=1)   # [E, 65]
        owq, osc, og = oracle.quantize_nv(case.w[np.arange(E)[:, None], rows])
        assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
        assert np.array_equal(torch_to_u32(wq)[:, colset], owq[:, :64])
        assert np.array_equal(sc.cpu().numpy()[:, colset], osc[:, :64])
        ref = oracle.gather_qmm_nv_rows(case.x, owq[:, :64], osc[:, :64], og, case.idx, pairs, sub)
    else:
        bits = 4 if mode == "mxfp4" else 8
        wq, sc = gpu_quantize_mx(case.w, dev, bits)
        out = _mq().mq_gather_qmm_mx(x, wq, sc, idx, bits=bits)
        owq, osc = oracle.quantize_mx(np.ascontiguousarray(case.w[:, colset]), ELEM[bits])
        assert np.array_equal(torch_to_u32(wq)[:, colset], owq)
        assert np.array_equal(sc.cpu().numpy()[:, colset], osc)
        ref = oracle.gather_qmm_mx_rows(case.x, owq, osc, case.idx, pairs, sub, ELEM[bits])
    torch.cuda.synchronize()
    o = torch_bf16_to_u16(out).reshape(-1, N)
    assert np.isfinite(bf16_u16_to_f64(o)).all()
    check_gate(bf16_u16_to_f64(o[pairs, colset[sub]]), ref, f"{mode} Mixtral up sampled")
