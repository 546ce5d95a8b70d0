"""Tail tiles split along K: the pieces, their slots and their reduce.

A tiled launch whose tail tiles run after every full tile (the kernel's rule,
or MQ_TAIL_TILES=1) and whose K holds two correction windows of 32 groups or
more cuts each tail tile into pieces of whole windows.  Each piece stores its
fp32 sums into a 64 KiB slot of the workspace's optional `part` region and
a second launch adds the pieces in piece order and stores bf16.  Here:

  * every non-GLU instance of 64- and 128-row launches with a split (4- and
    8-bit codes, groups of 32 and 64, three and four column blocks per
    wave), against the oracle, with tails of 1, 22, 32, 33, 62 and 64 rows,
    an empty expert and a segment with no tail;
  * the slots written are exactly npart * ntn * pieces (tail tiles x column
    tiles x pieces): a workspace pre-filled with 0xFF keeps every other slot;
  * fewer slots than windows (fewer, longer pieces), more windows than
    pieces (nine windows: five pieces of two), a partial last window;
  * the split result and the unsplit one (MQ_TAIL_SPLIT=0, or a workspace
    of exactly `part` bytes, which writes no slot) both pass the gate;
  * several rows per pair with x broadcast over the slots.
"""
import itertools
import re

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_torch, bf16_u16_to_f64, check_gate, i32_to_torch, torch_bf16_to_u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SLOT = 65536
WIN = 32            # groups per correction window
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


def routed_case(name, counts, K, N, seed, A=1, M=1, Ax=None, bits=4, gs=64):
    """A case whose experts get exactly `counts` pairs (in a seeded order)."""
    counts = np.asarray(counts)
    n = int(counts.sum())
    assert n % A == 0
    case = workloads.gather_case(name, n // A, A, len(counts), K, N, seed=seed, M=M, Ax=Ax,
                                 bits=bits, group_size=gs)
    idx = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(seed).shuffle(idx)
    case.idx = idx.reshape(n // A, A)
    return case


def expected_slots(counts, M, bm, N, cols, K, gs, slots):
    """Slots the launch fills: tail tiles x column tiles x pieces, as the
    kernel decides them (tails of at most bm / 2 rows; pieces of whole
    windows, at most 8, as many as the slots hold)."""
    rows = np.asarray(counts) * M
    npart = int(((rows % bm > 0) & (rows % bm <= bm // 2)).sum())
    ntn = -(-N // (64 * cols))
    nwin = -(-(K // gs) // WIN)
    tiles = npart * ntn
    if tiles == 0 or nwin < 2:
        return 0, 1
    s = min(8, nwin, slots // tiles)
    if s < 2:
        return 0, 1
    wpp = -(-nwin // s)
    s = -(-nwin // wpp)
    return tiles * s, s


def run(case, dev, ws_bytes=None, ret_ws=False):
    mq = _mq()
    gs, bits = case.group_size, case.bits
    T, Ax, M, K = case.x.shape
    A = case.idx.shape[1]
    N = case.w.shape[1]
    L = mq.mq_gather_qmm_workspace(T, A, M, K, N, case.E, gs, bits)
    nbytes = L.total if ws_bytes is None else ws_bytes(L)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
    wq = mq.mq_quantize(bf16_to_torch(case.w, dev), gs, bits)
    out = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), *wq, i32_to_torch(case.idx, dev), True,
                           gs, bits, False, workspace=ws)
    torch.cuda.synchronize()
    got = bf16_u16_to_f64(torch_bf16_to_u16(out))
    return (got, ws, L) if ret_ws else got


def written_slots(ws, L):
    """Indices of the whole slots after `part` that are no longer all 0xFF."""
    n = (ws.numel() - L.part) // SLOT
    region = ws[L.part:L.part + n * SLOT].view(n, SLOT)
    return torch.nonzero((region != 0xFF).any(dim=1)).flatten().cpu().numpy()


def oracle_out(case):
    gs, bits = case.group_size, case.bits
    return oracle.gather_qmm(case.x, *oracle.quantize(case.w, gs, bits), case.idx, gs, bits)


# Tails by tile height (rows % bm in (0, bm / 2]): 128-row tiles: 22, 62, 44,
# 64, 33, 1 (and 128: none; an empty expert); 64-row tiles: 6, 32, 1, 31 (36
# and 64: none; an empty expert).
COUNTS = {128: [150, 190, 300, 64, 33, 128, 0, 1], 64: [70, 96, 100, 1, 64, 0, 129, 31]}
# K: 72 groups = two windows and a partial third (8 groups)
K_OF = {64: 64 * 72, 32: 32 * 72}
N = 272                    # two column tiles of 256 or 192, the last one ragged


def test_split_every_instance(dev, monkeypatch, capfd):
    """Every non-GLU 64/128-row instance splits its tails; slots and parity."""
    monkeypatch.setenv("MQ_LOG", "1")
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    for bm, (bits, gs) in itertools.product((64, 128), ((4, 64), (4, 32), (8, 64), (8, 32))):
        K = K_OF[gs]
        case = routed_case("split", COUNTS[bm], K, N, seed=bm + bits + gs, bits=bits, gs=gs)
        ref = oracle_out(case)
        monkeypatch.setenv("MQ_FORCE_BM", str(bm))
        for cols in ((3, 4) if bits == 4 and gs == 64 else (4,)):
            monkeypatch.setenv("MQ_FORCE_COLS", str(cols))
            what = f"BM={bm} bits={bits} gs={gs} cols={cols}"
            _say(f"split tails {what}")
            got, ws, L = run(case, dev, ret_ws=True)
            check_gate(got, ref, what)
            slots = (L.total - L.part) // SLOT
            want, pieces = expected_slots(COUNTS[bm], 1, bm, N, cols, K, gs, slots)
            assert pieces == 3, what
            assert np.array_equal(written_slots(ws, L), np.arange(want)), what
            monkeypatch.setenv("MQ_TAIL_SPLIT", "0")
            plain, ws0, L0 = run(case, dev, ret_ws=True)
            monkeypatch.delenv("MQ_TAIL_SPLIT")
            assert written_slots(ws0, L0).size == 0, what
            check_gate(plain, ref, what + " unsplit")
    seen = set()
    for line in capfd.readouterr().err.splitlines():
        m = _LINE.match(line.strip())
        if m and m.group(1) == "tail_reduce":
            seen.add(tuple(int(v) for v in m.group(2).split(",")))
    assert seen == {(64, 3), (64, 4), (128, 3), (128, 4)}, seen


def test_split_workspace_of_part_bytes_runs_unsplit(dev, monkeypatch):
    """A workspace of exactly `part` bytes (no slots) is enough; nothing is
    split and the result equals MQ_TAIL_SPLIT=0 bit for bit."""
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    monkeypatch.setenv("MQ_FORCE_BM", "128")
    monkeypatch.setenv("MQ_FORCE_COLS", "4")
    case = routed_case("split-noslots", COUNTS[128], K_OF[64], N, seed=3)
    _say("split tails: workspace without slots")
    short = run(case, dev, ws_bytes=lambda L: L.part)
    monkeypatch.setenv("MQ_TAIL_SPLIT", "0")
    off = run(case, dev)
    assert np.array_equal(short, off)
    check_gate(short, oracle_out(case), "no slots")


def test_split_fewer_slots_than_windows(dev, monkeypatch):
    """Slots for two pieces per tail tile: K's three windows go 2 + 1."""
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    monkeypatch.setenv("MQ_FORCE_BM", "128")
    monkeypatch.setenv("MQ_FORCE_COLS", "4")
    case = routed_case("split-fewslots", COUNTS[128], K_OF[64], N, seed=4)
    tiles = 6 * 2
    _say("split tails: slots for two pieces")
    got, ws, L = run(case, dev, ws_bytes=lambda L: L.part + tiles * 2 * SLOT + 100, ret_ws=True)
    want, pieces = expected_slots(COUNTS[128], 1, 128, N, 4, K_OF[64], 64, tiles * 2)
    check_gate(got, oracle_out(case), "two pieces")
    assert pieces == 2
    assert np.array_equal(written_slots(ws, L), np.arange(want))


@pytest.mark.parametrize("K,gs,pieces", [(32 * 32 * 9, 32, 5), (64 * 40, 64, 2), (64 * 41, 64, 2),
                                         (64 * 32 * 7, 64, 7)],
                         ids=["9-windows", "partial-second-window", "odd-chunks", "7-windows"])
def test_split_window_counts(dev, monkeypatch, K, gs, pieces):
    """Nine windows: five pieces of two (the last of one); 40 groups: a full
    window and a partial one; 41 groups: the second piece has an odd number
    of chunks (its last code load of a chunk pair is half past K); seven
    windows (a Mixtral-shaped down projection's K): seven pieces."""
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    monkeypatch.setenv("MQ_FORCE_BM", "128")
    monkeypatch.setenv("MQ_FORCE_COLS", "4")
    counts = [150, 33, 1, 128]
    case = routed_case("split-windows", counts, K, 200, seed=5, gs=gs)
    _say(f"split tails: K={K} gs={gs}")
    got, ws, L = run(case, dev, ret_ws=True)
    slots = (L.total - L.part) // SLOT
    want, s = expected_slots(counts, 1, 128, 200, 4, K, gs, slots)
    check_gate(got, oracle_out(case), f"K={K} gs={gs}")
    assert s == pieces
    assert np.array_equal(written_slots(ws, L), np.arange(want))


def test_split_rows_per_pair_and_broadcast(dev, monkeypatch):
    """M = 3 rows per pair, x broadcast over A = 2 slots: tails counted in
    rows (pairs x M)."""
    monkeypatch.setenv("MQ_TAIL_TILES", "1")
    monkeypatch.setenv("MQ_FORCE_BM", "128")
    monkeypatch.setenv("MQ_FORCE_COLS", "4")
    counts = [50, 11, 22, 45]                   # rows 150, 33, 66, 135: tails 22, 33, 7 (66: full)
    case = routed_case("split-M3", counts, K_OF[64], 136, seed=6, A=2, M=3, Ax=1)
    _say("split tails: M=3, Ax=1")
    got, ws, L = run(case, dev, ret_ws=True)
    slots = (L.total - L.part) // SLOT
    want, s = expected_slots(counts, 3, 128, 136, 4, K_OF[64], 64, slots)
    check_gate(got, oracle_out(case), "M=3 Ax=1")
    assert s == 3 and want > 0
    assert np.array_equal(written_slots(ws, L), np.arange(want))


def test_default_rule_splits_the_mixtral_down_projection(dev, monkeypatch):
    """No test hooks: the Mixtral-shaped down projection (T = 2048, top-2 of
    E = 8, Zipf(1.2), K = 14336 -> N = 4096) runs its tails last and splits
    each of its 6 x 16 tail tiles into 7 pieces (672 slots written); the up
    projection (K = 4096 -> N = 14336, its full tiles take several rounds)
    keeps its tails in place and writes none.  Parity of both at this size:
    tests/test_gpu_fullsize.py."""
    for var in ("MQ_TAIL_TILES", "MQ_TAIL_SPLIT", "MQ_FORCE_BM", "MQ_FORCE_COLS"):
        monkeypatch.delenv(var, raising=False)
    for proj, want in (("down", 6 * 16 * 7), ("up", 0)):
        case = workloads.mixtral_ffn(0, 1.2, proj)
        counts = np.bincount(case.idx.reshape(-1), minlength=case.E)
        _say(f"default rule, Mixtral {proj}: rows per expert {counts.tolist()}")
        _, ws, L = run(case, dev, ret_ws=True)
        assert written_slots(ws, L).size == want, proj
        if want:
            assert np.array_equal(written_slots(ws, L), np.arange(want))
