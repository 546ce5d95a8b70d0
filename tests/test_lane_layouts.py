"""Lane layouts of the tiled GEMM's chunk-pair code loads, checked on the CPU.

Four-bit codes in 64-wide groups reach the MFMA B operand (v_mfma_f32_16x16x32
_bf16: lane (n = l16, quarter c4) holds 8 consecutive k of column n for k-step
slots 8 c4 .. 8 c4 + 7) from one 16-byte load per lane that covers two 64-k
chunks: dword i of lane (l16, c4) holds k 32 c4 + 8 i .. + 7 of the pair.  A
swap of lanes 32-63 of dwords (0, 1) and (2, 3) with lanes 0-31 of the other
(v_permlane32_swap: the swapped pair's first result keeps lanes 0-31 of the
first operand and takes lanes 0-31 of the second into lanes 32-63; the second
result takes lanes 32-63 of the first into lanes 0-31 and keeps lanes 32-63 of
the second, as measured on the GPU) leaves the first chunk's k-steps in
dwords 0 and 2 and the second chunk's in dwords 1 and 3.  The x fragment of
k-step ks of quarter c4 is the chunk's 8-k piece p(c4) + 2 ks with
p = 0, 4, 1, 5.  These tests model the load and the swap and check that every
MFMA pairs each code with the x of the same k, and that each chunk's 64 k are
used exactly once per column.
"""
import numpy as np

LANES = np.arange(64)
L16, C4 = LANES % 16, LANES // 16


def loaded_pair():
    """k (0..127, relative to the pair) of the 8 codes in dword i of each lane:
    array [4 dwords, 64 lanes] of the first k of each 8-code run."""
    return np.stack([32 * C4 + 8 * i for i in range(4)])


def permlane32_swap(a, b):
    """The measured semantics of the swap on two per-lane values."""
    r0 = np.concatenate([a[:32], b[:32]])
    r1 = np.concatenate([a[32:], b[32:]])
    return r0, r1


def exchanged():
    d = loaded_pair()
    d0, d1 = permlane32_swap(d[0], d[1])
    d2, d3 = permlane32_swap(d[2], d[3])
    return d0, d1, d2, d3


def piece(c4, ks):
    return ((c4 >> 1) | ((c4 & 1) << 2)) + 2 * ks


def test_swap_model_matches_the_measured_lane_semantics():
    a, b = 100 + LANES, 200 + LANES
    r0, r1 = permlane32_swap(a, b)
    assert list(r0[:32]) == list(100 + LANES[:32]) and list(r0[32:]) == list(200 + LANES[:32])
    assert list(r1[:32]) == list(100 + LANES[32:]) and list(r1[32:]) == list(200 + LANES[32:])


def test_each_kstep_pairs_codes_with_the_x_of_the_same_k():
    d0, d1, d2, d3 = exchanged()
    for chunk, steps in ((0, (d0, d2)), (1, (d1, d3))):
        for ks, codes in enumerate(steps):
            # the codes of this k-step, relative to the chunk, per lane
            k_codes = codes - 64 * chunk
            assert np.all((k_codes >= 0) & (k_codes < 64)), (chunk, ks)
            k_x = 8 * piece(C4, ks)
            assert np.array_equal(k_codes, k_x), (chunk, ks)


def test_each_chunk_k_is_used_once_per_column():
    d0, d1, d2, d3 = exchanged()
    for chunk, steps in ((0, (d0, d2)), (1, (d1, d3))):
        for n in range(16):
            ks = sorted(int(k) - 64 * chunk + j for codes in steps
                        for k in codes[L16 == n] for j in range(8))
            assert ks == list(range(64)), (chunk, n)


def pairs_match(d0, d1, d2, d3):
    for chunk, steps in ((0, (d0, d2)), (1, (d1, d3))):
        for ks, codes in enumerate(steps):
            if not np.array_equal(codes - 64 * chunk, 8 * piece(C4, ks)):
                return False
    return True


def test_plausible_mistakes_fail():
    """The checks reject a swap of the wrong dwords, the natural-order x
    pieces of one-chunk loads, and the swap's results taken the other way."""
    assert pairs_match(*exchanged())
    d = loaded_pair()
    a0, a2 = permlane32_swap(d[0], d[2])
    a1, a3 = permlane32_swap(d[1], d[3])
    assert not pairs_match(a0, a1, a2, a3)
    r0, r1 = permlane32_swap(d[0], d[1])
    r2, r3 = permlane32_swap(d[2], d[3])
    assert not pairs_match(r1, r0, r3, r2)
    global piece
    saved = piece
    try:
        piece = lambda c4, ks: 2 * c4 + ks          # the one-chunk loads' pieces
        assert not pairs_match(*exchanged())
    finally:
        piece = saved
