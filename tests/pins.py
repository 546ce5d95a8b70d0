"""Checks that pin the oracle to something other than itself.

Each ``check_*`` takes the functions under test as arguments and raises
AssertionError when they disagree with what the mathematics fixes: hand-worked
examples, exact rational arithmetic, library special cases (numpy's stable
argsort, plain float matmul of grid-exact weights), invariants and closed
forms.  ``test_oracle_pins.py`` runs them against the oracle (they must hold)
and ``test_oracle_mutants.py`` runs them against copies of the oracle with a
planted mistake (at least one must fail), which shows the pins have teeth.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

from workloads import bf16_bits_from_f32, f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- independent bit-level helpers (no oracle code) ---------------------------

def _bf16_value(bits: int) -> Fraction:
    """Exact value of a bf16 pattern, decoded from sign/exponent/mantissa."""
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    assert exp != 0xFF, "non-finite bf16"
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    v = Fraction(128 + man, 128)
    return sign * (v * (Fraction(2) ** (exp - 127)))


def _code(words, k: int, bits: int) -> int:
    per = 32 // bits
    return (int(words[k // per]) >> ((k % per) * bits)) & ((1 << bits) - 1)


def _load_golden():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, wv, sb, words = [p.strip() for p in line.split("|")]
            name, bits, gs = head.split()
            s_bits, b_bits = sb.split()
            rows.append(dict(name=name, bits=int(bits), gs=int(gs),
                             w=np.array([float(v) for v in wv.split()], np.float32),
                             scale=int(s_bits, 16), bias=int(b_bits, 16),
                             words=[int(v, 16) for v in words.split()]))
    return rows


def _rand_bf16(rng, shape, std=1.0):
    return bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


# --- quantize -------------------------------------------------------------------

def check_quantize_worked_examples(quantize):
    for g in _load_golden():
        wq, s, b = quantize(bf16_bits_from_f32(g["w"])[None, :], g["gs"], g["bits"])
        assert int(s[0, 0]) == g["scale"], (g["name"], hex(int(s[0, 0])))
        assert int(b[0, 0]) == g["bias"], (g["name"], hex(int(b[0, 0])))
        assert [int(v) for v in wq[0]] == g["words"], (g["name"], [hex(int(v)) for v in wq[0]])


def _exact_dequant_row(wq_row, s_row, b_row, gs, bits, K):
    return [_bf16_value(s_row[k // gs]) * _code(wq_row, k, bits) + _bf16_value(b_row[k // gs])
            for k in range(K)]


def check_quantize_round_trip(quantize, seed=0):
    """|w - w_hat| <= scale/2 per element (exact rationals), slack for the two
    fp32 roundings that precede rint."""
    rng = np.random.default_rng(seed)
    for bits in (4, 8):
        for gs in (32, 64, 128):
            for std in (1.0, 0.02, 300.0):
                w = _rand_bf16(rng, (3, 2 * gs), std)
                wq, s, b = quantize(w, gs, bits)
                for r in range(w.shape[0]):
                    wh = _exact_dequant_row(wq[r], s[r], b[r], gs, bits, w.shape[1])
                    for k in range(w.shape[1]):
                        sc = _bf16_value(s[r, k // gs])
                        err = abs(_bf16_value(w[r, k]) - wh[k])
                        assert err <= sc * (Fraction(1, 2) + Fraction(1, 2 ** 14)), \
                            (bits, gs, std, r, k, float(err), float(sc))


def check_quantize_argmin(quantize, seed=1):
    """Each code is a nearest grid point: no other code reconstructs w more
    closely (ties within the fp32 rounding slack allowed)."""
    rng = np.random.default_rng(seed)
    for bits in (4, 8):
        gs = 32
        w = _rand_bf16(rng, (2, gs))
        wq, s, b = quantize(w, gs, bits)
        for r in range(2):
            sc, bi = _bf16_value(s[r, 0]), _bf16_value(b[r, 0])
            for k in range(gs):
                wv = _bf16_value(w[r, k])
                q = _code(wq[r], k, bits)
                mine = abs(wv - (sc * q + bi))
                best = min(abs(wv - (sc * c + bi)) for c in range(2 ** bits))
                assert mine <= best + sc * Fraction(1, 2 ** 14), (bits, r, k, q)


def check_quantize_scale_rounding(quantize, seed=2):
    """scale is the smallest bf16 >= fp32(fp32(max-min)/(2^b-1)), bias the min,
    so the grid covers the group; the minimum maps to code 0 and the maximum
    to the code nearest (max-min)/scale."""
    rng = np.random.default_rng(seed)
    for bits in (4, 8):
        gs = 64
        w = _rand_bf16(rng, (8, gs))
        wq, s, b = quantize(w, gs, bits)
        wf = f32_from_bf16_bits(w)
        for r in range(8):
            lo, hi = wf[r].min(), wf[r].max()
            target = Fraction(float(np.float32(np.float32(hi - lo) / np.float32(2 ** bits - 1))))
            sc = _bf16_value(s[r, 0])
            assert sc >= target
            below = _bf16_value(int(s[r, 0]) - 1)        # next bf16 down (positive pattern)
            assert below < target, "scale is not the smallest bf16 >= the fp32 quotient"
            assert _bf16_value(b[r, 0]) == Fraction(float(lo))
            assert sc * (2 ** bits - 1) + _bf16_value(b[r, 0]) >= Fraction(float(hi))
            k_lo, k_hi = int(np.argmin(wf[r])), int(np.argmax(wf[r]))
            assert _code(wq[r], k_lo, bits) == 0
            top = _code(wq[r], k_hi, bits)
            # rounding up to bf16 raises the scale by less than 2^-7 relative
            # (7 stored mantissa bits), so the top code is rint((hi-lo)/scale)
            # >= rint(qmax / (1 + 2^-7)): 15 at 4 bits, 253..255 at 8 bits
            quot = Fraction(float(hi)) - Fraction(float(lo))
            quot /= sc
            assert abs(quot - top) <= Fraction(1, 2) + Fraction(1, 2 ** 14), (top, float(quot))
            assert top >= (15 if bits == 4 else 253), top


def check_quantize_closed_form(quantize, seed=3):
    """Weights on an exact grid b + s*q (s a power of two, every group using
    codes 0 and 2^b-1) quantise back to exactly (s, b, q)."""
    rng = np.random.default_rng(seed)
    for bits in (4, 8):
        gs = 32
        rows, G = 4, 3
        qmax = 2 ** bits - 1
        q = rng.integers(0, qmax + 1, size=(rows, G, gs))
        q[:, :, 0] = 0
        q[:, :, 1] = qmax
        e = rng.integers(-6, 0, size=(rows, G))
        s = np.ldexp(1.0, e)                                   # powers of two
        # bias = -c*s with an integer c < 256: then w/s is an integer of
        # magnitude <= 255, so every grid weight is exact in bf16
        b = -s * rng.integers(0, 256, size=(rows, G))
        w = b[..., None] + s[..., None] * q
        wb = bf16_bits_from_f32(w.astype(np.float32).reshape(rows, G * gs))
        assert np.array_equal(f32_from_bf16_bits(wb).astype(np.float64).reshape(rows, G, gs), w), \
            "fixture not exactly representable"
        wq, sb, bb = quantize(wb, gs, bits)
        assert np.array_equal(f32_from_bf16_bits(sb).astype(np.float64), s)
        assert np.array_equal(f32_from_bf16_bits(bb).astype(np.float64), b)
        for r in range(rows):
            for k in range(G * gs):
                assert _code(wq[r], k, bits) == q[r, k // gs, k % gs]


def check_quantize_constant_group(quantize):
    for bits in (4, 8):
        w = bf16_bits_from_f32(np.full((2, 64), -3.25, np.float32))
        w[1, 32:] = bf16_bits_from_f32(np.float32(7.5))
        wq, s, b = quantize(w, 32, bits)
        assert (s == 0).all()
        assert np.array_equal(f32_from_bf16_bits(b), np.array([[-3.25, -3.25], [-3.25, 7.5]], np.float32))
        assert (wq == 0).all()
        # signed zeros: a group of +-0.0 has scale and bias pattern +0.0
        z = np.zeros((1, 32), np.uint16)
        z[0, ::3] = 0x8000
        wq, s, b = quantize(z, 32, bits)
        assert int(s[0, 0]) == 0 and int(b[0, 0]) == 0 and (wq == 0).all()


# --- route --------------------------------------------------------------------------

def _route_cases(seed=4):
    rng = np.random.default_rng(seed)
    yield rng.integers(0, 8, size=(64, 2)), 8                  # uniform
    yield rng.integers(0, 64, size=(300, 8)), 64
    p = np.arange(1, 17, dtype=float) ** -2.5
    yield rng.choice(16, size=(200, 2), p=p / p.sum()), 16     # skewed, empty experts likely
    yield np.full((17, 3), 5), 9                               # all to one expert
    yield np.sort(rng.integers(0, 32, size=500)).reshape(500, 1), 32   # already sorted
    yield np.zeros((0, 4), dtype=np.int64), 4                  # empty


def check_route_library(route):
    """Equal to numpy's stable argsort and bincount/cumsum (library special case)."""
    for idx, E in _route_cases():
        counts, offsets, perm = route(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def check_route_brute_force(route):
    """perm is the concatenation over e of the pair indices routed to e, ascending."""
    for idx, E in _route_cases(seed=5):
        _, offsets, perm = route(idx, E)
        flat = [int(v) for v in idx.reshape(-1)]
        expect = [i for e in range(E) for i, v in enumerate(flat) if v == e]
        assert list(perm) == expect
        for e in range(E):
            assert offsets[e + 1] - offsets[e] == flat.count(e)
        if flat == sorted(flat):
            assert list(perm) == list(range(len(flat)))


# --- products -------------------------------------------------------------------------

def _grid_weights(rng, E, N, K, gs, bits):
    """Weights exactly on their own quantisation grid (see closed-form check)."""
    G = K // gs
    qmax = 2 ** bits - 1
    q = rng.integers(0, qmax + 1, size=(E, N, G, gs))
    q[..., 0] = 0
    q[..., 1] = qmax
    s = np.ldexp(1.0, rng.integers(-6, -1, size=(E, N, G)))
    b = -s * rng.integers(0, 256, size=(E, N, G))   # w/s integer, |w/s| <= 255
    w = (b[..., None] + s[..., None] * q).reshape(E, N, K)
    wb = bf16_bits_from_f32(w.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(wb).astype(np.float64), w)
    return wb, w


def check_gather_grid_exact(quantize, gather_qmm, seed=6):
    """For weights on their grid, gather_qmm of the quantised weight equals a
    plain float64 matmul of the *original* weight against the routed expert
    (numpy's matmul: a library special case; no dequantisation formula)."""
    rng = np.random.default_rng(seed)
    for bits, gs in ((4, 64), (8, 32)):
        T, A, E, K, N = 5, 3, 4, 128, 24
        wb, w = _grid_weights(rng, E, N, K, gs, bits)
        x = _rand_bf16(rng, (T, A, 1, K))
        idx = rng.integers(0, E, size=(T, A))
        wq, s, b = quantize(wb, gs, bits)
        out = gather_qmm(x, wq, s, b, idx, gs, bits)
        xf = f32_from_bf16_bits(x).astype(np.float64)
        ref = np.einsum("tamk,tank->tamn", xf, w[idx])
        assert out.shape == (T, A, 1, N)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        # x broadcast over A (Ax == 1)
        x1 = x[:, :1]
        out1 = gather_qmm(x1, wq, s, b, idx, gs, bits)
        ref1 = np.einsum("tmk,tank->tamn", f32_from_bf16_bits(x1[:, 0]).astype(np.float64), w[idx])
        assert np.allclose(out1, ref1, rtol=1e-12, atol=1e-12)


def check_gather_exact_rational(quantize, gather_qmm, seed=7):
    """Tiny shapes against an exact rational sum over the unpacked codes: the
    fp64 result lies within gamma_K * sum|x||w_hat| of the exact value."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 3, 2, 3, 64, 5, 32, 4
    w = _rand_bf16(rng, (E, N, K))
    x = _rand_bf16(rng, (T, A, 2, K))                  # M = 2 rows per pair
    idx = rng.integers(0, E, size=(T, A))
    wq, s, b = quantize(w, gs, bits)
    out = gather_qmm(x, wq, s, b, idx, gs, bits)
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            for m in range(2):
                xs = [_bf16_value(v) for v in x[t, a, m]]
                for n in range(N):
                    wh = _exact_dequant_row(wq[e, n], s[e, n], b[e, n], gs, bits, K)
                    exact = sum(xi * wi for xi, wi in zip(xs, wh))
                    mag = sum(abs(xi * wi) for xi, wi in zip(xs, wh))
                    assert abs(Fraction(float(out[t, a, m, n])) - exact) <= gamma * mag + Fraction(1, 10 ** 300)


def check_gather_one_hot(quantize, gather_qmm, dequant_exact=None, seed=8):
    """x row = unit vector e_k selects column k of the routed expert's grid
    weight exactly."""
    rng = np.random.default_rng(seed)
    E, N, K, gs, bits = 3, 16, 64, 32, 4
    wb, w = _grid_weights(rng, E, N, K, gs, bits)
    wq, s, b = quantize(wb, gs, bits)
    ks = [0, 5, 31, 32, 63]
    T = len(ks)
    xf = np.zeros((T, 1, 1, K), np.float32)
    for t, k in enumerate(ks):
        xf[t, 0, 0, k] = 1.0
    idx = np.array([[t % E] for t in range(T)])
    out = gather_qmm(bf16_bits_from_f32(xf), wq, s, b, idx, gs, bits)
    for t, k in enumerate(ks):
        assert np.array_equal(out[t, 0, 0], w[t % E, :, k])


def check_gather_all_equal_is_qmm(quantize, gather_qmm, qmm, seed=9):
    """All indices equal to e: gather_qmm equals the dense product against W[e]."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 6, 2, 3, 128, 12, 64, 4
    w = _rand_bf16(rng, (E, N, K))
    x = _rand_bf16(rng, (T, A, 1, K))
    wq, s, b = quantize(w, gs, bits)
    for e in range(E):
        idx = np.full((T, A), e)
        out = gather_qmm(x, wq, s, b, idx, gs, bits)
        ref = qmm(x.reshape(T * A, K), wq[e], s[e], b[e], gs, bits)
        assert np.allclose(out.reshape(T * A, N), ref, rtol=1e-13, atol=1e-13)


def check_gather_permutation(quantize, gather_qmm, seed=10):
    """Permuting the (token, slot) pairs permutes the outputs."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 7, 2, 4, 64, 8, 32, 8
    w = _rand_bf16(rng, (E, N, K))
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    wq, s, b = quantize(w, gs, bits)
    out = gather_qmm(x, wq, s, b, idx, gs, bits).reshape(T * A, N)
    p = rng.permutation(T * A)
    x2 = x.reshape(T * A, 1, 1, K)[p]
    idx2 = idx.reshape(-1)[p].reshape(T * A, 1)
    out2 = gather_qmm(x2, wq, s, b, idx2, gs, bits).reshape(T * A, N)
    assert np.allclose(out2, out[p], rtol=1e-13, atol=1e-13)


def check_integer_exact(quantize, gather_qmm, seed=11):
    """8-bit, scale 1, bias 0 (codes are the weights), small integer x: the
    result is an exact integer matmul."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 4, 2, 3, 64, 6, 32, 8
    qw = rng.integers(0, 256, size=(E, N, K))
    qw[..., 0] = 0
    qw[..., 1] = 255
    qw[..., 32] = 0
    qw[..., 33] = 255                                         # every group spans 0..255
    wb = bf16_bits_from_f32(qw.astype(np.float32))
    xi = rng.integers(-8, 9, size=(T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    wq, s, b = quantize(wb, gs, bits)
    out = gather_qmm(bf16_bits_from_f32(xi.astype(np.float32)), wq, s, b, idx, gs, bits)
    ref = np.einsum("tamk,tank->tamn", xi, qw[idx])
    assert np.array_equal(out, ref.astype(np.float64))


# --- the unquantised gather (bf16 weights) -------------------------------------------

def check_gather_mm_exact_rational(gather_mm, seed=12):
    """Tiny shapes against exact rational dot products of the bf16 values
    (decoded bit by bit here): the fp64 result lies within gamma_K of the
    exact sum.  M = 2 rows per pair, x per slot (Ax = A)."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 3, 2, 3, 48, 5
    w = _rand_bf16(rng, (E, N, K))
    x = _rand_bf16(rng, (T, A, 2, K))
    idx = rng.integers(0, E, size=(T, A))
    out = gather_mm(x, w, idx)
    assert out.shape == (T, A, 2, N)
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            for m in range(2):
                xs = [_bf16_value(v) for v in x[t, a, m]]
                for n in range(N):
                    ws = [_bf16_value(v) for v in w[e, n]]
                    exact = sum(xi * wi for xi, wi in zip(xs, ws))
                    mag = sum(abs(xi * wi) for xi, wi in zip(xs, ws))
                    assert abs(Fraction(float(out[t, a, m, n])) - exact) <= gamma * mag + Fraction(1, 10 ** 300)


def check_gather_mm_integer_exact(gather_mm, seed=13):
    """Small integers in x and w (exact in bf16): an exact integer matmul, with
    one x row per token broadcast over its slots (Ax = 1)."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 5, 3, 4, 40, 7
    wi = rng.integers(-16, 17, size=(E, N, K))
    xi = rng.integers(-8, 9, size=(T, 1, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    out = gather_mm(bf16_bits_from_f32(xi.astype(np.float32)),
                    bf16_bits_from_f32(wi.astype(np.float32)), idx)
    ref = np.einsum("tmk,tank->tamn", xi[:, 0], wi[idx])
    assert np.array_equal(out, ref.astype(np.float64))


def check_gather_mm_one_hot(gather_mm, seed=14):
    """x row = unit vector e_k returns column k of the routed expert's weight."""
    rng = np.random.default_rng(seed)
    E, N, K = 3, 9, 32
    w = _rand_bf16(rng, (E, N, K))
    ks = [0, 7, 16, 31]
    xf = np.zeros((len(ks), 1, 1, K), np.float32)
    for t, k in enumerate(ks):
        xf[t, 0, 0, k] = 1.0
    idx = np.array([[(t * 2) % E] for t in range(len(ks))])
    out = gather_mm(bf16_bits_from_f32(xf), w, idx)
    for t, k in enumerate(ks):
        assert np.array_equal(out[t, 0, 0], f32_from_bf16_bits(w[(t * 2) % E, :, k]).astype(np.float64))


def check_gather_mm_is_gather_qmm_on_grid(quantize, gather_qmm, gather_mm, seed=15):
    """Weights that lie exactly on a quantisation grid are the same matrix in
    both forms: the bf16 gather and the quantised gather agree to rounding."""
    rng = np.random.default_rng(seed)
    E, N, K, gs, bits = 3, 8, 64, 32, 4
    wb, _ = _grid_weights(rng, E, N, K, gs, bits)
    wq, s, b = quantize(wb, gs, bits)
    T, A = 5, 2
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    assert np.allclose(gather_mm(x, wb, idx), gather_qmm(x, wq, s, b, idx, gs, bits),
                       rtol=1e-13, atol=1e-13)


# --- the gated activation and the fused gate/up product -----------------------------------

def check_glu_odd_part(glu_act):
    """act(z) - act(-z) = z for both readings: z(sigmoid(z) + sigmoid(-z)) for
    SiLU, z/2 (2 + erf(u) + erf(-u)) for GELU (erf is odd)."""
    z = np.concatenate([np.linspace(-30, 30, 241), [1e-300, 1e-8, 0.5, 3.25]])
    for act in (1, 2):
        d = glu_act(z, act) - glu_act(-z, act) - z
        assert np.all(np.abs(d) <= 4 * np.finfo(np.float64).eps * np.maximum(1, np.abs(z))), act


def check_glu_library(glu_act, seed=16):
    """Against scipy's logistic and error functions on random points."""
    import scipy.special as sp
    z = np.random.default_rng(seed).normal(0, 4, 500)
    assert np.allclose(glu_act(z, 1), z * sp.expit(z), rtol=1e-14, atol=1e-300)
    assert np.allclose(glu_act(z, 2), 0.5 * z * (1 + sp.erf(z / np.sqrt(2))), rtol=1e-14, atol=1e-300)


def check_glu_closed_forms(glu_act):
    """SiLU(ln 3) = (3/4) ln 3 (sigmoid(ln 3) = 3/4); act(0) = 0; GELU at
    z = sqrt(2) * erfinv-free points: GELU(0) = 0, GELU(z) -> z and -> 0 in
    the tails; SiLU(-ln 3) = -(1/4) ln 3."""
    l3 = np.log(3.0)
    assert abs(glu_act(l3, 1) - 0.75 * l3) <= 1e-15
    assert abs(glu_act(-l3, 1) + 0.25 * l3) <= 1e-15
    for act in (1, 2):
        assert glu_act(0.0, act) == 0.0
        assert abs(glu_act(40.0, act) - 40.0) <= 1e-12
        assert abs(glu_act(-40.0, act)) <= 1e-12


def check_gather_qmm_glu_up_ones(quantize, gather_qmm, gather_qmm_glu, seed=17):
    """Up weights whose groups are constant 1.0 (scale 0, bias 1: exact ones)
    make u the plain row sum of x, so h = act(gate product) * sum_k x; with a
    gate of constant zero groups h vanishes.  Each expert routes both
    projections the same way."""
    rng = np.random.default_rng(seed)
    T, A, E, K, F, gs, bits = 5, 3, 4, 128, 6, 64, 4
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    wg = _rand_bf16(rng, (E, F, K))
    ones = bf16_bits_from_f32(np.ones((E, F, K), np.float32))
    zeros = bf16_bits_from_f32(np.zeros((E, F, K), np.float32))
    gq = quantize(wg, gs, bits)
    uq = quantize(ones, gs, bits)
    zq = quantize(zeros, gs, bits)
    rowsum = np.array([[sum(float(_bf16_value(v)) for v in x[t, a, 0]) for a in range(A)]
                       for t in range(T)])
    g = gather_qmm(x, *gq, idx, gs, bits)[..., 0, :]
    for act, f in ((1, lambda z: z / (1 + np.exp(-z))),
                   (2, lambda z: 0.5 * z * (1 + np.vectorize(__import__("math").erf)(z / np.sqrt(2))))):
        h = gather_qmm_glu(x, gq, uq, idx, gs, bits, act)[..., 0, :]
        assert np.allclose(h, f(g) * rowsum[..., None], rtol=1e-12, atol=1e-12), act
        h0 = gather_qmm_glu(x, zq, gq, idx, gs, bits, act)
        assert np.all(h0 == 0), act


# --- MXFP4 (OCP MX v1.0: E2M1 codes, 32-element blocks, E8M0 scales) ----------------

# The OCP specification's table of E2M1 magnitudes for codes 0..7; codes 8..15
# are their negatives.
_E2M1_TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
               Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _e2m1(code: int) -> Fraction:
    v = _E2M1_TABLE[code & 7]
    return -v if code & 8 else v


def check_mx_e2m1_table(e2m1_value):
    """The 16 code values against the specification's table, -0 included."""
    got = e2m1_value(np.arange(16))
    for c in range(16):
        assert Fraction(float(got[c])) == _e2m1(c), c
        assert bool(np.signbit(got[c])) == bool(c & 8), c


def _mx_grid_block(rng, s):
    """32 weights on the E2M1 grid scaled by 2^s, one of them +-6 (so that the
    block's amax fixes the shared exponent s)."""
    codes = rng.integers(0, 16, size=32)
    codes[rng.integers(0, 32)] = 7 + 8 * int(rng.integers(0, 2))
    vals = np.array([float(_e2m1(int(c))) for c in codes]) * 2.0 ** s
    return codes, vals


def check_mx_quantize_on_grid(quantize_mx, dequantize_mx, seed=20):
    """Weights already on a block's grid come back as the same codes (read
    from the words by this module's own unpacking), the same exponent and
    the same values."""
    rng = np.random.default_rng(seed)
    R, NB = 6, 4
    codes = np.zeros((R, NB * 32), np.int64)
    vals = np.zeros((R, NB * 32), np.float64)
    shifts = rng.integers(-40, 41, size=(R, NB))
    for r in range(R):
        for b in range(NB):
            codes[r, 32 * b:32 * b + 32], vals[r, 32 * b:32 * b + 32] = _mx_grid_block(rng, int(shifts[r, b]))
    wb = bf16_bits_from_f32(vals.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(wb).astype(np.float64), vals)
    wq, sc = quantize_mx(wb)
    assert wq.shape == (R, NB * 4) and wq.dtype == np.uint32
    assert sc.shape == (R, NB) and sc.dtype == np.uint8
    assert np.array_equal(sc.astype(np.int64), shifts + 127)
    for r in range(R):
        for k in range(NB * 32):
            c = _code(wq[r], k, 4)
            # +0 codes as 0; the grid has no -0 here unless drawn as code 8
            assert _e2m1(c) == _e2m1(int(codes[r, k])), (r, k)
    assert np.array_equal(dequantize_mx(wq, sc), vals)


def _mx_case_weights(rng):
    """Blocks at several magnitudes, a zero block, a -0 block, ties planted
    on the grid's midpoints and values past 6 X."""
    rows = []
    for std in (1.0, 3e-3, 250.0, 2.0 ** -100):
        rows.append(rng.standard_normal(128) * std)
    zero = np.zeros(128)
    zero[32:64] = -0.0
    zero[64:96] = rng.standard_normal(32) * 1e-2
    zero[96:128] = rng.integers(-7, 8, size=32) * 2.0 ** -133     # bf16 subnormals
    rows.append(zero)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)
    ties[1::2] *= -1
    tie_row = np.concatenate([ties, ties * 2.0 ** -3, ties * 2.0 ** 9,
                              np.array([7.0, 6.5, 7.5, 5.5] + [0.1] * 28)])
    rows.append(tie_row)
    return bf16_bits_from_f32(np.array(rows, dtype=np.float32))


def check_mx_quantize_nearest(quantize_mx, seed=21):
    """Brute force in exact rationals: every code is a nearest scaled E2M1
    value to its weight (ties to the even mantissa), weights past 6 X
    saturate to +-6 X, and the sign bit is the weight's."""
    rng = np.random.default_rng(seed)
    wb = _mx_case_weights(rng)
    wq, sc = quantize_mx(wb)
    R, K = wb.shape
    for r in range(R):
        for k in range(K):
            v = _bf16_value(int(wb[r, k]))
            X = Fraction(2) ** (int(sc[r, k // 32]) - 127)
            c = _code(wq[r], k, 4)
            assert bool(c & 8) == bool(int(wb[r, k]) & 0x8000), (r, k)
            got = _e2m1(c) * X
            if abs(v) > 6 * X:
                assert got == (6 * X if v > 0 else -6 * X), (r, k)
                continue
            dists = [abs(v - _e2m1(d) * X) for d in range(16)]
            best = min(dists)
            assert abs(v - got) == best, (r, k, v, got)
            ties = {d & 7 for d in range(16) if dists[d] == best}
            if len(ties) > 1:
                assert (c & 1) == 0, (r, k, "tie not to even")


def check_mx_scale_rule(quantize_mx, seed=22):
    """The shared exponent: 4 <= amax / X < 8 for every block whose amax is
    within the clamp, e = 0 for an all-zero block and for blocks below
    2^-125, and the largest bf16 block takes e = 252."""
    rng = np.random.default_rng(seed)
    wb = _mx_case_weights(rng)
    big = np.full((1, 128), np.float32(3.0e38))
    wb = np.concatenate([wb, bf16_bits_from_f32(big)])
    _, sc = quantize_mx(wb)
    R, K = wb.shape
    for r in range(R):
        for b in range(K // 32):
            amax = max(abs(_bf16_value(int(v))) for v in wb[r, 32 * b:32 * b + 32])
            e = int(sc[r, b])
            if amax == 0 or amax < Fraction(2) ** -125:
                assert e == 0, (r, b, e)
            else:
                ratio = amax / Fraction(2) ** (e - 127)
                assert 4 <= ratio < 8, (r, b, e, float(ratio))
    assert int(sc[-1, 0]) == 252


def check_mx_gather_exact_rational(gather_qmm_mx, seed=23):
    """Random codes and scales against exact rational dot products of the
    decoded weights: the fp64 result lies within gamma_K of the exact sum."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 3, 2, 3, 96, 4
    wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = rng.integers(110, 140, size=(E, N, K // 32)).astype(np.uint8)
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    out = gather_qmm_mx(x, wq, sc, idx)
    assert out.shape == (T, A, 1, N)
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            xs = [_bf16_value(v) for v in x[t, a, 0]]
            for n in range(N):
                ws = [_e2m1(_code(wq[e, n], k, 4)) * Fraction(2) ** (int(sc[e, n, k // 32]) - 127)
                      for k in range(K)]
                exact = sum(xi * wi for xi, wi in zip(xs, ws))
                mag = sum(abs(xi * wi) for xi, wi in zip(xs, ws))
                assert abs(Fraction(float(out[t, a, 0, n])) - exact) <= gamma * mag + Fraction(1, 10 ** 300)


def check_mx_gather_is_gather_mm(quantize_mx, gather_qmm_mx, gather_mm, seed=24):
    """Scaled E2M1 values are bf16 values: the MX gather equals the bf16
    gather of the same matrix, with x per slot and broadcast."""
    rng = np.random.default_rng(seed)
    E, N, K, T, A = 3, 6, 64, 5, 2
    vals = np.zeros((E, N, K))
    for e in range(E):
        for n in range(N):
            for b in range(K // 32):
                vals[e, n, 32 * b:32 * b + 32] = _mx_grid_block(rng, int(rng.integers(-8, 9)))[1]
    wb = bf16_bits_from_f32(vals.astype(np.float32))
    wq, sc = quantize_mx(wb)
    idx = rng.integers(0, E, size=(T, A))
    for Ax in (A, 1):
        x = _rand_bf16(rng, (T, Ax, 1, K))
        assert np.allclose(gather_qmm_mx(x, wq, sc, idx), gather_mm(x, wb, idx), rtol=1e-13, atol=1e-300)


# --- MXFP8 (OCP MX v1.0: E4M3 codes, 32-element blocks, E8M0 scales) ----------------

def _torch_e4m3_values():
    """The 256 E4M3 code values as torch's float8_e4m3fn decodes them (a
    library special case: torch implements the OCP E4M3 format)."""
    import torch
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_frac(code: int) -> Fraction:
    v = _torch_e4m3_values()[code]
    assert np.isfinite(v)
    return Fraction(float(v))


def check_mx8_e4m3_table(e4m3_value):
    """All 256 code values, NaN included, against torch's float8_e4m3fn."""
    ref = _torch_e4m3_values()
    got = e4m3_value(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def _mx8_weights(rng):
    rows = [rng.standard_normal(128) * s for s in (1.0, 3e-3, 250.0, 2.0 ** -60)]
    ties = []
    for m in range(8):               # midpoints between consecutive mantissas, two binades
        for e in (0, 3):
            ties.append((1 + (m + 0.5) / 8) * 2.0 ** e)
    ties = np.array(ties[:16] + [448.0, 460.0, 464.0, 470.0, 500.0, 511.0, 2.0 ** -10,
                                 3 * 2.0 ** -11, 5 * 2.0 ** -12, 1e-5, 0.0, -0.0, 1.0, -1.0,
                                 -464.0, -2.0 ** -10])
    ties[1::3] *= -1
    row = np.concatenate([ties, ties * 2.0 ** -20, ties * 2.0 ** 30, ties * 0.5])
    rows.append(row)
    zero = np.zeros(128)
    zero[32:64] = -0.0
    zero[64:96] = rng.integers(-50, 50, 32) * 2.0 ** -133
    zero[96:128] = rng.standard_normal(32) * 1e-3
    rows.append(zero)
    return bf16_bits_from_f32(np.array(rows, dtype=np.float32))


def check_mx8_quantize_library(quantize_mx, seed=25):
    """Given each block's exponent, every code is torch's float8_e4m3fn cast
    (round to nearest even) of w / X where |w / X| <= 464, and +-448 beyond
    (saturation, where torch's cast gives NaN); plus the scale rule
    2^8 <= amax / X < 2^9, e = 0 for zero and sub-2^-118 blocks."""
    import torch
    rng = np.random.default_rng(seed)
    wb = _mx8_weights(rng)
    wq, sc = quantize_mx(wb, "e4m3")
    R, K = wb.shape
    assert wq.shape == (R, K // 4) and sc.shape == (R, K // 32)
    w = f32_from_bf16_bits(wb).astype(np.float64)
    X = np.ldexp(1.0, np.repeat(sc.astype(np.int64), 32, axis=-1) - 127)
    y = w / X
    codes = np.array([[_code(wq[r], k, 8) for k in range(K)] for r in range(R)])
    cast = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    small = np.abs(y) <= 464
    assert np.array_equal(codes[small], cast[small])
    assert np.all((codes[~small] & 0x7F) == 0x7E)
    assert np.array_equal(codes >> 7, np.signbit(w).astype(np.int64))
    for r in range(R):
        for b in range(K // 32):
            amax = max(abs(_bf16_value(int(v))) for v in wb[r, 32 * b:32 * b + 32])
            e = int(sc[r, b])
            if amax == 0 or amax < Fraction(2) ** -118:
                assert e == 0, (r, b, e)
            else:
                assert 256 <= amax / Fraction(2) ** (e - 127) < 512, (r, b, e)


def check_mx8_quantize_on_grid(quantize_mx, dequantize_mx, seed=26):
    """Blocks of E4M3 values scaled by 2^s, each holding a +-448, come back as
    the same codes and exponents; -0 aside, the values are unchanged."""
    rng = np.random.default_rng(seed)
    R, NB = 5, 3
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    codes = np.zeros((R, NB * 32), np.int64)
    shifts = rng.integers(-30, 31, size=(R, NB))
    for r in range(R):
        for b in range(NB):
            cs = rng.choice(finite, 32)
            cs[rng.integers(0, 32)] = 0x7E | (0x80 * int(rng.integers(0, 2)))
            codes[r, 32 * b:32 * b + 32] = cs
    vals = np.array([[float(_e4m3_frac(int(c))) for c in row] for row in codes])
    vals *= np.ldexp(1.0, np.repeat(shifts, 32, axis=-1))
    wb = bf16_bits_from_f32(vals.astype(np.float32))
    wq, sc = quantize_mx(wb, "e4m3")
    assert np.array_equal(sc.astype(np.int64), shifts + 127)
    for r in range(R):
        for k in range(NB * 32):
            assert _e4m3_frac(_code(wq[r], k, 8)) == _e4m3_frac(int(codes[r, k])), (r, k)
    assert np.array_equal(dequantize_mx(wq, sc, "e4m3"), vals)


def check_mx8_gather_exact_rational(gather_qmm_mx, seed=27):
    """Random finite codes and exponents against exact rational products."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 3, 2, 3, 64, 4
    byte = rng.integers(0, 256, size=(E, N, K))
    byte[(byte & 0x7F) == 0x7F] = 0x11
    wq = np.zeros((E, N, K // 4), np.uint32)
    for j in range(4):
        wq |= byte[..., j::4].astype(np.uint32) << np.uint32(8 * j)
    sc = rng.integers(115, 135, size=(E, N, K // 32)).astype(np.uint8)
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    out = gather_qmm_mx(x, wq, sc, idx, "e4m3")
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            xs = [_bf16_value(v) for v in x[t, a, 0]]
            for n in range(N):
                ws = [_e4m3_frac(int(byte[e, n, k])) * Fraction(2) ** (int(sc[e, n, k // 32]) - 127)
                      for k in range(K)]
                exact = sum(xi * wi for xi, wi in zip(xs, ws))
                mag = sum(abs(xi * wi) for xi, wi in zip(xs, ws))
                assert abs(Fraction(float(out[t, a, 0, n])) - exact) <= gamma * mag + Fraction(1, 10 ** 300)


def check_mx8_gather_is_gather_mm(quantize_mx, gather_qmm_mx, gather_mm, seed=28):
    """Scaled E4M3 values are bf16 values: the MXFP8 gather of quantised
    weights equals the bf16 gather of their dequantised bf16 matrix."""
    rng = np.random.default_rng(seed)
    E, N, K, T, A = 3, 5, 96, 4, 2
    w = _rand_bf16(rng, (E, N, K))
    wq, sc = quantize_mx(w, "e4m3")
    vals = np.zeros((E, N, K))
    for e in range(E):
        for n in range(N):
            for k in range(K):
                vals[e, n, k] = float(_e4m3_frac(_code(wq[e, n], k, 8))) * 2.0 ** (int(sc[e, n, k // 32]) - 127)
    wb = bf16_bits_from_f32(vals.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(wb).astype(np.float64), vals)
    idx = rng.integers(0, E, size=(T, A))
    for Ax in (A, 1):
        x = _rand_bf16(rng, (T, Ax, 1, K))
        assert np.allclose(gather_qmm_mx(x, wq, sc, idx, "e4m3"), gather_mm(x, wb, idx),
                           rtol=1e-13, atol=1e-300)


# --- NVFP4 (E2M1 codes, an E4M3 scale per 16 weights, an fp32 scale per tensor) ------

def _f32_ulp(v: float) -> Fraction:
    v = abs(float(v))
    e = np.frexp(np.float32(v))[1] if v > 0 else -125
    return Fraction(2) ** (int(e) - 24)


def _nv_weights(rng):
    t0 = rng.standard_normal((4, 64))
    t0[1, :16] *= 1e-3                     # a block far below the tensor's largest
    t0[2, 16:32] = 0.0                     # a zero block
    t0[3, :16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75,
                  -2.5, -3.5, -5.0, -6.0]
    t1 = rng.standard_normal((4, 64)) * 300.0
    t2 = np.zeros((4, 64))                 # an all-zero tensor
    return bf16_bits_from_f32(np.stack([t0, t1, t2]).astype(np.float32))


def check_nv_scales(quantize_nv, seed=29):
    """g is amax / 2688 rounded to fp32 (exact rationals; 1 for a zero tensor);
    each block scale code is torch's float8_e4m3fn cast of the fp32 quotient
    amax_block / 6 / g, and its value lies within half an E4M3 quantum (plus
    the two fp32 roundings) of the exact quotient."""
    import torch
    rng = np.random.default_rng(seed)
    wb = _nv_weights(rng)
    wq, sc, g = quantize_nv(wb)
    Tn, R, K = wb.shape
    assert wq.shape == (Tn, R, K // 8) and sc.shape == (Tn, R, K // 16) and g.shape == (Tn,)
    assert g.dtype == np.float32
    for t in range(Tn):
        amax = max(abs(_bf16_value(int(v))) for v in wb[t].reshape(-1))
        if amax == 0:
            assert g[t] == 1.0
            assert np.all(sc[t] == 0)
            continue
        assert abs(Fraction(float(g[t])) - amax / 2688) <= _f32_ulp(g[t]) / 2
        for r in range(R):
            for b in range(K // 16):
                ab = max(abs(_bf16_value(int(v))) for v in wb[t, r, 16 * b:16 * b + 16])
                q = np.float32(np.float32(float(ab)) / np.float32(6.0)) / g[t]
                cast = torch.tensor([float(q)], dtype=torch.float32).to(torch.float8_e4m3fn)
                assert int(sc[t, r, b]) == int(cast.view(torch.uint8)[0]), (t, r, b)
                exact = ab / 6 / Fraction(float(g[t]))
                v = _e4m3_frac(int(sc[t, r, b]))
                quantum = Fraction(2) ** -9 if exact < Fraction(2) ** -6 else \
                    Fraction(2) ** (int(np.floor(np.log2(float(exact)))) - 3)
                assert abs(v - exact) <= quantum / 2 + 4 * _f32_ulp(float(exact)), (t, r, b)


def check_nv_codes_nearest(quantize_nv, seed=30):
    """Brute force in exact rationals: each code's value times the block's
    divisor d = fp32(e4m3(s) * g) is a nearest of the 16 (up to the fp32
    rounding of w / d), saturating at +-6 d, with the weight's sign bit."""
    rng = np.random.default_rng(seed)
    wb = _nv_weights(rng)
    wq, sc, g = quantize_nv(wb)
    Tn, R, K = wb.shape
    for t in range(Tn):
        for r in range(R):
            for k in range(K):
                w = _bf16_value(int(wb[t, r, k]))
                c = _code(wq[t, r], k, 4)
                assert bool(c & 8) == bool(int(wb[t, r, k]) & 0x8000), (t, r, k)
                d = Fraction(float(np.float32(float(_e4m3_frac(int(sc[t, r, k // 16])))) * g[t]))
                if d == 0:
                    assert c & 7 == 0
                    continue
                got = _e2m1(c) * d
                if abs(w) > 6 * d:
                    assert got == (6 * d if w > 0 else -6 * d), (t, r, k)
                    continue
                best = min(abs(w - _e2m1(j) * d) for j in range(16))
                assert abs(w - got) <= best + 6 * d * Fraction(1, 2 ** 22), (t, r, k)


def check_nv_gather_exact_rational(gather_qmm_nv, seed=31):
    """Random codes, block scales and tensor scales against exact rationals."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 3, 2, 3, 64, 4
    wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = rng.integers(0, 0x7F, size=(E, N, K // 16)).astype(np.uint8)
    g = (rng.random(E) * 3 + 0.1).astype(np.float32)
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    out = gather_qmm_nv(x, wq, sc, g, idx)
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            xs = [_bf16_value(v) for v in x[t, a, 0]]
            for n in range(N):
                ws = [_e2m1(_code(wq[e, n], k, 4)) * _e4m3_frac(int(sc[e, n, k // 16])) *
                      Fraction(float(g[e])) for k in range(K)]
                exact = sum(xi * wi for xi, wi in zip(xs, ws))
                mag = sum(abs(xi * wi) for xi, wi in zip(xs, ws))
                assert abs(Fraction(float(out[t, a, 0, n])) - exact) <= 2 * gamma * mag + Fraction(1, 10 ** 300)


def check_nv_gather_is_scaled_gather_mm(quantize_nv, gather_qmm_nv, gather_mm, seed=32):
    """e2m1(q) * e4m3(s) is a bf16 value: the NVFP4 gather equals the tensor
    scale of each routed expert times the bf16 gather of those products."""
    rng = np.random.default_rng(seed)
    E, N, K, T, A = 3, 5, 64, 4, 2
    w = _rand_bf16(rng, (E, N, K))
    wq, sc, g = quantize_nv(w)
    vals = np.zeros((E, N, K))
    for e in range(E):
        for n in range(N):
            for k in range(K):
                vals[e, n, k] = float(_e2m1(_code(wq[e, n], k, 4)) * _e4m3_frac(int(sc[e, n, k // 16])))
    wb = bf16_bits_from_f32(vals.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(wb).astype(np.float64), vals)
    idx = rng.integers(0, E, size=(T, A))
    for Ax in (A, 1):
        x = _rand_bf16(rng, (T, Ax, 1, K))
        ref = gather_mm(x, wb, idx) * g.astype(np.float64)[idx][:, :, None, None]
        assert np.allclose(gather_qmm_nv(x, wq, sc, g, idx), ref, rtol=1e-13, atol=1e-300)


def check_quantize_ties(quantize):
    """Quotients exactly halfway between two codes round to the even code
    (reading 3: rint of the fp32 quotient).  Groups spanning [0, 15] (4-bit)
    or [0, 255] (8-bit) have scale exactly 1, or a power of two times 1 when
    the group is scaled by 2^j; every k + 1/2 below is a bf16 value, so its
    quotient is exactly the tie."""
    for bits, gs in ((4, 32), (8, 32)):
        qmax = 2 ** bits - 1
        top = 15 if bits == 4 else 127                     # k + 1/2 exact in bf16 for k < top
        halves = [k + 0.5 for k in range(top)]
        for j in (0, -3, 4):
            rows = []
            for start in range(0, len(halves), gs - 2):
                vals = [0.0, float(qmax)] + halves[start:start + gs - 2]
                vals += [0.0] * (gs - len(vals))
                rows.append(vals)
            w = np.ldexp(np.array(rows, np.float64), j).astype(np.float32)
            wb = bf16_bits_from_f32(w)
            assert np.array_equal(f32_from_bf16_bits(wb), w)
            wq, s, b = quantize(wb, gs, bits)
            assert np.all(f32_from_bf16_bits(s) == np.float32(2.0 ** j)) and np.all(b == 0)
            for r, vals in enumerate(rows):
                for k, v in enumerate(vals):
                    want = int(v) if v == int(v) else (int(v) if int(v) % 2 == 0 else int(v) + 1)
                    assert _code(wq[r], k, bits) == want, (bits, j, v)


MX_QUANTIZE_CHECKS = [check_mx_quantize_on_grid, check_mx_quantize_nearest, check_mx_scale_rule]


QUANTIZE_CHECKS = [check_quantize_worked_examples, check_quantize_round_trip,
                   check_quantize_argmin, check_quantize_scale_rounding,
                   check_quantize_closed_form, check_quantize_constant_group,
                   check_quantize_ties]
ROUTE_CHECKS = [check_route_library, check_route_brute_force]
GATHER_CHECKS = [check_gather_grid_exact, check_gather_exact_rational, check_gather_one_hot,
                 check_gather_permutation, check_integer_exact]
GATHER_MM_CHECKS = [check_gather_mm_exact_rational, check_gather_mm_integer_exact,
                    check_gather_mm_one_hot]
GLU_CHECKS = [check_glu_odd_part, check_glu_library, check_glu_closed_forms]


# --- the row-sampling helpers (used where the full product is too large) ---------------

def _row_samples(rng, n_pairs, N, count=48):
    """Flat pair indices and columns: the corners plus random ones."""
    pairs = np.concatenate([[0, n_pairs - 1, 0, n_pairs - 1], rng.integers(0, n_pairs, count)])
    cols = np.concatenate([[0, 0, N - 1, N - 1], rng.integers(0, N, count)])
    return pairs, cols


def _check_rows(full_fn, rows_fn, draw_x, T, A, N, rng):
    """rows_fn(x, pairs, cols) against full_fn(x) at sampled (pair, column)
    points, for one x row per routed pair (Ax = A) and one per token (Ax = 1)."""
    for Ax in (A, 1):
        x = draw_x(Ax)
        full = full_fn(x).reshape(T * A, N)
        pairs, cols = _row_samples(rng, T * A, N)
        part = rows_fn(x, pairs, cols)
        assert np.allclose(part, full[pairs, cols], rtol=1e-12, atol=1e-12), Ax


def check_gather_qmm_rows(quantize, gather_qmm, gather_qmm_rows, seed=33):
    """gather_qmm_rows equals the (separately pinned) full gather_qmm."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 7, 3, 5, 128, 21
    for bits, gs in ((4, 64), (8, 32)):
        wq, s, b = quantize(_rand_bf16(rng, (E, N, K)), gs, bits)
        idx = rng.integers(0, E, size=(T, A))
        _check_rows(lambda x: gather_qmm(x, wq, s, b, idx, gs, bits),
                    lambda x, p, c: gather_qmm_rows(x, wq, s, b, idx, gs, bits, p, c),
                    lambda Ax: _rand_bf16(rng, (T, Ax, 1, K)), T, A, N, rng)


def check_gather_mm_rows(gather_mm, gather_mm_rows, seed=34):
    """gather_mm_rows equals the (separately pinned) full gather_mm."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 6, 4, 3, 96, 17
    w = _rand_bf16(rng, (E, N, K))
    idx = rng.integers(0, E, size=(T, A))
    _check_rows(lambda x: gather_mm(x, w, idx),
                lambda x, p, c: gather_mm_rows(x, w, idx, p, c),
                lambda Ax: _rand_bf16(rng, (T, Ax, 1, K)), T, A, N, rng)


def check_gather_qmm_mx_rows(quantize_mx, gather_qmm_mx, gather_qmm_mx_rows, seed=35):
    """gather_qmm_mx_rows equals the (separately pinned) full gather_qmm_mx,
    for both element formats."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 5, 3, 4, 128, 19
    for elem in ("e2m1", "e4m3"):
        wq, sc = quantize_mx(_rand_bf16(rng, (E, N, K)), elem)
        idx = rng.integers(0, E, size=(T, A))
        _check_rows(lambda x: gather_qmm_mx(x, wq, sc, idx, elem),
                    lambda x, p, c: gather_qmm_mx_rows(x, wq, sc, idx, p, c, elem),
                    lambda Ax: _rand_bf16(rng, (T, Ax, 1, K)), T, A, N, rng)


def check_gather_qmm_nv_rows(quantize_nv, gather_qmm_nv, gather_qmm_nv_rows, seed=36):
    """gather_qmm_nv_rows equals the (separately pinned) full gather_qmm_nv;
    the experts' weights differ in scale, so a wrong expert's tensor scale
    shows."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N = 5, 3, 4, 64, 18
    w = np.concatenate([_rand_bf16(rng, (1, N, K), std) for std in (1.0, 0.01, 30.0, 0.2)])
    wq, sc, g = quantize_nv(w)
    idx = rng.integers(0, E, size=(T, A))
    _check_rows(lambda x: gather_qmm_nv(x, wq, sc, g, idx),
                lambda x, p, c: gather_qmm_nv_rows(x, wq, sc, g, idx, p, c),
                lambda Ax: _rand_bf16(rng, (T, Ax, 1, K)), T, A, N, rng)


# --- transpose = False: the stored [E, K, N] stack applied untransposed ---------------

def check_gather_nn_grid_exact(quantize, gather_qmm, seed=37):
    """Weights on their own grid along N: gather_qmm(transpose=False) equals a
    plain float64 product x @ w[e] of the *original* [E, K, N] weight (numpy;
    no dequantisation formula), for Ax = A and Ax = 1.  K != N, so an
    operand applied transposed cannot pass."""
    rng = np.random.default_rng(seed)
    for bits, gs in ((4, 64), (8, 32)):
        T, A, E, K, N = 5, 3, 4, 96, 128
        wb, w = _grid_weights(rng, E, K, N, gs, bits)             # [E, K, N], grid along N
        idx = rng.integers(0, E, size=(T, A))
        wq, s, b = quantize(wb, gs, bits)
        for Ax in (A, 1):
            x = _rand_bf16(rng, (T, Ax, 1, K))
            out = gather_qmm(x, wq, s, b, idx, gs, bits, transpose=False)
            xf = f32_from_bf16_bits(x).astype(np.float64)
            xa = xf if Ax == A else np.repeat(xf, A, axis=1)
            ref = np.einsum("tamk,takn->tamn", xa, w[idx])
            assert out.shape == (T, A, 1, N)
            assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), (bits, Ax)


def check_gather_nn_exact_rational(quantize, gather_qmm, seed=38):
    """Tiny shapes against exact rational sums over the codes unpacked here:
    out[t, a, m, n] = sum_k x * (s[e, k, n / gs] * q[e, k, n] + b[e, k, n / gs])
    within gamma_K of the exact value; M = 2 rows per pair."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 3, 2, 3, 24, 64, 32, 4
    w = _rand_bf16(rng, (E, K, N))
    x = _rand_bf16(rng, (T, A, 2, K))
    idx = rng.integers(0, E, size=(T, A))
    wq, s, b = quantize(w, gs, bits)
    out = gather_qmm(x, wq, s, b, idx, gs, bits, transpose=False)
    assert out.shape == (T, A, 2, N)
    gamma = Fraction(K, 2 ** 53 - K)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            wh = [[_bf16_value(s[e, k, n // gs]) * _code(wq[e, k], n, bits)
                   + _bf16_value(b[e, k, n // gs]) for n in range(N)] for k in range(K)]
            for m in range(2):
                xs = [_bf16_value(v) for v in x[t, a, m]]
                for n in range(N):
                    terms = [xs[k] * wh[k][n] for k in range(K)]
                    exact = sum(terms)
                    mag = sum(abs(v) for v in terms)
                    assert abs(Fraction(float(out[t, a, m, n])) - exact) <= gamma * mag + Fraction(1, 10 ** 300)


def check_gather_nn_one_hot(quantize, gather_qmm, seed=39):
    """x row = unit vector e_k returns row k of the routed expert's grid
    weight (all N columns) exactly."""
    rng = np.random.default_rng(seed)
    E, K, N, gs, bits = 3, 40, 64, 32, 4
    wb, w = _grid_weights(rng, E, K, N, gs, bits)
    wq, s, b = quantize(wb, gs, bits)
    ks = [0, 7, 20, 39]
    xf = np.zeros((len(ks), 1, 1, K), np.float32)
    for t, k in enumerate(ks):
        xf[t, 0, 0, k] = 1.0
    idx = np.array([[(t + 1) % E] for t in range(len(ks))])
    out = gather_qmm(bf16_bits_from_f32(xf), wq, s, b, idx, gs, bits, transpose=False)
    for t, k in enumerate(ks):
        assert np.array_equal(out[t, 0, 0], w[(t + 1) % E, k, :])


def check_gather_nn_all_equal_is_qmm(quantize, gather_qmm, qmm, seed=40):
    """All indices equal to e: the transpose=False gather equals the dense
    transpose=False product against the stored W[e]."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 6, 2, 3, 72, 128, 64, 4
    w = _rand_bf16(rng, (E, K, N))
    x = _rand_bf16(rng, (T, A, 1, K))
    wq, s, b = quantize(w, gs, bits)
    for e in range(E):
        out = gather_qmm(x, wq, s, b, np.full((T, A), e), gs, bits, transpose=False)
        ref = qmm(x.reshape(T * A, K), wq[e], s[e], b[e], gs, bits, transpose=False)
        assert ref.shape == (T * A, N)
        assert np.allclose(out.reshape(T * A, N), ref, rtol=1e-13, atol=1e-13)


def check_gather_nn_is_gather_mm(quantize, gather_qmm, gather_mm, seed=41):
    """On weights exactly on their grid, the transpose=False gather of the
    stored [E, K, N] stack equals the (separately pinned) bf16 gather of the
    same matrix laid out as [E, N, K]."""
    rng = np.random.default_rng(seed)
    E, K, N, gs, bits = 3, 64, 96, 32, 8
    wb, _ = _grid_weights(rng, E, K, N, gs, bits)
    wq, s, b = quantize(wb, gs, bits)
    T, A = 5, 2
    x = _rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    w_nk = np.ascontiguousarray(wb.transpose(0, 2, 1))
    assert np.allclose(gather_qmm(x, wq, s, b, idx, gs, bits, transpose=False),
                       gather_mm(x, w_nk, idx), rtol=1e-13, atol=1e-13)


GATHER_NN_CHECKS = [check_gather_nn_grid_exact, check_gather_nn_exact_rational,
                    check_gather_nn_one_hot]
