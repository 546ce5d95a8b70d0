"""The fp32 C oracle (oracle/mq_oracle_c.c) against what the mathematics fixes.

The quantiser and the routing are pinned by the same checks as the fp64
oracle (worked examples, brute-force nearest codes, closed forms, numpy's
stable argsort, ...): their results do not depend on the accumulation
precision.  The product is pinned by checks that hold exactly in fp32
(one-hot rows, an exact integer product, all-equal indices = the dense
product, permutation of the pairs) and by exact rational sums with the fp32
error bound: |out - exact| <= (gamma_{K+1}) * sum |x| |w_hat| with
gamma_n = n u / (1 - n u), u = 2^-24 (one rounding per fused step of the
k-ascending sum, one for the dequantised weight).  Each planted mistake
(a copy of the library built with one MQ_MUTANT_* define) fails one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import pins
import workloads
from oracle import c_oracle

U = Fraction(1, 2 ** 24)


@pytest.fixture(scope="module")
def co():
    try:
        return c_oracle.Oracle()
    except RuntimeError as e:                  # no C compiler
        pytest.skip(str(e))


def _gamma(n):
    return n * U / (1 - n * U)


def check_c_exact_rational(quantize, gather_qmm, seed=40):
    """Tiny shapes, both code widths, M = 2 rows per pair and x broadcast
    over the slots: within the fp32 bound of the exact rational sum."""
    rng = np.random.default_rng(seed)
    for bits, gs, K in ((4, 32, 64), (8, 64, 128)):
        T, A, E, N = 3, 2, 3, 5
        w = pins._rand_bf16(rng, (E, N, K))
        for Ax in (A, 1):
            x = pins._rand_bf16(rng, (T, Ax, 2, K))
            idx = rng.integers(0, E, size=(T, A))
            wq, s, b = quantize(w, gs, bits)
            out = gather_qmm(x, wq, s, b, idx, gs, bits)
            g = _gamma(K + 1)
            for t in range(T):
                for a in range(A):
                    e = int(idx[t, a])
                    for m in range(2):
                        xs = [pins._bf16_value(v) for v in x[t, a if Ax > 1 else 0, m]]
                        for n in range(N):
                            wh = pins._exact_dequant_row(wq[e, n], s[e, n], b[e, n], gs, bits, K)
                            exact = sum(xi * wi for xi, wi in zip(xs, wh))
                            mag = sum(abs(xi * wi) for xi, wi in zip(xs, wh))
                            assert abs(Fraction(float(out[t, a, m, n])) - exact) <= g * mag


def check_c_untransposed_rational(quantize, gather_qmm, seed=41):
    """transpose = False (the stored [E, K, N] applied as x @ w_hat): within
    the fp32 bound of the exact rational sum."""
    rng = np.random.default_rng(seed)
    T, A, E, K, N, gs, bits = 3, 2, 2, 24, 64, 32, 4
    w = pins._rand_bf16(rng, (E, K, N))                   # quantised along N
    x = pins._rand_bf16(rng, (T, A, 1, K))
    idx = rng.integers(0, E, size=(T, A))
    wq, s, b = quantize(w, gs, bits)
    out = gather_qmm(x, wq, s, b, idx, gs, bits, transpose=False)
    g = _gamma(K + 1)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            xs = [pins._bf16_value(v) for v in x[t, a, 0]]
            cols = [pins._exact_dequant_row(wq[e, k], s[e, k], b[e, k], gs, bits, N) for k in range(K)]
            for n in range(N):
                exact = sum(xs[k] * cols[k][n] for k in range(K))
                mag = sum(abs(xs[k] * cols[k][n]) for k in range(K))
                assert abs(Fraction(float(out[t, a, 0, n])) - exact) <= g * mag


def _gather_checks(o):
    return [
        lambda: check_c_exact_rational(o.quantize, o.gather_qmm),
        lambda: check_c_untransposed_rational(o.quantize, o.gather_qmm),
        lambda: pins.check_gather_one_hot(o.quantize, o.gather_qmm),
        lambda: pins.check_integer_exact(o.quantize, o.gather_qmm),
        lambda: pins.check_gather_all_equal_is_qmm(o.quantize, o.gather_qmm, o.qmm),
        lambda: pins.check_gather_permutation(o.quantize, o.gather_qmm),
    ]


def _all_checks(o):
    return ([lambda c=c: c(o.quantize) for c in pins.QUANTIZE_CHECKS] +
            [lambda c=c: c(o.route) for c in pins.ROUTE_CHECKS] + _gather_checks(o))


@pytest.mark.parametrize("check", pins.QUANTIZE_CHECKS, ids=lambda c: c.__name__)
def test_c_quantize_pins(co, check):
    check(co.quantize)


@pytest.mark.parametrize("check", pins.ROUTE_CHECKS, ids=lambda c: c.__name__)
def test_c_route_pins(co, check):
    check(co.route)


@pytest.mark.parametrize("i", range(6))
def test_c_gather_pins(co, i):
    _gather_checks(co)[i]()


def test_c_agrees_with_fp64_oracle(co):
    """Codes and routing bit for bit with the fp64 oracle (each pinned on its
    own); the product within the fp32 bound of the fp64 one, on a shape with
    several groups, experts and a ragged routing."""
    case = workloads.gather_case("c-vs-fp64", 48, 4, 6, 512, 96, seed=42, routing="zipf")
    for gs, bits in ((64, 4), (32, 8)):
        a = co.quantize(case.w, gs, bits)
        b = oracle.quantize(case.w, gs, bits)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        got = co.gather_qmm(case.x, *a, case.idx, gs, bits).astype(np.float64)
        ref = oracle.gather_qmm(case.x, *b, case.idx, gs, bits)
        W = oracle.dequantize(*b, gs, bits)
        xf = oracle.bf16_to_f32(case.x).astype(np.float64)
        mag = np.einsum("tamk,tank->tamn", np.abs(xf), np.abs(W[case.idx]))
        K = case.K
        assert (np.abs(got - ref) <= float(_gamma(K + 1)) * mag + 1e-300).all()
    for x, y in zip(co.route(case.idx, case.E), oracle.route(case.idx, case.E)):
        assert np.array_equal(x, y)


def test_c_thread_count_does_not_matter(co):
    case = workloads.gather_case("c-threads", 64, 2, 4, 256, 64, seed=43)
    wq, s, b = co.quantize(case.w, 64, 4)
    n = co.threads()
    try:
        co.threads(1)
        one = co.gather_qmm(case.x, wq, s, b, case.idx, 64, 4)
    finally:
        co.threads(n)
    many = co.gather_qmm(case.x, wq, s, b, case.idx, 64, 4)
    assert np.array_equal(one, many)


def test_c_rejects_bad_indices(co):
    case = workloads.gather_case("c-bad", 4, 2, 3, 64, 16, seed=44)
    wq, s, b = co.quantize(case.w, 64, 4)
    idx = case.idx.copy()
    idx[1, 0] = 3
    with pytest.raises(ValueError):
        co.gather_qmm(case.x, wq, s, b, idx, 64, 4)
    with pytest.raises(ValueError):
        co.route(idx, 3)


@pytest.mark.parametrize("mutant", c_oracle.MUTANTS)
def test_c_mutant_is_caught(co, mutant):
    """A copy of the C oracle with one planted mistake fails a pin."""
    m = c_oracle.Oracle(mutant)
    failed = []
    for i, chk in enumerate(_all_checks(m)):
        try:
            chk()
        except (AssertionError, ValueError):
            failed.append(i)
    assert failed, f"no pin catches {mutant}"
