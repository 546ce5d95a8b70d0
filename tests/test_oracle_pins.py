"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.QUANTIZE_CHECKS, ids=lambda f: f.__name__)
def test_quantize(check):
    check(oracle.quantize)


@pytest.mark.parametrize("check", pins.ROUTE_CHECKS, ids=lambda f: f.__name__)
def test_route(check):
    check(oracle.route)


@pytest.mark.parametrize("check", pins.GATHER_CHECKS, ids=lambda f: f.__name__)
def test_gather(check):
    check(oracle.quantize, oracle.gather_qmm)


@pytest.mark.parametrize("check", pins.GATHER_MM_CHECKS, ids=lambda f: f.__name__)
def test_gather_mm(check):
    check(oracle.gather_mm)


def test_gather_mm_is_gather_qmm_on_grid():
    pins.check_gather_mm_is_gather_qmm_on_grid(oracle.quantize, oracle.gather_qmm, oracle.gather_mm)


@pytest.mark.parametrize("check", pins.GLU_CHECKS, ids=lambda f: f.__name__)
def test_glu_act(check):
    check(oracle.glu_act)


def test_gather_qmm_glu_up_ones():
    pins.check_gather_qmm_glu_up_ones(oracle.quantize, oracle.gather_qmm, oracle.gather_qmm_glu)


def test_gather_all_equal_is_qmm():
    pins.check_gather_all_equal_is_qmm(oracle.quantize, oracle.gather_qmm, oracle.qmm)


def test_route_rejects_out_of_range():
    import numpy as np
    with pytest.raises(ValueError):
        oracle.route(np.array([[0, 3]]), 3)
    with pytest.raises(ValueError):
        oracle.route(np.array([[-1]]), 3)


def test_gather_rows_matches_full():
    import numpy as np
    import workloads
    c = workloads.tiny_moe(seed=3)
    wq, s, b = oracle.quantize(c.w, c.group_size, c.bits)
    full = oracle.gather_qmm(c.x, wq, s, b, c.idx, c.group_size, c.bits).reshape(-1, c.N)
    rng = np.random.default_rng(0)
    pairs = rng.integers(0, c.T * c.A, 40)
    cols = rng.integers(0, c.N, 40)
    part = oracle.gather_qmm_rows(c.x, wq, s, b, c.idx, c.group_size, c.bits, pairs, cols)
    assert np.array_equal(part, full[pairs, cols])


def test_mx_e2m1_table():
    pins.check_mx_e2m1_table(oracle.e2m1_value)


def test_mx_quantize_on_grid():
    pins.check_mx_quantize_on_grid(oracle.quantize_mx, oracle.dequantize_mx)


def test_mx_quantize_nearest():
    pins.check_mx_quantize_nearest(oracle.quantize_mx)


def test_mx_scale_rule():
    pins.check_mx_scale_rule(oracle.quantize_mx)


def test_mx_gather_exact_rational():
    pins.check_mx_gather_exact_rational(oracle.gather_qmm_mx)


def test_mx_gather_is_gather_mm():
    pins.check_mx_gather_is_gather_mm(oracle.quantize_mx, oracle.gather_qmm_mx, oracle.gather_mm)


def test_mx_quantize_rejects():
    import numpy as np
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((2, 48), np.uint16))              # K not a multiple of 32
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.full((1, 32), 0x7F80, np.uint16))       # +inf


def test_mx8_e4m3_table():
    pins.check_mx8_e4m3_table(oracle.e4m3_value)


def test_mx8_quantize_library():
    pins.check_mx8_quantize_library(oracle.quantize_mx)


def test_mx8_quantize_on_grid():
    pins.check_mx8_quantize_on_grid(oracle.quantize_mx, oracle.dequantize_mx)


def test_mx8_gather_exact_rational():
    pins.check_mx8_gather_exact_rational(oracle.gather_qmm_mx)


def test_mx8_gather_is_gather_mm():
    pins.check_mx8_gather_is_gather_mm(oracle.quantize_mx, oracle.gather_qmm_mx, oracle.gather_mm)


def test_mx_quantize_rejects_unknown_element():
    import numpy as np
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((1, 32), np.uint16), "e5m2")


def test_nv_scales():
    pins.check_nv_scales(oracle.quantize_nv)


def test_nv_codes_nearest():
    pins.check_nv_codes_nearest(oracle.quantize_nv)


def test_nv_gather_exact_rational():
    pins.check_nv_gather_exact_rational(oracle.gather_qmm_nv)


def test_nv_gather_is_scaled_gather_mm():
    pins.check_nv_gather_is_scaled_gather_mm(oracle.quantize_nv, oracle.gather_qmm_nv,
                                             oracle.gather_mm)


def test_nv_quantize_rejects():
    import numpy as np
    with pytest.raises(ValueError):
        oracle.quantize_nv(np.zeros((1, 2, 24), np.uint16))          # K % 16
    with pytest.raises(ValueError):
        oracle.quantize_nv(np.zeros((2, 32), np.uint16))             # not [T, R, K]
