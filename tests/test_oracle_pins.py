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


def test_gather_qmm_rows():
    pins.check_gather_qmm_rows(oracle.quantize, oracle.gather_qmm, oracle.gather_qmm_rows)


def test_gather_mm_rows():
    pins.check_gather_mm_rows(oracle.gather_mm, oracle.gather_mm_rows)


def test_gather_qmm_mx_rows():
    pins.check_gather_qmm_mx_rows(oracle.quantize_mx, oracle.gather_qmm_mx,
                                  oracle.gather_qmm_mx_rows)


def test_gather_qmm_nv_rows():
    pins.check_gather_qmm_nv_rows(oracle.quantize_nv, oracle.gather_qmm_nv,
                                  oracle.gather_qmm_nv_rows)


@pytest.mark.parametrize("check", pins.GATHER_NN_CHECKS, ids=lambda f: f.__name__)
def test_gather_nn(check):
    check(oracle.quantize, oracle.gather_qmm)


def test_gather_nn_all_equal_is_qmm():
    pins.check_gather_nn_all_equal_is_qmm(oracle.quantize, oracle.gather_qmm, oracle.qmm)


def test_gather_nn_is_gather_mm():
    pins.check_gather_nn_is_gather_mm(oracle.quantize, oracle.gather_qmm, oracle.gather_mm)


def test_gather_rejects_mismatched_features():
    import numpy as np
    x = np.zeros((2, 1, 1, 64), np.uint16)
    wq, s, b = oracle.quantize(np.zeros((3, 32, 128), np.uint16), 64, 4)   # [E, K=32, N=128]
    with pytest.raises(ValueError):
        oracle.gather_qmm(x, wq, s, b, np.zeros((2, 1), np.int32), 64, 4, transpose=False)


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
