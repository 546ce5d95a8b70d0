"""Planted mistakes in the oracle (CPU only).

Each case edits one plausible bug into a private copy of the oracle's source
(a dropped term, a wrong rounding, a wrong index, a swapped operand) and
checks that at least one pin in ``pins.py`` rejects the copy.  The real oracle
is never modified.
"""
import inspect
import types

import pytest

import pins
from oracle import mq_oracle

MUTANTS = [
    # (id, original snippet, planted mistake, pin family)
    ("scale-rne", "scale_bits = bf16_round_up((span / levels).astype(np.float32))",
     "scale_bits = ((((span / levels).astype(np.float32)).view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)",
     "quantize"),
    ("levels-2^b", "levels = np.float32(2 ** bits - 1)", "levels = np.float32(2 ** bits)", "quantize"),
    ("bias-max", "lo = (w.min(axis=-1) + np.float32(0)).astype(np.float32)",
     "lo = (w.max(axis=-1) + np.float32(0)).astype(np.float32)", "quantize"),
    ("floor-codes", "q = np.rint(quot)", "q = np.floor(quot)", "quantize"),
    ("pack-reversed", "words |= q[:, j::per] << np.uint32(j * bits)",
     "words |= q[:, j::per] << np.uint32((per - 1 - j) * bits)", "quantize"),
    ("unpack-reversed", "out[..., j::per] = (wq >> np.uint32(j * bits)) & mask",
     "out[..., j::per] = (wq >> np.uint32((per - 1 - j) * bits)) & mask", "gather"),
    ("dequant-no-bias", "    return s * q + b\n", "    return s * q\n", "gather"),
    ("dequant-group-axis", "s = np.repeat(bf16_to_f32(scales).astype(np.float64), group_size, axis=-1)",
     "s = np.tile(bf16_to_f32(scales).astype(np.float64), group_size)", "gather"),
    ("route-unstable", "    for i, e in enumerate(flat):\n        perm[cursor[e]] = i",
     "    for i, e in reversed(list(enumerate(flat))):\n        perm[cursor[e]] = i", "route"),
    ("route-inclusive-scan", "    cursor = offsets[:E]", "    cursor = offsets[1:] + [0]", "route"),
    ("gather-ignores-slot", "out[t, a] = x[t, a if Ax == A else 0] @ W[e]\n    return out\n\n\ndef gather_qmm_rows",
     "out[t, a] = x[t, 0] @ W[e]\n    return out\n\n\ndef gather_qmm_rows", "gather"),
    ("gather-wrong-expert", "            e = int(idx[t, a])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e]\n    return out\n\n\ndef gather_qmm_rows",
     "            e = int(idx[t, 0])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e]\n    return out\n\n\ndef gather_qmm_rows", "gather"),
    ("mm-wrong-expert", "            e = int(idx[t, a])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_mm_rows",
     "            e = int(idx[t, 0])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_mm_rows", "gather_mm"),
    ("gather-x-times-w", "out[t, a] = x[t, a if Ax == A else 0] @ W[e]\n    return out\n\n\ndef gather_qmm_rows",
     "out[t, a] = (x[t, a if Ax == A else 0] @ W[e]) * (1 + 2.0 ** -20)\n    return out\n\n\ndef gather_qmm_rows", "gather"),
    # the bf16 gather
    ("mm-ignores-slot", "out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_mm_rows",
     "out[t, a] = x[t, 0] @ W[e].T\n    return out\n\n\ndef gather_mm_rows", "gather_mm"),
    ("mm-weight-not-transposed", "    W = bf16_to_f32(w_bits).astype(np.float64)                    # [E, N, K]",
     "    W = bf16_to_f32(w_bits).astype(np.float64)[:, ::-1, :]       # [E, N, K]", "gather_mm"),
    # the gated activation and the fused product
    ("silu-sign", "            return z / (1.0 + np.exp(-z))", "            return z / (1.0 + np.exp(z))", "glu"),
    ("gelu-no-sqrt2", "        return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))",
     "        return 0.5 * z * (1.0 + erf(z))", "glu"),
    ("glu-act-on-up", "    return glu_act(g, act) * u", "    return g * glu_act(u, act)", "glu"),
    ("glu-acts-swapped", "ACT_SILU, ACT_GELU = 1, 2", "ACT_SILU, ACT_GELU = 2, 1", "glu"),
    # MXFP4
    ("mx-emax-1", "    emax, bits = (2, 4) if elem == \"e2m1\" else (8, 8)",
     "    emax, bits = (1, 4) if elem == \"e2m1\" else (8, 8)", "mx"),
    ("mx-ties-away", "r = np.minimum(np.rint(mag / quantum) * quantum, 6.0)",
     "r = np.minimum(np.floor(mag / quantum + 0.5) * quantum, 6.0)", "mx"),
    ("mx-no-saturation", "r = np.minimum(np.rint(mag / quantum) * quantum, 6.0)",
     "r = np.rint(mag / quantum) * quantum", "mx"),
    ("mx-subnormal-quantum", "quantum = np.where(mag < 1.0, 0.5, np.ldexp(1.0, ex - 1))",
     "quantum = np.where(mag < 1.0, 0.25, np.ldexp(1.0, ex - 1))", "mx"),
    ("mx-sign-dropped", "return code | np.where(neg, np.uint32(8), np.uint32(0))",
     "return code | np.where(mag < 0, np.uint32(8), np.uint32(0))", "mx"),
    ("mx-nibbles-reversed", "        words |= codes[:, j::per] << np.uint32(bits * j)",
     "        words |= codes[:, j::per] << np.uint32(32 - bits - bits * j)", "mx"),
    ("mx-scale-bias-126", "    return value(codes) * np.ldexp(1.0, e - 127)",
     "    return value(codes) * np.ldexp(1.0, e - 126)", "mx"),
    ("mx-e2m1-exp-bias", "mag = np.where(ex == 0, man * 0.5, np.ldexp(1.0 + man / 2.0, ex - 1))",
     "mag = np.where(ex == 0, man * 0.5, np.ldexp(1.0 + man / 2.0, ex))", "mx"),
    ("mx-zero-block-scale", "shared = np.where(amax > 0, ex.astype(np.int64) - 1 - emax, -127)",
     "shared = np.where(amax > 0, ex.astype(np.int64) - 1 - emax, 0)", "mx"),
    ("mx-wrong-expert", "            e = int(idx[t, a])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_qmm_mx_rows",
     "            e = int(idx[t, 0])\n            if not 0 <= e < E:\n                raise ValueError(f\"expert index {e} outside [0, {E})\")\n            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_qmm_mx_rows", "mx"),
    ("mx-ignores-slot", "out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_qmm_mx_rows",
     "out[t, a] = x[t, 0] @ W[e].T\n    return out\n\n\ndef gather_qmm_mx_rows", "mx"),
    # MXFP8
    ("mx8-emax-7", "    emax, bits = (2, 4) if elem == \"e2m1\" else (8, 8)",
     "    emax, bits = (2, 4) if elem == \"e2m1\" else (7, 8)", "mx8"),
    ("mx8-subnormal-quantum", "quantum = np.where(mag < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 3))",
     "quantum = np.where(mag < 2.0 ** -6, 2.0 ** -10, np.ldexp(1.0, ex - 3))", "mx8"),
    ("mx8-quantum-binade", "quantum = np.where(mag < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 3))",
     "quantum = np.where(mag < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 2))", "mx8"),
    ("mx8-no-saturation", "r = np.minimum(np.rint(mag / quantum) * quantum, 448.0)",
     "r = np.minimum(np.rint(mag / quantum) * quantum, 480.0)", "mx8"),
    ("mx8-ties-away", "r = np.minimum(np.rint(mag / quantum) * quantum, 448.0)",
     "r = np.minimum(np.floor(mag / quantum + 0.5) * quantum, 448.0)", "mx8"),
    ("mx8-sign-dropped", "return code | np.where(neg, np.uint32(0x80), np.uint32(0))",
     "return code | np.where(mag < 0, np.uint32(0x80), np.uint32(0))", "mx8"),
    ("mx8-exp-bias-6", "mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, np.ldexp(1.0 + man / 8.0, ex - 7))",
     "mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, np.ldexp(1.0 + man / 8.0, ex - 6))", "mx8"),
    ("mx8-subnormal-exp", "mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, np.ldexp(1.0 + man / 8.0, ex - 7))",
     "mag = np.where(ex == 0, man / 8.0 * 2.0 ** -7, np.ldexp(1.0 + man / 8.0, ex - 7))", "mx8"),
    ("mx8-bytes-reversed", "        words |= codes[:, j::per] << np.uint32(bits * j)",
     "        words |= codes[:, j::per] << np.uint32(32 - bits - bits * j)", "mx8"),
    # NVFP4
    ("nv-2048", "    g = np.where(amax_t > 0, amax_t / f32(2688.0), f32(1.0)).astype(np.float32)",
     "    g = np.where(amax_t > 0, amax_t / f32(2048.0), f32(1.0)).astype(np.float32)", "nv"),
    ("nv-no-div6", "    sb = ((amax_b / f32(6.0)).astype(np.float32) / g[:, None, None]).astype(np.float32)",
     "    sb = ((amax_b / f32(4.0)).astype(np.float32) / g[:, None, None]).astype(np.float32)", "nv"),
    ("nv-dequant-no-g", "    return e2m1_value(codes) * s * g\n",
     "    return e2m1_value(codes) * s\n", "nv"),
    ("nv-block-scale-axis", "    s = np.repeat(e4m3_value(np.asarray(scales, dtype=np.int64)), NV_BLOCK, axis=-1)",
     "    s = np.tile(e4m3_value(np.asarray(scales, dtype=np.int64)), NV_BLOCK)", "nv"),
    ("nv-divisor-no-g", "    d = (s_val * g[:, None, None]).astype(np.float32)",
     "    d = (s_val * np.float32(1.0)).astype(np.float32)", "nv"),
    ("nv-sign-dropped", "    y = np.where(d[..., None] > 0, y, np.copysign(np.float32(0), blocks))",
     "    y = np.abs(np.where(d[..., None] > 0, y, np.float32(0)))", "nv"),
    ("nv-zero-tensor-g", "    g = np.where(amax_t > 0, amax_t / f32(2688.0), f32(1.0)).astype(np.float32)",
     "    g = np.where(amax_t > 0, amax_t / f32(2688.0), f32(2.0)).astype(np.float32)", "nv"),
    ("nv-wrong-expert", "            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T\n    return out\n\n\ndef gather_qmm_nv_rows",
     "            out[t, a] = x[t, a if Ax == A else 0] @ W[(e + 1) % E].T\n    return out\n\n\ndef gather_qmm_nv_rows", "nv"),
    ("mm-bf16-as-fp16", "    W = bf16_to_f32(w_bits).astype(np.float64)                    # [E, N, K]",
     "    W = w_bits.view(np.float16).astype(np.float64)                 # [E, N, K]", "gather_mm"),
    # the row-sampling helpers (each against its pinned full product)
    ("qmm-rows-wrong-expert", "        e = int(idx[t, a])\n        wrow = dequantize(wq[e, c:c + 1]",
     "        e = int(idx[t, 0])\n        wrow = dequantize(wq[e, c:c + 1]", "rows"),
    ("qmm-rows-wrong-column", "wrow = dequantize(wq[e, c:c + 1], scales[e, c:c + 1], biases[e, c:c + 1],",
     "wrow = dequantize(wq[e, c - 1:c], scales[e, c - 1:c], biases[e, c - 1:c],", "rows"),
    ("mm-rows-wrong-expert", "        e = int(idx[t, a])\n        wrow = bf16_to_f32(w_bits[e, c])",
     "        e = int(idx[t, 0])\n        wrow = bf16_to_f32(w_bits[e, c])", "rows"),
    ("mm-rows-wrong-column", "wrow = bf16_to_f32(w_bits[e, c]).astype(np.float64)",
     "wrow = bf16_to_f32(w_bits[e, c - 1]).astype(np.float64)", "rows"),
    ("mx-rows-wrong-expert", "        e = int(idx[t, a])\n        wrow = dequantize_mx(",
     "        e = int(idx[t, 0])\n        wrow = dequantize_mx(", "rows"),
    ("mx-rows-wrong-column", "wrow = dequantize_mx(wq[e, c:c + 1], scales[e, c:c + 1], elem)[0]",
     "wrow = dequantize_mx(wq[e, c:c + 1], scales[e, c - 1:c], elem)[0]", "rows"),
    ("mx-rows-slot", "        res[j] = _x_f64(x_bits[t, a if Ax == A else 0, 0]) @ wrow\n    return res\n\n\n# --- NVFP4",
     "        res[j] = _x_f64(x_bits[t, 0, 0]) @ wrow\n    return res\n\n\n# --- NVFP4", "rows"),
    ("nv-rows-wrong-expert", "wrow = dequantize_nv(wq[e:e + 1, c:c + 1], scales[e:e + 1, c:c + 1], gscale[e:e + 1])[0, 0]",
     "wrow = dequantize_nv(wq[e:e + 1, c:c + 1], scales[e:e + 1, c:c + 1], gscale[:1])[0, 0]", "rows"),
    ("nv-rows-wrong-column", "wrow = dequantize_nv(wq[e:e + 1, c:c + 1], scales[e:e + 1, c:c + 1], gscale[e:e + 1])[0, 0]",
     "wrow = dequantize_nv(wq[e:e + 1, c - 1:c], scales[e:e + 1, c - 1:c], gscale[e:e + 1])[0, 0]", "rows"),
    # transpose = False (the stored stack applied untransposed)
    ("nn-applied-transposed", "    return W.transpose(0, 2, 1) if transpose else W",
     "    return W.transpose(0, 2, 1)", "nn"),
    ("nn-roles-swapped", "    return W.transpose(0, 2, 1) if transpose else W",
     "    return W if transpose else W.transpose(0, 2, 1)", "nn"),
    ("qmm-nn-transposed", "    return _x_f64(x_bits) @ (W.T if transpose else W)",
     "    return _x_f64(x_bits) @ W.T", "nn"),
]


def _mutant(original: str, planted: str) -> types.ModuleType:
    src = inspect.getsource(mq_oracle)
    assert src.count(original) == 1, f"snippet not found exactly once: {original!r}"
    mod = types.ModuleType("mq_oracle_mutant")
    exec(compile(src.replace(original, planted), "<mutant>", "exec"), mod.__dict__)
    return mod


def _run_family(mod, family):
    if family == "quantize":
        for check in pins.QUANTIZE_CHECKS:
            check(mod.quantize)
    elif family == "route":
        for check in pins.ROUTE_CHECKS:
            check(mod.route)
    elif family == "glu":
        for check in pins.GLU_CHECKS:
            check(mod.glu_act)
        pins.check_gather_qmm_glu_up_ones(mod.quantize, mod.gather_qmm, mod.gather_qmm_glu)
    elif family == "mx":
        pins.check_mx_e2m1_table(mod.e2m1_value)
        pins.check_mx_quantize_on_grid(mod.quantize_mx, mod.dequantize_mx)
        pins.check_mx_quantize_nearest(mod.quantize_mx)
        pins.check_mx_scale_rule(mod.quantize_mx)
        pins.check_mx_gather_exact_rational(mod.gather_qmm_mx)
        pins.check_mx_gather_is_gather_mm(mod.quantize_mx, mod.gather_qmm_mx, mod.gather_mm)
    elif family == "mx8":
        pins.check_mx8_e4m3_table(mod.e4m3_value)
        pins.check_mx8_quantize_library(mod.quantize_mx)
        pins.check_mx8_quantize_on_grid(mod.quantize_mx, mod.dequantize_mx)
        pins.check_mx8_gather_exact_rational(mod.gather_qmm_mx)
        pins.check_mx8_gather_is_gather_mm(mod.quantize_mx, mod.gather_qmm_mx, mod.gather_mm)
    elif family == "nv":
        pins.check_nv_scales(mod.quantize_nv)
        pins.check_nv_codes_nearest(mod.quantize_nv)
        pins.check_nv_gather_exact_rational(mod.gather_qmm_nv)
        pins.check_nv_gather_is_scaled_gather_mm(mod.quantize_nv, mod.gather_qmm_nv, mod.gather_mm)
    elif family == "rows":
        pins.check_gather_qmm_rows(mod.quantize, mod.gather_qmm, mod.gather_qmm_rows)
        pins.check_gather_mm_rows(mod.gather_mm, mod.gather_mm_rows)
        pins.check_gather_qmm_mx_rows(mod.quantize_mx, mod.gather_qmm_mx, mod.gather_qmm_mx_rows)
        pins.check_gather_qmm_nv_rows(mod.quantize_nv, mod.gather_qmm_nv, mod.gather_qmm_nv_rows)
    elif family == "nn":
        for check in pins.GATHER_NN_CHECKS:
            check(mod.quantize, mod.gather_qmm)
        pins.check_gather_nn_all_equal_is_qmm(mod.quantize, mod.gather_qmm, mod.qmm)
        pins.check_gather_nn_is_gather_mm(mod.quantize, mod.gather_qmm, mod.gather_mm)
    elif family == "gather_mm":
        for check in pins.GATHER_MM_CHECKS:
            check(mod.gather_mm)
        pins.check_gather_mm_is_gather_qmm_on_grid(mod.quantize, mod.gather_qmm, mod.gather_mm)
    else:
        for check in pins.GATHER_CHECKS:
            check(mod.quantize, mod.gather_qmm)
        pins.check_gather_all_equal_is_qmm(mod.quantize, mod.gather_qmm, mod.qmm)


@pytest.mark.parametrize("name,original,planted,family", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(name, original, planted, family):
    mod = _mutant(original, planted)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        _run_family(mod, family)


def test_unmutated_copy_passes():
    """The copying machinery itself does not break the oracle."""
    mod = _mutant("q = np.rint(quot)", "q = np.rint(quot)")
    for fam in ("quantize", "route", "gather", "gather_mm", "glu", "mx", "mx8", "nv", "rows", "nn"):
        _run_family(mod, fam)
