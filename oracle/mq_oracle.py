"""CPU oracle for expert-routed affine-quantised matmul (gather_qmm).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library; the two see
the same bytes only through the seeded generators in ``workloads``.

What is computed, and where the pages say so
--------------------------------------------
ml-explore/mlx issue 4339 ("[CUDA] gather_qmm ~24x slower than equal-FLOPs
quantized_matmul ..."), section "Kernel microbenchmark", exercises three calls:

  * ``quantize(w, group_size, bits)`` returning packed codes, scales, biases
    of an *affine* quantisation of w along its last axis;
  * ``gather_qmm(x, wq, scales, biases, rhs_indices, transpose=True, ...)``:
    every token row x[t, a, :] is multiplied by the transposed dequantised
    weight of expert rhs_indices[t, a] (FLOPs = 2*T*A*H*F);
  * ``quantized_matmul(x, wq, scales, biases, transpose=True, ...)``: the
    same product against a single quantised weight (the dense control).

lablup/mlxcel issue 629, "Implementation plan" item 4b, names the routing step:
sort the tokens by expert on the device so that each expert sees one
contiguous block.  ``route`` below is that step written as a counting sort.

The pages never print the affine formula, the code packing, the rounding
modes or the output dtype.  The readings used here (all in fp32 where a
floating-point value decides an integer code, fp64 elsewhere) are:

  1. one bf16 scale and one bf16 bias per run of ``group_size`` weights
     along K, with w ~= scale * q + bias and q an unsigned ``bits``-bit code;
  2. bias = group minimum (signed zeros read as +0.0); scale = (max - min) / (2**bits - 1) computed in
     fp32 and rounded *up* to bf16, so that the code grid covers the group;
  3. q = clamp(rint((w - bias) / scale), 0, 2**bits - 1), fp32 subtraction
     and IEEE fp32 division, round half to even; a constant group has
     scale = 0 and q = 0;
  4. codes packed little-endian into uint32 words along K: code k sits in
     bits [(k % per) * bits, +bits) of word k // per, per = 32 // bits;
  5. the dequantised weight is scale * q + bias, evaluated exactly (fp64);
  6. the product is accumulated in fp64 and returned unrounded (fp64).

Readings 7-10 and 25-26 (the MX and NVFP4 modes) and those of the gated
activation sit with their functions below.

``transpose``.  The stored weight of one expert is always a matrix [R, C]
quantised along its last axis C.  With transpose=True (the microbenchmark's
call) x has C features and out = x @ w_hat^T has R; with transpose=False x
has R features and out = x @ w_hat has C.  ml-explore/mlx PR 4023, the
coverage reply (its second gap, the ``_nn`` kernels), names the second form:
the vector-Jacobian product of the first flips the transpose, so the
backward pass of a quantised MoE layer applies the same stored weight
untransposed (reading 11).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f32", "bf16_round_up", "quantize", "unpack_codes", "dequantize",
    "route", "gather_qmm", "gather_qmm_rows", "qmm", "gather_mm", "gather_mm_rows",
    "glu_act", "gather_qmm_glu", "ACT_SILU", "ACT_GELU",
    "MX_BLOCK", "MX_ELEMS", "e2m1_value", "e4m3_value", "quantize_mx", "dequantize_mx", "gather_qmm_mx",
    "gather_qmm_mx_rows", "NV_BLOCK", "quantize_nv", "dequantize_nv", "gather_qmm_nv",
    "gather_qmm_nv_rows",
]


# --- bf16 helpers (bit patterns held in uint16) ----------------------------

def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round_up(f: np.ndarray) -> np.ndarray:
    """Non-negative finite float32 -> the smallest bf16 >= f (bit pattern).

    Dropping the low 16 bits truncates toward zero; when any of them is set,
    the next bf16 pattern up is the rounded-up value (reading 2).
    """
    u = np.asarray(f, dtype=np.float32).view(np.uint32)
    hi = (u >> np.uint32(16)).astype(np.uint32)
    inexact = (u & np.uint32(0xFFFF)) != 0
    return (hi + inexact.astype(np.uint32)).astype(np.uint16)


# --- quantize ---------------------------------------------------------------

def quantize(w_bits: np.ndarray, group_size: int, bits: int):
    """Affine-quantise bf16 rows along the last axis.

    w_bits: uint16 [..., K] (bf16 bit patterns), K % group_size == 0.
    Returns (wq uint32 [..., K*bits/32], scales uint16 [..., K/gs],
    biases uint16 [..., K/gs]).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K = w_bits.shape[-1]
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    lead = w_bits.shape[:-1]
    G = K // group_size
    w = bf16_to_f32(w_bits).reshape(-1, G, group_size)            # fp32, exact

    # exact; "+ 0" turns a -0.0 extreme into +0.0 so the bias and a zero
    # scale have one bit pattern each
    lo = (w.min(axis=-1) + np.float32(0)).astype(np.float32)
    hi = (w.max(axis=-1) + np.float32(0)).astype(np.float32)
    bias_bits = (lo.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # lo is a bf16 value
    levels = np.float32(2 ** bits - 1)
    span = (hi - lo).astype(np.float32)                            # fp32 RNE
    scale_bits = bf16_round_up((span / levels).astype(np.float32))
    scale = bf16_to_f32(scale_bits)
    bias = bf16_to_f32(bias_bits)

    diff = (w - bias[..., None]).astype(np.float32)                # fp32 RNE
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (diff / scale[..., None]).astype(np.float32)        # IEEE fp32 division
    q = np.rint(quot)                                              # half to even
    q = np.where(scale[..., None] == 0, np.float32(0), q)
    q = np.clip(q, 0, 2 ** bits - 1).astype(np.uint32).reshape(-1, K)

    per = 32 // bits
    words = np.zeros((q.shape[0], K // per), dtype=np.uint32)
    for j in range(per):                                           # code k -> word k//per, slot k%per
        words |= q[:, j::per] << np.uint32(j * bits)
    return (words.reshape(*lead, K // per),
            scale_bits.reshape(*lead, G),
            bias_bits.reshape(*lead, G))


def unpack_codes(wq: np.ndarray, bits: int) -> np.ndarray:
    """uint32 words [..., K*bits/32] -> codes uint32 [..., K] (reading 4)."""
    per = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    wq = np.asarray(wq, dtype=np.uint32)
    out = np.empty(wq.shape[:-1] + (wq.shape[-1] * per,), dtype=np.uint32)
    for j in range(per):
        out[..., j::per] = (wq >> np.uint32(j * bits)) & mask
    return out


def dequantize(wq, scales, biases, group_size: int, bits: int) -> np.ndarray:
    """w_hat = scale * q + bias per group, in fp64 (exact for bf16 scale/bias
    and codes below 2**8: the product has at most 16 significant bits)."""
    q = unpack_codes(wq, bits).astype(np.float64)
    s = np.repeat(bf16_to_f32(scales).astype(np.float64), group_size, axis=-1)
    b = np.repeat(bf16_to_f32(biases).astype(np.float64), group_size, axis=-1)
    return s * q + b


# --- route --------------------------------------------------------------------

def route(idx: np.ndarray, E: int):
    """Stable counting sort of the flattened pair indices by expert.

    lablup/mlxcel issue 629, "Implementation plan" 4b (token sort by expert so
    each expert processes a contiguous block), written as its three steps:
    per-expert counts, exclusive prefix sum into segment offsets, and a
    scatter that visits pairs in increasing flat index (hence stable).

    Returns (counts int64 [E], offsets int64 [E+1], perm int64 [n]) with
    perm[offsets[e] + r] = the r-th flat pair index i (ascending) whose
    expert is e.
    """
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    counts = [0] * E
    for e in flat:
        if not 0 <= e < E:
            raise ValueError(f"expert index {e} outside [0, {E})")
        counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    perm = [0] * len(flat)
    for i, e in enumerate(flat):
        perm[cursor[e]] = i
        cursor[e] += 1
    return (np.array(counts, dtype=np.int64), np.array(offsets, dtype=np.int64),
            np.array(perm, dtype=np.int64))


# --- products -------------------------------------------------------------------

def _x_f64(x_bits):
    return bf16_to_f32(x_bits).astype(np.float64)


def _applied(W: np.ndarray, transpose: bool) -> np.ndarray:
    """The stored stack [E, R, C] as the matrix x multiplies from the right:
    w_hat^T [E, C, R] (transpose=True) or w_hat itself (transpose=False)."""
    return W.transpose(0, 2, 1) if transpose else W


def gather_qmm(x_bits, wq, scales, biases, rhs_indices, group_size: int, bits: int,
               transpose: bool = True) -> np.ndarray:
    """The routed product against a quantised expert stack.

    transpose=True:  wq / scales / biases quantise the stack [E, N, K] along K
                     and out[t, a, m, n] = sum_k x[t, a', m, k] * w_hat[e, n, k];
    transpose=False: they quantise the stack [E, K, N] along N and
                     out[t, a, m, n] = sum_k x[t, a', m, k] * w_hat[e, k, n];
    with e = rhs_indices[t, a], x_bits uint16 [T, Ax, M, K], Ax in {1, A}
    (a' = a if Ax == A else 0).  Returns fp64 [T, A, M, N], one dot product
    per output row, in order.
    """
    x = _x_f64(x_bits)
    T, Ax, M, K = x.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    if Ax not in (1, A):
        raise ValueError("x must have 1 or A rows per token")
    E = wq.shape[0]
    W = _applied(dequantize(wq, scales, biases, group_size, bits), transpose)   # [E, K, N]
    if W.shape[1] != K:
        raise ValueError("x's feature count does not match the weight")
    N = W.shape[2]
    out = np.zeros((T, A, M, N), dtype=np.float64)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            if not 0 <= e < E:
                raise ValueError(f"expert index {e} outside [0, {E})")
            out[t, a] = x[t, a if Ax == A else 0] @ W[e]
    return out


def gather_qmm_rows(x_bits, wq, scales, biases, rhs_indices, group_size: int, bits: int,
                    pairs, cols) -> np.ndarray:
    """Selected outputs of ``gather_qmm`` (transpose=True, M == 1):
    out[pairs[j], cols[j]] for flat pair indices ``pairs`` and output columns
    ``cols``, each one dot product over the dequantised weight row.  Used
    where the full product is too large for the oracle."""
    T, Ax, M, K = x_bits.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    res = np.empty(len(pairs), dtype=np.float64)
    for j, (p, c) in enumerate(zip(pairs, cols)):
        t, a = divmod(int(p), A)
        e = int(idx[t, a])
        wrow = dequantize(wq[e, c:c + 1], scales[e, c:c + 1], biases[e, c:c + 1],
                          group_size, bits)[0]
        res[j] = _x_f64(x_bits[t, a if Ax == A else 0, 0]) @ wrow
    return res


def qmm(x_bits, wq, scales, biases, group_size: int, bits: int,
        transpose: bool = True) -> np.ndarray:
    """Dense quantised matmul against one stored weight [R, C] quantised
    along C: out = x @ w_hat^T (transpose=True, x [M, C]) or x @ w_hat
    (transpose=False, x [M, R]); fp64."""
    W = dequantize(wq, scales, biases, group_size, bits)
    return _x_f64(x_bits) @ (W.T if transpose else W)


# --- the unquantised gather (bf16 weights) -----------------------------------------

def gather_mm(x_bits, w_bits, rhs_indices, transpose: bool = True) -> np.ndarray:
    """The same routed product with a bf16 expert weight (ml-explore/mlx issue
    4339, the follow-up comments on the bf16 MoE gather path, GatherMM):
    out[t, a, m, n] = sum_k x[t, a', m, k] * w[rhs_indices[t, a], n, k].

    x_bits uint16 [T, Ax, M, K] (Ax in {1, A}); w_bits uint16 bf16 [E, N, K];
    rhs_indices [T, A].  Products and sums in fp64; returns fp64 [T, A, M, N].
    """
    if not transpose:
        raise NotImplementedError("only the transposed (x @ W^T) product is defined here")
    x = _x_f64(x_bits)
    T, Ax, M, K = x.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    if Ax not in (1, A):
        raise ValueError("x must have 1 or A rows per token")
    W = bf16_to_f32(w_bits).astype(np.float64)                    # [E, N, K]
    E, N = W.shape[0], W.shape[1]
    out = np.zeros((T, A, M, N), dtype=np.float64)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            if not 0 <= e < E:
                raise ValueError(f"expert index {e} outside [0, {E})")
            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T
    return out


def gather_mm_rows(x_bits, w_bits, rhs_indices, pairs, cols) -> np.ndarray:
    """Selected outputs of ``gather_mm`` (M == 1): out[pairs[j], cols[j]], one
    dot product each (for shapes too large for the full product)."""
    T, Ax, M, K = x_bits.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    res = np.empty(len(pairs), dtype=np.float64)
    for j, (p, c) in enumerate(zip(pairs, cols)):
        t, a = divmod(int(p), A)
        e = int(idx[t, a])
        wrow = bf16_to_f32(w_bits[e, c]).astype(np.float64)
        res[j] = _x_f64(x_bits[t, a if Ax == A else 0, 0]) @ wrow
    return res



# --- gate and up projections with the gated activation ----------------------------------

# The pages' fused switch-GeGLU (lablup/mlxcel issue 629, its references) names
# the gated linear unit of an MoE FFN but not its activation function.  Two
# readings: SiLU (the SwiGLU of the Mixtral-shaped FFN) and GELU with the
# exact error function (GeGLU).
ACT_SILU, ACT_GELU = 1, 2


def glu_act(z, act: int) -> np.ndarray:
    """The activation applied to the gate projection, in fp64:
    SiLU(z) = z / (1 + exp(-z));  GELU(z) = z / 2 * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_SILU:
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-z))
    if act == ACT_GELU:
        erf = np.vectorize(math.erf, otypes=[np.float64])
        return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    raise ValueError(f"unknown activation {act}")


def gather_qmm_glu(x_bits, gate, up, rhs_indices, group_size: int, bits: int,
                   act: int) -> np.ndarray:
    """h[t, a, m, f] = act(g)[t, a, m, f] * u[t, a, m, f] with g and u the routed
    quantised products of x with the gate and up weights (each a (wq, scales,
    biases) triple of an [E, F, K] stack).  Returns fp64 [T, A, M, F]."""
    g = gather_qmm(x_bits, *gate, rhs_indices, group_size, bits)
    u = gather_qmm(x_bits, *up, rhs_indices, group_size, bits)
    return glu_act(g, act) * u


# --- MXFP4: E2M1 codes under a shared power-of-two scale ---------------------------

# The pages name the microscaling fp modes (mxfp4, nvfp4, mxfp8) beside the
# affine one (ml-explore/mlx pull 4023, the comment on the block-height
# coverage; ml-explore/mlx issue 4339, the maintainers' note that the CUDA
# backend keeps only the fp modes) without defining them.  The reading here is
# the published OCP Microscaling Formats (MX) v1.0 definition of MXFP4:
#
#  7. a block of 32 consecutive weights along K shares one scale X = 2^(e - 127),
#     e an unsigned 8-bit exponent (E8M0; 255 is NaN and never produced);
#  8. each weight is an FP4 E2M1 value: 1 sign bit, 2 exponent bits (bias 1),
#     1 mantissa bit, no infinities or NaN;  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
#  9. quantisation: the block's shared exponent is floor(log2(amax)) minus 2
#     (the largest E2M1 exponent), clamped to [-127, 127]; an all-zero block
#     takes the smallest scale (e = 0).  Each weight is divided by X and rounded
#     to E2M1 at the element's precision, ties to the even mantissa, magnitudes
#     beyond 6 saturating to 6; the sign is kept, so a negative weight that
#     rounds to zero becomes -0 (code 8);
# 10. the 4-bit codes are packed like the affine 4-bit codes (reading 4).
#
# MXFP8 is the same block structure with FP8 E4M3 elements (the specification's
# E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
# S.1111.111 the only NaN, largest magnitude 448); the shared exponent
# subtracts E4M3's largest exponent, 8; magnitudes past 448 saturate to 448;
# the 8-bit codes are packed like the affine 8-bit codes.
MX_BLOCK = 32
MX_ELEMS = ("e2m1", "e4m3")


def e2m1_value(code) -> np.ndarray:
    """Value of E2M1 codes from their bit fields (fp64): exponent field 0 is
    subnormal, m/2; otherwise 2^(exp - 1) * (1 + m/2)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    ex = (c >> 1) & 3
    man = (c & 1).astype(np.float64)
    mag = np.where(ex == 0, man * 0.5, np.ldexp(1.0 + man / 2.0, ex - 1))
    return sign * mag


def e4m3_value(code) -> np.ndarray:
    """Value of E4M3 codes from their bit fields (fp64): exponent field 0 is
    subnormal, m/8 * 2^-6; otherwise 2^(exp - 7) * (1 + m/8); S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 15
    man = (c & 7).astype(np.float64)
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, np.ldexp(1.0 + man / 8.0, ex - 7))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def _e4m3_encode(y: np.ndarray) -> np.ndarray:
    """fp64 y (|y| < 512, already divided by the block scale) -> E4M3 code.

    The quantum is 2^-9 below 2^-6 (the subnormal binade) and 2^(floor(log2|y|)
    - 3) above; np.rint on the multiple is round half to even on the last
    mantissa bit, and magnitudes past 448 saturate to 448."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    neg = np.signbit(y)
    ex = np.floor(np.log2(np.maximum(mag, 2.0 ** -6))).astype(np.int64)
    quantum = np.where(mag < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 3))
    r = np.minimum(np.rint(mag / quantum) * quantum, 448.0)
    table = {float(e4m3_value(c)): c for c in range(0x7F)}
    code = np.array([table.get(float(v), -1) for v in r.reshape(-1)], dtype=np.int64)
    if (code < 0).any():
        raise ValueError("a rounded magnitude is not an E4M3 value")
    code = code.astype(np.uint32).reshape(r.shape)
    return code | np.where(neg, np.uint32(0x80), np.uint32(0))


def _e2m1_encode(y: np.ndarray) -> np.ndarray:
    """fp64 y (|y| < 8, already divided by the block scale) -> E2M1 code.

    The element's quantum is 1/2 below 2 (the subnormal binade and the
    binade [1, 2) both step by 1/2) and 2^(floor(log2|y|) - 1) above;
    rounding |y| to a multiple of its quantum with np.rint is round half to
    even on the mantissa bit, and 8 saturates to 6."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    neg = np.signbit(y)
    ex = np.floor(np.log2(np.maximum(mag, 1.0))).astype(np.int64)   # 0, 1 or 2
    quantum = np.where(mag < 1.0, 0.5, np.ldexp(1.0, ex - 1))
    r = np.minimum(np.rint(mag / quantum) * quantum, 6.0)
    # the magnitude back to its fields: r = 2^(E - 1) (1 + m/2) or m/2
    code = np.zeros(r.shape, dtype=np.uint32)
    for c in range(8):
        code[r == e2m1_value(c)] = c
    return code | np.where(neg, np.uint32(8), np.uint32(0))


def quantize_mx(w_bits: np.ndarray, elem: str = "e2m1"):
    """MX-quantise bf16 rows along the last axis (readings 7-10): MXFP4
    (elem "e2m1") or MXFP8 (elem "e4m3").

    w_bits: uint16 [..., K] bf16 patterns, finite, K % 32 == 0.
    Returns (wq uint32 [..., K/8] (MXFP4) or [..., K/4] (MXFP8), scales uint8
    [..., K/32])."""
    if elem not in MX_ELEMS:
        raise ValueError(f"unknown element format {elem}")
    emax, bits = (2, 4) if elem == "e2m1" else (8, 8)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K = w_bits.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of the 32-element block")
    lead = w_bits.shape[:-1]
    w = bf16_to_f32(w_bits.reshape(-1, K // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    amax = np.abs(w).max(axis=-1)
    _, ex = np.frexp(amax)                                   # amax = f 2^ex, f in [0.5, 1)
    shared = np.where(amax > 0, ex.astype(np.int64) - 1 - emax, -127)
    shared = np.clip(shared, -127, 127)
    y = w / np.ldexp(1.0, shared)[..., None]                 # exact: a power of two
    codes = (_e2m1_encode(y) if elem == "e2m1" else _e4m3_encode(y)).reshape(-1, K)
    per = 32 // bits
    words = np.zeros((codes.shape[0], K // per), dtype=np.uint32)
    for j in range(per):
        words |= codes[:, j::per] << np.uint32(bits * j)
    scales = (shared + 127).astype(np.uint8)
    return words.reshape(*lead, K // per), scales.reshape(*lead, K // MX_BLOCK)


def dequantize_mx(wq: np.ndarray, scales: np.ndarray, elem: str = "e2m1") -> np.ndarray:
    """w_hat[..., k] = value(code k) * 2^(e[k // 32] - 127), exact in fp64."""
    wq = np.asarray(wq, dtype=np.uint32)
    bits = 4 if elem == "e2m1" else 8
    K = wq.shape[-1] * (32 // bits)
    codes = unpack_codes(wq, bits)
    e = np.repeat(np.asarray(scales, dtype=np.int64), MX_BLOCK, axis=-1)
    assert e.shape[-1] == K
    value = e2m1_value if elem == "e2m1" else e4m3_value
    return value(codes) * np.ldexp(1.0, e - 127)


def gather_qmm_mx(x_bits, wq, scales, rhs_indices, elem: str = "e2m1") -> np.ndarray:
    """The routed product against MX expert weights:
    out[t, a, m, n] = sum_k x[t, a', m, k] * w_hat[rhs_indices[t, a], n, k],
    wq uint32 [E, N, K/8] (MXFP4) or [E, N, K/4] (MXFP8), scales uint8
    [E, N, K/32].  fp64 [T, A, M, N]."""
    x = _x_f64(x_bits)
    T, Ax, M, K = x.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    if Ax not in (1, A):
        raise ValueError("x must have 1 or A rows per token")
    W = dequantize_mx(wq, scales, elem)                            # [E, N, K]
    E = W.shape[0]
    out = np.zeros((T, A, M, W.shape[1]), dtype=np.float64)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            if not 0 <= e < E:
                raise ValueError(f"expert index {e} outside [0, {E})")
            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T
    return out


def gather_qmm_mx_rows(x_bits, wq, scales, rhs_indices, pairs, cols,
                       elem: str = "e2m1") -> np.ndarray:
    """Selected outputs of ``gather_qmm_mx`` (M == 1), one dot product each."""
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    Ax = x_bits.shape[1]
    res = np.empty(len(pairs), dtype=np.float64)
    for j, (p, c) in enumerate(zip(pairs, cols)):
        t, a = divmod(int(p), A)
        e = int(idx[t, a])
        wrow = dequantize_mx(wq[e, c:c + 1], scales[e, c:c + 1], elem)[0]
        res[j] = _x_f64(x_bits[t, a if Ax == A else 0, 0]) @ wrow
    return res


# --- NVFP4: E2M1 codes, an E4M3 scale per 16 weights, an fp32 scale per tensor -------

# The pages name nvfp4 beside mxfp4 and mxfp8 (ml-explore/mlx pull 4023, the
# comment on block-height coverage) without defining it.  The reading is
# NVIDIA's published NVFP4:
#
# 25. blocks of 16 weights along K, each with a scale stored as FP8 E4M3, and
#     one fp32 scale g per tensor (here: per expert weight [N, K]); a weight is
#     e2m1(q) * e4m3(s) * g;
# 26. quantisation, every step in IEEE fp32 (round to nearest even):
#     g = amax_tensor / 2688 (2688 = 6 * 448, so that the largest block scale
#     lands on E4M3's largest value), g = 1 for an all-zero tensor;
#     s = e4m3(amax_block / 6 / g) (nearest, ties even, saturating at 448);
#     d = e4m3_value(s) * g;  q = e2m1(w / d) (nearest, ties even, saturating
#     at 6, the sign kept); a block whose scale rounds to 0 gets signed zeros.
NV_BLOCK = 16


def quantize_nv(w_bits: np.ndarray):
    """NVFP4-quantise a stack of bf16 tensors [T, R, K] (K % 16 == 0) along K.

    Returns (wq uint32 [T, R, K/8], scales uint8 [T, R, K/16] (E4M3 codes),
    gscale float32 [T])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 3 or w_bits.shape[-1] % NV_BLOCK:
        raise ValueError("w must be [T, R, K] with K a multiple of 16")
    Tn, R, K = w_bits.shape
    w = bf16_to_f32(w_bits)                                         # exact, fp32
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    f32 = np.float32
    amax_t = np.abs(w).reshape(Tn, -1).max(axis=1)
    g = np.where(amax_t > 0, amax_t / f32(2688.0), f32(1.0)).astype(np.float32)
    blocks = w.reshape(Tn, R, K // NV_BLOCK, NV_BLOCK)
    amax_b = np.abs(blocks).max(axis=-1)
    sb = ((amax_b / f32(6.0)).astype(np.float32) / g[:, None, None]).astype(np.float32)
    s_code = _e4m3_encode(sb.astype(np.float64))
    s_val = e4m3_value(s_code).astype(np.float32)
    d = (s_val * g[:, None, None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (blocks / d[..., None]).astype(np.float32)
    y = np.where(d[..., None] > 0, y, np.copysign(np.float32(0), blocks))
    codes = _e2m1_encode(y.astype(np.float64)).reshape(Tn * R, K)
    words = np.zeros((Tn * R, K // 8), dtype=np.uint32)
    for j in range(8):
        words |= codes[:, j::8] << np.uint32(4 * j)
    return words.reshape(Tn, R, K // 8), s_code.astype(np.uint8), g


def dequantize_nv(wq, scales, gscale) -> np.ndarray:
    """w_hat[t, r, k] = e2m1(q) * e4m3(s[t, r, k // 16]) * g[t], exact in fp64."""
    wq = np.asarray(wq, dtype=np.uint32)
    codes = unpack_codes(wq, 4)
    s = np.repeat(e4m3_value(np.asarray(scales, dtype=np.int64)), NV_BLOCK, axis=-1)
    g = np.asarray(gscale, dtype=np.float64).reshape(-1, *([1] * (wq.ndim - 1)))
    return e2m1_value(codes) * s * g


def gather_qmm_nv(x_bits, wq, scales, gscale, rhs_indices) -> np.ndarray:
    """The routed product against NVFP4 expert weights (wq [E, N, K/8], scales
    [E, N, K/16], gscale [E]): out[t, a, m, n] = sum_k x * w_hat.  fp64."""
    x = _x_f64(x_bits)
    T, Ax, M, K = x.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    if Ax not in (1, A):
        raise ValueError("x must have 1 or A rows per token")
    W = dequantize_nv(wq, scales, gscale)                           # [E, N, K]
    E = W.shape[0]
    out = np.zeros((T, A, M, W.shape[1]), dtype=np.float64)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            if not 0 <= e < E:
                raise ValueError(f"expert index {e} outside [0, {E})")
            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T
    return out


def gather_qmm_nv_rows(x_bits, wq, scales, gscale, rhs_indices, pairs, cols) -> np.ndarray:
    """Selected outputs of ``gather_qmm_nv`` (M == 1), one dot product each."""
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    Ax = x_bits.shape[1]
    res = np.empty(len(pairs), dtype=np.float64)
    for j, (p, c) in enumerate(zip(pairs, cols)):
        t, a = divmod(int(p), A)
        e = int(idx[t, a])
        wrow = dequantize_nv(wq[e:e + 1, c:c + 1], scales[e:e + 1, c:c + 1], gscale[e:e + 1])[0, 0]
        res[j] = _x_f64(x_bits[t, a if Ax == A else 0, 0]) @ wrow
    return res
