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
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f32", "bf16_round_up", "quantize", "unpack_codes", "dequantize",
    "route", "gather_qmm", "gather_qmm_rows", "qmm", "gather_mm", "gather_mm_rows",
    "glu_act", "gather_qmm_glu", "ACT_SILU", "ACT_GELU",
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


def gather_qmm(x_bits, wq, scales, biases, rhs_indices, group_size: int, bits: int,
               transpose: bool = True) -> np.ndarray:
    """out[t, a, m, n] = sum_k x[t, a', m, k] * w_hat[rhs_indices[t, a], n, k].

    x_bits: uint16 [T, Ax, M, K] with Ax in {1, A} (a' = a if Ax == A else 0);
    wq / scales / biases: the quantised [E, N, K] weight; rhs_indices [T, A].
    Returns fp64 [T, A, M, N].  One dot product per output row, in order.
    """
    if not transpose:
        raise NotImplementedError("only the transposed (x @ W^T) product is defined here")
    x = _x_f64(x_bits)
    T, Ax, M, K = x.shape
    idx = np.asarray(rhs_indices)
    A = idx.shape[1]
    if Ax not in (1, A):
        raise ValueError("x must have 1 or A rows per token")
    E = wq.shape[0]
    W = dequantize(wq, scales, biases, group_size, bits)         # [E, N, K]
    N = W.shape[1]
    out = np.zeros((T, A, M, N), dtype=np.float64)
    for t in range(T):
        for a in range(A):
            e = int(idx[t, a])
            if not 0 <= e < E:
                raise ValueError(f"expert index {e} outside [0, {E})")
            out[t, a] = x[t, a if Ax == A else 0] @ W[e].T
    return out


def gather_qmm_rows(x_bits, wq, scales, biases, rhs_indices, group_size: int, bits: int,
                    pairs, cols) -> np.ndarray:
    """Selected outputs of ``gather_qmm`` (M == 1): out[pairs[j], cols[j]] for
    flat pair indices ``pairs`` and output columns ``cols``, each one dot
    product over the dequantised weight row.  Used where the full product is
    too large for the oracle."""
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
    """Dense quantised matmul: out[m, n] = sum_k x[m, k] * w_hat[n, k] (fp64)."""
    if not transpose:
        raise NotImplementedError("only the transposed (x @ W^T) product is defined here")
    return _x_f64(x_bits) @ dequantize(wq, scales, biases, group_size, bits).T


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
