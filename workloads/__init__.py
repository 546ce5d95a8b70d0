"""Seeded synthetic inputs for gather_qmm, shared by the oracle tests, the GPU
parity tests and bench.py.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, no routing, no matmul).  Every array it
returns is plain host memory:

  * bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
    from float32 normals, the way a framework casts fp32 -> bf16);
  * expert indices are ``int32``.

Shapes and distributions follow the workloads on the pages:

  * ml-explore/mlx issue 4339, "Kernel microbenchmark": T=2048 tokens, A=8
    active experts, H=2048, F=768, E=64, x ~ N(0,1) of shape [T, A, 1, H],
    w ~ N(0,1) of shape [E, F, H], indices uniform in [0, E) of shape [T, A],
    and the equal-FLOPs dense control x [T*A, H] times one [F, H] weight.
  * ml-explore/mlx PR 4023 ("Pick BM from rows per expert ..."), the
    measurement paragraph: E=256, K=2048, N=512, 4-bit gs64, chained up and
    down projections, swept over rows per expert 4..128.
  * lablup/mlxcel issue 629, "Acceptance criteria": a Mixtral-8x7B-shaped
    expert FFN at a 2048-token prompt.
  * lablup/mlxcel issue 725, "The gap": small-M batched decode, B in [1, 8].

Seeding: ``numpy.random.SeedSequence(seed).spawn(4)`` in the fixed order
[x, W (up), W (down), idx].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "bf16_bits_from_f32", "f32_from_bf16_bits", "GatherCase", "gather_case",
    "tiny_moe", "prefill_microbench", "prefill_dense_control", "short_run_sweep",
    "mixtral_ffn", "small_m_dense", "moe_decode", "presort",
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits_from_f32(a)


@dataclasses.dataclass
class GatherCase:
    """One gather_qmm problem: out[t,a,m,:] = x[t, a*(Ax>1), m, :] @ W[idx[t,a]]^T.

    x    uint16 (bf16 bits) [T, Ax, M, K]
    w    uint16 (bf16 bits) [E, N, K]   unquantised weight, quantised along K
    idx  int32 [T, A]
    """
    name: str
    x: np.ndarray
    w: np.ndarray
    idx: np.ndarray
    E: int
    group_size: int = 64
    bits: int = 4
    sorted_indices: bool = False
    w_down: Optional[np.ndarray] = None   # [E, K, N] for chained up/down cases

    @property
    def T(self): return self.x.shape[0]
    @property
    def Ax(self): return self.x.shape[1]
    @property
    def M(self): return self.x.shape[2]
    @property
    def K(self): return self.x.shape[3]
    @property
    def A(self): return self.idx.shape[1]
    @property
    def N(self): return self.w.shape[1]
    @property
    def flops(self) -> int:
        return 2 * self.T * self.A * self.M * self.K * self.N


def _uniform_idx(rng, T, A, E):
    return rng.integers(0, E, size=(T, A), dtype=np.int64).astype(np.int32)


def _balanced_idx(rng, T, A, E):
    """Exactly T*A/E rows per expert: round-robin slots, then a seeded shuffle."""
    flat = (np.arange(T * A, dtype=np.int64) % E).astype(np.int32)
    rng.shuffle(flat)
    return flat.reshape(T, A)


def _zipf_idx(rng, T, A, E, s):
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return rng.choice(E, size=(T, A), replace=True, p=p).astype(np.int32)


def gather_case(name: str, T: int, A: int, E: int, K: int, N: int, seed: int,
                *, M: int = 1, Ax: Optional[int] = None, routing: str = "uniform",
                zipf_s: float = 1.2, w_std: float = 1.0, group_size: int = 64,
                bits: int = 4, with_down: bool = False) -> GatherCase:
    """Draw one case.  ``routing`` is "uniform", "balanced" or "zipf"."""
    Ax = A if Ax is None else Ax
    ss_x, ss_up, ss_down, ss_idx = np.random.SeedSequence(seed).spawn(4)
    x = _normal_bf16(np.random.default_rng(ss_x), (T, Ax, M, K))
    w = _normal_bf16(np.random.default_rng(ss_up), (E, N, K), w_std)
    r = np.random.default_rng(ss_idx)
    if routing == "uniform":
        idx = _uniform_idx(r, T, A, E)
    elif routing == "balanced":
        idx = _balanced_idx(r, T, A, E)
    elif routing == "zipf":
        idx = _zipf_idx(r, T, A, E, zipf_s)
    else:
        raise ValueError(routing)
    case = GatherCase(name, x, w, idx, E, group_size, bits)
    if with_down:
        # the down projection maps N back to K, same experts and routing
        case.w_down = _normal_bf16(np.random.default_rng(ss_down), (E, K, N), w_std)
    return case


def presort(case: GatherCase) -> tuple[GatherCase, np.ndarray]:
    """The pre-sorted variant of a case with Ax == A and M == 1.

    Pairs are stably sorted by expert; x rows follow them; the result has
    T' = T*A, A' = 1 and sorted_indices=True.  Returns (case', order) with
    out'[j] = out[order[j]] (flattened pair index).
    """
    assert case.Ax == case.A
    flat = case.idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    T2 = flat.size
    x2 = case.x.reshape(T2, 1, case.M, case.K)[order]
    idx2 = flat[order].reshape(T2, 1).astype(np.int32)
    c2 = GatherCase(case.name + "-presorted", np.ascontiguousarray(x2), case.w,
                    np.ascontiguousarray(idx2), case.E, case.group_size, case.bits,
                    sorted_indices=True)
    return c2, order


# --- the workloads --------------------------------------------------------

def tiny_moe(seed: int = 0) -> GatherCase:
    """T=64, A=2, E=8, K=256, N=128, 4-bit gs64, uniform routing."""
    return gather_case("tiny-moe", 64, 2, 8, 256, 128, seed)


def prefill_microbench(seed: int = 0) -> GatherCase:
    """T=2048, A=8, E=64, K=2048, N=768, 4-bit gs64, uniform routing (~256 rows/expert)."""
    return gather_case("prefill-T2048-A8-E64-K2048-N768", 2048, 8, 64, 2048, 768, seed)


def prefill_dense_control(seed: int = 0):
    """The equal-FLOPs dense control: x [16384, 2048] and one weight [768, 2048] (bf16 bits)."""
    ss_x, ss_w, _, _ = np.random.SeedSequence(seed + 1000).spawn(4)
    x = _normal_bf16(np.random.default_rng(ss_x), (2048 * 8, 2048))
    w = _normal_bf16(np.random.default_rng(ss_w), (768, 2048))
    return x, w


def short_run_sweep(rows_per_expert: int, seed: int = 0) -> GatherCase:
    """E=256, top-8, K=2048, N=512 (up; the down weight is [E, 2048, 512]),
    exactly ``rows_per_expert`` rows per expert: T = 32 * rows_per_expert."""
    T = 256 * rows_per_expert // 8
    return gather_case(f"short-run-r{rows_per_expert}", T, 8, 256, 2048, 512, seed,
                       routing="balanced", with_down=True)


def mixtral_ffn(seed: int = 0, zipf_s: float = 1.2, proj: str = "up") -> GatherCase:
    """E=8, top-2, T=2048; gate/up K=4096 -> N=14336, down K=14336 -> N=4096;
    W ~ N(0, 0.02); Zipf(s) routing drawn with replacement."""
    K, N = (4096, 14336) if proj in ("up", "gate") else (14336, 4096)
    return gather_case(f"mixtral-{proj}-zipf{zipf_s}", 2048, 2, 8, K, N, seed,
                       routing="zipf", zipf_s=zipf_s, w_std=0.02)


def small_m_dense(B: int, N: int, K: int, seed: int = 0):
    """Dense small-M decode: x [B, K] and one weight [N, K] (bf16 bits)."""
    ss_x, ss_w, _, _ = np.random.SeedSequence(seed + 2000).spawn(4)
    x = _normal_bf16(np.random.default_rng(ss_x), (B, K))
    w = _normal_bf16(np.random.default_rng(ss_w), (N, K))
    return x, w


def moe_decode(seed: int = 0) -> GatherCase:
    """MoE decode: E=128, top-8, K=2048, N=768, T=4 tokens, uniform routing."""
    return gather_case("moe-decode-T4-A8-E128", 4, 8, 128, 2048, 768, seed)
