// Gathered grouped GEMM on affine-quantised expert weights (gfx950, bf16 MFMA).
//
// What it computes (ml-explore/mlx issue 4339, "Kernel microbenchmark"): every
// routed row is multiplied by the transposed dequantised weight of its expert.
// How the work is cut follows the pages' diagnosis:
//   * lablup/mlxcel issue 629, "Implementation plan" 4a/4b, and the sm_86
//     comment on mlx issue 4339: one grouped GEMM over tokens sorted by expert,
//     never one workgroup per (token, expert) pair;
//   * ml-explore/mlx PR 4023, opening paragraphs: a tile never straddles two
//     experts, so no row is computed and thrown away, and each expert's BN x K
//     slab is streamed once per tile; the tile height BM is a template
//     parameter the host picks from the average rows per expert.
//
// Exactness.  A code q is fed to the MFMA as the bf16 value 128 + q (4-bit:
// exact, built by OR-ing the nibble into the mantissa of 128.0) or q itself
// (8-bit: exact via an integer->float conversion).  Per group g the MFMA
// accumulates P_g = sum_k x_k * (off + q_k) in fp32, and the epilogue adds
//     s_g * P_g + (b_g - off * s_g) * X_g,        X_g = sum_{k in g} x_k,
// in fp32, which equals sum_k x_k * (s_g q_k + b_g).  No bf16 rounding of the
// dequantised weight ever happens.
//
// Layout of one 256-thread workgroup (4 waves):
//   tile   BM routed rows of one expert x BN = 128 output columns;
//   wave w owns columns [32w, 32w + 32): BM/16 x 2 MFMA 16x16 blocks;
//   K      is walked in chunks of 64; x rows of the chunk are gathered through
//          perm, written to LDS (double buffered, k-pairs pre-permuted to the
//          order the code decode produces) with their per-group row sums;
//          codes go straight from global memory to registers, one chunk ahead.
//   store  fp32 -> bf16 (RNE) through LDS, then 16-byte row segments to
//          out[pair * M + m] (the unpermute of the routing is fused here).
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int XS_STRIDE = BK + 8;        // bf16 per LDS row (16-byte pad)
constexpr int YS_STRIDE = BN + 8;        // bf16 per staged output row

__device__ inline float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// (x0,x1),(x2,x3),(x4,x5),(x6,x7) -> (x0,x4),(x1,x5),(x2,x6),(x3,x7)
__device__ inline u32x4 pair_k_with_k4(u32x4 u) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(u[2], u[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(u[2], u[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(u[3], u[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(u[3], u[1], 0x07060302u);
  return r;
}

// 8 four-bit codes (k0..k7 in nibbles 0..7) -> bf16 (128+q) pairs in the
// order (k0,k4),(k1,k5),(k2,k6),(k3,k7).
__device__ inline u32x4 decode4(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

// 8 eight-bit codes (k0..k3 in w0, k4..k7 in w1) -> exact bf16 pairs in the
// same (k_j, k_j+4) order.
__device__ inline u32x4 decode8(uint32_t w0, uint32_t w1) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = __float_as_uint(float((w0 >> (8 * j)) & 0xFFu));
    const uint32_t b = __float_as_uint(float((w1 >> (8 * j)) & 0xFFu));
    r[j] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
  return r;
}

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int BM, int BITS, int GS>
__global__ __launch_bounds__(kThreads) void gather_gemm_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(GS == 32 || GS == 64, "GS");
  constexpr int MT = BM / 16;                    // MFMA row blocks per wave
  constexpr int NT = 2;                          // MFMA column blocks per wave
  constexpr int GPC = BK / GS;                   // groups per chunk
  constexpr int KS = BK / 32;                    // MFMA k-steps per chunk
  constexpr int PASSES = BM >= 32 ? BM / 32 : 1; // x-load passes
  constexpr int WPR = 32 / BITS;                 // codes per word
  constexpr float OFF = BITS == 4 ? 128.0f : 0.0f;

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * XS_STRIDE];
  __shared__ __attribute__((aligned(16))) float xsum[2][GPC][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;

  // ---- which tile ----------------------------------------------------------
  const int ntn = (a.N + BN - 1) / BN;          // column tiles; fastest in launch order
  const int t = int(blockIdx.x / unsigned(ntn));
  int e = 0;
  int64_t row0, seg_end;
  if (a.perm) {
    // a tile table built for another tile height (a workspace routed under a
    // different plan) is not used: nothing is written
    if (*a.tile_bm != BM) return;
    const int ntiles = a.tiles[a.E];
    if (t >= ntiles) return;
    int lo = 0, hi = a.E;                        // largest e with tiles[e] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tiles[mid] <= t) lo = mid; else hi = mid;
    }
    e = lo;
    // offsets come from the routing kernels; clamping them to [0, n] keeps
    // every access in bounds even if they were corrupted
    const int64_t nrows = a.n_pairs * a.M;
    row0 = min<int64_t>(max<int64_t>(int64_t(a.offsets[e]) * a.M, 0) +
                            int64_t(t - a.tiles[e]) * BM, nrows);
    seg_end = min<int64_t>(max<int64_t>(int64_t(a.offsets[e + 1]) * a.M, 0), nrows);
    if (row0 >= seg_end) return;
  } else {
    row0 = int64_t(t) * BM;
    seg_end = a.n_pairs * a.M;
    if (row0 >= seg_end) return;
  }
  const int rows = int(min<int64_t>(BM, seg_end - row0));
  const int n0 = int(blockIdx.x % unsigned(ntn)) * BN;

  // ---- per-thread x row pointers (gather through perm) ----------------------
  const int piece = tid & 7;                     // 16-byte piece of a 64-k chunk row
  const uint16_t* xrow[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = (tid >> 3) + 32 * p;
    xrow[p] = nullptr;
    if (r < BM && r < rows) {
      const int64_t j = row0 + r;
      int64_t xr;
      if (a.perm) {
        const int32_t pair = min<int64_t>(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1);
        const int m = int(j % a.M);
        const int tok = pair / a.A, slot = pair - tok * a.A;
        xr = (int64_t(tok) * a.Ax + (a.Ax > 1 ? slot : 0)) * a.M + m;
      } else {
        xr = j;
      }
      xrow[p] = a.x + xr * K + piece * 8;
    }
  }

  // ---- per-lane weight pointers --------------------------------------------
  const uint32_t* wrow[NT];
  const uint16_t* srow[NT];
  const uint16_t* brow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(n0 + 32 * wave + 16 * nt + l16, N - 1);
    const int64_t r = int64_t(e) * N + n;
    wrow[nt] = a.wq + r * (K / WPR);
    srow[nt] = a.scales + r * G;
    brow[nt] = a.biases + r * G;
  }

  // k offset (within a chunk) of this lane's 8 codes at k-step ks.  For GS=64
  // the two k-steps of a lane are adjacent (one 8/16-byte code load); for
  // GS=32 each k-step must stay inside one group.
  auto koff = [&](int ks) { return GS == 32 ? 32 * ks + 8 * c4 : 16 * c4 + 8 * ks; };

  // ---- register staging ------------------------------------------------------
  u32x4 xreg[PASSES];
  uint32_t creg[NT][KS * BITS / 4];              // code words of the next chunk
  auto load_x = [&](int chunk) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      if (xrow[p]) xreg[p] = *reinterpret_cast<const u32x4*>(xrow[p] + chunk * BK);
      else xreg[p] = u32x4{0, 0, 0, 0};
    }
  };
  auto load_codes = [&](int chunk) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int w0 = (chunk * BK + koff(ks)) / WPR;
        if constexpr (BITS == 4) {
          creg[nt][ks] = wrow[nt][w0];
        } else {
          creg[nt][2 * ks] = wrow[nt][w0];
          creg[nt][2 * ks + 1] = wrow[nt][w0 + 1];
        }
      }
    }
  };
  auto stage_x = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = (tid >> 3) + 32 * p;
      if (r < BM) {
        const u32x4 u = xreg[p];
        *reinterpret_cast<u32x4*>(&xs[buf][r * XS_STRIDE + piece * 8]) = pair_k_with_k4(u);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) s += bf16lo(u[j]) + bf16hi(u[j]);
        // reduce over the lanes holding the same (row, group)
        constexpr int LANES = GS / 8;
#pragma unroll
        for (int d = 1; d < LANES; d <<= 1) s += __shfl_xor(s, d, 64);
        if ((piece % LANES) == 0) xsum[buf][piece / LANES][r] = s;
      }
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = K / BK;
  load_x(0);
  load_codes(0);
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int buf = chunk & 1;
    stage_x(buf);
    uint32_t cur[NT][KS * BITS / 4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < KS * BITS / 4; ++i) cur[nt][i] = creg[nt][i];
    // scales / biases of this chunk's groups
    float sc[NT][GPC], cb[NT][GPC];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int gl = 0; gl < GPC; ++gl) {
        const int g = chunk * GPC + gl;
        const float s = __uint_as_float(uint32_t(srow[nt][g]) << 16);
        const float b = __uint_as_float(uint32_t(brow[nt][g]) << 16);
        sc[nt][gl] = s;
        cb[nt][gl] = b - OFF * s;
      }
    __syncthreads();
    if (chunk + 1 < nchunks) {
      load_x(chunk + 1);
      load_codes(chunk + 1);
    }

#pragma unroll
    for (int gl = 0; gl < GPC; ++gl) {
      f32x4 P[MT][NT];
#pragma unroll
      for (int ksg = 0; ksg < KS / GPC; ++ksg) {
        const int ks = gl * (KS / GPC) + ksg;
        u32x4 bfrag[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (BITS == 4) bfrag[nt] = decode4(cur[nt][ks]);
          else bfrag[nt] = decode8(cur[nt][2 * ks], cur[nt][2 * ks + 1]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4 afrag = *reinterpret_cast<const u32x4*>(
              &xs[buf][(mt * 16 + l16) * XS_STRIDE + koff(ks)]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            P[mt][nt] = mfma(afrag, bfrag[nt], ksg == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[mt][nt]);
        }
      }
      // epilogue of group gl: acc += s * P + (b - off*s) * X
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 X = *reinterpret_cast<const f32x4*>(&xsum[buf][gl][mt * 16 + 4 * c4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mt][nt][i] = fmaf(sc[nt][gl], P[mt][nt][i], fmaf(cb[nt][gl], X[i], acc[mt][nt][i]));
      }
    }
  }

  // ---- store: fp32 -> bf16 through LDS, then row segments --------------------
  __syncthreads();
  uint16_t* ys = &xs[0][0];
  static_assert(2 * BM * XS_STRIDE >= BM * YS_STRIDE, "staging fits in the x buffers");
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * c4 + i;
        const int c = 32 * wave + 16 * nt + l16;
        ys[r * YS_STRIDE + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mt][nt][i]));
      }
  __syncthreads();
  const bool vec_ok = (N % 8) == 0;
  for (int idx = tid; idx < BM * (BN / 8); idx += kThreads) {
    const int r = idx / (BN / 8), pc = idx % (BN / 8);
    if (r >= rows) continue;
    const int c = n0 + pc * 8;
    if (c >= N) continue;
    const int64_t j = row0 + r;
    int64_t orow;
    if (a.perm)
      orow = min<int64_t>(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1) * a.M + (j % a.M);
    else orow = j;
    uint16_t* dst = a.out + orow * N + c;
    const uint16_t* srcp = &ys[r * YS_STRIDE + pc * 8];
    if (vec_ok) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(srcp);
    } else {
      for (int q = 0; q < 8 && c + q < N; ++q) dst[q] = srcp[q];
    }
  }
}

template <int BM, int BITS>
hipError_t launch_bm_bits(const GemmArgs& a, dim3 grid, hipStream_t s) {
  if (a.group_size == 32)
    gather_gemm_kernel<BM, BITS, 32><<<grid, dim3(kThreads), 0, s>>>(a);
  else
    gather_gemm_kernel<BM, BITS, 64><<<grid, dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <int BM>
hipError_t launch_bm(const GemmArgs& a, dim3 grid, hipStream_t s) {
  return a.bits == 4 ? launch_bm_bits<BM, 4>(a, grid, s) : launch_bm_bits<BM, 8>(a, grid, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  const int64_t blocks = ceil_div(a.N, BN) * a.max_tiles;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  switch (a.bm) {
    case 16: return launch_bm<16>(a, grid, s);
    case 32: return launch_bm<32>(a, grid, s);
    case 64: return launch_bm<64>(a, grid, s);
    default: return launch_bm<128>(a, grid, s);
  }
}

}  // namespace mq
