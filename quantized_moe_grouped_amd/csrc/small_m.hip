// Weight-reusing small-M path: at most 16 rows per tile against a quantised
// weight, each weight byte read from memory once.
//
// lablup/mlxcel issue 725, "The gap" and "What's needed": batched decode with
// B <= 8 rows must not re-read the whole weight per row (per-row matrix-vector
// kernels make the traffic O(B)), and a 128-row tile wastes ~94% of its work
// at M = 8.  Here one workgroup owns 16 output columns of one row tile (dense:
// the M rows; gathered: the <= 16 routed rows of one expert) and its KW (4 or 8) waves
// split K; every code, scale and bias of those columns is loaded once and
// applied to all rows of the tile by one MFMA per 32 k.  The work is
// HBM-bound, so each wave requests the weights of up to 16 groups at once
// before it computes any of them.
//
// Arithmetic is the GEMM's (exact codes, per-group fp32 epilogue): per group
// P = x . (off + q) and X = x . 1 come from two MFMAs (the second against a
// constant all-ones operand gives the row sums in the same register layout),
// then acc += s P + (b - off s) X.  Partial sums of the waves meet in LDS in a
// fixed order, so results are deterministic.
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kNoRow = 0x80000000u;          // outside every descriptor range (< 2 GiB)
constexpr int GR = 16;                           // groups whose weights are in flight at once

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

__device__ inline u32x4 pair_k_with_k4(u32x4 u) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(u[2], u[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(u[2], u[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(u[3], u[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(u[3], u[1], 0x07060302u);
  return r;
}

__device__ inline u32x4 decode4(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

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

// One "step" of a wave covers 4*LB bytes of every column's code row: lane
// (l16, c4) loads LB contiguous bytes (16, or 8 for 4-bit groups of 32) of
// column l16, so each load instruction moves 64 lanes x LB useful bytes.  A
// step spans GPS = 4*LB / (bytes per group) groups, 1 or 2; with 2, lanes
// c4 < 2 hold group g and lanes c4 >= 2 group g+1, and one MFMA k-step would
// mix the two.  They are separated on the x side: a lane's x values form the
// A operand of the half (group) it serves, the other half's operand being
// zero in that lane, and every k-step runs one MFMA per half.  That doubles
// the (cheap) MFMA work of this memory-bound path but keeps every weight load
// wide.  Row sums per group come from MFMAs of the same operands against a
// ones operand.
template <int BITS, int GS, int KW, int NT>
__global__ __launch_bounds__(64 * KW) void small_m_kernel(GemmArgs a) {
  constexpr float OFF = BITS == 4 ? 128.0f : 0.0f;
  constexpr int GB = GS * BITS / 8;               // bytes of one group of one column
  constexpr int LB = (BITS == 4 && GS == 32) ? 8 : 16;   // bytes per lane per step
  constexpr int GPS = 4 * LB / GB;                // groups per step: 1 or 2
  constexpr int LPG = 4 / GPS;                    // lanes (c4 values) per group
  constexpr int CPL = LB * 8 / BITS;              // codes per lane per step
  constexpr int JS = CPL / 8;                     // MFMA k-steps per step
  static_assert(GPS == 1 || GPS == 2, "step layout");
  __shared__ float red[KW][NT * 256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;
  const int ctn = (N + 16 * NT - 1) / (16 * NT);

  const int t = int(blockIdx.x / unsigned(ctn));
  const int n0 = int(blockIdx.x % unsigned(ctn)) * 16 * NT;
  if (t >= a.max_tiles) return;
  int e = 0;
  int64_t row0, seg_end;
  if (a.perm) {
    if (*a.tile_bm != 16) return;               // workspace routed for another tiling
    if (t >= a.tiles[a.E]) return;
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tiles[mid] <= t) lo = mid; else hi = mid;
    }
    // the search runs on identical values in every lane; say so, so that the
    // buffer descriptors built from e live in SGPRs
    e = __builtin_amdgcn_readfirstlane(lo);
    const int64_t nrows = a.n_pairs * a.M;
    row0 = min<int64_t>(max<int64_t>(int64_t(a.offsets[e]) * a.M, 0) + int64_t(t - a.tiles[e]) * 16,
                        nrows);
    seg_end = min<int64_t>(max<int64_t>(int64_t(a.offsets[e + 1]) * a.M, 0), nrows);
  } else {
    row0 = int64_t(t) * 16;
    seg_end = a.n_pairs * a.M;
  }
  if (row0 >= seg_end) return;
  const int rows = int(min<int64_t>(16, seg_end - row0));

  // ---- per-lane offsets ---------------------------------------------------------
  // x: lane (row l16, c4); rows past the tile read zeros (offset outside the
  // descriptor)
  uint32_t xoff = kNoRow;
  if (l16 < rows) {
    const int64_t j = row0 + l16;
    int64_t xrow;
    if (a.perm) {
      const int32_t pair = min<int64_t>(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1);
      const int m = int(j % a.M);
      const int tok = pair / a.A, slot = pair - tok * a.A;
      xrow = (int64_t(tok) * a.Ax + (a.Ax > 1 ? slot : 0)) * a.M + m;
    } else {
      xrow = j;
    }
    xoff = uint32_t(xrow * K * 2);
  }
  const int64_t wrow_bytes = int64_t(K) * BITS / 8;
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq + int64_t(e) * N * (K * BITS / 32),
                                         uint32_t(int64_t(N) * wrow_bytes));
  const __amdgpu_buffer_rsrc_t sr = rsrc(a.scales + int64_t(e) * N * G, uint32_t(N) * G * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(a.biases + int64_t(e) * N * G, uint32_t(N) * G * 2u);
  uint32_t woff[NT], soff[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(n0 + 16 * j + l16, N - 1);
    woff[j] = uint32_t(n * wrow_bytes) + uint32_t(LB) * c4;
    soff[j] = uint32_t(n) * G * 2u;
  }
  const int gsub = c4 / LPG;                       // group of the step this lane serves
  const int kl = (c4 % LPG) * CPL;                 // its first code within that group

  // ---- steps of this wave ----------------------------------------------------------
  const int nsteps = (G + GPS - 1) / GPS;
  const int per = (nsteps + KW - 1) / KW;
  const int s_lo = min(nsteps, wave * per), s_hi = min(nsteps, s_lo + per);

  // Loads of a step are issued DEPTH steps before its compute, x together
  // with the codes: vector-memory counters retire in issue order, so a step's
  // data must not be issued after the data of later steps.
  constexpr int DEPTH = 4;
  u32x4 cw[DEPTH][NT], xq[DEPTH][JS];
  uint32_t sv[DEPTH][NT], bv[DEPTH][NT];
  // Lane-dependent parts of an address go into the vector offset, the step's
  // (wave-uniform) advance into the scalar offset.  The second group of the
  // last step may not exist (odd G): its loads then read the next column's or
  // row's data, or zeros past the end of the buffer, and are not used.
  const uint32_t xlane = xoff + uint32_t(gsub * GS + kl) * 2u;
  uint32_t slane[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) slane[j] = soff[j] + uint32_t(gsub) * 2u;
  auto load_step = [&](int st, int slot) {
#pragma unroll
    for (int js = 0; js < JS; ++js)
      xq[slot][js] = __builtin_amdgcn_raw_buffer_load_b128(xr, xlane, (st * GPS * GS + 8 * js) * 2, 0);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (LB == 16) {
        cw[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[j], st * 4 * LB, 0);
      } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, woff[j], st * 4 * LB, 0);
        cw[slot][j] = u32x4{v[0], v[1], 0u, 0u};
      }
      sv[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, slane[j], st * GPS * 2, 0);
      bv[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(br, slane[j], st * GPS * 2, 0);
    }
  };

  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const bool first_half = gsub == 0;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (s_lo + d < s_hi) load_step(s_lo + d, d);
  for (int st0 = s_lo; st0 < s_hi; st0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int st = st0 + d;
      if (st >= s_hi) break;
      const bool second = GPS > 1 && st * GPS + 1 < G;   // the step's second group exists
      f32x4 Plo[NT], Phi[NT], Xlo = {0.f, 0.f, 0.f, 0.f}, Xhi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        Plo[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        Phi[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        // x of this lane goes to the half of the group it serves; the other
        // half's operand is zero in this lane
        const u32x4 xv = pair_k_with_k4(xq[d][js]);
        const u32x4 alo = (GPS == 1 || first_half) ? xv : zero4;
        Xlo = mfma(alo, ones, Xlo);
        u32x4 ahi = zero4;
        if constexpr (GPS > 1) {
          ahi = first_half ? zero4 : xv;
          Xhi = mfma(ahi, ones, Xhi);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          u32x4 bfrag;
          if constexpr (BITS == 4) bfrag = decode4(cw[d][j][js]);
          else bfrag = decode8(cw[d][j][2 * js], cw[d][j][2 * js + 1]);
          Plo[j] = mfma(alo, bfrag, Plo[j]);
          if constexpr (GPS > 1) Phi[j] = mfma(ahi, bfrag, Phi[j]);
        }
      }
      // each lane loaded the scale / bias of its own half's group; both halves'
      // values are fetched from a lane of each half (c4 = 0 and c4 = LPG)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint32_t slo = __shfl(sv[d][j], l16, 64), blo = __shfl(bv[d][j], l16, 64);
        const float s0 = __uint_as_float(slo << 16);
        const float c0 = __uint_as_float(blo << 16) - OFF * s0;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(s0, Plo[j][q], fmaf(c0, Xlo[q], acc[j][q]));
        if (second) {
          const uint32_t shi = __shfl(sv[d][j], l16 + 16 * LPG, 64);
          const uint32_t bhi = __shfl(bv[d][j], l16 + 16 * LPG, 64);
          const float s1 = __uint_as_float(shi << 16);
          const float c1 = __uint_as_float(bhi << 16) - OFF * s1;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(s1, Phi[j][q], fmaf(c1, Xhi[q], acc[j][q]));
        }
      }
      if (st + DEPTH < s_hi) load_step(st + DEPTH, d);
    }
  }

  // ---- reduce the waves' partial sums in a fixed order and store ------------------
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][j * 256 + (4 * c4 + q) * 16 + l16] = acc[j][q];
  __syncthreads();
  for (int i = tid; i < NT * 256; i += 64 * KW) {
    const int j = i >> 8, r = (i >> 4) & 15, c = i & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) sum += red[w][i];
    const int col = n0 + 16 * j + c;
    if (r < rows && col < N) {
      const int64_t jr = row0 + r;
      int64_t orow;
      if (a.perm)
        orow = min<int64_t>(max<int32_t>(a.perm[jr / a.M], 0), a.n_pairs - 1) * a.M + (jr % a.M);
      else orow = jr;
      a.out[orow * N + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
    }
  }
}

template <int BITS, int GS, int NT>
hipError_t launch_kw(const GemmArgs& a, int kw, dim3 grid, hipStream_t s) {
  if (kw == 8) small_m_kernel<BITS, GS, 8, NT><<<grid, dim3(512), 0, s>>>(a);
  else small_m_kernel<BITS, GS, 4, NT><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_nt(const GemmArgs& a, int nt, int kw, dim3 grid, hipStream_t s) {
  if (nt == 4) return launch_kw<BITS, GS, 4>(a, kw, grid, s);
  if (nt == 2) return launch_kw<BITS, GS, 2>(a, kw, grid, s);
  return launch_kw<BITS, GS, 1>(a, kw, grid, s);
}

}  // namespace

// Column blocks of 16 per wave: as many as keep >= ~2048 waves for the
// weight (x rows are loaded once per wave and shared by its column blocks).
int small_m_cols(int64_t N, int64_t tiles) {
  const int64_t cb = ceil_div(N, 16) * tiles;
  if (cb >= 4 * 256) return 4;
  if (cb >= 2 * 256) return 2;
  return 1;
}

int small_m_waves(int64_t blocks, int G) {
  // 8 waves when 4 would leave fewer than ~4 waves per SIMD and K is long
  // enough for several steps per wave
  return (blocks * 4 < 4096 && G >= 32) ? 8 : 4;
}

hipError_t launch_small_m(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  const int nt = a.nt;
  const int64_t blocks = ceil_div(a.N, 16 * nt) * a.max_tiles;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int kw = a.waves;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  if (a.bits == 4)
    return a.group_size == 32 ? launch_nt<4, 32>(a, nt, kw, grid, s) : launch_nt<4, 64>(a, nt, kw, grid, s);
  return a.group_size == 32 ? launch_nt<8, 32>(a, nt, kw, grid, s) : launch_nt<8, 64>(a, nt, kw, grid, s);
}

}  // namespace mq
