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
// Exactness.  A code q enters the MFMA as the bf16 value 128 + q (4-bit: built
// by OR-ing the nibble into the mantissa of 128.0) or as q itself (8-bit: an
// exact integer -> float conversion).  Per group g the MFMA accumulates
// P_g = sum_k x_k (off + q_k) in fp32 and one fp32 FMA per output adds s_g P_g.
// The rest, sum_g X_g (b_g - off s_g) with X_g the row sum of x over the group,
// is added by "correction" MFMAs once per window of 32 groups: X_g is split
// into three bf16 parts whose sum is X_g to 2^-24, and b_g and -128 s_g are
// exact in bf16, so every product is exact and only fp32 summation rounds.
// No bf16 rounding of a dequantised weight ever happens.
//
// Layout of one workgroup (NW waves, NW in {4, 8}):
//   tile   BM routed rows of one expert x BN = 32*NW output columns;
//   wave w owns columns [32w, 32w + 32): BM/16 x 2 MFMA 16x16x32 blocks, so
//          every code is decoded once per workgroup;
//   loads  buffer loads through SGPR resource descriptors: per-lane 32-bit
//          offsets are computed once, the chunk advance rides in the scalar
//          offset, and gathered rows past the segment end fall outside the
//          descriptor's range and read as zeros;
//   K      walked in chunks of 64, register prefetch two chunks ahead; the
//          chunk's x rows are written to LDS (double buffered) with k pairs
//          permuted to the order the code decode produces, and their row sums
//          (v_dot2 against 1.0 plus DPP reductions) to a window table;
//   store  fp32 -> bf16 (RNE) through LDS, then 16-byte row segments to
//          out[pair * M + m] (the unpermute of the routing is fused here).
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;                   // k per chunk
constexpr int XS_STRIDE = BK + 8;        // bf16 per LDS row of the x chunk (16-byte pad)
constexpr int WIN = 32;                  // groups per correction window (one MFMA k-step)
constexpr int XW_STRIDE = WIN + 4;       // floats per row of the window's row sums
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // gfx9 raw buffer descriptor flags
constexpr uint32_t kNoRow = 0x80000000u;        // offset outside every descriptor range (< 2 GiB)

__device__ inline float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

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

// v . (1, 1) + c for a bf16 pair, exact products, fp32 sum
__device__ inline float dot2_ones(uint32_t v, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), c, false);
}

// fp32 -> three bf16 parts whose sum equals v to within 2^-24 relative
// (each part is the round-to-nearest-even of the remainder left by the ones
// before it).
__device__ inline void split3(float v, uint32_t& h, uint32_t& m, uint32_t& l) {
  const __bf16 bh = static_cast<__bf16>(v);
  const float r1 = v - static_cast<float>(bh);
  const __bf16 bm = static_cast<__bf16>(r1);
  const float r2 = r1 - static_cast<float>(bm);
  const __bf16 bl = static_cast<__bf16>(r2);
  h = __builtin_bit_cast(uint16_t, bh);
  m = __builtin_bit_cast(uint16_t, bm);
  l = __builtin_bit_cast(uint16_t, bl);
}

template <int BM, int NW>
struct Smem {
  static constexpr int BN = 32 * NW;
  static constexpr int YS_STRIDE = BN + 8;
  static constexpr int XS_BYTES = 2 * BM * XS_STRIDE * 2;
  static constexpr int XW_BYTES = BM * XW_STRIDE * 4;
  static constexpr int MAIN = XS_BYTES + XW_BYTES;
  static constexpr int STORE = BM * YS_STRIDE * 2;
  static constexpr int BYTES = MAIN > STORE ? MAIN : STORE;
};

template <int BM, int BITS, int GS, int NW>
__global__ __launch_bounds__(64 * NW) void gather_gemm_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(GS == 32 || GS == 64, "GS");
  constexpr int THREADS = 64 * NW;
  constexpr int BN = 32 * NW;
  constexpr int MT = BM / 16;                    // MFMA row blocks per wave
  constexpr int NT = 2;                          // MFMA column blocks per wave
  constexpr int GPC = BK / GS;                   // groups per chunk
  constexpr int KS = BK / 32;                    // MFMA k-steps per chunk
  constexpr int KSG = KS / GPC;                  // k-steps per group
  constexpr int ROWS_PER_PASS = THREADS / 8;     // x rows staged per pass (8 pieces a row)
  constexpr int PASSES = BM >= ROWS_PER_PASS ? BM / ROWS_PER_PASS : 1;
  constexpr int CW = KS * BITS / 4;              // code words per lane and column block per chunk
  constexpr int CPW = WIN / GPC;                 // chunks per window
  constexpr bool OFFSET = BITS == 4;             // codes enter the MFMA as 128 + q
  using S = Smem<BM, NW>;

  __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                    // [2][BM*XS_STRIDE]
  float* xw = reinterpret_cast<float*>(smem + S::XS_BYTES);            // [BM*XW_STRIDE]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;

  // ---- which tile: XCD-aware order ----------------------------------------
  // Workgroups are dealt to the 8 XCDs round-robin.  Renumbering them so that
  // each XCD receives a contiguous range of (row tile, column tile) pairs,
  // column tiles fastest, keeps a row tile's gathered x rows in one L2.
  const unsigned per_xcd = gridDim.x / 8u;       // the grid is padded to a multiple of 8
  const unsigned logical = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  const int ntn = (N + BN - 1) / BN;
  const int t = int(logical / unsigned(ntn));
  if (t >= a.max_tiles) return;
  const int n0 = int(logical % unsigned(ntn)) * BN;
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
    // the search runs on identical values in every lane; say so, so that the
    // buffer descriptors built from e live in SGPRs
    e = __builtin_amdgcn_readfirstlane(lo);
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

  // ---- descriptors and per-lane offsets ---------------------------------------
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const int64_t wrow_bytes = int64_t(K) * BITS / 8;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq + int64_t(e) * N * (K * BITS / 32),
                                         uint32_t(int64_t(N) * wrow_bytes));
  const __amdgpu_buffer_rsrc_t sr = rsrc(a.scales + int64_t(e) * N * G, uint32_t(N) * G * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(a.biases + int64_t(e) * N * G, uint32_t(N) * G * 2u);

  const int piece = tid & 7;                     // 16-byte piece of a 64-k chunk row
  uint32_t xoff[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = (tid >> 3) + ROWS_PER_PASS * p;
    xoff[p] = kNoRow;
    if (r < BM && r < rows) {
      const int64_t j = row0 + r;
      int64_t xrow;
      if (a.perm) {
        const int32_t pair = min<int64_t>(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1);
        const int m = int(j % a.M);
        const int tok = pair / a.A, slot = pair - tok * a.A;
        xrow = (int64_t(tok) * a.Ax + (a.Ax > 1 ? slot : 0)) * a.M + m;
      } else {
        xrow = j;
      }
      xoff[p] = uint32_t(xrow * K * 2 + piece * 16);
    }
  }
  uint32_t woff[NT], soff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(n0 + 32 * wave + 16 * nt + l16, N - 1);
    // this lane's 8 codes of k-step ks sit at k offset 16*c4 + 8*ks of the
    // chunk for GS=64 (both k-steps adjacent), 32*ks + 8*c4 for GS=32
    woff[nt] = uint32_t(n * wrow_bytes) + (GS == 64 ? 2 * BITS * c4 : BITS * c4);
    soff[nt] = uint32_t(n) * G * 2u;
  }

  // ---- loads (issued two chunks ahead) --------------------------------------
  auto load_x = [&](int chunk, u32x4 (&dst)[PASSES]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      dst[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[p], chunk * BK * 2, 0);
  };
  auto load_codes = [&](int chunk, uint32_t (&dst)[NT][CW]) {
    const int so = chunk * BK * BITS / 8;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (BITS == 4 && GS == 64) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, woff[nt], so, 0);
        dst[nt][0] = v[0];
        dst[nt][1] = v[1];
      } else if constexpr (BITS == 4) {
        dst[nt][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff[nt], so, 0);
        dst[nt][1] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff[nt], so + 16, 0);
      } else if constexpr (GS == 64) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[nt], so, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[nt][i] = v[i];
      } else {
        const u32x2 v0 = __builtin_amdgcn_raw_buffer_load_b64(wr, woff[nt], so, 0);
        const u32x2 v1 = __builtin_amdgcn_raw_buffer_load_b64(wr, woff[nt], so + 32, 0);
        dst[nt][0] = v0[0];
        dst[nt][1] = v0[1];
        dst[nt][2] = v1[0];
        dst[nt][3] = v1[1];
      }
    }
  };
  auto load_scales = [&](int chunk, uint32_t (&dst)[NT][GPC]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int gl = 0; gl < GPC; ++gl)
        dst[nt][gl] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff[nt], (chunk * GPC + gl) * 2, 0);
  };
  // bias and scale bf16 of the 8 groups w*WIN + 8*c4 .. +7 of this lane's
  // column, zero beyond the last group
  auto load_window = [&](int w, u32x4 (&bw)[NT], u32x4 (&sw)[NT]) {
    const int g0 = w * WIN + 8 * c4;
    if ((G % 8) == 0 && w * WIN + WIN <= G) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bw[nt] = __builtin_amdgcn_raw_buffer_load_b128(br, soff[nt] + 16u * c4, w * WIN * 2, 0);
        sw[nt] = OFFSET ? __builtin_amdgcn_raw_buffer_load_b128(sr, soff[nt] + 16u * c4, w * WIN * 2, 0)
                        : u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t bb[8], ss[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool in = g0 + i < G;
          const uint32_t o = soff[nt] + uint32_t(in ? g0 + i : 0) * 2u;
          const uint32_t bv = __builtin_amdgcn_raw_buffer_load_b16(br, o, 0, 0);
          const uint32_t sv = OFFSET ? __builtin_amdgcn_raw_buffer_load_b16(sr, o, 0, 0) : 0u;
          bb[i] = in ? bv : 0u;
          ss[i] = in ? sv : 0u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bw[nt][i] = bb[2 * i] | (bb[2 * i + 1] << 16);
          sw[nt][i] = ss[2 * i] | (ss[2 * i + 1] << 16);
        }
      }
    }
  };

  // ---- x staging: gathered rows -> LDS (k pairs permuted) + row sums ---------
  auto stage_x = [&](int buf, int gw0, const u32x4 (&src)[PASSES]) {
    uint16_t* xb = xs + buf * (BM * XS_STRIDE);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = (tid >> 3) + ROWS_PER_PASS * p;
      if (BM >= ROWS_PER_PASS || r < BM) {
        const u32x4 u = src[p];
        *reinterpret_cast<u32x4*>(&xb[r * XS_STRIDE + piece * 8]) = pair_k_with_k4(u);
        float s = dot2_ones(u[0], 0.f);
        s = dot2_ones(u[1], s);
        s = dot2_ones(u[2], s);
        s = dot2_ones(u[3], s);
        // sum over the lanes holding one (row, group): 8 lanes at GS=64
        // (quad pairs, quads, then row_ror:12, which hands lane i the value
        // of lane i+4 within its 16-lane row), 4 lanes at GS=32; the total
        // lands in the group's first lane
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
        s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
        if constexpr (GS == 64)
          s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x12C, 0xF, 0xF, false));
        constexpr int LANES = GS / 8;
        if ((piece % LANES) == 0) xw[r * XW_STRIDE + gw0 + piece / LANES] = s;
      }
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // main product of one chunk: per group and row block, P = x . (off + q) by
  // MFMA, then acc += s * P (bias and offset terms come from the correction)
  auto compute = [&](int buf, const uint32_t (&cw)[NT][CW], const uint32_t (&sv)[NT][GPC]) {
    const uint16_t* xb = xs + buf * (BM * XS_STRIDE);
    u32x4 bfrag[KS][NT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (BITS == 4) bfrag[ks][nt] = decode4(cw[nt][ks]);
        else bfrag[ks][nt] = decode8(cw[nt][2 * ks], cw[nt][2 * ks + 1]);
      }
#pragma unroll
    for (int gl = 0; gl < GPC; ++gl) {
      float s[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt] = bf16lo(sv[nt][gl]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 P[NT];
#pragma unroll
        for (int ksg = 0; ksg < KSG; ++ksg) {
          const int ks = gl * KSG + ksg;
          const int ko = GS == 32 ? 32 * ks + 8 * c4 : 16 * c4 + 8 * ks;
          const u32x4 afrag = *reinterpret_cast<const u32x4*>(&xb[(mt * 16 + l16) * XS_STRIDE + ko]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            P[nt] = mfma(afrag, bfrag[ks][nt], ksg == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(s[nt], P[nt][i], acc[mt][nt][i]);
      }
    }
  };

  // window correction: acc += sum_g X_g * b_g  (- 128 * X_g * s_g for 4-bit),
  // with X split into three exact bf16 parts, as MFMAs over the window's groups
  auto correct = [&](const u32x4 (&bw)[NT], const u32x4 (&sw)[NT]) {
    u32x4 bneg[NT];
    if constexpr (OFFSET) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = -128.0f * bf16lo(sw[nt][i]);     // exact: a power-of-two scaling
          const float hi = -128.0f * bf16hi(sw[nt][i]);
          bneg[nt][i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float* xp = &xw[(mt * 16 + l16) * XW_STRIDE + 8 * c4];
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(xp);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(xp + 4);
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        split3(v0[i], h[i], m[i], l[i]);
        split3(v1[i], h[4 + i], m[4 + i], l[4 + i]);
      }
      u32x4 ah, am, al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ah[i] = h[2 * i] | (h[2 * i + 1] << 16);
        am[i] = m[2 * i] | (m[2 * i + 1] << 16);
        al[i] = l[2 * i] | (l[2 * i + 1] << 16);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[mt][nt] = mfma(ah, bw[nt], acc[mt][nt]);
        acc[mt][nt] = mfma(am, bw[nt], acc[mt][nt]);
        acc[mt][nt] = mfma(al, bw[nt], acc[mt][nt]);
        if constexpr (OFFSET) {
          acc[mt][nt] = mfma(ah, bneg[nt], acc[mt][nt]);
          acc[mt][nt] = mfma(am, bneg[nt], acc[mt][nt]);
          acc[mt][nt] = mfma(al, bneg[nt], acc[mt][nt]);
        }
      }
    }
  };

  // the window's row sums start at zero so that a partial window adds nothing
  for (int i = tid; i < BM * XW_STRIDE; i += THREADS) xw[i] = 0.f;
  __syncthreads();                               // before any row sum is written

  const int nchunks = K / BK;
  u32x4 xA[PASSES], xB[PASSES];
  uint32_t cA[NT][CW], cB[NT][CW];
  uint32_t sA[NT][GPC], sB[NT][GPC];
  u32x4 bw[NT], sw[NT];
  load_x(0, xA);
  load_codes(0, cA);
  load_scales(0, sA);
  if (nchunks > 1) {
    load_x(1, xB);
    load_codes(1, cB);
    load_scales(1, sB);
  }

  auto chunk = [&](int c, u32x4 (&xr_)[PASSES], uint32_t (&cw)[NT][CW], uint32_t (&sv)[NT][GPC]) {
    const int buf = c & 1;
    if (c % CPW == 0) load_window(c / CPW, bw, sw);
    stage_x(buf, (c % CPW) * GPC, xr_);
    __syncthreads();
    uint32_t cur[NT][CW], scur[NT][GPC];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < CW; ++i) cur[nt][i] = cw[nt][i];
#pragma unroll
      for (int i = 0; i < GPC; ++i) scur[nt][i] = sv[nt][i];
    }
    if (c + 2 < nchunks) {
      load_x(c + 2, xr_);
      load_codes(c + 2, cw);
      load_scales(c + 2, sv);
    }
    compute(buf, cur, scur);
    if ((c + 1) % CPW == 0 || c + 1 == nchunks) {
      correct(bw, sw);
      __syncthreads();                           // xw is rewritten by the next window
    }
  };
  for (int c = 0; c < nchunks; c += 2) {
    chunk(c, xA, cA, sA);
    if (c + 1 < nchunks) chunk(c + 1, xB, cB, sB);
  }

  // ---- store: fp32 -> bf16 through LDS, then row segments --------------------
  __syncthreads();
  uint16_t* ys = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * c4 + i;
        const int c = 32 * wave + 16 * nt + l16;
        ys[r * S::YS_STRIDE + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mt][nt][i]));
      }
  __syncthreads();
  const bool vec_ok = (N % 8) == 0;
  for (int idx = tid; idx < BM * (BN / 8); idx += THREADS) {
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
    const uint16_t* srcp = &ys[r * S::YS_STRIDE + pc * 8];
    if (vec_ok) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(srcp);
    } else {
      for (int q = 0; q < 8 && c + q < N; ++q) dst[q] = srcp[q];
    }
  }
}

template <int BM, int BITS, int NW>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BN = 32 * NW;
  // padded to a multiple of 8 for the XCD-aware renumbering in the kernel
  const int64_t blocks = ceil_div(ceil_div(a.N, BN) * a.max_tiles, 8) * 8;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  if (a.group_size == 32)
    gather_gemm_kernel<BM, BITS, 32, NW><<<grid, dim3(64 * NW), 0, s>>>(a);
  else
    gather_gemm_kernel<BM, BITS, 64, NW><<<grid, dim3(64 * NW), 0, s>>>(a);
  return hipGetLastError();
}

template <int BM, int BITS>
hipError_t launch_bm_bits(const GemmArgs& a, hipStream_t s) {
  return a.waves == 8 ? launch_cfg<BM, BITS, 8>(a, s) : launch_cfg<BM, BITS, 4>(a, s);
}

template <int BM>
hipError_t launch_bm(const GemmArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_bm_bits<BM, 4>(a, s) : launch_bm_bits<BM, 8>(a, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  switch (a.bm) {
    case 16: return launch_bm<16>(a, s);
    case 32: return launch_bm<32>(a, s);
    case 64: return launch_bm<64>(a, s);
    default: return launch_bm<128>(a, s);
  }
}

}  // namespace mq
