// Gathered grouped GEMM on unquantised bf16 expert weights (gfx950, bf16 MFMA).
//
// What it computes (ml-explore/mlx issue 4339, the follow-up comments on the
// bf16 MoE gather path, GatherMM): every routed row is multiplied by the
// transposed bf16 weight of its expert, out = x . W[e]^T, fp32 accumulation,
// rounded to bf16 once.  The routing, the tile table and the tile shapes are
// the quantised GEMM's: a tile is BM routed rows of one expert x 64 * NW
// columns, never straddling experts, and the unpermute is fused into the
// store.  What differs is the weight path: a B fragment is eight bf16 weights
// of one column, loaded straight into registers (one 16-byte load per
// 16-column block and MFMA k-step), with no decode, no per-group scale and no
// correction, so the MFMAs accumulate into the output tile directly.
//
// Layout of one workgroup (NW waves): wave w owns columns [64 w, 64 w + 64) of
// the tile, BM / 16 x 4 MFMA 16x16x32 blocks; x chunks of 64 k go from HBM to
// LDS (buffer_load ... lds) in three stages, two chunks in flight, 16-byte
// pieces swizzled so that the fragment reads are free of bank conflicts; the
// weights of a chunk (8 KB per wave) are loaded two chunks ahead.
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BK = 64;                          // k per chunk: 128 bytes of an x row
constexpr int KS = BK / 32;                     // MFMA k-steps per chunk
constexpr int NT = 4;                           // 16-column MFMA blocks per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;    // gfx9 raw buffer descriptor flags
constexpr uint32_t kNoRow = 0x80000000u;        // offset outside every descriptor range

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding)
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ inline int uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(int(v)); }

__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, int(voff), uni(soff), 0, 0);
}

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int BM, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void gather_mm_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  constexpr int MT = BM / 16;
  constexpr int BN = 64 * NW;
  constexpr int STAGE = BM * 128;                      // bytes of one x chunk
  constexpr int XDMA = BM * 8 / (64 * NW);             // x copies per wave per chunk
  static_assert(XDMA >= 1 && XDMA * 64 * NW == BM * 8, "x copies per chunk");
  constexpr int PPS = BM / 16;                         // 2 KiB store patches per stage
  static_assert(NW <= 3 * PPS, "store patches");
  // VMEM instructions one chunk issues for the chunk two ahead
  constexpr int PER = XDMA + KS * NT;

  __shared__ __attribute__((aligned(16))) unsigned char xs0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs2[STAGE];
  __shared__ int32_t xrow_tab[BM];
  __shared__ int32_t orow_tab[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N;

  // ---- which tile: the quantised GEMM's XCD-aware order ------------------------
  const int ntn = (N + BN - 1) / BN;
  const int ntiles = a.perm ? min64(a.tiles[a.E], a.max_tiles) : int(a.max_tiles);
  const unsigned per_xcd = unsigned(ntiles * ntn + 7) / 8u;
  if (blockIdx.x / 8u >= per_xcd) return;
  const unsigned logical = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  const int t = int(logical / unsigned(ntn));
  if (t >= ntiles) return;
  const int n0 = int(logical % unsigned(ntn)) * BN;
  int e = 0;
  int64_t row0, seg_end;
  if (a.perm) {
    if (*a.tile_bm != BM) return;
    const int step = (a.E + 64) / 64;
    const int i1 = min(lane * step, a.E);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(a.tiles[i1] <= t);
    const int lo = (63 - __builtin_clzll(m1)) * step;
    const int i2 = min(lo + lane, a.E);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < step && a.tiles[i2] <= t);
    e = __builtin_amdgcn_readfirstlane(min(lo + (63 - __builtin_clzll(m2)), a.E - 1));
    const int64_t nrows = a.n_pairs * a.M;
    row0 = min64(max64(int64_t(a.offsets[e]) * a.M, 0) +
                            int64_t(t - a.tiles[e]) * BM, nrows);
    seg_end = min64(max64(int64_t(a.offsets[e + 1]) * a.M, 0), nrows);
    if (row0 >= seg_end) return;
  } else {
    row0 = int64_t(t) * BM;
    seg_end = a.n_pairs * a.M;
    if (row0 >= seg_end) return;
  }
  const int rows = int(min64(BM, seg_end - row0));

  if (tid < BM) {
    int32_t xr = -1, orr = -1;
    if (tid < rows) {
      const int64_t j = row0 + tid;
      if (a.perm) {
        const int32_t pair = int32_t(min64(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1));
        const int m = int(j % a.M);
        const int tok = pair / a.A, slot = pair - tok * a.A;
        xr = (tok * a.Ax + (a.Ax > 1 ? slot : 0)) * a.M + m;
        orr = pair * a.M + m;
      } else {
        xr = orr = int32_t(j);
      }
    }
    xrow_tab[tid] = xr;
    orow_tab[tid] = orr;
  }
  __syncthreads();

  // ---- descriptors and offsets ------------------------------------------------
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const int64_t wrow_bytes = int64_t(K) * 2;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.w_bf16 + int64_t(e) * N * K, uint32_t(int64_t(N) * wrow_bytes));
  const __amdgpu_buffer_rsrc_t none = rsrc(a.x, 0u);
  // x copy j of this wave: rows 8 (j NW + wave) .. +7; lane -> row r, LDS slot
  // lane & 7, which holds 16-byte piece (slot ^ (r & 7) ^ ((r >> 3) & 1))
  uint32_t xoff[XDMA];
#pragma unroll
  for (int j = 0; j < XDMA; ++j) {
    const int r = (j * NW + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
    const int32_t xrow = xrow_tab[r];
    xoff[j] = xrow < 0 ? kNoRow : uint32_t(xrow) * uint32_t(K) * 2u + uint32_t(piece) * 16u;
  }
  // B fragment of block nt, k-step ks: column n0 + 64 wave + 16 nt + l16, k =
  // 64 chunk + 32 ks + 8 c4 .. +7; the block's distance rides in soffset, so
  // columns past N read zeros (computed, never stored)
  const uint32_t woff = uint32_t(n0 + 64 * wave + l16) * uint32_t(wrow_bytes) + 16u * c4;
  const uint32_t wstep = 16u * uint32_t(wrow_bytes);
  // x fragment of k-step ks: row 16 mt + l16, piece 4 ks + c4, swizzled as above
  const uint32_t aoff0 = uint32_t(l16 * 128 + 16 * (c4 ^ (l16 & 7) ^ ((l16 >> 3) & 1)));

  auto issue_x = [&](__amdgpu_buffer_rsrc_t r, unsigned char* stage, int chunk) {
#pragma unroll
    for (int j = 0; j < XDMA; ++j)
      dma16(r, stage + (j * NW + wave) * 1024, xoff[j], uint32_t(chunk) * (BK * 2));
  };
  auto load_w = [&](__amdgpu_buffer_rsrc_t r, int chunk, u32x4 (&dst)[KS][NT]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        dst[ks][nt] = __builtin_amdgcn_raw_buffer_load_b128(
            r, woff, uni(uint32_t(chunk) * (BK * 2) + uint32_t(ks) * 64u + uint32_t(nt) * wstep), 0);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = K / BK;
  u32x4 wb0[KS][NT], wb1[KS][NT];

  // ---- prologue: chunks 0 and 1 in flight ----------------------------------------
  issue_x(xr, xs0, 0);
  load_w(wr, 0, wb0);
  const bool one = nchunks > 1;
  issue_x(one ? xr : none, xs1, 1);
  load_w(one ? wr : none, 1, wb1);

  // one chunk: x stage `cur` holds chunk c, its weights are in `wb`; chunk
  // c + 2's copy goes to `nxt` (chunk c - 1's stage) and its weights to `wb`
  // once this chunk's MFMAs have read them
  auto chunk = [&](int c, unsigned char* cur, unsigned char* nxt, u32x4 (&wb)[KS][NT]) {
    __builtin_amdgcn_sched_barrier(0);
    // this chunk's copies and weights were issued two chunks ago: at most the
    // previous chunk's PER loads may still be in flight
    wait_vmem<PER>();
    wait_lds();
    __builtin_amdgcn_s_barrier();
    const int cn = c + 2;
    const bool pre = cn < nchunks;
    issue_x(pre ? xr : none, nxt, cn);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(cur + mt * 2048 + (aoff0 ^ (ks ? 64u : 0u)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma(af, wb[ks][nt], acc[mt][nt]);
      }
    }
    load_w(pre ? wr : none, cn, wb);
  };
  for (int c = 0;; c += 6) {
    chunk(c, xs0, xs2, wb0);
    if (c + 1 >= nchunks) break;
    chunk(c + 1, xs1, xs0, wb1);
    if (c + 2 >= nchunks) break;
    chunk(c + 2, xs2, xs1, wb0);
    if (c + 3 >= nchunks) break;
    chunk(c + 3, xs0, xs2, wb1);
    if (c + 4 >= nchunks) break;
    chunk(c + 4, xs1, xs0, wb0);
    if (c + 5 >= nchunks) break;
    chunk(c + 5, xs2, xs1, wb1);
    if (c + 6 >= nchunks) break;
  }

  // ---- store: fp32 -> bf16 through a per-wave LDS patch, then row segments ------
  wait_vmem<0>();
  wait_lds();
  __syncthreads();
  unsigned char* patch_base = wave < PPS ? xs0 : (wave < 2 * PPS ? xs1 : xs2);
  uint16_t* patch = reinterpret_cast<uint16_t*>(patch_base + (wave % PPS) * 2048);
  const bool vec_ok = (N % 8) == 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * c4 + i, col = 16 * nt + l16;
        patch[r * 64 + (((col >> 3) ^ (r & 7)) << 3) + (col & 7)] =
            __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mt][nt][i]));
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int seg = lane + 64 * h;
      const int r = seg >> 3, cs = seg & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&patch[r * 64 + ((cs ^ (r & 7)) << 3)]);
      const int tr = mt * 16 + r;
      const int col = n0 + 64 * wave + 8 * cs;
      if (tr < rows && col < N) {
        uint16_t* dst = a.out + int64_t(orow_tab[tr]) * N + col;
        if (vec_ok) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (col + q < N) dst[q] = uint16_t(v[q >> 1] >> (16 * (q & 1)));
        }
      }
    }
  }
}

template <int BM>
hipError_t launch_mm_bm(const GemmArgs& a, hipStream_t s) {
  constexpr int NW = BM == 16 ? 2 : 4;
  constexpr int BN = 64 * NW;
  const int64_t blocks = ceil_div(ceil_div(a.N, BN) * a.max_tiles, 8) * 8;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  note_dispatch("gather_mm", {BM, NW});
  gather_mm_kernel<BM, NW><<<dim3(unsigned(blocks)), dim3(64 * NW), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_mm(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  switch (a.bm) {
    case 16: return launch_mm_bm<16>(a, s);
    case 32: return launch_mm_bm<32>(a, s);
    case 64: return launch_mm_bm<64>(a, s);
    default: return launch_mm_bm<128>(a, s);
  }
}

}  // namespace mq
