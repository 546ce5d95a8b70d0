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
// Exactness.  A code q enters the MFMA as the bf16 value 16 + q (4-bit: built
// by OR-ing the nibble into mantissa bits 3..6 of 16.0) or as q itself (8-bit:
// an exact integer -> float conversion).  Per group g the MFMA accumulates
// P_g = sum_k x_k (off + q_k) in fp32 and one fp32 FMA per output adds s_g P_g.
// The rest, sum_g X_g (b_g - off s_g) with X_g the row sum of x over group g,
// is added by "correction" MFMAs once per window of 32 groups: X_g comes from
// the routing launch's row-sum workgroups as three bf16 parts whose sum is X_g
// to 2^-24, b_g and -16 s_g are exact in bf16, so every product is exact and
// only fp32 summation rounds.  No bf16 rounding of a dequantised weight ever
// happens.  The offset is the smallest power of two above every 4-bit code:
// the fp32 sums then cancel the least (P_g is ~3x sum_k x_k q_k, against ~18x
// for an offset of 128).
//
// Layout of one workgroup (NW waves):
//   tile   BM routed rows of one expert x BN = 64*NW output columns;
//   wave w owns columns [64w, 64w + 64): BM/16 x 4 MFMA 16x16x32 blocks, so
//          every code is decoded once per workgroup and reused BM/16 times,
//          and every x fragment read from LDS feeds 4 MFMAs;
//   x      K is walked in chunks of 64.  The chunk's gathered rows go straight
//          from HBM into LDS (buffer_load ... lds, three stages, two chunks in
//          flight); 16-byte pieces are XOR-swizzled by row so that the MFMA
//          fragment reads are free of bank conflicts;
//   codes  buffer loads into registers, two chunks ahead, decoded to bf16 in
//          natural k order (the x fragment is 8 consecutive k of one row);
//   sums   the window's row-sum parts are fetched into LDS one window ahead;
//   store  fp32 -> bf16 (RNE) through a per-wave LDS patch, then 16-byte row
//          segments to out[pair * M + m] (the unpermute of the routing is
//          fused here).
// Pipeline waits are explicit: each stage is its own LDS array, so the
// compiler can tell which DMA a fragment read depends on; a wave waits for its
// own copies with s_waitcnt vmcnt and an s_barrier publishes them.
#include <type_traits>

#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BK = 64;                   // k per chunk: 128 bytes of an x row
constexpr int WIN = 32;                  // groups per correction window (one MFMA k-step)
// a piece of a tail tile split along K: up to 4 row blocks (64 rows) of 4
// waves x NT <= 4 column blocks, fp32, in a slot of kTailPieceBytes
constexpr int kPieceMT = 4;
// workgroups of the reduce at most (each takes items in turn)
constexpr int kReduceBlocks = 512;
constexpr int kPieceFloats = int(kTailPieceBytes / 4);
static_assert(4 * kPieceMT * 4 * 256 == kPieceFloats, "tail piece slot");
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // gfx9 raw buffer descriptor flags
constexpr uint32_t kNoRow = 0x80000000u;        // offset outside every descriptor range (< 2 GiB)

__device__ inline float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// every LDS access of this wave has completed
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// This lane's index, computed afresh: values derived from it that are only
// needed once per window or in the epilogue are then recomputed there rather
// than held in registers (or scratch) through the whole K loop.
__device__ inline int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// A uniform buffer offset, stated as such: the compiler may keep a uniform
// value in a VGPR when SGPRs run short, and a VGPR soffset is served by a
// loop over the distinct values of its lanes.
__device__ inline int uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(int(v)); }

// 16 bytes per lane from global (buffer offset voff + soff) to LDS at
// lds + 16 * lane; offsets outside the descriptor write zeros
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, int(voff), uni(soff), 0, 0);
}

// 8 four-bit codes (k0..k7 in nibbles 0..7) -> bf16 (16+q) pairs in natural
// order (k0,k1),(k2,k3),(k4,k5),(k6,k7).  16 + q = 2^4 (1 + q/16) is 16.0
// (0x4180) with q in mantissa bits 3..6: byte i of w << 3 holds k_2i in bits
// 3..6 and byte i of w >> 1 holds k_2i+1 there.  `mask` (0x00780078, in an
// SGPR) and `base` (0x41804180, in a VGPR) are passed in registers so that
// each pair is one v_perm_b32 + one v_and_or_b32 (a VOP3 instruction takes no
// literal operand on gfx9).
__device__ inline u32x4 decode4(uint32_t w, uint32_t mask, uint32_t base) {
  const uint32_t lo = w << 3, hi = w >> 1;
  u32x4 r;
  r[0] = (__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) & mask) | base;
  r[1] = (__builtin_amdgcn_perm(hi, lo, 0x0C050C01u) & mask) | base;
  r[2] = (__builtin_amdgcn_perm(hi, lo, 0x0C060C02u) & mask) | base;
  r[3] = (__builtin_amdgcn_perm(hi, lo, 0x0C070C03u) & mask) | base;
  return r;
}

// 8 eight-bit codes (k0..k3 in w0, k4..k7 in w1) -> exact bf16 pairs in
// natural order: q < 256 is exact in the upper half of its fp32 value.
__device__ inline u32x4 decode8(uint32_t w0, uint32_t w1) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t w = j == 0 ? w0 : w1;
    const uint32_t a = __float_as_uint(float(w & 0xFFu));
    const uint32_t b = __float_as_uint(float((w >> 8) & 0xFFu));
    const uint32_t c = __float_as_uint(float((w >> 16) & 0xFFu));
    const uint32_t d = __float_as_uint(float(w >> 24));
    r[2 * j] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    r[2 * j + 1] = __builtin_amdgcn_perm(d, c, 0x07060302u);
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
__device__ inline void split3(float v, uint16_t& h, uint16_t& m, uint16_t& l) {
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
struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int MT = BM / 16;
  static constexpr int STAGE = BM * 128;                 // bytes of one x chunk
  static constexpr int XDMA = BM * 8 / (64 * NW);        // x copies per wave per chunk
  static constexpr int SUMS = 3 * BM * 64;               // bytes of one window's row-sum parts
  static constexpr int SDMA_ALL = 3 * BM / 16;           // copies per window (16 rows x 1 part each)
  static constexpr int SDMA = (SDMA_ALL + NW - 1) / NW;  // per wave (the last one may repeat)
  static constexpr int PATCH_PER_STAGE = BM / 16;        // 2 KiB store patches per x stage
  static_assert(XDMA >= 1 && XDMA * 64 * NW == BM * 8, "x copies per chunk");
  static_assert(NW <= 3 * PATCH_PER_STAGE, "store patches");
};

// Short tiles are bound by memory latency, not by the matrix cores: their
// launch bounds ask for more resident waves (16-row tiles: 4 per SIMD, 128
// VGPRs; 32-row tiles: 3 per SIMD, 168 VGPRs) so that more of them have
// loads in flight.
template <int BM>
constexpr int waves_per_simd() { return BM == 16 ? 4 : (BM == 32 ? 3 : 2); }

// NT: 16-column MFMA blocks per wave, 4 (64 columns) or 3 (48 columns; the
// host picks it where tiles of 48 * NW columns spread more evenly over the
// CUs than tiles of 64 * NW).
// GLU: the gate and up projections of an MoE FFN in one pass.  Waves
// 0 .. NW/2 - 1 compute 64-column slices of the gate projection (a.wq /
// scales / biases), waves NW/2 .. NW - 1 the same slices of the up projection
// (a.wq2 / scales2 / biases2): every wave runs the plain product's loop on
// one weight, and the tile's x chunk in LDS serves both.  In the store each
// up wave hands its fp32 results to its gate partner through LDS, which forms
// act(gate) * up; a tile is 32 * NW output columns wide.
// One tile: rows row0 .. row0 + rows - 1 (rows <= BM) of expert e's segment
// (the dense product: of x), output columns n0 .. n0 + BN - 1, over the
// chunks c0 .. c1 - 1 of K (c0 a multiple of the chunks per correction
// window).  With part == nullptr the tile covers all of K and stores bf16
// outputs; otherwise (a piece of a tail tile split along K, BM <= 64) it
// stores its fp32 partial sums to part, in the layout tail_reduce_kernel
// reads.  The LDS arrays are the kernel's, sized for its tallest tile.
template <int BM, int BITS, int GS, int NW, bool GLU, int NT, bool PAIRS>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const int e, const int64_t row0,
                                          const int rows, const int n0, unsigned char* const xs0,
                                          unsigned char* const xs1, unsigned char* const xs2,
                                          unsigned char* const sums, int32_t* const xrow_tab,
                                          int32_t* const orow_tab, const int c0, const int c1,
                                          float* const part) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(GS == 32 || GS == 64, "GS");
  static_assert(NT == 4 || (NT == 3 && !GLU), "column blocks per wave");
  using C = Cfg<BM, NW>;
  constexpr int MT = C::MT;
  constexpr int WCOLS = 16 * NT;                 // weight columns per wave
  constexpr int HW = GLU ? NW / 2 : NW;          // waves per weight
  constexpr int BN = WCOLS * HW;                 // output columns per tile
  static_assert(!GLU || NW % 2 == 0, "gate and up waves in pairs");
  constexpr int GPC = BK / GS;                   // groups per chunk
  constexpr int KS = BK / 32;                    // MFMA k-steps per chunk
  constexpr int KSG = KS / GPC;                  // k-steps per group
  constexpr int CW = BITS == 4 ? 2 : 4;          // code words per lane and column block per chunk
  constexpr int CLOADS = GS == 64 ? 1 : 2;       // code loads per column block per chunk
  constexpr int CPW = WIN / GPC;                 // chunks per window
  constexpr bool OFFSET = BITS == 4;             // codes enter the MFMA as 16 + q
  // VMEM instructions one chunk issues for the chunk two ahead: its x
  // copies, its code loads and one scale load
  constexpr int PER = C::XDMA + NT * CLOADS + 1;
  // 4-bit codes in 64-wide groups (PAIRS: launches of 4 waves): each column
  // block's codes come in one 16-byte load per lane for two chunks (a chunk
  // pair), issued two chunks before the pair's first.  8-byte loads of one
  // chunk hold the memory pipeline to ~70 % of the rate 16-byte loads reach
  // on the same bytes.  The pair buffers take 8 more VGPRs: the 128-row
  // launches then keep 2-3 VGPRs in scratch (and run 5-9 % faster on long K
  // all the same); the 2-wave 16-row launch has no room for them.
  constexpr bool PAIR = PAIRS && BITS == 4 && GS == 64;
  // loads an odd chunk of a pair issues: its x copies and one scale load
  constexpr int PER_ODD = C::XDMA + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;


  // ---- the tile's x rows and output rows ------------------------------------
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

  // ---- descriptors and per-lane offsets ---------------------------------------
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t sumr = rsrc(a.sums, a.sums_bytes);
  const int64_t wrow_bytes = int64_t(K) * BITS / 8;
  // the wave's weight (GLU: gate or up) and its slice of that weight's columns
  const bool upw = GLU && wave >= HW;
  const int slice = GLU ? wave % HW : wave;
  const uint32_t* const wq_e = (upw ? a.wq2 : a.wq) + int64_t(e) * N * (K * BITS / 32);
  const uint16_t* const sc_e = (upw ? a.scales2 : a.scales) + int64_t(e) * N * G;
  const uint16_t* const bi_e = (upw ? a.biases2 : a.biases) + int64_t(e) * N * G;
  const __amdgpu_buffer_rsrc_t wr = rsrc(wq_e, uint32_t(int64_t(N) * wrow_bytes));
  const __amdgpu_buffer_rsrc_t sr = rsrc(sc_e, uint32_t(N) * G * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(bi_e, uint32_t(N) * G * 2u);

  // x copy j of this wave: rows 8 (j NW + wave) .. +7; lane -> row r, LDS
  // slot lane & 7, which holds 16-byte piece (slot ^ (r & 7)) of the row
  uint32_t xoff[C::XDMA];
#pragma unroll
  for (int j = 0; j < C::XDMA; ++j) {
    const int r = (j * NW + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
    const int32_t xrow = xrow_tab[r];
    xoff[j] = xrow < 0 ? kNoRow : uint32_t(xrow) * uint32_t(K) * 2u + uint32_t(piece) * 16u;
  }
  // row-sum copy j of this wave: 16 rows x one part; lane -> row 16 rb +
  // lane / 4, LDS slot lane & 3, which holds the 8 groups (slot ^ ((row >> 1)
  // & 3)) of the window.  Recomputed per window from the row table (the
  // offsets would otherwise hold registers through the whole K loop).
  auto sum_copy = [&](int j, uint32_t& voff, int& dst) {
    const int lane = fresh_lane();
    const int i = min(wave + NW * j, C::SDMA_ALL - 1);
    const int part = i / (BM / 16), rb = i % (BM / 16);
    const int row = rb * 16 + (lane >> 2);
    const int gslot = (lane & 3) ^ ((row >> 1) & 3);
    const int32_t xrow = xrow_tab[row];
    voff = xrow < 0 ? kNoRow
                    : (uint32_t(xrow) * 3u + uint32_t(part)) * uint32_t(a.Gp) * 2u +
                          uint32_t(gslot) * 16u;
    dst = part * BM * 64 + rb * 1024;
  };
  // Weight-side offsets.  The range check of a buffer load covers the
  // uniform soffset too, so column block nt's distance 16 nt rows rides in
  // soffset and columns past N read zeros (they are computed and never
  // stored).  This lane's 8 codes of k-step ks are k 16 c4 + 8 ks (GS = 64:
  // both k-steps in one load; chunk pairs: see load_pair) or 32 ks + 8 c4
  // (GS = 32: one load per k-step).
  const uint32_t ncol = uint32_t(n0 + WCOLS * slice + l16);     // column of block 0
  const uint32_t woff = ncol * uint32_t(wrow_bytes) + (GS == 64 ? 2 * BITS * c4 : BITS * c4);
  // (PAIR) lane (l16, c4) loads codes k 32 c4 .. 32 c4 + 31 of the pair
  const uint32_t woffp = ncol * uint32_t(wrow_bytes) + 16u * uint32_t(c4);
  const uint32_t wstep = 16u * uint32_t(wrow_bytes);            // between column blocks
  const uint32_t sstep = 16u * uint32_t(G) * 2u;
  // a chunk's scales are one load: lane (c4, l16) fetches those of column
  // block c4; every lane then picks its four from lanes 16 nt + l16
  const uint32_t soff_lane = (ncol + 16u * uint32_t(c4)) * uint32_t(G) * 2u;
  // x fragment of k-step ks: row 16 mt + l16, piece 2 c4 + ks (GS = 64) or
  // 4 ks + c4 (GS = 32), swizzled as the copies placed it; the piece of k-step
  // 1 differs from k-step 0's in one bit
  // (PAIR: after the exchange below, k-step 0 of quarter c4 holds the k of
  // piece 0, 4, 1, 5 and k-step 1 those of piece 2, 6, 3, 7)
  const int piece0 = GS == 64 ? (PAIR ? ((c4 >> 1) | ((c4 & 1) << 2)) : 2 * c4) : c4;
  const uint32_t aoff0 = uint32_t(l16 * 128 + 16 * (piece0 ^ (l16 & 7) ^ ((l16 >> 3) & 1)));
  auto aoff = [&](int ks) {
    return ks == 0 ? aoff0 : aoff0 ^ (GS == 64 ? (PAIR ? 32u : 16u) : 64u);
  };

  // ---- loads --------------------------------------------------------------------
  auto issue_x = [&](__amdgpu_buffer_rsrc_t r, unsigned char* stage, int chunk) {
#pragma unroll
    for (int j = 0; j < C::XDMA; ++j)
      dma16(r, stage + (j * NW + wave) * 1024, xoff[j], uint32_t(chunk) * (BK * 2));
  };
  auto issue_sums = [&](int w) {
#pragma unroll
    for (int j = 0; j < C::SDMA; ++j) {
      uint32_t voff;
      int dst;
      sum_copy(j, voff, dst);
      dma16(sumr, sums + dst, voff, uint32_t(w) * WIN * 2);
    }
  };
  auto load_codes = [&](__amdgpu_buffer_rsrc_t wr, int chunk, uint32_t (&dst)[NT][CW]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int so = uni(uint32_t(chunk) * (BK * BITS / 8) + uint32_t(nt) * wstep);
      if constexpr (BITS == 4 && GS == 64) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, woff, so, 0);
        dst[nt][0] = v[0];
        dst[nt][1] = v[1];
      } else if constexpr (BITS == 4) {
        dst[nt][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff, so, 0);
        dst[nt][1] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff + 16u, so, 0);
      } else if constexpr (GS == 64) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, so, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[nt][i] = v[i];
      } else {
        const u32x2 v0 = __builtin_amdgcn_raw_buffer_load_b64(wr, woff, so, 0);
        const u32x2 v1 = __builtin_amdgcn_raw_buffer_load_b64(wr, woff + 32u, so, 0);
        dst[nt][0] = v0[0];
        dst[nt][1] = v0[1];
        dst[nt][2] = v1[0];
        dst[nt][3] = v1[1];
      }
    }
  };
  // (PAIR) the codes of chunks `chunk` and `chunk` + 1 of every column block:
  // dword i of lane (l16, c4) holds k 32 c4 + 8 i .. + 7 of the pair, so
  // lanes 0-31 hold the first chunk's codes and lanes 32-63 the second's
  auto load_pair = [&](__amdgpu_buffer_rsrc_t wr, int chunk, u32x4 (&dst)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      dst[nt] = __builtin_amdgcn_raw_buffer_load_b128(
          wr, woffp, uni(uint32_t(chunk) * (BK * BITS / 8) + uint32_t(nt) * wstep), 0);
  };
  // (PAIR) after a pair has landed: swap lanes 32-63 of dwords 0 and 2 with
  // lanes 0-31 of dwords 1 and 3, so that dwords 0 and 2 hold the first
  // chunk's codes (k-steps 0 and 1) on all 64 lanes and dwords 1 and 3 the
  // second's.  Quarter c4 of k-step 0 then holds the 8 k of the chunk's
  // piece 0, 4, 1 or 5, of k-step 1 those of piece 2, 6, 3 or 7.
  auto exchange = [&](u32x4 (&p)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto r = __builtin_amdgcn_permlane32_swap(p[nt][2 * h], p[nt][2 * h + 1], false, false);
        p[nt][2 * h] = r[0];
        p[nt][2 * h + 1] = r[1];
      }
  };
  // one load instruction per chunk (the chunk's GPC scales are adjacent)
  auto load_scales = [&](__amdgpu_buffer_rsrc_t sr, int chunk, uint32_t (&dst)[GPC]) {
    // lane (c4, l16) loads column block c4's scales
    if constexpr (GPC == 1) {
      dst[0] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff_lane, uni(chunk * 2), 0);
    } else {
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(sr, soff_lane, uni(chunk * 4), 0);
      dst[0] = v & 0xFFFFu;
      dst[1] = v >> 16;
    }
  };
  // bias and scale bf16 of the 8 groups w*WIN + 8*c4 .. +7 of this lane's
  // column, zero beyond the last group
  auto load_window = [&](int w, u32x4 (&bw)[NT], u32x4 (&sw)[NT]) {
    const int fl = fresh_lane(), c4 = fl >> 4;
    const uint32_t ncol = uint32_t(n0 + WCOLS * slice + (fl & 15));
    const int g0 = w * WIN + 8 * c4;
    if ((G % 8) == 0) {
      // a lane's 8 groups are all in range or all past the last one (a
      // partial last window): those read zeros through an offset outside
      // the descriptor
      const uint32_t o = g0 < G ? ncol * uint32_t(G) * 2u + 16u * c4 : kNoRow;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int so = uni(uint32_t(w) * WIN * 2u + uint32_t(nt) * sstep);
        bw[nt] = __builtin_amdgcn_raw_buffer_load_b128(br, o, so, 0);
        sw[nt] = OFFSET ? __builtin_amdgcn_raw_buffer_load_b128(sr, o, so, 0) : u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t bb[8], ss[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool in = g0 + i < G;
          const uint32_t o = (ncol + 16u * uint32_t(nt)) * uint32_t(G) * 2u +
                             uint32_t(in ? g0 + i : 0) * 2u;
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

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t dmask = 0, dbase = 0;
  if constexpr (BITS == 4) {
    asm("s_mov_b32 %0, 0x00780078" : "=s"(dmask));
    asm("v_mov_b32 %0, 0x41804180" : "=v"(dbase));
  }
  // window correction: acc += sum_g X_g * b_g  (- 16 * X_g * s_g for 4-bit),
  // X in three exact bf16 parts from LDS, as MFMAs over the window's groups
  auto correct = [&](const u32x4 (&bw)[NT], const u32x4 (&sw)[NT]) {
    u32x4 bneg[NT];
    if constexpr (OFFSET) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = -16.0f * bf16lo(sw[nt][i]);      // exact: a power-of-two scaling
          const float hi = -16.0f * bf16hi(sw[nt][i]);
          bneg[nt][i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        }
    }
    const int fl = fresh_lane(), fl16 = fl & 15;
    const uint32_t sum_off = uint32_t(fl16 * 64 + 16 * ((fl >> 4) ^ ((fl16 >> 1) & 3)));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 xp[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        xp[p] = *reinterpret_cast<const u32x4*>(sums + p * BM * 64 + mt * 1024 + sum_off);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int p = 0; p < 3; ++p) acc[mt][nt] = mfma(xp[p], bw[nt], acc[mt][nt]);
        if constexpr (OFFSET) {
#pragma unroll
          for (int p = 0; p < 3; ++p) acc[mt][nt] = mfma(xp[p], bneg[nt], acc[mt][nt]);
        }
      }
    }
  };

  // main product of one chunk: per group and row block, P = x . (off + q) by
  // MFMA, then acc += s * P (bias and offset terms come from the correction)
  auto decode = [&](const uint32_t (&cw)[NT][CW], u32x4 (&bfrag)[KS][NT]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (BITS == 4) bfrag[ks][nt] = decode4(cw[nt][ks], dmask, dbase);
        else bfrag[ks][nt] = decode8(cw[nt][2 * ks], cw[nt][2 * ks + 1]);
      }
  };
  auto mma = [&](const unsigned char* xs, const u32x4 (&bfrag)[KS][NT], const float (&s)[GPC][NT]) {
#pragma unroll
    for (int gl = 0; gl < GPC; ++gl) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 P[NT];
#pragma unroll
        for (int ksg = 0; ksg < KSG; ++ksg) {
          const int ks = gl * KSG + ksg;
          const u32x4 afrag = *reinterpret_cast<const u32x4*>(xs + mt * 2048 + aoff(ks));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            P[nt] = mfma(afrag, bfrag[ks][nt], ksg == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(s[gl][nt], P[nt][i], acc[mt][nt][i]);
      }
    }
  };

  // chunks of this tile (relative to c0) and the window of chunk c0
  const int nchunks = c1 - c0;
  const int w0 = c0 / CPW;
  // Software pipeline (4-bit codes, 64-wide groups).  In-order issue means
  // that an FMA waiting on an MFMA result holds up the MFMAs behind it, so
  // the products P of row block mt are scaled into acc while the MFMAs of
  // row block mt + 1 run (two FMAs after each MFMA), and those of a chunk's
  // last row block during the first row block of the next chunk.  Pp and sp
  // carry them; sched_barrier pins the order.
  constexpr bool PIPE = BITS == 4 && GS == 64;
  f32x4 Pp[NT];
  float sp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { Pp[nt] = f32x4{0.f, 0.f, 0.f, 0.f}; sp[nt] = 0.f; }
  // codes and scales of even (0) and odd (1) chunks; a buffer is refilled
  // with chunk c + 2 as soon as chunk c has been decoded
  uint32_t cb0[NT][CW], cb1[NT][CW];
  uint32_t sb0[GPC], sb1[GPC];
  // (PAIR) chunk pairs: pa holds chunks 4 i, 4 i + 1, pb chunks 4 i + 2, 4 i + 3
  u32x4 pa[NT], pb[NT];
  // loads of chunks past the end go through an empty descriptor: they read
  // nothing, return zeros, and keep the number of loads per chunk fixed
  const __amdgpu_buffer_rsrc_t none = rsrc(a.x, 0u);

  // ---- prologue: window 0's corrections, chunks 0 and 1 in flight -------------
  {
    u32x4 bw[NT], sw[NT];
    issue_sums(w0);
    load_window(w0, bw, sw);
    // the row-sum copies must stay ahead of the x copies: the wait below
    // counts only the chunk loads issued after them
    __builtin_amdgcn_sched_barrier(0);
    issue_x(xr, xs0, c0);
    if constexpr (PAIR) load_pair(wr, c0, pa);
    else load_codes(wr, c0, cb0);
    load_scales(sr, c0, sb0);
    const bool one = nchunks > 1;
    issue_x(one ? xr : none, xs1, c0 + 1);
    if constexpr (!PAIR) load_codes(one ? wr : none, c0 + 1, cb1);
    load_scales(one ? sr : none, c0 + 1, sb1);
    // keep the corrections' arithmetic behind the chunk loads
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem<PAIR ? PER + PER_ODD : 2 * PER>();
    __builtin_amdgcn_s_barrier();
    correct(bw, sw);
  }

  // one chunk: x stage `cur` holds chunk c; the copy of chunk c + 2 goes to
  // stage `nxt`, whose chunk c - 1 every wave has finished reading once it
  // passes this chunk's barrier.
  // (PAIR: pc holds the chunk's pair, pn is the buffer the pair two chunks
  // ahead goes to; `odd` says which chunk of its pair this is)
  auto chunk = [&](int c, unsigned char* cur, unsigned char* nxt, uint32_t (&cw)[NT][CW],
                   uint32_t (&sv)[GPC], u32x4 (&pc)[NT], u32x4 (&pn)[NT], auto odd) {
    constexpr bool ODD = decltype(odd)::value;
    // chunks are scheduled one at a time: letting the scheduler interleave
    // neighbouring chunks costs more registers than two waves per SIMD allow
    __builtin_amdgcn_sched_barrier(0);
    if (c > 0 && c % CPW == 0) {
      // this window's row-sum parts arrived a window ago; its biases and
      // scales are fetched now, while no chunk holds registers
      u32x4 wb[NT], ws[NT];
      load_window(w0 + c / CPW, wb, ws);
      if constexpr (PIPE) {
        // the pending scale FMAs first: their registers are then free for
        // the correction
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[MT - 1][nt][i] = fmaf(sp[nt], Pp[nt][i], acc[MT - 1][nt][i]);
          Pp[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          sp[nt] = 0.f;
        }
      }
      correct(wb, ws);
    }
    // this chunk's x copies, codes and scales were issued two chunks ago (a
    // pair's codes three for its odd chunk): at most the previous chunk's
    // loads may still be in flight
    wait_vmem<!PAIR ? PER : (ODD ? PER : PER_ODD)>();
    wait_lds();
    __builtin_amdgcn_s_barrier();
    const int cn = c + 2;
    const bool pre = cn < nchunks;
    issue_x(pre ? xr : none, nxt, c0 + cn);
    if (c % CPW == 0 && c + CPW < nchunks) issue_sums(w0 + c / CPW + 1);
    if constexpr (PAIR) {
      // this chunk's two code words per column block
      if constexpr (!ODD) exchange(pc);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        cw[nt][0] = pc[nt][ODD ? 1 : 0];
        cw[nt][1] = pc[nt][ODD ? 3 : 2];
      }
    }
    u32x4 bfrag[KS][NT];
    float s[GPC][NT];
#pragma unroll
    for (int gl = 0; gl < GPC; ++gl) {
      const int sf = int(sv[gl] << 16);          // bf16 -> fp32 bits
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        s[gl][nt] = __int_as_float(__builtin_amdgcn_ds_bpermute((16 * nt + l16) * 4, sf));
    }
    if constexpr (PIPE) {
      // x fragments are read one row block ahead; row block 0 decodes each
      // B fragment one MFMA before its first use and then queues the code
      // and scale loads of chunk c + 2
      u32x4 af[2][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[0][ks] = *reinterpret_cast<const u32x4*>(cur + aoff(ks));
      bfrag[0][0] = decode4(cw[0][0], dmask, dbase);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + 1 < MT) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            af[(mt + 1) & 1][ks] = *reinterpret_cast<const u32x4*>(cur + (mt + 1) * 2048 + aoff(ks));
        }
        f32x4 Pc[NT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int j = ks * NT + nt;
            Pc[nt] = mfma(af[mt & 1][ks], bfrag[ks][nt], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Pc[nt]);
            if (mt == 0) {
              if (j + 1 < KS * NT)
                bfrag[(j + 1) / NT][(j + 1) % NT] = decode4(cw[(j + 1) % NT][(j + 1) / NT], dmask, dbase);
              if (j + 1 == KS * NT) {
                if constexpr (PAIR) {
                  if constexpr (!ODD) load_pair(pre ? wr : none, c0 + cn, pn);
                } else {
                  load_codes(pre ? wr : none, c0 + cn, cw);
                }
                load_scales(pre ? sr : none, c0 + cn, sv);
              }
            }
            // two of the 4 NT pending scale FMAs of the previous row block
            const int pm = mt == 0 ? MT - 1 : mt - 1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int e = 2 * j + h, pn = e / 4, pi = e % 4;
              acc[pm][pn][pi] = fmaf(sp[pn], Pp[pn][pi], acc[pm][pn][pi]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) { Pp[nt] = Pc[nt]; sp[nt] = s[0][nt]; }
      }
    } else {
      decode(cw, bfrag);
      load_codes(pre ? wr : none, c0 + cn, cw);
      load_scales(pre ? sr : none, c0 + cn, sv);
      mma(cur, bfrag, s);
    }
  };

  // x stages rotate with period 3, code buffers with period 2 (chunk pairs:
  // pair buffers with period 4, so 12 chunks a turn).  Leaving the
  // loop right after the last chunk (rather than skipping the rest of a
  // period) means no path reaches the back edge with a chunk left out, so
  // the compiler's count of loads in flight is the same on every path.
  using Ev = std::false_type;
  using Od = std::true_type;
  if constexpr (PAIR) {
    // pair buffers rotate with period 4: the loop holds 12 chunks
    for (int c = 0;; c += 12) {
      chunk(c, xs0, xs2, cb0, sb0, pa, pb, Ev{});
      if (c + 1 >= nchunks) break;
      chunk(c + 1, xs1, xs0, cb1, sb1, pa, pb, Od{});
      if (c + 2 >= nchunks) break;
      chunk(c + 2, xs2, xs1, cb0, sb0, pb, pa, Ev{});
      if (c + 3 >= nchunks) break;
      chunk(c + 3, xs0, xs2, cb1, sb1, pb, pa, Od{});
      if (c + 4 >= nchunks) break;
      chunk(c + 4, xs1, xs0, cb0, sb0, pa, pb, Ev{});
      if (c + 5 >= nchunks) break;
      chunk(c + 5, xs2, xs1, cb1, sb1, pa, pb, Od{});
      if (c + 6 >= nchunks) break;
      chunk(c + 6, xs0, xs2, cb0, sb0, pb, pa, Ev{});
      if (c + 7 >= nchunks) break;
      chunk(c + 7, xs1, xs0, cb1, sb1, pb, pa, Od{});
      if (c + 8 >= nchunks) break;
      chunk(c + 8, xs2, xs1, cb0, sb0, pa, pb, Ev{});
      if (c + 9 >= nchunks) break;
      chunk(c + 9, xs0, xs2, cb1, sb1, pa, pb, Od{});
      if (c + 10 >= nchunks) break;
      chunk(c + 10, xs1, xs0, cb0, sb0, pb, pa, Ev{});
      if (c + 11 >= nchunks) break;
      chunk(c + 11, xs2, xs1, cb1, sb1, pb, pa, Od{});
      if (c + 12 >= nchunks) break;
    }
  } else {
    for (int c = 0;; c += 6) {
      chunk(c, xs0, xs2, cb0, sb0, pa, pb, Ev{});
      if (c + 1 >= nchunks) break;
      chunk(c + 1, xs1, xs0, cb1, sb1, pa, pb, Od{});
      if (c + 2 >= nchunks) break;
      chunk(c + 2, xs2, xs1, cb0, sb0, pa, pb, Ev{});
      if (c + 3 >= nchunks) break;
      chunk(c + 3, xs0, xs2, cb1, sb1, pa, pb, Od{});
      if (c + 4 >= nchunks) break;
      chunk(c + 4, xs1, xs0, cb0, sb0, pa, pb, Ev{});
      if (c + 5 >= nchunks) break;
      chunk(c + 5, xs2, xs1, cb1, sb1, pa, pb, Od{});
      if (c + 6 >= nchunks) break;
    }
  }

  if constexpr (PIPE) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[MT - 1][nt][i] = fmaf(sp[nt], Pp[nt][i], acc[MT - 1][nt][i]);
  }
  // ---- store: fp32 -> bf16 through a per-wave LDS patch, then row segments ------
  // the patches reuse the x stages: the repeated copies of the last chunk
  // must have landed first
  wait_vmem<0>();
  wait_lds();
  __syncthreads();
  constexpr int PPS = C::PATCH_PER_STAGE;
  unsigned char* patch_base = wave < PPS ? xs0 : (wave < 2 * PPS ? xs1 : xs2);
  uint16_t* patch = reinterpret_cast<uint16_t*>(patch_base + (wave % PPS) * 2048);
  const bool vec_ok = (N % 8) == 0;
  const int lane_s = fresh_lane(), l16s = lane_s & 15, c4s = lane_s >> 4;
  if constexpr (GLU) {
    // Gate wave j and up wave HW + j hold the same outputs (lane (l16, c4)
    // of both holds the same rows and columns).  Per row block each hands the
    // other half of its fp32 results through LDS: the gate wave forms
    // h = act(gate) * up (act 1 = SiLU, 2 = GELU with the exact erf) for the
    // first 32 columns, the up wave for the last 32, each into a patch of its
    // own in xs2, and each stores its half's row segments.  Exchange space:
    // stage j (xs0 or xs1), or both for a single pair; two row blocks'
    // worth where the stage holds them, so that one barrier per row block
    // suffices.
    static_assert(NT == 4 && HW <= 2 && C::STAGE >= HW * 2048, "exchange and patch space");
    constexpr int XB = HW == 1 ? 2 * C::STAGE : C::STAGE;        // exchange bytes per pair
    constexpr int NB = XB >= 8192 ? 2 : 1;                        // row blocks in flight
    unsigned char* const xbase = HW == 1 ? xs0 : (slice == 0 ? xs0 : xs1);
    uint16_t* const hpatch = reinterpret_cast<uint16_t*>(xs2 + slice * 2048 + (upw ? 1024 : 0));
    const bool gelu = a.act == 2;
    auto glu = [&](float g, float u) {
      const float act = gelu ? 0.5f * g * (1.0f + erff(g * 0.70710678118654752f))
                             : g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      return act * u;
    };
    // the gate wave keeps column blocks 0, 1 and sends 2, 3; the up wave the
    // reverse.  One body per role, with constant indices into acc (a select
    // or a runtime index would hold copies of it, or put it in scratch).
    auto epilogue = [&](auto role) {
      constexpr bool UP = decltype(role)::value;
      constexpr int keep0 = UP ? 2 : 0, send0 = UP ? 0 : 2;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // [2 blocks][4][64 lanes] floats each way; the up wave's outbox is the
        // first 2 KiB (single pair: xs0, the gate wave's is xs1)
        unsigned char* const xb = xbase + (NB == 2 ? (mt & 1) * 4096 : 0);
        float* const up_out = reinterpret_cast<float*>(xb);
        float* const gate_out = reinterpret_cast<float*>(HW == 1 ? xs1 + (xb - xs0) : xb + 2048);
        float* const outbox = UP ? up_out : gate_out;
        const float* const inbox = UP ? gate_out : up_out;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) outbox[(j * 4 + i) * 64 + lane_s] = acc[mt][send0 + j][i];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float mine = acc[mt][keep0 + j][i], theirs = inbox[(j * 4 + i) * 64 + lane_s];
            const int r = 4 * c4s + i, col = 16 * j + l16s;
            hpatch[r * 32 + (((col >> 3) ^ (r & 3)) << 3) + (col & 7)] = __builtin_bit_cast(
                uint16_t, static_cast<__bf16>(UP ? glu(theirs, mine) : glu(mine, theirs)));
          }
        // [16 rows][32 columns]: one 16-byte segment per lane
        {
          const int r = lane_s >> 2, cs = lane_s & 3;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&hpatch[r * 32 + ((cs ^ (r & 3)) << 3)]);
          const int tr = mt * 16 + r;
          const int col = n0 + WCOLS * slice + 16 * keep0 + 8 * cs;
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
        // a buffer is written again two row blocks on (NB = 2), after the next
        // row block's barrier; with one buffer every read must end first
        if constexpr (NB == 1) __syncthreads();
      }
    };
    if (upw) epilogue(std::true_type{});
    else epilogue(std::false_type{});
    return;
  }
  if constexpr (MT <= kPieceMT) {
    if (part) {
      // a piece of a split tail tile: its fp32 sums as [wave][row block]
      // [column block][element][lane] (256 bytes per store instruction; one
      // element at a time, as storing whole f32x4 accumulators ties them to
      // register quadruples through the K loop and spills); rows past `rows`
      // hold the products of zero x rows and are never read
      float* const blk = part + size_t(wave) * (kPieceMT * NT * 256);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) blk[((mt * NT + nt) * 4 + i) * 64 + lane_s] = acc[mt][nt][i];
      return;
    }
  }
  {
  const int lane = lane_s, l16 = l16s, c4 = c4s;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // [16 rows][64 columns], 16-byte slots swizzled by row
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
      const int col = n0 + WCOLS * slice + 8 * cs;
      if (cs < 2 * NT && tr < rows && col < N) {
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
}


// ---- tiles ----------------------------------------------------------------------
// Tile heights follow each expert's measured rows (ml-explore/mlx PR 4023,
// opening paragraphs: a block taller than the run computes rows that are
// thrown away).  A segment of r rows is cut into tiles of BM rows; where its
// last r % BM rows number at most h = BM / 2 (BM >= 64) they may instead form
// a tail tile, run by the shortest body that holds them (32 rows with four
// 16-column blocks per wave, or 64).  The routing launch writes three prefix
// tables over the experts: tiles[e] (ceil(r / BM)), tiles[E+1 + e]
// (floor(r / BM) + [r % BM > h]) and tiles[2(E+1) + e] (0 < r % BM <= h).
//
// Tail tiles go after every full tile ("mixed") when the full tiles fit in
// one round of resident workgroups (two per CU) and the segments' last tiles
// would spill into a second: that round is then made of short tiles only.
// Where the full tiles take several rounds anyway, keeping each segment's
// last tile among its others measured faster (a Mixtral-shaped up projection:
// 571 us against 587 us).  In a mixed launch with K of two correction windows
// or more (and no GLU store), each tail tile is cut along K into `pieces` of
// whole windows: a lone short tile runs its K loop with one wave per SIMD,
// and a Mixtral-shaped down projection (K = 14336) spent 151 of 658 us on its
// tail round.  The pieces' fp32 sums go to a.part, and tail_reduce_kernel
// adds them in piece order and stores the bf16 result.
// a.mixed: 0 never, 1 by the rule above, 2 always.  Every workgroup of both
// kernels reads the same counts, so all take the same decisions.
struct TileCounts {
  const int32_t* ftab;   // prefix of full-height tiles per expert (routed)
  const int32_t* ptab;   // prefix of tail tiles per expert (routed)
  int nfull, npart;      // full-height and tail tiles (per column tile)
  int pieces;            // pieces per tail tile (1: not split)
};

// pieces per tail tile: windows of K shared out as evenly as the slots of
// a.part allow, at most kMaxTailPieces
__device__ inline int tail_pieces(const GemmArgs& a, int npart, int ntn) {
  const int nwin = (a.K / a.group_size + WIN - 1) / WIN;
  if (npart <= 0 || nwin < 2 || !a.part) return 1;
  const int64_t tiles = int64_t(npart) * ntn;
  const int s = int(min64(min64(kMaxTailPieces, nwin), a.part_pieces / tiles));
  if (s < 2) return 1;
  const int wpp = (nwin + s - 1) / s;              // windows per piece
  return (nwin + wpp - 1) / wpp;
}

template <int BM>
__device__ inline TileCounts tile_counts(const GemmArgs& a, int ntn, bool splittable) {
  constexpr int TAIL = BM >= 64 ? BM / 2 : 0;      // the routing's h
  const int E = a.E;
  const int64_t nrows = a.n_pairs * a.M;
  TileCounts t{};
  int64_t uniform, full;                           // tiles of BM rows without / with tails
  if (a.perm) {
    uniform = min64(a.tiles[E], a.max_full);
    full = min64(a.tiles[(E + 1) + E], a.max_full);
  } else {
    const int64_t rest = nrows % BM;
    uniform = min64((nrows + BM - 1) / BM, a.max_full);
    full = min64(nrows / BM + (rest > TAIL ? 1 : 0), a.max_full);
  }
  const int64_t round = 2 * kComputeUnits;
  const bool mixed = a.mixed == 2 || (a.mixed == 1 && full * ntn <= round && uniform * ntn > round);
  if (a.perm) {
    t.ftab = mixed ? a.tiles + (E + 1) : a.tiles;
    t.ptab = a.tiles + 2 * (E + 1);
    t.nfull = int(min64(t.ftab[E], a.max_full));
    t.npart = mixed ? int(min64(t.ptab[E], a.max_part)) : 0;
  } else {
    const int64_t rest = nrows % BM;
    const bool short_tail = mixed && rest > 0 && rest <= TAIL;
    t.nfull = int(min64(nrows / BM + (rest > 0 && !short_tail ? 1 : 0), a.max_full));
    t.npart = short_tail ? 1 : 0;
  }
  t.pieces = splittable && mixed ? tail_pieces(a, t.npart, ntn) : 1;
  return t;
}

struct TileCoords {
  int e;           // expert
  int64_t row0;    // first row (in routed order)
  int rows;        // rows of the tile (<= 0: none)
  int n0;          // first output column
};

// Tile `logical` of the full-height tiles (tail = false) or of the tail
// tiles: column tiles in groups of a.col_group (0: all); within a group
// column tiles fastest, then row tiles, so that the workgroups resident
// together on an XCD share both their x chunks and their weight chunks in L2.
// (With all of a row tile's column tiles first, a Mixtral-shaped up
// projection, 56 column tiles per row tile, fetched 6x its algorithmic bytes
// from beyond L2: each expert's slab once per row tile.)  Called by whole
// waves (the expert search is a ballot over 64 lanes).
__device__ inline TileCoords tile_coords(const GemmArgs& a, const TileCounts& tc,
                                         unsigned logical, bool tail, int ntn, int BN, int BM,
                                         int lane) {
  const int E = a.E;
  const int64_t nrows = a.n_pairs * a.M;
  const unsigned rows_here = tail ? unsigned(tc.npart) : unsigned(tc.nfull);
  const unsigned gcw = a.col_group > 0 ? min(unsigned(a.col_group), unsigned(ntn)) : unsigned(ntn);
  const unsigned cg = logical / (gcw * rows_here), rem = logical % (gcw * rows_here);
  const unsigned w = min(gcw, unsigned(ntn) - cg * gcw);
  const int t = int(rem / w);
  TileCoords c;
  c.n0 = int(cg * gcw + rem % w) * BN;
  c.e = 0;
  int64_t seg_beg, seg_end;
  if (a.perm) {
    // expert of tile t: the largest e with tab[e] <= t (tab is
    // non-decreasing, tab[0] = 0).  Two rounds of 64 lanes: coarse entries
    // every `step`, then the step between two of them.
    const int32_t* const tab = tail ? tc.ptab : tc.ftab;
    const int step = (E + 64) / 64;                   // E + 1 entries <= 64 * step
    const int i1 = min(lane * step, E);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(tab[i1] <= t);
    const int lo = (63 - __builtin_clzll(m1 | 1u)) * step;
    const int i2 = min(lo + lane, E);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < step && tab[i2] <= t);
    int e = min(lo + (63 - __builtin_clzll(m2 | 1u)), E - 1);
    e = __builtin_amdgcn_readfirstlane(e);
    c.e = e;
    // offsets come from the routing kernels; clamping them to [0, n] keeps
    // every access in bounds even if they were corrupted
    seg_beg = min64(max64(int64_t(a.offsets[e]) * a.M, 0), nrows);
    seg_end = min64(max64(int64_t(a.offsets[e + 1]) * a.M, 0), nrows);
    c.row0 = tail ? seg_beg : min64(seg_beg + int64_t(t - tab[e]) * BM, nrows);
  } else {
    seg_beg = 0;
    seg_end = nrows;
    c.row0 = tail ? 0 : int64_t(t) * BM;
  }
  if (tail) c.row0 += (max64(seg_end - seg_beg, 0) / BM) * BM;   // the last len % BM rows
  c.rows = c.row0 >= seg_end ? 0 : int(min64(BM, seg_end - c.row0));
  return c;
}

// Output row of routed row j: pair perm[j / M], row j % M of it (the dense
// product: j itself).
__device__ inline int32_t out_row(const GemmArgs& a, int64_t j) {
  if (!a.perm) return int32_t(j);
  const int32_t pair = int32_t(min64(max<int32_t>(a.perm[j / a.M], 0), a.n_pairs - 1));
  return pair * a.M + int32_t(j % a.M);
}

template <int BM, int BITS, int GS, int NW, bool GLU, int NT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(waves_per_simd<BM>())))
void gather_gemm_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(NT == 4 || (NT == 3 && !GLU), "column blocks per wave");
  using C = Cfg<BM, NW>;
  constexpr int BN = 16 * NT * (GLU ? NW / 2 : NW);   // output columns per tile
  // codes of two chunks per load in every body of a 4-wave launch (gemm_tile)
  constexpr bool PAIRS = NW == 4;

  __shared__ __attribute__((aligned(16))) unsigned char xs0[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs1[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs2[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char sums[C::SUMS];
  __shared__ int32_t xrow_tab[BM];
  __shared__ int32_t orow_tab[BM];

  const int lane = threadIdx.x & 63;

  // ---- which tile (tile_counts, tile_coords) ------------------------------------
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin
  // (blockIdx % 8).  The full-height tiles that exist (the routed count, not
  // the grid's upper bound) are cut into 8 contiguous ranges, one per XCD, so
  // that a row tile's gathered x rows and an expert's weight slab stay in one
  // L2; the tail tiles (or their pieces) follow the same way, after every
  // XCD's full tiles, so the short ones fill in at the end.  Surplus
  // workgroups exit at once.
  const int ntn = (a.N + BN - 1) / BN;
  // a tile table built for another tile height (a workspace routed under a
  // different plan) is not used: nothing is written
  if (a.perm && *a.tile_bm != BM) return;
  const TileCounts tc = tile_counts<BM>(a, ntn, !GLU);
  const int nfull = tc.nfull, npart = tc.npart, S = tc.pieces;
  const unsigned nb = unsigned(nfull) * unsigned(ntn);
  const unsigned ns = unsigned(npart) * unsigned(ntn) * unsigned(S);
  const unsigned pb = (nb + 7u) / 8u, ps = (ns + 7u) / 8u;
  const unsigned xcd = blockIdx.x % 8u, j = blockIdx.x / 8u;
  bool tail;
  unsigned logical;
  if (j < pb) {
    logical = xcd * pb + j;
    if (logical >= nb) return;
    tail = false;
  } else {
    if (j - pb >= ps) return;
    logical = xcd * ps + (j - pb);
    if (logical >= ns) return;
    tail = true;
  }
  // a split tail tile's pieces are adjacent: piece s of tail tile logical / S
  const unsigned slot = logical;
  const int piece = tail ? int(logical % unsigned(S)) : 0;
  if (tail) logical /= unsigned(S);
  const TileCoords tco = tile_coords(a, tc, logical, tail, ntn, BN, BM, lane);
  if (tco.rows <= 0) return;
  const int e = tco.e, rows = tco.rows, n0 = tco.n0;
  const int64_t row0 = tco.row0;
  // K range: the whole of K, or piece `piece`'s windows
  const int nch = a.K / BK;
  int c0 = 0, c1 = nch;
  float* part = nullptr;
  if constexpr (BM >= 64 && !GLU) {                // (no tail tiles below 64 rows)
    if (tail && S > 1) {
      constexpr int CPW = WIN * GS / BK;           // chunks per correction window
      const int nwin = (a.K / GS + WIN - 1) / WIN;
      const int wpp = (nwin + S - 1) / S;
      c0 = piece * wpp * CPW;
      c1 = min(c0 + wpp * CPW, nch);
      part = a.part + size_t(slot) * kPieceFloats;
    }
  }

  // the tail's body: the shortest that holds its rows (bodies of 32 rows for
  // four 16-column blocks per wave only)
  if constexpr (BM >= 64 && NW == 4 && NT == 4) {
    if (rows <= 32) {
      gemm_tile<32, BITS, GS, NW, GLU, NT, PAIRS>(a, e, row0, rows, n0, xs0, xs1, xs2, sums,
                                                  xrow_tab, orow_tab, c0, c1, part);
      return;
    }
  }
  if constexpr (BM == 128) {
    if (rows <= 64) {
      gemm_tile<64, BITS, GS, NW, GLU, NT, PAIRS>(a, e, row0, rows, n0, xs0, xs1, xs2, sums,
                                                  xrow_tab, orow_tab, c0, c1, part);
      return;
    }
  }
  // (a tail tile reaches this body only in 64-row launches with three
  // column blocks per wave: tiles of 16 or 32 rows have no tail tiles, and
  // a 128-row launch's tails have at most 64 rows)
  gemm_tile<BM, BITS, GS, NW, GLU, NT, PAIRS>(a, e, row0, rows, n0, xs0, xs1, xs2, sums,
                                              xrow_tab, orow_tab, c0, c1, BM == 64 ? part : nullptr);
}

// Grid: the upper bounds on full-height and tail tiles, each rounded up to a
// multiple of 8 for the XCD-aware numbering in the kernel.
// Whether a launch may split its tail tiles along K (the device decides from
// the routed counts): tail tiles possible, K of two correction windows or
// more, no GLU store, and slots for the pieces.
bool splits_tails(const GemmArgs& a) {
  return a.part && a.part_pieces > 0 && !a.glu && a.bm >= 64 && a.mixed != 0 && a.max_part > 0 &&
         a.K / a.group_size > WIN;
}

// Tail tiles may each be cut into up to min(kMaxTailPieces, windows of K)
// pieces, as many as the a.part_pieces slots of a.part hold.
int64_t gemm_blocks(const GemmArgs& a, int bn) {
  const int64_t ntn = ceil_div(a.N, bn);
  int64_t tails = a.max_part * ntn;
  if (splits_tails(a)) {
    const int64_t nwin = ceil_div(int64_t(a.K / a.group_size), int64_t(WIN));
    tails = std::max(tails, std::min(a.part_pieces, tails * std::min<int64_t>(kMaxTailPieces, nwin)));
  }
  return 8 * (ceil_div(a.max_full * ntn, 8) + ceil_div(tails, 8));
}

// Sums the pieces of every split tail tile in piece order and stores them as
// bf16.  A piece stored element i of column block nt of row block mt of
// GEMM wave w, lane l (row 16 mt + 4 (l / 16) + i, column
// n0 + 16 NT w + 16 nt + l % 16 of the tile) at [w][mt][nt][i][l] of its
// slot.  A workgroup takes (tail tile, row block, GEMM wave) items in turn
// (a grid of at most kReduceBlocks); thread q < 64 NT takes four
// neighbouring lanes of one (nt, i): 16-byte loads, four columns of one row,
// one 8-byte store.  Every piece's values are loaded before the first add
// (slots past the last piece load the last one again and are not added), so
// the loads of all pieces are in flight together.  The kernel takes the same
// decisions as the GEMM launch before it from the same tables and exits at
// once where that launch split nothing (the common case after a launch whose
// tails stayed in place: a few microseconds for a small grid).
template <int BM, int NT>
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs a) {
  constexpr int BN = 64 * NT;
  const int q = threadIdx.x;
  const int ntn = (a.N + BN - 1) / BN;
  if (a.perm && *a.tile_bm != BM) return;
  const TileCounts tc = tile_counts<BM>(a, ntn, true);
  const int S = tc.pieces;
  if (S < 2) return;
  const unsigned items = unsigned(tc.npart) * unsigned(ntn) * unsigned(kPieceMT * 4);
  for (unsigned b = blockIdx.x; b < items; b += gridDim.x) {
    const unsigned tl = b / (kPieceMT * 4);
    const int mt = int(b / 4 % kPieceMT), w = int(b % 4);
    // (whole waves call it: the expert search is a ballot)
    const TileCoords c = tile_coords(a, tc, tl, true, ntn, BN, BM, q & 63);
    if (16 * mt >= c.rows || q >= 64 * NT) continue;   // uniform per wave
    const int nt = q / 64, i = (q / 16) % 4;
    const int qi = q % 16;                            // lanes 4 qi .. 4 qi + 3
    const int c4 = qi / 4, l16 = 4 * (qi % 4);
    const int r = 16 * mt + 4 * c4 + i;
    const float* const src = a.part + size_t(tl) * S * kPieceFloats +
                             size_t(w) * (kPieceMT * NT * 256) + size_t(mt) * NT * 256 +
                             size_t((nt * 4 + i) * 64 + 4 * qi);
    f32x4 v[kMaxTailPieces];
#pragma unroll
    for (int p = 0; p < kMaxTailPieces; ++p)
      v[p] = *reinterpret_cast<const f32x4*>(src + size_t(min(p, S - 1)) * kPieceFloats);
    f32x4 sum = v[0];
#pragma unroll
    for (int p = 1; p < kMaxTailPieces; ++p)
      if (p < S) sum += v[p];
    if (r < c.rows) {
      const int col = c.n0 + 16 * NT * w + 16 * nt + l16;
      uint16_t* const dst = a.out + int64_t(out_row(a, c.row0 + r)) * a.N + col;
      uint16_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum[k]));
      if (col + 3 < a.N && (a.N % 4) == 0) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                               uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (col + k < a.N) dst[k] = h[k];
      }
    }
  }
}

// the reduce after a GEMM launch that may have split its tail tiles
template <int BM, int NT>
hipError_t launch_tail_reduce(const GemmArgs& a, hipStream_t s) {
  if constexpr (BM >= 64) {
    if (!splits_tails(a)) return hipSuccess;
    const int64_t blocks = std::min<int64_t>(a.max_part * ceil_div(a.N, 64 * NT) * kPieceMT * 4,
                                             kReduceBlocks);
    if (blocks <= 0) return hipSuccess;
    note_dispatch("tail_reduce", {BM, NT});
    tail_reduce_kernel<BM, NT><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int BM, int BITS, int NW, bool GLU, int NT>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BN = 16 * NT * (GLU ? NW / 2 : NW);    // output columns per tile
  const int64_t blocks = gemm_blocks(a, BN);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  note_dispatch("gather_gemm", {BM, BITS, a.group_size == 32 ? 32 : 64, NW, GLU, NT});
  if (a.group_size == 32)
    gather_gemm_kernel<BM, BITS, 32, NW, GLU, NT><<<grid, dim3(64 * NW), 0, s>>>(a);
  else
    gather_gemm_kernel<BM, BITS, 64, NW, GLU, NT><<<grid, dim3(64 * NW), 0, s>>>(a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || GLU) return err;
  return launch_tail_reduce<BM, NT>(a, s);
}

// 128-, 64- and 32-row tiles are 4 waves wide (256 columns, or 192 with
// three column blocks per wave for 64- and 128-row tiles); 16-row tiles are
// 2 waves wide, so that one chunk of x is still one 16-byte copy per lane.
template <int BM>
hipError_t launch_bm(const GemmArgs& a, hipStream_t s) {
  constexpr int NW = BM == 16 ? 2 : 4;
  if (a.glu)
    return a.bits == 4 ? launch_cfg<BM, 4, NW, true, 4>(a, s) : launch_cfg<BM, 8, NW, true, 4>(a, s);
  if constexpr (BM >= 64) {
    // three column blocks per wave: 4-bit codes in groups of 64 only
    if (a.ntw == 3) {
      if (a.bits != 4 || a.group_size != 64) return hipErrorInvalidValue;
      const int64_t blocks = gemm_blocks(a, 48 * NW);
      if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
      note_dispatch("gather_gemm", {BM, 4, 64, NW, 0, 3});
      gather_gemm_kernel<BM, 4, 64, NW, false, 3><<<dim3(unsigned(blocks)), dim3(64 * NW), 0, s>>>(a);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      return launch_tail_reduce<BM, 3>(a, s);
    }
  }
  return a.bits == 4 ? launch_cfg<BM, 4, NW, false, 4>(a, s) : launch_cfg<BM, 8, NW, false, 4>(a, s);
}

}  // namespace

// Tiles of BM rows and 256 columns (four 16-column blocks per wave) or 192
// columns (three): the width whose tiles come closest to an even number of
// tiles per compute unit wins, weighing the narrower tile's lower reuse of
// each x fragment (three MFMAs per fragment read instead of four; measured
// 18 % slower per tile of equal work) against it.  The prefill shape's dense
// control (128 row tiles x 4 = 512 tiles, two per CU) takes 192 columns; its
// routed call (about 160 row tiles with the experts' partial ones) keeps 256.
int gemm_tile_cols(int64_t rows, int64_t N, int bm, int E, int bits, int group_size, bool glu) {
  if (glu || bm < 64 || N <= 0 || bits != 4 || group_size != 64) return 4;
  // full row tiles, plus each routed expert's last, partial one (about half
  // the experts end in one; it costs a whole tile)
  const int64_t row_tiles = ceil_div(rows, bm) + (E > 1 ? ceil_div(std::min<int64_t>(E, rows), 2) : 0);
  auto cost = [&](int nt) {
    const int64_t bn = 64 * nt;
    const int64_t per_cu = ceil_div(row_tiles * ceil_div(N, bn), kComputeUnits);
    return double(per_cu * bn) * (nt == 3 ? 1.18 : 1.0);
  };
  return cost(3) < cost(4) ? 3 : 4;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.max_full < 0 || a.max_part < 0 || (a.max_part > 0 && !a.mixed)) return hipErrorInvalidValue;
  if (a.part && a.part_pieces <= 0) return hipErrorInvalidValue;
  if (a.max_full + a.max_part <= 0 || a.N <= 0) return hipSuccess;
  if (a.ntw != 0 && a.ntw != 3 && a.ntw != 4) return hipErrorInvalidValue;
  switch (a.bm) {
    case 16: return launch_bm<16>(a, s);
    case 32: return launch_bm<32>(a, s);
    case 64: return launch_bm<64>(a, s);
    default: return launch_bm<128>(a, s);
  }
}

}  // namespace mq
