// Gathered grouped GEMM on MX expert weights, MXFP4 and MXFP8 (gfx950, bf16
// MFMA).
//
// What it computes: the pages name the microscaling fp modes next to the affine
// one (ml-explore/mlx pull 4023, the comment on block-height coverage; issue
// 4339, the maintainers' note on the CUDA backend) without defining them; the
// formats are read as OCP MX v1.0 MXFP4 (E2M1 codes, eight to a uint32 word
// along K, low nibble first) and MXFP8 (E4M3 codes, four to a word, low byte
// first), with one E8M0 exponent e per 32 weights, the weight being
// value(code) * 2^(e - 127).  out = x . W[e]^T for every routed row, fp32
// accumulation, rounded to bf16 once.
//
// Why there is no correction step: a scaled E2M1 or E4M3 value is a bf16 value
// (two or four significant bits), so the weight is dequantised exactly into the
// MFMA's bf16 B operand by v_cvt_scalef32_pk_bf16_fp4 / _fp8 (two codes and the
// block's scale per instruction), and the MFMA products are exact.  Exponents
// 2..252 (MXFP4) or 10..246 (MXFP8) keep every weight a normal, finite bf16.
//
// The routing, tile table, tile shapes and the fused unpermute/store are the
// bf16 gather's.  The k order inside an MFMA k-step is free as long as both
// operands agree, and it is chosen for the weight loads: chunks (64 k) run in
// pairs, and lane (l16, c4) owns the 32 contiguous k from 32 c4 of its pair's
// 128 k, the first 16 in the even chunk and the rest in the odd one.  One
// 16-byte code load and one scale byte per 16-column block then serve two
// chunks (those 32 k are one 32-weight block).  Per-lane loads that gather a
// few bytes from 16 columns each are what limits this kernel, so halving the
// code loads and quartering the scale loads is what counts; the x copies into
// LDS fetch the matching 16-byte pieces of each row.
#include "mq_internal.h"

#include <type_traits>

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// 2^(e - 127) as fp32: the exponent field for e >= 1, the subnormal 2^-127 for
// e = 0 (255, the E8M0 NaN, is never produced by the quantiser)
__device__ inline float e8m0_scale(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// two E4M3 codes (one half of a word, low byte = lower k) times the block scale
// -> two bf16 (the OCP E4M3 format, as v_cvt_scalef32_pk_bf16_fp8 reads it)
template <bool HI>
__device__ inline uint32_t cvt_e4m3x2(uint32_t w, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, HI));
}

template <bool B, class T>
__device__ inline T& pick(T& a, T& b) {
  if constexpr (B) return a; else return b;
}

// eight E2M1 codes (one word, low nibble = lowest k) times the block scale ->
// eight bf16 in k order: byte b of the word gives bf16 pair (2b, 2b + 1)
__device__ inline u32x4 decode8(uint32_t w, float s) {
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
}

// value of a non-negative E4M3 code (< 0x7F), exactly, in fp32
__device__ inline float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0x1p-9f;
}

// eight E2M1 codes times an E4M3 block scale s.  The conversion instruction
// reads only the exponent field of its fp32 scale, as an E8M0 exponent (field
// 0 is 2^-127), so it gets the power-of-two part P of s, and the mantissa
// factor F = s / P in [1, 2) (0 when s == 0) multiplies each weight in fp32;
// e2m1 * s has at most six significant bits, so the bf16 results are exact
__device__ inline u32x4 decode8_nv(uint32_t w, float s) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t sb = __float_as_uint(s);
  const float P = __uint_as_float(sb & 0x7F800000u);
  const float F = (sb & 0x7F800000u) ? __uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u) : 0.0f;
  u32x4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x2 v;
    switch (b) {
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, P, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, P, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, P, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, P, 3); break;
    }
    r[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v * F, bf16x2));
  }
  return r;
}

// EB: element bits, 4 (MXFP4, E2M1) or 8 (MXFP8, E4M3).  NV (with EB = 4):
// NVFP4, an E4M3 scale per 16 weights and an fp32 scale per expert; a lane's
// 16 k of a chunk are then exactly one scale block (two per pair: one 2-byte
// load per 16-column block and pair), the block scale is applied exactly at
// decode (decode8_nv) and the expert's scale multiplies the fp32 sums.
template <int BM, int NW, int EB, bool SC4, bool NV>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void gather_mx_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  constexpr int MT = BM / 16;
  constexpr int BN = 64 * NW;
  constexpr int STAGE = BM * 128;                      // bytes of one x chunk
  constexpr int XDMA = BM * 8 / (64 * NW);             // x copies per wave per chunk
  static_assert(XDMA >= 1 && XDMA * 64 * NW == BM * 8, "x copies per chunk");
  constexpr int PPS = BM / 16;                         // 2 KiB store patches per stage
  static_assert(NW <= 3 * PPS, "store patches");
  // VMEM instructions a chunk issues: x copies for the chunk two ahead, and an
  // even chunk also the codes and scales of the next chunk pair (one 16-byte
  // code load and one scale byte per 16-column block)
  // (MXFP8: every chunk also loads its own codes, one 16-byte load per block,
  // two chunks ahead; the scales stay per pair)
  static_assert(EB == 4 || EB == 8, "element bits");
  static_assert(!NV || EB == 4, "NVFP4: E2M1 codes");
  constexpr int PER_ODD = XDMA + (EB == 8 ? NT : 0);
  constexpr int PER_EVEN = XDMA + NT + (SC4 ? 1 : NT);

  __shared__ __attribute__((aligned(16))) unsigned char xs0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xs2[STAGE];
  __shared__ int32_t xrow_tab[BM];
  __shared__ int32_t orow_tab[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N;

  // ---- which tile: the XCD-aware order of the other gathered GEMMs -------------
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
  const uint32_t crow_bytes = uint32_t(K) * EB / 8u;   // codes of one weight row
  const uint32_t srow_bytes = uint32_t(K) / (NV ? 16u : 32u);   // scales of one weight row
  const __amdgpu_buffer_rsrc_t cr =
      rsrc(reinterpret_cast<const unsigned char*>(a.wq) + int64_t(e) * N * crow_bytes,
           uint32_t(N) * crow_bytes);
  const __amdgpu_buffer_rsrc_t sr =
      rsrc(a.scales_e8 + int64_t(e) * N * srow_bytes, uint32_t(N) * srow_bytes);
  const __amdgpu_buffer_rsrc_t none = rsrc(a.x, 0u);
  // x copy j of this wave: rows 8 (j NW + wave) .. +7; lane -> row r, LDS slot
  // lane & 7, which holds 16-byte piece (slot ^ (r & 7) ^ ((r >> 3) & 1))
  // Piece s of a chunk (8 k) is, within its pair's 128 k, k = 32 (s >> 1) +
  // 8 (s & 1) + 16 h for chunk parity h: lane c4 then owns the 32 k from
  // 32 c4 of the pair, the first 16 in the even chunk, the rest in the odd.
  // xtail: the same offsets with the pieces past K (s >= 4) of a final half
  // pair (K / 64 odd) turned into zero reads.
  uint32_t xoff[XDMA], xtail[XDMA];
#pragma unroll
  for (int j = 0; j < XDMA; ++j) {
    const int r = (j * NW + wave) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
    const int32_t xrow = xrow_tab[r];
    xoff[j] = xrow < 0 ? kNoRow
                       : uint32_t(xrow) * uint32_t(K) * 2u + uint32_t(piece >> 1) * 64u +
                             uint32_t(piece & 1) * 16u;
    xtail[j] = piece >= 4 ? kNoRow : xoff[j];
  }
  // codes of block nt for pair q: column n0 + 64 wave + 16 nt + l16, k = 128 q
  // + 32 c4 .. +31 (MXFP4: four words, 16 bytes; MXFP8: 32 bytes, of which a
  // chunk of parity h loads the 16 from 16 h); their scale is that of 32-weight
  // block 4 q + c4.  The block's distance rides in soffset, so columns past N
  // read zeros (computed, never stored).  In a final half pair the lanes
  // c4 >= 2 lie past K and read zeros (ctail / stail).
  const uint32_t col = uint32_t(n0 + 64 * wave + l16);
  const uint32_t coff = col * crow_bytes + uint32_t(4 * EB) * uint32_t(c4);
  const uint32_t soff = col * srow_bytes + uint32_t(NV ? 2 * c4 : c4);
  const uint32_t ctail = c4 >= 2 ? kNoRow : coff, stail = c4 >= 2 ? kNoRow : soff;
  // SC4 (K % 128 == 0, no half pair): one 4-byte load per wave and pair
  // fetches the scales of all 64 columns (lane j: column n0 + 64 wave + j,
  // blocks 4 q .. 4 q + 3); each lane then takes its columns' words from the
  // lanes that hold them (ds_bpermute) and the byte of its c4
  // (NVFP4 with SC4: 8 bytes per column and pair, blocks 8 q .. 8 q + 7, and a
  // lane takes the two of its c4 from the dword c4 / 2 of its column's lane)
  const uint32_t s4off = uint32_t(n0 + 64 * wave + lane) * srow_bytes;
  const uint32_t cstep = 16u * crow_bytes, sstep = 16u * srow_bytes;
  // x fragment of k-step ks: row 16 mt + l16, piece 2 c4 + ks, swizzled as above
  const uint32_t aoff0 = uint32_t(l16 * 128 + 16 * ((2 * c4) ^ (l16 & 7) ^ ((l16 >> 3) & 1)));

  // the chunks run in whole pairs: for an odd count the last pair's second
  // half lies past K and reads zeros, as do its lanes c4 >= 2
  const bool odd = ((K / BK) & 1) != 0;
  const int nchunks = (K / BK + 1) & ~1;
  const int last_pair = nchunks / 2 - 1;
  auto issue_x = [&](__amdgpu_buffer_rsrc_t r, unsigned char* stage, int chunk) {
    const bool tail = odd && (chunk >> 1) == last_pair;
    const uint32_t so = uint32_t(chunk >> 1) * 256u + uint32_t(chunk & 1) * 32u;
#pragma unroll
    for (int j = 0; j < XDMA; ++j)
      dma16(r, stage + (j * NW + wave) * 1024, tail ? xtail[j] : xoff[j], so);
  };
  // codes of chunk c (MXFP8) or of its pair (MXFP4, c even), then the scales
  // of the pair (c even); the waits count VMEM instructions, so this is the
  // issue order
  auto load_c = [&](__amdgpu_buffer_rsrc_t rc, int c, u32x4 (&codes)[NT]) {
    const bool tail = odd && (c >> 1) == last_pair;
    const uint32_t co = tail ? ctail : coff;
    const uint32_t so = EB == 4 ? uint32_t(c >> 1) * 64u : uint32_t(c >> 1) * 128u + uint32_t(c & 1) * 16u;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      codes[nt] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, uni(so + uint32_t(nt) * cstep), 0);
  };
  auto load_s = [&](__amdgpu_buffer_rsrc_t rs, int q, uint32_t (&sc)[NT]) {
    const bool tail = odd && q == last_pair;
    const uint32_t so = tail ? stail : soff;
    if constexpr (SC4 && NV) {
      const u32x2 v = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, s4off, uni(uint32_t(q) * 8u), 0));
      sc[0] = v[0];
      sc[1] = v[1];
    } else if constexpr (SC4) {
      sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, s4off, uni(uint32_t(q) * 4u), 0);
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        sc[nt] = NV ? uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                          rs, so, uni(uint32_t(q) * 8u + uint32_t(nt) * sstep), 0))
                    : uint32_t(__builtin_amdgcn_raw_buffer_load_b8(
                          rs, so, uni(uint32_t(q) * 4u + uint32_t(nt) * sstep), 0));
    }
  };
  // NVFP4: the two block-scale bytes (chunk parity 0, 1) of this lane's column
  // of block nt and pair
  auto nv_pair = [&](const uint32_t (&sb)[NT], int nt) -> uint32_t {
    if constexpr (SC4) {
      const int src = (16 * nt + l16) * 4;
      const uint32_t lo = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sb[0])));
      const uint32_t hi = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(sb[1])));
      return ((c4 >> 1) ? hi : lo) >> (16 * (c4 & 1));
    } else {
      return sb[nt];
    }
  };
  auto scale_of = [&](const uint32_t (&sb)[NT], int nt) -> uint32_t {
    if constexpr (SC4) {
      const uint32_t w = uint32_t(__builtin_amdgcn_ds_bpermute((16 * nt + l16) * 4, int(sb[0])));
      return (w >> (8 * c4)) & 0xFFu;
    } else {
      return sb[nt];
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // code buffers: MXFP4 one per pair (parity of the pair), MXFP8 one per chunk
  // (parity of the chunk); scale buffers one per pair
  u32x4 cb0[NT], cb1[NT];
  uint32_t sb0[NT], sb1[NT];

  // ---- prologue: chunks 0 and 1 (pair 0) in flight ------------------------------
  issue_x(xr, xs0, 0);
  load_c(cr, 0, cb0);
  load_s(sr, 0, sb0);
  issue_x(xr, xs1, 1);
  if constexpr (EB == 8) load_c(cr, 1, cb1);

  // one chunk: x stage `cur` holds chunk c, its codes are in cb (MXFP4: words
  // 2 (c & 1), +1 of the pair's; MXFP8: the chunk's 16 bytes) and its pair's
  // scales in sb.  It issues chunk c + 2's x copy, then chunk c + 2's codes
  // (MXFP8, into cb once decoded) or, when c is even, the next pair's codes
  // (MXFP4, into nb), then, when c is even, the next pair's scales (into nsb).
  auto chunk = [&](int c, unsigned char* cur, unsigned char* nxt, u32x4 (&cb)[NT],
                   u32x4 (&nb)[NT], uint32_t (&sb)[NT], uint32_t (&nsb)[NT], auto parity) {
    constexpr int H = decltype(parity)::value;
    __builtin_amdgcn_sched_barrier(0);
    // this chunk's x copy was issued two chunks ago; what the previous chunk
    // issued may still be in flight
    wait_vmem<H ? PER_EVEN : PER_ODD>();
    wait_lds();
    __builtin_amdgcn_s_barrier();
    const int cn = c + 2;
    const bool pre = cn < nchunks;
    issue_x(pre ? xr : none, nxt, cn);
    u32x4 bf[KS][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float s = NV ? e4m3_to_f32((nv_pair(sb, nt) >> (8 * H)) & 0x7Fu)
                         : e8m0_scale(scale_of(sb, nt));
      if constexpr (NV) {
        bf[0][nt] = decode8_nv(cb[nt][2 * H], s);
        bf[1][nt] = decode8_nv(cb[nt][2 * H + 1], s);
      } else if constexpr (EB == 4) {
        bf[0][nt] = decode8(cb[nt][2 * H], s);
        bf[1][nt] = decode8(cb[nt][2 * H + 1], s);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bf[ks][nt] = u32x4{cvt_e4m3x2<false>(cb[nt][2 * ks], s), cvt_e4m3x2<true>(cb[nt][2 * ks], s),
                             cvt_e4m3x2<false>(cb[nt][2 * ks + 1], s),
                             cvt_e4m3x2<true>(cb[nt][2 * ks + 1], s)};
      }
    }
    if (EB == 8 || !H) load_c(pre ? cr : none, cn, nb);
    if (!H) load_s(pre ? sr : none, cn >> 1, nsb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(cur + mt * 2048 + (aoff0 ^ (ks ? 16u : 0u)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma(af, bf[ks][nt], acc[mt][nt]);
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int c = 0;; c += 12) {
    chunk(c, xs0, xs2, pick<EB == 4>(cb0, cb0), pick<EB == 4>(cb1, cb0), sb0, sb1, P0{});
    if (c + 1 >= nchunks) break;
    chunk(c + 1, xs1, xs0, pick<EB == 4>(cb0, cb1), pick<EB == 4>(cb1, cb1), sb0, sb1, P1{});
    if (c + 2 >= nchunks) break;
    chunk(c + 2, xs2, xs1, pick<EB == 4>(cb1, cb0), pick<EB == 4>(cb0, cb0), sb1, sb0, P0{});
    if (c + 3 >= nchunks) break;
    chunk(c + 3, xs0, xs2, pick<EB == 4>(cb1, cb1), pick<EB == 4>(cb0, cb1), sb1, sb0, P1{});
    if (c + 4 >= nchunks) break;
    chunk(c + 4, xs1, xs0, pick<EB == 4>(cb0, cb0), pick<EB == 4>(cb1, cb0), sb0, sb1, P0{});
    if (c + 5 >= nchunks) break;
    chunk(c + 5, xs2, xs1, pick<EB == 4>(cb0, cb1), pick<EB == 4>(cb1, cb1), sb0, sb1, P1{});
    if (c + 6 >= nchunks) break;
    chunk(c + 6, xs0, xs2, pick<EB == 4>(cb1, cb0), pick<EB == 4>(cb0, cb0), sb1, sb0, P0{});
    if (c + 7 >= nchunks) break;
    chunk(c + 7, xs1, xs0, pick<EB == 4>(cb1, cb1), pick<EB == 4>(cb0, cb1), sb1, sb0, P1{});
    if (c + 8 >= nchunks) break;
    chunk(c + 8, xs2, xs1, pick<EB == 4>(cb0, cb0), pick<EB == 4>(cb1, cb0), sb0, sb1, P0{});
    if (c + 9 >= nchunks) break;
    chunk(c + 9, xs0, xs2, pick<EB == 4>(cb0, cb1), pick<EB == 4>(cb1, cb1), sb0, sb1, P1{});
    if (c + 10 >= nchunks) break;
    chunk(c + 10, xs1, xs0, pick<EB == 4>(cb1, cb0), pick<EB == 4>(cb0, cb0), sb1, sb0, P0{});
    if (c + 11 >= nchunks) break;
    chunk(c + 11, xs2, xs1, pick<EB == 4>(cb1, cb1), pick<EB == 4>(cb0, cb1), sb1, sb0, P1{});
    if (c + 12 >= nchunks) break;
  }

  // ---- store: fp32 -> bf16 through a per-wave LDS patch, then row segments ------
  wait_vmem<0>();
  wait_lds();
  __syncthreads();
  unsigned char* patch_base = wave < PPS ? xs0 : (wave < 2 * PPS ? xs1 : xs2);
  uint16_t* patch = reinterpret_cast<uint16_t*>(patch_base + (wave % PPS) * 2048);
  const bool vec_ok = (N % 8) == 0;
  // NVFP4: the expert's fp32 scale, applied to the fp32 sums before rounding
  const float gsc = NV ? a.gscale[e] : 1.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * c4 + i, cc = 16 * nt + l16;
        const float v = NV ? acc[mt][nt][i] * gsc : acc[mt][nt][i];
        patch[r * 64 + (((cc >> 3) ^ (r & 7)) << 3) + (cc & 7)] =
            __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int seg = lane + 64 * h;
      const int r = seg >> 3, cs = seg & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&patch[r * 64 + ((cs ^ (r & 7)) << 3)]);
      const int tr = mt * 16 + r;
      const int oc = n0 + 64 * wave + 8 * cs;
      if (tr < rows && oc < N) {
        uint16_t* dst = a.out + int64_t(orow_tab[tr]) * N + oc;
        if (vec_ok) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (oc + q < N) dst[q] = uint16_t(v[q >> 1] >> (16 * (q & 1)));
        }
      }
    }
  }
}

template <int BM>
hipError_t launch_mx_bm(const GemmArgs& a, hipStream_t s) {
  constexpr int NW = BM == 16 ? 2 : 4;
  constexpr int BN = 64 * NW;
  const int64_t blocks = ceil_div(ceil_div(a.N, BN) * a.max_tiles, 8) * 8;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // the 4-byte scale loads need K % 128 == 0 (whole pairs, aligned rows) and
  // a 4-byte aligned scale array
  const bool sc4 = a.K % 128 == 0 && (reinterpret_cast<uintptr_t>(a.scales_e8) & 3u) == 0;
  const dim3 grid{unsigned(blocks)}, block{unsigned(64 * NW)};
  if (a.gscale) {
    // the 8-byte scale loads need K % 128 == 0 and an 8-byte aligned scale array
    const bool sc8 = a.K % 128 == 0 && (reinterpret_cast<uintptr_t>(a.scales_e8) & 7u) == 0;
    note_dispatch("gather_mx", {BM, NW, 4, sc8, 1});
    if (sc8)
      gather_mx_kernel<BM, NW, 4, true, true><<<grid, block, 0, s>>>(a);
    else
      gather_mx_kernel<BM, NW, 4, false, true><<<grid, block, 0, s>>>(a);
  } else if (a.bits == 8) {
    note_dispatch("gather_mx", {BM, NW, 8, sc4, 0});
    if (sc4) gather_mx_kernel<BM, NW, 8, true, false><<<grid, block, 0, s>>>(a);
    else gather_mx_kernel<BM, NW, 8, false, false><<<grid, block, 0, s>>>(a);
  } else {
    note_dispatch("gather_mx", {BM, NW, 4, sc4, 0});
    if (sc4) gather_mx_kernel<BM, NW, 4, true, false><<<grid, block, 0, s>>>(a);
    else gather_mx_kernel<BM, NW, 4, false, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_mx(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  switch (a.bm) {
    case 16: return launch_mx_bm<16>(a, s);
    case 32: return launch_mx_bm<32>(a, s);
    case 64: return launch_mx_bm<64>(a, s);
    default: return launch_mx_bm<128>(a, s);
  }
}

}  // namespace mq
