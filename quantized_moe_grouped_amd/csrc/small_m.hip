// Weight-reusing small-M path: row tiles of TR <= 8 rows against a quantised
// weight, each weight byte read from memory once per tile.
//
// lablup/mlxcel issue 725, "The gap" and "What's needed": batched decode with
// B <= 8 rows must not re-read the whole weight per row (per-row matrix-vector
// kernels make the traffic O(B)), and a 128-row tile wastes ~94% of its work
// at M = 8.  Here one workgroup owns NT blocks of 16 output columns of one row
// tile (dense: the M rows; gathered: the <= TR routed rows of one expert) and
// its KW waves split K; or, for short rows (CS, "column split"), each of its
// KW waves owns NT blocks of its own and walks the whole of K.  Every code, scale and bias of those columns is loaded
// once and applied to all rows of the tile.  The work is HBM-bound: each wave
// keeps the weights of D steps in flight and never waits on another wave.
//
// One MFMA k-step (v_mfma_f32_16x16x32_bf16, 16 rows x 16 columns x 32 k).
// Lane (l16, c4) holds 8 consecutive codes of column l16 in the B operand.  A
// wave step covers SK consecutive k of its columns; quarters c4 = 0, 1 hold the
// first half of them and quarters 2, 3 the second half, and each half lies in
// one quantisation group.  The 16 rows of the A operand are (half, x row):
// rows 0-7 carry the tile's x rows on the first half's k slots and zeros on
// the others, rows 8-15 the same x rows on the second half's slots.  One MFMA
// therefore gives the group partial sums of both halves for all rows, and
// output lane (column, c4) holds rows 4c4..4c4+3, all of one half: it applies
// the scale and bias of its own column and half.  The per-half row sums of x
// (for the bias and the code offset) come from an MFMA of the same A against
// ones.
//
// Arithmetic is the GEMM's (exact codes, per-group fp32 epilogue): per group
// P = x . (off + q) and X = x . 1, then acc += s P + (b - off s) X.  Partial
// sums of the waves and of the two halves meet in LDS in a fixed order, so
// results are deterministic.
//
// Every byte through the load path costs time, whether it comes from HBM, L2
// or an out-of-range offset (which reads zeros), so the loads are cut to the
// bytes the tile needs:
//   x       one dword-per-lane copy (buffer_load ... lds) per row and step,
//           into a per-wave LDS ring of D slots; rows padded to 272 bytes so
//           that the fragment reads are free of bank conflicts, A lanes that
//           carry zeros read a zero block;
//   scales  one dword per lane per round of D steps (the four lanes of a
//           column hold the round's four dwords; ds_bpermute hands each step
//           its dword);
//   tail    the last round issues no loads.
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kNoRow = 0x80000000u;          // outside every descriptor range (< 2 GiB)
constexpr int D = 4;                             // steps in flight per wave (a round)
constexpr int RS = 272;                          // LDS bytes of one x row (pair) of a slot
constexpr int ZERO_BYTES = 64;                   // zero block: four 16-byte k-steps
// LDS bytes for the workgroup's scale rows (and again for its bias rows),
// 16 * NT rows of G values: 4 KB (two column blocks, G <= 64), 8 KB (one
// block, G <= 256) or 32 KB (one block, G <= 1024; at most 8 waves, so that
// the ring still fits).  The column split's 4 waves hold 64 * NT rows in
// 8 KB blocks (G <= 64 for one block per wave, G <= 32 for two).
constexpr int kScaleSmall2 = 4096, kScaleSmall1 = 8192, kScaleLarge = 32768;
constexpr int kMaxSmallGroups = kScaleLarge / (16 * 2);

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

// a uniform value, stated as such (a VGPR soffset is served by a loop)
__device__ inline int uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(int(v)); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding)
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 8 four-bit codes (nibbles 0..7 = k0..k7) -> bf16 (16 + q) pairs in natural
// order: q goes to mantissa bits 3..6 of 16.0 (byte i of w << 3 holds k_2i
// there, byte i of w >> 1 holds k_2i+1); mask 0x00780078 and base 0x41804180
// come in registers (a VOP3 instruction takes no literal).  16 is the
// smallest power of two above every code, so the fp32 sums cancel the least.
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
// natural order (q < 256 is exact in the upper half of its fp32 value)
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

// Geometry of one wave step for a code format and tile height.
template <int BITS, int GS, int TR>
struct Step {
  static constexpr int LB = (BITS == 4 && GS == 32) ? 8 : 16;  // code bytes per lane
  static constexpr int CPL = LB * 8 / BITS;       // codes per lane: 32 or 16
  static constexpr int SK = 4 * CPL;              // k per step: 128 or 64
  static constexpr int JS = CPL / 8;              // MFMA k-steps per step: 4 or 2
  static constexpr int RB = SK * 2;               // bytes of one x row per step: 256 or 128
  static constexpr int RPC = 256 / RB;            // x rows per copy (a dword per lane): 1 or 2
  static constexpr int XI = (TR + RPC - 1) / RPC; // copies per step
  static constexpr int SLOT = XI * RS;            // LDS bytes of one step's x rows
  static constexpr int GPS = SK / GS;             // groups per step: 2, or 1 (8-bit gs64)
  static_assert(SK / 2 <= GS && GS % (SK / 2) == 0, "a half lies in one group");
  static_assert(JS * 16 <= ZERO_BYTES && TR >= 1 && TR <= 8, "step layout");
};

template <int BITS, int GS, int KW, int NT, int TR, int SCB, bool CS, bool FR>
__global__ __launch_bounds__(64 * KW, 4) void small_m_kernel(GemmArgs a) {
  using St = Step<BITS, GS, TR>;
  constexpr int LB = St::LB, SK = St::SK, JS = St::JS, RB = St::RB, SLOT = St::SLOT;
  constexpr int RPC = St::RPC, XI = St::XI, GPS = St::GPS;
  constexpr float OFF = BITS == 4 ? 16.0f : 0.0f;
  typedef typename std::conditional<LB == 16, u32x4, u32x2>::type codes_t;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[KW * SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[KW * SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[KW * SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[KW * SLOT];
  __shared__ __attribute__((aligned(64))) uint8_t zeros[ZERO_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sc_s[SCB];
  __shared__ __attribute__((aligned(1024))) uint8_t sc_b[SCB];
  // the tile's pairs when the workgroup routes the pairs itself (FR)
  __shared__ int32_t f_pairs[FR ? 8 : 1];
  // the partial sums of (column block j, half h) go to ring slot 2j + h
  static_assert(D == 4 && NT <= 2 && TR * 16 * 4 <= SLOT, "partials in the ring");
  static_assert(SCB >= (kFuseMaxExperts + 1) * 4, "routing scratch in the scale blocks");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;
  // columns of the workgroup (CS: KW times those of a wave)
  constexpr int WCOLS = CS ? 16 * NT * KW : 16 * NT;
  const int cbs = (N + WCOLS - 1) / WCOLS;

  // (the grid is exactly cbs * max_tiles workgroups, so t < max_tiles)
  const int t = int(blockIdx.x / unsigned(cbs));
  const int n0 = int(blockIdx.x % unsigned(cbs)) * WCOLS;
  // first column of this wave's blocks
  const int nw = CS ? n0 + 16 * NT * wave : n0;
  // Row counts fit in 31 bits on this path (pairs * M < 2^31 is checked on
  // the host), so row arithmetic is 32-bit.
  int e = 0, row0, seg_end;
  const bool routed = FR || a.perm;
  if constexpr (FR) {
    // ---- the routing of a decode step, in this workgroup ------------------------
    // (lablup/mlxcel issue 629, "Implementation plan" 4b: sort by expert on the
    // device.)  Histogram over E + 1 bins (bin E: indices outside [0, E)), then
    // the exclusive scans that give the segment offsets and the tile prefix,
    // as the routing kernels compute them; the scale blocks' LDS is free until
    // the scales are published.
    int32_t* const cnt = reinterpret_cast<int32_t*>(sc_s);
    int32_t* const tpre = reinterpret_cast<int32_t*>(sc_b);
    __shared__ int32_t f_invalid;
    const int n = int(a.n_pairs), bins = a.E + 1, nthr = 64 * KW;
    // Every index load is issued before the first is used (a loop of load,
    // then use, would wait for each in turn): up to HR per thread for the
    // histogram, and in wave 0 all chunks of 64 for the pair search and the
    // scatter below.
    constexpr int HR = (kFuseMaxPairs + 255) / 256;   // rounds of >= 256 threads
    constexpr int PC = kFuseMaxPairs / 64;            // chunks of 64 pairs
    int hv[HR], pv[PC];
#pragma unroll
    for (int r = 0; r < HR; ++r) hv[r] = a.idx[min(tid + r * nthr, n - 1)];
    if (wave == 0) {
#pragma unroll
      for (int c = 0; c < PC; ++c) pv[c] = a.idx[min(c * 64 + lane, n - 1)];
    }
    for (int b = tid; b < bins; b += nthr) cnt[b] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < HR; ++r) {
      const int v = hv[r];
      if (tid + r * nthr < n) atomicAdd(&cnt[uint32_t(v) < uint32_t(a.E) ? v : a.E], 1);
    }
    __syncthreads();
    if (wave == 0) {
      const int per = (bins + 63) / 64;
      const int b0 = min(lane * per, bins), b1 = min(b0 + per, bins);
      int sc = 0, st = 0;
      for (int b = b0; b < b1; ++b) {
        sc += cnt[b];
        st += b < a.E ? (cnt[b] + TR - 1) / TR : 0;
      }
      int ic = sc, it = st;
      for (int d = 1; d < 64; d <<= 1) {
        const int yc = __shfl_up(ic, d, 64), yt = __shfl_up(it, d, 64);
        if (lane >= d) {
          ic += yc;
          it += yt;
        }
      }
      int rc = ic - sc, rt = it - st;
      for (int b = b0; b < b1; ++b) {
        const int c = cnt[b];
        if (b == a.E) f_invalid = c;
        cnt[b] = rc;
        tpre[b] = rt;
        rc += c;
        rt += b < a.E ? (c + TR - 1) / TR : 0;
      }
    }
    __syncthreads();
    // this workgroup's tile: expert (the largest e with tpre[e] <= t), rows,
    // and the pairs of ranks r0 .. r0 + want - 1 among expert e's, in pair order
    const int ntiles = tpre[a.E];
    int want = 0;
    if (t < ntiles) {
      int lo = 0, hi = a.E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (tpre[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      e = __builtin_amdgcn_readfirstlane(lo);
      const int r0 = (t - tpre[e]) * TR;
      row0 = cnt[e] + r0;
      seg_end = cnt[e + 1];
      want = min(TR, seg_end - row0);
      if (wave == 0) {
        const uint64_t lt = (uint64_t(1) << lane) - 1;
        int run = 0;
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          const int i = c * 64 + lane;
          if (c * 64 >= n || run >= r0 + want) break;   // uniform
          const bool m = i < n && pv[c] == e;
          const uint64_t mask = __ballot(m);
          const int r = run + __popcll(mask & lt);
          if (m && r >= r0 && r < r0 + want) f_pairs[r - r0] = i;
          run += __popcll(mask);
        }
      }
    }
    if (blockIdx.x == 0) {
      // Workgroup 0 leaves the routing in the workspace, as the routing
      // kernels would: offsets, tile table, error word, and perm by a stable
      // counting sort (wave 0, 64 pairs a round; the offsets array serves as
      // the per-expert cursor, so ranks among equal experts follow the pair
      // order).  Rows of out-of-range pairs, the tail of perm, are zeroed.
      __syncthreads();                      // every wave has read cnt above
      for (int b = tid; b < bins; b += nthr) {
        a.r_offsets[b] = cnt[b];
        a.r_tiles[b] = tpre[b];
      }
      if (tid == 0) {
        a.r_error[0] = f_invalid;
        a.r_error[1] = TR;
      }
      const int valid_pairs = cnt[a.E];
      __syncthreads();                      // the offsets are copied before they move
      if (wave == 0) {
        int nbits = 0;
        while ((1 << nbits) < bins) ++nbits;
        const uint64_t lt = (uint64_t(1) << lane) - 1;
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          if (c * 64 >= n) break;                         // uniform
          const int i = c * 64 + lane;
          const bool valid = i < n;
          int v = valid ? pv[c] : 0;
          if (uint32_t(v) >= uint32_t(a.E)) v = a.E;
          uint64_t peers = __ballot(valid);
          for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (v >> bit) & 1;
            const uint64_t m = __ballot(set);
            peers &= set ? m : ~m;
          }
          const int rank = __popcll(peers & lt);
          // every lane reads its expert's cursor before the first lane of
          // each expert moves it (a wave's LDS accesses keep program order)
          const int base = cnt[v];
          if (valid) a.r_perm[base + rank] = i;
          if (valid && rank == 0) cnt[v] = base + __popcll(peers);
        }
      }
      const int ninv = f_invalid;
      if (ninv > 0) {
        __syncthreads();                    // wave 0's perm writes are visible to the block
        for (int w = tid; w < ninv * N; w += nthr) {
          const int pair = min(max(a.r_perm[valid_pairs + w / N], 0), n - 1);
          a.out[int64_t(pair) * N + w % N] = 0;
        }
      }
    }
    if (t >= ntiles) return;
    __syncthreads();                        // f_pairs
  } else if (a.perm) {
    if (*a.tile_bm != TR) return;               // workspace routed for another tiling
    if (t >= a.tiles[a.E]) return;
    // expert of tile t: the largest e with tiles[e] <= t (tiles is
    // non-decreasing).  Two rounds of 64 lanes: coarse entries every `step`,
    // then the step between two of them.
    const int step = (a.E + 64) / 64;                 // E + 1 entries <= 64 * step
    const int i1 = min(lane * step, a.E);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(a.tiles[i1] <= t);
    const int lo = (63 - __builtin_clzll(m1)) * step;  // lane 0 always qualifies (tiles[0] = 0)
    const int i2 = min(lo + lane, a.E);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < step && a.tiles[i2] <= t);
    e = __builtin_amdgcn_readfirstlane(min(lo + (63 - __builtin_clzll(m2)), a.E - 1));
    // offsets come from the routing kernels; clamping them to [0, rows] keeps
    // every access in bounds even if they were corrupted
    const int nrows = int(a.n_pairs * a.M);
    row0 = min(max(a.offsets[e] * a.M, 0) + (t - a.tiles[e]) * TR, nrows);
    seg_end = min(max(a.offsets[e + 1] * a.M, 0), nrows);
  } else {
    row0 = t * TR;
    seg_end = int(a.n_pairs * a.M);
  }
  if (row0 >= seg_end) return;
  const int rows = min(TR, seg_end - row0);

  // ---- steps of this wave and the weight codes: their loads go out first ---------
  // With 128-k steps and K = 64 mod 128 (an odd number of groups of 64) the
  // last step's second half lies past K: its x is copied from outside the
  // buffer, i.e. as zeros, and its scale index is clamped to a loaded value.
  const int S = (K + SK - 1) / SK;
  const bool ragged = (K % SK) != 0;
  const int per = CS ? S : (S + KW - 1) / KW;
  const int s_lo = CS ? 0 : min(S, wave * per), s_hi = min(S, s_lo + per);
  const uint32_t wrow_bytes = uint32_t(K) * BITS / 8;
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq + int64_t(e) * N * (K * BITS / 32), uint32_t(N) * wrow_bytes);
  // descriptors of a step past the wave's range: every access reads zeros
  const __amdgpu_buffer_rsrc_t none = rsrc(a.x, 0u);
  // Own slices (a.sw; split of K over 8 or 16 waves, one round per wave,
  // routing not folded in): each wave copies the scales and biases of its own groups (at most
  // 8 a column: 16 bytes) for the block's columns straight into 1 KB of LDS
  // of its own, so no wave waits for another's before the final reduction.
  // Otherwise wave w holds pieces w, w + KW, ... of each block (in registers
  // until the first barrier, where they go to LDS).
  constexpr bool SW_OK = !CS && !FR && SCB <= kScaleSmall1 && KW >= 8 && KW <= 2 * (SCB / 1024);
  const bool sw = SW_OK && a.sw != 0;
  uint8_t* const own = wave < SCB / 1024 ? sc_s + 1024 * wave : sc_b + 1024 * (wave - SCB / 1024);
  constexpr int PPW = (SCB / 1024 + KW - 1) / KW;                   // pieces per wave, at most
  const int pieces = (WCOLS * G * 2 + 1023) / 1024;                 // <= SCB / 1024 (checked at launch)
  u32x4 s_piece[PPW], b_piece[PPW];
  // last value of the block inside the array, and the wave holding its piece
  const int fix_at = (min(n0 + WCOLS, N) - n0) * G - 1;
  const bool fix_wave = (fix_at * 2 / 1024) % KW == wave;
  uint16_t s_fix, b_fix;
  {
    const __amdgpu_buffer_rsrc_t srs = rsrc(a.scales + int64_t(e) * N * G, uint32_t(N) * G * 2u);
    const __amdgpu_buffer_rsrc_t brs = rsrc(a.biases + int64_t(e) * N * G, uint32_t(N) * G * 2u);
    const uint32_t blk0 = uint32_t(n0) * uint32_t(G) * 2u;           // byte offset of the block
    if (sw) {
      // lane l < 32: the 16 bytes of column n0 + l from its first group of this
      // wave's steps (G is even: dword aligned); scales to own[16 l], biases to
      // own[512 + 16 l].  Past the wave's groups the 16 bytes run into later
      // groups or the next column's row: read, never used.
      const int col = n0 + lane;
      const uint32_t off = lane < WCOLS && col < N && s_lo < S
                               ? (uint32_t(col) * uint32_t(G) + uint32_t(s_lo * GPS)) * 2u
                               : kNoRow;
      if (lane < 32) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_ptr)own, 16, int(off), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_ptr)(own + 512), 16, int(off), 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int c = wave + p * KW;
        const uint32_t off = blk0 + 1024u * uint32_t(c) + 16u * lane;
        s_piece[p] = __builtin_amdgcn_raw_buffer_load_b128(c < pieces ? srs : none, off, 0, 0);
        b_piece[p] = __builtin_amdgcn_raw_buffer_load_b128(c < pieces ? brs : none, off, 0, 0);
      }
      // With N * G odd the expert's last value shares a dword with the 2 bytes
      // past its range, and a load reads that whole dword as zeros: the wave
      // whose piece holds the block's last value also loads it on its own.
      s_fix = __builtin_amdgcn_raw_buffer_load_b16(fix_wave ? srs : none, blk0 + uint32_t(fix_at) * 2u, 0, 0);
      b_fix = __builtin_amdgcn_raw_buffer_load_b16(fix_wave ? brs : none, blk0 + uint32_t(fix_at) * 2u, 0, 0);
    }
  }
  // the pieces to LDS, then a barrier (after which every wave reads the whole
  // blocks); the LDS writes have completed before the barrier, the loads of
  // the steps need not have
  auto publish_scales = [&]() {
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int c = wave + p * KW;
      if (c < pieces) {
        *reinterpret_cast<u32x4*>(sc_s + 1024 * c + 16 * lane) = s_piece[p];
        *reinterpret_cast<u32x4*>(sc_b + 1024 * c + 16 * lane) = b_piece[p];
      }
    }
    // (after the piece, in this wave's LDS order)
    if (fix_wave && lane == 0) {
      reinterpret_cast<uint16_t*>(sc_s)[fix_at] = s_fix;
      reinterpret_cast<uint16_t*>(sc_b)[fix_at] = b_fix;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
  };
  uint32_t woff[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) woff[j] = uint32_t(min(nw + 16 * j + l16, N - 1)) * wrow_bytes + uint32_t(LB) * c4;
  codes_t cw[D][NT];
  auto issue_codes = [&](int st, int d) {
    const __amdgpu_buffer_rsrc_t wr_ = st < s_hi ? wr : none;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (LB == 16)
        cw[d][j] = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[j], uni(uint32_t(st) * 4 * LB), 0);
      else
        cw[d][j] = __builtin_amdgcn_raw_buffer_load_b64(wr_, woff[j], uni(uint32_t(st) * 4 * LB), 0);
    }
  };
  // the x rows of this lane's copies: routed rows need their pair from perm,
  // loaded ahead of the first codes so that it does not hold them up
  int prow[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = min(RPC * i + lane / (64 / RPC), rows - 1);
    const int j = row0 + r;
    if constexpr (FR) prow[i] = f_pairs[r];
    else prow[i] = a.perm ? a.perm[a.M == 1 ? j : j / a.M] : 0;
  }
  issue_codes(s_lo, 0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- x rows of the tile ------------------------------------------------------------
  // copy i of a step: x rows RPC*i .. RPC*i + RPC - 1, a dword per lane, to
  // LDS slot + RS * i (rows of a pair back to back); rows past the tile are
  // copied from outside the buffer, as zeros
  uint32_t xv[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = RPC * i + lane / (64 / RPC);
    const int j = row0 + r;
    int xrow = j;
    if (routed) {
      const int jp = a.M == 1 ? j : j / a.M;
      const int pair = min(max(prow[i], 0), int(a.n_pairs) - 1);
      const int tok = pair / a.A, slot = pair - tok * a.A;
      xrow = (tok * a.Ax + (a.Ax > 1 ? slot : 0)) * a.M + (j - jp * a.M);
    }
    // < x_bytes < 2^31
    xv[i] = r < rows ? uint32_t(xrow) * uint32_t(K) * 2u + 4u * uint32_t(lane % (64 / RPC)) : kNoRow;
  }

  // ---- scale and bias rows of the workgroup's columns --------------------------------
  // Column n's G values are one row of the [N, G] arrays, so the workgroup's
  // WCOLS rows are one contiguous block of each array.  The waves copy the
  // two blocks into LDS in 1 KB pieces (whole cache lines: read lane by lane
  // from memory, the rows of 16 columns would touch 16 lines per load), the
  // first loads of the kernel; each lane then reads the value of its column
  // and half for every step from LDS.  (Past the last column the copy reads
  // the next rows, or zeros past the block; those columns are not stored.)
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const int half = c4 >> 1;

  // ---- LDS fragment addresses ----------------------------------------------------
  // A lane (row l16, quarter c4) carries x row b = l16 & 7 when its row half
  // (l16 >> 3) is the half its k slots belong to (c4 >> 1) and b < TR; else
  // zeros.  Both kinds of address are offsets from the slot's own ring array,
  // so the compiler ties each fragment read to the copies into that array.
  const int xb = l16 & 7;
  const bool alive = (l16 >> 3) == half && xb < TR;
  const uint32_t frag = uint32_t(RS * (xb / RPC) + RB * (xb % RPC) + 16 * JS * c4);
  auto ring_of = [&](int d) -> uint8_t* {
    return d == 0 ? ring0 : d == 1 ? ring1 : d == 2 ? ring2 : ring3;
  };
  uint8_t* rings[D];
#pragma unroll
  for (int d = 0; d < D; ++d) rings[d] = ring_of(d) + wave * SLOT;
  uint32_t voff[D];
#pragma unroll
  for (int d = 0; d < D; ++d) voff[d] = alive ? frag : uint32_t(zeros - rings[d]);
  // the wave's own zero block writes precede its own reads (LDS keeps a
  // wave's order); every wave writes the same zeros
  if (lane < ZERO_BYTES / 16) reinterpret_cast<u32x4*>(zeros)[lane] = u32x4{0u, 0u, 0u, 0u};
  asm volatile("" ::: "memory");

  // the step's x rows
  // copy offsets of the last, ragged step: the lanes of the half past K
  uint32_t xv_last[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) xv_last[i] = (lane % (64 / RPC)) * 4 < RB / 2 ? xv[i] : kNoRow;
  auto issue_x = [&](int st, int d) {
    const __amdgpu_buffer_rsrc_t xr_ = st < s_hi ? xr : none;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr_, (lds_ptr)(rings[d] + RS * i), 4,
                                               int(ragged && st == S - 1 ? xv_last[i] : xv[i]),
                                               uni(uint32_t(st) * RB), 0, 0);
  };
  // scale and bias of (column block j, this lane's column and half) at step st
  uint32_t sc_off[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    sc_off[j] = (uint32_t(nw - n0 + 16 * j + l16) * uint32_t(G) + uint32_t(half * (GPS - 1))) * 2u;
  // (clamped to the block: the second half of a ragged last step names the
  // group past the row, whose x is zero but whose value must be finite)
  const uint32_t sc_last = uint32_t(WCOLS * G - 1) * 2u;
  // (own slices: value (st - s_lo) GPS + half of column 16 j + l16's 16 bytes)
  auto scale_at = [&](int bias, int j, int st) -> float {
    uint16_t v;
    if (sw) {
      const uint32_t off = uint32_t(bias * 512 + (16 * j + l16) * 16 +
                                    ((st - s_lo) * GPS + half * (GPS - 1)) * 2);
      v = *reinterpret_cast<const uint16_t*>(own + off);
    } else {
      const uint32_t off = min(sc_off[j] + uint32_t(st) * GPS * 2u, sc_last);
      v = *reinterpret_cast<const uint16_t*>((bias ? sc_b : sc_s) + off);
    }
    return __uint_as_float(uint32_t(v) << 16);
  };

  uint32_t dmask, dbase;
  asm("s_mov_b32 %0, 0x00780078" : "=s"(dmask));
  asm("v_mov_b32 %0, 0x41804180" : "=v"(dbase));
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int rounds = (s_hi - s_lo + D - 1) / D;
  // the first round's loads, in the order of the later rounds (codes, then
  // x rows and scales, step by step), so that every round gets the same wait
  // counts; the scheduler keeps each step's loads together and in order
  issue_x(s_lo, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 1; d < D; ++d) {
    issue_codes(s_lo + d, d);
    issue_x(s_lo + d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One round of D steps.  The steps past the wave's range read zeros through
  // the empty descriptor and add nothing.  Every round but the last issues
  // the next round's loads as its steps free their slots; the last issues none.
  // (The round loop has no early exit: an exit from inside a round would add
  // never-taken paths from a step's issue back to its compute, and the
  // compiler's wait counts follow every path.)
  auto round = [&](int it, auto more) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s_lo + it * D + d;
      f32x4 P[NT], X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NT; ++j) P[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < JS; ++ks) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(rings[d] + voff[d] + 16 * ks);
        X = mfma(A, ones, X);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          u32x4 bfrag;
          if constexpr (BITS == 4) bfrag = decode4(cw[d][j][ks], dmask, dbase);
          else bfrag = decode8(cw[d][j][2 * ks], cw[d][j][2 * ks + 1]);
          P[j] = mfma(A, bfrag, P[j]);
        }
      }
      // The scale and bias pieces are the oldest loads of every wave, so
      // they have landed once the first step's codes have; they go to LDS and
      // a barrier (without a memory fence) makes every wave's pieces visible.
      // It sits here, after the first step's MFMAs, rather than before any
      // step, so that a wave is not held while its siblings still issue.
      // (own slices: the wave's copies are its oldest loads, landed with the
      // first step's codes, and LDS keeps the wave's order; no barrier)
      if (d == 0 && it == 0 && !sw) publish_scales();
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float s = scale_at(0, j, st);
        const float c = scale_at(1, j, st) - OFF * s;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(s, P[j][q], fmaf(c, X[q], acc[j][q]));
      }
      if constexpr (decltype(more)::value) {
        __builtin_amdgcn_sched_barrier(0);
        issue_codes(st + D, d);
        issue_x(st + D, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Waves without steps meet the others' barrier here (see the round).
  if (rounds == 0 && !sw) publish_scales();
  for (int it = 0; it + 1 < rounds; ++it) round(it, std::true_type{});
  if (rounds > 0) round(rounds - 1, std::false_type{});

  // ---- reduce the waves' and halves' partial sums in a fixed order, store ----------
  // every copy of this wave has landed before its ring is reused
  wait_vmem<0>();
  // partials of (block j, half h) of wave w: floats [x row b < TR][column] at
  // ring slot 2j + h of the wave; lane (n, c4) holds rows 4 (c4 & 1) .. + 3
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    // (a select of two addresses: indexing the slot table with the lane's
    // half would put the table in scratch memory)
    float* const p = reinterpret_cast<float*>(half ? ring_of(2 * j + 1) + wave * SLOT
                                                   : ring_of(2 * j) + wave * SLOT);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = 4 * (c4 & 1) + q;
      if (b < TR) p[b * 16 + l16] = acc[j][q];
    }
  }
  __syncthreads();
  // output (column block j, x row r, column c) of the workgroup (CS: of this
  // wave's blocks, from its own partials)
  auto store = [&](int j, int r, int c, int w0, int w1, int col0) {
    const uint8_t* const h0 = j == 0 ? ring0 : ring2;
    const uint8_t* const h1 = j == 0 ? ring1 : ring3;
    float sum = 0.f;
    for (int w = w0; w < w1; ++w) {
      sum += reinterpret_cast<const float*>(h0 + w * SLOT)[r * 16 + c];
      sum += reinterpret_cast<const float*>(h1 + w * SLOT)[r * 16 + c];
    }
    const int col = col0 + 16 * j + c;
    if (r < rows && col < N) {
      const int jr = row0 + r;
      int orow = jr;
      if constexpr (FR) {
        orow = f_pairs[r];
      } else if (a.perm) {
        const int jp = a.M == 1 ? jr : jr / a.M;
        orow = min(max(a.perm[jp], 0), int(a.n_pairs) - 1) * a.M + (jr - jp * a.M);
      }
      a.out[int64_t(orow) * N + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
    }
  };
  if constexpr (CS) {
    for (int i = lane; i < NT * TR * 16; i += 64)
      store(i / (TR * 16), (i / 16) % TR, i % 16, wave, wave + 1, nw);
  } else if (tid < NT * TR * 16) {
    store(tid / (TR * 16), (tid / 16) % TR, tid % 16, 0, KW, n0);
  }
}

template <int BITS, int GS, int NT, int TR, bool FR>
hipError_t launch_kw(const GemmArgs& a, int kw, bool large, dim3 grid, hipStream_t s) {
  constexpr int SCB = NT == 2 ? kScaleSmall2 : kScaleSmall1;
  if (a.cs) {
    // (the column split's 4 waves: 8 KB blocks for one or two column blocks)
    note_dispatch("small_m", {BITS, GS, 4, NT, TR, kScaleSmall1, 1, FR});
    small_m_kernel<BITS, GS, 4, NT, TR, kScaleSmall1, true, FR><<<grid, dim3(256), 0, s>>>(a);
    return hipGetLastError();
  }
  if constexpr (NT == 1 && !FR) {
    if (large) {
      note_dispatch("small_m", {BITS, GS, kw == 8 ? 8 : 4, NT, TR, kScaleLarge, 0, 0});
      if (kw == 8) small_m_kernel<BITS, GS, 8, NT, TR, kScaleLarge, false, false><<<grid, dim3(512), 0, s>>>(a);
      else small_m_kernel<BITS, GS, 4, NT, TR, kScaleLarge, false, false><<<grid, dim3(256), 0, s>>>(a);
      return hipGetLastError();
    }
  }
  note_dispatch("small_m", {BITS, GS, kw == 16 ? 16 : (kw == 8 ? 8 : 4), NT, TR, SCB, 0, FR});
  if (kw == 16) small_m_kernel<BITS, GS, 16, NT, TR, SCB, false, FR><<<grid, dim3(1024), 0, s>>>(a);
  else if (kw == 8) small_m_kernel<BITS, GS, 8, NT, TR, SCB, false, FR><<<grid, dim3(512), 0, s>>>(a);
  else small_m_kernel<BITS, GS, 4, NT, TR, SCB, false, FR><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, int GS, int NT>
hipError_t launch_tr(const GemmArgs& a, int kw, bool large, dim3 grid, hipStream_t s) {
  // routed tiles (the only ones the routing can be folded into) are 4 or 8 rows
  if (a.fuse) {
    if (a.bm == 4) return launch_kw<BITS, GS, NT, 4, true>(a, kw, large, grid, s);
    return launch_kw<BITS, GS, NT, 8, true>(a, kw, large, grid, s);
  }
  switch (a.bm) {
    case 1: return launch_kw<BITS, GS, NT, 1, false>(a, kw, large, grid, s);
    case 2: return launch_kw<BITS, GS, NT, 2, false>(a, kw, large, grid, s);
    case 4: return launch_kw<BITS, GS, NT, 4, false>(a, kw, large, grid, s);
    default: return launch_kw<BITS, GS, NT, 8, false>(a, kw, large, grid, s);
  }
}

template <int BITS, int GS>
hipError_t launch_nt(const GemmArgs& a, int nt, int kw, bool large, dim3 grid, hipStream_t s) {
  if constexpr (BITS == 4)
    if (nt == 2) return launch_tr<BITS, GS, 2>(a, kw, false, grid, s);
  return launch_tr<BITS, GS, 1>(a, kw, large, grid, s);
}

}  // namespace

int small_m_rows(int64_t rows, int64_t E) {
  if (E <= 1) return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
  // routed: a tile never spans two experts, and every tile streams its
  // expert's weights once.  A tile of TR rows moves ~TR/8 of its code bytes
  // again as x (its rows over all of K, zero rows included), so an expert of
  // r rows costs ceil(r/4) * 1.5 in 4-row tiles and ceil(r/8) * 2 in 8-row
  // ones: 4-row tiles up to 4 rows per expert on average (at exactly 4 rows
  // per expert, E = 256, K = 2048 <-> 512: 53 against 61 us per projection;
  // Poisson-spread runs of 4 cost about the same either way).
  return 4 * E >= rows ? 4 : 8;
}

// Column blocks of 16 per wave: for 4-bit codes two when that still leaves
// >= 256 workgroups (a wave's x copies, fragments and row sums serve all its
// column blocks) and the workgroup's scale rows fit their LDS block.  8-bit
// codes carry twice the bytes per k, so one block already gives the same x
// bytes per code byte (and two would not fit in 128 VGPRs).
int small_m_cols(int64_t N, int64_t tiles, int bits, int64_t G) {
  return bits == 4 && 32 * G * 2 <= kScaleSmall2 && ceil_div(N, 16) * tiles >= 512 ? 2 : 1;
}

// Column split (4 waves, each with NT blocks of its own over the whole of K)
// for rows too short to give each of 4 waves 2 steps, when the workgroup's
// 64 NT columns of scales fit the LDS block.
bool small_m_colsplit_fits(int64_t K, int group_size, int nt) {
  return int64_t(16) * nt * 4 * (K / group_size) * 2 <= kScaleSmall1;
}
// One column block per wave and no column split: the shape small_m_shape
// picks whenever the scale rows would not fit the small blocks.
bool small_m_fuse_fits(int64_t K, int group_size) {
  return int64_t(16) * (K / group_size) * 2 <= kScaleSmall1;
}
bool small_m_own_slices(int64_t K, int bits, int group_size, int waves, int nt, bool cs, bool fuse,
                        bool large) {
  if (cs || fuse || large) return false;
  const int64_t sk = (bits == 4 && group_size == 64) ? 128 : 64;   // k per step
  if (sk / group_size != 2 || (K / group_size) % 2 != 0) return false;
  const int64_t steps = ceil_div(K, sk), per = ceil_div(steps, waves);
  const int blocks = (nt == 2 ? kScaleSmall2 : kScaleSmall1) / 1024;
  // (8 or 16 waves: with 4 the other kernel instances' registers grow more
  // than a one-round split of K gains)
  return per <= D && waves >= 8 && waves <= 2 * blocks;
}

bool small_m_colsplit(int64_t K, int bits, int group_size, int nt) {
  const int64_t sk = (bits == 4 && group_size == 64) ? 128 : 64;
  return ceil_div(K, sk) < 8 && small_m_colsplit_fits(K, group_size, nt);
}

// Waves per workgroup (splitting K): enough for ~3 waves per SIMD over the
// chip, as long as each wave keeps >= 2 steps.
int small_m_waves(int64_t blocks, int64_t K, int bits, int group_size) {
  const int64_t sk = (bits == 4 && group_size == 64) ? 128 : 64;
  const int64_t steps = ceil_div(K, sk);
  // the 32 KB scale block of long rows leaves room for the ring of 8 waves
  const int kw_max = 16 * (K / group_size) * 2 > kScaleSmall1 ? 8 : 16;
  int kw = 4;
  while (kw < kw_max && blocks * kw < 3072 && 2 * kw * 2 <= steps) kw *= 2;
  return kw;
}

hipError_t launch_small_m(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  const int nt = a.nt;
  if (nt != 1 && !(nt == 2 && a.bits == 4)) return hipErrorInvalidValue;
  if (a.waves != 4 && a.waves != 8 && a.waves != 16) return hipErrorInvalidValue;
  if (a.bm != 1 && a.bm != 2 && a.bm != 4 && a.bm != 8) return hipErrorInvalidValue;
  if (!small_m_fits(a.N, a.K, a.group_size)) return hipErrorInvalidValue;
  // scale bytes per workgroup (the column split's blocks are 8 KB for one or
  // two column blocks per wave)
  const int64_t block = int64_t(16) * nt * (a.cs ? 4 : 1) * (a.K / a.group_size) * 2;
  const bool large = block > (nt == 2 && !a.cs ? kScaleSmall2 : kScaleSmall1);
  if (large && (a.cs || nt != 1 || block > kScaleLarge || a.waves > 8)) return hipErrorInvalidValue;
  if (a.cs && a.waves != 4) return hipErrorInvalidValue;
  // the folded routing needs routed tile heights, one row per pair, the
  // small scale blocks (its LDS scratch) and a decode-sized routing
  if (a.fuse && (large || (a.bm != 4 && a.bm != 8) || a.M != 1 || !a.idx || a.n_pairs > kFuseMaxPairs ||
                 a.E > kFuseMaxExperts || !a.r_offsets || !a.r_perm || !a.r_tiles || !a.r_error))
    return hipErrorInvalidValue;
  const int64_t blocks = ceil_div(a.N, 16 * nt * (a.cs ? 4 : 1)) * a.max_tiles;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int kw = a.waves;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  if (a.bits == 4)
    return a.group_size == 32 ? launch_nt<4, 32>(a, nt, kw, large, grid, s)
                              : launch_nt<4, 64>(a, nt, kw, large, grid, s);
  return a.group_size == 32 ? launch_nt<8, 32>(a, nt, kw, large, grid, s)
                            : launch_nt<8, 64>(a, nt, kw, large, grid, s);
}

}  // namespace mq
