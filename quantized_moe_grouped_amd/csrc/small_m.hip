// Weight-reusing small-M path: row tiles of at most 8 rows against a quantised
// weight, each weight byte read from memory once.
//
// lablup/mlxcel issue 725, "The gap" and "What's needed": batched decode with
// B <= 8 rows must not re-read the whole weight per row (per-row matrix-vector
// kernels make the traffic O(B)), and a 128-row tile wastes ~94% of its work
// at M = 8.  Here one workgroup owns NT blocks of 16 output columns of one row
// tile (dense: the M rows; gathered: the <= 8 routed rows of one expert) and
// its KW waves split K.  Every code, scale and bias of those columns is loaded
// once and applied to all rows of the tile.  The work is HBM-bound: each wave
// keeps the weights of D steps in flight and never waits on another wave.
//
// One MFMA k-step (v_mfma_f32_16x16x32_bf16, 16 rows x 16 columns x 32 k).
// Lane (l16, c4) holds 8 consecutive codes of column l16 in the B operand.  A
// wave step covers SK consecutive k of its columns; quarters c4 = 0, 1 hold the
// first half of them and quarters 2, 3 the second half, and each half lies in
// one quantisation group.  The 16 rows of the A operand are (half, x row):
// rows 0-7 carry the tile's 8 x rows on the first half's k slots and zeros on
// the others, rows 8-15 the same x rows on the second half's slots.  One MFMA
// therefore gives the group partial sums of both halves for all 8 rows, and
// output lane (column, c4) holds rows 4c4..4c4+3, all of one half: it applies
// the scale and bias it loaded itself.  The per-half row sums of x (for the
// bias and the code offset) come from an MFMA of the same A against ones.
//
// Arithmetic is the GEMM's (exact codes, per-group fp32 epilogue): per group
// P = x . (off + q) and X = x . 1, then acc += s P + (b - off s) X.  Partial
// sums of the waves and of the two halves meet in LDS in a fixed order, so
// results are deterministic.
//
// x goes from memory straight into LDS (buffer_load ... lds), a ring of D
// slots per wave laid out [16-byte chunk][row] so that one fragment read per
// k-step is free of bank conflicts; A lanes that carry zeros read a shared
// zero block.
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
constexpr int TR = 8;                            // rows per tile
constexpr int D = 4;                             // steps in flight per wave
constexpr int ZERO_BYTES = 512;                  // zero block: 4 k-steps x 128-byte stride

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

// 8 four-bit codes (nibbles 0..7 = k0..k7) -> bf16 (128 + q) pairs in natural
// order; mask 0x000F000F and base 0x43004300 come in registers (a VOP3
// instruction takes no literal)
__device__ inline u32x4 decode4(uint32_t w, uint32_t mask, uint32_t base) {
  const uint32_t w4 = w >> 4;
  u32x4 r;
  r[0] = (__builtin_amdgcn_perm(w4, w, 0x0C040C00u) & mask) | base;
  r[1] = (__builtin_amdgcn_perm(w4, w, 0x0C050C01u) & mask) | base;
  r[2] = (__builtin_amdgcn_perm(w4, w, 0x0C060C02u) & mask) | base;
  r[3] = (__builtin_amdgcn_perm(w4, w, 0x0C070C03u) & mask) | base;
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

// Geometry of one wave step for a code format.
template <int BITS, int GS>
struct Step {
  static constexpr int LB = (BITS == 4 && GS == 32) ? 8 : 16;  // code bytes per lane
  static constexpr int CPL = LB * 8 / BITS;       // codes per lane: 32 or 16
  static constexpr int SK = 4 * CPL;              // k per step: 128 or 64
  static constexpr int JS = CPL / 8;              // MFMA k-steps per step: 4 or 2
  static constexpr int RB = SK * 2;               // bytes of one x row per step
  static constexpr int SLOT = TR * RB;            // LDS bytes of one step's x rows
  static constexpr int XI = SLOT / 1024;          // 1 KB copies per step: 2 or 1
  static constexpr int GPS = SK / GS;             // groups per step: 2, or 1 (8-bit gs64)
  static constexpr int HG = SK / 2 / GS;          // group of the second half: +1 or +0
  static_assert(SK / 2 <= GS && GS % (SK / 2) == 0, "a half lies in one group");
  static_assert(JS * 128 <= ZERO_BYTES && XI >= 1, "step layout");
};

template <int BITS, int GS, int KW, int NT>
__global__ __launch_bounds__(64 * KW, 4) void small_m_kernel(GemmArgs a) {
  using St = Step<BITS, GS>;
  constexpr int LB = St::LB, SK = St::SK, JS = St::JS, RB = St::RB, SLOT = St::SLOT;
  constexpr int XI = St::XI, GPS = St::GPS, HG = St::HG;
  constexpr float OFF = BITS == 4 ? 128.0f : 0.0f;
  typedef typename std::conditional<LB == 16, u32x4, u32x2>::type codes_t;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[KW * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[KW * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[KW * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[KW * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t zeros[ZERO_BYTES];
  static_assert(D == 4 && NT <= 2, "four ring slots; partials of block j go to slot j");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, G = K / GS;
  const int cbs = (N + 16 * NT - 1) / (16 * NT);

  const int t = int(blockIdx.x / unsigned(cbs));
  const int n0 = int(blockIdx.x % unsigned(cbs)) * 16 * NT;
  if (t >= a.max_tiles) return;
  int e = 0;
  int64_t row0, seg_end;
  if (a.perm) {
    if (*a.tile_bm != TR) return;               // workspace routed for another tiling
    if (t >= a.tiles[a.E]) return;
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tiles[mid] <= t) lo = mid; else hi = mid;
    }
    e = __builtin_amdgcn_readfirstlane(lo);
    const int64_t nrows = a.n_pairs * a.M;
    row0 = min<int64_t>(max<int64_t>(int64_t(a.offsets[e]) * a.M, 0) + int64_t(t - a.tiles[e]) * TR,
                        nrows);
    seg_end = min<int64_t>(max<int64_t>(int64_t(a.offsets[e + 1]) * a.M, 0), nrows);
  } else {
    row0 = int64_t(t) * TR;
    seg_end = a.n_pairs * a.M;
  }
  if (row0 >= seg_end) return;
  const int rows = int(min<int64_t>(TR, seg_end - row0));

  // ---- x rows of the tile ------------------------------------------------------------
  // byte offset of x row r of the tile (kNoRow past the tile: the copy writes zeros)
  auto x_row_bytes = [&](int r) -> uint32_t {
    if (r >= rows) return kNoRow;
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
    return uint32_t(xrow * K * 2);
  };
  // copy i of a step: LDS chunk position 8q + b (16 bytes each) <- x row b,
  // chunk q of the step, for lane L = 8q + b - 64 i
  // With 128-k steps and K = 64 mod 128 the last step's second half lies past
  // K: its chunks are copied from offsets outside the buffer, i.e. as zeros,
  // so the A operand is zero there whatever the codes.
  const int S = (K + SK - 1) / SK;
  const bool ragged = (K % SK) != 0;
  uint32_t xv[XI], xv_last[XI];
  {
    const uint32_t rb = x_row_bytes(lane & 7);
    const int q_last = (K - (S - 1) * SK) / 8;         // chunks of the last step inside K
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int q = 8 * i + (lane >> 3);
      xv[i] = rb == kNoRow ? kNoRow : rb + 16u * uint32_t(q);
      xv_last[i] = q < q_last ? xv[i] : kNoRow;
    }
  }

  // ---- weight offsets ----------------------------------------------------------------
  const int64_t wrow_bytes = int64_t(K) * BITS / 8;
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq + int64_t(e) * N * (K * BITS / 32),
                                         uint32_t(int64_t(N) * wrow_bytes));
  const __amdgpu_buffer_rsrc_t sr = rsrc(a.scales + int64_t(e) * N * G, uint32_t(N) * G * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(a.biases + int64_t(e) * N * G, uint32_t(N) * G * 2u);
  // descriptors of a step past the wave's range: every access reads zeros and
  // moves no memory, so loads are issued unconditionally
  const __amdgpu_buffer_rsrc_t none = rsrc(a.x, 0u);
  const int half = c4 >> 1;
  // ---- steps of this wave ----------------------------------------------------------
  const int per = (S + KW - 1) / KW;
  const int s_lo = min(S, wave * per), s_hi = min(S, s_lo + per);

  // Scales and biases are fetched once per round of D steps, as dwords at
  // 4-byte offsets from the expert's block.  Lane (column n, half h) needs the
  // value of one group per step: with two groups per step these are every
  // other value, i.e. the same half (the lane's parity) of D consecutive
  // dwords; with one group per step they are D consecutive values, brought to
  // a dword boundary with a funnel shift.  A dword never straddles the end of
  // the block because the block holds an even number of values (N * G even is
  // a condition of this path).
  constexpr int SV = GPS == 2 ? D : 4;             // dwords of one round's run
  typedef u32x4 scales_t;
  uint32_t woff[NT], soff[NT], spar[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(n0 + 16 * j + l16, N - 1);
    woff[j] = uint32_t(n * wrow_bytes) + uint32_t(LB) * c4;
    if constexpr (GPS == 2) {
      const uint32_t e0 = uint32_t(n) * G + uint32_t(half);      // value at step 0
      soff[j] = (e0 >> 1) * 4u;
      spar[j] = e0 & 1u;
    } else {
      // rounds start at steps of the parity of s_lo (D is even)
      const uint32_t e0 = uint32_t(n) * G + uint32_t(s_lo & 1);
      soff[j] = (e0 >> 1) * 4u;
      spar[j] = (uint32_t(n) * G + uint32_t(s_lo)) & 1u;
    }
  }
  static_assert(SV == 4 && D % 2 == 0, "scale runs");

  // ---- LDS fragment addresses ----------------------------------------------------
  // A lane (row l16, quarter c4) carries x row (l16 & 7) when its row half
  // (l16 >> 3) is the half its k slots belong to (c4 >> 1); else zeros.
  const bool alive = (l16 >> 3) == half;
  const uint32_t frag = uint32_t(128 * JS * c4 + 16 * (l16 & 7));
  // the ring arrays by slot (a switch, not a table: the addresses stay
  // constants of the kernel instead of a table in memory)
  auto ring_of = [&](int d) -> uint8_t* {
    return d == 0 ? ring0 : d == 1 ? ring1 : d == 2 ? ring2 : ring3;
  };
  uint8_t* rings[D];
#pragma unroll
  for (int d = 0; d < D; ++d) rings[d] = ring_of(d) + wave * SLOT;
  // Both kinds of address are offsets from the slot's own ring array, so the
  // compiler ties each fragment read to the copies into that array alone.
  uint32_t voff[D];
#pragma unroll
  for (int d = 0; d < D; ++d) voff[d] = alive ? frag : uint32_t(zeros - rings[d]);
  // the wave's own zero block writes precede its own reads (LDS keeps a
  // wave's order); every wave writes the same zeros
  if (lane < ZERO_BYTES / 16) reinterpret_cast<u32x4*>(zeros)[lane] = u32x4{0u, 0u, 0u, 0u};
  asm volatile("" ::: "memory");

  codes_t cw[D][NT];
  scales_t sv_next[NT], bv_next[NT];
  auto issue = [&](int st, int d) {
    const bool live = st < s_hi;
    const __amdgpu_buffer_rsrc_t xr_ = live ? xr : none;
    const __amdgpu_buffer_rsrc_t wr_ = live ? wr : none;
    const __amdgpu_buffer_rsrc_t sr_ = live ? sr : none;
    const __amdgpu_buffer_rsrc_t br_ = live ? br : none;
    const bool last = ragged && st == S - 1;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr_, (lds_ptr)(rings[d] + 1024 * i), 16,
                                               int(last ? xv_last[i] : xv[i]),
                                               uni(uint32_t(st) * RB), 0, 0);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (LB == 16)
        cw[d][j] = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[j], uni(uint32_t(st) * 4 * LB), 0);
      else
        cw[d][j] = __builtin_amdgcn_raw_buffer_load_b64(wr_, woff[j], uni(uint32_t(st) * 4 * LB), 0);
    }
    // a round starts with slot 0: its scales and biases come with it (dword
    // offset of the round: st with two groups per step, (st - (s_lo & 1)) / 2
    // with one)
    if (d == 0) {
      const uint32_t rs = GPS == 2 ? uint32_t(st) * 4u : uint32_t(st - (s_lo & 1)) * 2u;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        sv_next[j] = __builtin_amdgcn_raw_buffer_load_b128(sr_, soff[j], uni(rs), 0);
        bv_next[j] = __builtin_amdgcn_raw_buffer_load_b128(br_, soff[j], uni(rs), 0);
      }
    }
  };
  // the run as D dwords whose upper halves are the bf16 values of the steps
  // of the round (fp32 bit patterns once the lower half is cleared)
  uint32_t psel[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) psel[j] = spar[j] ? 0x03020C0Cu : 0x01000C0Cu;
  auto run_values = [&](const scales_t& v, int j, float (&f)[D]) {
    if constexpr (GPS == 2) {
#pragma unroll
      for (int d = 0; d < D; ++d) f[d] = __uint_as_float(__builtin_amdgcn_perm(v[d], v[d], psel[j]));
    } else {
      const uint32_t sh = spar[j] * 16u;
      const uint32_t w0 = __builtin_amdgcn_alignbit(v[1], v[0], sh);
      const uint32_t w1 = __builtin_amdgcn_alignbit(v[2], v[1], sh);
      f[0] = __uint_as_float(w0 << 16);
      f[1] = __uint_as_float(w0 & 0xFFFF0000u);
      f[2] = __uint_as_float(w1 << 16);
      f[3] = __uint_as_float(w1 & 0xFFFF0000u);
    }
  };

  uint32_t dmask, dbase;
  asm("s_mov_b32 %0, 0x000f000f" : "=s"(dmask));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(dbase));
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A counted loop over rounds of D steps with no early exit: the steps past
  // the wave's range read zeros through the empty descriptor and add nothing.
  // (An exit from inside the round would add never-taken paths from a step's
  // issue back to its compute, and the compiler's wait counts follow every
  // path.)
  const int rounds = (s_hi - s_lo + D - 1) / D;
  // (the scheduler keeps each step's loads together and in step order, so the
  // wait counts above hold on the first round as on the others)
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(s_lo + d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One round of D steps; every round but the last issues the loads of the
  // next round as its steps free their slots.  (A load through the empty
  // descriptor moves no memory but costs the load path as much as a real
  // one, so the last round issues none.)
  auto round = [&](int it, auto more) {
    float sf[NT][D], bf[NT][D];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      run_values(sv_next[j], j, sf[j]);
      run_values(bv_next[j], j, bf[j]);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s_lo + it * D + d;
      f32x4 P[NT], X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NT; ++j) P[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < JS; ++ks) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(rings[d] + voff[d] + 128 * ks);
        X = mfma(A, ones, X);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          u32x4 bfrag;
          if constexpr (BITS == 4) bfrag = decode4(cw[d][j][ks], dmask, dbase);
          else bfrag = decode8(cw[d][j][2 * ks], cw[d][j][2 * ks + 1]);
          P[j] = mfma(A, bfrag, P[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float s = sf[j][d];
        const float c = bf[j][d] - OFF * s;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(s, P[j][q], fmaf(c, X[q], acc[j][q]));
      }
      if constexpr (decltype(more)::value) {
        __builtin_amdgcn_sched_barrier(0);
        issue(st + D, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int it = 0; it + 1 < rounds; ++it) round(it, std::true_type{});
  if (rounds > 0) round(rounds - 1, std::false_type{});

  // ---- reduce the waves' and halves' partial sums in a fixed order, store ----------
  // every copy of this wave has landed before its ring is reused
  wait_vmem<0>();
  // wave w's partials of column block j: [column][row 0..15] floats in its ring slot j
#pragma unroll
  for (int j = 0; j < NT; ++j)
    *reinterpret_cast<f32x4*>(rings[j] + (l16 * 16 + 4 * c4) * 4) = acc[j];
  __syncthreads();
  if (tid < NT * 16 * TR) {
    const int j = tid / (16 * TR), c = (tid / TR) % 16, r = tid % TR;
    const uint8_t* const base = j == 0 ? ring0 : ring1;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const float* p = reinterpret_cast<const float*>(base + w * SLOT) + c * 16;
      sum += p[r];
      sum += p[8 + r];
    }
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
  if (kw == 16) small_m_kernel<BITS, GS, 16, NT><<<grid, dim3(1024), 0, s>>>(a);
  else if (kw == 8) small_m_kernel<BITS, GS, 8, NT><<<grid, dim3(512), 0, s>>>(a);
  else small_m_kernel<BITS, GS, 4, NT><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_nt(const GemmArgs& a, int nt, int kw, dim3 grid, hipStream_t s) {
  if constexpr (BITS == 4)
    if (nt == 2) return launch_kw<BITS, GS, 2>(a, kw, grid, s);
  return launch_kw<BITS, GS, 1>(a, kw, grid, s);
}

}  // namespace

int small_m_rows() { return TR; }

// Column blocks of 16 per wave: for 4-bit codes two when that still leaves
// >= 256 workgroups (a wave's x copies, fragments and row sums serve all its
// column blocks).  8-bit codes carry twice the bytes per k, so one block
// already gives the same x bytes per code byte (and two would not fit in 128
// VGPRs).
int small_m_cols(int64_t N, int64_t tiles, int bits) {
  return bits == 4 && ceil_div(N, 16) * tiles >= 512 ? 2 : 1;
}

// Waves per workgroup (splitting K): enough for ~3 waves per SIMD over the
// chip, as long as each wave keeps >= 2 steps.
int small_m_waves(int64_t blocks, int64_t K, int bits, int group_size) {
  const int64_t sk = (bits == 4 && group_size == 64) ? 128 : 64;
  const int64_t steps = ceil_div(K, sk);
  int kw = 4;
  while (kw < 16 && blocks * kw < 3072 && 2 * kw * 2 <= steps) kw *= 2;
  return kw;
}

hipError_t launch_small_m(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  const int nt = a.nt;
  if (nt != 1 && !(nt == 2 && a.bits == 4)) return hipErrorInvalidValue;
  if (a.waves != 4 && a.waves != 8 && a.waves != 16) return hipErrorInvalidValue;
  const int64_t blocks = ceil_div(a.N, 16 * nt) * a.max_tiles;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int kw = a.waves;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  if (a.bits == 4)
    return a.group_size == 32 ? launch_nt<4, 32>(a, nt, kw, grid, s) : launch_nt<4, 64>(a, nt, kw, grid, s);
  return a.group_size == 32 ? launch_nt<8, 32>(a, nt, kw, grid, s) : launch_nt<8, 64>(a, nt, kw, grid, s);
}

}  // namespace mq
