// Routed product against the stored weight applied untransposed (transpose = 0).
//
// What it computes: ml-explore/mlx PR 4023, the coverage reply (its second
// gap, the _nn kernels): the vector-Jacobian product of x . w_hat^T flips the
// transpose, so the backward pass of a quantised MoE layer multiplies by the
// same stored weight untransposed.  Expert e's weight is stored [K, N] and
// quantised along N in groups of group_size:
//     out[t,a,m,n] = sum_k x[t,a',m,k] (s[e,k,n/gs] q[e,k,n] + b[e,k,n/gs]).
//
// Exactness.  The scale now varies along the reduction (one per k and column
// group), so it cannot be applied to a per-group MFMA sum as in the
// transposed kernel.  Instead the product s q of a bf16 scale (8 significant
// bits) and a code (at most 8 bits) is formed exactly in fp32 and split into
// two bf16 values: the high part keeps its leading 8 significant bits (the
// fp32 value with its low 16 bits cleared), the low part is the remainder,
// which has at most 8 significant bits and so is a bf16 value too.  Three
// MFMAs per row block and k-step multiply x by the high part, the low part
// and the bias (broadcast over the 16 columns of a block, which share one
// group): every product is exact, the sums are fp32 and the output is
// rounded to bf16 once.
//
// Layout of one workgroup (4 waves): a tile is BM routed rows of one expert
// (the routing and tile table of the other gathers) x 64 output columns; wave
// w owns columns [16 w, 16 w + 16), BM / 16 MFMA 16x16x32 blocks.  K is walked
// in steps of 64 (two MFMA k-steps).  Per step every thread loads the codes
// of one column (its lane) at two runs of 8 consecutive k (k-octets w and
// w + 4 of the step), their scales, and for its MFMA lane the biases of its
// block's group; it stages the gathered x rows and writes the column's split
// products, k contiguous, to LDS (double buffered, one barrier per step).
// The next step's loads are in flight during the current step's MFMAs; the
// loads are small (4 or 2 bytes) and many, so the step is as long as the
// memory latency allows.
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KSTEP = 64;                        // k per step (two MFMA k-steps)
constexpr int BNC = 64;                          // output columns per tile
constexpr uint32_t kRsrcWord3 = 0x00020000u;     // gfx9 raw buffer descriptor flags
constexpr uint32_t kNoRow = 0x80000000u;         // offset outside every descriptor range

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           int(kRsrcWord3));
}

__device__ inline int uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(int(v)); }

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// upper halves of two fp32 bit patterns -> one bf16 pair (lo in the low half)
__device__ inline uint32_t pack_hi(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

template <int BM, int BITS>
__global__ __launch_bounds__(256) void gather_nn_kernel(GemmArgs a) {
  static_assert(BM == 16 || BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(BITS == 4 || BITS == 8, "bits");
  constexpr int MT = BM / 16;
  constexpr int XP = (BM * 8 + 255) / 256;        // 16-byte x pieces per thread per step
  constexpr int CPW = 32 / BITS;                  // codes per 32-bit word

  // x rows and split products, 128 bytes (64 k) per row or column; 16-byte
  // slot o of row r sits at slot o ^ ((r >> 1) & 7), so that the 16 rows (or
  // columns) of a fragment read fall in distinct 16-byte bank slots
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][BM * 128];
  __shared__ __attribute__((aligned(16))) unsigned char bh[2][BNC * 128];
  __shared__ __attribute__((aligned(16))) unsigned char bl[2][BNC * 128];
  __shared__ int32_t xrow_tab[BM];
  __shared__ int32_t orow_tab[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, c4 = lane >> 4;
  const int K = a.K, N = a.N, gs = a.group_size, G = N / gs;

  // ---- which tile: routed tiles cut into 8 contiguous ranges, one per XCD --------
  const int ntn = (N + BNC - 1) / BNC;
  const int ntiles = a.perm ? min64(a.tiles[a.E], a.max_tiles) : int(a.max_tiles);
  const unsigned per_xcd = unsigned(ntiles * ntn + 7) / 8u;
  if (blockIdx.x / 8u >= per_xcd) return;
  const unsigned logical = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  const int t = int(logical / unsigned(ntn));
  if (t >= ntiles) return;
  const int n0 = int(logical % unsigned(ntn)) * BNC;
  int e = 0;
  int64_t row0, seg_end;
  if (a.perm) {
    // a tile table built for another tile height is not used: nothing is written
    if (*a.tile_bm != BM) return;
    // expert of tile t: the largest e with tiles[e] <= t (two ballot rounds)
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

  // ---- descriptors and per-lane offsets -----------------------------------------
  const int64_t row_bytes = int64_t(N) * BITS / 8;          // one stored row of codes
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq + int64_t(e) * K * (int64_t(N) * BITS / 32),
                                         uint32_t(int64_t(K) * row_bytes));
  const __amdgpu_buffer_rsrc_t sr = rsrc(a.scales + int64_t(e) * K * G, uint32_t(K) * G * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(a.biases + int64_t(e) * K * G, uint32_t(K) * G * 2u);

  // x piece j of this thread: row p / 8, 16-byte piece p % 8 of the step's
  // 128 bytes
  uint32_t xoff[XP];
  int xdst[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    const int p = tid + 256 * j;
    const int r = min(p >> 3, BM - 1), c = p & 7;
    const int32_t row = xrow_tab[r];
    xoff[j] = (p >= BM * 8 || row < 0) ? kNoRow : uint32_t(row) * uint32_t(K) * 2u + uint32_t(c) * 16u;
    xdst[j] = (p >= BM * 8) ? -1 : r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  }
  // this thread's column (lane) and k-octet (wave) for the dequantisation;
  // columns past N read whatever lies there and are never stored
  const int ncol = n0 + lane;
  const uint32_t code_off = uint32_t(ncol / CPW) * 4u;
  const int code_shift = (ncol % CPW) * BITS;
  const uint32_t scale_off = uint32_t(min(ncol / gs, G - 1)) * 2u;
  // this thread's two split-product slots: k-octets wave and wave + 4
  const int bdst0 = lane * 128 + ((wave ^ ((lane >> 1) & 7)) << 4);
  const int bdst1 = lane * 128 + (((wave + 4) ^ ((lane >> 1) & 7)) << 4);
  // this MFMA lane's bias offsets: its block's group, k-octet c4 (k-step 0)
  const int gblk = min((n0 + 16 * wave) / gs, G - 1);
  const uint32_t bias_off = (uint32_t(8 * c4) * uint32_t(G) + uint32_t(gblk)) * 2u;
  // fragment reads: x row 16 mt + l16 and B column 16 wave + l16, k-octet
  // c4 (k-step 0) or c4 + 4 (k-step 1)
  const int ncl = 16 * wave + l16;
  auto xfrag = [&](int ks) { return l16 * 128 + (((c4 + 4 * ks) ^ ((l16 >> 1) & 7)) << 4); };
  auto bfrag = [&](int ks) { return ncl * 128 + (((c4 + 4 * ks) ^ ((ncl >> 1) & 7)) << 4); };

  // ---- one step's loads ---------------------------------------------------------
  u32x4 xv[XP];
  uint32_t cw[16], sv[16], bv[16];
  auto load_step = [&](int st) {
    const uint32_t k0 = uint32_t(st) * KSTEP;
#pragma unroll
    for (int j = 0; j < XP; ++j) xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[j], uni(k0 * 2u), 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t kw = k0 + 32u * uint32_t(h) + 8u * uint32_t(wave);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        cw[8 * h + r] = __builtin_amdgcn_raw_buffer_load_b32(wr, code_off,
                                                             uni((kw + r) * uint32_t(row_bytes)), 0);
        sv[8 * h + r] = __builtin_amdgcn_raw_buffer_load_b16(sr, scale_off,
                                                             uni((kw + r) * uint32_t(G) * 2u), 0);
        bv[8 * h + r] = __builtin_amdgcn_raw_buffer_load_b16(
            br, bias_off + uint32_t(r) * uint32_t(G) * 2u, uni((k0 + 32u * h) * uint32_t(G) * 2u), 0);
      }
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / KSTEP;
  load_step(0);
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    // x rows and the split products of this step to LDS
#pragma unroll
    for (int j = 0; j < XP; ++j)
      if (xdst[j] >= 0) *reinterpret_cast<u32x4*>(&xs[buf][xdst[j]]) = xv[j];
    u32x4 vb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float q = float((cw[8 * h + r] >> code_shift) & ((1u << BITS) - 1u));
        const float p = __uint_as_float(sv[8 * h + r] << 16) * q;   // exact: <= 16 significant bits
        const uint32_t ph = __float_as_uint(p) & 0xFFFF0000u;       // leading 8 significant bits
        hi[r] = ph;
        lo[r] = __float_as_uint(p - __uint_as_float(ph));           // exact remainder, <= 8 bits
      }
      u32x4 vh, vl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vh[i] = pack_hi(hi[2 * i], hi[2 * i + 1]);
        vl[i] = pack_hi(lo[2 * i], lo[2 * i + 1]);
        vb[h][i] = (bv[8 * h + 2 * i] & 0xFFFFu) | (bv[8 * h + 2 * i + 1] << 16);
      }
      *reinterpret_cast<u32x4*>(&bh[buf][h ? bdst1 : bdst0]) = vh;
      *reinterpret_cast<u32x4*>(&bl[buf][h ? bdst1 : bdst0]) = vl;
    }
    // the next step's loads stay in flight during this step's MFMAs
    if (st + 1 < nsteps) load_step(st + 1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 fh = *reinterpret_cast<const u32x4*>(&bh[buf][bfrag(ks)]);
      const u32x4 fl = *reinterpret_cast<const u32x4*>(&bl[buf][bfrag(ks)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(&xs[buf][mt * 2048 + xfrag(ks)]);
        acc[mt] = mfma(af, fh, acc[mt]);
        acc[mt] = mfma(af, fl, acc[mt]);
        acc[mt] = mfma(af, vb[ks], acc[mt]);
      }
    }
  }

  // ---- store: fp32 -> bf16 (nearest even), row r of block mt at its pair's row --------
  const int col = n0 + 16 * wave + l16;
  if (col < N) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * c4 + i;
        if (r < rows)
          a.out[int64_t(orow_tab[r]) * N + col] =
              __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[mt][i]));
      }
  }
}

template <int BM>
hipError_t launch_bm(const GemmArgs& a, hipStream_t s) {
  // padded to a multiple of 8 for the XCD-aware renumbering in the kernel
  const int64_t blocks = ceil_div(ceil_div(a.N, BNC) * a.max_tiles, 8) * 8;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  note_dispatch("gather_nn", {BM, a.bits});
  if (a.bits == 4) gather_nn_kernel<BM, 4><<<grid, dim3(256), 0, s>>>(a);
  else gather_nn_kernel<BM, 8><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_nn(const GemmArgs& a, hipStream_t s) {
  if (a.max_tiles <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % KSTEP || a.N % a.group_size || (a.bits != 4 && a.bits != 8)) return hipErrorInvalidValue;
  switch (a.bm) {
    case 16: return launch_bm<16>(a, s);
    case 32: return launch_bm<32>(a, s);
    case 64: return launch_bm<64>(a, s);
    default: return launch_bm<128>(a, s);
  }
}

}  // namespace mq
