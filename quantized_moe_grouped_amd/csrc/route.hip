// Device-side routing: expert histogram, prefix scan, stable scatter, in one
// launch that also computes the per-group row sums of x for the GEMM.
//
// lablup/mlxcel issue 629, "Implementation plan" 4b: sort tokens by expert on
// the device before the grouped call so that each expert sees one contiguous
// block (its step 2 suspects a serialising host-side sort; nothing here touches
// the host).  ml-explore/mlx PR 4023 walks exactly such a sorted index array.
//
// Two launches (one for at most 1024 pairs), no host synchronisation, no
// inter-workgroup waiting:
//   route_count    one workgroup per 1024 consecutive pairs builds a histogram
//                  over E+1 bins in LDS (bin E collects indices outside
//                  [0, E)) and writes it to counts[block][*];
//   route_scatter  workgroup b re-reads the (small) count table, forms the
//                  exclusive scan over experts (segment offsets) plus its own
//                  per-expert base (counts of earlier blocks), then ranks its
//                  pairs stably: wavefront match masks give the rank among
//                  equal experts inside a wave, an LDS table the rank across
//                  the 4 waves, and a per-expert cursor carries it across the
//                  chunk's four rounds.  Workgroup 0 also writes offsets, the
//                  GEMM's tile table and the error word.  The same launch
//                  carries the row-sum workgroups: one thread per (x row,
//                  group) sums the group's x values in fp32 and stores three
//                  bf16 parts whose sum is the row sum to 2^-24 (the GEMM's
//                  bias and offset terms multiply them exactly).
// The routing result is unique (a stable sort), so it is bit-exact with the
// oracle.
#include "mq_internal.h"

namespace mq {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kRouteThreads / 64;
constexpr int kRounds = kRouteChunk / kRouteThreads;

// Exclusive scan of v[0..len) in place (LDS), returns the total.  All threads
// of the block must call it.
__device__ int32_t block_exclusive_scan(int32_t* v, int len, int32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (len + kRouteThreads - 1) / kRouteThreads;
  const int beg = min(tid * per, len), end = min(beg + per, len);
  int32_t local = 0;
  for (int i = beg; i < end; ++i) local += v[i];
  // inclusive scan of `local` across the wave
  int32_t inc = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) before += wave_tot[w];
    total += wave_tot[w];
  }
  int32_t run = before + inc - local;
  for (int i = beg; i < end; ++i) {
    const int32_t c = v[i];
    v[i] = run;
    run += c;
  }
  __syncthreads();
  return total;
}

// lanes of this wave whose bin equals this lane's (among lanes with `valid`)
__device__ inline uint64_t match_peers(int e, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t m = __ballot(set);
    peers &= set ? m : ~m;
  }
  return peers;
}

__device__ inline float dot2_ones(uint32_t v, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), c, false);
}

// fp32 -> three bf16 parts whose sum equals v to within 2^-24 relative (each
// part is the round-to-nearest-even of the remainder left by the ones before)
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

// Row sums of x per quantisation group: sums[(row * 3 + part) * Gp + g],
// zero for g >= G.  Thread i of the row-sum workgroups owns (row, g).
template <int GS>
__device__ void row_sums(const RowSumArgs& s, int64_t i) {
  if (i >= s.xrows * s.Gp) return;
  const int64_t row = i / s.Gp;
  const int g = int(i - row * s.Gp);
  float acc = 0.f;
  if (g < s.G) {
    const u32x4* p = reinterpret_cast<const u32x4*>(s.x + row * s.K + int64_t(g) * GS);
    u32x4 v[GS / 8];
#pragma unroll
    for (int q = 0; q < GS / 8; ++q) v[q] = p[q];
#pragma unroll
    for (int q = 0; q < GS / 8; ++q) {
      acc = dot2_ones(v[q][0], acc);
      acc = dot2_ones(v[q][1], acc);
      acc = dot2_ones(v[q][2], acc);
      acc = dot2_ones(v[q][3], acc);
    }
  }
  uint16_t h, m, l;
  split3(acc, h, m, l);
  uint16_t* o = s.sums + row * 3 * s.Gp + g;
  o[0] = h;
  o[s.Gp] = m;
  o[2 * s.Gp] = l;
}

// This thread's indices of chunk [base, base + kRouteChunk): unconditional
// loads of clamped positions, all issued before any is used (base < n).
__device__ inline void chunk_indices(const int32_t* __restrict__ idx, int64_t n, int64_t base,
                                     int (&ev)[kRounds]) {
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    ev[r] = idx[min64(base + r * kRouteThreads + threadIdx.x, n - 1)];
}

// Adds the pairs of chunk [base, base + kRouteChunk) (this thread's indices in
// ev) to hist (LDS, E + 1 bins, zeroed by the caller): one LDS add per
// distinct bin of each wave's 64 pairs, since sorted indices would otherwise
// send most adds to one counter.  Every thread of the block calls it.
__device__ void chunk_histogram(const int (&ev)[kRounds], int64_t n, int32_t E, int64_t base,
                                int32_t* hist) {
  if (base >= n) return;
  const int bins = E + 1;
  int nbits = 0;
  while ((1 << nbits) < bins) ++nbits;
  const uint64_t lt_mask = (uint64_t(1) << (threadIdx.x & 63)) - 1;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const bool valid = base + r * kRouteThreads + threadIdx.x < n;
    int e = ev[r];
    if (uint32_t(e) >= uint32_t(E)) e = E;
    const uint64_t peers = match_peers(e, valid, nbits);
    if (valid && __popcll(peers & lt_mask) == 0) atomicAdd(&hist[e], __popcll(peers));
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_count(const int32_t* __restrict__ idx,
                                                              int64_t n, int32_t E,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t hist[kMaxExperts + 1];
  const int bins = E + 1;
  const int64_t base = int64_t(blockIdx.x) * kRouteChunk;
  int ev[kRounds];
  chunk_indices(idx, n, base, ev);
  for (int e = threadIdx.x; e < bins; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  chunk_histogram(ev, n, E, base, hist);
  __syncthreads();
  for (int e = threadIdx.x; e < bins; e += kRouteThreads)
    counts[int64_t(blockIdx.x) * bins + e] = hist[e];
}

template <int MAXB>
__device__ void route_block(const RouteArgs& a, int blk, int nblk) {
  __shared__ int32_t s_off[MAXB];       // totals, then segment offsets
  __shared__ int32_t s_cur[MAXB];       // pairs before this chunk, then the next free slot
  __shared__ int32_t s_wcnt[kWaves][MAXB];
  __shared__ int32_t s_tmp[kWaves];

  const int bins = a.E + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < bins) ++nbits;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int64_t base = int64_t(blk) * kRouteChunk;
  // this chunk's indices, loaded first so that their latency overlaps the
  // count table's.  A workgroup whose chunk starts at or past n (only
  // workgroup 0 of an empty routing) has nothing to place and must not touch
  // idx (it may be null).
  int ev[kRounds];
  if (base < a.n) chunk_indices(a.idx, a.n, base, ev);

  // totals and the counts of earlier chunks, per bin.  A routing of a single
  // chunk (up to kRouteChunk pairs, e.g. a decode step) counts its own chunk
  // here and needs no count launch.
  if (nblk == 1) {
    for (int e = tid; e < bins; e += kRouteThreads) {
      s_off[e] = 0;
      s_cur[e] = 0;
      for (int w = 0; w < kWaves; ++w) s_wcnt[w][e] = 0;
    }
    __syncthreads();
    chunk_histogram(ev, a.n, a.E, base, s_off);
  }
  // Otherwise sixteen rows of the count table are loaded before any is added
  // (the loop is bound by load latency, and a load under a condition would
  // be waited for on its own).
  if (nblk > 1) {
    for (int e = tid; e < bins; e += kRouteThreads) {
      int32_t tot = 0, before = 0;
      constexpr int U = 16;
      for (int b0 = 0; b0 < nblk; b0 += U) {
        int32_t c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = a.counts[int64_t(min(b0 + u, nblk - 1)) * bins + e];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int b = b0 + u;
          const int32_t v = b < nblk ? c[u] : 0;
          tot += v;
          before += b < blk ? v : 0;
        }
      }
      s_off[e] = tot;
      s_cur[e] = before;
      for (int w = 0; w < kWaves; ++w) s_wcnt[w][e] = 0;
    }
  }
  __syncthreads();

  // The out-of-range bin E is scanned last, so its offset is the number of
  // valid pairs and its pairs land at the tail of perm.
  const int32_t invalid = s_off[a.E];
  block_exclusive_scan(s_off, bins, s_tmp);

  if (blk == 0) {
    for (int e = tid; e < bins; e += kRouteThreads) a.offsets[e] = s_off[e];
    if (tid == 0 && a.error) {
      a.error[0] = invalid;
      a.error[1] = a.tiles ? a.bm : 0;
    }
    if (a.tiles) {
      // tile tables, each a prefix over the experts e' < e of their rows r,
      // with h = bm / 2 for bm >= 64 (else 0): row 0 ceil(r / bm) (tiles of
      // bm rows); row 1 floor(r / bm) + [r % bm > h] (the tiles of bm rows
      // when the last h rows or fewer of a segment go to a tail tile); row 2
      // [0 < r % bm <= h] (those tail tiles)
      // (the three tables side by side, one scan over all of them: table k's
      // prefix is the scan minus its value at the table's start)
      int32_t* t = &s_wcnt[0][0];          // reused as scratch (zero again below)
      static_assert(kWaves >= 3, "three tables in the per-wave count rows");
      const int64_t h = a.bm >= 64 ? a.bm / 2 : 0;
      for (int e = tid; e < bins; e += kRouteThreads) {
        const int64_t rows = e < a.E ? int64_t(s_off[e + 1] - s_off[e]) * a.rows_per_pair : 0;
        const int64_t rest = rows % a.bm;
        t[e] = int32_t((rows + a.bm - 1) / a.bm);
        t[bins + e] = int32_t(rows / a.bm + (rest > h ? 1 : 0));
        t[2 * bins + e] = int32_t(rest > 0 && rest <= h ? 1 : 0);
      }
      __syncthreads();
      block_exclusive_scan(t, 3 * bins, s_tmp);
      for (int i = tid; i < 3 * bins; i += kRouteThreads) a.tiles[i] = t[i] - t[i / bins * bins];
      __syncthreads();
      for (int i = tid; i < 3 * bins; i += kRouteThreads) t[i] = 0;
    }
  }
  for (int e = tid; e < bins; e += kRouteThreads) s_cur[e] += s_off[e];
  __syncthreads();

  // ---- stable scatter of this chunk ------------------------------------------------
  if (base >= a.n) return;
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = base + r * kRouteThreads + tid;
    const bool valid = i < a.n;
    int e = ev[r];
    if (uint32_t(e) >= uint32_t(a.E)) e = a.E;
    const uint64_t peers = match_peers(e, valid, nbits);
    const int rank = __popcll(peers & lt_mask);
    const bool leader = valid && rank == 0;
    if (leader) s_wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int32_t pos = s_cur[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
      if (pos >= 0 && pos < a.n) a.perm[pos] = int32_t(i);
      if (e == a.E && a.out) {
        uint16_t* row = a.out + i * a.out_row_elems;
        for (int64_t k = 0; k < a.out_row_elems; ++k) row[k] = 0;
      }
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&s_cur[e], s_wcnt[wave][e]);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// Workgroups [0, route_blocks) route (route_blocks is the grid of route_count);
// the rest compute row sums.
template <int MAXB>
__global__ __launch_bounds__(kRouteThreads) void route_scatter(RouteArgs a, RowSumArgs s,
                                                               int route_blocks) {
  if (int(blockIdx.x) < route_blocks) {
    route_block<MAXB>(a, blockIdx.x, route_blocks);
    return;
  }
  const int64_t i = int64_t(blockIdx.x - route_blocks) * kRouteThreads + threadIdx.x;
  if (s.group_size == 32) row_sums<32>(s, i);
  else row_sums<64>(s, i);
}

}  // namespace

hipError_t launch_route(const RouteArgs* a, const RowSumArgs* s, hipStream_t stream) {
  const int64_t rblocks = a ? route_blocks(a->n) : 0;
  const int64_t sthreads = s ? s->xrows * s->Gp : 0;
  const int64_t sblocks = ceil_div(sthreads, kRouteThreads);
  const int64_t blocks = rblocks + sblocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  RouteArgs ra{};
  if (a) {
    ra = *a;
    // a single chunk is counted by its routing workgroup itself
    if (rblocks > 1) {
      note_dispatch("route_count", {});
      route_count<<<dim3(unsigned(rblocks)), dim3(kRouteThreads), 0, stream>>>(a->idx, a->n, a->E,
                                                                               a->counts);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  RowSumArgs rs{};
  if (s) rs = *s;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  note_dispatch("route_scatter", {!a || a->E < 257 ? 257 : kMaxExperts + 1});
  if (!a || a->E < 257)
    route_scatter<257><<<grid, dim3(kRouteThreads), 0, stream>>>(ra, rs, int(rblocks));
  else
    route_scatter<kMaxExperts + 1><<<grid, dim3(kRouteThreads), 0, stream>>>(ra, rs, int(rblocks));
  return hipGetLastError();
}

}  // namespace mq
