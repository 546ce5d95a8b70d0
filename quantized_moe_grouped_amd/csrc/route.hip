// Device-side routing: expert histogram, prefix scan, stable scatter.
//
// lablup/mlxcel issue 629, "Implementation plan" 4b: sort tokens by expert on
// the device before the grouped call so that each expert sees one contiguous
// block (its step 2 suspects a serialising host-side sort; nothing here touches
// the host).  ml-explore/mlx PR 4023 walks exactly such a sorted index array.
//
// Two launches, no host synchronisation:
//   route_count    one workgroup per 1024 consecutive pairs builds a
//                  histogram over E+1 bins in LDS (bin E collects indices
//                  outside [0, E)) and writes it to counts[block][*];
//   route_scatter  each workgroup re-reads the (small) count table, forms the
//                  exclusive scan over experts (segment offsets) plus its own
//                  per-expert base (counts of earlier blocks), then ranks its
//                  pairs stably: wavefront ballots give the rank among equal
//                  experts inside a wave, an LDS table the rank across the 4
//                  waves, and a per-expert cursor carries it across the block's
//                  four rounds.  Workgroup 0 also writes offsets, the tile
//                  table for the GEMM and the error word.
// The result is unique (a stable sort), so it is bit-exact with the oracle.
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kWaves = kRouteThreads / 64;
constexpr int kRounds = kRouteChunk / kRouteThreads;
constexpr int kMaxBins = 2049;  // E <= 2048, plus the out-of-range bin

__global__ __launch_bounds__(kRouteThreads) void route_count(const int32_t* __restrict__ idx,
                                                              int64_t n, int32_t E,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t hist[kMaxBins];
  const int bins = E + 1;
  for (int e = threadIdx.x; e < bins; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kRouteChunk;
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = base + r * kRouteThreads + threadIdx.x;
    if (i < n) {
      int e = idx[i];
      if (uint32_t(e) >= uint32_t(E)) e = E;
      atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < bins; e += kRouteThreads)
    counts[int64_t(blockIdx.x) * bins + e] = hist[e];
}

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

__global__ __launch_bounds__(kRouteThreads) void route_scatter(RouteArgs a) {
  __shared__ int32_t s_off[kMaxBins];     // segment offsets (exclusive scan of totals)
  __shared__ int32_t s_cur[kMaxBins];     // this block's next free slot per expert
  __shared__ int32_t s_wcnt[kWaves][kMaxBins];
  __shared__ int32_t s_tmp[kWaves];

  const int bins = a.E + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = gridDim.x;

  for (int e = tid; e < bins; e += kRouteThreads) {
    int32_t tot = 0, before = 0;
    for (int b = 0; b < nblk; ++b) {
      const int32_t c = a.counts[int64_t(b) * bins + e];
      before += (b < int(blockIdx.x)) ? c : 0;
      tot += c;
    }
    s_off[e] = tot;
    s_cur[e] = before;
    for (int w = 0; w < kWaves; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();
  // The out-of-range bin E is scanned last, so its offset is the number of
  // valid pairs and its pairs land at the tail of perm.
  const int32_t invalid = s_off[a.E];
  block_exclusive_scan(s_off, bins, s_tmp);

  if (blockIdx.x == 0) {
    for (int e = tid; e < bins; e += kRouteThreads) a.offsets[e] = s_off[e];
    if (tid == 0 && a.error) {
      a.error[0] = invalid;
      a.error[1] = a.tiles ? a.bm : 0;
    }
    if (a.tiles) {
      // tile table: tiles[e] = sum over e' < e of ceil(rows(e') / bm)
      int32_t* t = &s_wcnt[0][0];          // reuse as scratch (zero again below)
      for (int e = tid; e < bins; e += kRouteThreads) {
        const int64_t rows =
            e < a.E ? int64_t(s_off[e + 1] - s_off[e]) * a.rows_per_pair : 0;
        t[e] = int32_t((rows + a.bm - 1) / a.bm);
      }
      __syncthreads();
      block_exclusive_scan(t, bins, s_tmp);
      for (int e = tid; e < bins; e += kRouteThreads) {
        a.tiles[e] = t[e];
        t[e] = 0;
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < bins; e += kRouteThreads) s_cur[e] += s_off[e];
  __syncthreads();

  int nbits = 0;
  while ((1 << nbits) < bins) ++nbits;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int64_t base = int64_t(blockIdx.x) * kRouteChunk;
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = base + r * kRouteThreads + tid;
    const bool valid = i < a.n;
    int e = 0;
    if (valid) {
      e = a.idx[i];
      if (uint32_t(e) >= uint32_t(a.E)) e = a.E;
    }
    // lanes of this wave holding the same bin
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
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

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int64_t blocks = route_blocks(a.n);
  route_count<<<dim3(unsigned(blocks)), dim3(kRouteThreads), 0, s>>>(a.idx, a.n, a.E, a.counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  route_scatter<<<dim3(unsigned(blocks)), dim3(kRouteThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mq
