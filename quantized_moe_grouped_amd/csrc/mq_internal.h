// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units.  Host-only; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

namespace mq {

// int64 minimum and maximum.  (In device code `min<int64_t>(a, b)` with an
// int b, or `max<int64_t>(a, 0)`, resolves to a double overload: the result
// is then a double, and an integer division of it is not one.)
__host__ __device__ constexpr int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ constexpr int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// MQ_LOG=1 (read on every call): one stderr line per kernel launch naming the
// template instance launched, "[mq-dispatch] kernel<p0,p1,...>".
void note_dispatch(const char* kernel, std::initializer_list<int> params);

// Pairs handled by one routing workgroup (256 threads x 4 pairs each).
constexpr int kRouteChunk = 1024;
constexpr int kRouteThreads = 256;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Routing: number of workgroups for n pairs (at least one, so that the
// offsets are always written).
inline int64_t route_blocks(int64_t n) { return n > 0 ? ceil_div(n, kRouteChunk) : 1; }

// Largest number of experts the routing supports.
constexpr int kMaxExperts = 2048;

struct RouteArgs {
  const int32_t* idx;   // [n]
  int64_t n;
  int32_t E;
  int32_t* perm;        // [n]
  int32_t* offsets;     // [E+1]
  int32_t* counts;      // [route_blocks(n), E+1] scratch: per-block histograms
  int32_t* error;       // optional: [0] number of out-of-range indices,
                        //           [1] the tile height the tile table was built for
  int32_t* tiles;       // optional: [3, E+1] tile prefixes for tile height bm
  int32_t rows_per_pair;  // M: routed rows per pair (tile table counts rows)
  int32_t bm;           // tile height for the tile table
  // optional zero-fill of the output rows of out-of-range pairs
  uint16_t* out;
  int64_t out_row_elems;  // M * N
};

// Per-group row sums of x for the tiled GEMM's bias and offset terms.
struct RowSumArgs {
  const uint16_t* x;    // bf16 [xrows, K]
  int64_t xrows;
  int32_t K, G, Gp, group_size;
  uint16_t* sums;       // [xrows, 3, Gp] bf16 parts
};

// One launch: the routing of a (if not null) and the row sums of s (if not
// null) run side by side in one grid.
hipError_t launch_route(const RouteArgs* a, const RowSumArgs* s, hipStream_t stream);

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t cols, int group_size,
                           int bits, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                           hipStream_t s);

// Gathered grouped GEMM over the routed rows (or the identity routing when
// perm == nullptr, which is the dense product).
struct GemmArgs {
  const uint16_t* x;         // bf16 rows
  uint32_t x_bytes;          // size of x (buffer-descriptor range; <= kMaxXBytes)
  const uint32_t* wq;        // [E, N, K*bits/32]
  const uint16_t* w_bf16;    // unquantised gather: bf16 [E, N, K]
  const uint8_t* scales_e8;  // MX gathers: E8M0 exponents [E, N, K / 32] (codes in wq);
                             // NVFP4: E4M3 block scales [E, N, K / 16]
  const float* gscale;       // NVFP4: fp32 scale per expert [E]
  // gate/up in one pass (glu != 0): wq / scales / biases hold the gate weight,
  // these the up weight (both [E, N, K]); out has N = F columns,
  // act(gate) * up with act 1 = SiLU, 2 = GELU
  const uint32_t* wq2;
  const uint16_t* scales2;
  const uint16_t* biases2;
  int32_t glu, act;
  const uint16_t* scales;    // [E, N, K/gs]
  const uint16_t* biases;    // [E, N, K/gs]
  uint16_t* out;             // bf16 rows of N
  const int32_t* perm;       // [n pairs] or nullptr (dense: identity, E == 1)
  const int32_t* offsets;    // [E+1] pair offsets per expert (routed only)
  const int32_t* tiles;      // [3, E+1] tile prefixes (routed only): ceil(rows / bm),
                             // floor(rows / bm), experts with rows % bm > 0
  const int32_t* tile_bm;    // tile height the tile table was built for (routed only)
  uint16_t* sums;            // [x rows, 3, Gp] bf16 parts of the per-group row sums of x
  uint32_t sums_bytes;       // size of sums (buffer-descriptor range)
  int32_t Gp;                // groups per row of sums: K / group_size rounded up to 32
  int64_t n_pairs;           // pairs (routed) or rows (dense)
  int32_t E;
  int32_t A;                 // slots per token (x row mapping)
  int32_t Ax;                // x rows per token: 1 or A
  int32_t M;                 // rows per pair
  int32_t K, N;
  int32_t group_size, bits;
  int32_t bm;                // tile height
  int32_t ntw;               // tiled GEMM: 16-column blocks per wave (3 or 4; 0 = 4)
  int32_t col_group;         // tiled GEMM: column tiles per group of the tile order (0 = all)
  // small-M path with the routing folded in (a decode-sized routing, M = 1):
  // every workgroup routes the pairs of idx in LDS; workgroup 0 also writes
  // the routing (offsets, perm, tile table, error word) to r_* and zeroes the
  // output rows of out-of-range pairs
  int32_t fuse;
  const int32_t* idx;        // [n_pairs] expert of each pair
  int32_t* r_offsets;        // [E+1]
  int32_t* r_perm;           // [n_pairs]
  int32_t* r_tiles;          // [E+1]
  int32_t* r_error;          // [2]
  int32_t waves;             // small-M path: waves splitting K (4, 8 or 16)
  int32_t cs;                // small-M path: 1 = the 4 waves split the columns, not K
  int32_t nt;                // small-M path: 16-column blocks per wave (1, or 2 for 4-bit)
  int32_t sw;                // small-M path: each wave copies its own groups' scales and
                             // biases (split of K, one round per wave, see small_m_own_slices)
  int64_t max_tiles;         // upper bound on row tiles (grid size)
  // tiled GEMM (launch_gemm): tail tiles (a segment's last rows, up to half a
  // tile, in a shorter tile after every full one; tables rows 1 and 2) never
  // (mixed = 0), when the full tiles fit in one round of resident workgroups
  // and the segments' last tiles would spill into another (1), or always
  // (2); else tiles of bm rows (table row 0).  Grid bounds on tiles of bm
  // rows and on tail tiles (max_part is 0 when mixed is 0).
  int32_t mixed;
  int64_t max_full, max_part;
  // tiled GEMM, non-GLU: slots for the fp32 sums of tail-tile pieces (a tail
  // tile split along K), kTailPieceBytes each; nullptr: tails are not split
  float* part;
  int64_t part_pieces;
};
// one piece of a split tail tile: up to 64 rows x 256 columns of fp32 sums
constexpr int64_t kTailPieceBytes = 65536;
// pieces per tail tile at most
constexpr int kMaxTailPieces = 8;
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// Compute units of the MI355X, for the host's choice of tile width.
constexpr int kComputeUnits = 256;
// 16-column blocks per wave of the tiled GEMM (tiles of 64 * ntw columns) for
// `rows` routed rows in tiles of `bm` rows and N output columns.
int gemm_tile_cols(int64_t rows, int64_t N, int bm, int E, int bits, int group_size, bool glu);
// the stored weight applied untransposed (transpose = 0): a.wq [E, K, N*bits/32],
// a.scales / a.biases [E, K, N/group_size]; same routing and tile heights as
// launch_gemm, tiles of 64 columns, K % 32 == 0, N % group_size == 0
hipError_t launch_gather_nn(const GemmArgs& a, hipStream_t s);
// unquantised bf16 weights (a.w_bf16), same tiles and routing as launch_gemm
hipError_t launch_gather_mm(const GemmArgs& a, hipStream_t s);
// MX weights (a.wq codes, a.scales_e8 exponents; a.bits 4 = MXFP4, 8 = MXFP8),
// same tiles and routing
hipError_t launch_gather_mx(const GemmArgs& a, hipStream_t s);
// MX quantisation of bf16 rows [rows, cols], cols % 32 == 0, bits 4 or 8
hipError_t launch_quantize_mx(const uint16_t* w, int64_t rows, int64_t cols, int bits,
                              uint32_t* wq, uint8_t* scales, hipStream_t s);
// NVFP4 quantisation of a bf16 stack [tensors, rows, cols], cols % 16 == 0
hipError_t launch_quantize_nv(const uint16_t* w, int64_t tensors, int64_t rows, int64_t cols,
                              uint32_t* wq, uint8_t* scales, float* gscale, hipStream_t s);
// Groups per row of the row-sum planes for K / group_size groups.
inline int32_t sums_groups(int64_t K, int group_size) {
  return int32_t(ceil_div(K / group_size, 32) * 32);
}
inline uint64_t sums_bytes(int64_t xrows, int64_t K, int group_size) {
  return uint64_t(xrows) * 3u * uint64_t(sums_groups(K, group_size)) * 2u;
}

// Small-M path: row tiles of a.bm in {1, 2, 4, 8} rows (dense, or a tile
// table built for that height), 16 * a.nt output columns per workgroup,
// a.waves in {4, 8, 16} waves splitting K.
hipError_t launch_small_m(const GemmArgs& a, hipStream_t s);
// tile height of the small-M path for `rows` rows over E experts (E = 1: dense)
int small_m_rows(int64_t rows, int64_t E);
// Whether the small-M kernel takes K / group_size groups per row: it holds the
// scale and bias rows of a workgroup's 16 columns in LDS (at most 1024 values
// each).  The choice of the small-M path for a routed call depends on the
// rows and experts only (a routing may serve several K), so plans that pick
// it reject longer rows.
inline bool small_m_fits(int64_t N, int64_t K, int group_size) {
  (void)N;
  return K / group_size <= 1024;
}
// waves per small-M workgroup for `blocks` workgroups over a K-long reduction
int small_m_waves(int64_t blocks, int64_t K, int bits, int group_size);
// Largest routing the small-M kernel routes itself (M = 1): pairs, experts.
// Every workgroup routes all pairs: up to 512 that cost less than the
// separate routing launch (a batched decode of 64 tokens, top-8: 42.3 against
// 45.6 us), at 1024 more (59.3 against 55.7 us).
constexpr int kFuseMaxPairs = 512;
constexpr int kFuseMaxExperts = 1023;
// Whether the small-M kernel can route the pairs itself for rows of K: its
// routing scratch shares LDS with the small scale block, which holds the
// scale rows of K / group_size <= 256 groups.
bool small_m_fuse_fits(int64_t K, int group_size);
// Whether each small-M wave can copy the scales and biases of its own groups
// (at most 8 per column) instead of the workgroup staging the block's rows
// behind a barrier: the split of K over 8 or 16 waves with one round of
// steps per wave, two groups per step, an even number of groups per row, no
// folded routing, the small scale blocks (whose LDS holds 1 KB a wave).
bool small_m_own_slices(int64_t K, int bits, int group_size, int waves, int nt, bool cs, bool fuse,
                        bool large);
// whether short rows take the column split (each of 4 waves walks all of K),
// and whether the column split can take rows of K (its scale rows fit LDS)
bool small_m_colsplit(int64_t K, int bits, int group_size, int nt);
bool small_m_colsplit_fits(int64_t K, int group_size, int nt);
// 16-column blocks per small-M wave for N columns, `tiles` row tiles,
// `bits`-bit codes and G groups per row
int small_m_cols(int64_t N, int64_t tiles, int bits, int64_t G);

// Largest x (bytes) the kernels address with 32-bit buffer offsets; offsets
// from 2^31 up mark rows that read as zeros.
constexpr uint64_t kMaxXBytes = 0x7FFFFF00ull;

}  // namespace mq
