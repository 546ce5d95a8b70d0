// C ABI of libmq.so: argument validation, the host-side plan (tile height,
// workspace carve-up) and the kernel launches.  See include/mq.h for the
// contract of every entry point.
//
// Nothing here allocates device memory or synchronises: each call enqueues its
// kernels on the caller's stream.  All validation happens before the first HIP
// call, so a rejected call leaves the device untouched.
//
// Environment (read on every call, never cached, so that a test can steer
// one call at a time onto a path it wants to reach):
//   MQ_LOG=1        print each dispatch decision to stderr;
//   MQ_FORCE_BM=n   force the gather tile height n in {16, 32, 64, 128};
//   MQ_FORCE_COLS=n force n in {3, 4} 16-column blocks per wave of the tiled
//                   GEMM where both exist (tiles of 64 or 128 rows, 4-bit
//                   codes in groups of 64);
//   MQ_SMALL_M=0|1  force the gather off / onto the small-M path;
//   MQ_SMALL_WAVES=n, MQ_SMALL_COLS=n  force the small-M path's waves per
//                   workgroup (4, 8 or 16) and 16-column blocks per wave (1,
//                   or 2 for 4-bit codes whose scale rows fit), so that a test
//                   can reach every small-M kernel instance;
//   MQ_SMALL_COLSPLIT=0|1  force the small-M path's column split (each of 4
//                   waves walks all of K for columns of its own) off / on
//                   (on only where the workgroup's scale rows fit);
//   MQ_SMALL_OWN=0  keep the small-M path's staged scale block where each
//                   wave would copy its own groups' scales;
//   MQ_TAIL_TILES=0|1  tail tiles of the tiled GEMM (an expert's last rows,
//                   up to half a tile, in a shorter tile after the full ones)
//                   never / always, instead of when the full-height tiles fit
//                   in one round of resident workgroups and the experts' last
//                   tiles would spill into a second;
//   MQ_TAIL_SPLIT=0 never split tail tiles along K (by default they are,
//                   into pieces of whole correction windows, where K has two
//                   windows or more and the workspace holds the pieces' slots);
//   MQ_COL_GROUP=n  the tiled GEMM's tile order takes column tiles in groups of
//                   n (0: all of a row tile's) instead of 8;
//   MQ_FUSE_ROUTE=0 keep a decode-sized routing in its own launch instead of
//                   inside the small-M kernel.
#include <cstdio>
#include <cstdlib>

#include "../../include/mq.h"
#include "mq_internal.h"

using namespace mq;

namespace {

// scratch of the routing: one histogram of E+1 bins per block of pairs
size_t route_ws_bytes(int64_t n, int32_t E) {
  return align256(size_t(route_blocks(n)) * size_t(E + 1) * 4);
}

bool log_enabled() {
  const char* v = std::getenv("MQ_LOG");
  return v && v[0] && v[0] != '0';
}

}  // namespace

void mq::note_dispatch(const char* kernel, std::initializer_list<int> params) {
  if (!log_enabled()) return;
  char buf[160];
  int n = std::snprintf(buf, sizeof buf, "[mq-dispatch] %s<", kernel);
  bool first = true;
  for (const int p : params) {
    n += std::snprintf(buf + n, sizeof buf - size_t(n), first ? "%d" : ",%d", p);
    first = false;
  }
  std::fprintf(stderr, "%s>\n", buf);
}

namespace {

// -1: no preference, 0: never the small-M path, 1: always.
int forced_small() {
  const char* v = std::getenv("MQ_SMALL_M");
  if (!v || !v[0]) return -1;
  return v[0] == '0' ? 0 : 1;
}

// 16-column blocks per wave of the tiled GEMM: the heuristic's choice unless
// MQ_FORCE_COLS names one the kernel has for this tile height and format
int tile_cols(int64_t rows, int64_t N, int bm, int E, int bits, int group_size, bool glu) {
  const int nt = gemm_tile_cols(rows, N, bm, E, bits, group_size, glu);
  const char* v = std::getenv("MQ_FORCE_COLS");
  if (!v || !v[0] || glu || bm < 64 || bits != 4 || group_size != 64) return nt;
  const int f = std::atoi(v);
  return (f == 3 || f == 4) ? f : nt;
}

int forced_bm() {
  const char* v = std::getenv("MQ_FORCE_BM");
  if (!v || !v[0]) return 0;
  const int bm = std::atoi(v);
  return (bm == 16 || bm == 32 || bm == 64 || bm == 128) ? bm : 0;
}

// Workgroups (at one 16-column block per wave) from which the small-M path
// takes the column split whatever the row length.
constexpr int64_t kColSplitWorkgroups = 1024;

// small-M launch shape: column blocks per wave, waves splitting K, and the
// column split for short rows or many row tiles
void small_m_shape(GemmArgs& g, int64_t tiles, int64_t K, int bits, int group_size) {
  g.nt = small_m_cols(g.N, tiles, bits, K / group_size);
  bool forced_cols = false;
  if (const char* v = std::getenv("MQ_SMALL_COLS")) {
    const int nt = std::atoi(v);
    if (nt == 1 || (nt == 2 && bits == 4 && 32 * (K / group_size) * 2 <= 4096)) {
      g.nt = nt;
      forced_cols = true;
    }
  }
  g.waves = small_m_waves(ceil_div(g.N, 16 * g.nt) * tiles, K, bits, group_size);
  if (const char* v = std::getenv("MQ_SMALL_WAVES")) {
    const int kw = std::atoi(v);
    // the large scale block (K / group_size > 256) leaves LDS for 8 waves
    if (kw == 4 || kw == 8 || (kw == 16 && 16 * (K / group_size) * 2 <= 8192)) g.waves = kw;
  }
  g.cs = 0;
  // short rows: the 4 waves split the columns (MQ_SMALL_COLSPLIT=0|1 overrides)
  bool cs = small_m_colsplit(K, bits, group_size, g.nt);
  // Many row tiles (short runs over many experts): the column split too,
  // with one column block per wave where two would not fit its scale rows.
  // Splitting K there gives workgroups of a few steps per wave whose partial
  // sums meet in LDS; E = 256 with 2 .. 8 rows per expert, K = 2048 -> 512:
  // 4-bit 38 / 50 / 62 against 46 / 53 / 67 us, 8-bit gs32 59 / 74 / 84
  // against 71 / 79 / 101 us; K = 1024 -> 2048, 4-bit: 70 / 82 / 96 against
  // 143 / 123 / 166 us.  A decode step over 128 experts (40 tiles) keeps the
  // split of K.
  if (!cs && ceil_div(g.N, 64) * tiles >= kColSplitWorkgroups) {
    if (small_m_colsplit_fits(K, group_size, g.nt)) {
      cs = true;
    } else if (g.nt == 2 && !forced_cols && small_m_colsplit_fits(K, group_size, 1)) {
      g.nt = 1;
      cs = true;
    }
  }
  if (const char* v = std::getenv("MQ_SMALL_COLSPLIT"))
    cs = v[0] == '1' && small_m_colsplit_fits(K, group_size, g.nt);
  if (cs) {
    g.cs = 1;
    g.waves = 4;
  }
  // MQ_SMALL_OWN=0 keeps the staged scale block (a test hook)
  const int64_t block = int64_t(16) * g.nt * (K / group_size) * 2;
  const bool large = !g.cs && block > (g.nt == 2 ? 4096 : 8192);
  g.sw = small_m_own_slices(K, bits, group_size, g.waves, g.nt, g.cs != 0, g.fuse != 0, large);
  if (const char* v = std::getenv("MQ_SMALL_OWN"))
    if (v[0] == '0') g.sw = 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tail tiles of the tiled GEMM (a segment's last r % bm rows, when they are
// at most bm / 2 for bm >= 64, in a tile of 32 or 64 rows, after every full
// tile): the kernel takes them when its full tiles fit in one round of
// resident workgroups and the segments' last tiles would spill into a second.
// Test hook MQ_TAIL_TILES: 0 never, 1 always.
int tail_tiles() {
  const char* v = std::getenv("MQ_TAIL_TILES");
  if (v && v[0] == '0') return 0;
  if (v && v[0] == '1') return 2;
  return 1;
}

// Tail tiles split along K (the kernel decides per launch).  Test hook
// MQ_TAIL_SPLIT=0: never.
bool tail_split() {
  const char* v = std::getenv("MQ_TAIL_SPLIT");
  return !(v && v[0] == '0');
}

// Grid bounds of the tiled GEMM for `rows` rows over `segments` segments at
// most: max_tiles tiles of bm rows (ceil(rows / bm) + segments bounds them
// however the rows fall), plus one tail tile per segment with tail tiles.
void gemm_tiles(GemmArgs& g, int64_t rows, int64_t segments, int64_t max_tiles) {
  // tile order: groups of 8 column tiles (Mixtral-shaped projections, 56
  // and 16 column tiles per row tile: 4 % and 3 % faster than all columns of
  // a row tile first; the prefill shape has 3); MQ_COL_GROUP=n overrides
  g.col_group = 8;
  if (const char* v = std::getenv("MQ_COL_GROUP")) g.col_group = std::atoi(v);
  g.mixed = g.bm >= 64 ? tail_tiles() : 0;
  g.max_full = max_tiles;
  g.max_part = g.mixed ? std::min<int64_t>(segments, rows) : 0;
}

// Tile height from the average run of rows per expert (ml-explore/mlx PR 4023,
// "The change": a shorter block when the average run is short, so that a run
// is not padded out to a much taller block).  Thresholds are gfx950's own.
// `short16`: runs too short for 32-row tiles take 16-row tiles; else (the
// quantised gathers) 32-row tiles, whose launch loads 4-bit gs64 codes in
// chunk pairs and streams the weights faster (E = 256, 16 rows per expert,
// K = 2048 <-> 512: 59 against 67 us).  The quantised gathers' tile height
// must not depend on the format: a routing is shared by projections of
// other formats (mq_gather_route, mq_gather_qmm_routed).
int pick_bm(int64_t rows, int32_t E, bool short16) {
  const int f = forced_bm();
  if (f) return f;
  const double avg = double(rows) / double(E);
  if (avg >= 96) return 128;
  if (avg >= 48) return 64;
  if (avg >= 24 || !short16) return 32;
  return 16;
}

// transpose = 1: the stored weight [N, K] is quantised along K (the
// reduction); transpose = 0: it is [K, N], quantised along N (the output).
mq_status check_quant_params(int64_t K, int64_t N, int group_size, int bits, int transpose) {
  if (K <= 0) return MQ_ERR_INVALID;
  if (transpose != 0 && transpose != 1) return MQ_ERR_INVALID;
  if (bits != 4 && bits != 8) return MQ_ERR_UNSUPPORTED;
  if (group_size != 32 && group_size != 64) return MQ_ERR_UNSUPPORTED;
  if (transpose && K % group_size) return MQ_ERR_INVALID;
  if (!transpose && N % group_size) return MQ_ERR_INVALID;
  if (K % 64) return MQ_ERR_UNSUPPORTED;            // the GEMMs walk K in chunks of 64 (or 32)
  if (K > (int64_t(1) << 30)) return MQ_ERR_UNSUPPORTED;
  return MQ_OK;
}

struct Layout {
  size_t offsets, perm, error, tiles, counts, sums, part, total;
};

// The routing regions come first and do not depend on K, so a workspace
// routed by mq_gather_route serves every projection that shares the routing;
// the row sums of x (sized for xrows rows) follow.  Everything up to `part`
// is required; the slots for split tail-tile pieces after it (part_pieces of
// kTailPieceBytes) are used when the workspace holds them.
Layout gather_layout(int64_t n, int32_t E, int64_t xrows, int64_t K, int group_size,
                     int64_t part_pieces = 0) {
  Layout L;
  size_t at = 0;
  L.offsets = at; at += align256(size_t(E + 1) * 4);
  L.perm = at;    at += align256(size_t(n > 0 ? n : 1) * 4);
  L.error = at;   at += 256;
  L.tiles = at;   at += align256(size_t(E + 1) * 3 * 4);
  L.counts = at;  at += route_ws_bytes(n, E);
  L.sums = at;    at += align256(size_t(sums_bytes(xrows, K, group_size)));
  L.part = at;    at += size_t(part_pieces) * size_t(kTailPieceBytes);
  L.total = at;
  return L;
}

// Piece slots for the tiled GEMM's split tail tiles (see launch_gemm): one
// tail tile per expert at most, as many column tiles as the narrowest tile
// (192 columns) gives, up to kMaxTailPieces pieces each (one per correction
// window of 32 groups), at most kMaxPartPieces slots (64 MiB) in all.
constexpr int64_t kMaxPartPieces = 1024;
int64_t tail_piece_slots(int64_t rows, int32_t E, int64_t K, int64_t N, int group_size, int bm) {
  const int64_t nwin = ceil_div(K / group_size, int64_t(32));
  if (bm < 64 || N <= 0 || rows <= 0 || nwin < 2) return 0;
  const int64_t tails = std::min<int64_t>(E, rows) * ceil_div(N, int64_t(192));
  return std::min(kMaxPartPieces, tails * std::min<int64_t>(kMaxTailPieces, nwin));
}


}  // namespace

extern "C" {

const char* mq_status_str(mq_status status) {
  switch (status) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_INVALID: return "MQ_ERR_INVALID";
    case MQ_ERR_UNSUPPORTED: return "MQ_ERR_UNSUPPORTED";
    case MQ_ERR_WORKSPACE: return "MQ_ERR_WORKSPACE";
    case MQ_ERR_HIP: return "MQ_ERR_HIP";
  }
  return "MQ_ERR_UNKNOWN";
}

mq_status mq_quantize(const mq_bf16* w, int64_t rows, int64_t cols, int group_size, int bits,
                      uint32_t* wq, mq_bf16* scales, mq_bf16* biases, void* stream) {
  if (rows < 0 || cols <= 0) return MQ_ERR_INVALID;
  if (bits != 4 && bits != 8) return MQ_ERR_UNSUPPORTED;
  if (group_size != 32 && group_size != 64) return MQ_ERR_UNSUPPORTED;
  if (cols % group_size) return MQ_ERR_INVALID;
  if (cols > (int64_t(1) << 30)) return MQ_ERR_UNSUPPORTED;
  if (rows > 0 && (!w || !wq || !scales || !biases)) return MQ_ERR_INVALID;
  if (rows == 0) return MQ_OK;
  const hipError_t e = launch_quantize(w, rows, cols, group_size, bits, wq, scales, biases,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

mq_status mq_quantize_mx(const mq_bf16* w, int64_t rows, int64_t cols, int bits, uint32_t* wq,
                         uint8_t* scales, void* stream) {
  if (bits != 4 && bits != 8) return MQ_ERR_UNSUPPORTED;
  if (rows < 0 || cols <= 0 || cols % 32) return MQ_ERR_INVALID;
  if (cols > (int64_t(1) << 30)) return MQ_ERR_UNSUPPORTED;
  if (rows > 0 && (!w || !wq || !scales)) return MQ_ERR_INVALID;
  if ((w && !aligned16(w)) || (wq && !aligned16(wq))) return MQ_ERR_INVALID;
  if (rows == 0) return MQ_OK;
  const hipError_t e = launch_quantize_mx(w, rows, cols, bits, wq, scales,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

mq_status mq_quantize_nv(const mq_bf16* w, int64_t tensors, int64_t rows, int64_t cols,
                         uint32_t* wq, uint8_t* scales, float* gscale, void* stream) {
  if (tensors < 0 || rows < 0 || cols <= 0 || cols % 16) return MQ_ERR_INVALID;
  if (cols > (int64_t(1) << 30) || tensors > 0x7FFFFFFF) return MQ_ERR_UNSUPPORTED;
  if (tensors > 0 && rows > 0 && (!w || !wq || !scales || !gscale)) return MQ_ERR_INVALID;
  if ((w && !aligned16(w)) || (wq && !aligned16(wq)) ||
      (gscale && (reinterpret_cast<uintptr_t>(gscale) & 3u)))
    return MQ_ERR_INVALID;
  if (tensors == 0 || rows == 0) return MQ_OK;
  const hipError_t e = launch_quantize_nv(w, tensors, rows, cols, wq, scales, gscale,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

mq_status mq_route_workspace(int64_t n, int32_t E, size_t* bytes) {
  if (!bytes || n < 0 || E <= 0) return MQ_ERR_INVALID;
  if (E > 2048) return MQ_ERR_UNSUPPORTED;
  if (n > 0x7FFFFFFF) return MQ_ERR_UNSUPPORTED;
  *bytes = route_ws_bytes(n, E);
  return MQ_OK;
}

mq_status mq_route(const int32_t* idx, int64_t n, int32_t E, int sorted_indices, int32_t* perm,
                   int32_t* offsets, void* ws, size_t ws_bytes, void* stream) {
  (void)sorted_indices;   // a hint only: the stable sort of sorted input is the identity
  if (n < 0 || E <= 0) return MQ_ERR_INVALID;
  if (E > 2048 || n > 0x7FFFFFFF) return MQ_ERR_UNSUPPORTED;
  if (!offsets || (n > 0 && (!idx || !perm))) return MQ_ERR_INVALID;
  if (!ws || ws_bytes < route_ws_bytes(n, E)) return MQ_ERR_WORKSPACE;
  RouteArgs r{};
  r.idx = idx;
  r.n = n;
  r.E = E;
  r.perm = perm;
  r.offsets = offsets;
  r.counts = static_cast<int32_t*>(ws);
  r.error = nullptr;
  r.tiles = nullptr;
  r.rows_per_pair = 1;
  r.bm = 1;
  r.out = nullptr;
  r.out_row_elems = 0;
  return launch_route(&r, nullptr, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK
                                                                                   : MQ_ERR_HIP;
}

namespace {

struct GatherPlan {
  int64_t n, rows;
  int bm;
  bool nn;             // transpose = 0: the stored [K, N] weight applied untransposed
  bool small;          // small-M path: short row tiles, split-K workgroups
  int64_t max_tiles;
  Layout L;
};

// Average runs of a few rows per expert (batched decode through a MoE layer,
// lablup/mlxcel issue 725) are weight-bandwidth bound: the small-M path reads
// each routed expert's weight once with K split across waves.  Longer runs go
// to the tiled GEMM.
// The choice depends on the rows and experts only, as does the tile height:
// a routing written by mq_gather_route serves calls of any K.
bool pick_small(int64_t rows, int32_t E) {
  const int f = forced_small();
  if (f >= 0) return f == 1;
  if (forced_bm()) return false;
  return double(rows) / double(E) <= 8.0;
}

// One expert's codes, scales and biases are each addressed through a buffer
// descriptor with 32-bit offsets; a code offset may run up to 16 columns past
// the last one (a column block's distance rides in the uniform offset), and
// offsets from 2^31 up mark rows that read as zeros.
bool expert_weight_fits(int64_t N, int64_t K, int group_size, int bits, int transpose) {
  if (!transpose)   // [K, N]: codes and scales of one expert
    return uint64_t(K) * uint64_t(N) * uint64_t(bits) / 8u <= kMaxXBytes &&
           uint64_t(K) * uint64_t(N / group_size) * 2u <= kMaxXBytes;
  const uint64_t row_bytes = uint64_t(K) * uint64_t(bits) / 8u;
  return uint64_t(N + 16) * row_bytes <= kMaxXBytes &&
         uint64_t(N + 16) * uint64_t(K / group_size) * 2u <= kMaxXBytes;
}

// allow_small = false: the caller runs the tiled GEMM whatever the rows per
// expert (the fused gate/up), so the small-M path's limits do not apply.
mq_status plan_gather(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N, int32_t E,
                      int group_size, int bits, int transpose, GatherPlan* p,
                      bool allow_small = true) {
  if (T < 0 || A <= 0 || M <= 0 || N < 0 || E <= 0) return MQ_ERR_INVALID;
  const mq_status q = check_quant_params(K, N, group_size, bits, transpose);
  if (q != MQ_OK) return q;
  if (E > 2048) return MQ_ERR_UNSUPPORTED;
  if (N > 0x7FFFFFFF || T * A > 0x7FFFFFFF / M) return MQ_ERR_UNSUPPORTED;
  if (uint64_t(T) * uint64_t(A) * uint64_t(M) * uint64_t(K) * 2u > kMaxXBytes)
    return MQ_ERR_UNSUPPORTED;
  if (!expert_weight_fits(N, K, group_size, bits, transpose)) return MQ_ERR_UNSUPPORTED;
  // the row sums are sized for x [T, A, M, K], the largest x (Ax = A)
  if (sums_bytes(T * A * M, K, group_size) > kMaxXBytes) return MQ_ERR_UNSUPPORTED;
  p->n = T * A;
  p->rows = p->n * M;
  p->nn = transpose == 0;
  // the untransposed product has no small-M path: short runs take 32-row tiles
  p->small = allow_small && !p->nn && pick_small(p->rows, E);
  // the small-M kernel keeps a workgroup's scale rows in LDS
  if (p->small && !small_m_fits(N, K, group_size)) return MQ_ERR_UNSUPPORTED;
  p->bm = p->small ? small_m_rows(p->rows, E) : pick_bm(p->rows, E, false);
  p->max_tiles = ceil_div(p->rows, p->bm) + E;
  const int64_t slots = p->small || p->nn ? 0 : tail_piece_slots(p->rows, E, K, N, group_size, p->bm);
  p->L = gather_layout(p->n, E, p->rows, K, group_size, slots);
  return MQ_OK;
}

RouteArgs route_args(const GatherPlan& p, const int32_t* rhs_indices, int32_t E, int64_t M,
                     int64_t N, mq_bf16* out, char* base) {
  RouteArgs r{};
  r.idx = rhs_indices;
  r.n = p.n;
  r.E = E;
  r.perm = reinterpret_cast<int32_t*>(base + p.L.perm);
  r.offsets = reinterpret_cast<int32_t*>(base + p.L.offsets);
  r.counts = reinterpret_cast<int32_t*>(base + p.L.counts);
  r.error = reinterpret_cast<int32_t*>(base + p.L.error);
  r.tiles = reinterpret_cast<int32_t*>(base + p.L.tiles);
  r.rows_per_pair = int32_t(M);
  r.bm = p.bm;
  r.out = N > 0 ? out : nullptr;
  r.out_row_elems = M * N;
  return r;
}

// Whether the small-M kernel routes the pairs itself: one row per pair, a
// routing small enough for every workgroup to redo it in LDS (a decode step),
// and rows short enough for the routing scratch to share LDS with the scale
// rows.  MQ_FUSE_ROUTE=0 keeps the separate routing launch.
bool fuse_routing(const GatherPlan& p, int64_t M, int32_t E, int64_t N, int64_t K,
                  int group_size) {
  if (const char* v = std::getenv("MQ_FUSE_ROUTE"))
    if (v[0] == '0') return false;
  return p.small && M == 1 && N > 0 && p.n >= 1 && p.n <= kFuseMaxPairs &&
         E <= kFuseMaxExperts && small_m_fuse_fits(K, group_size);
}

// The tiled GEMM reads per-group row sums of x; the small-M path and the
// untransposed product do not.
bool needs_sums(const GatherPlan& p, int64_t N) { return !p.small && !p.nn && p.n > 0 && N > 0; }

RowSumArgs sum_args(const mq_bf16* x, int64_t xrows, int64_t K, int group_size, uint16_t* sums) {
  RowSumArgs rs{};
  rs.x = x;
  rs.xrows = xrows;
  rs.K = int32_t(K);
  rs.G = int32_t(K / group_size);
  rs.Gp = sums_groups(K, group_size);
  rs.group_size = group_size;
  rs.sums = sums;
  return rs;
}

// the up weight and activation of a fused gate/up call
struct GluWeights {
  const uint32_t* wq;
  const mq_bf16* scales;
  const mq_bf16* biases;
  int act;
};

mq_status enqueue_gemm(const GatherPlan& p, const mq_bf16* x, int64_t T, int64_t A, int64_t Ax, int64_t M,
                       int64_t K, const uint32_t* wq, const mq_bf16* scales,
                       const mq_bf16* biases, int32_t E, int64_t N, int group_size, int bits,
                       mq_bf16* out, char* base, size_t ws_bytes, hipStream_t s,
                       const int32_t* fuse_idx = nullptr, const GluWeights* glu = nullptr) {
  if (p.n == 0 || N == 0) return MQ_OK;
  GemmArgs g{};
  g.x = x;
  g.x_bytes = uint32_t(uint64_t(T) * uint64_t(Ax) * uint64_t(M) * uint64_t(K) * 2u);
  g.wq = wq;
  g.scales = scales;
  g.biases = biases;
  g.out = out;
  g.perm = reinterpret_cast<const int32_t*>(base + p.L.perm);
  g.offsets = reinterpret_cast<const int32_t*>(base + p.L.offsets);
  g.tiles = reinterpret_cast<const int32_t*>(base + p.L.tiles);
  g.tile_bm = reinterpret_cast<const int32_t*>(base + p.L.error) + 1;
  g.n_pairs = p.n;
  g.E = E;
  g.A = int32_t(A);
  g.Ax = int32_t(Ax);
  g.M = int32_t(M);
  g.K = int32_t(K);
  g.N = int32_t(N);
  g.group_size = group_size;
  g.bits = bits;
  g.bm = p.bm;
  g.max_tiles = p.max_tiles;
  if (p.nn) return launch_gather_nn(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
  if (p.small) {
    if (fuse_idx) {
      // the small-M kernel routes the pairs itself (and leaves the routing in ws)
      g.fuse = 1;
      g.idx = fuse_idx;
      g.r_offsets = reinterpret_cast<int32_t*>(base + p.L.offsets);
      g.r_perm = reinterpret_cast<int32_t*>(base + p.L.perm);
      g.r_tiles = reinterpret_cast<int32_t*>(base + p.L.tiles);
      g.r_error = reinterpret_cast<int32_t*>(base + p.L.error);
    }
    // The grid: sum over experts of ceil(rows_e / bm) <= rows / bm + (experts
    // touched) <= ceil(rows / bm) + min(E, rows) tiles.  For a decode step
    // (32 pairs over 128 experts) that is 40 tiles where the plan's bound,
    // ceil(rows / bm) + E, gives 136; surplus workgroups (which, with the
    // routing folded in, each route the pairs before finding no tile) cost
    // launch time.
    const int64_t tiles = std::min<int64_t>(p.max_tiles, ceil_div(p.rows, p.bm) + std::min<int64_t>(E, p.rows));
    g.max_tiles = tiles;
    small_m_shape(g, tiles, K, bits, group_size);
    return launch_small_m(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
  }
  if (glu) {
    g.glu = 1;
    g.act = glu->act;
    g.wq2 = glu->wq;
    g.scales2 = glu->scales;
    g.biases2 = glu->biases;
  }
  g.ntw = tile_cols(p.rows, N, p.bm, E, bits, group_size, glu != nullptr);
  gemm_tiles(g, p.rows, std::min<int64_t>(E, p.rows), p.max_tiles);
  // the per-group row sums of x were written by the routing launch
  g.sums = reinterpret_cast<uint16_t*>(base + p.L.sums);
  g.Gp = sums_groups(K, group_size);
  g.sums_bytes = uint32_t(sums_bytes(T * Ax * M, K, group_size));
  // the piece slots this workspace holds (none: tail tiles are not split)
  const int64_t slots = std::min<int64_t>(int64_t((p.L.total - p.L.part) / kTailPieceBytes),
                                          ws_bytes > p.L.part ? int64_t((ws_bytes - p.L.part) / kTailPieceBytes) : 0);
  if (!glu && slots > 0 && tail_split()) {
    g.part = reinterpret_cast<float*>(base + p.L.part);
    g.part_pieces = slots;
  }
  return launch_gemm(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

// The unquantised (bf16 weight) gather: the tiled GEMM's routing and tile
// heights, no row sums (nothing to correct), no small-M path.
mq_status plan_gather_mm(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N, int32_t E,
                         int transpose, GatherPlan* p) {
  if (T < 0 || A <= 0 || M <= 0 || N < 0 || E <= 0 || K <= 0) return MQ_ERR_INVALID;
  if (transpose != 0 && transpose != 1) return MQ_ERR_INVALID;
  if (transpose != 1) return MQ_ERR_UNSUPPORTED;
  if (K % 64) return MQ_ERR_UNSUPPORTED;            // the GEMM walks K in chunks of 64
  if (K > (int64_t(1) << 30) || E > 2048) return MQ_ERR_UNSUPPORTED;
  if (N > 0x7FFFFFFF || T * A > 0x7FFFFFFF / M) return MQ_ERR_UNSUPPORTED;
  if (uint64_t(T) * uint64_t(A) * uint64_t(M) * uint64_t(K) * 2u > kMaxXBytes)
    return MQ_ERR_UNSUPPORTED;
  // one expert's weight is one buffer-descriptor range
  if (uint64_t(N) * uint64_t(K) * 2u > kMaxXBytes) return MQ_ERR_UNSUPPORTED;
  p->n = T * A;
  p->rows = p->n * M;
  p->small = false;
  p->bm = pick_bm(p->rows, E, true);
  p->max_tiles = ceil_div(p->rows, p->bm) + E;
  p->L = gather_layout(p->n, E, 0, K, 64);
  return MQ_OK;
}

void log_gather(const char* what, const GatherPlan& p, int64_t T, int64_t A, int64_t Ax,
                int64_t M, int64_t K, int64_t N, int32_t E, int bits, int gs) {
  if (!log_enabled()) return;
  std::fprintf(stderr,
               "[mq] %s T=%lld A=%lld Ax=%lld M=%lld K=%lld N=%lld E=%d bits=%d gs=%d "
               "rows/expert=%.1f -> BM=%d max_tiles=%lld kernel=%s<%d,%d>\n",
               what, (long long)T, (long long)A, (long long)Ax, (long long)M, (long long)K,
               (long long)N, E, bits, gs, double(p.rows) / E, p.bm, (long long)p.max_tiles,
               p.small ? "small_m" : (p.nn ? "gather_nn" : "gather_gemm"), bits, gs);
}

}  // namespace

mq_status mq_gather_qmm_workspace(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N,
                                  int32_t E, int group_size, int bits, mq_ws_layout* layout) {
  if (!layout) return MQ_ERR_INVALID;
  GatherPlan p;
  // the layout is the same on every path, so the small-M path's own limit is
  // left to the call that takes it (the fused gate/up never does)
  const mq_status st = plan_gather(T, A, M, K, N, E, group_size, bits, 1, &p, false);
  if (st != MQ_OK) return st;
  layout->offsets = p.L.offsets;
  layout->perm = p.L.perm;
  layout->error = p.L.error;
  layout->tiles = p.L.tiles;
  layout->sums = p.L.sums;
  layout->part = p.L.part;
  layout->total = p.L.total;
  return MQ_OK;
}

mq_status mq_gather_route(const int32_t* rhs_indices, int64_t T, int64_t A, int64_t M,
                          int32_t E, void* ws, size_t ws_bytes, void* stream) {
  GatherPlan p;
  // the routing does not depend on K, N or the quantisation: plan with
  // neutral values; only the routing regions (everything before the row
  // sums) are written
  const mq_status st = plan_gather(T, A, M, 64, 0, E, 64, 4, 1, &p);
  if (st != MQ_OK) return st;
  if (p.n > 0 && !rhs_indices) return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.sums || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather("gather_route", p, T, A, A, M, 0, 0, E, 0, 0);
  const RouteArgs r = route_args(p, rhs_indices, E, M, 0, nullptr, static_cast<char*>(ws));
  return launch_route(&r, nullptr, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK
                                                                                   : MQ_ERR_HIP;
}

mq_status mq_gather_sums(const mq_bf16* x, int64_t T, int64_t Ax, int64_t A, int64_t M,
                         int64_t K, int32_t E, int group_size, void* ws, size_t ws_bytes,
                         void* stream) {
  GatherPlan p;
  const mq_status st = plan_gather(T, A, M, K, 0, E, group_size, 4, 1, &p);
  if (st != MQ_OK) return st;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && !x) return MQ_ERR_INVALID;
  if (x && !aligned16(x)) return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  if (p.n == 0) return MQ_OK;
  const RowSumArgs rs = sum_args(x, T * Ax * M, K, group_size,
                                 reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.L.sums));
  return launch_route(nullptr, &rs, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK
                                                                                    : MQ_ERR_HIP;
}

mq_status mq_gather_qmm_routed(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                               const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                               int32_t E, int64_t N, int64_t A, int transpose, int group_size,
                               int bits, mq_bf16* out, const void* ws, size_t ws_bytes,
                               void* stream) {
  GatherPlan p;
  const mq_status st = plan_gather(T, A, M, K, N, E, group_size, bits, transpose, &p);
  if (st != MQ_OK) return st;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && (!x || (N > 0 && !out))) return MQ_ERR_INVALID;
  if (N > 0 && (!wq || !scales || !biases)) return MQ_ERR_INVALID;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || (wq && !aligned16(wq)))
    return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather("gather_qmm_routed", p, T, A, Ax, M, K, N, E, bits, group_size);
  return enqueue_gemm(p, x, T, A, Ax, M, K, wq, scales, biases, E, N, group_size, bits, out,
                      const_cast<char*>(static_cast<const char*>(ws)), ws_bytes,
                      static_cast<hipStream_t>(stream));
}

mq_status mq_gather_qmm(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                        const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                        int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                        int transpose, int group_size, int bits, int sorted_indices,
                        mq_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  (void)sorted_indices;   // a hint only; see mq_route
  GatherPlan p;
  const mq_status st = plan_gather(T, A, M, K, N, E, group_size, bits, transpose, &p);
  if (st != MQ_OK) return st;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && (!x || !rhs_indices || (N > 0 && !out))) return MQ_ERR_INVALID;
  if (N > 0 && (!wq || !scales || !biases)) return MQ_ERR_INVALID;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || (wq && !aligned16(wq)))
    return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather("gather_qmm", p, T, A, Ax, M, K, N, E, bits, group_size);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  // A decode-sized routing on the small-M path is done by the small-M kernel
  // itself (one launch instead of two); otherwise one launch routes the
  // pairs and (for the tiled GEMM) sums the x rows.
  if (fuse_routing(p, M, E, N, K, group_size)) {
    log_gather("gather_qmm (routing in the small-M kernel)", p, T, A, Ax, M, K, N, E, bits,
               group_size);
    return enqueue_gemm(p, x, T, A, Ax, M, K, wq, scales, biases, E, N, group_size, bits, out,
                        base, ws_bytes, s, rhs_indices);
  }
  const RouteArgs r = route_args(p, rhs_indices, E, M, N, out, base);
  const RowSumArgs rs =
      sum_args(x, T * Ax * M, K, group_size, reinterpret_cast<uint16_t*>(base + p.L.sums));
  if (launch_route(&r, needs_sums(p, N) ? &rs : nullptr, s) != hipSuccess) return MQ_ERR_HIP;
  return enqueue_gemm(p, x, T, A, Ax, M, K, wq, scales, biases, E, N, group_size, bits, out, base,
                      ws_bytes, s);
}

mq_status mq_gather_qmm_glu(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                            const uint32_t* wq_gate, const mq_bf16* scales_gate,
                            const mq_bf16* biases_gate, const uint32_t* wq_up,
                            const mq_bf16* scales_up, const mq_bf16* biases_up, int32_t E,
                            int64_t F, const int32_t* rhs_indices, int64_t A, int transpose,
                            int group_size, int bits, int sorted_indices, int act, mq_bf16* out,
                            void* ws, size_t ws_bytes, void* stream) {
  (void)sorted_indices;   // a hint only; see mq_route
  GatherPlan p;
  // the fused store exists on the tiled path only: short runs take 32-row tiles
  const mq_status st = plan_gather(T, A, M, K, F, E, group_size, bits, transpose, &p, false);
  if (st != MQ_OK) return st;
  if (p.nn) return MQ_ERR_UNSUPPORTED;     // the fused gate/up is a forward-pass call
  if (act != 1 && act != 2) return MQ_ERR_UNSUPPORTED;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && (!x || !rhs_indices || (F > 0 && !out))) return MQ_ERR_INVALID;
  if (F > 0 && (!wq_gate || !scales_gate || !biases_gate || !wq_up || !scales_up || !biases_up))
    return MQ_ERR_INVALID;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || (wq_gate && !aligned16(wq_gate)) ||
      (wq_up && !aligned16(wq_up)))
    return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather("gather_qmm_glu", p, T, A, Ax, M, K, F, E, bits, group_size);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const RouteArgs r = route_args(p, rhs_indices, E, M, F, out, base);
  const RowSumArgs rs =
      sum_args(x, T * Ax * M, K, group_size, reinterpret_cast<uint16_t*>(base + p.L.sums));
  if (launch_route(&r, needs_sums(p, F) ? &rs : nullptr, s) != hipSuccess) return MQ_ERR_HIP;
  const GluWeights up{wq_up, scales_up, biases_up, act};
  return enqueue_gemm(p, x, T, A, Ax, M, K, wq_gate, scales_gate, biases_gate, E, F, group_size,
                      bits, out, base, ws_bytes, s, nullptr, &up);
}

mq_status mq_gather_mm_workspace(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N,
                                 int32_t E, mq_ws_layout* layout) {
  if (!layout) return MQ_ERR_INVALID;
  GatherPlan p;
  const mq_status st = plan_gather_mm(T, A, M, K, N, E, 1, &p);
  if (st != MQ_OK) return st;
  layout->offsets = p.L.offsets;
  layout->perm = p.L.perm;
  layout->error = p.L.error;
  layout->tiles = p.L.tiles;
  layout->sums = p.L.sums;
  layout->part = p.L.part;
  layout->total = p.L.total;
  return MQ_OK;
}

mq_status mq_gather_mm(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                       const mq_bf16* w, int32_t E, int64_t N, const int32_t* rhs_indices,
                       int64_t A, int transpose, int sorted_indices, mq_bf16* out, void* ws,
                       size_t ws_bytes, void* stream) {
  (void)sorted_indices;   // a hint only; see mq_route
  GatherPlan p;
  const mq_status st = plan_gather_mm(T, A, M, K, N, E, transpose, &p);
  if (st != MQ_OK) return st;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && (!x || !rhs_indices || (N > 0 && !out))) return MQ_ERR_INVALID;
  if (N > 0 && !w) return MQ_ERR_INVALID;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || (w && !aligned16(w)))
    return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather("gather_mm", p, T, A, Ax, M, K, N, E, 16, 0);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const RouteArgs r = route_args(p, rhs_indices, E, M, N, out, base);
  if (launch_route(&r, nullptr, s) != hipSuccess) return MQ_ERR_HIP;
  if (p.n == 0 || N == 0) return MQ_OK;
  GemmArgs g{};
  g.x = x;
  g.x_bytes = uint32_t(uint64_t(T) * uint64_t(Ax) * uint64_t(M) * uint64_t(K) * 2u);
  g.w_bf16 = w;
  g.out = out;
  g.perm = reinterpret_cast<const int32_t*>(base + p.L.perm);
  g.offsets = reinterpret_cast<const int32_t*>(base + p.L.offsets);
  g.tiles = reinterpret_cast<const int32_t*>(base + p.L.tiles);
  g.tile_bm = reinterpret_cast<const int32_t*>(base + p.L.error) + 1;
  g.n_pairs = p.n;
  g.E = E;
  g.A = int32_t(A);
  g.Ax = int32_t(Ax);
  g.M = int32_t(M);
  g.K = int32_t(K);
  g.N = int32_t(N);
  g.bits = 16;
  g.bm = p.bm;
  g.max_tiles = p.max_tiles;
  return launch_gather_mm(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

}  // extern "C"

namespace {

// The MX and NVFP4 gathers: the bf16 gather's plan and routing, then the MX
// GEMM (gscale != NULL selects NVFP4).
mq_status gather_mx_common(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                           const uint32_t* wq, const uint8_t* scales, const float* gscale,
                           int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                           int transpose, int bits, int sorted_indices, mq_bf16* out, void* ws,
                           size_t ws_bytes, void* stream, const char* what) {
  (void)sorted_indices;   // a hint only; see mq_route
  if (bits != 4 && bits != 8) return MQ_ERR_UNSUPPORTED;
  GatherPlan p;
  // the bf16 gather's plan: its per-expert weight limit (N*K*2 bytes) is
  // stricter than the codes' (N*K/2)
  const mq_status st = plan_gather_mm(T, A, M, K, N, E, transpose, &p);
  if (st != MQ_OK) return st;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (p.n > 0 && (!x || !rhs_indices || (N > 0 && !out))) return MQ_ERR_INVALID;
  if (N > 0 && (!wq || !scales)) return MQ_ERR_INVALID;
  if ((x && !aligned16(x)) || (out && !aligned16(out)) || (wq && !aligned16(wq)))
    return MQ_ERR_INVALID;
  if (!ws || ws_bytes < p.L.part || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  log_gather(what, p, T, A, Ax, M, K, N, E, bits, gscale ? 16 : 32);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const RouteArgs r = route_args(p, rhs_indices, E, M, N, out, base);
  if (launch_route(&r, nullptr, s) != hipSuccess) return MQ_ERR_HIP;
  if (p.n == 0 || N == 0) return MQ_OK;
  GemmArgs g{};
  g.x = x;
  g.x_bytes = uint32_t(uint64_t(T) * uint64_t(Ax) * uint64_t(M) * uint64_t(K) * 2u);
  g.wq = wq;
  g.scales_e8 = scales;
  g.gscale = gscale;
  g.out = out;
  g.bits = bits;
  g.perm = reinterpret_cast<const int32_t*>(base + p.L.perm);
  g.offsets = reinterpret_cast<const int32_t*>(base + p.L.offsets);
  g.tiles = reinterpret_cast<const int32_t*>(base + p.L.tiles);
  g.tile_bm = reinterpret_cast<const int32_t*>(base + p.L.error) + 1;
  g.n_pairs = p.n;
  g.E = E;
  g.A = int32_t(A);
  g.Ax = int32_t(Ax);
  g.M = int32_t(M);
  g.K = int32_t(K);
  g.N = int32_t(N);
  g.bm = p.bm;
  g.max_tiles = p.max_tiles;
  return launch_gather_mx(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

}  // namespace

extern "C" {

mq_status mq_gather_qmm_mx(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                           const uint32_t* wq, const uint8_t* scales, int32_t E, int64_t N,
                           const int32_t* rhs_indices, int64_t A, int transpose, int bits,
                           int sorted_indices, mq_bf16* out, void* ws, size_t ws_bytes,
                           void* stream) {
  return gather_mx_common(x, T, Ax, M, K, wq, scales, nullptr, E, N, rhs_indices, A, transpose,
                          bits, sorted_indices, out, ws, ws_bytes, stream, "gather_qmm_mx");
}

mq_status mq_gather_qmm_nv(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                           const uint32_t* wq, const uint8_t* scales, const float* gscale,
                           int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                           int transpose, int sorted_indices, mq_bf16* out, void* ws,
                           size_t ws_bytes, void* stream) {
  if (N > 0 && (!gscale || (reinterpret_cast<uintptr_t>(gscale) & 3u))) return MQ_ERR_INVALID;
  return gather_mx_common(x, T, Ax, M, K, wq, scales, gscale, E, N, rhs_indices, A, transpose,
                          4, sorted_indices, out, ws, ws_bytes, stream, "gather_qmm_nv");
}

mq_status mq_qmm_workspace(int64_t M, int64_t K, int group_size, size_t* bytes) {
  if (!bytes || M < 0 || K <= 0) return MQ_ERR_INVALID;
  if (group_size != 32 && group_size != 64) return MQ_ERR_UNSUPPORTED;
  if (K % group_size) return MQ_ERR_INVALID;
  if (sums_bytes(M, K, group_size) > kMaxXBytes) return MQ_ERR_UNSUPPORTED;
  *bytes = size_t(sums_bytes(M, K, group_size));
  return MQ_OK;
}

mq_status mq_qmm(const mq_bf16* x, int64_t M, int64_t K, const uint32_t* wq,
                 const mq_bf16* scales, const mq_bf16* biases, int64_t N, int transpose,
                 int group_size, int bits, mq_bf16* out, void* ws, size_t ws_bytes,
                 void* stream) {
  if (M < 0 || N < 0) return MQ_ERR_INVALID;
  const mq_status q = check_quant_params(K, N, group_size, bits, transpose);
  if (q != MQ_OK) return q;
  if (M > 0x7FFFFFFF || N > 0x7FFFFFFF) return MQ_ERR_UNSUPPORTED;
  if (uint64_t(M) * uint64_t(K) * 2u > kMaxXBytes) return MQ_ERR_UNSUPPORTED;
  if (!expert_weight_fits(N, K, group_size, bits, transpose)) return MQ_ERR_UNSUPPORTED;
  if (sums_bytes(M, K, group_size) > kMaxXBytes) return MQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return MQ_OK;
  if (!x || !wq || !scales || !biases || !out) return MQ_ERR_INVALID;
  if (!aligned16(x) || !aligned16(out) || !aligned16(wq)) return MQ_ERR_INVALID;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  GemmArgs g{};
  g.x = x;
  g.x_bytes = uint32_t(uint64_t(M) * uint64_t(K) * 2u);
  g.wq = wq;
  g.scales = scales;
  g.biases = biases;
  g.out = out;
  g.perm = nullptr;
  g.offsets = nullptr;
  g.tiles = nullptr;
  g.n_pairs = M;
  g.E = 1;
  g.A = 1;
  g.Ax = 1;
  g.M = 1;
  g.K = int32_t(K);
  g.N = int32_t(N);
  g.group_size = group_size;
  g.bits = bits;
  g.bm = M <= 16 ? 16 : (M <= 32 ? 32 : (M <= 64 ? 64 : 128));
  const int f = forced_bm();
  if (f) g.bm = f;
  g.max_tiles = ceil_div(M, g.bm);
  if (!transpose) {
    // the stored [K, N] weight applied untransposed: the routed kernel with
    // identity rows (no row sums, no small-M path)
    if (log_enabled())
      std::fprintf(stderr, "[mq] qmm M=%lld K=%lld N=%lld bits=%d gs=%d transpose=0 -> BM=%d "
                   "kernel=gather_nn<%d,%d>\n", (long long)M, (long long)K, (long long)N, bits,
                   group_size, g.bm, g.bm, bits);
    return launch_gather_nn(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
  }
  if (M <= 16 && !f && forced_small() != 0 && small_m_fits(N, K, group_size)) {
    // lablup/mlxcel issue 725: one pass over the weight per tile of <= 8 rows
    g.bm = small_m_rows(M, 1);
    g.max_tiles = ceil_div(M, g.bm);
    small_m_shape(g, g.max_tiles, K, bits, group_size);
    if (log_enabled())
      std::fprintf(stderr,
                   "[mq] qmm M=%lld K=%lld N=%lld bits=%d gs=%d -> kernel=small_m<%d,%d> "
                   "waves=%d col_blocks=%d\n",
                   (long long)M, (long long)K, (long long)N, bits, group_size, bits, group_size,
                   g.waves, g.nt);
    return launch_small_m(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
  }
  g.ntw = tile_cols(M, N, g.bm, 1, bits, group_size, false);
  gemm_tiles(g, M, 1, g.max_tiles);
  // the tiled GEMM reads the per-group row sums of x from the workspace
  const uint64_t need = sums_bytes(M, K, group_size);
  if (!ws || ws_bytes < need || !aligned16(ws)) return MQ_ERR_WORKSPACE;
  g.sums = static_cast<uint16_t*>(ws);
  g.sums_bytes = uint32_t(need);
  g.Gp = sums_groups(K, group_size);
  if (log_enabled())
    std::fprintf(stderr, "[mq] qmm M=%lld K=%lld N=%lld bits=%d gs=%d -> BM=%d kernel=gather_gemm<%d,%d,%d> "
                 "col_blocks=%d\n",
                 (long long)M, (long long)K, (long long)N, bits, group_size, g.bm, g.bm, bits,
                 group_size, g.ntw);
  const RowSumArgs rs = sum_args(x, M, K, group_size, g.sums);
  if (launch_route(nullptr, &rs, s) != hipSuccess) return MQ_ERR_HIP;
  return launch_gemm(g, s) == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

}  // extern "C"
