/*
 * mq.h — expert-routed affine-quantised matmul (gather_qmm) on AMD Instinct
 * MI355X (gfx950).  C ABI of libmq.so.
 *
 * Sources for what each call computes (the pages are cited by title and
 * section):
 *   [mlx-4339]   ml-explore/mlx issue 4339, "[CUDA] gather_qmm ~24x slower than
 *                equal-FLOPs quantized_matmul on GB10 (sm_121)", section
 *                "Kernel microbenchmark": the quantize / gather_qmm /
 *                quantized_matmul calls and their keyword arguments.
 *   [mlxcel-629] lablup/mlxcel issue 629, "fix MoE prefill collapse on CUDA",
 *                section "Implementation plan", 4a/4b: a grouped GEMM per
 *                expert group over tokens sorted by expert on the device.
 *   [mlx-4023]   ml-explore/mlx PR 4023, "Pick BM from rows per expert in
 *                gather_qmm_rhs_nax", opening paragraphs and "The change":
 *                block height chosen from the average run of rows per expert;
 *                weight traffic set by the experts a block touches.
 *   [mlxcel-725] lablup/mlxcel issue 725, "amortizing small-M quantized GEMM
 *                for batched decode", sections "The gap" / "What's needed":
 *                read each weight tile once for all B <= 8 rows.
 *   [mlx-4339-bf16] the same mlx issue 4339, its follow-up comments on the
 *                bf16 MoE gather path (GatherMM): the routed product with
 *                unquantised bf16 expert weights, slow on the same hardware.
 *   [mlx-fp-modes] the microscaling fp modes the pages name beside the affine
 *                one: mlx PR 4023, the comment on block-height coverage (the
 *                mxfp4 / nvfp4 / mxfp8 kernels of the same gather), and mlx
 *                issue 4339, the maintainers' note that the CUDA backend keeps
 *                only the fp modes.  The pages define no format; MXFP4 is read
 *                as the OCP Microscaling Formats (MX) v1.0 specification's.
 *
 * Data formats (the pages name the calls but print no formats; these are the
 * library's readings and are identical to the CPU oracle's):
 *   bf16       raw IEEE bfloat16 bit patterns (mq_bf16).
 *   Quantised  a weight of R rows by K columns, quantised along K in groups of
 *   weight     group_size: for row r and group g = k / group_size,
 *                  w_hat[r,k] = scale[r,g] * q[r,k] + bias[r,g]
 *              with q an unsigned `bits`-bit code.
 *                wq      uint32 [R, K*bits/32]: code k of a row sits in bits
 *                        [(k % (32/bits))*bits, +bits) of word k / (32/bits)
 *                scales  bf16   [R, K/group_size]
 *                biases  bf16   [R, K/group_size]
 *              An expert stack [E, N, K] is the same with R = E*N, row
 *              r = e*N + n.  A stored weight is always quantised along its
 *              last axis: [E, N, K] for transpose = 1 (x @ w_hat^T, groups
 *              along the reduction K), [E, K, N] for transpose = 0 (x @ w_hat,
 *              groups along the output N; the orientation of the backward
 *              product of a forward call on the same stored weight).
 *   MXFP4      (OCP MX v1.0) per 32 weights along K one E8M0 exponent e and
 *   weight     per weight a 4-bit E2M1 code c (sign, 2 exponent bits with
 *              bias 1, 1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6):
 *                  w_hat[r,k] = e2m1(q[r,k]) * 2^(e[r, k/32] - 127)
 *                wq      uint32 [R, K/8]: packed like the 4-bit affine codes
 *                scales  uint8  [R, K/32]
 *   NVFP4      (NVIDIA's NVFP4) per 16 weights along K one E4M3 scale s and per
 *   weight     tensor (expert) one fp32 scale g; 4-bit E2M1 codes as MXFP4:
 *                  w_hat[e,n,k] = e2m1(q) * e4m3(s[e, n, k/16]) * g[e]
 *                wq uint32 [E, N, K/8], scales uint8 [E, N, K/16] (E4M3
 *                codes, sign bit clear, < 0x7F), gscale float [E]
 *   MXFP8      the same with an 8-bit E4M3 code (sign, 4 exponent bits with
 *   weight     bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN, largest
 *              magnitude 448): wq uint32 [R, K/4], packed like the 8-bit
 *              affine codes.
 *
 * Conventions for every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller, contiguous
 *     row-major, and must stay valid until the enqueued work completes.
 *     Pointers of zero-sized tensors may be NULL.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     enqueues its kernels on it and returns without synchronising; nothing
 *     is copied between host and device.
 *   - The library allocates no device memory and keeps no mutable global
 *     state: concurrent calls on different streams with distinct outputs and
 *     workspaces are safe.
 *   - Arguments are validated on the host BEFORE any HIP call.  Bad shapes or
 *     NULL pointers give MQ_ERR_INVALID, valid but unimplemented parameters
 *     MQ_ERR_UNSUPPORTED, a short workspace MQ_ERR_WORKSPACE; in each case no
 *     work is enqueued.  A failed launch gives MQ_ERR_HIP.
 *   - Supported parameters: bits in {4, 8}; group_size in {32, 64}; the
 *     quantised axis a multiple of group_size (K for transpose = 1, N for
 *     transpose = 0; MQ_ERR_INVALID otherwise); for the matmuls K % 64 == 0
 *     (MQ_ERR_UNSUPPORTED otherwise); transpose in {0, 1} for the affine
 *     gather, its routed and no-alloc forms and the dense product, 1 for the
 *     others (any other value: MQ_ERR_INVALID, 0 where only 1 exists:
 *     MQ_ERR_UNSUPPORTED); at most 2048 experts; x, out and wq 16-byte
 *     aligned (MQ_ERR_INVALID otherwise).
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t mq_bf16;

typedef enum {
    MQ_OK = 0,
    MQ_ERR_INVALID = 1,      /* bad shape, NULL pointer, out-of-range argument */
    MQ_ERR_UNSUPPORTED = 2,  /* valid request this library does not implement */
    MQ_ERR_WORKSPACE = 3,    /* workspace too small (or NULL when needed)      */
    MQ_ERR_HIP = 4           /* a HIP launch/runtime call failed               */
} mq_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char* mq_status_str(mq_status status);

/*
 * mq_quantize — affine-quantise a bf16 matrix along its rows.   [mlx-4339]
 *
 * w       bf16 [rows, cols], finite values.
 * wq      uint32 [rows, cols*bits/32]      (output)
 * scales  bf16   [rows, cols/group_size]   (output)
 * biases  bf16   [rows, cols/group_size]   (output)
 *
 * Per group: bias = minimum; scale = fp32(max - min) / (2^bits - 1) in IEEE
 * fp32, rounded UP to bf16; a -0.0 minimum or maximum is read as +0.0, so a
 * zero bias and a zero scale each have one bit pattern;
 * q = clamp(rint_half_even(fp32(w - bias) / scale), 0, 2^bits - 1) with IEEE
 * fp32 division; a constant group gets scale 0 and q 0.  The result is
 * bit-identical to the oracle's.
 * Errors: rows < 0 or cols <= 0 or cols % group_size != 0 -> MQ_ERR_INVALID.
 */
mq_status mq_quantize(const mq_bf16* w, int64_t rows, int64_t cols, int group_size,
                      int bits, uint32_t* wq, mq_bf16* scales, mq_bf16* biases,
                      void* stream);

/*
 * mq_route_workspace — bytes of workspace mq_route needs for n indices.
 */
mq_status mq_route_workspace(int64_t n, int32_t E, size_t* bytes);

/*
 * mq_route — group flat pair indices by expert (stable).       [mlxcel-629]
 *
 * idx      int32 [n]: expert of flat pair i (i = t*A + a).
 * perm     int32 [n]     (output) perm[offsets[e] + r] = the r-th pair i, in
 *                        increasing i, with idx[i] == e.
 * offsets  int32 [E+1]   (output) offsets[0] = 0, offsets[e+1] = offsets[e] +
 *                        count of e.  Pairs whose index lies outside [0, E)
 *                        are placed, in increasing i, at perm[offsets[E] .. n);
 *                        n - offsets[E] is their number (0 for valid input).
 * sorted_indices  a hint that idx is non-decreasing; the result is identical
 *                 either way.
 * ws / ws_bytes   device workspace of at least mq_route_workspace() bytes.
 * Errors: n < 0, E <= 0 -> MQ_ERR_INVALID; E > 2048 -> MQ_ERR_UNSUPPORTED;
 * short ws -> MQ_ERR_WORKSPACE.
 */
mq_status mq_route(const int32_t* idx, int64_t n, int32_t E, int sorted_indices,
                   int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * Workspace of mq_gather_qmm.  All offsets are in bytes from the start of the
 * caller's workspace and 256-byte aligned; after a call the routing it used
 * can be read back from there:
 *   offsets  int32 [E+1]  as in mq_route
 *   perm     int32 [n]    as in mq_route (n = T*A)
 *   error    int32 [2]    [0]: number of pairs whose index was outside
 *                         [0, E) (their output rows are written as zeros);
 *                         [1]: the tile height the tile table was built for
 *   tiles    int32 [3, E+1]  over the experts e' < e of their rows r, with
 *                         h the tile height in error[1] and t = h / 2 for
 *                         h >= 64 (else 0):
 *                         [0][e] = sum of ceil(r / h) (tiles of h rows),
 *                         [1][e] = sum of floor(r / h) + [r % h > t],
 *                         [2][e] = number with 0 < r % h <= t: the tiled
 *                         GEMM runs such a segment's last r % h rows as one
 *                         tail tile of 32 or 64 rows
 *   (then the routing's per-block histograms)
 *   sums     bf16 [...]   per-group row sums of x, sized for x [T, A, M, K]
 *                         (the tiled GEMM's bias and offset terms read them)
 *   part     fp32 [...]   optional: slots of 64 KiB for the fp32 sums of tail
 *                         tiles split along K (at most 64 MiB; empty unless
 *                         the tiled GEMM may run with tail tiles and K holds
 *                         two windows of 32 groups or more)
 * The routing regions precede `sums`: mq_gather_route needs only the first
 * `sums` bytes.  mq_gather_qmm and mq_gather_qmm_routed need at least `part`
 * bytes; with `total` bytes the GEMM may split its tail tiles along K (a
 * workspace in between offers as many whole slots as it holds).  Results are
 * within the same bound either way, not bit-identical: a split tile sums its
 * pieces in fp32 in piece order.
 */
typedef struct {
    size_t offsets, perm, error, tiles, sums, part, total;
} mq_ws_layout;

mq_status mq_gather_qmm_workspace(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N,
                                  int32_t E, int group_size, int bits,
                                  mq_ws_layout* layout);

/*
 * mq_gather_qmm — expert-routed quantised matmul.     [mlx-4339], [mlxcel-629],
 *                                                      [mlx-4023]
 *
 * x            bf16 [T, Ax, M, K], Ax in {1, A} (Ax == 1 broadcasts one row
 *              block per token over its A experts).
 * wq, scales, biases   quantised expert stack: [E, N, K] (transpose = 1) or
 *              [E, K, N] (transpose = 0), see above.
 * rhs_indices  int32 [T, A], expert of each (token, slot) pair.
 * out          bf16 [T, A, M, N] (output):
 *                transpose = 1 (the pages' microbenchmark):
 *                  out[t,a,m,n] = sum_k x[t, a*(Ax>1), m, k] * w_hat[idx[t,a], n, k]
 *                transpose = 0 (ml-explore/mlx PR 4023, the coverage reply: the
 *                vector-Jacobian product flips the transpose):
 *                  out[t,a,m,n] = sum_k x[t, a*(Ax>1), m, k] * w_hat[idx[t,a], k, n]
 *              accumulated in fp32 and rounded to nearest even.  With
 *              transpose = 0 each product of a scale and a code is split into
 *              two exact bf16 parts, so every MFMA product is exact; there is
 *              no small-M path (short runs take 32-row tiles).
 * sorted_indices  a hint that rhs_indices (flattened) is non-decreasing; the
 *              output is identical either way.
 * ws           device workspace of at least layout.part bytes from
 *              mq_gather_qmm_workspace() (layout.total recommended).
 * Index values outside [0, E) are a precondition violation: those rows are
 * written as zeros and counted in the workspace error word; nothing traps.
 * Errors: shapes < 0, E <= 0, Ax not in {1, A}, NULL non-empty tensors ->
 * MQ_ERR_INVALID; see the general conventions for the rest.  With a few rows
 * per expert (on average at most 8, the batched-decode regime) K / group_size
 * may not exceed 1024 (MQ_ERR_UNSUPPORTED; mq_gather_qmm_workspace does not
 * check this, as the layout is the same on every path).  One expert's codes
 * and its scales must each stay below 2 GiB (MQ_ERR_UNSUPPORTED).
 */
mq_status mq_gather_qmm(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                        const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                        int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                        int transpose, int group_size, int bits, int sorted_indices,
                        mq_bf16* out, void* ws, size_t ws_bytes, void* stream);

/*
 * mq_gather_route — the routing half of mq_gather_qmm, on its own.
 *                                                     [mlxcel-629], [mlx-4023]
 *
 * Writes offsets, perm, the error word and the tile table into ws for the
 * pairs of rhs_indices [T, A] (M rows per pair).  Several projections that
 * share one routing (the gate, up and down matmuls of one MoE layer) can then
 * each call mq_gather_qmm_routed without routing again.
 * ws needs at least layout.sums bytes (the routing regions of the layout);
 * a workspace later passed to mq_gather_qmm_routed needs layout.part (and
 * takes layout.total) for that call's K, N and group size.
 * Errors: as mq_gather_qmm's routing arguments.
 */
mq_status mq_gather_route(const int32_t* rhs_indices, int64_t T, int64_t A, int64_t M,
                          int32_t E, void* ws, size_t ws_bytes, void* stream);

/*
 * mq_gather_sums — per-group row sums of x into ws (layout.sums), the other
 * input mq_gather_qmm_routed reads besides the routing: the tiled matmul adds
 * the bias and the code offset of each group as (row sum of x over the group)
 * x (bias, scale) products.  They depend on x only, so the projections that
 * share one x (gate and up) share them too.
 * x bf16 [T, Ax, M, K], Ax in {1, A}; ws as for mq_gather_qmm (K, group size).
 * Errors: as mq_gather_qmm.
 */
mq_status mq_gather_sums(const mq_bf16* x, int64_t T, int64_t Ax, int64_t A, int64_t M,
                         int64_t K, int32_t E, int group_size, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * mq_gather_qmm_routed — the matmul half of mq_gather_qmm.
 *
 * Same arguments and result as mq_gather_qmm, without rhs_indices: the routing
 * is read from ws, which must hold the result of mq_gather_route (or of
 * mq_gather_qmm) for the same T, A, M and E, and — unless every routed
 * expert's run is short enough for the small-M path (at most 8 rows per
 * expert on average) — the row sums of this x from mq_gather_sums (or
 * mq_gather_qmm with this x), both enqueued earlier in stream order and not
 * overwritten since.  Rows of out-of-range pairs are not written.  If the
 * workspace was routed for a different tile height, nothing is written.
 */
mq_status mq_gather_qmm_routed(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                               const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                               int32_t E, int64_t N, int64_t A, int transpose, int group_size,
                               int bits, mq_bf16* out, const void* ws, size_t ws_bytes,
                               void* stream);

/*
 * mq_qmm_workspace — bytes of workspace mq_qmm needs for x [M, K] (the
 * per-group row sums of x; at most a few hundred bytes per row).
 */
mq_status mq_qmm_workspace(int64_t M, int64_t K, int group_size, size_t* bytes);

/*
 * mq_qmm — dense quantised matmul, the equal-FLOPs control and the small-M
 * (batched decode) path.                          [mlx-4339], [mlxcel-725]
 *
 * x    bf16 [M, K];  wq / scales / biases: one quantised [N, K] weight
 *      (transpose = 1) or [K, N] weight (transpose = 0).
 * out  bf16 [M, N] = x @ w_hat^T (or x @ w_hat), fp32 accumulation, round to
 *      nearest even.  transpose = 0 needs no workspace.
 * ws   device workspace of at least mq_qmm_workspace() bytes (16-byte
 *      aligned); for M <= 16 (with K / group_size <= 1024) it is not used
 *      and may be NULL.
 * For M <= 16 (with K / group_size <= 1024) each weight tile is read from
 * memory once per tile of at most 8 rows and applied to all of them.
 * Errors: as mq_gather_qmm.
 */
mq_status mq_qmm(const mq_bf16* x, int64_t M, int64_t K, const uint32_t* wq,
                 const mq_bf16* scales, const mq_bf16* biases, int64_t N,
                 int transpose, int group_size, int bits, mq_bf16* out,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * mq_gather_qmm_glu — the gate and up projections of an MoE FFN in one pass,
 * with the gated activation applied before the store.
 *                     [mlxcel-629] (its references: the fused switch-GeGLU)
 *
 * Arguments as mq_gather_qmm, with two quantised [E, F, K] stacks (gate and
 * up, same group size and bits) and
 * act          1 = SiLU (SwiGLU), 2 = GELU with the exact error function
 *              (GeGLU); anything else -> MQ_ERR_UNSUPPORTED.
 * out          bf16 [T, A, M, F] (output):
 *                out[t,a,m,f] = act(g) * u,  g = sum_k x . w_hat_gate[e, f, :],
 *                                            u = sum_k x . w_hat_up[e, f, :]
 *              with g and u accumulated in fp32, act evaluated in fp32, one
 *              rounding to bf16.
 * ws           as for mq_gather_qmm with N = F (mq_gather_qmm_workspace).
 * One routing launch, one GEMM launch; every x row and routing is read once
 * for both projections and only F columns are written.  Always the tiled
 * GEMM (short runs take 32-row tiles).  Errors as mq_gather_qmm.
 */
mq_status mq_gather_qmm_glu(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                            const uint32_t* wq_gate, const mq_bf16* scales_gate,
                            const mq_bf16* biases_gate, const uint32_t* wq_up,
                            const mq_bf16* scales_up, const mq_bf16* biases_up, int32_t E,
                            int64_t F, const int32_t* rhs_indices, int64_t A, int transpose,
                            int group_size, int bits, int sorted_indices, int act, mq_bf16* out,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * mq_gather_mm_workspace / mq_gather_mm — the routed product with unquantised
 * bf16 expert weights.                                    [mlx-4339-bf16]
 *
 * x            bf16 [T, Ax, M, K], Ax in {1, A}.
 * w            bf16 [E, N, K], 16-byte aligned; one expert's N*K*2 bytes must
 *              stay below 2 GiB (MQ_ERR_UNSUPPORTED otherwise).
 * rhs_indices  int32 [T, A], expert of each (token, slot) pair.
 * out          bf16 [T, A, M, N] (output):
 *                out[t,a,m,n] = sum_k x[t, a*(Ax>1), m, k] * w[idx[t,a], n, k]
 *              accumulated in fp32 and rounded to nearest even.
 * transpose    must be 1; sorted_indices is a hint (the output is identical).
 * ws           device workspace of at least layout.total bytes from
 *              mq_gather_mm_workspace() (the routing only: layout.sums ==
 *              layout.total); after the call it holds the routing it used, laid
 *              out as for mq_gather_qmm.
 * The routing and the tile heights are mq_gather_qmm's (tile height from the
 * average rows per expert); there is no small-M path.  K % 64 == 0; other
 * errors as mq_gather_qmm (index values outside [0, E) give zero rows and
 * are counted in the workspace error word).
 */
mq_status mq_gather_mm_workspace(int64_t T, int64_t A, int64_t M, int64_t K, int64_t N,
                                 int32_t E, mq_ws_layout* layout);

mq_status mq_gather_mm(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                       const mq_bf16* w, int32_t E, int64_t N, const int32_t* rhs_indices,
                       int64_t A, int transpose, int sorted_indices, mq_bf16* out, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * mq_quantize_mx — MX-quantise a bf16 matrix along its rows:    [mlx-fp-modes]
 *                  MXFP4 (bits = 4, E2M1) or MXFP8 (bits = 8, E4M3).
 *
 * w       bf16 [rows, cols], finite values, 16-byte aligned, cols % 32 == 0.
 * wq      uint32 [rows, cols*bits/32]  (output), 16-byte aligned
 * scales  uint8  [rows, cols/32]       (output)
 *
 * Per block of 32: e = max(exponent field of the largest |w| - emax, 0), i.e.
 * floor(log2 amax) - emax clamped at -127 (emax = 2 for E2M1, 8 for E4M3; an
 * all-zero block gets e = 0); each weight's code is the element value nearest
 * to w / 2^(e - 127), ties to the even mantissa, magnitudes beyond the
 * largest (6, or 448) saturating to it, the sign bit always the weight's (a
 * negative weight that rounds to zero is -0).  The result is bit-identical to
 * the oracle's.  Non-finite weights give an unspecified block.
 * Errors: bits not 4 or 8 -> MQ_ERR_UNSUPPORTED; rows < 0, cols <= 0,
 * cols % 32 != 0 or a misaligned pointer -> MQ_ERR_INVALID; cols > 2^30 ->
 * MQ_ERR_UNSUPPORTED.
 */
mq_status mq_quantize_mx(const mq_bf16* w, int64_t rows, int64_t cols, int bits, uint32_t* wq,
                         uint8_t* scales, void* stream);

/*
 * mq_gather_qmm_mx — the routed product against MX expert weights
 *                    (bits = 4: MXFP4, bits = 8: MXFP8).    [mlx-fp-modes]
 *
 * x            bf16 [T, Ax, M, K], Ax in {1, A}, 16-byte aligned.
 * wq, scales   the MX expert stack [E, N, K] (see the data formats),
 *              wq 16-byte aligned.
 * rhs_indices  int32 [T, A]; out bf16 [T, A, M, N], 16-byte aligned:
 *                out[t,a,m,n] = sum_k x[t, a*(Ax>1), m, k] * w_hat[idx[t,a], n, k]
 *              accumulated in fp32 and rounded to nearest even.  Every
 *              product is exact for exponents 2..252 (MXFP4) or 10..246
 *              (MXFP8), where every weight is a normal, finite bf16; other
 *              exponents are outside that range.
 * transpose    must be 1; sorted_indices is a hint (the output is identical).
 * ws           device workspace of at least layout.total bytes from
 *              mq_gather_mm_workspace() with the same T, A, M, K, N, E (the
 *              routing only); after the call it holds the routing it used.
 * Tile heights and routing as mq_gather_mm; K % 64 == 0; other errors as
 * mq_gather_mm (index values outside [0, E) give zero rows and are counted
 * in the workspace error word).
 */
mq_status mq_gather_qmm_mx(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                           const uint32_t* wq, const uint8_t* scales, int32_t E, int64_t N,
                           const int32_t* rhs_indices, int64_t A, int transpose, int bits,
                           int sorted_indices, mq_bf16* out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * mq_quantize_nv — NVFP4-quantise a stack of bf16 tensors.   [mlx-fp-modes]
 *
 * w       bf16 [tensors, rows, cols], finite, 16-byte aligned, cols % 16 == 0.
 * wq      uint32 [tensors, rows, cols/8]   (output), 16-byte aligned
 * scales  uint8  [tensors, rows, cols/16]  (output, E4M3 codes)
 * gscale  float  [tensors]                 (output, 4-byte aligned)
 *
 * Per tensor g = amax / 2688 (6 * 448) in IEEE fp32, 1 for an all-zero tensor;
 * per 16 weights s = e4m3(fp32(fp32(amax_block / 6) / g)), nearest with ties
 * to even, saturating at 448; per weight q = e2m1(fp32(w / d)) with
 * d = fp32(e4m3(s) * g), nearest with ties to even, saturating at 6, the sign
 * bit the weight's (a block whose scale is 0 gets signed zeros).  The
 * reading of the pages' nvfp4 is NVIDIA's published format; the result is
 * bit-identical to the oracle's.  Two launches (the tensor scales, then the
 * blocks).
 * Errors: tensors < 0, rows < 0, cols <= 0, cols % 16 != 0, a NULL or
 * misaligned pointer -> MQ_ERR_INVALID; cols > 2^30 -> MQ_ERR_UNSUPPORTED.
 */
mq_status mq_quantize_nv(const mq_bf16* w, int64_t tensors, int64_t rows, int64_t cols,
                         uint32_t* wq, uint8_t* scales, float* gscale, void* stream);

/*
 * mq_gather_qmm_nv — the routed product against NVFP4 expert weights.
 *                                                           [mlx-fp-modes]
 *
 * As mq_gather_qmm_mx with bits = 4, except: scales uint8 [E, N, K/16] (E4M3
 * block scales) and gscale float [E] (each expert's fp32 scale, 4-byte
 * aligned):
 *     out[t,a,m,n] = g[e] * sum_k x[t, a*(Ax>1), m, k] * e2m1(q) * e4m3(s)
 * with e = idx[t,a]; the products e2m1 * e4m3 are bf16 values, so every MFMA
 * product is exact; the sums are fp32, multiplied by g[e] in fp32, rounded
 * to bf16 once.  Workspace from mq_gather_mm_workspace(); K % 64 == 0;
 * transpose must be 1.  Errors as mq_gather_qmm_mx (a NULL or misaligned
 * gscale with N > 0 -> MQ_ERR_INVALID).
 */
mq_status mq_gather_qmm_nv(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                           const uint32_t* wq, const uint8_t* scales, const float* gscale,
                           int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                           int transpose, int sorted_indices, mq_bf16* out, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * mq_gather_qmm_noalloc — mq_gather_qmm without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Arguments and result as mq_gather_qmm, minus ws / ws_bytes.  The workspace
 * is the library's own scratch: one device array of MQ_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, held from the first call on that GPU until the process
 * ends.  The call allocates nothing (no hipMalloc, no library allocation).
 * Errors: as mq_gather_qmm; MQ_ERR_WORKSPACE when the call would need more
 * than MQ_NOALLOC_SCRATCH_BYTES of workspace (mq_gather_qmm_workspace's
 * layout.part: the routing regions plus per-group row sums of x, e.g.
 * 3.2 MB for 16384 routed rows at K = 2048, group size 64; the optional
 * piece slots after it are used as far as the scratch holds them); MQ_ERR_INVALID
 * for a stream that does not belong to the current device; MQ_ERR_HIP if the
 * device or its scratch cannot be looked up.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (its routing can be read back from there as from a
 * workspace): calls that overlap on one GPU (several streams or threads)
 * race.
 */
#define MQ_NOALLOC_SCRATCH_BYTES (16u << 20)

mq_status mq_gather_qmm_noalloc(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                                const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                                int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                                int transpose, int group_size, int bits, int sorted_indices,
                                mq_bf16* out, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
