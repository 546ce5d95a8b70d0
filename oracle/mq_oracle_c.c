/*
 * The oracle's fp32 form in plain C: quantise, route, and the routed product
 * accumulated in fp32.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests and the CPU baseline of the
 * benchmark load this library (through oracle/c_oracle.py).  It shares no
 * code with the HIP library, and nothing here comes from it.
 *
 * What is computed (the same definitions as oracle/mq_oracle.py, which holds
 * the citations and the readings in full):
 *   ml-explore/mlx issue 4339, "Kernel microbenchmark": quantize(w, group_size,
 *   bits) gives packed codes and one scale and one bias per group along the
 *   last axis; gather_qmm multiplies every (token, slot) row of x by the
 *   dequantised weight of the expert its index names (transposed for
 *   transpose = 1); quantized_matmul is the same against one weight.
 *   lablup/mlxcel issue 629, "Implementation plan" 4b: routing groups the
 *   pairs by expert, here a stable counting sort.
 *
 * Readings (the same as the fp64 oracle's where they decide an integer):
 *   quantise   per group: lo = min, hi = max (-0 read as +0); bias = lo;
 *              scale = fp32(hi - lo) / (2^bits - 1) in fp32, rounded up to
 *              bf16; q = clamp(rint((w - bias) / scale), 0, 2^bits - 1) with
 *              fp32 subtraction and IEEE division, ties to even; scale 0 gives
 *              q = 0; codes little-endian in uint32 words along the group axis.
 *   dequantise w_hat = fp32(scale) * q + fp32(bias) in fp32: the product is
 *              exact (at most 16 significant bits), the sum rounds once.
 *   product    out = sum over k ascending of x_k * w_hat_k, each step one fp32
 *              fused multiply-add (acc <- fl(acc + x_k w_hat_k)), acc from 0.
 *              The benchmark spec asks for an fp32-accumulated oracle; the fp64
 *              oracle is the stricter reference, this one the plain fp32 form.
 *   routing    perm = the pairs stably sorted by expert (indices outside [0, E)
 *              are an error here: the caller's precondition).
 *
 * Work is split over output rows only (OpenMP when built with -fopenmp), so
 * results do not depend on the thread count.
 *
 * Planted mistakes for the pin tests (each build defines at most one):
 *   MQ_MUTANT_NO_BIAS      dequantise without the bias;
 *   MQ_MUTANT_ROUND_AWAY   codes rounded half away from zero;
 *   MQ_MUTANT_GROUP_SHIFT  the scale of group g taken from group g + 1;
 *   MQ_MUTANT_UNSTABLE     routing places a segment's pairs in reverse;
 *   MQ_MUTANT_SKIP_LAST_K  the product drops the last k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* threads for the parallel loops (n <= 0: leave the default); returns the
 * number in use */
int mqo_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* Smallest bf16 >= f (f finite and >= 0 here). */
static uint16_t bf16_round_up(float f) {
  const uint32_t u = f32_bits(f);
  uint16_t hi = (uint16_t)(u >> 16);
  if (u & 0xFFFFu) hi = (uint16_t)(hi + 1); /* positive: the next pattern is larger */
  return hi;
}

static float code_of(float w, float bias, float scale, int qmax) {
  if (scale == 0.0f) return 0.0f;
  const float t = (w - bias) / scale;
#ifdef MQ_MUTANT_ROUND_AWAY
  float q = roundf(t);
#else
  float q = rintf(t); /* default rounding mode: ties to even */
#endif
  if (q < 0.0f) q = 0.0f;
  if (q > (float)qmax) q = (float)qmax;
  return q;
}

/* w bf16 [rows, cols] -> wq uint32 [rows, cols*bits/32], scales and biases
 * bf16 [rows, cols/gs].  Returns 0, or -1 for unsupported parameters. */
int mqo_quantize(const uint16_t* w, int64_t rows, int64_t cols, int gs, int bits,
                 uint32_t* wq, uint16_t* scales, uint16_t* biases) {
  if ((bits != 4 && bits != 8) || gs <= 0 || cols % gs || gs % (32 / bits)) return -1;
  const int per = 32 / bits, qmax = (1 << bits) - 1;
  const int64_t G = cols / gs, words = cols / per;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    memset(wq + r * words, 0, (size_t)words * 4);
    for (int64_t g = 0; g < G; ++g) {
      const uint16_t* wg = w + r * cols + g * gs;
      float lo = bf16_to_f32(wg[0]), hi = lo;
      for (int i = 1; i < gs; ++i) {
        const float v = bf16_to_f32(wg[i]);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      if (lo == 0.0f) lo = 0.0f; /* signed zeros read as +0 */
      if (hi == 0.0f) hi = 0.0f;
      const uint16_t sb = bf16_round_up((hi - lo) / (float)qmax);
      const uint16_t bb = (uint16_t)(f32_bits(lo) >> 16); /* lo is a bf16 value: exact */
      scales[r * G + g] = sb;
      biases[r * G + g] = bb;
      const float s = bf16_to_f32(sb);
      for (int i = 0; i < gs; ++i) {
        const uint32_t q = (uint32_t)code_of(bf16_to_f32(wg[i]), lo, s, qmax);
        const int64_t k = g * gs + i;
        wq[r * words + k / per] |= q << ((k % per) * bits);
      }
    }
  }
  return 0;
}

/* wq/scales/biases of `rows` rows of `cols` -> w_hat fp32 [rows, cols] */
static void dequantize_rows(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            int64_t rows, int64_t cols, int gs, int bits, float* out) {
  const int per = 32 / bits;
  const int64_t G = cols / gs, words = cols / per;
  const uint32_t mask = (1u << bits) - 1u;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < cols; ++k) {
      const int64_t g = k / gs;
#ifdef MQ_MUTANT_GROUP_SHIFT
      const int64_t gsrc = g + 1 < G ? g + 1 : g;
#else
      const int64_t gsrc = g;
#endif
      const float s = bf16_to_f32(scales[r * G + gsrc]);
#ifdef MQ_MUTANT_NO_BIAS
      const float b = 0.0f;
#else
      const float b = bf16_to_f32(biases[r * G + g]);
#endif
      const uint32_t q = (wq[r * words + k / per] >> ((k % per) * bits)) & mask;
      out[r * cols + k] = s * (float)q + b; /* exact product, one rounding */
    }
}

int mqo_dequantize(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                   int64_t rows, int64_t cols, int gs, int bits, float* out) {
  if ((bits != 4 && bits != 8) || gs <= 0 || cols % gs) return -1;
  dequantize_rows(wq, scales, biases, rows, cols, gs, bits, out);
  return 0;
}

/* counts [E], offsets [E+1], perm [n]: the pairs stably sorted by expert.
 * Returns 0, or -1 if an index lies outside [0, E). */
int mqo_route(const int32_t* idx, int64_t n, int32_t E, int32_t* counts, int32_t* offsets,
              int32_t* perm) {
  for (int64_t i = 0; i < n; ++i)
    if (idx[i] < 0 || idx[i] >= E) return -1;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n; ++i) counts[idx[i]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  if (!cur) return -2;
  for (int32_t e = 0; e < E; ++e) cur[e] = offsets[e];
  for (int64_t i = 0; i < n; ++i) perm[cur[idx[i]]++] = (int32_t)i;
#ifdef MQ_MUTANT_UNSTABLE
  for (int32_t e = 0; e < E; ++e)
    for (int32_t a = offsets[e], b = offsets[e + 1] - 1; a < b; ++a, --b) {
      const int32_t t = perm[a];
      perm[a] = perm[b];
      perm[b] = t;
    }
#endif
  free(cur);
  return 0;
}

/* out fp32 [T, A, M, NO]: x bf16 [T, Ax, M, KI] (Ax = 1 or A), the stored
 * stack [E, R, C] quantised along C, idx int32 [T, A].  transpose = 1: KI = C
 * and NO = R, out[t,a,m,n] = sum_k x[t,a',m,k] w_hat[e,n,k]; transpose = 0:
 * KI = R and NO = C, out[t,a,m,n] = sum_k x[t,a',m,k] w_hat[e,k,n].
 * Returns 0, -1 for bad parameters or an index outside [0, E), -2 if memory
 * runs out. */
int mqo_gather_qmm(const uint16_t* x, int64_t T, int64_t Ax, int64_t M, const uint32_t* wq,
                   const uint16_t* scales, const uint16_t* biases, int32_t E, int64_t R,
                   int64_t C, const int32_t* idx, int64_t A, int transpose, int gs, int bits,
                   float* out) {
  if ((bits != 4 && bits != 8) || gs <= 0 || C % gs || (Ax != 1 && Ax != A) || E <= 0) return -1;
  for (int64_t p = 0; p < T * A; ++p)
    if (idx[p] < 0 || idx[p] >= E) return -1;
  const int64_t KI = transpose ? C : R, NO = transpose ? R : C;
  float* w = (float*)malloc(sizeof(float) * (size_t)(E * R * C));
  if (!w) return -2;
  dequantize_rows(wq, scales, biases, (int64_t)E * R, C, gs, bits, w);
#ifdef MQ_MUTANT_SKIP_LAST_K
  const int64_t kend = KI - 1;
#else
  const int64_t kend = KI;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < T * A; ++p) {
    const int64_t t = p / A, a = p % A;
    const float* we = w + (int64_t)idx[p] * R * C;
    for (int64_t m = 0; m < M; ++m) {
      const uint16_t* xr = x + ((t * Ax + (Ax > 1 ? a : 0)) * M + m) * KI;
      float* o = out + (p * M + m) * NO;
      for (int64_t n = 0; n < NO; ++n) {
        float acc = 0.0f;
        for (int64_t k = 0; k < kend; ++k) {
          const float wv = transpose ? we[n * C + k] : we[k * C + n];
          acc = fmaf(bf16_to_f32(xr[k]), wv, acc);
        }
        o[n] = acc;
      }
    }
  }
  free(w);
  return 0;
}
