// Affine quantisation of bf16 rows (mq_quantize).
//
// ml-explore/mlx issue 4339, "Kernel microbenchmark": the weight is quantised
// with a group size and a bit width in "affine" mode before gather_qmm.  The
// page does not print the formula; this kernel implements the reading the
// library documents in mq.h (bias = group min, scale = fp32 span / (2^b - 1)
// rounded up to bf16, codes = rint of the IEEE fp32 quotient), operation for
// operation in fp32 so that codes, scales and biases are bit-exact with the
// CPU oracle.  Built without fast-math and without FP contraction.
//
// One thread per (row, group): the work is offline (weight preparation), so
// the kernel favours a plain, checkable structure over bandwidth.
#include "mq_internal.h"

namespace mq {
namespace {

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                       int cols, int gs,
                                                       uint32_t* __restrict__ wq,
                                                       uint16_t* __restrict__ scales,
                                                       uint16_t* __restrict__ biases) {
  constexpr int PER = 32 / BITS;              // codes per uint32 word
  constexpr uint32_t QMAX = (1u << BITS) - 1;
  const int G = cols / gs;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * G) return;
  const int64_t r = gid / G;
  const int g = int(gid - r * G);
  const uint16_t* src = w + r * cols + int64_t(g) * gs;

  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int k = 0; k < gs; ++k) {
    const float v = bf16_to_f32(src[k]);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  lo = lo + 0.0f;                              // -0.0 -> +0.0
  hi = hi + 0.0f;
  const float span = hi - lo;                  // IEEE fp32, round to nearest even
  const float q32 = __fdiv_rn(span, float(QMAX));
  const uint32_t qu = __float_as_uint(q32);
  const uint32_t sbits = (qu >> 16) + ((qu & 0xFFFFu) != 0u);   // round up (q32 >= 0)
  const float scale = __uint_as_float(sbits << 16);
  const uint32_t bbits = __float_as_uint(lo) >> 16;              // lo is a bf16 value

  uint32_t* dst = wq + r * (int64_t(cols) / PER) + int64_t(g) * gs / PER;
  for (int k0 = 0; k0 < gs; k0 += PER) {
    uint32_t word = 0;
    for (int j = 0; j < PER; ++j) {
      const float d = bf16_to_f32(src[k0 + j]) - lo;            // fp32 RNE
      uint32_t q = 0;
      if (scale != 0.0f) {
        float qf = __builtin_rintf(__fdiv_rn(d, scale));        // half to even
        qf = fminf(fmaxf(qf, 0.0f), float(QMAX));
        q = uint32_t(qf);
      }
      word |= q << (j * BITS);
    }
    dst[k0 / PER] = word;
  }
  scales[r * G + g] = uint16_t(sbits);
  biases[r * G + g] = uint16_t(bbits);
}

// ---- MXFP4 / MXFP8 (mq_quantize_mx) -------------------------------------------------
//
// OCP MX v1.0 MXFP4, the reading of the pages' mxfp4 mode (ml-explore/mlx pull
// 4023, the comment on block-height coverage): per 32 weights along K an E8M0
// exponent e = max(exponent field of the block's largest magnitude - 2, 0), i.e.
// floor(log2 amax) - 2 clamped at -127, and per weight the E2M1 code nearest to
// w / 2^(e - 127), ties to the even mantissa, magnitudes past 6 saturating, the
// sign bit kept.  The quotient is formed exactly in fp64 from the bf16 bits
// (no fp32 denormal mode can flush a subnormal weight) and the code is the
// number of E2M1 rounding thresholds it passes: a threshold is strict where
// the tie rounds down (to an even code) and inclusive where it rounds up.

// |w| of a bf16 pattern, exactly, in fp64
__device__ inline double bf16_mag_f64(uint32_t h) {
  const uint32_t ex = (h >> 7) & 0xFFu, m = h & 0x7Fu;
  return ex ? __hiloint2double(int(((ex + 896u) << 20) | (m << 13)), 0)
            : double(m) * 0x1p-133;
}

// E2M1 magnitude code of y >= 0
__device__ inline uint32_t e2m1_mag(double y) {
  return uint32_t(y > 0.25) + uint32_t(y >= 0.75) + uint32_t(y > 1.25) + uint32_t(y >= 1.75) +
         uint32_t(y > 2.5) + uint32_t(y >= 3.5) + uint32_t(y > 5.0);
}

__device__ inline uint32_t e2m1_code(uint32_t h, double inv_scale) {
  return e2m1_mag(bf16_mag_f64(h) * inv_scale) | ((h >> 12) & 8u);   // exact quotient
}

// MXFP8 (E4M3 elements): e = max(exponent field of amax - 8, 0); the quotient
// y < 512 is rounded at its binade's quantum by rint (half to even) on the
// scaled mantissa, a carry into the next binade falling out of the field
// arithmetic, and codes past 0x7E (448) saturate to it.
// E4M3 magnitude code of y >= 0
__device__ inline uint32_t e4m3_mag(double y) {
  uint32_t code;
  if (y < 0x1p-6) {
    code = uint32_t(rint(y * 0x1p9));                         // subnormal quantum 2^-9
  } else {
    const int ex = ilogb(y);                                   // -6 .. 8
    const int m = int(rint(ldexp(y, -ex) * 8.0));              // 8 .. 16
    code = uint32_t((ex + 7) * 8 + m - 8);
  }
  return min(code, 0x7Eu);
}

__device__ inline uint32_t e4m3_code(uint32_t h, double inv_scale) {
  return e4m3_mag(bf16_mag_f64(h) * inv_scale) | ((h >> 8) & 0x80u);  // exact quotient
}

// value of a non-negative E4M3 code (< 0x7F), exactly, in fp32
__device__ inline float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0x1p-9f;
}

template <int EB>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const uint16_t* __restrict__ w,
                                                          int64_t rows, int cols,
                                                          uint32_t* __restrict__ wq,
                                                          uint8_t* __restrict__ scales) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int NB = cols / 32;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * NB) return;
  const int64_t r = gid / NB;
  const int b = int(gid - r * NB);
  const u32x4* src = reinterpret_cast<const u32x4*>(w + r * cols + int64_t(b) * 32);
  u32x4 v[4];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = max(amax, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
  }
  const int e8 = max(int(amax >> 7) - (EB == 4 ? 2 : 8), 0);
  const double inv_scale = ldexp(1.0, 127 - e8);
  if constexpr (EB == 4) {
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {           // word i: weights 8 i .. 8 i + 7
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pair = v[i][j];
        word |= e2m1_code(pair & 0xFFFFu, inv_scale) << (8 * j);
        word |= e2m1_code(pair >> 16, inv_scale) << (8 * j + 4);
      }
      out[i] = word;
    }
    *reinterpret_cast<u32x4*>(wq + r * (cols / 8) + int64_t(b) * 4) = out;
  } else {
    uint32_t word[8];                       // word k: weights 4 k .. 4 k + 3
#pragma unroll
    for (int i = 0; i < 4; ++i)             // v[i][j]: weights 8 i + 2 j, +1
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pair = v[i][j];
        const uint32_t two = e4m3_code(pair & 0xFFFFu, inv_scale) | (e4m3_code(pair >> 16, inv_scale) << 8);
        const int k = 2 * i + (j >> 1);
        word[k] = (j & 1) ? (word[k] | (two << 16)) : two;
      }
    u32x4* d = reinterpret_cast<u32x4*>(wq + r * (cols / 4) + int64_t(b) * 8);
    d[0] = u32x4{word[0], word[1], word[2], word[3]};
    d[1] = u32x4{word[4], word[5], word[6], word[7]};
  }
  scales[r * NB + b] = uint8_t(e8);
}

// ---- NVFP4 (mq_quantize_nv) ---------------------------------------------------------
//
// NVIDIA's published NVFP4, the reading of the pages' nvfp4 mode (ml-explore/mlx
// pull 4023, the comment on block-height coverage): per tensor g = amax / 2688
// (1 for a zero tensor), per 16 weights s = e4m3(amax_block / 6 / g), per weight
// q = e2m1(w / (e4m3(s) * g)), every step an IEEE fp32 operation as the oracle
// performs it (built without contraction), so codes, scales and g are
// bit-identical.

// one workgroup per tensor: g[t] from the largest |w| of tensor t
__global__ __launch_bounds__(256) void nv_gscale_kernel(const uint16_t* __restrict__ w,
                                                        int64_t elems, float* __restrict__ g) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ uint32_t red[256];
  const int64_t t = blockIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + t * elems);
  uint32_t amax = 0;
  for (int64_t i = threadIdx.x; i < elems / 8; i += 256) {
    const u32x4 v = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float a = __uint_as_float(red[0] << 16);
    g[t] = red[0] ? __fdiv_rn(a, 2688.0f) : 1.0f;
  }
}

// one thread per (tensor, row, 16-weight block)
__global__ __launch_bounds__(256) void nv_quant_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                       int64_t rows_per_tensor, int cols,
                                                       const float* __restrict__ g,
                                                       uint32_t* __restrict__ wq,
                                                       uint8_t* __restrict__ scales) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int NB = cols / 16;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * NB) return;
  const int64_t r = gid / NB;
  const int b = int(gid - r * NB);
  const float gt = g[r / rows_per_tensor];
  const u32x4* src = reinterpret_cast<const u32x4*>(w + r * cols + int64_t(b) * 16);
  const u32x4 v[2] = {src[0], src[1]};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
  const float sb = __fdiv_rn(__fdiv_rn(__uint_as_float(amax << 16), 6.0f), gt);
  const uint32_t sc = e4m3_mag(double(sb));
  const float d = __fmul_rn(e4m3_to_f32(sc), gt);
  u32x2 out;
#pragma unroll
  for (int i = 0; i < 2; ++i) {             // word i: weights 8 i .. 8 i + 7
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t h = (v[i][j] >> (16 * half)) & 0xFFFFu;
        const float y = d > 0.0f ? __fdiv_rn(__uint_as_float(h << 16), d) : 0.0f;
        const uint32_t q = e2m1_mag(fabs(double(y))) | ((h >> 12) & 8u);
        word |= q << (8 * j + 4 * half);
      }
    out[i] = word;
  }
  *reinterpret_cast<u32x2*>(wq + r * (cols / 8) + int64_t(b) * 2) = out;
  scales[r * NB + b] = uint8_t(sc);
}

}  // namespace

hipError_t launch_quantize_nv(const uint16_t* w, int64_t tensors, int64_t rows, int64_t cols,
                              uint32_t* wq, uint8_t* scales, float* gscale, hipStream_t s) {
  if (tensors == 0 || rows == 0) return hipSuccess;
  note_dispatch("nv_gscale", {});
  nv_gscale_kernel<<<dim3(unsigned(tensors)), dim3(256), 0, s>>>(w, rows * cols, gscale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = tensors * rows * (cols / 16);
  const int64_t blocks = ceil_div(items, 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  note_dispatch("nv_quant", {});
  nv_quant_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, tensors * rows, rows, int(cols),
                                                                gscale, wq, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t* w, int64_t rows, int64_t cols, int bits,
                              uint32_t* wq, uint8_t* scales, hipStream_t s) {
  const int64_t items = rows * (cols / 32);
  if (items == 0) return hipSuccess;
  const int64_t blocks = ceil_div(items, 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  note_dispatch("quantize_mx", {bits == 8 ? 8 : 4});
  if (bits == 8)
    quantize_mx_kernel<8><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), wq, scales);
  else
    quantize_mx_kernel<4><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), wq, scales);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t cols, int group_size,
                           int bits, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                           hipStream_t s) {
  const int64_t items = rows * (cols / group_size);
  if (items == 0) return hipSuccess;
  const int64_t blocks = ceil_div(items, 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  note_dispatch("quantize", {bits == 4 ? 4 : 8});
  if (bits == 4)
    quantize_kernel<4><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), group_size,
                                                                    wq, scales, biases);
  else
    quantize_kernel<8><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), group_size,
                                                                    wq, scales, biases);
  return hipGetLastError();
}

}  // namespace mq
