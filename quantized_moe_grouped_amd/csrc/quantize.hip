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

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t cols, int group_size,
                           int bits, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                           hipStream_t s) {
  const int64_t items = rows * (cols / group_size);
  if (items == 0) return hipSuccess;
  const int64_t blocks = ceil_div(items, 256);
  if (bits == 4)
    quantize_kernel<4><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), group_size,
                                                                    wq, scales, biases);
  else
    quantize_kernel<8><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(w, rows, int(cols), group_size,
                                                                    wq, scales, biases);
  return hipGetLastError();
}

}  // namespace mq
