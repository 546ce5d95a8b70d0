// Calibration probes (libmq_probe.so, C ABI in include/mq_probe.h): the HBM
// read bandwidth and the dense bf16 MFMA rate this GPU delivers, measured by
// the caller (events around the call).  They are the references next to which
// the benchmark reads the roofline fractions of the GEMM and small-M kernels
// (the published peaks are 8 TB/s and 2.5 PFLOP/s).  Not part of libmq.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mq_probe.h"

namespace mq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;                     // 16-byte loads in flight per lane

// Every lane reads 16-byte elements i, i + stride, ... (consecutive lanes,
// consecutive elements: each wave load is 1 KB of one contiguous range),
// kInFlight of them issued before any is used; the XOR of all words goes to
// the lane's sink word so that no load can be dropped.
__global__ __launch_bounds__(kThreads) void probe_stream(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// Eight independent accumulators per wave, each one v_mfma_f32_16x16x32_bf16
// per round on register operands (no memory traffic inside the loop).  The
// operands are random bf16 (random sign and mantissa, exponents 2^-4 .. 2^3)
// and change from one MFMA to the next, as a GEMM's do: the matrix cores
// draw power by the bits they switch, and with near-constant operands this
// loop runs about 20% faster than any real GEMM can.
__device__ inline uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  return h;
}
__device__ inline uint32_t rand_bf16x2(uint32_t seed) {
  const uint32_t h = mix32(seed);
  const uint32_t lo = (h & 0x807Fu) | ((0x3Bu + ((h >> 7) & 7u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807Fu) | ((0x3Bu + ((h >> 23) & 7u)) << 7);
  return lo | (hi << 16);
}
__global__ __launch_bounds__(kThreads) void probe_mfma(int iters, float* __restrict__ sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  u32x4 a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[j][i] = rand_bf16x2(t * 32u + uint32_t(j * 4 + i));
      b[j][i] = rand_bf16x2(t * 32u + 16u + uint32_t(j * 4 + i));
    }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j & 3]),
                                                       __builtin_bit_cast(bf16x8, b[(j >> 1) & 3]),
                                                       acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace mq

extern "C" {

mq_status mq_probe_stream(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                          void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || workgroups < 1 ||
      (reinterpret_cast<uintptr_t>(src) & 15u))
    return MQ_ERR_INVALID;
  mq::probe_stream<<<dim3(unsigned(workgroups)), dim3(mq::kThreads), 0,
                     static_cast<hipStream_t>(stream)>>>(static_cast<const mq::u32x4*>(src),
                                                        bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

mq_status mq_probe_mfma(int32_t iters, float* sink, int32_t workgroups, void* stream) {
  if (!sink || iters < 1 || workgroups < 1) return MQ_ERR_INVALID;
  mq::probe_mfma<<<dim3(unsigned(workgroups)), dim3(mq::kThreads), 0,
                   static_cast<hipStream_t>(stream)>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_HIP;
}

}  // extern "C"
