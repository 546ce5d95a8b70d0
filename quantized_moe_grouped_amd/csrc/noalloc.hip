// mq_gather_qmm_noalloc: mq_gather_qmm with the library's own scratch as its
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch is one file-scope device array of MQ_NOALLOC_SCRATCH_BYTES.
// Each GPU the library runs on holds its own copy until the process ends.
// Its device address is looked up once per device, with that device current,
// on the first call there (hipGetSymbolAddress); host code only ever uses
// that address, never the array's name (which in host code is a host-side
// stand-in, not a device address).  The call then enqueues exactly what
// mq_gather_qmm enqueues, with the scratch as the workspace: every kernel
// takes the address as an argument, as it takes a caller's workspace.
//
// Nothing in the scratch needs clearing: each call's routing launch writes
// every workspace region the GEMM reads (counts, offsets, permutation, tile
// table, error word, row sums) before the GEMM runs, in stream order.  Calls
// that overlap on one GPU (other streams, other threads) share the array and
// race.
#include <algorithm>
#include <mutex>

#include "../../include/mq.h"
#include "mq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// The scratch of the current device (looked up on first use); nullptr if the
// lookup fails.
void* device_scratch(int dev) {
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

mq_status mq_gather_qmm_noalloc(const mq_bf16* x, int64_t T, int64_t Ax, int64_t M, int64_t K,
                                const uint32_t* wq, const mq_bf16* scales, const mq_bf16* biases,
                                int32_t E, int64_t N, const int32_t* rhs_indices, int64_t A,
                                int transpose, int group_size, int bits, int sorted_indices,
                                mq_bf16* out, void* stream) {
  // the workspace this call needs, from the same plan mq_gather_qmm makes
  // (host arithmetic only: shapes are validated before any HIP call)
  mq_ws_layout layout;
  const mq_status st = mq_gather_qmm_workspace(T, A, M, K, N, E, group_size, bits, &layout);
  if (st != MQ_OK) return st;
  // mq_gather_qmm's own checks, ahead of the device lookup below so that no
  // HIP call precedes them
  const int64_t n = T * A;
  if (Ax != 1 && Ax != A) return MQ_ERR_INVALID;
  if (n > 0 && (!x || !rhs_indices || (N > 0 && !out))) return MQ_ERR_INVALID;
  if (N > 0 && (!wq || !scales || !biases)) return MQ_ERR_INVALID;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if ((x && misaligned(x)) || (out && misaligned(out)) || (wq && misaligned(wq)))
    return MQ_ERR_INVALID;
  // the required regions must fit; the optional piece slots after them are
  // used as far as the scratch holds them
  if (layout.part > MQ_NOALLOC_SCRATCH_BYTES) return MQ_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MQ_ERR_HIP;
  if (stream) {
    // the scratch looked up is the current device's: the stream must be one
    // of its streams
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return MQ_ERR_HIP;
    if (sdev != dev) return MQ_ERR_INVALID;
  }
  void* ws = device_scratch(dev);
  if (!ws) return MQ_ERR_HIP;
  return mq_gather_qmm(x, T, Ax, M, K, wq, scales, biases, E, N, rhs_indices, A, transpose,
                       group_size, bits, sorted_indices, out, ws,
                       std::min<size_t>(layout.total, MQ_NOALLOC_SCRATCH_BYTES), stream);
}

}  // extern "C"
