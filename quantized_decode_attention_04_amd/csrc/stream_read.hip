// A plain streaming read of device memory, the measured reference beside the
// decode kernels' HBM figures: every byte of the buffer is loaded once with
// 16-byte loads (eight independent loads in flight per thread and round), and
// the words are folded into one value per thread so that the loads stay live.
// A result is stored only if it equals a value no realistic buffer folds to,
// so the kernel writes (almost) nothing.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const v4u* __restrict__ buf, uint64_t n16,
                                                               uint32_t* sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    v4u v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  stream_read_kernel<<<dim3(blocks), dim3(kThreads), 0, stream>>>(static_cast<const v4u*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace tq
