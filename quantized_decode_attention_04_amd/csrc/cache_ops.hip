// Token-record copies between compressed caches of one codec ("omlx
// turboquant_kv.py", BatchTurboQuantKVCache.filter / extract / extend /
// merge: batch rows are selected, split off or joined; the packed state moves
// as it is, never re-quantised).
//
// A cache is structure-of-arrays [batch][heads][cap][width] per field, so the
// tokens s0 .. s0+n-1 of one (sequence, head) are one contiguous run of n *
// width 32-bit elements in every field.  One launch copies, for every
// destination sequence and head, that run of every field: workgroup (x, h, b)
// streams a slice of the runs of sequence b, head h with 16-byte vector
// copies where both ends are aligned and 4-byte copies otherwise.
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ void copy_run(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t n,
                                         int64_t first, int64_t stride) {
  const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  if (vec) {
    const int64_t n4 = n / 4;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (int64_t e = first; e < n4; e += stride) d4[e] = s4[e];
    for (int64_t e = 4 * n4 + first; e < n; e += stride) dst[e] = src[e];
  } else {
    for (int64_t e = first; e < n; e += stride) dst[e] = src[e];
  }
}

__global__ __launch_bounds__(256) void cache_gather_kernel(CacheGather g) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int sb = g.src_batch[b];
  if (sb < 0) return;
  const int64_t n = g.count[b];
  const int64_t s_slot = ((int64_t)sb * g.heads + h) * g.src_cap + g.src_start[b];
  const int64_t d_slot = ((int64_t)b * g.heads + h) * g.dst_cap;
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int f = 0; f < g.n_fields; ++f) {
    const int w = g.width[f];
    copy_run(g.src[f] + s_slot * w, g.dst[f] + d_slot * w, n * w, first, stride);
  }
}

}  // namespace

hipError_t launch_cache_gather(const CacheGather& g, int64_t max_count, hipStream_t stream) {
  if (g.dst_batch < 1 || g.dst_batch > kMaxGatherBatch || g.heads < 1 || g.heads > 65535) return hipErrorInvalidValue;
  int wmax = 1;
  for (int f = 0; f < g.n_fields; ++f) wmax = g.width[f] > wmax ? g.width[f] : wmax;
  // about 16 KiB of the widest field per workgroup
  int64_t blocks = (max_count * wmax + 4095) / 4096;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  cache_gather_kernel<<<dim3((unsigned)blocks, (unsigned)g.heads, (unsigned)g.dst_batch), dim3(256), 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace tq
