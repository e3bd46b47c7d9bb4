// tq_decode_attention_noalloc: the decode call for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid it).  Its scratch -- the per-chunk partial results that
// tq_decode_attention keeps in a caller workspace -- lives in a file-scope
// device array of kScratchBytes that every device the library runs on holds
// until the process ends.
//
// Host code must not pass `scratch` itself to a kernel: in host code the name
// is a host-side stand-in, not a device address.  The device address of each
// device's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; only that pointer is used.
#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array (looked up on the
// first call on that device).
tq_status scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(TQ_ERR_NO_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(TQ_ERR_UNSUPPORTED, "device index above 15");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(TQ_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_decode_attention_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q,
                                                 int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t q_len, const tq_cache* k,
                                                 const tq_cache* v, const int32_t* d_len, int64_t max_len,
                                                 float scale, float* out, void* stream) {
  // the size check is host arithmetic only; it also validates the shapes
  size_t need = 0;
  tq_status st = tq_decode_workspace_size(kc, vc, batch, n_q_heads, n_kv_heads, q_len, max_len, &need);
  if (st != TQ_OK) return st;
  if (need > tq::kScratchBytes)
    return tq::set_error(TQ_ERR_WORKSPACE, "tq_decode_attention_noalloc: these sizes need " + std::to_string(need) +
                                               " bytes of scratch, more than the " +
                                               std::to_string(tq::kScratchBytes) +
                                               " the library holds per device (use tq_decode_attention)");
  void* ws = nullptr;
  st = tq::scratch_on_device(&ws);
  if (st != TQ_OK) return st;
  return tq::decode_attention_in("tq_decode_attention_noalloc", kc, vc, q, q_dtype, batch, n_q_heads, n_kv_heads,
                                 q_len, k, v, d_len, max_len, scale, out, ws, tq::kScratchBytes, stream);
}
