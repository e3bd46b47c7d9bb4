// Kernel launchers of libtq.so replaced by stubs, for a host-only build of the
// C ABI, the codec builder and the dispatch logic under the address and
// undefined-behaviour sanitizers.  A stub reports hipErrorNoDevice; the host
// checks only call entry points whose validation refuses the arguments before
// any launch, so a stub being reached is itself reported by the driver.
#include "tq_internal.h"

namespace tq {

int g_stub_launches = 0;

hipError_t launch_quantize(const QuantizeSets&, int, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_qprep(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_merge(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_decode_bf16_kernel(const DecodeParams&, const dim3, hipStream_t) {
  ++g_stub_launches;
  return hipErrorNoDevice;
}
hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_decode_fast(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_prefill_fast(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_prefill_bf16(const DecodeParams&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_cache_gather(const CacheGather&, int64_t, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_hybrid_stage(const HybridStage&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_hybrid_lens(const int32_t*, int32_t*, int, int, hipStream_t) {
  ++g_stub_launches;
  return hipErrorNoDevice;
}
hipError_t launch_hybrid_combine(const HybridAttn&, hipStream_t) { ++g_stub_launches; return hipErrorNoDevice; }
hipError_t launch_stream_read(const void*, uint64_t, uint32_t*, int, hipStream_t) {
  ++g_stub_launches;
  return hipErrorNoDevice;
}
hipError_t launch_decode_read(const DecodeParams&, uint32_t*, uint32_t, hipStream_t) {
  ++g_stub_launches;
  return hipErrorNoDevice;
}

}  // namespace tq
