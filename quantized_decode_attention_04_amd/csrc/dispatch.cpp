// Which kernel takes a decode launch, and the chunk plan and workspace
// layout of each decode path.  Host code only (no HIP kernels), so that it can
// be built and checked on hosts without a GPU.
#include <algorithm>

#include "tq_internal.h"

namespace tq {
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// ---- which decode kernel covers which codecs ---------------------------------

// int8 matrix-core kernel (decode_fast.hip): head_dim 128, 3-bit MSE keys and
// values, up to 16 rows.
bool fast_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows) {
  return d == 128 && kmode == TQ_MODE_MSE && kbits == 3 && vmode == TQ_MODE_MSE && vbits == 3 && rows <= 16;
}

// bf16 split-operand kernel (decode_bf16.hip): head_dim 128 or 256, key codes
// of 1, 2 or 3 bits (MSE, or the MSE part of 2- to 4-bit Prod keys), MSE values of
// 1 to 4 bits or 2-bit group values, up to 16 rows (8 at head_dim 256).
bool bf16_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows) {
  const bool kok = (kmode == TQ_MODE_MSE || kmode == TQ_MODE_PROD) && kbits >= 1 && kbits <= 3;
  const bool vok = (vmode == TQ_MODE_MSE && vbits >= 1 && vbits <= 4) || (vmode == TQ_MODE_GROUP && vbits == 2);
  return (d == 128 || d == 256) && kok && vok && rows >= 1 && rows <= (d == 128 ? 16 : 8);
}

// Its shared-tile prefill kernel: the same codecs.
bool bf16_prefill_supported(int d, int kmode, int kbits, int vmode, int vbits) {
  return bf16_decode_supported(d, kmode, kbits, vmode, vbits, 1);
}

// fp32 matrix-core kernel (decode_mfma.hip).
bool mfma_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows) {
  const bool kok = (kmode == TQ_MODE_MSE || kmode == TQ_MODE_PROD) && kbits >= 1 && kbits <= 4;
  const bool vok = (vmode == TQ_MODE_MSE && (vbits == 1 || vbits == 2 || vbits == 4)) ||
                   (vmode == TQ_MODE_GROUP && (vbits == 2 || vbits == 4));
  return (d == 128 || d == 256) && kok && vok && rows >= 1 && rows <= (d == 128 ? 16 : 8);
}

// Split keys and values, each part half of head_dim 128 or 256: the fp32
// matrix-core kernel's split variant (decode_mfma.hip), at any row count.
bool mfma_split_supported(int d, int kmode, int kbits, int k_dlo, int vmode, int vbits, int v_dlo, int rows) {
  return (d == 128 || d == 256) && kmode == TQ_MODE_SPLIT && vmode == TQ_MODE_SPLIT && k_dlo == d / 2 &&
         v_dlo == d / 2 && kbits >= 1 && kbits <= 3 && vbits >= 1 && vbits <= 3 && rows >= 1 &&
         rows <= (d == 128 ? 16 : 8);
}

// Measured on MI355X: at head_dim 128 with more than 8 rows (prefill blocks,
// multi-token decode) the fp32 matrix-core kernel takes half the general
// kernel's time (whose work grows with the rows); at 8 rows or fewer, and at
// head_dim 256, the general kernel is as fast or faster.  Launches the bf16
// kernel covers (either head_dim) go through launch_decode_mfma as well.
bool mfma_decode_preferred(int d, int kmode, int kbits, int vmode, int vbits, int rows) {
  if (bf16_decode_supported(d, kmode, kbits, vmode, vbits, rows)) return true;
  return d == 128 && rows > 8 && mfma_decode_supported(d, kmode, kbits, vmode, vbits, rows);
}

// ---- chunk plans and workspace layouts ---------------------------------------

DecodePlan plan_decode(int batch, int hkv, int rows, int d, int64_t max_len, bool prod) {
  DecodePlan p{};
  p.rows = rows;
  const int64_t tile = 256;
  // about two 256-token tiles per workgroup: measured 6-7% faster than one
  // (the query prologue is amortised) and than four (fewer workgroups)
  const int64_t target_items = 512;
  const int64_t total = (int64_t)batch * hkv * max_len;
  int64_t chunk = (total + target_items - 1) / target_items;
  chunk = ((chunk + tile - 1) / tile) * tile;
  chunk = std::max<int64_t>(tile, std::min<int64_t>(chunk, 16384));
  p.chunk = (int)chunk;
  p.n_chunks = (int)((max_len + chunk - 1) / chunk);
  const size_t bg = (size_t)batch * hkv;
  size_t off = 0;
  p.off_qrot = off;
  off = align256(off + bg * rows * d * sizeof(float));
  p.off_qs = off;
  if (prod) off = align256(off + bg * rows * d * sizeof(float));
  p.off_part_o = off;
  off = align256(off + bg * p.n_chunks * rows * d * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + bg * p.n_chunks * rows * 2 * sizeof(float));
  p.total = off;
  return p;
}

// Compute units of the current device (256 on MI355X; the fallback when no
// device answers keeps workspace sizing usable on hosts without a GPU).
static int device_cus() {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Largest chunk of a batched launch on the matrix-core paths (tokens).
constexpr int64_t kRaggedChunk = 8192;
// The same for the four-wave decode kernels (two workgroups per compute unit).
// A ragged batch leaves the last chunk of every sequence short and the chunks
// past its end empty, so the busy workgroups come in uneven rounds; halving
// the cap doubles the rounds and evens them out.  Measured on 32 sequences of
// 1.2k..64k tokens (8 KV heads): 546 us per call at 8192, 473..488 us at
// 3072..6144, 551 us at 2048 (more partials for the merge).
constexpr int64_t kRaggedDecodeChunk = 4096;

DecodePlan plan_decode_mfma(int batch, int hkv, int rows, int d, int64_t max_len, bool prod, int wg_per_cu) {
  DecodePlan p{};
  p.rows = rows;
  const int64_t step = 256;  // four waves x 64-token tiles
  const int64_t heads = (int64_t)batch * hkv;
  // about wg_per_cu workgroups per compute unit (as many as the kernel keeps
  // resident); every wave writes a partial and the merge takes at most 4096
  // of them per row
  const int64_t per_head = std::max<int64_t>(1, (wg_per_cu * device_cus() + heads - 1) / heads);
  int64_t chunk = (max_len + per_head - 1) / per_head;
  // a batch may be ragged: the host knows only the longest sequence, so the
  // chunk is capped and a long sequence spreads over several workgroups
  // (chunks past a sequence's end exit at once)
  if (batch > 1) chunk = std::min<int64_t>(chunk, kRaggedDecodeChunk);
  chunk = std::max<int64_t>(step, ((chunk + step - 1) / step) * step);
  chunk = std::min<int64_t>(chunk, (int64_t)1 << 24);  // the bf16 kernel's 24-bit token offsets
  chunk = std::max<int64_t>(chunk, ((max_len + 1023) / 1024 + step - 1) / step * step);  // <= 1024 chunks
  p.chunk = (int)chunk;
  p.n_chunks = (int)((max_len + chunk - 1) / chunk);
  const size_t bg = (size_t)batch * hkv;
  const size_t parts = (size_t)p.n_chunks * 4;
  size_t off = 0;
  p.off_qrot = off;
  off = align256(off + bg * rows * d * sizeof(float));
  p.off_qs = off;
  if (prod) off = align256(off + bg * rows * d * sizeof(float));
  p.off_part_o = off;
  off = align256(off + bg * parts * rows * d * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + bg * parts * rows * 2 * sizeof(float));
  p.total = off;
  return p;
}

DecodePlan plan_decode_fast(int batch, int hkv, int rows, int d, int64_t max_len) {
  DecodePlan p{};
  p.rows = rows;
  p.fast = true;
  const int64_t step = 512;                 // eight waves x 64-token tiles
  const int64_t heads = (int64_t)batch * hkv;
  const int64_t per_head = std::max<int64_t>(1, (device_cus() + heads - 1) / heads);  // one workgroup per CU
  int64_t chunk = (max_len + per_head - 1) / per_head;
  if (batch > 1) chunk = std::min<int64_t>(chunk, kRaggedChunk);  // as in plan_decode_mfma
  chunk = ((chunk + step - 1) / step) * step;
  chunk = std::max<int64_t>(step, chunk);
  // at most 2^19 tokens per chunk (the kernel's int32 accumulator bound),
  // which with max_len <= 2^26 still leaves <= 128 chunks
  chunk = std::min<int64_t>(chunk, (int64_t)1 << 19);
  chunk = std::max<int64_t>(chunk, ((max_len + 127) / 128 + step - 1) / step * step);  // <= 128 chunks
  p.chunk = (int)chunk;
  p.n_chunks = (int)((max_len + chunk - 1) / chunk);
  const size_t bg = (size_t)batch * hkv;
  size_t off = 0;
  p.off_part_o = off;
  off = align256(off + bg * p.n_chunks * rows * d * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + bg * p.n_chunks * rows * 2 * sizeof(float));
  p.total = off;
  return p;
}

DecodePlan plan_prefill_fast(int batch, int hkv, int rows, int64_t max_len) {
  DecodePlan p{};
  p.rows = rows;
  p.fast = true;
  const int64_t tile = 64;                    // every wave walks every tile of its chunk
  const int64_t max_chunk = (int64_t)1 << 16;  // the int32 value-accumulator bound of a wave
  const int64_t max_chunks = 128;              // merge weights kept in LDS
  const int64_t row_groups = (rows + 127) / 128;
  const int64_t units = (int64_t)batch * hkv * row_groups;
  // about one workgroup per compute unit (one fits, at 120 KB of LDS)
  const int64_t per = std::max<int64_t>(1, (device_cus() + units - 1) / units);
  int64_t chunk = (max_len + per - 1) / per;
  if (batch > 1) chunk = std::min<int64_t>(chunk, kRaggedChunk);  // as in plan_decode_mfma
  chunk = std::max<int64_t>(tile, (chunk + tile - 1) / tile * tile);
  chunk = std::min<int64_t>(chunk, max_chunk);
  chunk = std::max<int64_t>(chunk, ((max_len + max_chunks - 1) / max_chunks + tile - 1) / tile * tile);
  if (chunk > max_chunk || chunk * max_chunks < max_len || ((max_len + chunk - 1) / chunk) * row_groups > 65535) {
    p.n_chunks = 0;  // longer than the merge takes: the caller falls back to row blocks
    return p;
  }
  p.chunk = (int)chunk;
  p.n_chunks = (int)((max_len + chunk - 1) / chunk);
  const size_t bg = (size_t)batch * hkv;
  size_t off = 0;
  p.off_qrot = off;
  off = align256(off + bg * rows * 128 * sizeof(float));
  p.off_qs = off;
  p.off_part_o = off;
  off = align256(off + bg * p.n_chunks * rows * 128 * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + bg * p.n_chunks * rows * 2 * sizeof(float));
  p.total = off;
  return p;
}

DecodePlan plan_prefill_bf16(int batch, int hkv, int rows, int d, int64_t max_len) {
  DecodePlan p{};
  p.rows = rows;
  const int64_t tile = 64;                    // a multiple of both kernels' tiles
  const int64_t max_chunks = 4096;            // the merge kernel's weights in LDS
  const int64_t group = d == 128 ? 128 : 64;  // rows per workgroup
  const int64_t row_groups = (rows + group - 1) / group;
  const int64_t units = (int64_t)batch * hkv * row_groups;
  // about one workgroup per compute unit (one fits, at 130 KB of LDS)
  const int64_t per = std::max<int64_t>(1, (device_cus() + units - 1) / units);
  int64_t chunk = (max_len + per - 1) / per;
  if (batch > 1) chunk = std::min<int64_t>(chunk, kRaggedChunk);  // as in plan_decode_mfma
  chunk = std::max<int64_t>(tile, (chunk + tile - 1) / tile * tile);
  chunk = std::max<int64_t>(chunk, ((max_len + max_chunks - 1) / max_chunks + tile - 1) / tile * tile);
  if (chunk > ((int64_t)1 << 24) || ((max_len + chunk - 1) / chunk) * row_groups > 0x7fffffff) {
    p.n_chunks = 0;  // the caller falls back to row blocks
    return p;
  }
  p.chunk = (int)chunk;
  p.n_chunks = (int)((max_len + chunk - 1) / chunk);
  const size_t bg = (size_t)batch * hkv;
  size_t off = 0;
  p.off_qrot = off;
  off = align256(off + bg * rows * d * sizeof(float));
  p.off_qs = off;
  off = align256(off + bg * rows * d * sizeof(float));
  p.off_part_o = off;
  off = align256(off + bg * p.n_chunks * rows * d * sizeof(float));
  p.off_part_ml = off;
  off = align256(off + bg * p.n_chunks * rows * 2 * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace tq
