// Internal declarations shared by the C ABI, the host codec builder and the
// HIP kernels of libtq.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "tq.h"

namespace tq {

constexpr int kMaxDevices = 16;
// Longest attended length a decode or prefill call takes (tokens per
// sequence): the general path merges at most 4096 chunks of at most 16384
// tokens, and the int8 matrix-core path keeps each wave's exact int32 value
// accumulators below 2^31 with chunks of at most 2^19 tokens (128 chunks).
constexpr int64_t kMaxDecodeLen = (int64_t)1 << 26;
constexpr int kGridMax = 16256;  // 127 * 128: |centroid| * 2^E bound
constexpr float kQjlConstNumer = 1.2533141373155003f;  // sqrt(pi/2)

// Host tables of a codec (float32 as stored; see tq_codec_export).
struct HostCodec {
  int d = 0, bits = 0, mode = 0, mse_bits = 0, levels = 0, grid_exp = 0;
  int split_dhi = 0;              // SPLIT: channels of the high part (the parts are separate codecs)
  uint64_t seed = 0;
  std::vector<float> rot;         // Pi [d][d] row-major, y = Pi x
  std::vector<float> sketch;      // S  [d][d] row-major (Prod)
  std::vector<float> centroids;   // [levels]
  std::vector<float> boundaries;  // [levels-1]
};

// Builds the codec; returns false with a message on unsupported parameters.
// The rotation's Gaussian is stream rot_stream of the seed (0; the high part of
// a split codec uses 2).
bool build_codec(int d, int bits, uint64_t seed, int mode, HostCodec* out, std::string* err, int rot_stream = 0);

// Device copies of the tables on one device.
struct DevTables {
  float* pit = nullptr;   // Pi^T [d][d]: pit[j*d + i] = Pi[i][j]
  float* pi = nullptr;    // Pi   [d][d] row-major
  float* st = nullptr;    // S^T  [d][d]: st[j*d + i] = S[i][j] (Prod)
  float* s = nullptr;     // S    [d][d] row-major (Prod)
  float* spt = nullptr;   // (S Pi)^T [d][d]: spt[j*d + i] = (S Pi)[i][j] (Prod)
  float* cent = nullptr;  // centroids [16] (SPLIT: the low part's)
  float* bnd = nullptr;   // boundaries [16]
  float* cent2 = nullptr; // SPLIT: the high part's centroids [16]
  float* bnd2 = nullptr;  // SPLIT: the high part's boundaries [16]
  void* block = nullptr;  // single allocation holding all of the above
};

}  // namespace tq

struct tq_codec {
  tq::HostCodec h;
  std::mutex mu;
  bool uploaded[tq::kMaxDevices] = {};
  tq::DevTables dev[tq::kMaxDevices];
  tq_codec* part[2] = {nullptr, nullptr};  // SPLIT: the low and high MSE codecs (owned)
};

namespace tq {

// ---- kernel launch parameters -------------------------------------------

struct QuantizeParams {
  const void* x;
  int x_bf16;
  int64_t s0, s1, s2;  // element strides of batch, head, token (coordinate stride 1)
  int batch, heads, n_new;
  int d, mode, mse_bits, levels, words, sign_words, groups, gbits;
  int x_vec16;        // x, its strides and element size allow 16-byte loads
  const float* pit;   // Pi^T
  const float* pi;    // Pi (row-major)
  const float* st;    // S^T (Prod)
  const float* s;     // S (row-major, Prod)
  const float* cent;  // centroids
  const float* bnd;   // boundaries
  uint32_t* idx;
  int idx_stride;     // words per token record of idx (= words, or a split cache's two parts' words)
  float* norm;
  float* rnorm;
  uint32_t* sign;
  float* scale;
  float* gmin;
  int64_t cap;
  const int32_t* pos;
  // hybrid-cache flush (0: an ordinary append at pos[b] + t): x is the
  // recent-token buffer of flush_block tokens, pos[b] the sequence's length
  // before the step's flush_new appended tokens; the buffer is quantised into
  // slots start .. start+flush_block-1, start = floor(pos[b] / flush_block) *
  // flush_block, when those tokens complete it, and nothing is written
  // otherwise
  int flush_block, flush_new;
};

// One or two parameter blocks (a key and a value append) in one launch;
// blockIdx.y selects the block.
struct QuantizeSets {
  QuantizeParams s[2];
};

// Appends of at most this many vectors per set use one workgroup per vector.
constexpr int64_t kSmallAppend = 4096;

hipError_t launch_quantize(const QuantizeSets& sets, int n_sets, hipStream_t stream);

struct DecodeParams {
  // query
  const void* q;
  int q_bf16;
  int batch, hq, hkv, q_len, group, rows;  // rows of this launch (<= 16)
  int row0;  // first row of the launch among the group * q_len rows of a KV head
  int d;
  float scale;
  // key codec / cache
  int kmode, kbits, kwords, ksign_words;
  const float* k_pit;   // Pi_k^T
  const float* k_pi;    // Pi_k row-major
  const float* k_spt;   // (S Pi)^T (Prod): the prologue's S q_rot = (S Pi) q
  const float* k_cent;
  const uint32_t* k_idx;
  const float* k_norm;
  const float* k_rnorm;
  const uint32_t* k_sign;
  // split keys: the high part starts at group ksplit_g (0: not split), its
  // codes have kbits + 1 bits, its centroids k_cent_hi, its norms k_norm_hi
  int ksplit_g;
  const float* k_cent_hi;
  const float* k_norm_hi;
  // value codec / cache
  int vmode, vbits, vwords, vgroups;
  int vsplit_g;               // as ksplit_g, for split values
  const float* v_cent_hi;
  const float* v_norm_hi;
  const float* v_pi;    // Pi_v row-major (inverse rotation of the output)
  const float* v_cent;
  const uint32_t* v_idx;
  const float* v_norm;
  const float* v_scale;
  const float* v_gmin;
  int64_t cap;
  const int32_t* len;
  // optional: the length the causal rule counts from (row i sees t <= lm -
  // q_len + i), when it differs from len (a hybrid cache: len its compressed
  // tokens, lm its whole length); NULL: len
  const int32_t* len_mask;
  // optional: the merge also writes each output row's softmax reference M and
  // sum L (log2 domain) as [batch][hq][q_len][2]; NULL: not written
  float* row_ml;
  // split over the token axis
  int chunk, n_chunks;
  // workspace pieces
  float* qrot;         // [batch*hkv][rows][d]
  float* qs;           // [batch*hkv][rows][d] (Prod)
  float* part_o;       // [batch*hkv][n_chunks][rows][d]
  float* part_ml;      // [batch*hkv][n_chunks][rows][2]
  float* out;          // [batch][hq][q_len][d]
  // MFMA path: the byte look-up tables of the two codebooks
  uint32_t klut[4];    // key centroid pieces: hi bytes 0-3, 4-7, lo bytes 0-3, 4-7
  uint32_t vlut[4];    // value centroid pieces
  int kgrid, vgrid;    // grid exponents E (centroid = integer * 2^-E)
};

// Chunk length of the token split and the workspace layout for it.
struct DecodePlan {
  int rows, chunk, n_chunks;
  size_t off_qrot, off_qs, off_part_o, off_part_ml, total;
  bool fast;
};
DecodePlan plan_decode(int batch, int hkv, int rows, int d, int64_t max_len, bool prod);

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// The general path's query rotation (qrot, qs) and cross-chunk merge, also
// used by the fp32 matrix-core kernel (head_dim 128 and 256).
hipError_t launch_qprep(const DecodeParams& p, hipStream_t stream);
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream);

// fp32 matrix-core decode for the modes the int8 kernel does not cover:
// head_dim 128/256, MSE or Prod keys of 1-4 index bits, MSE values of 1, 2
// or 4 bits or group values of 2 or 4 bits, up to 16 rows.  The plan splits
// each sequence's tokens into chunks; every wave of a workgroup writes its own
// partial, so the merge sees 4 partials per chunk.
bool mfma_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows);
bool mfma_decode_preferred(int d, int kmode, int kbits, int vmode, int vbits, int rows);
// fp32 matrix-core kernel over split keys and values (head_dim 128 or 256,
// each part half the channels, low parts of 1 to 3 bits); k_dlo, v_dlo: the
// low parts' channels
bool mfma_split_supported(int d, int kmode, int kbits, int k_dlo, int vmode, int vbits, int v_dlo, int rows);
// its resident 256-thread workgroups per compute unit at head_dim 128 (the
// launch bound and the chunk plan; two at 256)
constexpr int kSplitWgPerCu = 4;
// bf16 split-operand matrix-core kernel (head_dim 128, 1/2-bit MSE key codes,
// 1/2/4-bit MSE values), launched by launch_decode_mfma when it applies
bool bf16_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows);
bool bf16_prefill_supported(int d, int kmode, int kbits, int vmode, int vbits);
hipError_t launch_decode_bf16_kernel(const DecodeParams& p, const dim3 grid, hipStream_t stream);
DecodePlan plan_decode_mfma(int batch, int hkv, int rows, int d, int64_t max_len, bool prod, int wg_per_cu = 2);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);

// MFMA decode path: which shapes it covers, its plan and its launcher.
bool fast_decode_supported(int d, int kmode, int kbits, int vmode, int vbits, int rows);
DecodePlan plan_decode_fast(int batch, int hkv, int rows, int d, int64_t max_len);
hipError_t launch_decode_fast(const DecodeParams& p, hipStream_t stream);

// Prefill on the same codecs: query rows per launch (128 per workgroup), the
// plan (n_chunks = 0: the lengths need more chunks than the merge takes, and
// the caller uses the decode path per row block) and the launcher (query
// prologue, prefill kernel, merge).
constexpr int kPrefillRows = 1024;
DecodePlan plan_prefill_fast(int batch, int hkv, int rows, int64_t max_len);
hipError_t launch_prefill_fast(const DecodeParams& p, hipStream_t stream);
// prefill on the bf16 / int8 kernel's codecs (head_dim 128 or 256): 128 or
// 64 rows per workgroup over shared tiles (decode_bf16.hip), qprep and merge
// around it
DecodePlan plan_prefill_bf16(int batch, int hkv, int rows, int d, int64_t max_len);
hipError_t launch_prefill_bf16(const DecodeParams& p, hipStream_t stream);

// ---- token-record copies between caches of one codec ----------------------

constexpr int kMaxGatherBatch = 256;  // destination sequences per call
constexpr int kMaxFields = 4;         // idx + norm (MSE); idx, norm, rnorm, sign (Prod); idx, scale, gmin (group)

struct CacheGather {
  const uint32_t* src[kMaxFields];
  uint32_t* dst[kMaxFields];
  int width[kMaxFields];  // 32-bit elements per token-head of each field
  int n_fields;
  int heads, dst_batch;
  int64_t src_cap, dst_cap;
  int32_t src_batch[kMaxGatherBatch];  // -1: destination sequence not written
  int32_t src_start[kMaxGatherBatch];
  int32_t count[kMaxGatherBatch];
};

hipError_t launch_cache_gather(const CacheGather& g, int64_t max_count, hipStream_t stream);

// ---- the decode call behind the entry point that allocates nothing ------------

// tq_decode_attention's checks, plan and launches with the given workspace,
// refusing (instead of uploading) a codec whose tables are not on the current
// device yet; name prefixes the error messages.
tq_status decode_attention_in(const char* name, const tq_codec* kc, const tq_codec* vc, const void* q,
                              int32_t q_dtype, int32_t batch, int32_t hq, int32_t hkv, int32_t q_len,
                              const tq_cache* k, const tq_cache* v, const int32_t* d_len, int64_t max_len,
                              float scale, float* out, void* ws, size_t ws_bytes, void* stream);
// Records msg as the thread's last error and returns s.
tq_status set_error(tq_status s, const std::string& msg);

// ---- hybrid cache: the recent-token buffer --------------------------------------

// Copy of a step's new tokens into the rings (phase 0: the tokens of the block
// being filled; phase 1: those after it, once the full block is flushed).
struct HybridStage {
  const void* x[2];
  int64_t xs[2][3];   // element strides of batch, head, token (coordinate stride 1)
  void* buf[2];       // rings [batch][heads][block][d]
  int n_sets, bf16, batch, heads, n_new, d, block, phase;
  const int32_t* len; // tokens of each sequence before the step
};
hipError_t launch_hybrid_stage(const HybridStage& s, hipStream_t stream);
hipError_t launch_hybrid_lens(const int32_t* len, int32_t* lens_c, int batch, int block, hipStream_t stream);

// Exact attention over the rings and the merge with the compressed decode.
struct HybridAttn {
  const void* q;
  int q_bf16, batch, hq, hkv, q_len, group, d;
  float scale;
  const void* kbuf;
  const void* vbuf;
  int buf_bf16, block, has_compressed;
  const int32_t* len;    // whole length N of each sequence
  const float* row_ml;   // the compressed decode's (M, L) per output row
  float* out;            // holds the compressed decode's output; overwritten with the merge
};
hipError_t launch_hybrid_combine(const HybridAttn& a, hipStream_t stream);

// ---- measurement ------------------------------------------------------------

// Threads per workgroup of the streaming-read kernel.
constexpr int kStreamThreads = 256;
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, hipStream_t stream);
// decode_fast_kernel's loads (grid, chunks, tiles, two tiles in flight per
// wave) over the packed K/V state, with no arithmetic
hipError_t launch_decode_read(const DecodeParams& p, uint32_t* sink, uint32_t sink_words, hipStream_t stream);

}  // namespace tq
