/*
 * tq.h -- TurboQuant compressed KV cache for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libtq.so.  Three operations:
 *   tq_codec_create       build a codec (rotation, Lloyd-Max codebook, QJL sketch)
 *   tq_quantize_append    compress new K or V head vectors into a cache
 *   tq_decode_attention   decode attention of queries over a compressed cache
 *
 * Sources ("the pages"):
 *   [plan]   "lightning-mlx plan.md": feasibility of TurboQuant at 256k
 *            context; decode is bound by reading the whole KV of every layer
 *            each step; decompression = unpack + Lloyd-Max lookup,
 *            denormalise, inverse rotation; a fused attention kernel over
 *            the codes is what makes it viable.
 *   [omlx]   "omlx turboquant_kv.py": BatchTurboQuantKVCache; the state
 *            types TurboQuantMSEState(norms, indices) and
 *            TurboQuantProdState(norms, mse_indices, residual_norms,
 *            qjl_signs); packed width ceil(head_dim*bits/32) uint32 words
 *            (_infer_head_dim); codecs rebuilt from (head_dim, bits, seed)
 *            with the K codec on seed s and the V codec on seed s+1
 *            (_rebuild_codecs); new tokens are written at the written end
 *            (update_and_fetch) and see the cache causally (make_mask);
 *            mixed (bits, seed) caches are refused (merge).
 *   [val]    "turboquant validate_moe_phase2.py": TurboQuantProd keys
 *            (3-bit = 2-bit MSE + 1-bit QJL), value group quantisation
 *            quantize_values(v, bits, group_size=32) -> data, scales, zeros;
 *            attention scores scaled by 1/sqrt(head_dim); Pi and S are
 *            d x d float32 matrices.
 *
 * Conventions
 *   - All device pointers are caller-owned device memory on the current HIP
 *     device.  The library owns only codec objects and their tables.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every device operation is asynchronous on that stream; nothing
 *     synchronises implicitly (except the one-time table upload of a codec
 *     on a device, which uses hipMemcpy).
 *   - Arguments are validated on the host before any launch; a failing call
 *     launches nothing and returns a status, with a message retrievable via
 *     tq_last_error() on the same thread.  No exception crosses the ABI.
 *   - head_dim is a multiple of 32, at most 256.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,     /* null pointer, bad size, bad stride */
  TQ_ERR_UNSUPPORTED = 2,     /* parameter combination not implemented */
  TQ_ERR_CONFIG_MISMATCH = 3, /* K/V codecs or caches disagree ([omlx] merge) */
  TQ_ERR_CAPACITY = 4,        /* a length exceeds the cache capacity */
  TQ_ERR_WORKSPACE = 5,       /* workspace missing or too small */
  TQ_ERR_HIP = 6,             /* a HIP runtime call or launch failed */
  TQ_ERR_NO_DEVICE = 7        /* no usable HIP device */
} tq_status;

/* Quantiser modes.
 *   MSE:   rotate, store the float32 norm and the packed nearest-centroid
 *          indices of the normalised rotated vector ([omlx] TurboQuantMSEState).
 *          bits 1..4.
 *   PROD:  MSE at bits-1 plus 1-bit QJL signs of the rotated residual and its
 *          float32 norm ([omlx] TurboQuantProdState; [val] 3-bit keys =
 *          MSE + QJL).  bits 2..5.  Keys only.
 *   GROUP: asymmetric min-max quantisation of the unrotated vector in groups
 *          of 32 coordinates with float32 scale and minimum per group ([val]
 *          quantize_values).  bits 1..4.  Values only.
 *   SPLIT: a fractional width b ([omlx] TurboQuantSplitState(low, high)):
 *          the first d_lo channels through a floor(b)-bit MSE codec ("low"),
 *          the last d_hi = round((b - floor b) * head_dim / 32) * 32 channels
 *          through a ceil(b)-bit one ("high"), each with its own rotation,
 *          norm and codebook.  Built by tq_codec_create_split only.  Keys or
 *          values.                                                         */
typedef enum { TQ_MODE_MSE = 0, TQ_MODE_PROD = 1, TQ_MODE_GROUP = 2, TQ_MODE_SPLIT = 3 } tq_mode;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef struct tq_codec tq_codec; /* opaque, immutable after creation */

typedef struct {
  int32_t head_dim;
  int32_t bits;        /* bits per coordinate as requested (Prod includes the sign bit); SPLIT: floor(b) */
  int32_t mode;        /* tq_mode */
  int32_t mse_bits;    /* bits of the packed index stream: bits (MSE, GROUP) or bits-1 (PROD); SPLIT: low part's */
  int32_t levels;      /* 2^mse_bits (MSE, PROD, SPLIT low part); 0 in GROUP mode */
  int32_t idx_words;   /* words per token-head of idx: head_dim*mse_bits/32 ([omlx] _infer_head_dim);
                          SPLIT: the low part's words plus the high part's (= ceil(head_dim*b/32)
                          when (b - floor b)*head_dim is a multiple of 32) */
  int32_t sign_words;  /* head_dim/32 in PROD mode, else 0 */
  int32_t groups;      /* head_dim/32 in GROUP mode, else 0 */
  int32_t grid_exp;    /* E: every centroid is an integer multiple of 2^-E (|c| 2^E <= 16256); SPLIT: low part's */
  int32_t split_high_dim; /* SPLIT: d_hi, channels of the high part (the last ones); else 0 */
  uint64_t seed;
  uint64_t bytes_per_token; /* compressed bytes per token-head (state only) */
} tq_codec_info;

/* A compressed cache for one of K or V: caller-owned device arrays laid out
 * [batch][heads][cap][...] in row-major order.  Which arrays are used
 * depends on the codec's mode; unused ones may be NULL.
 *   idx    uint32 [..][cap][idx_words]   MSE indices / Prod mse_indices / group data
 *   norm   float  [..][cap]              MSE and Prod: vector norm
 *   rnorm  float  [..][cap]              Prod: residual norm
 *   sign   uint32 [..][cap][sign_words]  Prod: QJL sign bits, bit j = coordinate j
 *   scale  float  [..][cap][groups]      GROUP: (max-min)/(2^bits-1) per group
 *   gmin   float  [..][cap][groups]      GROUP: minimum per group ("zeros")
 * A SPLIT cache holds both sub-states of [omlx] TurboQuantSplitState(low,
 * high) in one token record: idx is the low part's packed words followed by
 * the high part's (idx_words in all), norm the low part's norm and rnorm the
 * high part's.
 * Packed layout of idx: see the codec section of the library's design notes;
 * for 1, 2 and 4 bits it is an LSB-first stream (index j at bits
 * [b*j, b*j+b) of the word stream); 3-bit indices use a byte-lane layout
 * in which each 32 coordinates own three words. */
typedef struct {
  uint32_t* idx;
  float* norm;
  float* rnorm;
  uint32_t* sign;
  float* scale;
  float* gmin;
  int32_t batch;
  int32_t heads;
  int64_t cap;
} tq_cache;

/* Build a codec, deterministic in (head_dim, bits, seed, mode) ([omlx]
 * _rebuild_codecs).  Host-only: tables are uploaded to a device on first
 * use there (or by tq_codec_upload).  Caller owns *out; release it with
 * tq_codec_destroy.  Errors: INVALID_ARG (out == NULL), UNSUPPORTED (head_dim
 * not a multiple of 32 in 32..256, bits out of range for the mode). */
tq_status tq_codec_create(int32_t head_dim, int32_t bits, uint64_t seed, int32_t mode, tq_codec** out);

/* The two codecs of a cache of width `bits` ([omlx] _rebuild_codecs): when
 * bits is fractional (not within 1e-6 of an integer) the key codec takes
 * floor(bits) and the value codec ceil(bits), else both take bits; both are
 * MSE codecs, the key one on `seed` and the value one on seed + 1.  The
 * caller owns both (tq_codec_destroy).  Errors: INVALID_ARG (NULL), UNSUPPORTED
 * (a resulting width outside 1..4 bits, head_dim as for tq_codec_create). */
tq_status tq_codec_create_kv(int32_t head_dim, double bits, uint64_t seed, tq_codec** key_out, tq_codec** value_out);

/* A SPLIT codec of fractional width `bits` (see tq_mode): the low part is the
 * MSE codec (d_lo, floor(bits), seed) with its rotation from stream 0 of the
 * seed, the high part the MSE codec (d_hi, ceil(bits), seed) with its
 * rotation from stream 2.  Errors: INVALID_ARG (out NULL), UNSUPPORTED
 * (bits within 1e-6 of an integer, a part with fewer than 32 channels, a
 * part outside 1..4 bits, head_dim not a multiple of 32 in 64..256). */
tq_status tq_codec_create_split(int32_t head_dim, double bits, uint64_t seed, tq_codec** out);

/* The low (which = 0) or high (which = 1) part of a SPLIT codec, as an MSE
 * codec of the part's channels, owned by `codec` (valid until it is
 * destroyed; never pass it to tq_codec_destroy).  Use it to export a part's
 * tables.  Errors: INVALID_ARG (not a SPLIT codec, which not 0 or 1). */
tq_status tq_codec_part(const tq_codec* codec, int32_t which, const tq_codec** out);

/* Free a codec and its device tables.  NULL is a no-op.  The caller must make
 * sure no work using it is still queued on any stream. */
void tq_codec_destroy(tq_codec* codec);

/* Describe a codec (sizes of the state it produces). */
tq_status tq_codec_get_info(const tq_codec* codec, tq_codec_info* info);

/* Copy the codec's float32 tables to host memory.  Any pointer may be NULL.
 *   rot        [head_dim][head_dim] Pi, row-major; the rotation is y = Pi x
 *   centroids  [levels] ascending
 *   boundaries [levels-1] midpoints of neighbouring centroids
 *   sketch     [head_dim][head_dim] S (PROD only; left untouched otherwise)
 * GROUP codecs have no tables (returns OK and writes nothing).  SPLIT codecs
 * write the block-diagonal rotation (low part's rotation on channels 0..d_lo-1,
 * the high part's on the rest) and the low part's centroids and boundaries
 * (tq_codec_part exports either part's own tables). */
tq_status tq_codec_export(const tq_codec* codec, float* rot, float* centroids, float* boundaries, float* sketch);

/* Upload the codec's tables to the current device now (otherwise done on
 * first use, with a blocking hipMemcpy).  Idempotent per device. */
tq_status tq_codec_upload(const tq_codec* codec);

/* Quantise-on-append ([omlx] update_and_fetch: only the new tokens are
 * quantised and written at the written end; [plan]: append incremental per
 * token).
 *   x        device, n_new new head vectors per (batch, head), element
 *            (b, h, t, j) at x + b*s0 + h*s1 + t*s2 + j*s3 (element strides
 *            x_strides[0..3], s3 == 1 required), dtype x_dtype
 *   dst      the cache to write; dst->batch == batch, dst->heads == heads
 *   d_pos    device int32[batch]: token t of sequence b goes to position
 *            d_pos[b] + t
 *   pos_end  host bound on the written end after the append: the caller
 *            guarantees d_pos[b] + n_new <= pos_end for every b (the
 *            positions live on the device, so the library checks the bound,
 *            not the positions).  pos_end > dst->cap is refused with
 *            CAPACITY before anything is launched.  A device position that
 *            breaks the caller's guarantee (d_pos[b] < 0, or a token at or
 *            past cap) is never written out of bounds: such tokens are
 *            dropped.
 * Errors: INVALID_ARG (pos_end < n_new, ...), CONFIG_MISMATCH (cache shape),
 * CAPACITY (pos_end > cap), HIP. */
tq_status tq_quantize_append(const tq_codec* codec, const void* x, int32_t x_dtype, int32_t batch, int32_t heads,
                             int32_t n_new, const int64_t* x_strides, const tq_cache* dst, const int32_t* d_pos,
                             int64_t pos_end, void* stream);

/* Quantise the new keys and values of one decode step in one call ([omlx]
 * update_and_fetch appends keys and values together): one kernel launch when
 * both codecs take the same append kernel, two when they differ (at head_dim
 * <= 128 MSE caches take a per-group kernel, Prod and group caches a
 * per-vector one).  Same semantics and
 * errors as two tq_quantize_append calls, one with (kc, k, k_strides, kdst)
 * and one with (vc, v, v_strides, vdst), sharing dtype, sizes, d_pos and
 * pos_end (CAPACITY if pos_end exceeds either cache's cap); kc and vc must
 * have the same head_dim (else CONFIG_MISMATCH). */
tq_status tq_quantize_append_kv(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v,
                                int32_t x_dtype, int32_t batch, int32_t heads, int32_t n_new,
                                const int64_t* k_strides, const int64_t* v_strides, const tq_cache* kdst,
                                const tq_cache* vdst, const int32_t* d_pos, int64_t pos_end, void* stream);

/* Bytes of device workspace tq_decode_attention needs for these sizes (the
 * per-chunk partial results of the split over the token axis). */
tq_status tq_decode_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t q_len, int64_t max_len, size_t* bytes);

/* Decode attention over the compressed cache ([val] Tests 1 and 5: scaled
 * scores, softmax, weighted values, compared in the original domain; [plan]:
 * a fused kernel over the codes instead of dequantising K and V).
 *   q        device [batch][n_q_heads][q_len][head_dim], dtype q_dtype
 *   k, v     caches written by tq_quantize_append with kc and vc
 *            (kc: MSE or PROD; vc: MSE or GROUP; equal head_dim)
 *   d_len    device int32[batch]: attended length N_b of each sequence
 *            (after the q_len new tokens were appended); clamped to cap;
 *            every N_b must be <= max_len (tokens beyond max_len are ignored)
 *   max_len  host bound on the lengths, 1 <= max_len <= cap and
 *            max_len <= 2^26 (67,108,864 tokens per sequence; UNSUPPORTED
 *            above); sizes the grid
 *   scale    softmax scale (1/sqrt(head_dim) in [val])
 *   out      device float [batch][n_q_heads][q_len][head_dim]
 *   ws       device workspace of ws_bytes >= tq_decode_workspace_size(...),
 *            caller-owned; its contents need no initialisation.  Calls that
 *            share a workspace must not run concurrently.
 * Query head h reads KV head h / (n_q_heads / n_kv_heads); row i of q_len
 * sees tokens t <= N_b - q_len + i ([omlx] make_mask: causal for new tokens).
 * A row that sees no token gets zeros.
 * Errors: INVALID_ARG, UNSUPPORTED (more than 16 rows per KV head, 8 above
 * head_dim 128: use tq_prefill_attention; max_len above 2^26), CONFIG_MISMATCH, CAPACITY
 * (max_len > cap), WORKSPACE, HIP. */
tq_status tq_decode_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t q_len, const tq_cache* k,
                              const tq_cache* v, const int32_t* d_len, int64_t max_len, float scale, float* out,
                              void* ws, size_t ws_bytes, void* stream);

/* tq_decode_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  Same arguments, semantics and errors, without ws / ws_bytes:
 * the per-chunk partial results go to a device array the library holds, 64
 * MiB per device (every device the library runs on keeps it until the
 * process ends).  The call allocates nothing -- no hipMalloc, hipFree or
 * allocating library routine -- so both codecs' tables must already be on
 * the current device (tq_codec_upload, or any earlier call that used them
 * there), else INVALID_ARG.  Sizes whose workspace (tq_decode_workspace_size)
 * exceeds 64 MiB are refused with WORKSPACE.  Every call on one device shares
 * that device's array, which keeps the last call's contents (the decode
 * writes every partial it reads, so nothing needs clearing): calls that
 * overlap on one device -- on different streams or threads -- race, and must
 * be ordered by the caller. */
tq_status tq_decode_attention_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype,
                                      int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t q_len,
                                      const tq_cache* k, const tq_cache* v, const int32_t* d_len, int64_t max_len,
                                      float scale, float* out, void* stream);

/* Bytes of device workspace tq_prefill_attention needs for these sizes (one
 * launch of rows at a time reuses it). */
tq_status tq_prefill_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t q_len, int64_t max_len, size_t* bytes);

/* Prefill attention over the compressed cache ([omlx] prefill_attention:
 * many new tokens attend to the cache and, causally, to each other, as in
 * make_mask).  Same arguments, layouts, masking, ownership and errors as
 * tq_decode_attention, with any q_len >= 1.  The (n_q_heads / n_kv_heads) *
 * q_len rows of each KV head run in launches of up to 1024 rows, one after
 * the other on the stream: on the 3-bit MSE head_dim 128 codecs and on the
 * codecs of the bf16 decode kernel (key codes of 1 to 3 bits, 1- to 4-bit
 * MSE or 2-bit group values, head_dim 128 or 256) a workgroup takes 128 rows (64
 * at head_dim 256) and reads each tile of the state once for them; other
 * codecs run the rows in blocks of 16 (8 above head_dim 128) through the
 * decode kernels, so their cost grows with the number of blocks.  ws must
 * hold tq_prefill_workspace_size(...) bytes.  UNSUPPORTED above 2^30 rows per
 * KV head. */
tq_status tq_prefill_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t q_len, const tq_cache* k,
                               const tq_cache* v, const int32_t* d_len, int64_t max_len, float scale, float* out,
                               void* ws, size_t ws_bytes, void* stream);

/* Copy token records between caches of one codec, for batch bookkeeping
 * ([omlx] BatchTurboQuantKVCache filter, extract, extend and merge select,
 * split off or join batch rows; merge refuses caches of different bits or
 * seed).  For every destination sequence b < dst->batch with
 * src_batch[b] >= 0, the records of tokens src_start[b] .. src_start[b] +
 * count[b] - 1 of source sequence src_batch[b] (every head, every field of
 * the codec's mode) are copied unchanged to slots 0 .. count[b] - 1 of
 * destination sequence b; other slots, and rows with src_batch[b] < 0, are
 * left as they are.  Lengths are the caller's (as for decode); trimming the
 * last tokens of a sequence is a length change only.
 *   src_codec, dst_codec  the codecs the caches were written with: head_dim,
 *                         bits, mode and seed must agree (else
 *                         CONFIG_MISMATCH, like [omlx] merge)
 *   src, dst              caches with equal head counts; the copied ranges
 *                         must not overlap (distinct allocations)
 *   src_batch, src_start, count  host int32 arrays of dst->batch entries
 * At most 256 destination sequences per call (UNSUPPORTED above).
 * Errors: INVALID_ARG (NULL, index out of range, negative start or count),
 * CONFIG_MISMATCH, CAPACITY (src_start + count > src->cap, count >
 * dst->cap), UNSUPPORTED, HIP. */
tq_status tq_cache_gather(const tq_codec* src_codec, const tq_cache* src, const tq_codec* dst_codec,
                          const tq_cache* dst, const int32_t* src_batch, const int32_t* src_start,
                          const int32_t* count, void* stream);

/* Hybrid cache ("turboquant validate_moe_phase2.py": Test 5's buffer_size
 * and the commit note's hybrid decode): the most recent tokens of each
 * sequence stay unquantised in a ring buffer of buf_size tokens per
 * (sequence, KV head), caller-owned device memory [batch][heads][buf_size]
 * [head_dim] of the tokens' dtype, one for keys and one for values, each
 * 16-byte aligned (INVALID_ARG otherwise).  A
 * sequence of N tokens holds tokens 0 .. Nc-1, Nc = floor(N / buf_size) *
 * buf_size, in the compressed caches and token t >= Nc in ring slot t - Nc;
 * whenever appends fill a ring, its buf_size tokens are quantised into the
 * compressed caches at Nc at once and the ring starts over.
 *
 * tq_hybrid_append: append n_new (<= buf_size) new key and value tokens per
 * (sequence, head) -- k, v, strides and dtype as tq_quantize_append_kv -- to
 * sequences holding d_len[b] tokens before the call (device int32[batch]);
 * len_end is the caller's host bound on d_len[b] + n_new, and the compressed
 * caches must hold floor(len_end / buf_size) * buf_size tokens (CAPACITY
 * otherwise).  The caller then holds d_len[b] + n_new tokens per sequence.
 * Errors: INVALID_ARG, UNSUPPORTED (n_new > buf_size), CONFIG_MISMATCH,
 * CAPACITY, HIP. */
tq_status tq_hybrid_append(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v, int32_t x_dtype,
                           int32_t batch, int32_t heads, int32_t n_new, const int64_t* k_strides,
                           const int64_t* v_strides, const tq_cache* kdst, const tq_cache* vdst, void* kbuf,
                           void* vbuf, int32_t buf_size, const int32_t* d_len, int64_t len_end, void* stream);

/* Workspace bytes of tq_hybrid_decode_attention for these sizes. */
tq_status tq_hybrid_decode_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t n_q_heads,
                                          int32_t n_kv_heads, int32_t q_len, int64_t max_len, int32_t buf_size,
                                          size_t* bytes);

/* Decode attention over a hybrid cache: every query row attends, with one
 * softmax and the causal rule of tq_decode_attention counted from the whole
 * length d_len[b] (device int32[batch], 1 <= d_len[b] <= max_len), to the
 * compressed tokens through their codes and to the ring's tokens exactly (in
 * float32 from buf_dtype values).  Arguments as tq_decode_attention plus the
 * rings (kbuf, vbuf, buf_dtype, buf_size); ws holds
 * tq_hybrid_decode_workspace_size(...) bytes.  Errors as tq_decode_attention. */
tq_status tq_hybrid_decode_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype,
                                     int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t q_len,
                                     const tq_cache* k, const tq_cache* v, const void* kbuf, const void* vbuf,
                                     int32_t buf_dtype, int32_t buf_size, const int32_t* d_len, int64_t max_len,
                                     float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* Measurement: read `bytes` of device memory once, as a plain streaming read
 * (16-byte loads, eight in flight per thread), the reference a decode
 * kernel's HBM rate is compared with.  Nothing in the library's path uses it.
 *   buf      device, 16-byte aligned; bytes a positive multiple of 16
 *   sink     device uint32[blocks * 256] (caller-owned; written only in the
 *            rare case that a thread's folded words equal one fixed value)
 *   blocks   workgroups of 256 threads, 1..2^20
 * Errors: INVALID_ARG, HIP. */
tq_status tq_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* Measurement: read the packed K and V state that tq_decode_attention reads
 * for these caches (indices and norms of the first len[b] tokens of every
 * sequence and KV head), once, in the int8 decode kernel's own grid, chunks,
 * tile loads and prefetch depth, with no arithmetic: the rate that the decode
 * kernel's access pattern reaches by itself.  Nothing in the library's path
 * uses it.  Codecs: 3-bit MSE keys and values at head_dim 128 only.
 *   k, v        device caches [batch][n_kv_heads][cap] (as for decode)
 *   d_len       device int32 [batch], clamped to 0..cap
 *   max_len     1..cap, the largest length (sets the chunk plan)
 *   sink        device uint32[sink_words], caller-owned; written only in the
 *               rare case that a thread's folded words equal one fixed value
 * Errors: INVALID_ARG, UNSUPPORTED (other codecs), CONFIG_MISMATCH, CAPACITY,
 * HIP. */
tq_status tq_decode_read_reference(const tq_codec* k_codec, const tq_codec* v_codec, int32_t batch,
                                   int32_t n_kv_heads, const tq_cache* k, const tq_cache* v, const int32_t* d_len,
                                   int64_t max_len, uint32_t* sink, uint32_t sink_words, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* tq_last_error(void);

/* Name of a status code. */
const char* tq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
