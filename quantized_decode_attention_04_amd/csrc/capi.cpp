// C ABI of libtq.so: argument validation, codec objects, per-device table
// upload and workspace planning.  Every device operation is a kernel launch
// on the caller's stream; nothing here computes on the host except the codec
// build.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>

#include "tq_internal.h"

namespace {

thread_local std::string g_error;

tq_status fail(tq_status s, const std::string& msg) {
  g_error = msg;
  return s;
}

tq_status hip_fail(hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(TQ_ERR_HIP, m);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// words of the low part of a split codec (its high part follows)
int split_low_words(const tq::HostCodec& h) { return (h.d - h.split_dhi) * h.mse_bits / 32; }
int idx_words(const tq::HostCodec& h) {
  if (h.mode == TQ_MODE_SPLIT) return split_low_words(h) + h.split_dhi * (h.mse_bits + 1) / 32;
  return h.d * h.mse_bits / 32;
}
int sign_words(const tq::HostCodec& h) { return h.mode == TQ_MODE_PROD ? h.d / 32 : 0; }
int group_count(const tq::HostCodec& h) { return h.mode == TQ_MODE_GROUP ? h.d / 32 : 0; }

uint64_t bytes_per_token(const tq::HostCodec& h) {
  uint64_t b = 4ull * idx_words(h);
  if (h.mode == TQ_MODE_MSE) b += 4;
  if (h.mode == TQ_MODE_PROD) b += 8 + 4ull * sign_words(h);
  if (h.mode == TQ_MODE_GROUP) b += 8ull * group_count(h);
  if (h.mode == TQ_MODE_SPLIT) b += 8;  // the two parts' norms
  return b;
}

// Upload the codec's tables to the current device (once per device).  With
// may_upload false a codec whose tables are not on the device yet is refused
// instead (the entry point that allocates nothing).
tq_status ensure_tables(const tq_codec* cc, tq::DevTables** out, bool may_upload = true) {
  tq_codec* c = const_cast<tq_codec*>(cc);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TQ_ERR_NO_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= tq::kMaxDevices) return fail(TQ_ERR_UNSUPPORTED, "device index above 15");
  std::lock_guard<std::mutex> lock(c->mu);
  tq::DevTables& t = c->dev[dev];
  if (!c->uploaded[dev] && c->h.mode != TQ_MODE_GROUP && !may_upload)
    return fail(TQ_ERR_INVALID_ARG, "codec tables are not on this device yet: call tq_codec_upload first");
  if (!c->uploaded[dev] && c->h.mode != TQ_MODE_GROUP) {
    const int d = c->h.d;
    const size_t dd = (size_t)d * d;
    const size_t nfl = 5 * dd + 64;
    void* block = nullptr;
    e = hipMalloc(&block, nfl * sizeof(float));
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(codec tables)");
    std::vector<float> host(nfl, 0.0f);
    float* pit = host.data();
    float* pi = pit + dd;
    float* st = pi + dd;
    float* sk = st + dd;
    float* spt = sk + dd;
    float* cent = spt + dd;
    float* bnd = cent + 16;
    float* cent2 = bnd + 16;
    float* bnd2 = cent2 + 16;
    // a split codec's rotation is block diagonal: each part rotates its own
    // channels (the query rotation and the output's inverse rotation then act
    // on the whole vector at once)
    const tq::HostCodec* blk[2] = {&c->h, nullptr};
    int off[2] = {0, 0};
    if (c->h.mode == TQ_MODE_SPLIT) {
      blk[0] = &c->part[0]->h;
      blk[1] = &c->part[1]->h;
      off[1] = blk[0]->d;
    }
    for (int q = 0; q < 2 && blk[q]; ++q) {
      const tq::HostCodec& hb = *blk[q];
      const int db = hb.d, o = off[q];
      for (int i = 0; i < db; ++i)
        for (int j = 0; j < db; ++j) {
          const float r = hb.rot[(size_t)i * db + j];
          pit[(size_t)(o + j) * d + o + i] = r;
          pi[(size_t)(o + i) * d + o + j] = r;
          if (!hb.sketch.empty()) {
            st[(size_t)(o + j) * d + o + i] = hb.sketch[(size_t)i * db + j];
            sk[(size_t)(o + i) * d + o + j] = hb.sketch[(size_t)i * db + j];
          }
        }
      float* ce = q == 0 ? cent : cent2;
      float* bo = q == 0 ? bnd : bnd2;
      if (!hb.sketch.empty()) {
        // (S Pi)^T, so that the query prologue forms S q_rot = (S Pi) q in
        // the same pass as q_rot = Pi q (the product taken in double)
        std::vector<double> row(db);
        for (int i = 0; i < db; ++i) {
          std::fill(row.begin(), row.end(), 0.0);
          for (int k = 0; k < db; ++k) {
            const double sik = hb.sketch[(size_t)i * db + k];
            const float* rk = &hb.rot[(size_t)k * db];
            for (int j = 0; j < db; ++j) row[j] += sik * (double)rk[j];
          }
          for (int j = 0; j < db; ++j) spt[(size_t)(o + j) * d + o + i] = (float)row[j];
        }
      }
      for (int k = 0; k < hb.levels; ++k) ce[k] = hb.centroids[k];
      for (int k = 0; k + 1 < hb.levels; ++k) bo[k] = hb.boundaries[k];
    }
    e = hipMemcpy(block, host.data(), nfl * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(block);
      return hip_fail(e, "hipMemcpy(codec tables)");
    }
    float* base = static_cast<float*>(block);
    t.block = block;
    t.pit = base;
    t.pi = base + dd;
    t.st = base + 2 * dd;
    t.s = base + 3 * dd;
    t.spt = base + 4 * dd;
    t.cent = base + 5 * dd;
    t.bnd = base + 5 * dd + 16;
    t.cent2 = base + 5 * dd + 32;
    t.bnd2 = base + 5 * dd + 48;
    c->uploaded[dev] = true;
  }
  *out = &t;
  return TQ_OK;
}

bool cache_ok(const tq_cache* c, const tq::HostCodec& h, std::string* why) {
  if (!c->idx) { *why = "cache idx is NULL"; return false; }
  if (h.mode != TQ_MODE_GROUP && !c->norm) { *why = "cache norm is NULL"; return false; }
  if (h.mode == TQ_MODE_PROD && (!c->rnorm || !c->sign)) { *why = "Prod cache needs rnorm and sign"; return false; }
  if (h.mode == TQ_MODE_SPLIT && !c->rnorm) { *why = "split cache needs rnorm (the high part's norm)"; return false; }
  if (h.mode == TQ_MODE_GROUP && (!c->scale || !c->gmin)) { *why = "group cache needs scale and gmin"; return false; }
  if (c->batch <= 0 || c->heads <= 0 || c->cap <= 0) { *why = "cache batch, heads and cap must be positive"; return false; }
  return true;
}

}  // namespace


namespace {

// int8 piece tables of an 8-level codebook: centroid * 2^E = 256*hi + lo with
// lo in [-128, 127]; bytes hi[0..3], hi[4..7], lo[0..3], lo[4..7].
void piece_tables(const tq::HostCodec& h, uint32_t* lut) {
  lut[0] = lut[1] = lut[2] = lut[3] = 0;
  for (int k = 0; k < h.levels && k < 8; ++k) {
    const int c = (int)std::ldexp((double)h.centroids[k], h.grid_exp);
    const int hi = (int)std::floor((c + 128) / 256.0);
    const int lo = c - 256 * hi;
    lut[k / 4] |= ((uint32_t)hi & 0xffu) << (8 * (k % 4));
    lut[2 + k / 4] |= ((uint32_t)lo & 0xffu) << (8 * (k % 4));
  }
}

bool use_fast(const tq_codec* kc, const tq_codec* vc, int rows) {
  return tq::fast_decode_supported(kc->h.d, kc->h.mode, kc->h.mse_bits, vc->h.mode, vc->h.mse_bits, rows);
}

bool use_mfma(const tq_codec* kc, const tq_codec* vc, int rows) {
  if (kc->h.mode == TQ_MODE_SPLIT || vc->h.mode == TQ_MODE_SPLIT)
    return tq::mfma_split_supported(kc->h.d, kc->h.mode, kc->h.mse_bits, kc->h.d - kc->h.split_dhi, vc->h.mode,
                                    vc->h.mse_bits, vc->h.d - vc->h.split_dhi, rows);
  return !use_fast(kc, vc, rows) &&
         tq::mfma_decode_preferred(kc->h.d, kc->h.mode, kc->h.mse_bits, vc->h.mode, vc->h.mse_bits, rows);
}

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_error.c_str(); }

const char* tq_status_string(int32_t s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_CONFIG_MISMATCH: return "TQ_ERR_CONFIG_MISMATCH";
    case TQ_ERR_CAPACITY: return "TQ_ERR_CAPACITY";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_NO_DEVICE: return "TQ_ERR_NO_DEVICE";
    default: return "TQ_ERR_UNKNOWN";
  }
}

tq_status tq_codec_create(int32_t head_dim, int32_t bits, uint64_t seed, int32_t mode, tq_codec** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_create: out is NULL");
  *out = nullptr;
  tq::HostCodec h;
  std::string err;
  if (!tq::build_codec(head_dim, bits, seed, mode, &h, &err)) return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create: " + err);
  tq_codec* c = new (std::nothrow) tq_codec();
  if (!c) return fail(TQ_ERR_INVALID_ARG, "tq_codec_create: out of host memory");
  c->h = std::move(h);
  *out = c;
  g_error.clear();
  return TQ_OK;
}

tq_status tq_codec_create_kv(int32_t head_dim, double bits, uint64_t seed, tq_codec** key_out,
                             tq_codec** value_out) {
  if (!key_out || !value_out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_create_kv: NULL argument");
  *key_out = *value_out = nullptr;
  if (!std::isfinite(bits) || bits < 0.5 || bits > 16.0)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create_kv: bits out of range");
  // [omlx] _rebuild_codecs: fractional unless within 1e-6 of an integer;
  // keys floor(bits), values ceil(bits)
  const double r = std::nearbyint(bits);
  const bool fractional = std::fabs(bits - r) > 1e-6;
  const int kb = fractional ? (int)std::floor(bits) : (int)r;
  const int vb = fractional ? (int)std::ceil(bits) : (int)r;
  tq_codec *k = nullptr, *v = nullptr;
  tq_status st = tq_codec_create(head_dim, kb, seed, TQ_MODE_MSE, &k);
  if (st != TQ_OK) return st;
  st = tq_codec_create(head_dim, vb, seed + 1, TQ_MODE_MSE, &v);
  if (st != TQ_OK) {
    tq_codec_destroy(k);
    return st;
  }
  *key_out = k;
  *value_out = v;
  return TQ_OK;
}

tq_status tq_codec_create_split(int32_t head_dim, double bits, uint64_t seed, tq_codec** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_create_split: out is NULL");
  *out = nullptr;
  if (!std::isfinite(bits) || std::fabs(bits - std::nearbyint(bits)) <= 1e-6)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create_split: bits must be fractional (not within 1e-6 of an integer)");
  if (head_dim < 64 || head_dim > 256 || head_dim % 32)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create_split: head_dim must be a multiple of 32 in [64, 256]");
  const int lo = (int)std::floor(bits), hi = lo + 1;
  const int d_hi = (int)std::lround((bits - lo) * head_dim / 32.0) * 32;
  const int d_lo = head_dim - d_hi;
  if (lo < 1 || hi > 4 || d_hi < 32 || d_lo < 32)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create_split: each part needs 32..head_dim-32 channels and 1..4 bits");
  tq::HostCodec hl, hh;
  std::string err;
  if (!tq::build_codec(d_lo, lo, seed, TQ_MODE_MSE, &hl, &err, 0) ||
      !tq::build_codec(d_hi, hi, seed, TQ_MODE_MSE, &hh, &err, 2))
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_create_split: " + err);
  tq_codec* c = new (std::nothrow) tq_codec();
  tq_codec* pl = new (std::nothrow) tq_codec();
  tq_codec* ph = new (std::nothrow) tq_codec();
  if (!c || !pl || !ph) {
    delete c;
    delete pl;
    delete ph;
    return fail(TQ_ERR_INVALID_ARG, "tq_codec_create_split: out of host memory");
  }
  tq::HostCodec& h = c->h;
  h.d = head_dim;
  h.bits = lo;
  h.mode = TQ_MODE_SPLIT;
  h.mse_bits = lo;
  h.levels = 1 << lo;
  h.grid_exp = hl.grid_exp;
  h.seed = seed;
  h.split_dhi = d_hi;
  // the block-diagonal rotation and the low part's codebook, for export
  h.rot.assign((size_t)head_dim * head_dim, 0.0f);
  for (int i = 0; i < d_lo; ++i)
    for (int j = 0; j < d_lo; ++j) h.rot[(size_t)i * head_dim + j] = hl.rot[(size_t)i * d_lo + j];
  for (int i = 0; i < d_hi; ++i)
    for (int j = 0; j < d_hi; ++j) h.rot[(size_t)(d_lo + i) * head_dim + d_lo + j] = hh.rot[(size_t)i * d_hi + j];
  h.centroids = hl.centroids;
  h.boundaries = hl.boundaries;
  pl->h = std::move(hl);
  ph->h = std::move(hh);
  c->part[0] = pl;
  c->part[1] = ph;
  *out = c;
  g_error.clear();
  return TQ_OK;
}

tq_status tq_codec_part(const tq_codec* c, int32_t which, const tq_codec** out) {
  if (!c || !out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_part: NULL argument");
  if (c->h.mode != TQ_MODE_SPLIT) return fail(TQ_ERR_INVALID_ARG, "tq_codec_part: not a split codec");
  if (which != 0 && which != 1) return fail(TQ_ERR_INVALID_ARG, "tq_codec_part: which must be 0 (low) or 1 (high)");
  *out = c->part[which];
  return TQ_OK;
}

void tq_codec_destroy(tq_codec* c) {
  if (!c) return;
  for (int i = 0; i < tq::kMaxDevices; ++i)
    if (c->uploaded[i] && c->dev[i].block) (void)hipFree(c->dev[i].block);
  tq_codec_destroy(c->part[0]);
  tq_codec_destroy(c->part[1]);
  delete c;
}

tq_status tq_codec_get_info(const tq_codec* c, tq_codec_info* info) {
  if (!c || !info) return fail(TQ_ERR_INVALID_ARG, "tq_codec_get_info: NULL argument");
  const tq::HostCodec& h = c->h;
  std::memset(info, 0, sizeof(*info));
  info->head_dim = h.d;
  info->bits = h.bits;
  info->mode = h.mode;
  info->mse_bits = h.mse_bits;
  info->levels = h.levels;
  info->idx_words = idx_words(h);
  info->sign_words = sign_words(h);
  info->groups = group_count(h);
  info->grid_exp = h.grid_exp;
  info->split_high_dim = h.mode == TQ_MODE_SPLIT ? h.split_dhi : 0;
  info->seed = h.seed;
  info->bytes_per_token = bytes_per_token(h);
  return TQ_OK;
}

tq_status tq_codec_export(const tq_codec* c, float* rot, float* centroids, float* boundaries, float* sketch) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "tq_codec_export: codec is NULL");
  const tq::HostCodec& h = c->h;
  if (h.mode == TQ_MODE_GROUP) return TQ_OK;
  if (rot) std::memcpy(rot, h.rot.data(), h.rot.size() * sizeof(float));
  if (centroids) std::memcpy(centroids, h.centroids.data(), h.centroids.size() * sizeof(float));
  if (boundaries) std::memcpy(boundaries, h.boundaries.data(), h.boundaries.size() * sizeof(float));
  if (sketch && !h.sketch.empty()) std::memcpy(sketch, h.sketch.data(), h.sketch.size() * sizeof(float));
  return TQ_OK;
}

tq_status tq_codec_upload(const tq_codec* c) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "tq_codec_upload: codec is NULL");
  tq::DevTables* t = nullptr;
  return ensure_tables(c, &t);
}

}  // extern "C"

// Checks one append and fills its kernel parameters; *empty is set when
// n_new == 0 (nothing to launch).
static tq_status prepare_append(const char* who, const tq_codec* c, const void* x, int32_t x_dtype, int32_t batch,
                                int32_t heads, int32_t n_new, const int64_t* x_strides, const tq_cache* dst,
                                const int32_t* d_pos, int64_t pos_end, tq::QuantizeParams* out, bool* empty) {
  const std::string w(who);
  if (!c || !x || !dst || !d_pos) return fail(TQ_ERR_INVALID_ARG, w + ": NULL argument");
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, w + ": bad x_dtype");
  if (batch <= 0 || heads <= 0 || n_new < 0)
    return fail(TQ_ERR_INVALID_ARG, w + ": batch and heads must be positive, n_new >= 0");
  const tq::HostCodec& h = c->h;
  std::string why;
  if (!cache_ok(dst, h, &why)) return fail(TQ_ERR_INVALID_ARG, w + ": " + why);
  if (dst->batch != batch || dst->heads != heads)
    return fail(TQ_ERR_CONFIG_MISMATCH, w + ": cache batch/heads differ from the input's");
  // the written end after the append, bounded on the host ([omlx]
  // update_and_fetch writes at the written end; a write past the allocated
  // capacity must not be lost silently)
  if (pos_end < n_new) return fail(TQ_ERR_INVALID_ARG, w + ": pos_end is below n_new");
  if (pos_end > dst->cap)
    return fail(TQ_ERR_CAPACITY, w + ": the append ends at " + std::to_string(pos_end) + ", past the cache capacity " +
                                     std::to_string(dst->cap));
  int64_t s0, s1, s2;
  if (x_strides) {
    if (x_strides[3] != 1) return fail(TQ_ERR_INVALID_ARG, w + ": coordinate stride must be 1");
    s0 = x_strides[0];
    s1 = x_strides[1];
    s2 = x_strides[2];
    if (s0 < 0 || s1 < 0 || s2 < 0) return fail(TQ_ERR_INVALID_ARG, w + ": negative stride");
  } else {
    s2 = h.d;
    s1 = (int64_t)n_new * h.d;
    s0 = (int64_t)heads * s1;
  }
  *empty = n_new == 0;
  tq::QuantizeParams& p = *out;
  p = tq::QuantizeParams{};
  p.x = x;
  p.x_bf16 = x_dtype == TQ_BF16;
  p.s0 = s0;
  p.s1 = s1;
  p.s2 = s2;
  p.batch = batch;
  p.heads = heads;
  p.n_new = n_new;
  p.d = h.d;
  p.mode = h.mode;
  p.mse_bits = h.mse_bits;
  p.levels = h.levels;
  p.words = idx_words(h);
  p.sign_words = sign_words(h);
  p.groups = group_count(h);
  p.gbits = h.mode == TQ_MODE_GROUP ? h.bits : 0;
  {
    // 16-byte row loads need a 16-byte aligned base and strides
    const int64_t es = p.x_bf16 ? 2 : 4;
    p.x_vec16 = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (s0 * es) % 16 == 0 && (s1 * es) % 16 == 0 &&
                (s2 * es) % 16 == 0;
  }
  p.idx = dst->idx;
  p.idx_stride = p.words;
  p.norm = dst->norm;
  p.rnorm = dst->rnorm;
  p.sign = dst->sign;
  p.scale = dst->scale;
  p.gmin = dst->gmin;
  p.cap = dst->cap;
  p.pos = d_pos;
  return TQ_OK;
}

// After every argument of a call has been checked: the codec's device tables
// (uploaded on first use on this device) go into its parameter block.
static tq_status bind_tables(const tq_codec* c, tq::QuantizeParams* p);

// The parameter blocks of one checked append: one, or for a split codec one
// per part (each an MSE append of the part's channels into the part's words
// of the shared token record and the part's norm array).  Tables bound.
static tq_status append_blocks(const tq_codec* c, const tq::QuantizeParams& whole, std::vector<tq::QuantizeParams>* out,
                               std::vector<const tq_codec*>* codecs) {
  if (c->h.mode != TQ_MODE_SPLIT) {
    out->push_back(whole);
    codecs->push_back(c);
    return TQ_OK;
  }
  const tq_codec* part[2] = {c->part[0], c->part[1]};
  const int w_lo = idx_words(part[0]->h);
  const int64_t es = whole.x_bf16 ? 2 : 4;
  for (int q = 0; q < 2; ++q) {
    const tq::HostCodec& h = part[q]->h;
    tq::QuantizeParams p = whole;
    p.d = h.d;
    p.mode = TQ_MODE_MSE;
    p.mse_bits = h.mse_bits;
    p.levels = h.levels;
    p.words = idx_words(h);
    p.sign_words = 0;
    p.groups = 0;
    p.gbits = 0;
    p.idx = whole.idx + (q == 0 ? 0 : w_lo);
    p.idx_stride = whole.words;
    p.norm = q == 0 ? whole.norm : whole.rnorm;
    p.rnorm = nullptr;
    if (q == 1) {
      p.x = static_cast<const char*>(whole.x) + (int64_t)part[0]->h.d * es;
      p.x_vec16 = whole.x_vec16 && ((int64_t)part[0]->h.d * es) % 16 == 0;
    }
    out->push_back(p);
    codecs->push_back(part[q]);
  }
  return TQ_OK;
}

// Launch checked append blocks: neighbours with the same head_dim share one
// launch (the kernel is chosen by sizes only, so grouping changes no bit).
static tq_status launch_blocks(const char* who, std::vector<tq::QuantizeParams>& blocks,
                               const std::vector<const tq_codec*>& codecs, void* stream) {
  for (size_t i = 0; i < blocks.size(); ++i) {
    tq_status st = bind_tables(codecs[i], &blocks[i]);
    if (st != TQ_OK) return st;
  }
  for (size_t i = 0; i < blocks.size();) {
    tq::QuantizeSets sets{};
    int n = 1;
    sets.s[0] = blocks[i];
    if (i + 1 < blocks.size() && blocks[i + 1].d == blocks[i].d) {
      sets.s[1] = blocks[i + 1];
      n = 2;
    }
    const hipError_t e = tq::launch_quantize(sets, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, (std::string(who) + " launch").c_str());
    i += n;
  }
  return TQ_OK;
}

static tq_status bind_tables(const tq_codec* c, tq::QuantizeParams* p) {
  if (c->h.mode == TQ_MODE_GROUP) return TQ_OK;
  tq::DevTables* t = nullptr;
  const tq_status st = ensure_tables(c, &t);
  if (st != TQ_OK) return st;
  p->pit = t->pit;
  p->pi = t->pi;
  p->st = t->st;
  p->s = t->s;
  p->cent = t->cent;
  p->bnd = t->bnd;
  return TQ_OK;
}

extern "C" {

tq_status tq_quantize_append(const tq_codec* c, const void* x, int32_t x_dtype, int32_t batch, int32_t heads,
                             int32_t n_new, const int64_t* x_strides, const tq_cache* dst, const int32_t* d_pos,
                             int64_t pos_end, void* stream) {
  tq::QuantizeSets sets{};
  bool empty = false;
  tq_status st = prepare_append("tq_quantize_append", c, x, x_dtype, batch, heads, n_new, x_strides, dst, d_pos,
                                pos_end, &sets.s[0], &empty);
  if (st != TQ_OK) return st;
  if (empty) return TQ_OK;
  std::vector<tq::QuantizeParams> blocks;
  std::vector<const tq_codec*> codecs;
  append_blocks(c, sets.s[0], &blocks, &codecs);
  return launch_blocks("tq_quantize_append", blocks, codecs, stream);
}

tq_status tq_quantize_append_kv(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v,
                                int32_t x_dtype, int32_t batch, int32_t heads, int32_t n_new,
                                const int64_t* k_strides, const int64_t* v_strides, const tq_cache* kdst,
                                const tq_cache* vdst, const int32_t* d_pos, int64_t pos_end, void* stream) {
  tq::QuantizeSets sets{};
  bool empty_k = false, empty_v = false;
  tq_status st = prepare_append("tq_quantize_append_kv (keys)", kc, k, x_dtype, batch, heads, n_new, k_strides, kdst,
                                d_pos, pos_end, &sets.s[0], &empty_k);
  if (st != TQ_OK) return st;
  st = prepare_append("tq_quantize_append_kv (values)", vc, v, x_dtype, batch, heads, n_new, v_strides, vdst, d_pos,
                      pos_end, &sets.s[1], &empty_v);
  if (st != TQ_OK) return st;
  if (kc->h.d != vc->h.d)
    return fail(TQ_ERR_CONFIG_MISMATCH, "tq_quantize_append_kv: key and value codecs have different head_dim");
  if (empty_k) return TQ_OK;
  std::vector<tq::QuantizeParams> blocks;
  std::vector<const tq_codec*> codecs;
  append_blocks(kc, sets.s[0], &blocks, &codecs);
  append_blocks(vc, sets.s[1], &blocks, &codecs);
  return launch_blocks("tq_quantize_append_kv", blocks, codecs, stream);
}

// Rows per launch: 16 up to head_dim 128, 8 above (the general kernel's
// register budget).  Decode takes one launch; prefill walks the rows of each
// KV head in blocks of this size.
static int row_block(const tq_codec* kc) { return kc->h.d <= 128 ? 16 : 8; }

static tq_status check_decode_shapes(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                                     int32_t q_len, int64_t max_len, bool blocks = false) {
  if (!kc || !vc) return fail(TQ_ERR_INVALID_ARG, "decode: codec is NULL");
  if (kc->h.mode != TQ_MODE_MSE && kc->h.mode != TQ_MODE_PROD && kc->h.mode != TQ_MODE_SPLIT)
    return fail(TQ_ERR_UNSUPPORTED, "decode: the key codec must be MSE, Prod or split");
  if (vc->h.mode != TQ_MODE_MSE && vc->h.mode != TQ_MODE_GROUP && vc->h.mode != TQ_MODE_SPLIT)
    return fail(TQ_ERR_UNSUPPORTED, "decode: the value codec must be MSE, group or split");
  if (kc->h.d != vc->h.d) return fail(TQ_ERR_CONFIG_MISMATCH, "decode: key and value codecs have different head_dim");
  if (batch <= 0 || hq <= 0 || hkv <= 0 || q_len <= 0)
    return fail(TQ_ERR_INVALID_ARG, "decode: batch, heads and q_len must be positive");
  if (hq % hkv) return fail(TQ_ERR_INVALID_ARG, "decode: n_q_heads must be a multiple of n_kv_heads");
  if (max_len <= 0) return fail(TQ_ERR_INVALID_ARG, "decode: max_len must be positive");
  if (max_len > tq::kMaxDecodeLen)
    return fail(TQ_ERR_UNSUPPORTED, "decode: max_len above " + std::to_string(tq::kMaxDecodeLen) + " tokens");
  const int64_t rows = (int64_t)(hq / hkv) * q_len;
  const int rmax = row_block(kc);
  if (blocks) {
    if (rows > (int64_t)1 << 30) return fail(TQ_ERR_UNSUPPORTED, "prefill: more than 2^30 query rows per KV head");
    return TQ_OK;
  }
  if (rows > rmax)
    return fail(TQ_ERR_UNSUPPORTED, "decode: (n_q_heads/n_kv_heads)*q_len above " + std::to_string(rmax) +
                                        " for this head_dim");
  return TQ_OK;
}

// The decode path and its plan for these sizes: one function for the
// workspace size queries and the calls, so that a workspace sized through the
// API always fits the call.
enum class DecodePath { kFast, kMfma, kGeneral, kPrefillFast, kPrefillBf16 };

static tq::DecodePlan choose_plan(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                                  int32_t q_len, int64_t max_len, DecodePath* path, bool blocks = false) {
  const int64_t rows_total = (int64_t)(hq / hkv) * q_len;
  const int rows = (int)std::min<int64_t>(rows_total, row_block(kc));
  const bool prod = kc->h.mode == TQ_MODE_PROD;
  // prefill on the 3-bit int8 path: one launch takes up to kPrefillRows rows
  // of every KV head and reads each tile once per 128 of them
  if (blocks && rows_total > 16 && use_fast(kc, vc, 16)) {
    const int prows = (int)std::min<int64_t>(rows_total, tq::kPrefillRows);
    const tq::DecodePlan pp = tq::plan_prefill_fast(batch, hkv, prows, max_len);
    if (pp.n_chunks > 0) {
      *path = DecodePath::kPrefillFast;
      return pp;
    }
  }
  // prefill on the bf16 / int8 kernel's codecs: likewise, per 128 rows at
  // head_dim 128 and per 64 at 256
  if (blocks && rows_total > row_block(kc) &&
      tq::bf16_prefill_supported(kc->h.d, kc->h.mode, kc->h.mse_bits, vc->h.mode, vc->h.mse_bits)) {
    const int prows = (int)std::min<int64_t>(rows_total, tq::kPrefillRows);
    const tq::DecodePlan pp = tq::plan_prefill_bf16(batch, hkv, prows, kc->h.d, max_len);
    if (pp.n_chunks > 0) {
      *path = DecodePath::kPrefillBf16;
      return pp;
    }
  }
  if (use_fast(kc, vc, rows)) {
    *path = DecodePath::kFast;
    return tq::plan_decode_fast(batch, hkv, rows, kc->h.d, max_len);
  }
  if (use_mfma(kc, vc, rows)) {
    *path = DecodePath::kMfma;
    const bool split = kc->h.mode == TQ_MODE_SPLIT || vc->h.mode == TQ_MODE_SPLIT;
    return tq::plan_decode_mfma(batch, hkv, rows, kc->h.d, max_len, prod, (split && kc->h.d == 128) ? tq::kSplitWgPerCu : 2);
  }
  *path = DecodePath::kGeneral;
  return tq::plan_decode(batch, hkv, rows, kc->h.d, max_len, prod);
}

static size_t attention_workspace(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                                  int32_t q_len, int64_t max_len, bool blocks = false) {
  DecodePath path;
  return choose_plan(kc, vc, batch, hq, hkv, q_len, max_len, &path, blocks).total;
}

tq_status tq_decode_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                                   int32_t q_len, int64_t max_len, size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "tq_decode_workspace_size: bytes is NULL");
  tq_status st = check_decode_shapes(kc, vc, batch, hq, hkv, q_len, max_len);
  if (st != TQ_OK) return st;
  *bytes = attention_workspace(kc, vc, batch, hq, hkv, q_len, max_len);
  return TQ_OK;
}

tq_status tq_prefill_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                                    int32_t q_len, int64_t max_len, size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "tq_prefill_workspace_size: bytes is NULL");
  tq_status st = check_decode_shapes(kc, vc, batch, hq, hkv, q_len, max_len, true);
  if (st != TQ_OK) return st;
  *bytes = attention_workspace(kc, vc, batch, hq, hkv, q_len, max_len, true);
  return TQ_OK;
}

static tq_status attention_impl(const char* name, bool blocks, const tq_codec* kc, const tq_codec* vc, const void* q,
                                int32_t q_dtype, int32_t batch, int32_t hq, int32_t hkv, int32_t q_len,
                                const tq_cache* k, const tq_cache* v, const int32_t* d_len, int64_t max_len,
                                float scale, float* out, void* ws, size_t ws_bytes, void* stream,
                                bool may_upload = true, const int32_t* len_mask = nullptr,
                                float* row_ml = nullptr) {
  const std::string fn(name);
  tq_status st = check_decode_shapes(kc, vc, batch, hq, hkv, q_len, max_len, blocks);
  if (st != TQ_OK) return st;
  if (!q || !k || !v || !d_len || !out) return fail(TQ_ERR_INVALID_ARG, fn + ": NULL argument");
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, fn + ": bad q_dtype");
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, fn + ": scale is not finite");
  std::string why;
  if (!cache_ok(k, kc->h, &why)) return fail(TQ_ERR_INVALID_ARG, fn + ": key " + why);
  if (!cache_ok(v, vc->h, &why)) return fail(TQ_ERR_INVALID_ARG, fn + ": value " + why);
  if (k->batch != batch || v->batch != batch || k->heads != hkv || v->heads != hkv)
    return fail(TQ_ERR_CONFIG_MISMATCH, fn + ": cache batch/heads differ from the call's");
  if (k->cap != v->cap) return fail(TQ_ERR_CONFIG_MISMATCH, fn + ": key and value caps differ");
  if (max_len > k->cap) return fail(TQ_ERR_CAPACITY, fn + ": max_len exceeds the cache capacity");
  const int64_t rows_total = (int64_t)(hq / hkv) * q_len;
  const int rows = (int)std::min<int64_t>(rows_total, row_block(kc));  // rows per launch
  const bool prod = kc->h.mode == TQ_MODE_PROD;
  DecodePath path;
  const tq::DecodePlan plan = choose_plan(kc, vc, batch, hq, hkv, q_len, max_len, &path, blocks);
  const bool prefill_bf16 = path == DecodePath::kPrefillBf16;
  const bool prefill = path == DecodePath::kPrefillFast || prefill_bf16;
  const bool fast = path == DecodePath::kFast || path == DecodePath::kPrefillFast;
  const bool mfma = path == DecodePath::kMfma;
  if (!ws || ws_bytes < plan.total)
    return fail(TQ_ERR_WORKSPACE, fn + ": workspace needs " + std::to_string(plan.total) + " bytes");
  tq::DevTables* kt = nullptr;
  tq::DevTables* vt = nullptr;
  st = ensure_tables(kc, &kt, may_upload);
  if (st != TQ_OK) return st;
  if (vc->h.mode != TQ_MODE_GROUP) {
    st = ensure_tables(vc, &vt, may_upload);
    if (st != TQ_OK) return st;
  }
  char* w = static_cast<char*>(ws);
  tq::DecodeParams p{};
  p.q = q;
  p.q_bf16 = q_dtype == TQ_BF16;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.q_len = q_len;
  p.group = hq / hkv;
  p.rows = rows;
  p.d = kc->h.d;
  p.scale = scale;
  p.kmode = kc->h.mode;
  p.kbits = kc->h.mse_bits;
  p.kwords = idx_words(kc->h);
  p.ksign_words = sign_words(kc->h);
  p.k_pit = kt->pit;
  p.k_pi = kt->pi;
  p.k_spt = kt->spt;
  p.k_cent = kt->cent;
  p.k_idx = k->idx;
  p.k_norm = k->norm;
  p.k_rnorm = k->rnorm;
  p.k_sign = k->sign;
  const bool ksplit = kc->h.mode == TQ_MODE_SPLIT, vsplit = vc->h.mode == TQ_MODE_SPLIT;
  p.ksplit_g = ksplit ? (kc->h.d - kc->h.split_dhi) / 32 : 0;
  p.k_cent_hi = ksplit ? kt->cent2 : nullptr;
  p.k_norm_hi = ksplit ? k->rnorm : nullptr;
  p.vsplit_g = vsplit ? (vc->h.d - vc->h.split_dhi) / 32 : 0;
  p.v_cent_hi = vsplit ? vt->cent2 : nullptr;
  p.v_norm_hi = vsplit ? v->rnorm : nullptr;
  p.vmode = vc->h.mode;
  p.vbits = vc->h.mse_bits;
  p.vwords = idx_words(vc->h);
  p.vgroups = group_count(vc->h);
  p.v_pi = vt ? vt->pi : nullptr;
  p.v_cent = vt ? vt->cent : nullptr;
  p.v_idx = v->idx;
  p.v_norm = v->norm;
  p.v_scale = v->scale;
  p.v_gmin = v->gmin;
  p.cap = k->cap;
  p.len = d_len;
  p.len_mask = len_mask;
  p.row_ml = row_ml;
  p.chunk = plan.chunk;
  p.n_chunks = plan.n_chunks;
  p.part_o = reinterpret_cast<float*>(w + plan.off_part_o);
  p.part_ml = reinterpret_cast<float*>(w + plan.off_part_ml);
  p.out = out;
  // int8 centroid pieces (the matrix-core paths; centroids lie on the 2^-E grid)
  piece_tables(kc->h, p.klut);
  p.kgrid = kc->h.grid_exp;
  if (fast) {
    piece_tables(vc->h, p.vlut);
    p.vgrid = vc->h.grid_exp;
  }
  if (!fast || prefill) {
    p.qrot = reinterpret_cast<float*>(w + plan.off_qrot);
    p.qs = prod ? reinterpret_cast<float*>(w + plan.off_qs) : nullptr;
  }
  // one launch per block of rows; the blocks reuse the workspace in stream order
  const int block = prefill ? plan.rows : rows;
  for (int64_t r0 = 0; r0 < rows_total; r0 += block) {
    p.row0 = (int)r0;
    p.rows = (int)std::min<int64_t>(block, rows_total - r0);
    const hipError_t e = prefill_bf16 ? tq::launch_prefill_bf16(p, static_cast<hipStream_t>(stream))
                         : prefill ? tq::launch_prefill_fast(p, static_cast<hipStream_t>(stream))
                         : fast  ? tq::launch_decode_fast(p, static_cast<hipStream_t>(stream))
                         : mfma  ? tq::launch_decode_mfma(p, static_cast<hipStream_t>(stream))
                                 : tq::launch_decode(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, (fn + " launch").c_str());
  }
  return TQ_OK;
}

}  // extern "C"

namespace tq {

tq_status decode_attention_in(const char* name, const tq_codec* kc, const tq_codec* vc, const void* q,
                              int32_t q_dtype, int32_t batch, int32_t hq, int32_t hkv, int32_t q_len,
                              const tq_cache* k, const tq_cache* v, const int32_t* d_len, int64_t max_len,
                              float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  return attention_impl(name, false, kc, vc, q, q_dtype, batch, hq, hkv, q_len, k, v, d_len, max_len, scale, out, ws,
                        ws_bytes, stream, false);
}

tq_status set_error(tq_status s, const std::string& msg) { return fail(s, msg); }

}  // namespace tq

extern "C" {

tq_status tq_decode_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype, int32_t batch,
                              int32_t hq, int32_t hkv, int32_t q_len, const tq_cache* k, const tq_cache* v,
                              const int32_t* d_len, int64_t max_len, float scale, float* out, void* ws,
                              size_t ws_bytes, void* stream) {
  return attention_impl("tq_decode_attention", false, kc, vc, q, q_dtype, batch, hq, hkv, q_len, k, v, d_len, max_len,
                        scale, out, ws, ws_bytes, stream);
}

tq_status tq_prefill_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype, int32_t batch,
                               int32_t hq, int32_t hkv, int32_t q_len, const tq_cache* k, const tq_cache* v,
                               const int32_t* d_len, int64_t max_len, float scale, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  return attention_impl("tq_prefill_attention", true, kc, vc, q, q_dtype, batch, hq, hkv, q_len, k, v, d_len,
                        max_len, scale, out, ws, ws_bytes, stream);
}

// ---- hybrid cache -------------------------------------------------------------

static bool hybrid_buffers_ok(const void* kbuf, const void* vbuf, int32_t buf_dtype, int32_t buf_size,
                              std::string* why) {
  if (!kbuf || !vbuf) { *why = "buffer pointer is NULL"; return false; }
  if (buf_dtype != TQ_F32 && buf_dtype != TQ_BF16) { *why = "bad buffer dtype"; return false; }
  if (buf_size < 1 || buf_size > (1 << 16)) { *why = "buffer size must be in 1..65536"; return false; }
  if ((reinterpret_cast<uintptr_t>(kbuf) | reinterpret_cast<uintptr_t>(vbuf)) & 15u) {
    *why = "buffers must be 16-byte aligned";  // the combine kernel's 16-byte key reads
    return false;
  }
  return true;
}

tq_status tq_hybrid_append(const tq_codec* kc, const tq_codec* vc, const void* k, const void* v, int32_t x_dtype,
                           int32_t batch, int32_t heads, int32_t n_new, const int64_t* k_strides,
                           const int64_t* v_strides, const tq_cache* kdst, const tq_cache* vdst, void* kbuf,
                           void* vbuf, int32_t buf_size, const int32_t* d_len, int64_t len_end, void* stream) {
  const char* who = "tq_hybrid_append";
  std::string why;
  if (!hybrid_buffers_ok(kbuf, vbuf, x_dtype, buf_size, &why)) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": " + why);
  if (n_new > buf_size) return fail(TQ_ERR_UNSUPPORTED, std::string(who) + ": more new tokens than the buffer holds");
  if (len_end < n_new) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": len_end is below n_new");
  // the compressed cache holds floor(len / buf_size) * buf_size tokens
  const int64_t comp_end = (len_end / buf_size) * buf_size;
  tq::QuantizeSets sets{};
  bool empty_k = false, empty_v = false;
  if (!kc || !vc) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": codec is NULL");
  if (kc->h.d != vc->h.d) return fail(TQ_ERR_CONFIG_MISMATCH, std::string(who) + ": key and value codecs differ in head_dim");
  const int d = kc->h.d;
  // a flush appends a whole ring (buf_size tokens, read in its own layout)
  // into the compressed cache, ending at most at comp_end; with comp_end 0 no
  // ring can fill in this call
  const bool may_flush = comp_end >= buf_size;
  if (may_flush) {
    const int64_t ring_strides[4] = {(int64_t)heads * buf_size * d, (int64_t)buf_size * d, d, 1};
    tq_status st = prepare_append("tq_hybrid_append (keys)", kc, kbuf, x_dtype, batch, heads, buf_size, ring_strides,
                                  kdst, d_len, comp_end, &sets.s[0], &empty_k);
    if (st != TQ_OK) return st;
    st = prepare_append("tq_hybrid_append (values)", vc, vbuf, x_dtype, batch, heads, buf_size, ring_strides, vdst,
                        d_len, comp_end, &sets.s[1], &empty_v);
    if (st != TQ_OK) return st;
  } else if (batch <= 0 || heads <= 0 || n_new < 0 || !d_len) {
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": bad sizes or NULL lengths");
  }
  if (!k || !v) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": NULL input");
  tq::HybridStage hs{};
  hs.x[0] = k;
  hs.x[1] = v;
  for (int q = 0; q < 2; ++q) {
    const int64_t* xs = q == 0 ? k_strides : v_strides;
    if (xs) {
      if (xs[3] != 1 || xs[0] < 0 || xs[1] < 0 || xs[2] < 0)
        return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": bad input strides");
      hs.xs[q][0] = xs[0];
      hs.xs[q][1] = xs[1];
      hs.xs[q][2] = xs[2];
    } else {
      hs.xs[q][2] = d;
      hs.xs[q][1] = (int64_t)n_new * d;
      hs.xs[q][0] = (int64_t)heads * n_new * d;
    }
  }
  hs.buf[0] = kbuf;
  hs.buf[1] = vbuf;
  hs.n_sets = 2;
  hs.bf16 = x_dtype == TQ_BF16;
  hs.batch = batch;
  hs.heads = heads;
  hs.n_new = n_new;
  hs.d = d;
  hs.block = buf_size;
  hs.len = d_len;
  if (n_new == 0) return TQ_OK;
  // every check passed: stage, flush full rings, stage the rest
  hs.phase = 0;
  hipError_t e = tq::launch_hybrid_stage(hs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_hybrid_append stage launch");
  if (!may_flush) return TQ_OK;
  for (int q = 0; q < 2; ++q) {
    sets.s[q].flush_block = buf_size;
    sets.s[q].flush_new = n_new;
  }
  std::vector<tq::QuantizeParams> blocks;
  std::vector<const tq_codec*> codecs;
  append_blocks(kc, sets.s[0], &blocks, &codecs);
  append_blocks(vc, sets.s[1], &blocks, &codecs);
  tq_status st = launch_blocks("tq_hybrid_append flush", blocks, codecs, stream);
  if (st != TQ_OK) return st;
  hs.phase = 1;
  e = tq::launch_hybrid_stage(hs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_hybrid_append stage launch");
  return TQ_OK;
}

// workspace: the compressed decode's, then the compressed lengths, then the
// rows' (M, L)
static tq_status hybrid_layout(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq, int32_t hkv,
                               int32_t q_len, int64_t max_len, int32_t buf_size, size_t* base, size_t* off_lens,
                               size_t* off_ml, size_t* total, bool* has_compressed) {
  if (buf_size < 1 || buf_size > (1 << 16)) return fail(TQ_ERR_INVALID_ARG, "hybrid decode: bad buffer size");
  const int64_t comp = (max_len / buf_size) * buf_size;
  *has_compressed = comp > 0;
  tq_status st = check_decode_shapes(kc, vc, batch, hq, hkv, q_len, std::max<int64_t>(comp, 1));
  if (st != TQ_OK) return st;
  if (max_len <= 0) return fail(TQ_ERR_INVALID_ARG, "hybrid decode: max_len must be positive");
  *base = *has_compressed ? attention_workspace(kc, vc, batch, hq, hkv, q_len, comp) : 0;
  *off_lens = align256(*base);
  *off_ml = align256(*off_lens + 4 * (size_t)batch);
  *total = align256(*off_ml + 8 * (size_t)batch * hq * q_len);
  return TQ_OK;
}

tq_status tq_hybrid_decode_workspace_size(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t hq,
                                          int32_t hkv, int32_t q_len, int64_t max_len, int32_t buf_size,
                                          size_t* bytes) {
  if (!bytes) return fail(TQ_ERR_INVALID_ARG, "tq_hybrid_decode_workspace_size: bytes is NULL");
  size_t base, ol, om, total;
  bool hc;
  tq_status st = hybrid_layout(kc, vc, batch, hq, hkv, q_len, max_len, buf_size, &base, &ol, &om, &total, &hc);
  if (st != TQ_OK) return st;
  *bytes = total;
  return TQ_OK;
}

tq_status tq_hybrid_decode_attention(const tq_codec* kc, const tq_codec* vc, const void* q, int32_t q_dtype,
                                     int32_t batch, int32_t hq, int32_t hkv, int32_t q_len, const tq_cache* k,
                                     const tq_cache* v, const void* kbuf, const void* vbuf, int32_t buf_dtype,
                                     int32_t buf_size, const int32_t* d_len, int64_t max_len, float scale,
                                     float* out, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "tq_hybrid_decode_attention";
  size_t base, off_lens, off_ml, total;
  bool has_comp;
  tq_status st = hybrid_layout(kc, vc, batch, hq, hkv, q_len, max_len, buf_size, &base, &off_lens, &off_ml, &total,
                               &has_comp);
  if (st != TQ_OK) return st;
  std::string why;
  if (!hybrid_buffers_ok(kbuf, vbuf, buf_dtype, buf_size, &why)) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": " + why);
  if (!q || !d_len || !out || !k || !v) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": NULL argument");
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": bad q_dtype");
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": scale is not finite");
  if (!ws || ws_bytes < total)
    return fail(TQ_ERR_WORKSPACE, std::string(who) + ": workspace needs " + std::to_string(total) + " bytes");
  char* w = static_cast<char*>(ws);
  int32_t* lens_c = reinterpret_cast<int32_t*>(w + off_lens);
  float* row_ml = reinterpret_cast<float*>(w + off_ml);
  if (has_comp) {
    const int64_t comp = (max_len / buf_size) * buf_size;
    // argument checks of the compressed decode before any launch
    std::string cw;
    if (!cache_ok(k, kc->h, &cw) || !cache_ok(v, vc->h, &cw)) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": " + cw);
    if (comp > k->cap) return fail(TQ_ERR_CAPACITY, std::string(who) + ": the compressed part exceeds the cache capacity");
    hipError_t e = tq::launch_hybrid_lens(d_len, lens_c, batch, buf_size, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "tq_hybrid_decode_attention lens launch");
    st = attention_impl(who, false, kc, vc, q, q_dtype, batch, hq, hkv, q_len, k, v, lens_c, comp, scale, out, ws,
                        base, stream, true, d_len, row_ml);
    if (st != TQ_OK) return st;
  }
  tq::HybridAttn a{};
  a.q = q;
  a.q_bf16 = q_dtype == TQ_BF16;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.q_len = q_len;
  a.group = hq / hkv;
  a.d = kc->h.d;
  a.scale = scale;
  a.kbuf = kbuf;
  a.vbuf = vbuf;
  a.buf_bf16 = buf_dtype == TQ_BF16;
  a.block = buf_size;
  a.has_compressed = has_comp ? 1 : 0;
  a.len = d_len;
  a.row_ml = row_ml;
  a.out = out;
  const hipError_t e = tq::launch_hybrid_combine(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_hybrid_decode_attention combine launch");
  return TQ_OK;
}

tq_status tq_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!buf || !sink) return fail(TQ_ERR_INVALID_ARG, "tq_stream_read: NULL argument");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(TQ_ERR_INVALID_ARG, "tq_stream_read: bytes must be a positive multiple of 16, buf 16-byte aligned");
  if (blocks < 1 || blocks > (1 << 20)) return fail(TQ_ERR_INVALID_ARG, "tq_stream_read: blocks out of range");
  const hipError_t e = tq::launch_stream_read(buf, bytes, sink, blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_stream_read launch");
  return TQ_OK;
}

tq_status tq_decode_read_reference(const tq_codec* kc, const tq_codec* vc, int32_t batch, int32_t n_kv_heads,
                                   const tq_cache* k, const tq_cache* v, const int32_t* d_len, int64_t max_len,
                                   uint32_t* sink, uint32_t sink_words, void* stream) {
  const std::string fn = "tq_decode_read_reference";
  if (!kc || !vc || !k || !v || !d_len || !sink) return fail(TQ_ERR_INVALID_ARG, fn + ": NULL argument");
  if (!k->idx || !k->norm || !v->idx || !v->norm) return fail(TQ_ERR_INVALID_ARG, fn + ": cache buffers missing");
  if (!use_fast(kc, vc, 16))
    return fail(TQ_ERR_UNSUPPORTED, fn + ": only the 3-bit MSE head_dim 128 key and value codecs (the int8 decode kernel)");
  if (batch < 1 || n_kv_heads < 1 || batch > 65535 || n_kv_heads > 65535 || sink_words < 1)
    return fail(TQ_ERR_INVALID_ARG, fn + ": batch, heads or sink_words out of range");
  if (k->batch != batch || v->batch != batch || k->heads != n_kv_heads || v->heads != n_kv_heads || k->cap != v->cap)
    return fail(TQ_ERR_CONFIG_MISMATCH, fn + ": caches disagree with batch / heads");
  if (max_len < 1 || max_len > k->cap) return fail(TQ_ERR_CAPACITY, fn + ": max_len outside 1..cap");
  const tq::DecodePlan plan = tq::plan_decode_fast(batch, n_kv_heads, 16, kc->h.d, max_len);
  tq::DecodeParams p{};
  p.batch = batch;
  p.hkv = n_kv_heads;
  p.d = kc->h.d;
  p.k_idx = k->idx;
  p.k_norm = k->norm;
  p.v_idx = v->idx;
  p.v_norm = v->norm;
  p.cap = k->cap;
  p.len = d_len;
  p.chunk = plan.chunk;
  p.n_chunks = plan.n_chunks;
  const hipError_t e = tq::launch_decode_read(p, sink, sink_words, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, (fn + " launch").c_str());
  return TQ_OK;
}

tq_status tq_cache_gather(const tq_codec* src_codec, const tq_cache* src, const tq_codec* dst_codec,
                          const tq_cache* dst, const int32_t* src_batch, const int32_t* src_start,
                          const int32_t* count, void* stream) {
  if (!src_codec || !dst_codec || !src || !dst || !src_batch || !src_start || !count)
    return fail(TQ_ERR_INVALID_ARG, "tq_cache_gather: NULL argument");
  const tq::HostCodec& a = src_codec->h;
  const tq::HostCodec& c = dst_codec->h;
  if (a.d != c.d || a.bits != c.bits || a.mode != c.mode || a.seed != c.seed || a.split_dhi != c.split_dhi)
    return fail(TQ_ERR_CONFIG_MISMATCH, "tq_cache_gather: the caches belong to codecs of different head_dim, bits, "
                                        "mode or seed");
  std::string why;
  if (!cache_ok(src, a, &why)) return fail(TQ_ERR_INVALID_ARG, "tq_cache_gather: source " + why);
  if (!cache_ok(dst, c, &why)) return fail(TQ_ERR_INVALID_ARG, "tq_cache_gather: destination " + why);
  if (src->heads != dst->heads) return fail(TQ_ERR_CONFIG_MISMATCH, "tq_cache_gather: head counts differ");
  if (dst->batch > tq::kMaxGatherBatch)
    return fail(TQ_ERR_UNSUPPORTED, "tq_cache_gather: more than " + std::to_string(tq::kMaxGatherBatch) +
                                        " destination sequences in one call");
  tq::CacheGather g{};
  int64_t max_count = 0;
  for (int b = 0; b < dst->batch; ++b) {
    const int32_t sb = src_batch[b], s0 = src_start[b], n = count[b];
    g.src_batch[b] = sb;
    g.src_start[b] = s0;
    g.count[b] = n;
    if (sb < 0) {
      g.src_batch[b] = -1;
      continue;
    }
    if (sb >= src->batch) return fail(TQ_ERR_INVALID_ARG, "tq_cache_gather: source sequence index out of range");
    if (s0 < 0 || n < 0) return fail(TQ_ERR_INVALID_ARG, "tq_cache_gather: negative start or count");
    if ((int64_t)s0 + n > src->cap) return fail(TQ_ERR_CAPACITY, "tq_cache_gather: range past the source capacity");
    if (n > dst->cap) return fail(TQ_ERR_CAPACITY, "tq_cache_gather: count above the destination capacity");
    max_count = std::max<int64_t>(max_count, n);
  }
  if (max_count == 0) return TQ_OK;
  auto field = [&](const void* s, void* d, int w) {
    g.src[g.n_fields] = static_cast<const uint32_t*>(s);
    g.dst[g.n_fields] = static_cast<uint32_t*>(d);
    g.width[g.n_fields] = w;
    ++g.n_fields;
  };
  field(src->idx, dst->idx, idx_words(a));
  if (a.mode != TQ_MODE_GROUP) field(src->norm, dst->norm, 1);
  if (a.mode == TQ_MODE_PROD) {
    field(src->rnorm, dst->rnorm, 1);
    field(src->sign, dst->sign, sign_words(a));
  }
  if (a.mode == TQ_MODE_GROUP) {
    field(src->scale, dst->scale, group_count(a));
    field(src->gmin, dst->gmin, group_count(a));
  }
  if (a.mode == TQ_MODE_SPLIT) field(src->rnorm, dst->rnorm, 1);  // the high part's norm
  g.heads = dst->heads;
  g.dst_batch = dst->batch;
  g.src_cap = src->cap;
  g.dst_cap = dst->cap;
  const hipError_t e = tq::launch_cache_gather(g, max_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_cache_gather launch");
  return TQ_OK;
}

}  // extern "C"
