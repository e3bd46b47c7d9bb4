// Host-only checks of libtq.so's C ABI, codec builder and dispatch logic, built
// with -fsanitize=address,undefined (tests/test_host_sanitizers.py).  Every
// codec the library accepts is built, described and exported; every argument
// check is driven with placeholder pointers that the host refuses before any
// launch.  Exit status 0 and "host checks passed" on success.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tq.h"

namespace tq {
extern int g_stub_launches;
}

static int g_failures = 0;

#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_failures;                                                       \
    }                                                                     \
  } while (0)

static tq_cache fake_cache(int batch, int heads, int64_t cap, bool group) {
  static uint32_t word = 0;
  float* f = reinterpret_cast<float*>(&word);
  tq_cache c{&word, group ? nullptr : f, f, &word, f, f, batch, heads, cap};
  return c;
}

static void codecs() {
  const int modes[3][2] = {{TQ_MODE_MSE, 1}, {TQ_MODE_PROD, 2}, {TQ_MODE_GROUP, 1}};
  for (int d = 32; d <= 256; d += 32) {
    for (const auto& m : modes) {
      for (int bits = m[1]; bits < m[1] + 4; ++bits) {
        tq_codec* c = nullptr;
        CHECK(tq_codec_create(d, bits, 1234567u + d, m[0], &c) == TQ_OK);
        if (!c) continue;
        tq_codec_info info{};
        CHECK(tq_codec_get_info(c, &info) == TQ_OK);
        CHECK(info.head_dim == d && info.bits == bits && info.mode == m[0]);
        std::vector<float> rot((size_t)d * d), sk((size_t)d * d), cent(16), bnd(16);
        CHECK(tq_codec_export(c, rot.data(), cent.data(), bnd.data(), sk.data()) == TQ_OK);
        if (m[0] != TQ_MODE_GROUP) {
          // orthogonal rotation, ascending centroids, midpoint boundaries
          double worst = 0.0;
          for (int i = 0; i < d; i += 7)
            for (int j = 0; j < d; j += 5) {
              double acc = 0.0;
              for (int k = 0; k < d; ++k) acc += (double)rot[(size_t)k * d + i] * rot[(size_t)k * d + j];
              worst = std::fmax(worst, std::fabs(acc - (i == j ? 1.0 : 0.0)));
            }
          CHECK(worst < 1e-5);
          for (int k = 0; k + 1 < info.levels; ++k) {
            CHECK(cent[k] < cent[k + 1]);
            CHECK(bnd[k] == 0.5f * (cent[k] + cent[k + 1]));
          }
        }
        tq_codec_destroy(c);
      }
    }
  }
  // fractional widths: the key/value pair rule and split codecs with their parts
  for (double b : {1.5, 2.5, 3.5, 3.25, 2.75, 3.0, 4.0000001}) {
    tq_codec *k = nullptr, *v = nullptr;
    CHECK(tq_codec_create_kv(128, b, 3, &k, &v) == TQ_OK);
    tq_codec_info ki{}, vi{};
    CHECK(tq_codec_get_info(k, &ki) == TQ_OK && tq_codec_get_info(v, &vi) == TQ_OK);
    CHECK(ki.bits == (int)std::floor(b + 1e-6) && vi.bits == (int)std::ceil(b - 1e-6) && vi.seed == 4);
    tq_codec_destroy(k);
    tq_codec_destroy(v);
    tq_codec* sp = nullptr;
    const bool frac = std::fabs(b - std::nearbyint(b)) > 1e-6;
    CHECK((tq_codec_create_split(128, b, 3, &sp) == TQ_OK) == frac);
    if (sp) {
      tq_codec_info si{}, li{}, hi{};
      const tq_codec *lo = nullptr, *hp = nullptr;
      CHECK(tq_codec_get_info(sp, &si) == TQ_OK && si.mode == TQ_MODE_SPLIT);
      CHECK(tq_codec_part(sp, 0, &lo) == TQ_OK && tq_codec_part(sp, 1, &hp) == TQ_OK);
      CHECK(tq_codec_get_info(lo, &li) == TQ_OK && tq_codec_get_info(hp, &hi) == TQ_OK);
      CHECK(li.head_dim + hi.head_dim == 128 && hi.head_dim == si.split_high_dim && hi.bits == li.bits + 1);
      CHECK(si.idx_words == li.idx_words + hi.idx_words && si.idx_words == (int)std::ceil(128 * b / 32));
      CHECK(tq_codec_part(sp, 2, &lo) == TQ_ERR_INVALID_ARG);
      std::vector<float> rot(128 * 128);
      CHECK(tq_codec_export(sp, rot.data(), nullptr, nullptr, nullptr) == TQ_OK);
      CHECK(rot[(size_t)0 * 128 + 127] == 0.0f && rot[(size_t)127 * 128 + 0] == 0.0f);  // block diagonal
      tq_codec_destroy(sp);
    }
  }
  tq_codec* c = nullptr;
  CHECK(tq_codec_create_split(128, 3.1, 0, &c) == TQ_ERR_UNSUPPORTED);   // a part below 32 channels
  CHECK(tq_codec_create_split(128, 4.5, 0, &c) == TQ_ERR_UNSUPPORTED);   // 5 bits
  CHECK(tq_codec_create_split(32, 2.5, 0, &c) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codec_create_kv(128, 3.5, 0, nullptr, &c) == TQ_ERR_INVALID_ARG);
  CHECK(tq_codec_part(nullptr, 0, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_codec_create(100, 3, 0, TQ_MODE_MSE, &c) == TQ_ERR_UNSUPPORTED && c == nullptr);
  CHECK(tq_codec_create(288, 3, 0, TQ_MODE_MSE, &c) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codec_create(128, 5, 0, TQ_MODE_MSE, &c) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codec_create(128, 1, 0, TQ_MODE_PROD, &c) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codec_create(128, 3, 0, 7, &c) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codec_create(128, 3, 0, TQ_MODE_MSE, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_codec_get_info(nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  tq_codec_destroy(nullptr);
}

static void decode_and_append() {
  tq_codec *kc = nullptr, *vc = nullptr, *kp = nullptr, *vg = nullptr;
  CHECK(tq_codec_create(128, 3, 0, TQ_MODE_MSE, &kc) == TQ_OK);
  CHECK(tq_codec_create(128, 3, 1, TQ_MODE_MSE, &vc) == TQ_OK);
  CHECK(tq_codec_create(256, 3, 0, TQ_MODE_PROD, &kp) == TQ_OK);
  CHECK(tq_codec_create(256, 2, 1, TQ_MODE_GROUP, &vg) == TQ_OK);
  size_t need = 0, other = 0;
  // workspace sizes over every path and a range of shapes
  for (int rows_q : {1, 2, 4, 8, 16})
    for (int64_t n : {1, 63, 64, 4097, 262144, 1 << 26}) {
      CHECK(tq_decode_workspace_size(kc, vc, 1, 8 * rows_q, 8, 1, n, &need) == TQ_OK);
      CHECK(tq_prefill_workspace_size(kc, vc, 3, 8, 8, 500, n, &other) == TQ_OK);
      CHECK(tq_decode_workspace_size(kp, vg, 2, 2 * (rows_q > 8 ? 8 : rows_q), 2, 1, n, &need) == TQ_OK);
    }
  CHECK(tq_decode_workspace_size(kc, vc, 1, 8, 8, 1, ((int64_t)1 << 26) + 1, &need) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_decode_workspace_size(kc, vc, 1, 68, 2, 1, 10, &need) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_decode_workspace_size(kc, vc, 1, 8, 8, 1, 10, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_decode_workspace_size(vg, vc, 1, 8, 8, 1, 10, &need) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_decode_workspace_size(kc, kp, 1, 8, 8, 1, 10, &need) == TQ_ERR_UNSUPPORTED);

  static char placeholder[64];
  void* P = placeholder;
  tq_cache k = fake_cache(1, 8, 100, false), v = fake_cache(1, 8, 100, false);
  CHECK(tq_decode_workspace_size(kc, vc, 1, 64, 8, 1, 100, &need) == TQ_OK);
  auto dec = [&](tq_cache* kk, tq_cache* vv, int64_t max_len, size_t ws, const void* q, float scale) {
    return tq_decode_attention(kc, vc, q, TQ_BF16, 1, 64, 8, 1, kk, vv, (const int32_t*)P, max_len, scale,
                               (float*)P, P, ws, nullptr);
  };
  CHECK(dec(&k, &v, 100, need, nullptr, 0.1f) == TQ_ERR_INVALID_ARG);
  CHECK(dec(&k, &v, 100, need, P, NAN) == TQ_ERR_INVALID_ARG);
  CHECK(dec(&k, &v, 100, need - 1, P, 0.1f) == TQ_ERR_WORKSPACE);
  CHECK(dec(&k, &v, 101, need, P, 0.1f) == TQ_ERR_CAPACITY);
  tq_cache v99 = fake_cache(1, 8, 99, false), k4 = fake_cache(1, 4, 100, false);
  CHECK(dec(&k, &v99, 50, need, P, 0.1f) == TQ_ERR_CONFIG_MISMATCH);
  CHECK(dec(&k4, &v, 100, need, P, 0.1f) == TQ_ERR_CONFIG_MISMATCH);
  tq_cache bad = fake_cache(1, 8, 100, false);
  bad.norm = nullptr;
  CHECK(dec(&bad, &v, 100, need, P, 0.1f) == TQ_ERR_INVALID_ARG);
  tq_cache huge = fake_cache(1, 8, ((int64_t)1 << 26) + 1, false);
  CHECK(dec(&huge, &huge, ((int64_t)1 << 26) + 1, need, P, 0.1f) == TQ_ERR_UNSUPPORTED);

  const int64_t strides[4] = {8 * 2 * 128, 2 * 128, 128, 1}, bad_strides[4] = {0, 0, 0, 2};
  auto app = [&](tq_cache* c, const void* x, int n, const int64_t* st, int dt, int64_t end) {
    return tq_quantize_append(kc, x, dt, 1, 8, n, st, c, (const int32_t*)P, end, nullptr);
  };
  CHECK(app(&k, nullptr, 2, strides, TQ_BF16, 100) == TQ_ERR_INVALID_ARG);
  CHECK(app(&k, P, 2, strides, 5, 100) == TQ_ERR_INVALID_ARG);
  CHECK(app(&k, P, -1, strides, TQ_BF16, 100) == TQ_ERR_INVALID_ARG);
  CHECK(app(&k, P, 2, bad_strides, TQ_BF16, 100) == TQ_ERR_INVALID_ARG);
  CHECK(app(&k, P, 2, strides, TQ_BF16, 101) == TQ_ERR_CAPACITY);
  CHECK(app(&k, P, 2, strides, TQ_BF16, 1) == TQ_ERR_INVALID_ARG);
  CHECK(app(&k, P, 0, strides, TQ_BF16, 0) == TQ_OK);  // nothing to do
  tq_cache b2 = fake_cache(2, 8, 100, false);
  CHECK(app(&b2, P, 2, strides, TQ_BF16, 100) == TQ_ERR_CONFIG_MISMATCH);
  tq_cache v50 = fake_cache(1, 8, 50, false);
  CHECK(tq_quantize_append_kv(kc, vc, P, P, TQ_BF16, 1, 8, 2, strides, strides, &k, &v50, (const int32_t*)P, 51,
                              nullptr) == TQ_ERR_CAPACITY);

  // record copies: codec guard, heads, ranges
  int32_t sb[2] = {0, -1}, s0[2] = {0, 0}, cnt[2] = {10, 0};
  tq_cache src = fake_cache(1, 8, 100, false), dst = fake_cache(2, 8, 40, false);
  CHECK(tq_cache_gather(kc, &src, vc, &dst, sb, s0, cnt, nullptr) == TQ_ERR_CONFIG_MISMATCH);  // seeds differ
  tq_cache dst4 = fake_cache(2, 4, 40, false);
  CHECK(tq_cache_gather(kc, &src, kc, &dst4, sb, s0, cnt, nullptr) == TQ_ERR_CONFIG_MISMATCH);
  int32_t cnt_big[2] = {41, 0}, sb_bad[2] = {1, -1}, s0_far[2] = {95, 0};
  CHECK(tq_cache_gather(kc, &src, kc, &dst, sb, s0, cnt_big, nullptr) == TQ_ERR_CAPACITY);
  CHECK(tq_cache_gather(kc, &src, kc, &dst, sb_bad, s0, cnt, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_cache_gather(kc, &src, kc, &dst, sb, s0_far, cnt, nullptr) == TQ_ERR_CAPACITY);

  for (int s = 0; s <= 8; ++s) CHECK(tq_status_string(s) != nullptr);
  CHECK(tq_last_error() != nullptr);
  tq_codec_destroy(kc);
  tq_codec_destroy(vc);
  tq_codec_destroy(kp);
  tq_codec_destroy(vg);
}

int main() {
  codecs();
  decode_and_append();
  CHECK(tq::g_stub_launches == 0);  // every refused call was refused before a launch
  if (g_failures) {
    std::fprintf(stderr, "%d host checks failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
