// Decode attention over the compressed cache on the bf16 matrix cores, with
// every fp32 operand split into two bf16 pieces, for head_dim 128 or 256 keys
// whose MSE part has 1 or 2 bits (MSE keys, or Prod keys of 2 or 3 bits) and
// MSE values of 1, 2 or 4 bits or 2-bit group values, at up to 16 query rows
// per KV head.
//
// What is computed is the fp32 kernels' ("turboquant validate_moe_phase2.py",
// Tests 1, 2 and 5; "omlx turboquant_kv.py", make_mask):
//     s_t = scale * ( n_t <q_rot, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q_rot, sigma_t> )
//     o_rot = sum_t p_t n^v_t c_v[idx^v_t]        (MSE values; out = Pi_v^T o_rot / l)
//     o     = sum_t p_t (q_t s_g + mn_g)          (group values; out = o / l)
// Each product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A
// value x is held as x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (round
// to nearest even: |x - hi - lo| <= 2^-17 |x|), and a product of two split
// operands as a_hi b_hi + a_hi b_lo + a_lo b_hi, which leaves out
// a_lo b_lo (<= 2^-16 |a b|).  The QJL signs are +-1, exact in bf16, so that
// term takes two products; the probabilities are split by truncation (hi =
// the top half of the fp32 word, lo = the truncated rest: |p - hi - lo| <
// 2^-15 |p|).  The scores and outputs therefore carry relative errors of
// order 1e-5 against the exact fp32 sums, an order below the decode's
// tolerance.
//
// Layout (lane l, m = l % 16, g = l / 16; A[i][k] B[k][j] summed over k, and
// lane l supplies A[m][k] and B[k][m] for the same eight k of its group g):
//   scores  token slot i, row j.  k-step s (D/32 of them) of lane group g
//           takes the key coordinates (D/4) g + 8 s + v (v = 0..7) of token
//           16 tg + m; the codes are spread into bytes (twice the code per
//           byte) and turned into byte selectors of a v_perm over the
//           4-entry centroid table (bf16 entry c at bytes 2c, 2c+1), for the
//           hi and the lo pieces.  The QJL term of k-step s takes sign word
//           s / 4 of the lane's D/4 coordinates and pairs its bits
//           (4 (s % 4) + e, +16), so one shift and one mask make the pair of
//           bf16 +-1.  Output: lane (m, g) holds the scores of tokens
//           16 tg + 4 g + r (r = 0..3) for row m, kept as two sums (MSE and
//           QJL) that the token's n and gamma scale afterwards.
//   values  coordinate slot i, row j, k = token: the 32 tokens of half h are
//           the ones whose probabilities the lane already holds (16 tg + 4 g
//           + r, tg = 2h, 2h + 1), so the probabilities never move between
//           lanes; lane m owns the coordinates (D/16) m .. (D/16) m + D/16 - 1,
//           one contiguous run of the token's packed value codes, inside one
//           32-coordinate group.  MSE values: the centroids come from a
//           16-entry (hi | lo << 16) table in LDS.  Group values: the lane
//           builds, per token, the 4-entry table q s + mn of its group (hi
//           and lo pieces, two dwords each) and looks two coordinates of the
//           run up at once with one v_perm per piece.
//
// One 256-thread workgroup per (chunk, KV head, sequence); wave w takes the
// 64-token tiles w, w + 4, ... of the chunk with its own online softmax; the
// four waves' (m, l, o) are combined in LDS (the query operands' space,
// reused once the tiles are done) into the chunk's partial, which the
// general path's merge kernel merges across chunks.
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStep = 256;  // chunks are multiples of this many tokens
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFlushGap = 8.f;  // log2 headroom of the lazy softmax reference

__device__ __forceinline__ v4f mfma(const v4u& a, const v4u& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// A value loaded from a valid address (the caller clamps it), or zero; the
// load itself is unconditional.
template <class T>
__device__ __forceinline__ T pick(T v, bool ok) {
  return ok ? v : T(0);
}

// The T at a byte offset from a base pointer.
template <class T>
__device__ __forceinline__ T ld(const char* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

// bf16 bits of x, rounded to nearest even (finite x)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_rne(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}

// (hi, lo) pairs of two split values, element a in the low half
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  uint32_t ha, la, hb, lb;
  split_rne(a, ha, la);
  split_rne(b, hb, lb);
  hi = ha | (hb << 16);
  lo = la | (lb << 16);
}

// maximum over the four 16-lane groups (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rowmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Twice the code of coordinate (8/KB) k + t of word w, in byte k (t < 8/KB).
template <int KB>
__device__ __forceinline__ uint32_t spread(uint32_t w, int t) {
  constexpr uint32_t mask = KB == 2 ? 0x06060606u : 0x02020202u;
  const int sh = KB * t;
  return (sh == 0 ? (w << 1) : (w >> (sh - 1))) & mask;
}

// Byte selectors of k-step s (coordinates 8 s .. 8 s + 7 of the lane's run):
// dword e covers the coordinates 8 s + 2e and 8 s + 2e + 1.
template <int KB>
__device__ __forceinline__ void key_selectors(const uint32_t* w, int s, uint32_t (&sel)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t lo, hi;
    int k;
    if constexpr (KB == 2) {
      const uint32_t word = w[s >> 1];
      k = 2 * (s & 1) + (e >> 1);
      lo = spread<2>(word, 2 * (e & 1));
      hi = spread<2>(word, 2 * (e & 1) + 1);
    } else {
      const uint32_t word = w[s >> 2];
      k = s & 3;
      lo = spread<1>(word, 2 * e);
      hi = spread<1>(word, 2 * e + 1);
    }
    const uint32_t dup = perm(hi, lo, 0x04040000u + 0x01010101u * (uint32_t)k);
    sel[e] = dup | 0x01000100u;
  }
}

// v_perm selector of two entries of a 4-entry bf16 table (entry c at bytes
// 2c, 2c+1 of the 8-byte pool): the 2-bit codes of run coordinates u (low
// half of the result) and u + NU/2 (high half); run = the lane's codes from
// bit 0, NU of them
template <int NU>
__device__ __forceinline__ uint32_t pair_selector(uint32_t run, int u) {
  if constexpr (NU == 16) {
    // the two codes sit 16 bits apart: bytes 0 and 2 after one shift and mask
    return ((run >> (2 * u)) & 0x00030003u) * 0x0202u + 0x01000100u;
  } else {
    const uint32_t a = (run >> (2 * u)) & 3u, b = (run >> (2 * u + NU)) & 3u;
    return a * 0x0202u + b * 0x02020000u + 0x01000100u;
  }
}

template <int D, int KB, int VB, bool PROD, bool VGROUP>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_bf16_kernel(DecodeParams p) {
  constexpr int KS = D / 32;          // k-steps of the score product
  constexpr int LC = D / 4;           // key coordinates of a lane group
  constexpr int KW = KB * LC / 32;    // key index words of a lane group's coordinates
  constexpr int SW = LC / 32;         // QJL sign words of them
  constexpr int NU = D / 16;          // value coordinates per lane
  constexpr int VRB = NU * VB;        // bits of a lane's value run (8 .. 64)
  constexpr int VW = (VRB + 31) / 32; // words of it
  constexpr uint32_t VMASK = (1u << VB) - 1u;
  // 16-token groups of a wave's tile: 64 tokens at head_dim 128, 32 at 256
  // (the wider head's operands and accumulators leave registers for half as
  // many tokens at two waves per SIMD); NT of them per lane
  constexpr int TG = D == 128 ? 4 : 2;
  constexpr int kTile = 16 * TG;
  constexpr int NT = 4 * TG;
  static_assert(D == 128 || D == 256, "head_dim 128 or 256");
  static_assert(kStep % (kWaves * kTile) == 0, "chunks hold whole workgroup steps");
  static_assert(!VGROUP || VB == 2, "group values of 2 bits");
  // the query operands during the tiles, the waves' partial outputs after them
  constexpr int kQopBytes = KS * 4 * 64 * 16;
  // the waves' outputs: kRows rows of kRS floats, coordinate j at
  // j + 16 (j / GW) (GW = 4 NU coordinates per lane group): kRS = 1 mod 64
  // and the 16-float step per lane group put the 64 lanes of one store
  // (row m, lane group g) in 64 different banks
  constexpr int kRows = D == 128 ? 16 : 8;
  constexpr int GW = 4 * NU;
  constexpr int kRS = ((D + 48 - 1) / 64 + 1) * 64 + 1;
  constexpr int kOutBytes = kWaves * kRows * kRS * 4;
  constexpr int kRawBytes = kQopBytes > kOutBytes ? kQopBytes : kOutBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawBytes];
  __shared__ uint32_t s_vt[16];           // MSE value centroid c: bf16 hi | lo << 16
  __shared__ float s_ml[kWaves][16][2];   // the waves' (m, l) per row
  v4u* s_qop = reinterpret_cast<v4u*>(s_raw);     // [k-step][q hi, q lo, S q hi, S q lo][lane]
  float* s_o = reinterpret_cast<float*>(s_raw);   // [wave][row][kRS]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int chunk_id = blockIdx.x, gh = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + gh;
  const int rows = p.rows;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int ntok = (c0 + p.chunk < len ? c0 + p.chunk : len) - c0;  // may be <= 0
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;  // the causal rule's length
  const int lim = lenm - p.q_len + ((p.row0 + m) % p.q_len) + 1 - c0;  // row m sees tokens < lim

  if constexpr (!VGROUP) {
    if (threadIdx.x < 16) {
      uint32_t hi = 0, lo = 0;
      if (threadIdx.x <= VMASK) split_rne(p.v_cent[threadIdx.x], hi, lo);
      s_vt[threadIdx.x] = hi | (lo << 16);
    }
  }
  // key centroid pools of v_perm: entries 0, 1 in the low word, 2, 3 in the high
  uint32_t kh[2] = {0u, 0u}, kl[2] = {0u, 0u};
#pragma unroll
  for (int c = 0; c < (1 << KB); ++c) {
    uint32_t hi, lo;
    split_rne(p.k_cent[c], hi, lo);
    kh[c >> 1] |= hi << (16 * (c & 1));
    kl[c >> 1] |= lo << (16 * (c & 1));
  }
  // query operands of row m, per k-step s and lane, in LDS (the same for
  // every wave): MSE term q_rot[(D/4) g + 8 s + v] (hi, lo), QJL term
  // (S q_rot)[(D/4) g + 32 (s/4) + 4 (s%4) + e] and [.. + 16] as the pair e
  // (hi, lo); wave w builds the k-steps w, w + 4, ...
  for (int s = wave; s < KS; s += kWaves) {
    const bool rok = m < rows;
    const size_t qoff = ((size_t)bg * rows + (rok ? m : 0)) * D + LC * g;
    v4u qh, ql, ch, cl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, l;
      split_pair(pick(p.qrot[qoff + 8 * s + 2 * e], rok), pick(p.qrot[qoff + 8 * s + 2 * e + 1], rok), h, l);
      qh[e] = h;
      ql[e] = l;
      ch[e] = cl[e] = 0u;
      if constexpr (PROD) {
        const int c = 32 * (s >> 2) + 4 * (s & 3) + e;
        split_pair(pick(p.qs[qoff + c], rok), pick(p.qs[qoff + c + 16], rok), h, l);
        ch[e] = h;
        cl[e] = l;
      }
    }
    s_qop[(4 * s + 0) * 64 + lane] = qh;
    s_qop[(4 * s + 1) * 64 + lane] = ql;
    s_qop[(4 * s + 2) * 64 + lane] = ch;
    s_qop[(4 * s + 3) * 64 + lane] = cl;
  }
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  const float qjl = kQjlConstNumer / (float)D;
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)c0;  // slot of token 0 of the chunk
  // the chunk's fields (uniform bases); a token index t < ntok (< 2^24)
  // addresses them with 24-bit products and 32-bit byte offsets
  const char* kidx = reinterpret_cast<const char*>(p.k_idx + base * p.kwords);
  const char* ksgn = PROD ? reinterpret_cast<const char*>(p.k_sign + base * p.ksign_words) : nullptr;
  const char* knrm = reinterpret_cast<const char*>(p.k_norm + base);
  const char* krnm = PROD ? reinterpret_cast<const char*>(p.k_rnorm + base) : nullptr;
  const char* vnrm = VGROUP ? nullptr : reinterpret_cast<const char*>(p.v_norm + base);
  const char* vscl = VGROUP ? reinterpret_cast<const char*>(p.v_scale + base * p.vgroups) : nullptr;
  const char* vmin = VGROUP ? reinterpret_cast<const char*>(p.v_gmin + base * p.vgroups) : nullptr;
  const char* vidx = reinterpret_cast<const char*>(p.v_idx + base * p.vwords);
  const uint32_t kstride = 4u * p.kwords, sstride = 4u * p.ksign_words, vstride = 4u * p.vwords;
  const uint32_t gstride = 4u * p.vgroups;
  const uint32_t koff = 4u * g * KW, soff = 4u * g * SW, voff = 4u * ((m * VRB) >> 5);
  const uint32_t goff = 4u * ((m * NU) >> 5);  // the group of the lane's value run
  const int vshift = (m * VRB) & 31;
  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  // Tokens past the chunk's end read the last token instead: every load is
  // valid, and their scores are masked, so they weigh nothing.
  // ---- key words of token T0 + 16 tg + m, coordinates (D/4) g .. (D/4) g +
  // D/4 - 1: each tile's are loaded one tile ahead (the scores need them
  // first; the other fields are used only after the scores)
  uint32_t nkw[TG][KW], nksw[TG][SW];
  auto load_keys = [&](int T0) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const uint32_t t = (uint32_t)max(min(T0 + 16 * tg + m, ntok - 1), 0);
#pragma unroll
      for (int w = 0; w < KW; ++w) nkw[tg][w] = ld<uint32_t>(kidx, __umul24(t, kstride) + koff + 4u * w);
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        nksw[tg][w] = 0u;
        if constexpr (PROD) nksw[tg][w] = ld<uint32_t>(ksgn, __umul24(t, sstride) + soff + 4u * w);
      }
    }
  };
  if (wave * kTile < ntok) load_keys(wave * kTile);

  for (int T0 = wave * kTile; T0 < ntok; T0 += kWaves * kTile) {
    uint32_t kw[TG][KW], ksw[TG][SW];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
      for (int w = 0; w < KW; ++w) kw[tg][w] = nkw[tg][w];
#pragma unroll
      for (int w = 0; w < SW; ++w) ksw[tg][w] = nksw[tg][w];
    }
    // ---- key norms and value fields of the lane's tokens T0 + 16 tg + 4 g
    // + r (token i: tg = i / 4, r = i % 4)
    float kn[NT], kq[NT], vn[NT], vs[NT];
    uint32_t vw[NT][VW];
    auto token_of = [&](int i) { return (uint32_t)min(T0 + 16 * (i >> 2) + 4 * g + (i & 3), ntok - 1); };
    auto load_values = [&](int i) {
      const uint32_t t = token_of(i);
      if constexpr (VGROUP) {
        vs[i] = ld<float>(vscl, __umul24(t, gstride) + goff);
        vn[i] = ld<float>(vmin, __umul24(t, gstride) + goff);
      } else {
        vn[i] = ld<float>(vnrm, 4u * t);
        vs[i] = 0.f;
      }
#pragma unroll
      for (int w = 0; w < VW; ++w) vw[i][w] = ld<uint32_t>(vidx, __umul24(t, vstride) + voff + 4u * w);
      if constexpr (VW == 1) vw[i][0] >>= vshift;
    };
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint32_t t = token_of(i);
      kn[i] = ld<float>(knrm, 4u * t);
      kq[i] = 0.f;
      if constexpr (PROD) kq[i] = ld<float>(krnm, 4u * t) * qjl;
      load_values(i);
    }
    // the next tile's key words (the last tile's reads of the chunk's last
    // token are never used)
    load_keys(T0 + kWaves * kTile);

    // ---- scores
    v4f sm[TG], sq[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) sm[tg] = sq[tg] = v4f{0.f, 0.f, 0.f, 0.f};
    // the query operands of k-step s + 1 are read while k-step s computes;
    // the scheduling barrier at the end of each k-step keeps the compiler from
    // hoisting every k-step's reads (their registers) to the top
    v4u nbh = s_qop[0 * 64 + lane], nbl = s_qop[1 * 64 + lane];
    v4u nch = v4u{0u, 0u, 0u, 0u}, ncl = v4u{0u, 0u, 0u, 0u};
    if constexpr (PROD) {
      nch = s_qop[2 * 64 + lane];
      ncl = s_qop[3 * 64 + lane];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const v4u bh = nbh, bl = nbl, ch = nch, cl = ncl;
      if (s + 1 < KS) {
        nbh = s_qop[(4 * s + 4) * 64 + lane];
        nbl = s_qop[(4 * s + 5) * 64 + lane];
        if constexpr (PROD) {
          nch = s_qop[(4 * s + 6) * 64 + lane];
          ncl = s_qop[(4 * s + 7) * 64 + lane];
        }
      }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        uint32_t sel[4];
        key_selectors<KB>(kw[tg], s, sel);
        v4u ah, al;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ah[e] = perm(kh[1], kh[0], sel[e]);
          al[e] = perm(kl[1], kl[0], sel[e]);
        }
        sm[tg] = mfma(ah, bh, sm[tg]);
        sm[tg] = mfma(ah, bl, sm[tg]);
        sm[tg] = mfma(al, bh, sm[tg]);
        if constexpr (PROD) {
          const uint32_t ns = ~ksw[tg][s >> 2];
          const int sb = 4 * (s & 3);
          v4u as;
#pragma unroll
          for (int e = 0; e < 4; ++e) as[e] = ((ns << (15 - (sb + e))) & 0x80008000u) | 0x3f803f80u;
          sq[tg] = mfma(as, ch, sq[tg]);
          sq[tg] = mfma(as, cl, sq[tg]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax of row m over this lane's NT tokens
    float sc[NT];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int tok = T0 + 16 * (i >> 2) + 4 * g + (i & 3);
      const float raw = PROD ? fmaf(kn[i], sm[i >> 2][i & 3], kq[i] * sq[i >> 2][i & 3]) : kn[i] * sm[i >> 2][i & 3];
      const float v = (tok < ntok && tok < lim) ? raw * sl2 : -INFINITY;
      sc[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = rowmax4(tmax);
    if (__ballot(tmax > m_ref + kFlushGap) != 0) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = exp2f(m_ref - m_new);
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] *= alpha;
      l_run *= alpha;
      m_ref = m_new;
    }
    float pv[NT];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float pr = exp2f(sc[i] - m_ref);
      psum += pr;
      pv[i] = VGROUP ? pr : pr * vn[i];
    }
    l_run += psum;

    // ---- values: half h takes the tokens i = 8 h .. 8 h + 7 of the lane
#pragma unroll
    for (int h = 0; h < TG / 2; ++h) {
      v4u bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = __float_as_uint(pv[8 * h + 2 * e]), c = __float_as_uint(pv[8 * h + 2 * e + 1]);
        bh[e] = perm(c, a, 0x07060302u);
        const float ra = pv[8 * h + 2 * e] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[8 * h + 2 * e + 1] - __uint_as_float(c & 0xffff0000u);
        bl[e] = perm(__float_as_uint(rc), __float_as_uint(ra), 0x07060302u);
      }
      if constexpr (VGROUP) {
        // the 4-entry table q s + mn of each token's group: entries 0, 1 in
        // the low dword, 2, 3 in the high one, hi and lo pieces apart
        uint32_t th[8][2], tl[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = vs[8 * h + i], mn = vn[8 * h + i];
          split_pair(mn, mn + sg, th[i][0], tl[i][0]);
          split_pair(fmaf(2.f, sg, mn), fmaf(3.f, sg, mn), th[i][1], tl[i][1]);
        }
#pragma unroll
        for (int u = 0; u < NU / 2; ++u) {
          // coordinates u and u + NU/2 of the run, for the token pairs e
          v4u ah0, al0, ah1, al1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ia = 2 * e, ib = 2 * e + 1;
            const uint32_t sa = pair_selector<NU>(vw[8 * h + ia][0], u);
            const uint32_t sb = pair_selector<NU>(vw[8 * h + ib][0], u);
            const uint32_t xa = perm(th[ia][1], th[ia][0], sa), xb = perm(th[ib][1], th[ib][0], sb);
            const uint32_t ya = perm(tl[ia][1], tl[ia][0], sa), yb = perm(tl[ib][1], tl[ib][0], sb);
            ah0[e] = perm(xb, xa, 0x05040100u);
            ah1[e] = perm(xb, xa, 0x07060302u);
            al0[e] = perm(yb, ya, 0x05040100u);
            al1[e] = perm(yb, ya, 0x07060302u);
          }
          acc[u] = mfma(ah0, bh, acc[u]);
          acc[u] = mfma(ah0, bl, acc[u]);
          acc[u] = mfma(al0, bh, acc[u]);
          acc[u + NU / 2] = mfma(ah1, bh, acc[u + NU / 2]);
          acc[u + NU / 2] = mfma(ah1, bl, acc[u + NU / 2]);
          acc[u + NU / 2] = mfma(al1, bh, acc[u + NU / 2]);
        }
      } else {
        // LDS byte offsets of the value codes: byte k of va[i][w][t] is 4 x
        // the code of run coordinate (32 w + 8 k) / VB + t of token i
        constexpr int TPB = 8 / VB;
        uint32_t va[8][VW][TPB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int w = 0; w < VW; ++w)
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
              const int sh = 2 - VB * t;
              const uint32_t x = vw[8 * h + i][w];
              va[i][w][t] = (sh >= 0 ? (x << sh) : (x >> -sh)) & (0x01010101u * (VMASK << 2));
            }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          constexpr int kBitsPerWord = 32;
          const int bit = u * VB, w = bit / kBitsPerWord, byte = (bit % kBitsPerWord) / 8;
          v4u ah, al;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // byte `byte`, zero-extended (selector 0x0c gives a zero byte)
            const uint32_t bsel = 0x0c0c0c00u + (uint32_t)byte;
            const uint32_t oa = perm(0u, va[2 * e][w][u % TPB], bsel);
            const uint32_t oc = perm(0u, va[2 * e + 1][w][u % TPB], bsel);
            const uint32_t ta = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oa);
            const uint32_t tc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oc);
            ah[e] = perm(tc, ta, 0x05040100u);
            al[e] = perm(tc, ta, 0x07060302u);
          }
          acc[u] = mfma(ah, bh, acc[u]);
          acc[u] = mfma(ah, bl, acc[u]);
          acc[u] = mfma(al, bh, acc[u]);
        }
      }
    }
  }

  // ---- the workgroup's partial: the four waves' (m, l, o) of each row,
  // rescaled to their common maximum and summed through LDS (over the query
  // operands, which every wave has finished with at the barrier)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  if (g == 0) {
    s_ml[wave][m][0] = m_ref;
    s_ml[wave][m][1] = l_run;
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (4 * g + r) * NU + u;
      if (m < rows) s_o[(wave * kRows + m) * kRS + j + 16 * (j / GW)] = acc[u][r];
    }
  __syncthreads();
  float* po = p.part_o + ((size_t)bg * gridDim.x + chunk_id) * rows * D;
  for (int e = threadIdx.x; e < rows * D; e += kWaves * 64) {
    const int r = e / D, j = e % D;
    float mx = s_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][r][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      o = fmaf(s_o[(w * kRows + r) * kRS + j + 16 * (j / GW)], exp2f(s_ml[w][r][0] - mx), o);
    po[e] = o;
  }
  if (threadIdx.x < rows) {
    const int r = threadIdx.x;
    float mx = s_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][r][0]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l = fmaf(s_ml[w][r][1], exp2f(s_ml[w][r][0] - mx), l);
    float* pml = p.part_ml + (((size_t)bg * gridDim.x + chunk_id) * rows + r) * 2;
    pml[0] = mx;
    pml[1] = l;
  }
}

template <int D, int KB, bool PROD>
hipError_t launch_vb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (p.vmode == TQ_MODE_GROUP) {
    if (p.vbits != 2) return hipErrorInvalidValue;
    decode_bf16_kernel<D, KB, 2, PROD, true><<<grid, block, 0, stream>>>(p);
    return hipGetLastError();
  }
  switch (p.vbits) {
    case 1: decode_bf16_kernel<D, KB, 1, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 2: decode_bf16_kernel<D, KB, 2, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 4: decode_bf16_kernel<D, KB, 4, PROD, false><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  const bool prod = p.kmode == TQ_MODE_PROD;
  if (p.kbits == 1) return prod ? launch_vb<D, 1, true>(p, grid, stream) : launch_vb<D, 1, false>(p, grid, stream);
  return prod ? launch_vb<D, 2, true>(p, grid, stream) : launch_vb<D, 2, false>(p, grid, stream);
}

}  // namespace

// The decode kernel of this file for a launch that bf16_decode_supported
// accepts; the query prologue and the merge are the caller's.  Token indices
// inside a chunk use 24-bit products: chunks hold at most 2^24 tokens.
hipError_t launch_decode_bf16_kernel(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  if (!bf16_decode_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits, p.rows) || p.chunk % kStep ||
      p.chunk > (1 << 24))
    return hipErrorInvalidValue;
  return p.d == 128 ? launch_d<128>(p, grid, stream) : launch_d<256>(p, grid, stream);
}

}  // namespace tq
