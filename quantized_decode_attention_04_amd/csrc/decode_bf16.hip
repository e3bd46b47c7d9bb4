// Decode attention over the compressed cache on the bf16 matrix cores, with
// every fp32 operand split into two bf16 pieces, for head_dim 128 keys whose
// MSE part has 1 or 2 bits (MSE keys, or Prod keys of 2 or 3 bits) and MSE
// values of 1, 2 or 4 bits, at up to 16 query rows per KV head.
//
// What is computed is the fp32 kernels' ("turboquant validate_moe_phase2.py",
// Tests 1 and 5; "omlx turboquant_kv.py", make_mask):
//     s_t = scale * ( n_t <q_rot, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q_rot, sigma_t> )
//     o_rot = sum_t p_t n^v_t c_v[idx^v_t]        (out = Pi_v^T o_rot / l)
// Each product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A
// value x is held as x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (round
// to nearest even: |x - hi - lo| <= 2^-17 |x|), and a product of two split
// operands as a_hi b_hi + a_hi b_lo + a_lo b_hi, which leaves out
// a_lo b_lo (<= 2^-18 |a b|).  The QJL signs are +-1, exact in bf16, so that
// term takes two products; the probabilities are split by truncation (hi =
// the top half of the fp32 word, lo = the truncated rest: |p - hi - lo| <=
// 2^-16 |p|).  The scores and outputs therefore carry relative errors of
// order 1e-5 against the exact fp32 sums, an order below the decode's
// tolerance.
//
// Layout (lane l, m = l % 16, g = l / 16; A[i][k] B[k][j] summed over k, and
// lane l supplies A[m][k] and B[k][m] for the same eight k of its group g):
//   scores  token slot i, row j.  k-step s of lane group g takes the key
//           coordinates 32 g + 8 s + v (v = 0..7) of token 16 tg + m; the
//           codes are spread into bytes (twice the code per byte) and turned
//           into byte selectors of a v_perm over the 4-entry centroid table
//           (bf16 entry c at bytes 2c, 2c+1), for the hi and the lo pieces.
//           The QJL term pairs the coordinates (32 g + 4 s + e, +16), whose
//           sign bits sit 16 apart, so one shift and one mask make the pair
//           of bf16 +-1.  Output: lane (m, g) holds the scores of tokens
//           16 tg + 4 g + r (r = 0..3) for row m, kept as two sums (MSE and
//           QJL) that the token's n and gamma scale afterwards.
//   values  coordinate slot i, row j, k = token: the 32 tokens of half h are
//           the ones whose probabilities the lane already holds (16 tg + 4 g
//           + r, tg = 2h, 2h + 1), so the probabilities never move between
//           lanes; lane m owns the coordinates 8 m .. 8 m + 7, one contiguous
//           run of the token's packed value codes; the value centroids come
//           from a 16-entry (hi | lo << 16) table in LDS.
//
// One 256-thread workgroup per (chunk, KV head, sequence); wave w takes the
// 64-token tiles w, w + 4, ... of the chunk with its own online softmax; the
// four waves' (m, l, o) are combined in LDS into the chunk's partial, which
// the general path's merge kernel merges across chunks.
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTile = 64;
constexpr int kDim = 128;
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

// Byte selectors of k-step s (coordinates 8 s .. 8 s + 7 of the lane's 32):
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
      k = s;
      lo = spread<1>(w[0], 2 * e);
      hi = spread<1>(w[0], 2 * e + 1);
    }
    const uint32_t dup = perm(hi, lo, 0x04040000u + 0x01010101u * (uint32_t)k);
    sel[e] = dup | 0x01000100u;
  }
}

template <int KB, int VB, bool PROD>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_bf16_kernel(DecodeParams p) {
  constexpr int D = kDim;
  constexpr int NU = D / 16;   // value coordinates per lane
  constexpr int VRB = NU * VB; // bits of a lane's value run (8, 16 or 32)
  constexpr uint32_t VMASK = (1u << VB) - 1u;
  __shared__ uint32_t s_vt[16];  // value centroid c: bf16 hi | lo << 16
  __shared__ v4u s_qop[4][4][64];  // [k-step][q hi, q lo, S q hi, S q lo][lane]
  __shared__ float s_o[kWaves][16][D];  // the waves' partial outputs
  __shared__ float s_ml[kWaves][16][2];  // and their (m, l) per row

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

  if (threadIdx.x < 16) {
    uint32_t hi = 0, lo = 0;
    if (threadIdx.x <= VMASK) split_rne(p.v_cent[threadIdx.x], hi, lo);
    s_vt[threadIdx.x] = hi | (lo << 16);
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
  // every wave): MSE term q_rot[32 g + 8 s + v] (hi, lo), QJL term
  // (S q_rot)[32 g + 4 s + e] and [.. + 16] as the pair e (hi, lo); wave w
  // builds k-step w
  {
    const int s = wave;
    const bool rok = m < rows;
    const size_t qoff = ((size_t)bg * rows + (rok ? m : 0)) * D + 32 * g;
    v4u qh, ql, ch, cl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, l;
      split_pair(pick(p.qrot[qoff + 8 * s + 2 * e], rok), pick(p.qrot[qoff + 8 * s + 2 * e + 1], rok), h, l);
      qh[e] = h;
      ql[e] = l;
      ch[e] = cl[e] = 0u;
      if constexpr (PROD) {
        split_pair(pick(p.qs[qoff + 4 * s + e], rok), pick(p.qs[qoff + 4 * s + e + 16], rok), h, l);
        ch[e] = h;
        cl[e] = l;
      }
    }
    s_qop[s][0][lane] = qh;
    s_qop[s][1][lane] = ql;
    s_qop[s][2][lane] = ch;
    s_qop[s][3][lane] = cl;
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
  const char* vnrm = reinterpret_cast<const char*>(p.v_norm + base);
  const char* vidx = reinterpret_cast<const char*>(p.v_idx + base * p.vwords);
  const uint32_t kstride = 4u * p.kwords, sstride = 4u * p.ksign_words, vstride = 4u * p.vwords;
  const uint32_t koff = 4u * g * KB, soff = 4u * g, voff = 4u * ((m * VRB) >> 5);
  const int vshift = (m * VRB) & 31;
  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int T0 = wave * kTile; T0 < ntok; T0 += kWaves * kTile) {
    // Tokens past the chunk's end read the last token instead: every load is
    // valid, and their scores are masked, so they weigh nothing.
    // ---- key words of token T0 + 16 tg + m, coordinates 32 g .. 32 g + 31
    uint32_t kw[4][KB], ksw[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const uint32_t t = (uint32_t)min(T0 + 16 * tg + m, ntok - 1);
#pragma unroll
      for (int w = 0; w < KB; ++w) kw[tg][w] = ld<uint32_t>(kidx, __umul24(t, kstride) + koff + 4u * w);
      ksw[tg] = 0u;
      if constexpr (PROD) ksw[tg] = ld<uint32_t>(ksgn, __umul24(t, sstride) + soff);
    }
    // ---- norms and value runs of the lane's tokens T0 + 16 tg + 4 g + r
    float kn[16], kq[16], vn[16];
    uint32_t vw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t t = (uint32_t)min(T0 + 16 * (i >> 2) + 4 * g + (i & 3), ntok - 1);
      kn[i] = ld<float>(knrm, 4u * t);
      kq[i] = 0.f;
      if constexpr (PROD) kq[i] = ld<float>(krnm, 4u * t) * qjl;
      vn[i] = ld<float>(vnrm, 4u * t);
      vw[i] = ld<uint32_t>(vidx, __umul24(t, vstride) + voff) >> vshift;
    }

    // ---- scores
    v4f sm[4], sq[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) sm[tg] = sq[tg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4u bh = s_qop[s][0][lane], bl = s_qop[s][1][lane];
      const v4u ch = s_qop[s][2][lane], cl = s_qop[s][3][lane];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
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
          const uint32_t ns = ~ksw[tg];
          v4u as;
#pragma unroll
          for (int e = 0; e < 4; ++e) as[e] = ((ns << (15 - (4 * s + e))) & 0x80008000u) | 0x3f803f80u;
          sq[tg] = mfma(as, ch, sq[tg]);
          sq[tg] = mfma(as, cl, sq[tg]);
        }
      }
    }

    // ---- online softmax of row m over this lane's 16 tokens
    float sc[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
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
    float pv[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pr = exp2f(sc[i] - m_ref);
      psum += pr;
      pv[i] = pr * vn[i];
    }
    l_run += psum;

    // ---- values: half h takes the tokens i = 8 h .. 8 h + 7 of the lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4u bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = __float_as_uint(pv[8 * h + 2 * e]), c = __float_as_uint(pv[8 * h + 2 * e + 1]);
        bh[e] = perm(c, a, 0x07060302u);
        const float ra = pv[8 * h + 2 * e] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[8 * h + 2 * e + 1] - __uint_as_float(c & 0xffff0000u);
        bl[e] = perm(__float_as_uint(rc), __float_as_uint(ra), 0x07060302u);
      }
      // LDS byte offsets of the value codes: byte k of va[i][t] is 4 x the
      // code of coordinate (8/VB) k + t of token i
      constexpr int TPB = 8 / VB;
      uint32_t va[8][TPB];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int t = 0; t < TPB; ++t) {
          const int sh = 2 - VB * t;
          const uint32_t w = vw[8 * h + i];
          va[i][t] = (sh >= 0 ? (w << sh) : (w >> -sh)) & (0x01010101u * (VMASK << 2));
        }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        v4u ah, al;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // byte u / TPB, zero-extended (selector 0x0c gives a zero byte)
          const uint32_t bsel = 0x0c0c0c00u + (uint32_t)(u / TPB);
          const uint32_t oa = perm(0u, va[2 * e][u % TPB], bsel);
          const uint32_t oc = perm(0u, va[2 * e + 1][u % TPB], bsel);
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

  // ---- the workgroup's partial: the four waves' (m, l, o) of each row,
  // rescaled to their common maximum and summed through LDS
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    s_ml[wave][m][0] = m_ref;
    s_ml[wave][m][1] = l_run;
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][m][(4 * g + r) * NU + u] = acc[u][r];
  __syncthreads();
  float* po = p.part_o + ((size_t)bg * gridDim.x + chunk_id) * rows * D;
  for (int e = threadIdx.x; e < rows * D; e += kWaves * 64) {
    const int r = e / D, j = e % D;
    float mx = s_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][r][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o = fmaf(s_o[w][r][j], exp2f(s_ml[w][r][0] - mx), o);
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

template <int KB, bool PROD>
hipError_t launch_vb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.vbits) {
    case 1: decode_bf16_kernel<KB, 1, PROD><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 2: decode_bf16_kernel<KB, 2, PROD><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 4: decode_bf16_kernel<KB, 4, PROD><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The decode kernel of this file for a launch that bf16_decode_supported
// accepts; the query prologue and the merge are the caller's.
hipError_t launch_decode_bf16_kernel(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  if (!bf16_decode_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits, p.rows) || p.chunk % (kWaves * kTile))
    return hipErrorInvalidValue;
  const bool prod = p.kmode == TQ_MODE_PROD;
  if (p.kbits == 1) return prod ? launch_vb<1, true>(p, grid, stream) : launch_vb<1, false>(p, grid, stream);
  return prod ? launch_vb<2, true>(p, grid, stream) : launch_vb<2, false>(p, grid, stream);
}

}  // namespace tq
