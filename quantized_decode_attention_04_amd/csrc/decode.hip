// Decode attention over the compressed cache for gfx950.
//
// What is computed ("turboquant validate_moe_phase2.py", Tests 1 and 5:
// scores scaled by 1/sqrt(head_dim), softmax, weighted values, compared in
// the original domain; "omlx turboquant_kv.py", make_mask: new tokens see the
// cache causally): for each sequence b, KV head g and query row r (query
// head g*G + r/q_len, new-token row r%q_len) the softmax over the visible
// cached tokens of
//     s_t = scale * ( n_t <Pi_k q, c_k[idx_t]>
//                     + gamma_t sqrt(pi/2)/d <S Pi_k q, sigma_t> )     (Prod)
// weights the values; MSE values are accumulated in the rotated domain,
//     o_rot = sum_t p_t n^v_t c_v[idx^v_t],   out = Pi_v^T o_rot / l,
// group values in the original domain, o = sum_t p_t (q_t s_g + mn_g).
//
// Structure (the token axis is split across workgroups, "split-K"):
//   qprep_kernel   one workgroup per (row, b, g): q_rot = Pi_k q (and S q_rot);
//   decode_kernel  one workgroup per (chunk, g, b): tiles of 256 tokens;
//                  phase A scores one token per thread against the rotated
//                  queries in LDS (centroid look-up table in LDS), phase B
//                  runs the online softmax per row, phase C accumulates the
//                  values with one thread per coordinate; the partial
//                  (m, l, o) of the chunk goes to the workspace;
//   merge_kernel   one workgroup per (row, g, b): merges the chunks and applies
//                  the single inverse rotation Pi_v^T (a stream-ordered second
//                  kernel: a last-arriving-workgroup merge would need a
//                  device-scope fence per workgroup, which writes back and
//                  invalidates the L2 of every XCD).
// Scores are kept in the log2 domain (multiplied by log2 e) so that the
// softmax uses exp2.
#include "chunk_order.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kTile = 256;
constexpr int kMaxMergeChunks = 4096;  // merge weights kept in LDS
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float load_q(const void* q, int64_t off, int bf16) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(q)[off]) << 16);
  return static_cast<const float*>(q)[off];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Field of coordinate r (0..31) of one 32-coordinate group whose B words are
// w[0..B-1] (the packed layout: LSB-first for 1, 2, 4 bits; byte lanes X, Y, Z
// for 3 bits).
template <int B>
__device__ __forceinline__ uint32_t group_field(const uint32_t* w, int r) {
  if constexpr (B == 3) {
    const int a = r >> 2, s = 8 * (r & 3);
    switch (a) {
      case 0: return (w[0] >> s) & 7u;
      case 1: return (w[0] >> (s + 3)) & 7u;
      case 2: return ((w[0] >> (s + 6)) & 3u) | (((w[2] >> (s + 6)) & 1u) << 2);
      case 3: return (w[1] >> s) & 7u;
      case 4: return (w[1] >> (s + 3)) & 7u;
      case 5: return ((w[1] >> (s + 6)) & 3u) | (((w[2] >> (s + 7)) & 1u) << 2);
      case 6: return (w[2] >> s) & 7u;
      default: return (w[2] >> (s + 3)) & 7u;
    }
  } else {
    const int bit = r * B;
    return (w[bit >> 5] >> (bit & 31)) & ((1u << B) - 1u);
  }
}

// Same, reading the words of coordinate j of a token straight from memory.
template <int B>
__device__ __forceinline__ uint32_t token_field(const uint32_t* tokw, int j) {
  const uint32_t* w = tokw + (j >> 5) * B;
  if constexpr (B == 3) {
    uint32_t ww[3] = {w[0], w[1], w[2]};
    return group_field<3>(ww, j & 31);
  } else {
    const int bit = (j & 31) * B;
    return (w[bit >> 5] >> (bit & 31)) & ((1u << B) - 1u);
  }
}

// q_rot = Pi_k q, and for Prod keys S q_rot = (S Pi_k) q, for one query row:
// one workgroup of 4 D threads per (row, sequence x KV head, product), the
// two products in parallel workgroups (blockIdx.z); thread (i, k) sums the
// quarter k of coordinate i's D terms, with all of its table loads issued
// before the query row is staged (coalesced across i), and the quarters are
// added through LDS.
template <int D>
__global__ __launch_bounds__(4 * D) void qprep_kernel(DecodeParams p) {
  constexpr int Q = D / 4;  // terms per thread
  static_assert(D % 4 == 0, "quarters");
  __shared__ float s_in[D], s_part[4][D];
  const int r = blockIdx.x, bg = blockIdx.y;
  const bool sq = blockIdx.z == 1;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int i = threadIdx.x % D, k = threadIdx.x / D;
  const int R = p.row0 + r;  // row among the KV head's group * q_len rows
  const int h = g * p.group + R / p.q_len, qi = R % p.q_len;
  const int64_t qoff = (((int64_t)b * p.hq + h) * p.q_len + qi) * D;
  const float* mt = sq ? p.k_spt : p.k_pit;
  float pv[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) pv[t] = mt[(size_t)(k * Q + t) * D + i];
  if (k == 0) s_in[i] = load_q(p.q, qoff + i, p.q_bf16);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < Q; ++t) acc = fmaf(pv[t], s_in[k * Q + t], acc);
  s_part[k][i] = acc;
  __syncthreads();
  const size_t e = ((size_t)bg * p.rows + r) * D + i;
  if (k == 0) (sq ? p.qs : p.qrot)[e] = (s_part[0][i] + s_part[1][i]) + (s_part[2][i] + s_part[3][i]);
}

// the prologue's grid: rows x (sequence x KV head) x (1, or 2 for Prod keys)
inline dim3 qprep_grid(const DecodeParams& p) {
  return dim3(p.rows, p.batch * p.hkv, p.kmode == TQ_MODE_PROD ? 2 : 1);
}

// Scores of one token against all rows (rows beyond p.rows read zeros).
template <int D, int RMAX, int KB, bool PROD>
__device__ __forceinline__ void score_token(const DecodeParams& p, int64_t slot, const float* s_q, const float* s_qs,
                                            const float* s_kc, float (&s)[RMAX]) {
  float am[RMAX], aq[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) am[r] = aq[r] = 0.f;
  const uint32_t* kw = p.k_idx + slot * (int64_t)(D * KB / 32);
  for (int gi = 0; gi < D / 32; ++gi) {
    uint32_t w[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) w[u] = kw[gi * KB + u];
    uint32_t sw = 0;
    if constexpr (PROD) sw = p.k_sign[slot * (int64_t)(D / 32) + gi];
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      const int j = gi * 32 + rr;
      const float c = s_kc[group_field<KB>(w, rr)];
      const float sg = ((sw >> rr) & 1u) ? 1.f : -1.f;
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        am[r] = fmaf(s_q[r * D + j], c, am[r]);
        if constexpr (PROD) aq[r] = fmaf(s_qs[r * D + j], sg, aq[r]);
      }
    }
  }
  const float n = p.k_norm[slot];
  float gq = 0.f;
  if constexpr (PROD) gq = p.k_rnorm[slot] * (kQjlConstNumer / (float)D);
#pragma unroll
  for (int r = 0; r < RMAX; ++r) s[r] = n * am[r] + (PROD ? gq * aq[r] : 0.f);
}

// Scores of one token of a split key cache: the low part's groups (KB-bit
// codes, centroids s_kc, norm k_norm) and the high part's (KB+1 bits, s_kc2,
// k_norm_hi) against the rotated query (the block-diagonal rotation rotates
// each part's channels by its own matrix).
template <int D, int RMAX, int KB>
__device__ __forceinline__ void score_token_split(const DecodeParams& p, int64_t slot, const float* s_q,
                                                  const float* s_kc, const float* s_kc2, float (&s)[RMAX]) {
  constexpr int KH = KB + 1;
  float al[RMAX], ah[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) al[r] = ah[r] = 0.f;
  const int glo = p.ksplit_g;
  const uint32_t* kw = p.k_idx + slot * (int64_t)p.kwords;
  for (int gi = 0; gi < glo; ++gi) {
    uint32_t w[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) w[u] = kw[gi * KB + u];
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      const int j = gi * 32 + rr;
      const float c = s_kc[group_field<KB>(w, rr)];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) al[r] = fmaf(s_q[r * D + j], c, al[r]);
    }
  }
  const uint32_t* kh = kw + glo * KB;
  for (int gi = glo; gi < D / 32; ++gi) {
    uint32_t w[KH];
#pragma unroll
    for (int u = 0; u < KH; ++u) w[u] = kh[(gi - glo) * KH + u];
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      const int j = gi * 32 + rr;
      const float c = s_kc2[group_field<KH>(w, rr)];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) ah[r] = fmaf(s_q[r * D + j], c, ah[r]);
    }
  }
  const float nl = p.k_norm[slot], nh = p.k_norm_hi[slot];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) s[r] = fmaf(nl, al[r], nh * ah[r]);
}

template <int D, int RMAX>
__device__ __forceinline__ void score_dispatch(const DecodeParams& p, int64_t slot, const float* s_q,
                                               const float* s_qs, const float* s_kc, float (&s)[RMAX]) {
  const bool prod = p.kmode == TQ_MODE_PROD;
  switch (p.kbits * 2 + (prod ? 1 : 0)) {
    case 2: score_token<D, RMAX, 1, false>(p, slot, s_q, s_qs, s_kc, s); break;
    case 3: score_token<D, RMAX, 1, true>(p, slot, s_q, s_qs, s_kc, s); break;
    case 4: score_token<D, RMAX, 2, false>(p, slot, s_q, s_qs, s_kc, s); break;
    case 5: score_token<D, RMAX, 2, true>(p, slot, s_q, s_qs, s_kc, s); break;
    case 6: score_token<D, RMAX, 3, false>(p, slot, s_q, s_qs, s_kc, s); break;
    case 7: score_token<D, RMAX, 3, true>(p, slot, s_q, s_qs, s_kc, s); break;
    case 8: score_token<D, RMAX, 4, false>(p, slot, s_q, s_qs, s_kc, s); break;
    default: score_token<D, RMAX, 4, true>(p, slot, s_q, s_qs, s_kc, s); break;
  }
}

// Value of coordinate j of token t of the tile staged in LDS (MSE: c_v[idx];
// the norm is folded into the softmax weight.  Group: q s_g + mn_g).
template <int D, int VB, bool GROUP>
__device__ __forceinline__ float value_coord(const uint32_t* s_vw, const float* s_vs, int t, int j,
                                             const float* s_vc) {
  constexpr int VW = D * VB / 32;
  const uint32_t f = token_field<VB>(s_vw + t * VW, j);
  if constexpr (GROUP) {
    const int gi = t * (D / 32) + (j >> 5);
    return fmaf((float)f, s_vs[2 * gi], s_vs[2 * gi + 1]);
  } else {
    return s_vc[f];
  }
}

// Stage the value words (and group scales / minima) of the tile's tokens in
// LDS with coalesced loads, so that the per-coordinate loop reads LDS.
template <int D, int VB, bool GROUP>
__device__ __forceinline__ void stage_values(const DecodeParams& p, int64_t slot0, int cnt, uint32_t* s_vw,
                                             float* s_vs) {
  constexpr int VW = D * VB / 32;
  const uint32_t* src = p.v_idx + slot0 * VW;
  for (int e = threadIdx.x; e < cnt * VW; e += 256) s_vw[e] = src[e];
  if constexpr (GROUP) {
    constexpr int NG = D / 32;
    for (int e = threadIdx.x; e < cnt * NG; e += 256) {
      s_vs[2 * e] = p.v_scale[slot0 * NG + e];
      s_vs[2 * e + 1] = p.v_gmin[slot0 * NG + e];
    }
  }
}

template <int D, int RMAX, int VB, bool GROUP>
__device__ __forceinline__ void accumulate_values(const DecodeParams& p, int64_t slot0, int cnt, int j, int rg,
                                                  const float* s_p, const float* s_vc, float* o, uint32_t* s_vw,
                                                  float* s_vs) {
  constexpr int NRG = 256 / D;
  constexpr int RPT = (RMAX + NRG - 1) / NRG;
  stage_values<D, VB, GROUP>(p, slot0, cnt, s_vw, s_vs);
  __syncthreads();
  if (rg >= NRG) return;
  for (int t = 0; t < cnt; ++t) {
    const float cv = value_coord<D, VB, GROUP>(s_vw, s_vs, t, j, s_vc);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = rg + NRG * k;
      if (r < RMAX) o[k] = fmaf(s_p[t * (RMAX + 1) + r], cv, o[k]);
    }
  }
}

// Values of a split cache: coordinate j < d_lo reads the low part's VB-bit
// codes (words 0 .. wlo-1 of the record), the rest the high part's VB+1-bit
// codes; each part's norm multiplies its own coordinates (the softmax weights
// in s_p carry no value norm for split values).
template <int D, int RMAX, int VB>
__device__ __forceinline__ void accumulate_values_split(const DecodeParams& p, int64_t slot0, int cnt, int j, int rg,
                                                        const float* s_p, const float* s_vc, const float* s_vc2,
                                                        const float* s_nv, const float* s_nv2, float* o,
                                                        uint32_t* s_vw) {
  constexpr int NRG = 256 / D;
  constexpr int RPT = (RMAX + NRG - 1) / NRG;
  const int vw = p.vwords, dlo = 32 * p.vsplit_g, wlo = p.vsplit_g * VB;
  const uint32_t* src = p.v_idx + slot0 * vw;
  for (int e = threadIdx.x; e < cnt * vw; e += 256) s_vw[e] = src[e];
  __syncthreads();
  if (rg >= NRG) return;
  const bool low = j < dlo;
  for (int t = 0; t < cnt; ++t) {
    const uint32_t* tw = s_vw + t * vw;
    const float cv = low ? s_vc[token_field<VB>(tw, j)] * s_nv[t]
                         : s_vc2[token_field<VB + 1>(tw + wlo, j - dlo)] * s_nv2[t];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = rg + NRG * k;
      if (r < RMAX) o[k] = fmaf(s_p[t * (RMAX + 1) + r], cv, o[k]);
    }
  }
}

template <int D, int RMAX>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int NRG = 256 / D;
  constexpr int RPT = (RMAX + NRG - 1) / NRG;
  __shared__ float s_q[RMAX * D];
  __shared__ float s_qs[RMAX * D];
  __shared__ float s_p[kTile * (RMAX + 1)];
  __shared__ float s_nv[kTile];
  __shared__ float s_nv2[kTile];                 // split values: the high part's norms
  __shared__ float s_m[RMAX], s_l[RMAX], s_alpha[RMAX];
  __shared__ float s_kc[16], s_vc[16];
  __shared__ float s_kc2[16], s_vc2[16];         // split codecs: the high parts' centroids
  __shared__ uint32_t s_vw[kTile * D * 4 / 32];  // the tile's value words (up to 4 bits)
  __shared__ float s_vs[kTile * (D / 32) * 2];   // group scale and minimum pairs

  const int chunk_id = rotated_chunk(blockIdx.x, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g;
  const int tid = threadIdx.x;
  const bool prod = p.kmode == TQ_MODE_PROD;
  const bool vgroup = p.vmode == TQ_MODE_GROUP;
  const bool ksplit = p.ksplit_g > 0, vsplit = p.vsplit_g > 0;
  int64_t len = p.len[b];
  len = len < 0 ? 0 : (len > p.cap ? p.cap : len);
  // the causal rule's length (a hybrid cache's whole length; else len)
  const int64_t lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : (int64_t)p.len_mask[b]) : len;
  const int64_t c0 = (int64_t)chunk_id * p.chunk;
  const int64_t c1 = c0 + p.chunk < len ? c0 + p.chunk : len;
  const int rows = p.rows;

  for (int e = tid; e < RMAX * D; e += 256) {
    s_q[e] = e < rows * D ? p.qrot[(size_t)bg * rows * D + e] : 0.f;
    s_qs[e] = (prod && e < rows * D) ? p.qs[(size_t)bg * rows * D + e] : 0.f;
  }
  if (tid < 16) {
    s_kc[tid] = tid < (1 << p.kbits) ? p.k_cent[tid] : 0.f;
    s_vc[tid] = (!vgroup && tid < (1 << p.vbits)) ? p.v_cent[tid] : 0.f;
    s_kc2[tid] = (ksplit && tid < (2 << p.kbits)) ? p.k_cent_hi[tid] : 0.f;
    s_vc2[tid] = (vsplit && tid < (2 << p.vbits)) ? p.v_cent_hi[tid] : 0.f;
  }
  if (tid < RMAX) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float o[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) o[k] = 0.f;
  __syncthreads();

  const int64_t base = (int64_t)bg * p.cap;  // token-head slot of token 0 of (b, g)
  const float sl2 = p.scale * kLog2e;
  const int j = tid % D, rg = tid / D;
  for (int64_t t0 = c0; t0 < c1; t0 += kTile) {
    const int cnt = (int)((c1 - t0) < kTile ? (c1 - t0) : kTile);
    // phase A: one token per thread
    {
      const int64_t tok = t0 + tid;
      float s[RMAX];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) s[r] = 0.f;
      if (tid < cnt) {
        if (ksplit) {
          switch (p.kbits) {
            case 1: score_token_split<D, RMAX, 1>(p, base + tok, s_q, s_kc, s_kc2, s); break;
            case 2: score_token_split<D, RMAX, 2>(p, base + tok, s_q, s_kc, s_kc2, s); break;
            default: score_token_split<D, RMAX, 3>(p, base + tok, s_q, s_kc, s_kc2, s); break;
          }
        } else {
          score_dispatch<D, RMAX>(p, base + tok, s_q, s_qs, s_kc, s);
        }
        s_nv[tid] = vgroup ? 1.f : p.v_norm[base + tok];
        if (vsplit) s_nv2[tid] = p.v_norm_hi[base + tok];
      }
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const bool vis = tid < cnt && r < rows && tok < lenm - p.q_len + ((p.row0 + r) % p.q_len) + 1;
        s_p[tid * (RMAX + 1) + r] = vis ? s[r] * sl2 : -INFINITY;
      }
    }
    __syncthreads();
    // phase B: online softmax, wave w owns rows w, w+4, ...
    {
      const int wave = tid >> 6, lane = tid & 63;
      for (int r = wave; r < rows; r += 4) {
        float mx = -INFINITY;
        for (int k = lane; k < cnt; k += 64) mx = fmaxf(mx, s_p[k * (RMAX + 1) + r]);
        mx = wave_max(mx);
        const float m_old = s_m[r];
        const float m_new = fmaxf(m_old, mx);
        float sum = 0.f;
        for (int k = lane; k < cnt; k += 64) {
          const float sv = s_p[k * (RMAX + 1) + r];
          const float pr = m_new == -INFINITY ? 0.f : exp2f(sv - m_new);
          sum += pr;
          s_p[k * (RMAX + 1) + r] = vsplit ? pr : pr * s_nv[k];
        }
        sum = wave_sum(sum);
        if (lane == 0) {
          const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_old - m_new);
          s_alpha[r] = alpha;
          s_m[r] = m_new;
          s_l[r] = s_l[r] * alpha + sum;
        }
      }
    }
    __syncthreads();
    // phase C: values, one coordinate per thread
    {
      if (rg < NRG) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          const int r = rg + NRG * k;
          if (r < rows) o[k] *= s_alpha[r];
        }
      }
      const int64_t slot0 = base + t0;
      if (vsplit) {
        switch (p.vbits) {
          case 1: accumulate_values_split<D, RMAX, 1>(p, slot0, cnt, j, rg, s_p, s_vc, s_vc2, s_nv, s_nv2, o, s_vw); break;
          case 2: accumulate_values_split<D, RMAX, 2>(p, slot0, cnt, j, rg, s_p, s_vc, s_vc2, s_nv, s_nv2, o, s_vw); break;
          default: accumulate_values_split<D, RMAX, 3>(p, slot0, cnt, j, rg, s_p, s_vc, s_vc2, s_nv, s_nv2, o, s_vw); break;
        }
      } else
      switch (p.vbits * 2 + (vgroup ? 1 : 0)) {
        case 2: accumulate_values<D, RMAX, 1, false>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 3: accumulate_values<D, RMAX, 1, true>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 4: accumulate_values<D, RMAX, 2, false>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 5: accumulate_values<D, RMAX, 2, true>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 6: accumulate_values<D, RMAX, 3, false>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 7: accumulate_values<D, RMAX, 3, true>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        case 8: accumulate_values<D, RMAX, 4, false>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
        default: accumulate_values<D, RMAX, 4, true>(p, slot0, cnt, j, rg, s_p, s_vc, o, s_vw, s_vs); break;
      }
    }
    __syncthreads();
  }

  // partial (m, l, o) of this chunk
  float* po = p.part_o + ((size_t)bg * p.n_chunks + chunk_id) * rows * D;
  float* pml = p.part_ml + ((size_t)bg * p.n_chunks + chunk_id) * rows * 2;
  if (rg < NRG) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = rg + NRG * k;
      if (r < rows) po[r * D + j] = o[k];
    }
  }
  if (tid < rows) {
    pml[2 * tid] = s_m[tid];
    pml[2 * tid + 1] = s_l[tid];
  }
}

// Cross-chunk merge, one workgroup of 4 D threads per (query row, KV head,
// sequence), stream-ordered after the decode kernel: weights 2^(m_c - M) / L
// from every chunk's (m, l), the merged row o = sum_c w_c o_c, then the
// single inverse rotation out = Pi_v^T o for MSE values (group values are
// already in the original domain).  Thread (j, k) takes coordinate j of the
// chunks c = k (mod 4), sixteen at a time, and the quarter k of the rotation's
// terms, whose loads it issues first; the quarters meet in LDS.
template <int D>
__global__ __launch_bounds__(4 * D) void merge_kernel(DecodeParams p) {
  constexpr int NT = 4 * D, NW = NT / 64, Q = D / 4;
  static_assert(D % 16 == 0, "whole waves");
  __shared__ float s_o[D];
  __shared__ float s_part[4][D];
  __shared__ float s_red[2][NW];
  __shared__ float s_w[kMaxMergeChunks];
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid % D, k = tid / D;
  const int nch = p.n_chunks, rows = p.rows;
  const bool rotate = p.vmode != TQ_MODE_GROUP;
  const float* pml = p.part_ml + (size_t)bg * nch * rows * 2;
  const float* po = p.part_o + (size_t)bg * nch * rows * D;
  float pv[Q];
  if (rotate) {
#pragma unroll
    for (int t = 0; t < Q; ++t) pv[t] = p.v_pi[(size_t)(k * Q + t) * D + j];
  }
  float M = -INFINITY;
  for (int c = tid; c < nch; c += NT) M = fmaxf(M, pml[((size_t)c * rows + r) * 2]);
  M = wave_max(M);
  if (lane == 0) s_red[0][wave] = M;
  __syncthreads();
  M = s_red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[0][w]);
  float L = 0.f;
  for (int c = tid; c < nch; c += NT) {
    const float mc = pml[((size_t)c * rows + r) * 2];
    const float w = (M == -INFINITY || mc == -INFINITY) ? 0.f : exp2f(mc - M);
    s_w[c] = w;
    L = fmaf(w, pml[((size_t)c * rows + r) * 2 + 1], L);
  }
  L = wave_sum(L);
  if (lane == 0) s_red[1][wave] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += s_red[1][w];
  float o = 0.f;
  int c = k;
  for (; c + 4 * 15 < nch; c += 4 * 16) {  // sixteen loads in flight per thread
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = po[((size_t)(c + 4 * t) * rows + r) * D + j];
#pragma unroll
    for (int t = 0; t < 16; ++t) o = fmaf(s_w[c + 4 * t], v[t], o);
  }
  for (; c < nch; c += 4) o = fmaf(s_w[c], po[((size_t)c * rows + r) * D + j], o);
  s_part[k][j] = o;
  __syncthreads();
  if (k == 0) {
    o = (s_part[0][j] + s_part[1][j]) + (s_part[2][j] + s_part[3][j]);
    s_o[j] = L > 0.f ? o / L : 0.f;
  }
  __syncthreads();
  const int R = p.row0 + r;
  const int h = g * p.group + R / p.q_len, qi = R % p.q_len;
  const int64_t orow = ((int64_t)b * p.hq + h) * p.q_len + qi;
  float* out = p.out + orow * D;
  if (p.row_ml && tid == 0) {  // the row's softmax reference and sum (log2 domain), for a later combine
    p.row_ml[2 * orow] = M;
    p.row_ml[2 * orow + 1] = L;
  }
  if (!rotate) {
    if (k == 0) out[j] = s_o[j];
    return;
  }
  float res = 0.f;
#pragma unroll
  for (int t = 0; t < Q; ++t) res = fmaf(s_o[k * Q + t], pv[t], res);
  s_part[k][j] = res;
  __syncthreads();
  if (k == 0) out[j] = (s_part[0][j] + s_part[1][j]) + (s_part[2][j] + s_part[3][j]);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  qprep_kernel<D><<<qprep_grid(p), dim3(4 * D), 0, stream>>>(p);
  const dim3 grid(p.n_chunks, p.hkv, p.batch);
  if (p.rows <= 4) {
    decode_kernel<D, 4><<<grid, dim3(256), 0, stream>>>(p);
  } else if (p.rows <= 8) {
    decode_kernel<D, 8><<<grid, dim3(256), 0, stream>>>(p);
  } else if constexpr (D <= 128) {
    decode_kernel<D, 16><<<grid, dim3(256), 0, stream>>>(p);
  } else {
    return hipErrorInvalidValue;  // more than 8 rows at head_dim > 128 is refused on the host
  }
  merge_kernel<D><<<dim3(p.rows, p.hkv, p.batch), dim3(4 * D), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qprep(const DecodeParams& p, hipStream_t stream) {
  switch (p.d) {
    case 128: qprep_kernel<128><<<qprep_grid(p), dim3(4 * 128), 0, stream>>>(p); break;
    case 256: qprep_kernel<256><<<qprep_grid(p), dim3(4 * 256), 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  if (p.n_chunks > kMaxMergeChunks) return hipErrorInvalidValue;
  switch (p.d) {
    case 128: merge_kernel<128><<<dim3(p.rows, p.hkv, p.batch), dim3(4 * 128), 0, stream>>>(p); break;
    case 256: merge_kernel<256><<<dim3(p.rows, p.hkv, p.batch), dim3(4 * 256), 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.n_chunks > kMaxMergeChunks || p.hkv > 65535 || p.batch > 65535 || p.rows > 16) return hipErrorInvalidValue;
  switch (p.d) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 96: return launch_d<96>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 160: return launch_d<160>(p, stream);
    case 192: return launch_d<192>(p, stream);
    case 224: return launch_d<224>(p, stream);
    case 256: return launch_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
