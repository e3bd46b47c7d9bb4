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
//   qprep_kernel   one workgroup per (b, g): q_rot = Pi_k q (and S q_rot),
//                  and clears the (b, g) arrival counter;
//   decode_kernel  one workgroup per (chunk, g, b): tiles of 256 tokens;
//                  phase A scores one token per thread against the rotated
//                  queries in LDS (centroid look-up table in LDS), phase B
//                  runs the online softmax per row, phase C accumulates the
//                  values with one thread per coordinate; the partial
//                  (m, l, o) of the chunk goes to the workspace; the last
//                  workgroup of (b, g) to arrive merges all chunks and applies
//                  the single inverse rotation Pi_v^T.
// Scores are kept in the log2 domain (multiplied by log2 e) so that the
// softmax uses exp2.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kTile = 256;
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

template <int D>
__global__ __launch_bounds__(256) void qprep_kernel(DecodeParams p) {
  __shared__ float s_qr[2048];
  const int bg = blockIdx.x;
  const int b = bg / p.hkv, g = bg % p.hkv;
  if (threadIdx.x == 0) p.counters[bg] = 0u;
  const int n = p.rows * D;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int r = e / D, i = e % D;
    const int h = g * p.group + r / p.q_len, qi = r % p.q_len;
    const int64_t qoff = (((int64_t)b * p.hq + h) * p.q_len + qi) * D;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = fmaf(p.k_pit[(size_t)j * D + i], load_q(p.q, qoff + j, p.q_bf16), acc);
    s_qr[e] = acc;
    p.qrot[(size_t)bg * n + e] = acc;
  }
  if (p.kmode != TQ_MODE_PROD) return;
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += 256) {
    const int r = e / D, i = e % D;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = fmaf(p.k_st[(size_t)j * D + i], s_qr[r * D + j], acc);
    p.qs[(size_t)bg * n + e] = acc;
  }
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

// Value of coordinate j of one token (MSE: c_v[idx]; the norm is folded into
// the softmax weight.  Group: q s_g + mn_g).
template <int VB, bool GROUP>
__device__ __forceinline__ float value_coord(const DecodeParams& p, int64_t slot, int j, const float* s_vc) {
  const uint32_t f = token_field<VB>(p.v_idx + slot * (int64_t)p.vwords, j);
  if constexpr (GROUP) {
    const int64_t gidx = slot * p.vgroups + (j >> 5);
    return fmaf((float)f, p.v_scale[gidx], p.v_gmin[gidx]);
  } else {
    return s_vc[f];
  }
}

template <int D, int RMAX, int VB, bool GROUP>
__device__ __forceinline__ void accumulate_values(const DecodeParams& p, int64_t slot0, int cnt, int j, int rg,
                                                  const float* s_p, const float* s_vc, float* o) {
  constexpr int NRG = 256 / D;
  constexpr int RPT = (RMAX + NRG - 1) / NRG;
  for (int t = 0; t < cnt; ++t) {
    const float cv = value_coord<VB, GROUP>(p, slot0 + t, j, s_vc);
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
  __shared__ float s_m[RMAX], s_l[RMAX], s_alpha[RMAX];
  __shared__ float s_kc[16], s_vc[16];
  __shared__ int s_last;

  const int chunk_id = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g;
  const int tid = threadIdx.x;
  const bool prod = p.kmode == TQ_MODE_PROD;
  const bool vgroup = p.vmode == TQ_MODE_GROUP;
  int64_t len = p.len[b];
  len = len < 0 ? 0 : (len > p.cap ? p.cap : len);
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
        score_dispatch<D, RMAX>(p, base + tok, s_q, s_qs, s_kc, s);
        s_nv[tid] = vgroup ? 1.f : p.v_norm[base + tok];
      }
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const bool vis = tid < cnt && r < rows && tok < len - p.q_len + (r % p.q_len) + 1;
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
          s_p[k * (RMAX + 1) + r] = pr * s_nv[k];
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
    if (rg < NRG) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int r = rg + NRG * k;
        if (r < rows) o[k] *= s_alpha[r];
      }
      const int64_t slot0 = base + t0;
      switch (p.vbits * 2 + (vgroup ? 1 : 0)) {
        case 2: accumulate_values<D, RMAX, 1, false>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 3: accumulate_values<D, RMAX, 1, true>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 4: accumulate_values<D, RMAX, 2, false>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 5: accumulate_values<D, RMAX, 2, true>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 6: accumulate_values<D, RMAX, 3, false>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 7: accumulate_values<D, RMAX, 3, true>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        case 8: accumulate_values<D, RMAX, 4, false>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
        default: accumulate_values<D, RMAX, 4, true>(p, slot0, cnt, j, rg, s_p, s_vc, o); break;
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
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(p.counters + bg, 1u) == (unsigned)(p.n_chunks - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // last workgroup of (b, g): merge the chunks, then one inverse rotation
  float* s_o = s_p;
  const float* pml0 = p.part_ml + (size_t)bg * p.n_chunks * rows * 2;
  const float* po0 = p.part_o + (size_t)bg * p.n_chunks * rows * D;
  for (int e = tid; e < rows * D; e += 256) {
    const int r = e / D;
    float M = -INFINITY;
    for (int c = 0; c < p.n_chunks; ++c) M = fmaxf(M, pml0[(size_t)c * rows * 2 + 2 * r]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int c = 0; c < p.n_chunks; ++c) {
        const float mc = pml0[(size_t)c * rows * 2 + 2 * r];
        const float w = mc == -INFINITY ? 0.f : exp2f(mc - M);
        L = fmaf(w, pml0[(size_t)c * rows * 2 + 2 * r + 1], L);
        acc = fmaf(w, po0[(size_t)c * rows * D + e], acc);
      }
    }
    s_o[e] = L > 0.f ? acc / L : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < rows * D; e += 256) {
    const int r = e / D, jj = e % D;
    float res;
    if (vgroup) {
      res = s_o[e];
    } else {
      res = 0.f;
      for (int i = 0; i < D; ++i) res = fmaf(p.v_pi[(size_t)i * D + jj], s_o[r * D + i], res);
    }
    const int h = g * p.group + r / p.q_len, qi = r % p.q_len;
    p.out[(((int64_t)b * p.hq + h) * p.q_len + qi) * D + jj] = res;
  }
  if (tid == 0) p.counters[bg] = 0u;
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  qprep_kernel<D><<<dim3(p.batch * p.hkv), dim3(256), 0, stream>>>(p);
  const dim3 grid(p.n_chunks, p.hkv, p.batch);
  if (p.rows <= 4) {
    decode_kernel<D, 4><<<grid, dim3(256), 0, stream>>>(p);
  } else if constexpr (D <= 128) {
    decode_kernel<D, 16><<<grid, dim3(256), 0, stream>>>(p);
  } else {
    decode_kernel<D, 8><<<grid, dim3(256), 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.n_chunks > 65535 || p.hkv > 65535 || p.batch > 65535) return hipErrorInvalidValue;
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
