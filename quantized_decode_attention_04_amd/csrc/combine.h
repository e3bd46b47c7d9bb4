// Cross-chunk merge of split-K partials, shared by the decode kernels.
//
// Each chunk of the token axis leaves, per query row r, its running maximum
// m_c (log2 domain), its softmax denominator l_c and its unnormalised output
// o_c (rotated domain for MSE values).  The merged row is
//     M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  O = sum_c o_c 2^(m_c - M) / L,
// and MSE values are rotated back once: out = Pi_v^T O.  Rows that saw no
// token (M = -inf) are written as zeros.
#pragma once

#include "tq_internal.h"

namespace tq {

// Called by every thread of the last-arriving workgroup of (b, g); s_o is LDS
// scratch of rows*d floats.
__device__ inline void merge_chunks(const DecodeParams& p, int b, int g, float* s_o) {
  const int rows = p.rows, D = p.d;
  const int bg = b * p.hkv + g;
  const float* pml0 = p.part_ml + (size_t)bg * p.n_chunks * rows * 2;
  const float* po0 = p.part_o + (size_t)bg * p.n_chunks * rows * D;
  for (int e = threadIdx.x; e < rows * D; e += blockDim.x) {
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
  const bool vgroup = p.vmode == TQ_MODE_GROUP;
  for (int e = threadIdx.x; e < rows * D; e += blockDim.x) {
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
}

// Publish this workgroup's partial and, if it is the last of (b, g) to
// arrive, merge all chunks.  Every thread must call it after writing its
// share of the partial.
__device__ inline void arrive_and_merge(const DecodeParams& p, int b, int g, float* s_o, int* s_last) {
  const int bg = b * p.hkv + g;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *s_last = atomicAdd(p.counters + bg, 1u) == (unsigned)(p.n_chunks - 1);
  __syncthreads();
  if (!*s_last) return;
  __threadfence();
  merge_chunks(p, b, g, s_o);
  if (threadIdx.x == 0) p.counters[bg] = 0u;
}

}  // namespace tq
