// Hybrid cache: a recent-token buffer in front of the compressed state.
//
// ("turboquant validate_moe_phase2.py", Test 5: caches built with
// buffer_size=128; its commit note: "hybrid decode".)  The most recent tokens
// of a sequence stay unquantised in a ring of B slots per (sequence, KV head);
// a sequence of N tokens holds tokens 0 .. Nc-1, Nc = floor(N / B) B, in the
// compressed cache and token t >= Nc in slot t - Nc of the ring.  A full ring
// is quantised into the compressed cache at once (by the append kernels, in
// their flush mode) and starts over.
//
//   hybrid_stage_kernel    copies a step's new tokens into the ring: first
//                          those of the block being filled, then -- after the
//                          flush -- those that start the next block;
//   hybrid_lens_kernel     Nc of every sequence, for the compressed decode;
//   hybrid_combine_kernel  exact attention of each query row over the ring's
//                          tokens, merged with the compressed decode's output
//                          through its softmax reference and sum.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float load_elem(const void* base, int64_t off, int bf16) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[off]) << 16);
  return static_cast<const float*>(base)[off];
}

// One workgroup of 64 threads per (new token, sequence x head, K or V).
__global__ __launch_bounds__(64) void hybrid_stage_kernel(HybridStage s) {
  const int set = blockIdx.y;
  const int64_t vec = blockIdx.x;
  const int i = (int)(vec % s.n_new);
  const int64_t bh = vec / s.n_new;
  const int h = (int)(bh % s.heads), b = (int)(bh / s.heads);
  const int64_t n = s.len[b] < 0 ? 0 : s.len[b];
  const int64_t pos = n + i, end = (n / s.block) * s.block + s.block;  // end of the block being filled
  if ((s.phase == 0) != (pos < end)) return;
  const int64_t slot = pos % s.block;
  const int64_t src = (int64_t)b * s.xs[set][0] + (int64_t)h * s.xs[set][1] + (int64_t)i * s.xs[set][2];
  const int64_t dst = (((int64_t)b * s.heads + h) * s.block + slot) * s.d;
  if (s.bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(s.x[set]) + src;
    uint16_t* y = static_cast<uint16_t*>(s.buf[set]) + dst;
    for (int j = threadIdx.x; j < s.d; j += 64) y[j] = x[j];
  } else {
    const float* x = static_cast<const float*>(s.x[set]) + src;
    float* y = static_cast<float*>(s.buf[set]) + dst;
    for (int j = threadIdx.x; j < s.d; j += 64) y[j] = x[j];
  }
}

__global__ __launch_bounds__(256) void hybrid_lens_kernel(const int32_t* len, int32_t* lens_c, int batch, int block) {
  for (int b = threadIdx.x; b < batch; b += 256) {
    const int32_t n = len[b] < 0 ? 0 : len[b];
    lens_c[b] = (n / block) * block;
  }
}

constexpr int kTok = 16;  // ring tokens per round

// One workgroup of 256 threads per (KV head, sequence): the G * q_len query
// rows of the head against the ring's tokens, online softmax in the log2
// domain (as the compressed decode), then the merge with the compressed
// output: out = (O_c L_c 2^(M_c - M) + o_b 2^(m_b - M)) / (L_c 2^(M_c - M) +
// l_b 2^(m_b - M)), M = max(M_c, m_b).
template <int D>
__global__ __launch_bounds__(256) void hybrid_combine_kernel(HybridAttn a) {
  constexpr int NRG = 256 / D;                 // row groups (thread j % D owns coordinate j)
  constexpr int RPT = (16 + NRG - 1) / NRG;    // rows per thread
  __shared__ float s_q[16][D + 1];
  __shared__ float s_k[kTok][D + 1];
  __shared__ float s_v[kTok][D];
  __shared__ float s_s[16][kTok];
  __shared__ float s_m[16], s_l[16], s_alpha[16];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int rows = a.group * a.q_len;
  const int64_t n = a.len[b] < 0 ? 0 : a.len[b];
  const int64_t nc = (n / a.block) * a.block;
  const int nb = (int)(n - nc);
  const float sl2 = a.scale * kLog2e;
  for (int e = tid; e < rows * D; e += 256) {
    const int r = e / D, j = e % D;
    const int h = g * a.group + r / a.q_len, qi = r % a.q_len;
    s_q[r][j] = load_elem(a.q, (((int64_t)b * a.hq + h) * a.q_len + qi) * D + j, a.q_bf16) * sl2;
  }
  if (tid < 16) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  const int j = tid % D, rg = tid / D;
  float o[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) o[k] = 0.f;
  const int64_t ring = ((int64_t)b * a.hkv + g) * a.block * D;
  __syncthreads();
  for (int t0 = 0; t0 < nb; t0 += kTok) {
    const int cnt = nb - t0 < kTok ? nb - t0 : kTok;
    for (int e = tid; e < cnt * D; e += 256) {
      const int i = e / D, jj = e % D;
      s_k[i][jj] = load_elem(a.kbuf, ring + (int64_t)(t0 + i) * D + jj, a.buf_bf16);
      s_v[i][jj] = load_elem(a.vbuf, ring + (int64_t)(t0 + i) * D + jj, a.buf_bf16);
    }
    __syncthreads();
    {
      const int r = tid / kTok, i = tid % kTok;
      if (r < rows) {
        // token nc + t0 + i is seen by row r when it is at most n - q_len + r % q_len
        const bool vis = i < cnt && nc + t0 + i <= n - a.q_len + r % a.q_len;
        float dot = 0.f;
        if (vis)
          for (int jj = 0; jj < D; ++jj) dot = fmaf(s_q[r][jj], s_k[i][jj], dot);
        s_s[r][i] = vis ? dot : -INFINITY;
      }
    }
    __syncthreads();
    if (tid < rows) {
      const int r = tid;
      float mx = -INFINITY;
      for (int i = 0; i < cnt; ++i) mx = fmaxf(mx, s_s[r][i]);
      const float m_old = s_m[r], m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int i = 0; i < cnt; ++i) {
        const float pr = m_new == -INFINITY ? 0.f : exp2f(s_s[r][i] - m_new);
        s_s[r][i] = pr;
        sum += pr;
      }
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_old - m_new);
      s_alpha[r] = alpha;
      s_m[r] = m_new;
      s_l[r] = s_l[r] * alpha + sum;
    }
    __syncthreads();
    if (rg < NRG) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int r = rg + NRG * k;
        if (r < rows) {
          float acc = o[k] * s_alpha[r];
          for (int i = 0; i < cnt; ++i) acc = fmaf(s_s[r][i], s_v[i][j], acc);
          o[k] = acc;
        }
      }
    }
    __syncthreads();
  }
  if (rg >= NRG) return;
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int r = rg + NRG * k;
    if (r >= rows) continue;
    const int h = g * a.group + r / a.q_len, qi = r % a.q_len;
    const int64_t orow = ((int64_t)b * a.hq + h) * a.q_len + qi;
    float mc = -INFINITY, lc = 0.f, oc = 0.f;
    if (a.has_compressed) {
      mc = a.row_ml[2 * orow];
      lc = a.row_ml[2 * orow + 1];
      oc = a.out[orow * D + j];
    }
    const float mb = s_m[r], lb = s_l[r];
    const float mm = fmaxf(mc, mb);
    const float wc = lc > 0.f ? lc * exp2f(mc - mm) : 0.f;
    const float wb = lb > 0.f ? exp2f(mb - mm) : 0.f;
    const float den = wc + lb * wb;
    a.out[orow * D + j] = den > 0.f ? (oc * wc + o[k] * wb) / den : 0.f;
  }
}

}  // namespace

hipError_t launch_hybrid_stage(const HybridStage& s, hipStream_t stream) {
  const int64_t vecs = (int64_t)s.batch * s.heads * s.n_new;
  if (vecs <= 0) return hipSuccess;
  if (vecs > 0x7fffffff || s.n_sets < 1 || s.n_sets > 2) return hipErrorInvalidValue;
  hybrid_stage_kernel<<<dim3((unsigned)vecs, (unsigned)s.n_sets), dim3(64), 0, stream>>>(s);
  return hipGetLastError();
}

hipError_t launch_hybrid_lens(const int32_t* len, int32_t* lens_c, int batch, int block, hipStream_t stream) {
  hybrid_lens_kernel<<<dim3(1), dim3(256), 0, stream>>>(len, lens_c, batch, block);
  return hipGetLastError();
}

hipError_t launch_hybrid_combine(const HybridAttn& a, hipStream_t stream) {
  if (a.group * a.q_len > 16 || a.hkv > 65535 || a.batch > 65535) return hipErrorInvalidValue;
  const dim3 grid(a.hkv, a.batch), block(256);
  switch (a.d) {
    case 32: hybrid_combine_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: hybrid_combine_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 96: hybrid_combine_kernel<96><<<grid, block, 0, stream>>>(a); break;
    case 128: hybrid_combine_kernel<128><<<grid, block, 0, stream>>>(a); break;
    case 160: hybrid_combine_kernel<160><<<grid, block, 0, stream>>>(a); break;
    case 192: hybrid_combine_kernel<192><<<grid, block, 0, stream>>>(a); break;
    case 224: hybrid_combine_kernel<224><<<grid, block, 0, stream>>>(a); break;
    case 256: hybrid_combine_kernel<256><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
