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
//                          tokens (one workgroup per row), merged with the
//                          compressed decode's output through its softmax
//                          reference and sum.
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

constexpr int kThreads = 256;  // combine workgroup
constexpr int kRound = 64;     // ring tokens per round (four threads score one)

// Coordinates j .. j+7 of a ring row as floats (16-byte reads of bf16, two of
// float32; rows of D >= 32 coordinates stay 16-byte aligned).
__device__ __forceinline__ void load8(const void* base, int64_t off, int bf16, float* x) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 c = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
  }
}

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* s_red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // s_red's previous use is over
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  v = s_red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) v = is_max ? fmaxf(v, s_red[w]) : v + s_red[w];
  return v;
}

// One workgroup of 256 threads per (query row, KV head, sequence): the row
// against the ring's tokens with an online softmax in the log2 domain (the
// compressed decode's), 64 tokens per round -- four threads score a token,
// each over a quarter of the coordinates, while the round's value rows are
// staged in LDS with 16-byte reads; thread j < D accumulates coordinate j --
// then the merge with the compressed output: out = (O_c L_c 2^(M_c - M) +
// o_b 2^(m_b - M)) / (L_c 2^(M_c - M) + l_b 2^(m_b - M)), M = max(M_c, m_b).
template <int D>
__global__ __launch_bounds__(kThreads) void hybrid_combine_kernel(HybridAttn a) {
  constexpr int Q4 = D / 4;  // coordinates per scoring thread (a multiple of 8)
  __shared__ float s_q[D];
  __shared__ float s_p[kRound];
  __shared__ float s_red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) float s_v[kRound][D];
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int h = g * a.group + r / a.q_len, qi = r % a.q_len;
  const int64_t orow = ((int64_t)b * a.hq + h) * a.q_len + qi;
  const int64_t n = a.len[b] < 0 ? 0 : a.len[b];
  const int64_t nc = (n / a.block) * a.block;
  const int nb = (int)(n - nc);
  const int64_t vis = n - a.q_len + qi + 1 - nc;  // ring tokens 0 .. vis-1 are seen by the row
  const float sl2 = a.scale * kLog2e;
  for (int j = tid; j < D; j += kThreads) s_q[j] = load_elem(a.q, orow * D + j, a.q_bf16) * sl2;
  const int64_t ring = ((int64_t)b * a.hkv + g) * a.block * D;
  const int tt = tid >> 2, part = tid & 3;  // scoring: token tt of the round, coordinates part * Q4 ..
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  __syncthreads();
  for (int t0 = 0; t0 < nb; t0 += kRound) {
    const int cnt = nb - t0 < kRound ? nb - t0 : kRound;
    // the round's value rows into LDS (as float), eight coordinates a read
    for (int e = tid; e < cnt * (D / 8); e += kThreads) {
      const int i = e / (D / 8), j0 = 8 * (e % (D / 8));
      float x[8];
      load8(a.vbuf, ring + (int64_t)(t0 + i) * D + j0, a.buf_bf16, x);
      *reinterpret_cast<float4*>(&s_v[i][j0]) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(&s_v[i][j0 + 4]) = make_float4(x[4], x[5], x[6], x[7]);
    }
    float dot = 0.f;
    const bool seen = tt < cnt && t0 + tt < vis;
    if (seen) {
      float x[Q4];
#pragma unroll
      for (int j0 = 0; j0 < Q4; j0 += 8) load8(a.kbuf, ring + (int64_t)(t0 + tt) * D + part * Q4 + j0, a.buf_bf16, x + j0);
#pragma unroll
      for (int j = 0; j < Q4; ++j) dot = fmaf(s_q[part * Q4 + j], x[j], dot);
    }
    dot += __shfl_xor(dot, 1, 64);
    dot += __shfl_xor(dot, 2, 64);
    const float sc = seen ? dot : -INFINITY;
    const float mx = block_reduce(sc, true, s_red);
    const float m_new = fmaxf(m_run, mx);
    const float pr = (m_new == -INFINITY || sc == -INFINITY) ? 0.f : exp2f(sc - m_new);
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    if (part == 0 && tt < kRound) s_p[tt] = pr;
    // each token's probability counted once (the four scoring threads agree)
    const float sum = block_reduce(part == 0 ? pr : 0.f, false, s_red);  // (its barriers publish s_p, s_v)
    l_run = l_run * alpha + sum;
    m_run = m_new;
    if (tid < D) {
      float acc = o * alpha;
      for (int i = 0; i < cnt; ++i) acc = fmaf(s_p[i], s_v[i][tid], acc);
      o = acc;
    }
    __syncthreads();  // s_p and s_v are rewritten by the next round
  }
  if (tid >= D) return;
  float mc = -INFINITY, lc = 0.f, oc = 0.f;
  if (a.has_compressed) {
    mc = a.row_ml[2 * orow];
    lc = a.row_ml[2 * orow + 1];
    oc = a.out[orow * D + tid];
  }
  const float mm = fmaxf(mc, m_run);
  const float wc = lc > 0.f ? lc * exp2f(mc - mm) : 0.f;
  const float wb = l_run > 0.f ? exp2f(m_run - mm) : 0.f;
  const float den = wc + l_run * wb;
  a.out[orow * D + tid] = den > 0.f ? (oc * wc + o * wb) / den : 0.f;
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
  const dim3 grid(a.group * a.q_len, a.hkv, a.batch), block(kThreads);
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
