// Quantise-on-append for gfx950 ("omlx turboquant_kv.py", update_and_fetch:
// only the new tokens are quantised and written at the written end).
//
// Bulk appends: one wave64 per head vector; lane l owns coordinates l, l+64,
// ...  Steps:
// load (bf16 or f32) -> wave-reduced norm -> y = Pi x with x broadcast from
// LDS and Pi^T read row by row (coalesced across lanes, L2-resident) ->
// nearest centroid by counting boundaries below u = y/n -> pack the indices
// into the word layout with LDS atomic OR -> vector stores.  Prod keys then
// form the rotated residual rho = y - n c[idx], its norm, z = S rho, and
// write sign(z) as 64-lane ballots.  Group values skip the rotation and
// quantise 32-coordinate groups (one half-wave each) by min/max.
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ float load_x(const void* x, int64_t off, int bf16) {
  if (bf16) {
    const uint16_t v = static_cast<const uint16_t*>(x)[off];
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  return static_cast<const float*>(x)[off];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// OR the b-bit field `v` of coordinate j into the word buffer (layout of the
// packed index stream: LSB-first for 1, 2, 4 bits; byte lanes for 3 bits).
__device__ __forceinline__ void pack_field(uint32_t* w, int j, int b, uint32_t v) {
  if (b == 3) {
    const int g = j >> 5, r = j & 31, a = r >> 2, k = r & 3;
    uint32_t* X = w + 3 * g;
    uint32_t* Y = X + 1;
    uint32_t* Z = X + 2;
    const int s = 8 * k;
    switch (a) {
      case 0: atomicOr(X, v << s); break;
      case 1: atomicOr(X, v << (s + 3)); break;
      case 2: atomicOr(X, (v & 3u) << (s + 6)); atomicOr(Z, (v >> 2) << (s + 6)); break;
      case 3: atomicOr(Y, v << s); break;
      case 4: atomicOr(Y, v << (s + 3)); break;
      case 5: atomicOr(Y, (v & 3u) << (s + 6)); atomicOr(Z, (v >> 2) << (s + 7)); break;
      case 6: atomicOr(Z, v << s); break;
      default: atomicOr(Z, v << (s + 3)); break;
    }
  } else {
    const int bit = j * b;
    atomicOr(w + (bit >> 5), v << (bit & 31));
  }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantizeSets sets) {
  constexpr int NC = (D + 63) / 64;
  const QuantizeParams& p = sets.s[blockIdx.y];
  __shared__ float xs[4][D];
  __shared__ uint32_t wbuf[4][32];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t vec = (int64_t)blockIdx.x * 4 + wave;

  bool active = vec < total;
  int b = 0, h = 0, t = 0;
  int64_t pos = 0;
  if (active) {
    t = (int)(vec % p.n_new);
    const int64_t bh = vec / p.n_new;
    h = (int)(bh % p.heads);
    b = (int)(bh / p.heads);
    pos = (int64_t)p.pos[b] + t;
    active = pos >= 0 && pos < p.cap;
  }
  const int64_t tok = ((int64_t)b * p.heads + h) * p.cap + pos;  // token-head slot in the cache

  float x[NC];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = lane + 64 * c;
    x[c] = (active && i < D) ? load_x(p.x, (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2 + i, p.x_bf16) : 0.f;
    ss += x[c] * x[c];
  }
  if (lane < 32) wbuf[wave][lane] = 0u;

  if (p.mode == TQ_MODE_GROUP) {
    // groups of 32 coordinates = half-waves; min/max stay inside a half-wave
    const int top = (1 << p.gbits) - 1;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = lane + 64 * c;
      const bool valid = i < D;
      float mn = valid ? x[c] : INFINITY;
      float mx = valid ? x[c] : -INFINITY;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      }
      const float rng = mx - mn;
      uint32_t q = 0;
      if (valid && rng > 0.f) {
        const float tq = (x[c] - mn) * (float)top / rng;
        q = (uint32_t)fminf(fmaxf(rintf(tq), 0.f), (float)top);
      }
      if (active && valid) {
        pack_field(wbuf[wave], i, p.gbits, q);
        if ((i & 31) == 0) {
          p.scale[tok * p.groups + (i >> 5)] = rng / (float)top;
          p.gmin[tok * p.groups + (i >> 5)] = mn;
        }
      }
    }
    __syncthreads();
    if (active && lane < p.words) p.idx[tok * p.words + lane] = wbuf[wave][lane];
    return;
  }

  const float n = sqrtf(wave_sum(ss));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = lane + 64 * c;
    if (i < D) xs[wave][i] = x[c];
  }
  __syncthreads();

  // y = Pi x, with Pi^T[j][i] = Pi[i][j] read along i (coalesced)
  float y[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) y[c] = 0.f;
  for (int j = 0; j < D; ++j) {
    const float xj = xs[wave][j];
    const float* row = p.pit + (size_t)j * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = lane + 64 * c;
      if (i < D) y[c] = fmaf(row[i], xj, y[c]);
    }
  }

  const float inv = n > 0.f ? 1.f / n : 0.f;
  uint32_t idx[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float u = y[c] * inv;
    uint32_t k = 0;
    for (int m = 0; m < p.levels - 1; ++m) k += u > p.bnd[m] ? 1u : 0u;
    idx[c] = k;
    const int i = lane + 64 * c;
    if (active && i < D) pack_field(wbuf[wave], i, p.mse_bits, k);
  }
  __syncthreads();
  if (active) {
    if (lane < p.words) p.idx[tok * p.words + lane] = wbuf[wave][lane];
    if (lane == 0) p.norm[tok] = n;
  }
  if (p.mode != TQ_MODE_PROD) return;

  // Prod: rotated residual, its norm, z = S rho, sign bits
  float rho[NC];
  float rs = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = lane + 64 * c;
    rho[c] = i < D ? y[c] - n * p.cent[idx[c]] : 0.f;
    rs += rho[c] * rho[c];
  }
  const float gamma = sqrtf(wave_sum(rs));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = lane + 64 * c;
    if (i < D) xs[wave][i] = rho[c];
  }
  __syncthreads();
  float z[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) z[c] = 0.f;
  for (int j = 0; j < D; ++j) {
    const float rj = xs[wave][j];
    const float* row = p.st + (size_t)j * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = lane + 64 * c;
      if (i < D) z[c] = fmaf(row[i], rj, z[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = lane + 64 * c;
    const uint64_t m = __ballot(i < D && z[c] >= 0.f);
    if (active) {
      if (lane == 0) p.sign[tok * p.sign_words + 2 * c] = (uint32_t)m;
      if (lane == 1 && 2 * c + 1 < p.sign_words) p.sign[tok * p.sign_words + 2 * c + 1] = (uint32_t)(m >> 32);
    }
  }
  if (active && lane == 0) p.rnorm[tok] = gamma;
}

// Small appends (a few tokens per sequence and head, the decode-step case):
// one 256-thread workgroup per vector, so that the rotation's loads are all
// in flight at once instead of one wave streaming Pi^T through L2 in many
// round trips.  Thread t owns coordinate i = t % D and the slice of the
// contraction j in [part*JN, (part+1)*JN), part = t / D; the rotation and
// sketch rows it needs are loaded before x arrives.  Every mode (group mode
// needs no rotation), head_dim 32, 64 and 128.
template <int D>
__global__ __launch_bounds__(256) void quantize_small_kernel(QuantizeSets sets) {
  constexpr int PARTS = 256 / D;
  constexpr int JN = D / PARTS;
  static_assert(PARTS * D == 256 && JN <= 64, "one to eight slices of at most 64 terms");
  const QuantizeParams& p = sets.s[blockIdx.y];
  __shared__ float xs[D];
  __shared__ float part_sum[PARTS][D];
  __shared__ uint32_t wbuf[32];
  __shared__ float red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = tid % D, part = tid / D, j0 = part * JN;
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t vec = blockIdx.x;
  if (vec >= total) return;  // whole workgroup
  const int t = (int)(vec % p.n_new);
  const int64_t bh = vec / p.n_new;
  const int h = (int)(bh % p.heads), b = (int)(bh / p.heads);
  const int64_t pos = (int64_t)p.pos[b] + t;
  if (pos < 0 || pos >= p.cap) return;  // whole workgroup: nothing is written for it
  const int64_t tok = ((int64_t)b * p.heads + h) * p.cap + pos;
  const bool prod = p.mode == TQ_MODE_PROD;

  if (p.mode == TQ_MODE_GROUP) {
    // unrotated 32-coordinate groups, one per half-wave (min/max stay inside it)
    const int top = (1 << p.gbits) - 1;
    if (tid < 32) wbuf[tid] = 0u;
    __syncthreads();
    if (tid < D) {
      const float xv = load_x(p.x, (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2 + tid, p.x_bf16);
      float mn = xv, mx = xv;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 64));
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      }
      const float rng = mx - mn;
      uint32_t q = 0;
      if (rng > 0.f) q = (uint32_t)fminf(fmaxf(rintf((xv - mn) * (float)top / rng), 0.f), (float)top);
      pack_field(wbuf, tid, p.gbits, q);
      if ((tid & 31) == 0) {
        p.scale[tok * p.groups + (tid >> 5)] = rng / (float)top;
        p.gmin[tok * p.groups + (tid >> 5)] = mn;
      }
    }
    __syncthreads();
    if (tid < p.words) p.idx[tok * p.words + tid] = wbuf[tid];
    return;
  }

  // rotation (and sketch) slices first, then x
  float pr[JN], sr[JN];
#pragma unroll
  for (int k = 0; k < JN; ++k) pr[k] = p.pit[(size_t)(j0 + k) * D + i];
  if (prod) {
#pragma unroll
    for (int k = 0; k < JN; ++k) sr[k] = p.st[(size_t)(j0 + k) * D + i];
  }
  float xv = 0.f;
  if (tid < D) xv = load_x(p.x, (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2 + tid, p.x_bf16);
  if (tid < 32) wbuf[tid] = 0u;
  if (tid < D) xs[tid] = xv;
  float sq = wave_sum(xv * xv);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  const float n = sqrtf(red[0] + red[1] + red[2] + red[3]);

  // y = Pi x
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < JN; ++k) acc = fmaf(pr[k], xs[j0 + k], acc);
  part_sum[part][i] = acc;
  __syncthreads();
  float y = 0.f;
  uint32_t idx = 0;
  if (tid < D) {
#pragma unroll
    for (int q = 0; q < PARTS; ++q) y += part_sum[q][tid];
    const float u = y * (n > 0.f ? 1.f / n : 0.f);
    for (int m = 0; m < p.levels - 1; ++m) idx += u > p.bnd[m] ? 1u : 0u;
    pack_field(wbuf, tid, p.mse_bits, idx);
  }
  __syncthreads();
  if (tid < p.words) p.idx[tok * p.words + tid] = wbuf[tid];
  if (tid == 0) p.norm[tok] = n;
  if (!prod) return;

  // Prod: rotated residual, its norm, z = S rho, sign bits
  const float rho = tid < D ? y - n * p.cent[idx] : 0.f;
  const float rs = wave_sum(rho * rho);
  __syncthreads();  // every read of xs, part_sum and red above is done
  if (tid < D) xs[tid] = rho;
  if (lane == 0) red[wave] = rs;
  __syncthreads();
  const float gamma = sqrtf(red[0] + red[1] + red[2] + red[3]);
  acc = 0.f;
#pragma unroll
  for (int k = 0; k < JN; ++k) acc = fmaf(sr[k], xs[j0 + k], acc);
  part_sum[part][i] = acc;
  __syncthreads();
  float z = 0.f;
  if (tid < D) {
#pragma unroll
    for (int q = 0; q < PARTS; ++q) z += part_sum[q][tid];
  }
  const uint64_t m = __ballot(tid < D && z >= 0.f);
  if (tid < D) {
    if (lane == 0) p.sign[tok * p.sign_words + 2 * wave] = (uint32_t)m;
    if (lane == 1 && 2 * wave + 1 < p.sign_words) p.sign[tok * p.sign_words + 2 * wave + 1] = (uint32_t)(m >> 32);
  }
  if (tid == 0) p.rnorm[tok] = gamma;
}

}  // namespace

hipError_t launch_quantize(const QuantizeSets& sets, int n_sets, hipStream_t stream) {
  if (n_sets < 1 || n_sets > 2) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int k = 0; k < n_sets; ++k) {
    const QuantizeParams& p = sets.s[k];
    if (p.d != sets.s[0].d) return hipErrorInvalidValue;
    const int64_t v = (int64_t)p.batch * p.heads * p.n_new;
    total = v > total ? v : total;
  }
  const int d = sets.s[0].d;
  // the choice depends only on the sizes, so a key and a value append made
  // together or one by one take the same kernel and write the same bits
  const bool small = total <= kSmallAppend && (d == 32 || d == 64 || d == 128);
  if (small) {
    const dim3 grid((unsigned)total, (unsigned)n_sets), block(256);
    switch (d) {
      case 32: quantize_small_kernel<32><<<grid, block, 0, stream>>>(sets); break;
      case 64: quantize_small_kernel<64><<<grid, block, 0, stream>>>(sets); break;
      default: quantize_small_kernel<128><<<grid, block, 0, stream>>>(sets); break;
    }
    return hipGetLastError();
  }
  const int64_t blocks = (total + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)n_sets), block(256);
  switch (d) {
    case 32: quantize_kernel<32><<<grid, block, 0, stream>>>(sets); break;
    case 64: quantize_kernel<64><<<grid, block, 0, stream>>>(sets); break;
    case 96: quantize_kernel<96><<<grid, block, 0, stream>>>(sets); break;
    case 128: quantize_kernel<128><<<grid, block, 0, stream>>>(sets); break;
    case 160: quantize_kernel<160><<<grid, block, 0, stream>>>(sets); break;
    case 192: quantize_kernel<192><<<grid, block, 0, stream>>>(sets); break;
    case 224: quantize_kernel<224><<<grid, block, 0, stream>>>(sets); break;
    case 256: quantize_kernel<256><<<grid, block, 0, stream>>>(sets); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
