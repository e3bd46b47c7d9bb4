// Quantise-on-append for gfx950 ("omlx turboquant_kv.py", update_and_fetch:
// only the new tokens are quantised and written at the written end).
//
// One wave64 per head vector; lane l owns coordinates l, l+64, ...  Steps:
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
__global__ __launch_bounds__(256) void quantize_kernel(QuantizeParams p) {
  constexpr int NC = (D + 63) / 64;
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

}  // namespace

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t blocks = (total + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  switch (p.d) {
    case 32: quantize_kernel<32><<<grid, block, 0, stream>>>(p); break;
    case 64: quantize_kernel<64><<<grid, block, 0, stream>>>(p); break;
    case 96: quantize_kernel<96><<<grid, block, 0, stream>>>(p); break;
    case 128: quantize_kernel<128><<<grid, block, 0, stream>>>(p); break;
    case 160: quantize_kernel<160><<<grid, block, 0, stream>>>(p); break;
    case 192: quantize_kernel<192><<<grid, block, 0, stream>>>(p); break;
    case 224: quantize_kernel<224><<<grid, block, 0, stream>>>(p); break;
    case 256: quantize_kernel<256><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
