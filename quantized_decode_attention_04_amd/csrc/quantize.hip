// Quantise-on-append for gfx950 ("omlx turboquant_kv.py", update_and_fetch:
// only the new tokens are quantised and written at the written end).
//
// For every head vector x: n = |x|, u = Pi x / n, the index of each rotated
// coordinate counts the codebook boundaries below it, and the indices are
// packed into the word layout; Prod keys add the rotated residual
// rho = Pi x - n c[idx], its norm and the signs of S rho; group values
// quantise 32-coordinate groups of the unrotated vector by their min and max.
//
// Two kernels, chosen by the size of the append only (so that keys and values
// appended together or one by one take the same kernel and write the same
// bits): bulk appends tile 64 vectors per workgroup and run the rotations on
// the fp32 matrix cores; small appends (the decode step) give each vector a
// whole workgroup so that its rotation's loads are all in flight at once.
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

__device__ __forceinline__ double wave_sum_d(double v) {
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

// Cache slot position of token t of sequence b (negative: not written).  A
// hybrid-cache flush writes the recent-token buffer's block only when this
// step's appends complete it.
__device__ __forceinline__ int64_t append_position(const QuantizeParams& p, int b, int t) {
  const int64_t base = p.pos[b];
  if (p.flush_block > 0) {
    const int64_t blk = p.flush_block, start = base < 0 ? -1 : (base / blk) * blk;
    return (start >= 0 && base - start + p.flush_new >= blk) ? start + t : -1;
  }
  return base + t;
}

// ---- bulk appends on the matrix cores --------------------------------------
//
// One 256-thread workgroup per tile of kMV = 64 vectors.  The tile is staged
// in LDS as fp32 rows; the rotation of every vector, Y = X Pi^T, runs on
// v_mfma_f32_16x16x4f32 (wave w computes the output columns 16c .. 16c+15,
// c = w, w+4, ...; four row tiles of 16 vectors each).  The contraction index
// is permuted so that each lane reads contiguous runs: in k-step s lane l
// supplies the term j = (l/16) (D/4) + s, i.e. A = X[v][j] from LDS and
// B = Pi[16c + l%16][j] from the row-major rotation.  Lane l then holds
// Y[16r + 4(l/16) + e][16c + l%16], e = 0..3, and quantises those elements in
// registers: u = y / n, the index counts the boundaries below u, and the
// index bytes go to LDS, from where one thread per (vector, word) packs the
// words.  Prod keys write the rotated residual rho = y - n c[idx] over the
// tile, take its norm per vector and run Z = rho S^T the same way for the
// sign bits.  Group values need no rotation: one thread per (vector, group)
// quantises from the tile.
constexpr int kMV = 64;

typedef float v4f_t __attribute__((ext_vector_type(4)));

template <int D>
struct __attribute__((aligned(16))) BulkLds {
  float xs[kMV][D + 4];   // x tile, then the rotated residual (Prod); +4 spreads rows over banks
  uint8_t codes[kMV][D];  // per-coordinate index, sign or group code
  float nrm[kMV];
  int64_t src[kMV];       // element offset of each vector's row in x, -1 past the end
  int64_t slot[kMV];      // cache slot, -1 when the vector is not written
};

// Word w of one vector from its per-coordinate codes (the packed layout:
// LSB-first for 1, 2, 4 bits; byte lanes X, Y, Z per 32 coordinates for 3).
__device__ __forceinline__ uint32_t pack_word(const uint8_t* codes, int w, int b) {
  if (b == 3) {
    const uint32_t* c = reinterpret_cast<const uint32_t*>(codes + 32 * (w / 3));
    switch (w % 3) {
      case 0: return c[0] | (c[1] << 3) | ((c[2] & 0x03030303u) << 6);
      case 1: return c[3] | (c[4] << 3) | ((c[5] & 0x03030303u) << 6);
      default:
        return c[6] | (c[7] << 3) | (((c[2] >> 2) & 0x01010101u) << 6) | (((c[5] >> 2) & 0x01010101u) << 7);
    }
  }
  const int per = 32 / b;
  const uint32_t* c = reinterpret_cast<const uint32_t*>(codes + per * w);
  uint32_t word = 0;
  for (int q = 0; q < per / 4; ++q) {
    const uint32_t cw = c[q];
#pragma unroll
    for (int k = 0; k < 4; ++k) word |= ((cw >> (8 * k)) & 0xffu) << (b * (4 * q + k));
  }
  return word;
}

// Y = A B^T for the tile (A = L.xs, B = `mat` row-major [D][D]); calls
// f(v, coord, y) for every element this lane holds.
template <int D, typename F>
__device__ __forceinline__ void tile_gemm(const BulkLds<D>& L, const float* __restrict__ mat, F&& f) {
  constexpr int KS = D / 4;  // contraction terms per lane
  constexpr int NCT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int cc = 0; cc < (NCT + 3) / 4; ++cc) {
    const int c = wave + 4 * cc;
    if (c >= NCT) break;
    v4f_t bq[KS / 4];
    const v4f_t* brow = reinterpret_cast<const v4f_t*>(mat + (size_t)(16 * c + r16) * D + g4 * KS);
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) bq[q] = brow[q];
    v4f_t acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v4f_t a = *reinterpret_cast<const v4f_t*>(&L.xs[16 * r + r16][g4 * KS + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bq[q][e], acc[r], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) f(cc, r, e, 16 * r + 4 * g4 + e, 16 * c + r16, acc[r][e]);
  }
}

// Same, in float64 on v_mfma_f64_16x16x4f64 (the fp32 operands widen
// exactly, so every product is exact and only the float64 accumulation
// rounds).  Used for the rotation of Prod keys, whose residual y - n c[idx] is
// a difference of nearly equal terms.  The operands sit in the lanes as for
// the fp32 instruction, but register e of lane l holds output row l/16 + 4e
// (measured on gfx950), not 4 (l/16) + e.
typedef double v4d_t __attribute__((ext_vector_type(4)));

template <int D, typename F>
__device__ __forceinline__ void tile_gemm_f64(const BulkLds<D>& L, const float* __restrict__ mat, F&& f) {
  constexpr int KS = D / 4;
  constexpr int NCT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int cc = 0; cc < (NCT + 3) / 4; ++cc) {
    const int c = wave + 4 * cc;
    if (c >= NCT) break;
    const v4f_t* brow = reinterpret_cast<const v4f_t*>(mat + (size_t)(16 * c + r16) * D + g4 * KS);
    v4d_t acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = v4d_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
    for (int q = 0; q < KS / 4; ++q) {
      const v4f_t bq = brow[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v4f_t a = *reinterpret_cast<const v4f_t*>(&L.xs[16 * r + r16][g4 * KS + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[r] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[e], (double)bq[e], acc[r], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) f(cc, r, e, 16 * r + g4 + 4 * e, 16 * c + r16, acc[r][e]);
  }
}

// The rotated modes after the norms: y = Pi x on the matrix cores, the
// nearest centroid of every element (NB = levels - 1 boundaries, unrolled),
// the packed indices and norms; for Prod keys the residual, its norm and the
// sign bits of z = S rho.
template <int D, int NB, bool PROD>
__device__ __forceinline__ void quantize_rotated(const QuantizeParams& p, BulkLds<D>& L) {
  constexpr int NCT = D / 16;
  constexpr int NCC = (NCT + 3) / 4;  // column tiles per wave
  constexpr bool prod = PROD;
  const int tid = threadIdx.x;
  float bnd[NB], cent[NB + 1];  // uniform: scalar registers
#pragma unroll
  for (int m = 0; m < NB; ++m) bnd[m] = p.bnd[m];
#pragma unroll
  for (int m = 0; m <= NB; ++m) cent[m] = PROD ? p.cent[m] : 0.f;
  float rho[NCC][4][4];
  if constexpr (PROD) {
    // float64 rotation: the residual keeps the accuracy of its own size
    tile_gemm_f64<D>(L, p.pi, [&](int cc, int r, int e, int v, int coord, double y) {
      const double n = (double)L.nrm[v];
      const double u = n > 0.0 ? y / n : 0.0;
      uint32_t k = 0;
      float c = cent[0];
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const bool above = u > (double)bnd[m];
        k += above ? 1u : 0u;
        c = above ? cent[m + 1] : c;
      }
      L.codes[v][coord] = (uint8_t)k;
      rho[cc][r][e] = (float)(y - n * (double)c);
    });
  } else {
    tile_gemm<D>(L, p.pi, [&](int cc, int r, int e, int v, int coord, float y) {
      const float n = L.nrm[v];
      const float inv = n > 0.f ? 1.f / n : 0.f;
      const float u = y * inv;
      // the boundaries are sorted: the last one below u names the centroid
      uint32_t k = 0;
#pragma unroll
      for (int m = 0; m < NB; ++m) k += u > bnd[m] ? 1u : 0u;
      L.codes[v][coord] = (uint8_t)k;
      rho[cc][r][e] = 0.f;
    });
  }
  __syncthreads();  // every read of the x tile and write of the codes is done
  for (int e = tid; e < kMV * p.words; e += 256) {
    const int v = e / p.words, w = e % p.words;
    const int64_t slot = L.slot[v];
    if (slot >= 0) p.idx[slot * p.idx_stride + w] = pack_word(L.codes[v], w, p.mse_bits);
  }
  if (tid < kMV && L.slot[tid] >= 0) p.norm[L.slot[tid]] = L.nrm[tid];
  if (!prod) return;

  // ---- Prod: the rotated residual over the tile, its norm, z = S rho
  {
    const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const int c = wave + 4 * cc;
      if (c >= NCT) break;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) L.xs[16 * r + g4 + 4 * e][16 * c + r16] = rho[cc][r][e];  // float64 layout
    }
  }
  __syncthreads();  // the residual is complete; the index packing has read the codes
  float gam = 0.f;
  {
    const int v = tid >> 2, part = tid & 3;
    double ss = 0.0;
    for (int j = part * (D / 4); j < (part + 1) * (D / 4); ++j) ss = fma((double)L.xs[v][j], (double)L.xs[v][j], ss);
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    gam = (float)sqrt(ss);
  }
  tile_gemm<D>(L, p.s, [&](int, int, int, int v, int coord, float z) { L.codes[v][coord] = z >= 0.f ? 1 : 0; });
  __syncthreads();
  for (int e = tid; e < kMV * p.sign_words; e += 256) {
    const int v = e / p.sign_words, w = e % p.sign_words;
    const int64_t slot = L.slot[v];
    if (slot >= 0) p.sign[slot * p.sign_words + w] = pack_word(L.codes[v], w, 1);
  }
  if ((tid & 3) == 0 && L.slot[tid >> 2] >= 0) p.rnorm[L.slot[tid >> 2]] = gam;
}

// two waves per SIMD where the registers allow it (head_dim up to 128)
template <int D>
__global__ __launch_bounds__(256, D <= 128 ? 2 : 1) void quantize_bulk_kernel(QuantizeSets sets) {
  const QuantizeParams& p = sets.s[blockIdx.y];
  __shared__ BulkLds<D> L;
  const int tid = threadIdx.x;
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t v0 = (int64_t)blockIdx.x * kMV;

  if (tid < kMV) {
    const int64_t vec = v0 + tid;
    int64_t src = -1, slot = -1;
    if (vec < total) {
      const int t = (int)(vec % p.n_new);
      const int64_t bh = vec / p.n_new;
      const int h = (int)(bh % p.heads), b = (int)(bh / p.heads);
      src = (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2;
      const int64_t pos = append_position(p, b, t);
      if (pos >= 0 && pos < p.cap) slot = ((int64_t)b * p.heads + h) * p.cap + pos;
    }
    L.src[tid] = src;
    L.slot[tid] = slot;
  }
  // a tile with nothing to write (a hybrid flush of sequences whose buffer is
  // not full) stops here
  if (!__syncthreads_or(tid < kMV && L.slot[tid] >= 0)) return;

  // ---- the x tile (zeros for rows past the end)
  if (p.x_vec16) {
    constexpr int PER = 8;  // bf16 elements per 16 bytes; f32 uses 4
    if (p.x_bf16) {
      for (int e = tid; e < kMV * D / PER; e += 256) {
        const int v = e / (D / PER), q = e % (D / PER);
        const int64_t src = L.src[v];
        uint4 w = {0u, 0u, 0u, 0u};
        if (src >= 0) w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + src + PER * q);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          L.xs[v][PER * q + 2 * k] = __uint_as_float(ww[k] << 16);
          L.xs[v][PER * q + 2 * k + 1] = __uint_as_float(ww[k] & 0xffff0000u);
        }
      }
    } else {
      for (int e = tid; e < kMV * D / 4; e += 256) {
        const int v = e / (D / 4), q = e % (D / 4);
        const int64_t src = L.src[v];
        v4f_t w = v4f_t{0.f, 0.f, 0.f, 0.f};
        if (src >= 0) w = *reinterpret_cast<const v4f_t*>(static_cast<const float*>(p.x) + src + 4 * q);
        *reinterpret_cast<v4f_t*>(&L.xs[v][4 * q]) = w;
      }
    }
  } else {
    for (int e = tid; e < kMV * D; e += 256) {
      const int v = e / D, j = e % D;
      const int64_t src = L.src[v];
      L.xs[v][j] = src >= 0 ? load_x(p.x, src + j, p.x_bf16) : 0.f;
    }
  }
  __syncthreads();

  if (p.mode == TQ_MODE_GROUP) {
    // asymmetric min/max per 32 coordinates of the unrotated vector
    const int top = (1 << p.gbits) - 1;
    for (int e = tid; e < kMV * (D / 32); e += 256) {
      const int v = e / (D / 32), g = e % (D / 32);
      const float* xv = &L.xs[v][32 * g];
      float mn = xv[0], mx = xv[0];
      for (int r = 1; r < 32; ++r) {
        mn = fminf(mn, xv[r]);
        mx = fmaxf(mx, xv[r]);
      }
      const float rng = mx - mn;
      for (int r = 0; r < 32; ++r) {
        uint32_t q = 0;
        if (rng > 0.f) q = (uint32_t)fminf(fmaxf(rintf((xv[r] - mn) * (float)top / rng), 0.f), (float)top);
        L.codes[v][32 * g + r] = (uint8_t)q;
      }
      const int64_t slot = L.slot[v];
      if (slot >= 0) {
        p.scale[slot * p.groups + g] = rng / (float)top;
        p.gmin[slot * p.groups + g] = mn;
      }
    }
    __syncthreads();
    for (int e = tid; e < kMV * p.words; e += 256) {
      const int v = e / p.words, w = e % p.words;
      const int64_t slot = L.slot[v];
      if (slot >= 0) p.idx[slot * p.idx_stride + w] = pack_word(L.codes[v], w, p.gbits);
    }
    return;
  }

  // ---- norms: four threads per vector (float64 sum of squares, so that the
  // stored float32 norm is the correctly rounded one)
  {
    const int v = tid >> 2, part = tid & 3;
    double ss = 0.0;
    for (int j = part * (D / 4); j < (part + 1) * (D / 4); ++j) ss = fma((double)L.xs[v][j], (double)L.xs[v][j], ss);
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (part == 0) L.nrm[v] = (float)sqrt(ss);
  }
  __syncthreads();

  const bool prod = p.mode == TQ_MODE_PROD;
  switch (p.levels) {
    case 2: prod ? quantize_rotated<D, 1, true>(p, L) : quantize_rotated<D, 1, false>(p, L); break;
    case 4: prod ? quantize_rotated<D, 3, true>(p, L) : quantize_rotated<D, 3, false>(p, L); break;
    case 8: prod ? quantize_rotated<D, 7, true>(p, L) : quantize_rotated<D, 7, false>(p, L); break;
    default: prod ? quantize_rotated<D, 15, true>(p, L) : quantize_rotated<D, 15, false>(p, L); break;
  }
}

// Small appends (a few tokens per sequence and head, the decode-step case):
// one workgroup per vector (256 threads, 1024 at head_dim 256), so that the
// rotation's loads are all in flight at once instead of one wave streaming
// Pi^T through L2 in many round trips.  Thread t owns coordinate i = t % D
// and the slice of the contraction j in [part*JN, (part+1)*JN), part = t / D;
// the rotation rows it needs (and the sketch rows, up to head_dim 128) are
// loaded before x arrives.  Every mode (group mode needs no rotation),
// head_dim 32, 64, 128 and 256.
template <int D>
constexpr int small_threads() { return D <= 128 ? 256 : 1024; }

template <int D>
__global__ __launch_bounds__(small_threads<D>()) void quantize_small_kernel(QuantizeSets sets) {
  constexpr int T = small_threads<D>();
  constexpr int NW = T / 64;
  constexpr int PARTS = T / D;
  constexpr int JN = D / PARTS;
  constexpr bool kEarlySketch = D <= 128;  // at 1024 threads the sketch rows wait for the registers
  static_assert(PARTS * D == T && JN <= 64, "one to eight slices of at most 64 terms");
  const QuantizeParams& p = sets.s[blockIdx.y];
  __shared__ float xs[D];
  __shared__ float part_sum[PARTS][D];
  __shared__ double part_sum_d[PARTS][D];  // Prod: the rotation in float64
  __shared__ uint32_t wbuf[32];
  __shared__ double red[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = tid % D, part = tid / D, j0 = part * JN;
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t vec = blockIdx.x;
  if (vec >= total) return;  // whole workgroup
  const int t = (int)(vec % p.n_new);
  const int64_t bh = vec / p.n_new;
  const int h = (int)(bh % p.heads), b = (int)(bh / p.heads);
  const int64_t pos = append_position(p, b, t);
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
    if (tid < p.words) p.idx[tok * p.idx_stride + tid] = wbuf[tid];
    return;
  }

  // rotation (and sketch) slices first, then x
  // row slice j0 .. j0+JN-1 of row i: from the transposed table (coalesced
  // across threads), or at 1024 threads as 16-byte loads of the row-major one
  // (one address instead of JN)
  auto load_slice = [&](const float* t, const float* rowmajor, float (&r)[JN]) {
    if constexpr (kEarlySketch) {
#pragma unroll
      for (int k = 0; k < JN; ++k) r[k] = t[(size_t)(j0 + k) * D + i];
    } else {
      const float4* src = reinterpret_cast<const float4*>(rowmajor + (size_t)i * D + j0);
#pragma unroll
      for (int k = 0; k < JN / 4; ++k) {
        const float4 v = src[k];
        r[4 * k] = v.x;
        r[4 * k + 1] = v.y;
        r[4 * k + 2] = v.z;
        r[4 * k + 3] = v.w;
      }
    }
  };
  float pr[JN], sr[JN];
  load_slice(p.pit, p.pi, pr);
  if (kEarlySketch && prod) load_slice(p.st, p.s, sr);
  float xv = 0.f;
  if (tid < D) xv = load_x(p.x, (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2 + tid, p.x_bf16);
  if (tid < 32) wbuf[tid] = 0u;
  if (tid < D) xs[tid] = xv;
  // the norm from a float64 sum of squares (the stored float32 norm is the
  // correctly rounded one)
  const double sq = wave_sum_d((double)xv * (double)xv);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  double n2 = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n2 += red[w];
  const float n = (float)sqrt(n2);

  // y = Pi x (Prod keys in float64: their residual y - n c[idx] is a
  // difference of nearly equal terms)
  if (prod) {
    double accd = 0.0;
#pragma unroll
    for (int k = 0; k < JN; ++k) accd = fma((double)pr[k], (double)xs[j0 + k], accd);
    part_sum_d[part][i] = accd;
  } else {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < JN; ++k) acc = fmaf(pr[k], xs[j0 + k], acc);
    part_sum[part][i] = acc;
  }
  __syncthreads();
  double yd = 0.0;
  uint32_t idx = 0;
  if (tid < D) {
    if (prod) {
#pragma unroll
      for (int q = 0; q < PARTS; ++q) yd += part_sum_d[q][tid];
      const double u = n > 0.f ? yd / (double)n : 0.0;
      for (int m = 0; m < p.levels - 1; ++m) idx += u > (double)p.bnd[m] ? 1u : 0u;
    } else {
      float y = 0.f;
#pragma unroll
      for (int q = 0; q < PARTS; ++q) y += part_sum[q][tid];
      const float u = y * (n > 0.f ? 1.f / n : 0.f);
      for (int m = 0; m < p.levels - 1; ++m) idx += u > p.bnd[m] ? 1u : 0u;
    }
    pack_field(wbuf, tid, p.mse_bits, idx);
  }
  __syncthreads();
  if (tid < p.words) p.idx[tok * p.idx_stride + tid] = wbuf[tid];
  if (tid == 0) p.norm[tok] = n;
  if (!prod) return;

  // Prod: rotated residual (float64), its norm, z = S rho, sign bits
  const double rho = tid < D ? yd - (double)n * (double)p.cent[idx] : 0.0;
  const double rs = wave_sum_d(rho * rho);
  __syncthreads();  // every read of xs, part_sum and red above is done
  if (tid < D) xs[tid] = (float)rho;
  if (lane == 0) red[wave] = rs;
  if (!kEarlySketch) load_slice(p.st, p.s, sr);
  __syncthreads();
  double g2 = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) g2 += red[w];
  const float gamma = (float)sqrt(g2);
  float acc = 0.f;
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

// MSE appends of a decode step at head_dim <= 128: one wave per (vector,
// 32-coordinate group), so that each workgroup streams 32 rows of Pi instead
// of all of them and needs no workgroup barrier.  Lane (c, k) = (lane / 2, lane % 2) loads half
// k of x and of row 32 g + c of Pi (16-byte loads, all in flight at once);
// the two halves of ||x||^2 and of (Pi x)_{32 g + c} meet by one lane
// exchange.  The group's b packed words (aligned in every layout: words
// b g .. b g + b - 1) are written by the wave that owns them.  Every wave of
// a vector computes the same norm; the group-0 one stores it.
template <int D>
__global__ __launch_bounds__(64) void quantize_mse_split_kernel(QuantizeSets sets) {
  constexpr int NS = D / 32, JN = D / 2;
  static_assert(D % 32 == 0 && JN % 8 == 0, "whole groups, 16-byte slices");
  const QuantizeParams& p = sets.s[blockIdx.y];
  __shared__ uint32_t wbuf[4];
  const int lane = threadIdx.x, c = lane >> 1, part = lane & 1;
  const int64_t total = (int64_t)p.batch * p.heads * p.n_new;
  const int64_t vec = blockIdx.x / NS;
  const int g = (int)(blockIdx.x % NS);
  if (vec >= total) return;  // whole workgroup
  const int t = (int)(vec % p.n_new);
  const int64_t bh = vec / p.n_new;
  const int h = (int)(bh % p.heads), b = (int)(bh / p.heads);
  // the write position is needed only by the stores: its load is in flight
  // with the others
  const int64_t pos = append_position(p, b, t);
  // a hybrid flush of a sequence whose buffer is not full writes nothing
  if (p.flush_block > 0 && (pos < 0 || pos >= p.cap)) return;

  float4 pr[JN / 4];
  const float4* src = reinterpret_cast<const float4*>(p.pi + (size_t)(32 * g + c) * D + part * JN);
#pragma unroll
  for (int k = 0; k < JN / 4; ++k) pr[k] = src[k];
  float xv[JN];
  const int64_t x0 = (int64_t)b * p.s0 + (int64_t)h * p.s1 + (int64_t)t * p.s2 + part * JN;
  if (p.x_vec16 && p.x_bf16) {  // eight bf16 per 16-byte load
    const uint4* xs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + x0);
#pragma unroll
    for (int k = 0; k < JN / 8; ++k) {
      const uint4 w = xs[k];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[8 * k + 2 * e] = __uint_as_float(ww[e] << 16);
        xv[8 * k + 2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
      }
    }
  } else if (p.x_vec16) {  // four floats per 16-byte load
    const float4* xs = reinterpret_cast<const float4*>(static_cast<const float*>(p.x) + x0);
#pragma unroll
    for (int k = 0; k < JN / 4; ++k) {
      const float4 w = xs[k];
      xv[4 * k] = w.x;
      xv[4 * k + 1] = w.y;
      xv[4 * k + 2] = w.z;
      xv[4 * k + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < JN; ++k) xv[k] = load_x(p.x, x0 + k, p.x_bf16);
  }
  if (lane < 4) wbuf[lane] = 0u;
  float sq0 = 0.f, sq1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int k = 0; k < JN / 4; ++k) {
    sq0 = fmaf(xv[4 * k], xv[4 * k], sq0);
    sq1 = fmaf(xv[4 * k + 1], xv[4 * k + 1], sq1);
    sq0 = fmaf(xv[4 * k + 2], xv[4 * k + 2], sq0);
    sq1 = fmaf(xv[4 * k + 3], xv[4 * k + 3], sq1);
    a0 = fmaf(pr[k].x, xv[4 * k], a0);
    a1 = fmaf(pr[k].y, xv[4 * k + 1], a1);
    a0 = fmaf(pr[k].z, xv[4 * k + 2], a0);
    a1 = fmaf(pr[k].w, xv[4 * k + 3], a1);
  }
  float sq = sq0 + sq1, acc = a0 + a1;
  // lane pairs (2c, 2c + 1) hold the two halves; the half-0 sum goes first in
  // both lanes so that every lane of the vector forms the same norm
  const float sq_o = __shfl_xor(sq, 1, 64), acc_o = __shfl_xor(acc, 1, 64);
  sq = part == 0 ? sq + sq_o : sq_o + sq;
  acc = part == 0 ? acc + acc_o : acc_o + acc;
  const float n = sqrtf(sq);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (part == 0) {
    const float u = acc * (n > 0.f ? 1.f / n : 0.f);
    uint32_t idx = 0;
    for (int m = 0; m < p.levels - 1; ++m) idx += u > p.bnd[m] ? 1u : 0u;
    pack_field(wbuf, c, p.mse_bits, idx);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (pos < 0 || pos >= p.cap) return;  // nothing is written for this vector
  const int64_t tok = ((int64_t)b * p.heads + h) * p.cap + pos;
  if (lane < p.mse_bits) p.idx[tok * p.idx_stride + g * p.mse_bits + lane] = wbuf[lane];
  if (g == 0 && lane == 0) p.norm[tok] = n;
}

template <int D>
void launch_small(const QuantizeSets& sets, int n_sets, int64_t total, hipStream_t stream) {
  if constexpr (D > 128) {
    quantize_small_kernel<D><<<dim3((unsigned)total, (unsigned)n_sets), small_threads<D>(), 0, stream>>>(sets);
  } else {
    // MSE sets take the split kernel, the others one workgroup per vector; a
    // key and a value append of the same modes stay one launch
    bool mse[2] = {false, false};
    for (int k = 0; k < n_sets; ++k) mse[k] = sets.s[k].mode == TQ_MODE_MSE;
    if (n_sets == 1 || mse[0] == mse[1]) {
      if (mse[0])
        quantize_mse_split_kernel<D><<<dim3((unsigned)(total * (D / 32)), (unsigned)n_sets), 64, 0, stream>>>(sets);
      else
        quantize_small_kernel<D><<<dim3((unsigned)total, (unsigned)n_sets), small_threads<D>(), 0, stream>>>(sets);
      return;
    }
    for (int k = 0; k < 2; ++k) {
      QuantizeSets one;
      one.s[0] = sets.s[k];
      one.s[1] = sets.s[k];
      if (mse[k])
        quantize_mse_split_kernel<D><<<dim3((unsigned)(total * (D / 32)), 1u), 64, 0, stream>>>(one);
      else
        quantize_small_kernel<D><<<dim3((unsigned)total, 1u), small_threads<D>(), 0, stream>>>(one);
    }
  }
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
  const bool small = total <= kSmallAppend && (d == 32 || d == 64 || d == 128 || d == 256);
  if (small) {
    switch (d) {
      case 32: launch_small<32>(sets, n_sets, total, stream); break;
      case 64: launch_small<64>(sets, n_sets, total, stream); break;
      case 128: launch_small<128>(sets, n_sets, total, stream); break;
      default: launch_small<256>(sets, n_sets, total, stream); break;
    }
    return hipGetLastError();
  }
  const int64_t blocks = (total + kMV - 1) / kMV;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)n_sets), block(256);
  switch (d) {
    case 32: quantize_bulk_kernel<32><<<grid, block, 0, stream>>>(sets); break;
    case 64: quantize_bulk_kernel<64><<<grid, block, 0, stream>>>(sets); break;
    case 96: quantize_bulk_kernel<96><<<grid, block, 0, stream>>>(sets); break;
    case 128: quantize_bulk_kernel<128><<<grid, block, 0, stream>>>(sets); break;
    case 160: quantize_bulk_kernel<160><<<grid, block, 0, stream>>>(sets); break;
    case 192: quantize_bulk_kernel<192><<<grid, block, 0, stream>>>(sets); break;
    case 224: quantize_bulk_kernel<224><<<grid, block, 0, stream>>>(sets); break;
    case 256: quantize_bulk_kernel<256><<<grid, block, 0, stream>>>(sets); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
