// Decode attention over the compressed cache on the fp32 matrix cores, for
// the codec modes the int8 kernel does not cover: Prod keys (the QJL term
// included), 1/2/4-bit MSE values, group values.  Taken at head_dim 128 when
// a launch has more than 8 query rows per KV head (prefill blocks,
// multi-token decode), where it halves the general kernel's time.  A variant
// below takes split keys and values (two 64-channel parts at head_dim 128)
// at any row count.
//
// What is computed is the general kernel's ("turboquant validate_moe_phase2.py",
// Tests 1 and 5; "omlx turboquant_kv.py", make_mask):
//     s_t = scale * ( n_t <q_rot, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q_rot, sigma_t> )
//     o_rot = sum_t p_t n^v_t c_v[idx^v_t]   (MSE values; out = Pi_v^T o_rot / l)
//     o     = sum_t p_t (q_t s_g + mn_g)     (group values)
// with both products on v_mfma_f32_16x16x4f32 over dequantised operands, so
// the accumulation is plain fp32:
//
//   scores  S[token][row] = sum_j A[token][j] Q[j][row], A = n c[idx] (and,
//           for Prod keys, gamma sqrt(pi/2)/d sigma against S q_rot, in the
//           same accumulator).  The contraction index is permuted: in k-step
//           s lane l supplies coordinate j = (l/16) (D/4) + s, so each lane
//           decodes one contiguous run of its token's packed words.
//   values  O^T[slot][row] = sum_t V[t][coord(slot)] P[row][t]: the k-step s
//           of token group tg takes token 16 tg + 4 (l/16) + s from lane l,
//           which is exactly a score the lane holds, so the probabilities
//           never move between lanes; lane l%16 = m owns the coordinates
//           m (D/16) .. m (D/16) + D/16 - 1, one contiguous bit run of the
//           token's packed value words.
//
// One 256-thread workgroup per (chunk, KV head, sequence); wave w takes the
// 64-token tiles w, w+4, ... of the chunk with its own online softmax and
// writes its own partial (m, l, o) (4 per chunk), merged by the general
// path's merge kernel.  The query rows (rotated by the general path's qprep
// kernel) sit in LDS.
#include "chunk_order.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTile = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFlushGap = 8.f;  // log2 headroom of the lazy softmax reference

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A value loaded from a valid address (the callers clamp it), or zero: the
// load is unconditional so that the loads of a tile issue back to back.
template <class T>
__device__ __forceinline__ T pick(T v, bool ok) {
  return ok ? v : T(0);
}

// maximum over the four 16-lane groups (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rowmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Index of coordinate r (0..31) of a 32-coordinate group with words w[0..B-1]
// (LSB-first for 1, 2, 4 bits; byte lanes X, Y, Z for 3 bits).
template <int B>
__device__ __forceinline__ uint32_t group_code(const uint32_t* w, int r) {
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

template <int D, int KB, int VB>
__global__ __launch_bounds__(kWaves * 64) void decode_mfma_kernel(DecodeParams p) {
  constexpr int KS = D / 4;          // contraction terms per lane (k-steps)
  constexpr int KG = KS / 32;        // 32-coordinate groups in a lane's key slice
  constexpr int KW = KB * KG;        // index words of the slice
  constexpr int NU = D / 16;         // value coordinate tiles = coordinates per lane run
  constexpr int VRB = NU * VB;       // bits of a lane's value run (8..64)
  constexpr int VW = (VRB + 31) / 32;
  constexpr int QSTR = D + 4;        // LDS row stride of the query tables
  static_assert(KG >= 1 && VRB % 8 == 0, "head_dim 128 or 256");
  __shared__ __attribute__((aligned(16))) float s_q[16 * QSTR];
  __shared__ __attribute__((aligned(16))) float s_qs[16 * QSTR];
  __shared__ float s_kc[16], s_vc[16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;  // token slot / query row, lane group
  const int chunk_id = rotated_chunk(blockIdx.x, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int gh = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + gh;
  const int rows = p.rows;
  const bool prod = p.kmode == TQ_MODE_PROD;
  const bool vgroup = p.vmode == TQ_MODE_GROUP;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int ntok = (c0 + p.chunk < len ? c0 + p.chunk : len) - c0;  // may be <= 0
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;  // the causal rule's length
  const int lim = lenm - p.q_len + ((p.row0 + m) % p.q_len) + 1 - c0;  // row m sees tokens < lim

  for (int e = threadIdx.x; e < 16 * D; e += kWaves * 64) {
    const int r = e / D, j = e % D;
    const size_t src = ((size_t)bg * rows + r) * D + j;
    s_q[r * QSTR + j] = r < rows ? p.qrot[src] : 0.f;
    s_qs[r * QSTR + j] = (prod && r < rows) ? p.qs[src] : 0.f;
  }
  if (threadIdx.x < 16) {
    const int t = threadIdx.x;
    s_kc[t] = t < (1 << p.kbits) ? p.k_cent[t] : 0.f;
    s_vc[t] = (!vgroup && t < (1 << p.vbits)) ? p.v_cent[t] : 0.f;
  }
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  const float qjl = kQjlConstNumer / (float)D;
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)c0;  // slot of token 0 of the chunk
  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int T0 = wave * kTile; T0 < ntok; T0 += kWaves * kTile) {
    // ---- key operands: token T0 + 16 tg + m, coordinates g*KS .. g*KS + KS - 1
    uint32_t kw[4][KW], ksw[4][KG];
    float kn[4], kq[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int tok = T0 + 16 * tg + m;
      const bool ok = tok < ntok;
      const size_t slot = base + (ok ? tok : 0);
#pragma unroll
      for (int w = 0; w < KW; ++w) kw[tg][w] = pick(p.k_idx[slot * p.kwords + g * KW + w], ok);
#pragma unroll
      for (int w = 0; w < KG; ++w) ksw[tg][w] = prod ? pick(p.k_sign[slot * p.ksign_words + g * KG + w], ok) : 0u;
      kn[tg] = pick(p.k_norm[slot], ok);
      kq[tg] = prod ? pick(p.k_rnorm[slot], ok) * qjl : 0.f;
    }
    // ---- scores: sacc[tg][i] = score of token T0 + 16 tg + 4 g + i for row m
    v4f sacc[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) sacc[tg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t4 = 0; t4 < KS / 4; ++t4) {
      const v4f qv = *reinterpret_cast<const v4f*>(&s_q[m * QSTR + g * KS + 4 * t4]);
      const v4f qsv = *reinterpret_cast<const v4f*>(&s_qs[m * QSTR + g * KS + 4 * t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * t4 + e;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const uint32_t code = group_code<KB>(&kw[tg][KB * (s >> 5)], s & 31);
          sacc[tg] = mfma4(kn[tg] * s_kc[code], qv[e], sacc[tg]);
          if (prod) {
            const bool bit = (ksw[tg][s >> 5] >> (s & 31)) & 1u;
            sacc[tg] = mfma4(bit ? kq[tg] : -kq[tg], qsv[e], sacc[tg]);
          }
        }
      }
    }

    // ---- online softmax of row m over this lane's 16 tokens
    float sc[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = T0 + 16 * tg + 4 * g + i;
        const float v = (tok < ntok && tok < lim) ? sacc[tg][i] * sl2 : -INFINITY;
        sc[4 * tg + i] = v;
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
    // value norms (MSE values) of the lane's tokens: four consecutive ones per group
    float pv[16];
    float psum = 0.f;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int t0 = T0 + 16 * tg + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = exp2f(sc[4 * tg + i] - m_ref);
        psum += pr;
        const bool ok = t0 + i < ntok;
        float nv = 1.f;
        if (!vgroup) {
          const float x = p.v_norm[base + (ok ? t0 + i : 0)];
          nv = ok ? x : 1.f;
        }
        pv[4 * tg + i] = pr * nv;
      }
    }
    l_run += psum;

    // ---- values: token 16 tg + 4 g + s, coordinates m*NU .. m*NU + NU - 1
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tok = T0 + 16 * tg + 4 * g + s;
        const bool ok = tok < ntok;
        const size_t slot = base + (ok ? tok : 0);
        const int bit0 = m * VRB;
        uint32_t run[VW];
#pragma unroll
        for (int w = 0; w < VW; ++w) run[w] = pick(p.v_idx[slot * p.vwords + (bit0 >> 5) + w], ok);
        float gs = 0.f, gm = 0.f;
        if (vgroup) {
          const int grp = (m * NU) >> 5;
          gs = pick(p.v_scale[slot * p.vgroups + grp], ok);
          gm = pick(p.v_gmin[slot * p.vgroups + grp], ok);
        }
        const int sh = bit0 & 31;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int bit = u * VB;  // within the run
          uint32_t code;
          if constexpr (VW == 1) {
            code = (run[0] >> (sh + bit)) & ((1u << VB) - 1u);
          } else {
            code = (run[bit >> 5] >> (bit & 31)) & ((1u << VB) - 1u);
          }
          const float a = vgroup ? fmaf((float)code, gs, gm) : s_vc[code];
          acc[u] = mfma4(a, pv[4 * tg + s], acc[u]);
        }
      }
    }
  }

  // ---- this wave's partial: o[row m][coord (4g + i) NU + u], m and l of row m
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int part = chunk_id * kWaves + wave;
  const int n_parts = gridDim.x * kWaves;
  if (m < rows) {
    float* po = p.part_o + (((size_t)bg * n_parts + part) * rows + m) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(4 * g + i) * NU + u] = acc[u][i];
    if (g == 0) {
      float* pml = p.part_ml + (((size_t)bg * n_parts + part) * rows + m) * 2;
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
}

// ---- split caches ("omlx turboquant_kv.py", TurboQuantSplitState): a low part
// of channels 0..63 with KB-bit codes and a high part of channels 64..127
// with KB+1-bit codes, each an MSE instance with its own norm and centroids
// (head_dim 128, keys and values both split this way).  The products are the
// kernel above's; only which lane supplies which coordinate changes, so that
// every k-step (keys) and every value product reads one part, with a code
// extraction the same for all lanes up to a per-lane shift:
//   keys    k-steps 0..15 take the low part, 16..31 the high part; in a
//           part of B-bit codes k-step s of lane group g takes coordinate
//           16 g + s (B = 1, 2, 4: a run of 16 codes of the part's LSB-first
//           stream) or, for B = 3, 32 (g/2) + 4 (s/2) + 2 (g%2) + s%2 (field
//           s/2 of byte 2 (g%2) + s%2 of the byte-lane group g/2).  The query
//           rows are staged in LDS in this order.  A = n_part c_part[code].
//   values  products 0..3 take the low part, 4..7 the high part; in a part
//           lane m owns coordinates 4 m .. 4 m + 3 (B = 1, 2, 4: 4 B bits of
//           the stream; B = 3: field m%8 of the four bytes of group m/8), and
//           the part's norm scales the probability operand.
// Words of a B-bit code group (32 channels) and of a 64-channel part: B, 2 B.

// key coordinate (within a part) of k-step s of lane group g
template <int B>
__device__ __forceinline__ int split_kcoord(int g, int s) {
  if constexpr (B == 3) return 32 * (g >> 1) + 4 * (s >> 1) + 2 * (g & 1) + (s & 1);
  return 16 * g + s;
}

// words of a part a lane group loads per token, the first one's index in the
// part, and the right shift that brings its codes to bit 0 (byte 0 for B = 3)
template <int B>
constexpr int split_klw() {
  return B == 3 ? 3 : (B == 4 ? 2 : 1);
}
template <int B>
__device__ __forceinline__ int split_kword0(int g) {
  if constexpr (B == 3) return 3 * (g >> 1);
  if constexpr (B == 4) return 2 * g;
  if constexpr (B == 2) return g;
  return g >> 1;
}
template <int B>
__device__ __forceinline__ uint32_t split_kshift(int g) {
  return (B == 3 || B == 1) ? 16u * (uint32_t)(g & 1) : 0u;
}

// code of k-step s (compile-time) from the lane group's shifted words
template <int B>
__device__ __forceinline__ uint32_t split_kcode(const uint32_t* w, int s) {
  if constexpr (B == 3) {
    const int kb = 8 * (s & 1);
    switch (s >> 1) {
      case 0: return (w[0] >> kb) & 7u;
      case 1: return (w[0] >> (kb + 3)) & 7u;
      case 2: return ((w[0] >> (kb + 6)) & 3u) | (((w[2] >> (kb + 6)) & 1u) << 2);
      case 3: return (w[1] >> kb) & 7u;
      case 4: return (w[1] >> (kb + 3)) & 7u;
      case 5: return ((w[1] >> (kb + 6)) & 3u) | (((w[2] >> (kb + 7)) & 1u) << 2);
      case 6: return (w[2] >> kb) & 7u;
      default: return (w[2] >> (kb + 3)) & 7u;
    }
  } else if constexpr (B == 4) {
    return (w[s >> 3] >> (4 * (s & 7))) & 15u;
  } else {
    return (w[0] >> (B * s)) & ((1u << B) - 1u);
  }
}

// A lane's value codes of one part: the word(s) to load and how to bring
// its four codes to fixed places (code u at bits B u; for B = 3 in byte u)
template <int B>
struct SplitValueLane {
  int w0, wz;  // word indices in the part (wz: the group's third word, B = 3)
  uint32_t sh, m1, m2, zsh;
  __device__ __forceinline__ explicit SplitValueLane(int m) {
    if constexpr (B == 3) {
      // field a of the four bytes of group G: bits 3 (a%3) of word a/3, and
      // for fields 2 and 5 two bits there plus bit 6 or 7 of the third word
      const int G = m >> 3, a = m & 7;
      w0 = 3 * G + a / 3;
      wz = 3 * G + 2;
      sh = 3u * (uint32_t)(a % 3);
      const bool two = a % 3 == 2;
      m1 = two ? 0x03030303u : 0x07070707u;
      m2 = two ? 0x04040404u : 0u;
      zsh = a == 5 ? 5u : 4u;
    } else {
      const int bit = 4 * m * B;
      w0 = wz = bit >> 5;
      sh = (uint32_t)(bit & 31);
      m1 = m2 = zsh = 0u;
    }
  }
  __device__ __forceinline__ uint32_t run(uint32_t w, uint32_t z) const {
    if constexpr (B == 3) return ((w >> sh) & m1) | ((z >> zsh) & m2);
    return w >> sh;
  }
  __device__ __forceinline__ static uint32_t code(uint32_t run, int u) {
    if constexpr (B == 3) return (run >> (8 * u)) & 7u;
    return (run >> (B * u)) & ((1u << B) - 1u);
  }
};

template <int KB, int VB>
__global__ __launch_bounds__(kWaves * 64, kSplitWgPerCu) void decode_mfma_split_kernel(DecodeParams p) {
  constexpr int D = 128, NU = 8, QSTR = D + 4;
  constexpr int KH = KB + 1, VH = VB + 1;
  constexpr int KLW = split_klw<KB>(), KHW = split_klw<KH>();
  __shared__ __attribute__((aligned(16))) float s_q[16 * QSTR];
  __shared__ float s_kc[32], s_vc[32];  // low part's centroids at 0, high part's at 16

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int chunk_id = rotated_chunk(blockIdx.x, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int gh = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + gh;
  const int rows = p.rows;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int ntok = (c0 + p.chunk < len ? c0 + p.chunk : len) - c0;  // may be <= 0
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;  // the causal rule's length
  const int lim = lenm - p.q_len + ((p.row0 + m) % p.q_len) + 1 - c0;  // row m sees tokens < lim

  // query rows in k-step order: entry g 32 + s of a row is the coordinate
  // that k-step s of lane group g takes
  for (int e = threadIdx.x; e < 16 * D; e += kWaves * 64) {
    const int r = e / D, c = e % D;
    const int gg = c >> 5, s = c & 31;
    const int j = s < 16 ? split_kcoord<KB>(gg, s) : 64 + split_kcoord<KH>(gg, s - 16);
    s_q[r * QSTR + c] = r < rows ? p.qrot[((size_t)bg * rows + r) * D + j] : 0.f;
  }
  if (threadIdx.x < 32) {
    const int t = threadIdx.x & 15;
    const bool hi = threadIdx.x >= 16;
    s_kc[threadIdx.x] = hi ? (t < (1 << KH) ? p.k_cent_hi[t] : 0.f) : (t < (1 << KB) ? p.k_cent[t] : 0.f);
    s_vc[threadIdx.x] = hi ? (t < (1 << VH) ? p.v_cent_hi[t] : 0.f) : (t < (1 << VB) ? p.v_cent[t] : 0.f);
  }
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)c0;  // slot of token 0 of the chunk
  const int klo = split_kword0<KB>(g), khi = 2 * KB + split_kword0<KH>(g);
  const uint32_t kslo = split_kshift<KB>(g), kshi = split_kshift<KH>(g);
  const SplitValueLane<VB> vl(m);
  const SplitValueLane<VH> vh(m);
  const int vhw = 2 * VB;  // the high part's first word in a value record
  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int T0 = wave * kTile; T0 < ntok; T0 += kWaves * kTile) {
    // ---- key operands: token T0 + 16 tg + m, lane group g's words of each part
    uint32_t kl[4][KLW], kh[4][KHW];
    float nl[4], nh[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int tok = T0 + 16 * tg + m;
      const bool ok = tok < ntok;
      const size_t slot = base + (ok ? tok : 0);
      const uint32_t* rec = p.k_idx + slot * p.kwords;
#pragma unroll
      for (int w = 0; w < KLW; ++w) kl[tg][w] = pick(rec[klo + w], ok) >> kslo;
#pragma unroll
      for (int w = 0; w < KHW; ++w) kh[tg][w] = pick(rec[khi + w], ok) >> kshi;
      nl[tg] = pick(p.k_norm[slot], ok);
      nh[tg] = pick(p.k_norm_hi[slot], ok);
    }
    // ---- scores: sacc[tg][i] = score of token T0 + 16 tg + 4 g + i for row m
    v4f sacc[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) sacc[tg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t4 = 0; t4 < 8; ++t4) {
      const v4f qv = *reinterpret_cast<const v4f*>(&s_q[m * QSTR + g * 32 + 4 * t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * t4 + e;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const float a = s < 16 ? nl[tg] * s_kc[split_kcode<KB>(kl[tg], s)]
                                 : nh[tg] * s_kc[16 + split_kcode<KH>(kh[tg], s - 16)];
          sacc[tg] = mfma4(a, qv[e], sacc[tg]);
        }
      }
    }

    // ---- online softmax of row m over this lane's 16 tokens
    float sc[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = T0 + 16 * tg + 4 * g + i;
        const float v = (tok < ntok && tok < lim) ? sacc[tg][i] * sl2 : -INFINITY;
        sc[4 * tg + i] = v;
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
    // ---- values: token 16 tg + 4 g + s; lane m's coordinates 4 m .. 4 m + 3
    // of each part, the probabilities times each part's value norm formed one
    // token group at a time (fewer live registers: four waves per SIMD)
    float psum = 0.f;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int t0 = T0 + 16 * tg + 4 * g;
      float pl[4], ph[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float pr = exp2f(sc[4 * tg + s] - m_ref);
        psum += pr;
        const bool ok = t0 + s < ntok;
        const size_t slot = base + (ok ? t0 + s : 0);
        pl[s] = pr * pick(p.v_norm[slot], ok);
        ph[s] = pr * pick(p.v_norm_hi[slot], ok);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bool ok = t0 + s < ntok;
        const size_t slot = base + (ok ? t0 + s : 0);
        const uint32_t* rec = p.v_idx + slot * p.vwords;
        const uint32_t rl = vl.run(pick(rec[vl.w0], ok), VB == 3 ? pick(rec[vl.wz], ok) : 0u);
        const uint32_t rh = vh.run(pick(rec[vhw + vh.w0], ok), VH == 3 ? pick(rec[vhw + vh.wz], ok) : 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc[u] = mfma4(s_vc[SplitValueLane<VB>::code(rl, u)], pl[s], acc[u]);
          acc[4 + u] = mfma4(s_vc[16 + SplitValueLane<VH>::code(rh, u)], ph[s], acc[4 + u]);
        }
      }
    }
    l_run += psum;
  }

  // ---- this wave's partial: o[row m][64 (u / 4) + 4 (4 g + i) + u % 4], m and l of row m
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int part = chunk_id * kWaves + wave;
  const int n_parts = gridDim.x * kWaves;
  if (m < rows) {
    float* po = p.part_o + (((size_t)bg * n_parts + part) * rows + m) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[64 * (u >> 2) + 4 * (4 * g + i) + (u & 3)] = acc[u][i];
    if (g == 0) {
      float* pml = p.part_ml + (((size_t)bg * n_parts + part) * rows + m) * 2;
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
}

template <int KB>
hipError_t launch_split_kb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.vbits) {
    case 1: decode_mfma_split_kernel<KB, 1><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 2: decode_mfma_split_kernel<KB, 2><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 3: decode_mfma_split_kernel<KB, 3><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_split(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.kbits) {
    case 1: return launch_split_kb<1>(p, grid, stream);
    case 2: return launch_split_kb<2>(p, grid, stream);
    case 3: return launch_split_kb<3>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int KB>
hipError_t launch_kb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  if (p.vbits == 2) {
    decode_mfma_kernel<D, KB, 2><<<grid, dim3(kWaves * 64), 0, stream>>>(p);
  } else if (p.vbits == 4) {
    decode_mfma_kernel<D, KB, 4><<<grid, dim3(kWaves * 64), 0, stream>>>(p);
  } else if (p.vbits == 1 && p.vmode == TQ_MODE_MSE) {
    decode_mfma_kernel<D, KB, 1><<<grid, dim3(kWaves * 64), 0, stream>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dd(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.kbits) {
    case 1: return launch_kb<D, 1>(p, grid, stream);
    case 2: return launch_kb<D, 2>(p, grid, stream);
    case 3: return launch_kb<D, 3>(p, grid, stream);
    case 4: return launch_kb<D, 4>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  const bool split = p.kmode == TQ_MODE_SPLIT || p.vmode == TQ_MODE_SPLIT;
  const bool bf16 = !split && bf16_decode_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits, p.rows);
  const bool ok = split ? mfma_split_supported(p.d, p.kmode, p.kbits, 32 * p.ksplit_g, p.vmode, p.vbits,
                                               32 * p.vsplit_g, p.rows)
                        : bf16 || mfma_decode_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits, p.rows);
  if (!ok || p.hkv > 65535 ||
      p.batch > 65535 || p.n_chunks < 1 || (int64_t)p.n_chunks * kWaves > 4096 || p.chunk % (kWaves * kTile))
    return hipErrorInvalidValue;
  hipError_t e = launch_qprep(p, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(p.n_chunks, p.hkv, p.batch);
  if (bf16)
    e = launch_decode_bf16_kernel(p, grid, stream);
  else if (split)
    e = launch_split(p, grid, stream);
  else
    e = p.d == 128 ? launch_dd<128>(p, grid, stream) : launch_dd<256>(p, grid, stream);
  if (e != hipSuccess) return e;
  DecodeParams pm = p;
  if (!bf16) pm.n_chunks = p.n_chunks * kWaves;  // one partial per wave (per workgroup for bf16)
  return launch_merge(pm, stream);
}

}  // namespace tq
