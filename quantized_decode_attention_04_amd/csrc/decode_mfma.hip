// Decode attention over the compressed cache on the fp32 matrix cores, for
// the codec modes the int8 kernel does not cover: Prod keys (the QJL term
// included), 1/2/4-bit MSE values, group values.  Taken at head_dim 128 when
// a launch has more than 8 query rows per KV head (prefill blocks,
// multi-token decode), where it halves the general kernel's time.  A variant
// below takes split keys and values (two parts of half the head each) at any
// row count.
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
// of channels 0 .. D/2 - 1 with KB-bit codes and a high part of the other D/2
// channels with KB+1-bit codes, each an MSE instance with its own norm and
// centroids (head_dim 128 or 256, keys and values both split this way).  The
// products are the kernel above's; only which lane supplies which coordinate
// changes, so that every k-step (keys) and every value product reads one
// part, with a code extraction the same for all lanes up to a per-lane shift:
//   keys    k-steps 0 .. D/8 - 1 take the low part, the rest the high part.
//           In a part of B-bit codes k-step s of lane group g takes
//           coordinate 32 g + s at head_dim 256 (the lane group's own code
//           group); at 128, 16 g + s (B = 1, 2, 4: a run of 16 codes of the
//           part's LSB-first stream) or, for B = 3, 32 (g/2) + 4 (s/2) +
//           2 (g%2) + s%2 (field s/2 of byte 2 (g%2) + s%2 of the byte-lane
//           group g/2).  The query rows are staged in LDS in this order.
//           A = n_part c_part[code].
//   values  products 0 .. D/32 - 1 take the low part, the rest the high part;
//           in a part lane m owns the coordinates NP m .. NP m + NP - 1 (NP =
//           D/32; B = 1, 2, 4: NP B bits of the stream; B = 3: NP/4 fields
//           of the four bytes of one group, see SplitValueLane), and the
//           part's norm scales the probability operand.
// Words of a B-bit code group (32 channels): B.

// key coordinate (within a part) of k-step s of lane group g
template <int D, int B>
__device__ __forceinline__ int split_kcoord(int g, int s) {
  if constexpr (D == 256) return 32 * g + s;
  if constexpr (B == 3) return 32 * (g >> 1) + 4 * (s >> 1) + 2 * (g & 1) + (s & 1);
  return 16 * g + s;
}

// words of a part a lane group loads per token, the first one's index in the
// part, and the right shift that brings its codes to bit 0 (byte 0 for B = 3)
template <int D, int B>
constexpr int split_klw() {
  return D == 256 ? B : (B == 3 ? 3 : (B == 4 ? 2 : 1));
}
template <int D, int B>
__device__ __forceinline__ int split_kword0(int g) {
  if constexpr (D == 256 || B == 3) return B * (D == 256 ? g : (g >> 1));
  if constexpr (B == 4) return 2 * g;
  if constexpr (B == 2) return g;
  return g >> 1;
}
template <int D, int B>
__device__ __forceinline__ uint32_t split_kshift(int g) {
  return (D == 128 && (B == 3 || B == 1)) ? 16u * (uint32_t)(g & 1) : 0u;
}

// code of k-step s (compile-time) from the lane group's shifted words
template <int D, int B>
__device__ __forceinline__ uint32_t split_kcode(const uint32_t* w, int s) {
  if constexpr (D == 256) return group_code<B>(w, s);
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

// A lane's NP value codes of one part (NP = 4 or 8): the word(s) to load and
// how to bring its codes to fixed places.  B = 1, 2, 4: code u at bits B u of
// one shifted word.  B = 3: NP / 4 fields of the four bytes of group G (field
// a of byte k is coordinate 32 G + 4 a + k): at NP = 4 field m % 8 of group
// m / 8, at NP = 8 fields 2 (m % 4) and 2 (m % 4) + 1 of group m / 4, so that
// lane m's coordinates are NP m .. NP m + NP - 1 either way; code u in byte
// u % 4 of selector f = u / 4.  A field a lies at bits 3 (a % 3) of word a / 3
// of the group, and fields 2 and 5 take two bits there plus bit 6 or 7 of the
// third word.
template <int B, int NP>
struct SplitValueLane {
  static constexpr int NF = B == 3 ? NP / 4 : 1;  // words (selectors) per token
  int w[NF], wz;
  uint32_t sh[NF], m1[NF], m2[NF], zsh[NF];
  __device__ __forceinline__ explicit SplitValueLane(int m) {
    if constexpr (B == 3) {
      const int G = NP == 4 ? (m >> 3) : (m >> 2);
      wz = 3 * G + 2;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int a = NP == 4 ? (m & 7) : 2 * (m & 3) + f;
        w[f] = 3 * G + a / 3;
        sh[f] = 3u * (uint32_t)(a % 3);
        const bool two = a % 3 == 2;
        m1[f] = two ? 0x03030303u : 0x07070707u;
        m2[f] = two ? 0x04040404u : 0u;
        zsh[f] = a == 5 ? 5u : 4u;
      }
    } else {
      const int bit = NP * m * B;
      w[0] = wz = bit >> 5;
      sh[0] = (uint32_t)(bit & 31);
      m1[0] = m2[0] = zsh[0] = 0u;
    }
  }
  __device__ __forceinline__ uint32_t run(int f, uint32_t x, uint32_t z) const {
    if constexpr (B == 3) return ((x >> sh[f]) & m1[f]) | ((z >> zsh[f]) & m2[f]);
    return x >> sh[0];
  }
  // code u from the runs
  __device__ __forceinline__ static uint32_t code(const uint32_t* r, int u) {
    if constexpr (B == 3) return (r[u >> 2] >> (8 * (u & 3))) & 7u;
    return (r[0] >> (B * u)) & ((1u << B) - 1u);
  }
};

// resident 256-thread workgroups per CU: at head_dim 128 kSplitWgPerCu, at
// 256 two (twice the accumulators)
template <int D>
constexpr int split_wg_per_cu() {
  return D == 128 ? kSplitWgPerCu : 2;
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(kWaves * 64, split_wg_per_cu<D>()) void decode_mfma_split_kernel(DecodeParams p) {
  constexpr int KS = D / 4;       // k-steps; the first KS / 2 take the low part
  constexpr int NU = D / 16;      // value products; the first NU / 2 take the low part
  constexpr int NP = D / 32;      // coordinates a lane owns in each part
  constexpr int QSTR = D + 4;
  constexpr int KH = KB + 1, VH = VB + 1;
  constexpr int KLW = split_klw<D, KB>(), KHW = split_klw<D, KH>();
  constexpr int LO_W = D * KB / 64, VLO_W = D * VB / 64;  // words of the low parts
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

  // query rows in k-step order: entry KS g + s of a row is the coordinate
  // that k-step s of lane group g takes
  for (int e = threadIdx.x; e < 16 * D; e += kWaves * 64) {
    const int r = e / D, c = e % D;
    const int gg = c / KS, s = c % KS;
    const int j = s < KS / 2 ? split_kcoord<D, KB>(gg, s) : D / 2 + split_kcoord<D, KH>(gg, s - KS / 2);
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
  const int klo = split_kword0<D, KB>(g), khi = LO_W + split_kword0<D, KH>(g);
  const uint32_t kslo = split_kshift<D, KB>(g), kshi = split_kshift<D, KH>(g);
  const SplitValueLane<VB, NP> vl(m);
  const SplitValueLane<VH, NP> vh(m);
  constexpr int VLF = SplitValueLane<VB, NP>::NF, VHF = SplitValueLane<VH, NP>::NF;
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
    for (int t4 = 0; t4 < KS / 4; ++t4) {
      const v4f qv = *reinterpret_cast<const v4f*>(&s_q[m * QSTR + g * KS + 4 * t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * t4 + e;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          const float a = s < KS / 2 ? nl[tg] * s_kc[split_kcode<D, KB>(kl[tg], s)]
                                     : nh[tg] * s_kc[16 + split_kcode<D, KH>(kh[tg], s - KS / 2)];
          sacc[tg] = mfma4(a, qv[e], sacc[tg]);
        }
      }
      // keep each group of four k-steps' look-ups next to its products: at
      // four waves per SIMD (128 registers) the look-ups the compiler
      // otherwise hoists ahead spill to scratch memory
      __builtin_amdgcn_sched_barrier(0);
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
    // ---- values: token 16 tg + 4 g + s; lane m's coordinates NP m ..
    // NP m + NP - 1 of each part, the probabilities times each part's value
    // norm formed one token group at a time (fewer live registers)
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
        uint32_t rl[VLF], rh[VHF];
        const uint32_t zl = VB == 3 ? pick(rec[vl.wz], ok) : 0u;
        const uint32_t zh = VH == 3 ? pick(rec[VLO_W + vh.wz], ok) : 0u;
#pragma unroll
        for (int f = 0; f < VLF; ++f) rl[f] = vl.run(f, pick(rec[vl.w[f]], ok), zl);
#pragma unroll
        for (int f = 0; f < VHF; ++f) rh[f] = vh.run(f, pick(rec[VLO_W + vh.w[f]], ok), zh);
#pragma unroll
        for (int u = 0; u < NU / 2; ++u) {
          acc[u] = mfma4(s_vc[SplitValueLane<VB, NP>::code(rl, u)], pl[s], acc[u]);
          acc[NU / 2 + u] = mfma4(s_vc[16 + SplitValueLane<VH, NP>::code(rh, u)], ph[s], acc[NU / 2 + u]);
        }
      }
    }
    l_run += psum;
  }

  // ---- this wave's partial: o[row m][(D/2) (u / (NU/2)) + NP (4 g + i) + u % (NU/2)], m and l of row m
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int part = chunk_id * kWaves + wave;
  const int n_parts = gridDim.x * kWaves;
  if (m < rows) {
    float* po = p.part_o + (((size_t)bg * n_parts + part) * rows + m) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        po[(D / 2) * (u / (NU / 2)) + NP * (4 * g + i) + (u % (NU / 2))] = acc[u][i];
    if (g == 0) {
      float* pml = p.part_ml + (((size_t)bg * n_parts + part) * rows + m) * 2;
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
}

template <int D, int KB>
hipError_t launch_split_kb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.vbits) {
    case 1: decode_mfma_split_kernel<D, KB, 1><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 2: decode_mfma_split_kernel<D, KB, 2><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    case 3: decode_mfma_split_kernel<D, KB, 3><<<grid, dim3(kWaves * 64), 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  switch (p.kbits) {
    case 1: return launch_split_kb<D, 1>(p, grid, stream);
    case 2: return launch_split_kb<D, 2>(p, grid, stream);
    case 3: return launch_split_kb<D, 3>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  return p.d == 128 ? launch_split_d<128>(p, grid, stream) : launch_split_d<256>(p, grid, stream);
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
