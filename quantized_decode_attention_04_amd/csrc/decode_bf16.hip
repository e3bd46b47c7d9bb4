// Decode attention over the compressed cache on the bf16 matrix cores, with
// every fp32 operand split into two bf16 pieces, for head_dim 128 or 256 keys
// whose MSE part has 1, 2 or 3 bits (MSE keys, or Prod keys of 2 to 4 bits) and
// MSE values of 1, 2 or 4 bits or 2-bit group values, at up to 16 query rows
// per KV head.
//
// What is computed is the fp32 kernels' ("turboquant validate_moe_phase2.py",
// Tests 1, 2 and 5; "omlx turboquant_kv.py", make_mask):
//     s_t = scale * ( n_t <q_rot, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q_rot, sigma_t> )
//     o_rot = sum_t p_t n^v_t c_v[idx^v_t]        (MSE values; out = Pi_v^T o_rot / l)
//     o     = sum_t p_t (q_t s_g + mn_g)          (group values; out = o / l)
// Each product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A
// value x is held as x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (round
// to nearest even: |x - hi - lo| <= 2^-17 |x|), and a product of two split
// operands as a_hi b_hi + a_hi b_lo + a_lo b_hi, which leaves out
// a_lo b_lo (<= 2^-16 |a b|).  The QJL signs are +-1, exact in bf16, so that
// term takes two products; the probabilities are split by truncation (hi =
// the top half of the fp32 word, lo = the truncated rest: |p - hi - lo| <
// 2^-15 |p|).  The scores and outputs therefore carry relative errors of
// order 1e-5 against the exact fp32 sums, an order below the decode's
// tolerance.
//
// Layout (lane l, m = l % 16, g = l / 16; A[i][k] B[k][j] summed over k, and
// lane l supplies A[m][k] and B[k][m] for the same eight k of its group g):
//   scores  token slot i, row j.  k-step s (D/32 of them) of lane group g
//           takes the key coordinates (D/4) g + 8 s + v (v = 0..7) of token
//           16 tg + m; the codes are spread into bytes (twice the code per
//           byte) and turned into byte selectors of a v_perm over the
//           4-entry centroid table (bf16 entry c at bytes 2c, 2c+1), for the
//           hi and the lo pieces.  The QJL term of k-step s takes sign word
//           s / 4 of the lane's D/4 coordinates and pairs its bits
//           (4 (s % 4) + e, +16), so one shift and one mask make the pair of
//           bf16 +-1.  Output: lane (m, g) holds the scores of tokens
//           16 tg + 4 g + r (r = 0..3) for row m, kept as two sums (MSE and
//           QJL) that the token's n and gamma scale afterwards.
//   values  coordinate slot i, row j, k = token: the 32 tokens of half h are
//           the ones whose probabilities the lane already holds (16 tg + 4 g
//           + r, tg = 2h, 2h + 1), so the probabilities never move between
//           lanes; lane m owns the coordinates (D/16) m .. (D/16) m + D/16 - 1,
//           one contiguous run of the token's packed value codes, inside one
//           32-coordinate group.  MSE values: the centroids come from a
//           16-entry (hi | lo << 16) table in LDS.  Group values: the lane
//           builds, per token, the 4-entry table q s + mn of its group (hi
//           and lo pieces, two dwords each) and looks two coordinates of the
//           run up at once with one v_perm per piece.
//
// One 256-thread workgroup per (chunk, KV head, sequence); wave w takes the
// 64-token tiles w, w + 4, ... of the chunk with its own online softmax; the
// four waves' (m, l, o) are combined in LDS (the query operands' space,
// reused once the tiles are done) into the chunk's partial, which the
// general path's merge kernel merges across chunks.
#include "chunk_order.h"
#include "codes3.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStep = 256;  // chunks are multiples of this many tokens
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFlushGap = 8.f;  // log2 headroom of the lazy softmax reference
constexpr float kQMax = 8355711.f;  // three-digit query bound (2^23 - 0x8081)

__device__ __forceinline__ v4f mfma(const v4u& a, const v4u& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

__device__ __forceinline__ v4i mfma8(const v4i& a, const v4i& b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Coordinate (within a lane group's D/4) of byte f = 4 e + b of the int8
// K-step ks fragments: the key selectors below put the codes in this order.
template <int KB>
__device__ __forceinline__ int kstep_coord(int ks, int e, int b) {
  if constexpr (KB == 3) return 16 * ks + 4 * e + b;
  if constexpr (KB == 2) return 16 * ks + 4 * b + e;
  return 32 * (ks >> 1) + 8 * b + 4 * (ks & 1) + e;
}

// int8 K-step ks selectors of a lane's key words: byte b of dword e is the
// code of coordinate kstep_coord(ks, e, b)
template <int KB>
__device__ __forceinline__ uint32_t key_sel8(const uint32_t* w, int ks, int e) {
  if constexpr (KB == 3) {
    // K-steps 2 j and 2 j + 1 take the two halves of 32-coordinate group j
    uint32_t s[8];
    selectors3(w[3 * (ks >> 1)], w[3 * (ks >> 1) + 1], w[3 * (ks >> 1) + 2], s);
    return s[4 * (ks & 1) + e];
  }
  if constexpr (KB == 2) return (w[ks] >> (2 * e)) & 0x03030303u;
  return (w[ks >> 1] >> (4 * (ks & 1) + e)) & 0x01010101u;
}

// key_sel8 at a run-time K-step ks < KS8: every K-step's selectors with
// compile-time indices, then a select (a register array takes no run-time
// index without going through scratch memory)
template <int KB, int KS8>
__device__ __forceinline__ uint32_t key_sel8_rt(const uint32_t* w, int ks, int e) {
  uint32_t x = 0u;
#pragma unroll
  for (int kk = 0; kk < KS8; ++kk) {
    const uint32_t y = key_sel8<KB>(w, kk, e);
    x = kk == ks ? y : x;
  }
  return x;
}

// A value loaded from a valid address (the caller clamps it), or zero; the
// load itself is unconditional.
template <class T>
__device__ __forceinline__ T pick(T v, bool ok) {
  return ok ? v : T(0);
}

// The T at a byte offset from a base pointer.
template <class T>
__device__ __forceinline__ T ld(const char* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

// A raw buffer resource over `bytes` bytes from `base`: loads at offsets
// past the end return zero without touching memory.
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, gfx9 data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint32_t bld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float bldf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// bf16 bits of x, rounded to nearest even (finite x)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_rne(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}

// (hi, lo) pairs of two split values, element a in the low half
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  uint32_t ha, la, hb, lb;
  split_rne(a, ha, la);
  split_rne(b, hb, lb);
  hi = ha | (hb << 16);
  lo = la | (lb << 16);
}

// maximum over the four 16-lane groups (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float rowmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// v_perm selector of two entries of a 4-entry bf16 table (entry c at bytes
// 2c, 2c+1 of the 8-byte pool): the 2-bit codes of run coordinates u (low
// half of the result) and u + NU/2 (high half); run = the lane's codes from
// bit 0, NU of them
template <int NU>
__device__ __forceinline__ uint32_t pair_selector(uint32_t run, int u) {
  if constexpr (NU == 16) {
    // the two codes sit 16 bits apart: bytes 0 and 2 after one shift and mask
    return ((run >> (2 * u)) & 0x00030003u) * 0x0202u + 0x01000100u;
  } else {
    const uint32_t a = (run >> (2 * u)) & 3u, b = (run >> (2 * u + NU)) & 3u;
    return a * 0x0202u + b * 0x02020000u + 0x01000100u;
  }
}

// 3-bit values (byte-lane layout, 32 coordinates in words X, Y, Z): lane
// slot i at value step u takes coordinate 32 G + 4 (u % 8) + i % 4 of the
// cache, G = i / 4 at head_dim 128 and 2 (i / 4) + u / 8 at 256 -- byte i % 4
// of selector dword u % 8 of one group, so every lane extracts its codes
// with the same instructions at a lane-dependent bit offset.
template <int D>
__device__ __forceinline__ int coord3(int i, int u) {
  const int grp = D == 128 ? i / 4 : 2 * (i / 4) + u / 8;
  return 32 * grp + 4 * (u % 8) + (i % 4);
}

// 4 x the code of selector dword q (a compile-time constant), byte k, of a
// 3-bit byte-lane group; kb = 8 k
__device__ __forceinline__ uint32_t code3x4(uint32_t X, uint32_t Y, uint32_t Z, int q, uint32_t kb) {
  switch (q) {
    case 0: return __builtin_amdgcn_ubfe(X, kb, 3) << 2;
    case 1: return __builtin_amdgcn_ubfe(X, kb + 3, 3) << 2;
    case 2: return (__builtin_amdgcn_ubfe(X, kb + 6, 2) << 2) | (__builtin_amdgcn_ubfe(Z, kb + 6, 1) << 4);
    case 3: return __builtin_amdgcn_ubfe(Y, kb, 3) << 2;
    case 4: return __builtin_amdgcn_ubfe(Y, kb + 3, 3) << 2;
    case 5: return (__builtin_amdgcn_ubfe(Y, kb + 6, 2) << 2) | (__builtin_amdgcn_ubfe(Z, kb + 7, 1) << 4);
    case 6: return __builtin_amdgcn_ubfe(Z, kb, 3) << 2;
    default: return __builtin_amdgcn_ubfe(Z, kb + 3, 3) << 2;
  }
}

template <int D, int KB, int VB, bool PROD, bool VGROUP>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_bf16_kernel(DecodeParams p) {
  constexpr int KS = D / 32;          // bf16 k-steps of the QJL product
  constexpr int KS8 = D / 64;         // int8 K-steps of the MSE product
  constexpr int LC = D / 4;           // key coordinates of a lane group
  constexpr int KW = KB * LC / 32;    // key index words of a lane group's coordinates
  constexpr int SW = LC / 32;         // QJL sign words of them
  constexpr int NU = D / 16;          // value coordinates per lane
  constexpr bool V3 = VB == 3;        // 3-bit MSE values (byte-lane groups)
  constexpr int VRB = NU * VB;        // bits of a lane's value run (8 .. 64)
  // words of it (3-bit values: the lane's one or two whole 32-coordinate groups)
  constexpr int VW = V3 ? 3 * (D / 128) : (VRB + 31) / 32;
  constexpr uint32_t VMASK = (1u << VB) - 1u;
  // 16-token groups of a wave's tile: 64 tokens at head_dim 128, 32 at 256
  // (the wider head's operands and accumulators leave registers for half as
  // many tokens at two waves per SIMD); NT of them per lane
  constexpr int TG = D == 128 ? 4 : 2;
  constexpr int kTile = 16 * TG;
  constexpr int NT = 4 * TG;
  static_assert(D == 128 || D == 256, "head_dim 128 or 256");
  static_assert(kStep % (kWaves * kTile) == 0, "chunks hold whole workgroup steps");
  static_assert(!VGROUP || VB == 2, "group values of 2 bits");
  // the query operands during the tiles (int8 digits, then the QJL pieces),
  // the waves' partial outputs after them
  constexpr int kQdBytes = KS8 * 3 * 64 * 16;
  constexpr int kQopBytes = kQdBytes + (PROD ? KS * 2 * 64 * 16 : 0);
  // the waves' outputs: kRows rows of kRS floats, coordinate j at
  // j + 16 (j / GW) (GW = 4 NU coordinates per lane group): kRS = 1 mod 64
  // and the 16-float step per lane group put the 64 lanes of one store
  // (row m, lane group g) in 64 different banks
  constexpr int kRows = D == 128 ? 16 : 8;
  constexpr int GW = 4 * NU;
  constexpr int kRS = ((D + 48 - 1) / 64 + 1) * 64 + 1;
  constexpr int kOutBytes = kWaves * kRows * kRS * 4;
  constexpr int kRawBytes = kQopBytes > kOutBytes ? kQopBytes : kOutBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawBytes];
  __shared__ uint32_t s_vt[16];           // MSE value centroid c: bf16 hi | lo << 16
  __shared__ float s_ml[kWaves][16][2];   // the waves' (m, l) per row
  v4i* s_qd = reinterpret_cast<v4i*>(s_raw);                 // [K-step][digit a, b, c][lane]
  v4u* s_qop = reinterpret_cast<v4u*>(s_raw + kQdBytes);     // [k-step][S q hi, S q lo][lane]
  float* s_o = reinterpret_cast<float*>(s_raw);   // [wave][row][kRS]

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
  const int lim_all = lenm - p.q_len + 1 - c0;                           // tokens every row sees

  if constexpr (!VGROUP) {
    if (threadIdx.x < 16) {
      uint32_t hi = 0, lo = 0;
      if (threadIdx.x <= VMASK) split_rne(p.v_cent[threadIdx.x], hi, lo);
      s_vt[threadIdx.x] = hi | (lo << 16);
    }
  }
  const float qjl = p.scale * kLog2e * kQjlConstNumer / (float)D;  // log2-domain QJL factor
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)c0;  // slot of token 0 of the chunk
  // the chunk's fields (uniform bases); a token index t < ntok (< 2^24)
  // addresses them with 24-bit products and 32-bit byte offsets
  const char* kidx = reinterpret_cast<const char*>(p.k_idx + base * p.kwords);
  const char* ksgn = PROD ? reinterpret_cast<const char*>(p.k_sign + base * p.ksign_words) : nullptr;
  const char* knrm = reinterpret_cast<const char*>(p.k_norm + base);
  const char* krnm = PROD ? reinterpret_cast<const char*>(p.k_rnorm + base) : nullptr;
  const char* vnrm = VGROUP ? nullptr : reinterpret_cast<const char*>(p.v_norm + base);
  const char* vscl = VGROUP ? reinterpret_cast<const char*>(p.v_scale + base * p.vgroups) : nullptr;
  const char* vmin = VGROUP ? reinterpret_cast<const char*>(p.v_gmin + base * p.vgroups) : nullptr;
  const char* vidx = reinterpret_cast<const char*>(p.v_idx + base * p.vwords);
  const uint32_t kstride = 4u * p.kwords, sstride = 4u * p.ksign_words, vstride = 4u * p.vwords;
  const uint32_t gstride = 4u * p.vgroups;
  const uint32_t koff = 4u * g * KW, soff = 4u * g * SW;
  const uint32_t voff = V3 ? 12u * (uint32_t)((D / 128) * (m / 4)) : 4u * ((m * VRB) >> 5);
  const uint32_t goff = 4u * ((m * NU) >> 5);  // the group of the lane's value run
  const int vshift = (m * VRB) & 31;
  // the chunk's fields as buffer resources that end at its last token
  const uint32_t nt = ntok > 0 ? (uint32_t)ntok : 0u;
  const __amdgpu_buffer_rsrc_t rki = rsrc(kidx, nt * kstride);
  const __amdgpu_buffer_rsrc_t rks = rsrc(PROD ? ksgn : kidx, PROD ? nt * sstride : 0u);
  const __amdgpu_buffer_rsrc_t rkn = rsrc(knrm, nt * 4u);
  const __amdgpu_buffer_rsrc_t rkr = rsrc(PROD ? krnm : knrm, PROD ? nt * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rvn = rsrc(VGROUP ? vidx : vnrm, VGROUP ? 0u : nt * 4u);
  const __amdgpu_buffer_rsrc_t rvs = rsrc(VGROUP ? vscl : vidx, VGROUP ? nt * gstride : 0u);
  const __amdgpu_buffer_rsrc_t rvm = rsrc(VGROUP ? vmin : vidx, VGROUP ? nt * gstride : 0u);
  const __amdgpu_buffer_rsrc_t rvi = rsrc(vidx, nt * vstride);

  // ---- tile loads, one tile ahead of their use.  Key words of token T0 +
  // 16 tg + m, coordinates (D/4) g .. (D/4) g + D/4 - 1; key norms and value
  // fields of the lane's tokens T0 + 16 tg + 4 g + r (token i: tg = i / 4,
  // r = i % 4).  Tokens past the chunk's end read zeros, without touching
  // memory; their scores are masked, so they weigh nothing.
  uint32_t nkw[TG][KW], nksw[TG][SW];
  float kn[NT], kq[NT], vn[NT], vs[NT];
  uint32_t vw[NT][VW];
  auto load_keys = [&](int T0) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const uint32_t t = (uint32_t)(T0 + 16 * tg + m);
#pragma unroll
      for (int w = 0; w < KW; ++w) nkw[tg][w] = bld(rki, __umul24(t, kstride) + koff + 4u * w);
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        nksw[tg][w] = 0u;
        if constexpr (PROD) nksw[tg][w] = bld(rks, __umul24(t, sstride) + soff + 4u * w);
      }
    }
  };
  auto load_fields = [&](int T0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint32_t t = (uint32_t)(T0 + 16 * (i >> 2) + 4 * g + (i & 3));
      kn[i] = bldf(rkn, 4u * t);
      kq[i] = 0.f;
      if constexpr (PROD) kq[i] = bldf(rkr, 4u * t) * qjl;
      if constexpr (VGROUP) {
        vs[i] = bldf(rvs, __umul24(t, gstride) + goff);
        vn[i] = bldf(rvm, __umul24(t, gstride) + goff);
      } else {
        vn[i] = bldf(rvn, 4u * t);
        vs[i] = 0.f;
      }
#pragma unroll
      for (int w = 0; w < VW; ++w) vw[i][w] = bld(rvi, __umul24(t, vstride) + voff + 4u * w);
    }
  };

  // ---- the prologue's reads of the query rows first, then the first
  // tile's key words: loads complete in issue order, so the prologue waits
  // for its own reads alone and the key words arrive while it computes
  const bool rok = m < rows;
  const size_t qoff = ((size_t)bg * rows + (rok ? m : 0)) * D + LC * g;
  // (16-byte reads: the rows are 16-byte aligned)
  float qv[LC];
#pragma unroll
  for (int c = 0; c < LC; c += 4) {
    const v4f x = *reinterpret_cast<const v4f*>(p.qrot + qoff + c);
#pragma unroll
    for (int t = 0; t < 4; ++t) qv[c + t] = x[t];
  }
  // this wave's QJL k-steps s = wave + 4 j: coordinates 32 j + 4 wave + e and + 16
  constexpr int KSW = (KS + kWaves - 1) / kWaves;
  float qsv[KSW][4][2];
#pragma unroll
  for (int jj = 0; jj < KSW; ++jj)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      v4f x = v4f{0.f, 0.f, 0.f, 0.f};
      if constexpr (PROD) x = *reinterpret_cast<const v4f*>(p.qs + qoff + 32 * jj + 4 * wave + 16 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) qsv[jj][e][hh] = x[e];
    }
  __builtin_amdgcn_sched_barrier(0);
  load_keys(wave * kTile);
  __builtin_amdgcn_sched_barrier(0);

  // key centroid pieces: centroid c * 2^E = 256 hi + lo (int8 hi, lo),
  // entries 0..3 in the bytes of one dword each
  // (up to 8 entries: the high dwords hold entries 4..7 of 3-bit codes)
  const uint32_t kth = p.klut[0], ktl = p.klut[2], kth1 = KB == 3 ? p.klut[1] : 0u, ktl1 = KB == 3 ? p.klut[3] : 0u;
  // Query operands, the same for every wave, in LDS.  MSE term: row m of
  // q_rot quantised to 24 bits, q = round(q_rot sc) = 65536 a + 256 b + c
  // with balanced int8 digits, sc = kQMax / max_j |q_rot[m][j]|; byte f =
  // 4 e + b of K-step ks is coordinate (D/4) g + kstep_coord(ks, e, b).  QJL
  // term: (S q_rot)[(D/4) g + 32 (s/4) + 4 (s%4) + e] and [.. + 16] as the
  // bf16 pair e (hi, lo) of k-step s.  Every wave finds the row maximum; wave
  // w writes the K-steps and k-steps w, w + 4, ...
  float rowc;  // log2-domain score per unit of 2^16 t24 + 2^8 t16 + t8, 0 for a zero row
  {
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < LC; ++c) mx = fmaxf(mx, fabsf(qv[c]));
    mx = rok ? rowmax4(mx) : 0.f;
    const float sc = mx > 0.f ? kQMax / mx : 0.f;
    // (with the log2-domain score scale folded in)
    rowc = mx > 0.f ? p.scale * kLog2e * 256.f * exp2f(-(float)p.kgrid) / sc : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
      if (ks % kWaves != wave) continue;
      v4i da, db, dc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t u[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // the product may round one past the bound: clamp so the top digit fits
          const float q = rok ? qv[kstep_coord<KB>(ks, e, bb)] : 0.f;
          const float x = fminf(fmaxf(rintf(q * sc), -kQMax), kQMax);
          u[bb] = (uint32_t)((int)x + 0x808080);  // bytes 2, 1, 0: a, b, c, each + 128
        }
        const uint32_t lo01 = perm(u[1], u[0], 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
        const uint32_t lo23 = perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = perm(u[1], u[0], 0x0c0c0602u);  // u0.b2 u1.b2 0 0
        const uint32_t hi23 = perm(u[3], u[2], 0x0c0c0602u);
        da[e] = (int)(perm(hi23, hi01, 0x05040100u) ^ 0x80808080u);
        db[e] = (int)(perm(lo23, lo01, 0x07060302u) ^ 0x80808080u);
        dc[e] = (int)(perm(lo23, lo01, 0x05040100u) ^ 0x80808080u);
      }
      s_qd[(3 * ks + 0) * 64 + lane] = da;
      s_qd[(3 * ks + 1) * 64 + lane] = db;
      s_qd[(3 * ks + 2) * 64 + lane] = dc;
    }
  }
  if constexpr (PROD) {
#pragma unroll
    for (int jj = 0; jj < KSW; ++jj) {
      const int s = wave + kWaves * jj;
      if (s >= KS) continue;
      v4u ch, cl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t h, l;
        split_pair(rok ? qsv[jj][e][0] : 0.f, rok ? qsv[jj][e][1] : 0.f, h, l);
        ch[e] = h;
        cl[e] = l;
      }
      s_qop[(2 * s + 0) * 64 + lane] = ch;
      s_qop[(2 * s + 1) * 64 + lane] = cl;
    }
  }
  // the first tile's other fields (the wait counter tracks at most 63 loads:
  // issued after the prologue's waits, they do not hold them up)
  load_fields(wave * kTile);
  __syncthreads();

  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int T0 = wave * kTile; T0 < ntok; T0 += kWaves * kTile) {
    uint32_t kw[TG][KW], ksw[TG][SW];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
      for (int w = 0; w < KW; ++w) kw[tg][w] = nkw[tg][w];
#pragma unroll
      for (int w = 0; w < SW; ++w) ksw[tg][w] = nksw[tg][w];
    }
    // the next tile's key words (the last tile's reads of the chunk's last
    // token are never used)
    load_keys(T0 + kWaves * kTile);
    uint32_t run[NT][VW];  // the value runs of this tile, from bit 0
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int w = 0; w < VW; ++w) run[i][w] = (VW == 1 && !V3) ? vw[i][w] >> vshift : vw[i][w];

    // ---- scores.  MSE term on the int8 matrix cores: sm[tg][i] = rowc (2^16
    // t24 + 2^8 t16 + t8), exact integer digit products; the query operands
    // of K-step ks + 1 are read while K-step ks computes, and the scheduling
    // barriers keep the compiler from hoisting every step's reads (their
    // registers) to the top
    v4f sm[TG], sq[TG];
    {
      v4i t24[TG], t16[TG], t8[TG];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) t24[tg] = t16[tg] = t8[tg] = v4i{0, 0, 0, 0};
      v4i na = s_qd[0 * 64 + lane], nb = s_qd[1 * 64 + lane], nc = s_qd[2 * 64 + lane];
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const v4i qa = na, qb = nb, qc = nc;
        if (ks + 1 < KS8) {
          na = s_qd[(3 * ks + 3) * 64 + lane];
          nb = s_qd[(3 * ks + 4) * 64 + lane];
          nc = s_qd[(3 * ks + 5) * 64 + lane];
        }
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          v4i ah, al;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = key_sel8<KB>(kw[tg], ks, e);
            ah[e] = (int)perm(kth1, kth, x);
            al[e] = (int)perm(ktl1, ktl, x);
          }
          // Q C = 2^24 a Ch + 2^16 (a Cl + b Ch) + 2^8 (b Cl + c Ch) [+ c Cl,
          // below 2^-23 of the product]
          t24[tg] = mfma8(ah, qa, t24[tg]);
          t16[tg] = mfma8(al, qa, t16[tg]);
          t8[tg] = mfma8(al, qb, t8[tg]);
          t16[tg] = mfma8(ah, qb, t16[tg]);
          t8[tg] = mfma8(ah, qc, t8[tg]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // 2^8 t16 + t8 stays below 2^31 (|t16|, |t8| <= D 64 128 + D 128 128)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lo = (int)(((uint32_t)t16[tg][i] << 8) + (uint32_t)t8[tg][i]);
          sm[tg][i] = rowc * fmaf(65536.f, (float)t24[tg][i], (float)lo);
        }
    }
    // QJL term on the bf16 matrix cores (the signs are exact in bf16)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) sq[tg] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (PROD) {
      // the sign-bit mask in a register, so that mask and +1.0 bits make one
      // v_and_or_b32 (its three-operand form takes no literal constant)
      uint32_t sgn = 0x80008000u;
      asm volatile("" : "+v"(sgn));
      v4u nch = s_qop[0 * 64 + lane], ncl = s_qop[1 * 64 + lane];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v4u ch = nch, cl = ncl;
        if (s + 1 < KS) {
          nch = s_qop[(2 * s + 2) * 64 + lane];
          ncl = s_qop[(2 * s + 3) * 64 + lane];
        }
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          const uint32_t ns = ~ksw[tg][s >> 2];
          v4u as;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // bits k and k + 16 of the negated signs become the bf16 sign bits
            const int k = 4 * (s & 3) + e;
            as[e] = ((ns << (15 - k)) & sgn) | 0x3f803f80u;
          }
          sq[tg] = mfma(as, ch, sq[tg]);
          sq[tg] = mfma(as, cl, sq[tg]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax of row m over this lane's NT tokens
    float sc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
      sc[i] = PROD ? fmaf(kn[i], sm[i >> 2][i & 3], kq[i] * sq[i >> 2][i & 3]) : kn[i] * sm[i >> 2][i & 3];
    if (!(T0 + kTile <= ntok && T0 + kTile <= lim_all)) {
      // a tile with masked tokens (the chunk's end, the causal edge); the
      // empty asm statement keeps the selects behind the wave-uniform branch
      asm volatile("");
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int tok = T0 + 16 * (i >> 2) + 4 * g + (i & 3);
        if (!(tok < ntok && tok < lim)) sc[i] = -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) tmax = fmaxf(tmax, sc[i]);
    tmax = rowmax4(tmax);
    if (__ballot(tmax > m_ref + kFlushGap) != 0) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] *= alpha;
      l_run *= alpha;
      m_ref = m_new;
    }
    float pv[NT];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      // the hardware exp2: arguments are at most kFlushGap, or -inf (masked)
      const float pr = __builtin_amdgcn_exp2f(sc[i] - m_ref);
      psum += pr;
      pv[i] = VGROUP ? pr : pr * vn[i];
    }
    l_run += psum;

    // ---- values: half h takes the tokens i = 8 h .. 8 h + 7 of the lane
#pragma unroll
    for (int h = 0; h < TG / 2; ++h) {
      v4u bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = __float_as_uint(pv[8 * h + 2 * e]), c = __float_as_uint(pv[8 * h + 2 * e + 1]);
        bh[e] = perm(c, a, 0x07060302u);
        const float ra = pv[8 * h + 2 * e] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[8 * h + 2 * e + 1] - __uint_as_float(c & 0xffff0000u);
        bl[e] = perm(__float_as_uint(rc), __float_as_uint(ra), 0x07060302u);
      }
      if constexpr (VGROUP) {
        // the 4-entry table q s + mn of each token's group: entries 0, 1 in
        // the low dword, 2, 3 in the high one, hi and lo pieces apart
        uint32_t th[8][2], tl[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = vs[8 * h + i], mn = vn[8 * h + i];
          split_pair(mn, mn + sg, th[i][0], tl[i][0]);
          split_pair(fmaf(2.f, sg, mn), fmaf(3.f, sg, mn), th[i][1], tl[i][1]);
        }
#pragma unroll
        for (int u = 0; u < NU / 2; ++u) {
          // coordinates u and u + NU/2 of the run, for the token pairs e
          v4u ah0, al0, ah1, al1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ia = 2 * e, ib = 2 * e + 1;
            const uint32_t sa = pair_selector<NU>(run[8 * h + ia][0], u);
            const uint32_t sb = pair_selector<NU>(run[8 * h + ib][0], u);
            const uint32_t xa = perm(th[ia][1], th[ia][0], sa), xb = perm(th[ib][1], th[ib][0], sb);
            const uint32_t ya = perm(tl[ia][1], tl[ia][0], sa), yb = perm(tl[ib][1], tl[ib][0], sb);
            ah0[e] = perm(xb, xa, 0x05040100u);
            ah1[e] = perm(xb, xa, 0x07060302u);
            al0[e] = perm(yb, ya, 0x05040100u);
            al1[e] = perm(yb, ya, 0x07060302u);
          }
          acc[u] = mfma(ah0, bh, acc[u]);
          acc[u] = mfma(ah0, bl, acc[u]);
          acc[u] = mfma(al0, bh, acc[u]);
          acc[u + NU / 2] = mfma(ah1, bh, acc[u + NU / 2]);
          acc[u + NU / 2] = mfma(ah1, bl, acc[u + NU / 2]);
          acc[u + NU / 2] = mfma(al1, bh, acc[u + NU / 2]);
        }
      } else if constexpr (V3) {
        // 3-bit values: slot m's code at step u (coord3) from its group's
        // words, as an LDS byte offset (4 x the code) into the centroid table
        const uint32_t kb = 8u * (uint32_t)(m & 3);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int w0 = 3 * (u / 8);
          v4u ah, al;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t* xa = run[8 * h + 2 * e];
            const uint32_t* xc = run[8 * h + 2 * e + 1];
            const uint32_t oa = code3x4(xa[w0], xa[w0 + 1], xa[w0 + 2], u % 8, kb);
            const uint32_t oc = code3x4(xc[w0], xc[w0 + 1], xc[w0 + 2], u % 8, kb);
            const uint32_t ta = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oa);
            const uint32_t tc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oc);
            ah[e] = perm(tc, ta, 0x05040100u);
            al[e] = perm(tc, ta, 0x07060302u);
          }
          acc[u] = mfma(ah, bh, acc[u]);
          acc[u] = mfma(ah, bl, acc[u]);
          acc[u] = mfma(al, bh, acc[u]);
        }
      } else {
        // LDS byte offsets of the value codes: byte k of va[i][w][t] is 4 x
        // the code of run coordinate (32 w + 8 k) / VB + t of token i
        constexpr int TPB = 8 / VB;
        uint32_t va[8][VW][TPB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int w = 0; w < VW; ++w)
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
              const int sh = 2 - VB * t;
              const uint32_t x = run[8 * h + i][w];
              va[i][w][t] = (sh >= 0 ? (x << sh) : (x >> -sh)) & (0x01010101u * (VMASK << 2));
            }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          constexpr int kBitsPerWord = 32;
          const int bit = u * VB, w = bit / kBitsPerWord, byte = (bit % kBitsPerWord) / 8;
          v4u ah, al;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // byte `byte`, zero-extended (selector 0x0c gives a zero byte)
            const uint32_t bsel = 0x0c0c0c00u + (uint32_t)byte;
            const uint32_t oa = perm(0u, va[2 * e][w][u % TPB], bsel);
            const uint32_t oc = perm(0u, va[2 * e + 1][w][u % TPB], bsel);
            const uint32_t ta = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oa);
            const uint32_t tc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oc);
            ah[e] = perm(tc, ta, 0x05040100u);
            al[e] = perm(tc, ta, 0x07060302u);
          }
          acc[u] = mfma(ah, bh, acc[u]);
          acc[u] = mfma(ah, bl, acc[u]);
          acc[u] = mfma(al, bh, acc[u]);
        }
      }
    }
    // the next tile's key norms and value fields (into registers whose
    // contents this tile no longer needs)
    load_fields(T0 + kWaves * kTile);
  }

  // ---- the workgroup's partial: the four waves' (m, l, o) of each row,
  // rescaled to their common maximum and summed through LDS (over the query
  // operands, which every wave has finished with at the barrier)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  if (g == 0) {
    s_ml[wave][m][0] = m_ref;
    s_ml[wave][m][1] = l_run;
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = V3 ? coord3<D>(4 * g + r, u) : (4 * g + r) * NU + u;
      if (m < rows) s_o[(wave * kRows + m) * kRS + j + 16 * (j / GW)] = acc[u][r];
    }
  __syncthreads();
  float* po = p.part_o + ((size_t)bg * gridDim.x + chunk_id) * rows * D;
  for (int e = threadIdx.x; e < rows * D; e += kWaves * 64) {
    const int r = e / D, j = e % D;
    float mx = s_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][r][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      o = fmaf(s_o[(w * kRows + r) * kRS + j + 16 * (j / GW)], exp2f(s_ml[w][r][0] - mx), o);
    po[e] = o;
  }
  if (threadIdx.x < rows) {
    const int r = threadIdx.x;
    float mx = s_ml[0][r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_ml[w][r][0]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l = fmaf(s_ml[w][r][1], exp2f(s_ml[w][r][0] - mx), l);
    float* pml = p.part_ml + (((size_t)bg * gridDim.x + chunk_id) * rows + r) * 2;
    pml[0] = mx;
    pml[1] = l;
  }
}

// ---- prefill: many query rows over shared tiles ------------------------------
//
// A launch with more query rows per KV head than the decode kernel takes
// would expand every tile's codes once per 16 rows.  Here the waves of a
// workgroup each own 16 rows of the same KV head and walk the chunk's tiles
// together: eight waves over 64-token tiles at head_dim 128, four waves over
// 32-token tiles at head_dim 256 (the same operand bytes per tile, so two
// tile buffers fit in LDS either way; and at head_dim 256 the wave's query
// operands and value accumulators take twice the registers, which four waves
// of 512 leave room for).  A tile's operands come in eight key pieces (token
// group, K-step), sixteen QJL sign operands (token group, k-step) and sixteen
// value operands (half, coordinate); wave w expands its equal share of each
// -- the ones the decode kernel's lanes build for themselves -- into one of
// two LDS buffers, and wave 0 the tile's per-token norms; after one barrier
// every wave runs its own rows' products, softmax and value products over all
// of them.  A wave that reaches the barrier of tile t has finished with tile
// t-1's buffer, which the expansion of tile t+1 (after that barrier) then
// overwrites.  The rows' operands (int8 query digits, the QJL pieces) come
// from qprep_kernel's rotated rows and stay in registers; each wave writes
// its rows' partial (m, l, o) for the chunk, merged by merge_kernel.
template <int D>
struct PbShape {
  static constexpr int kWaves = D == 128 ? 8 : 4;
  static constexpr int kRows = kWaves * 16;   // rows per workgroup
  static constexpr int TG = D == 128 ? 4 : 2; // 16-token groups per tile
};

template <int D, int KB, int VB, bool PROD, bool VGROUP>
struct PbLayout {
  static constexpr int KS = D / 32, KS8 = D / 64, TG = PbShape<D>::TG, kTile = 16 * TG, NU = D / 16;
  static constexpr int kKey = TG * KS8 * 2 * 64 * 16;             // [tg][ks][hi, lo][lane] v4i
  static constexpr int kQjl = PROD ? TG * KS * 64 * 16 : 0;       // [tg][s][lane] v4u
  static constexpr int kVal = (TG / 2) * NU * 2 * 64 * 16;        // [h][u][hi, lo][lane] v4u
  static constexpr int kFld = 3 * kTile * 4;                      // kn, kq, vn per token
  static constexpr int kBuf = kKey + kQjl + kVal + kFld;
  static_assert(TG * KS8 == 8 && TG * KS == 16 && (TG / 2) * NU == 16, "operand pieces per tile");
};

template <int D, int KB, int VB, bool PROD, bool VGROUP>
__global__ __launch_bounds__(PbShape<D>::kWaves * 64, 1) void prefill_bf16_kernel(DecodeParams p) {
  using Lay = PbLayout<D, KB, VB, PROD, VGROUP>;
  constexpr int kPbWaves = PbShape<D>::kWaves, kPbRows = PbShape<D>::kRows;
  constexpr int KS = Lay::KS, KS8 = Lay::KS8, TG = Lay::TG, kTile = Lay::kTile, NU = Lay::NU;
  constexpr int LC = D / 4;
  constexpr int KW = KB * LC / 32;
  constexpr int SW = LC / 32;
  constexpr int NT = 4 * TG;
  constexpr int VRB = NU * VB;
  constexpr bool V3 = VB == 3;  // 3-bit MSE values (byte-lane groups, the decode kernel's coord3 slots)
  constexpr int VW = V3 ? 3 * (D / 128) : (VRB + 31) / 32;
  constexpr uint32_t VMASK = (1u << VB) - 1u;
  constexpr int kBuf = Lay::kBuf;
  static_assert(!VGROUP || VB == 2, "group values of 2 bits");
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[2 * kBuf];
  __shared__ uint32_t s_vt[16];  // MSE value centroid c: bf16 hi | lo << 16

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int chunk_id = rotated_chunk(blockIdx.x % p.n_chunks, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int rg = blockIdx.x / p.n_chunks;
  const int gh = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + gh;
  const int rows = p.rows;
  const int rl = rg * kPbRows + wave * 16 + m;  // this lane's row among the launch's rows
  const bool rok = rl < rows;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int ntok = (c0 + p.chunk < len ? c0 + p.chunk : len) - c0;  // may be <= 0
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;
  const int lim = lenm - p.q_len + ((p.row0 + rl) % p.q_len) + 1 - c0;  // row rl sees tokens < lim
  const int lim_all = lenm - p.q_len + 1 - c0;                            // tokens every row sees

  if constexpr (!VGROUP) {
    if (threadIdx.x < 16) {
      uint32_t hi = 0, lo = 0;
      if (threadIdx.x <= VMASK) split_rne(p.v_cent[threadIdx.x], hi, lo);
      s_vt[threadIdx.x] = hi | (lo << 16);
    }
  }
  const float qjl = p.scale * kLog2e * kQjlConstNumer / (float)D;
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)(c0 > 0 ? c0 : 0);
  const char* kidx = reinterpret_cast<const char*>(p.k_idx + base * p.kwords);
  const char* ksgn = PROD ? reinterpret_cast<const char*>(p.k_sign + base * p.ksign_words) : nullptr;
  const char* knrm = reinterpret_cast<const char*>(p.k_norm + base);
  const char* krnm = PROD ? reinterpret_cast<const char*>(p.k_rnorm + base) : nullptr;
  const char* vnrm = VGROUP ? nullptr : reinterpret_cast<const char*>(p.v_norm + base);
  const char* vscl = VGROUP ? reinterpret_cast<const char*>(p.v_scale + base * p.vgroups) : nullptr;
  const char* vmin = VGROUP ? reinterpret_cast<const char*>(p.v_gmin + base * p.vgroups) : nullptr;
  const char* vidx = reinterpret_cast<const char*>(p.v_idx + base * p.vwords);
  const uint32_t kstride = 4u * p.kwords, sstride = 4u * p.ksign_words, vstride = 4u * p.vwords;
  const uint32_t gstride = 4u * p.vgroups;
  const uint32_t koff = 4u * g * KW, soff = 4u * g * SW, voff = V3 ? 12u * (uint32_t)((D / 128) * (m / 4)) : 4u * ((m * VRB) >> 5);
  const uint32_t goff = 4u * ((m * NU) >> 5);
  const int vshift = (m * VRB) & 31;
  // a token index of the chunk, clamped to a valid one (tokens past the end
  // are read from the last token, or token 0 of an empty chunk, and masked)
  auto tok = [&](int t) -> uint32_t { return (uint32_t)max(min(t, ntok - 1), 0); };

  // ---- this wave's share of the expansion: of the tile's pieces numbered
  // (tg, ks), (tg, s) and (h, u) in that order, the KJ key pieces, QJ QJL
  // operands and VJ value operands from wave x the count (one token group or
  // half, and for the QJL operands one sign word, per wave); group values go
  // by pairs (u, u + NU/2), GJ of them
  constexpr int KJ = 8 / kPbWaves, QJ = 16 / kPbWaves, VJ = 16 / kPbWaves, GJ = VJ / 2;
  const int ktg = wave * KJ / KS8, kks0 = wave * KJ % KS8;
  const bool early = kPbWaves == 8 && (wave & 4) != 0;  // expands before its products
  const bool late = kPbWaves == 8 && (wave & 4) == 0;   // after them
  const int qtg = wave * QJ / KS, qs0 = wave * QJ % KS;
  const int vh = wave * VJ / NU, vu0 = wave * VJ % NU;
  uint32_t rkw[KW], rsw = 0u;
  uint32_t rvw[8][VW];
  float rvs[8], rvm[8];
  float rfk = 0.f, rfq = 0.f, rfv = 0.f;
  auto stage_load = [&](int T0) {
    {
      const uint32_t t = tok(T0 + 16 * ktg + m);
#pragma unroll
      for (int w = 0; w < KW; ++w) rkw[w] = ld<uint32_t>(kidx, __umul24(t, kstride) + koff + 4u * w);
    }
    if constexpr (PROD) {
      const uint32_t t = tok(T0 + 16 * qtg + m);
      rsw = ld<uint32_t>(ksgn, __umul24(t, sstride) + soff + 4u * (qs0 >> 2));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t t = tok(T0 + 16 * (2 * vh + (i >> 2)) + 4 * g + (i & 3));
#pragma unroll
      for (int w = 0; w < VW; ++w) rvw[i][w] = ld<uint32_t>(vidx, __umul24(t, vstride) + voff + 4u * w);
      if constexpr (VGROUP) {
        rvs[i] = ld<float>(vscl, __umul24(t, gstride) + goff);
        rvm[i] = ld<float>(vmin, __umul24(t, gstride) + goff);
      }
    }
    if (wave == 0) {
      const uint32_t t = tok(T0 + (lane & (kTile - 1)));
      rfk = ld<float>(knrm, 4u * t);
      if constexpr (PROD) rfq = ld<float>(krnm, 4u * t) * qjl;
      if constexpr (!VGROUP) rfv = ld<float>(vnrm, 4u * t);
    }
  };
  const uint32_t kth = p.klut[0], ktl = p.klut[2], kth1 = KB == 3 ? p.klut[1] : 0u, ktl1 = KB == 3 ? p.klut[3] : 0u;
  auto stage_expand = [&](int T0) {
    uint8_t* buf = s_buf + ((T0 / kTile) & 1) * kBuf;
    v4i* kop = reinterpret_cast<v4i*>(buf);
    v4u* qop = reinterpret_cast<v4u*>(buf + Lay::kKey);
    v4u* vop = reinterpret_cast<v4u*>(buf + Lay::kKey + Lay::kQjl);
    float* fld = reinterpret_cast<float*>(buf + Lay::kKey + Lay::kQjl + Lay::kVal);
#pragma unroll
    for (int i = 0; i < KJ; ++i) {
      const int kks = kks0 + i;
      v4i ah, al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = KB == 3 ? key_sel8_rt<KB, KS8>(rkw, kks, e) : key_sel8<KB>(rkw, kks, e);
        ah[e] = (int)perm(kth1, kth, x);
        al[e] = (int)perm(ktl1, ktl, x);
      }
      kop[((ktg * KS8 + kks) * 2 + 0) * 64 + lane] = ah;
      kop[((ktg * KS8 + kks) * 2 + 1) * 64 + lane] = al;
    }
    if constexpr (PROD) {
      const uint32_t ns = ~rsw;
      uint32_t sgn = 0x80008000u;  // in a register: one v_and_or_b32 below
      asm volatile("" : "+v"(sgn));
#pragma unroll
      for (int j = 0; j < QJ; ++j) {
        const int s = qs0 + j;
        v4u as;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // bits k and k + 16 of the negated signs become the bf16 sign bits
          const int k = 4 * (s & 3) + e;
          as[e] = ((ns << (15 - k)) & sgn) | 0x3f803f80u;
        }
        qop[(qtg * KS + s) * 64 + lane] = as;
      }
    }
    uint32_t run[8][VW];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int w = 0; w < VW; ++w) run[i][w] = VW == 1 ? rvw[i][w] >> vshift : rvw[i][w];
    if constexpr (VGROUP) {
      uint32_t th[8][2], tl[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sg = rvs[i], mn = rvm[i];
        split_pair(mn, mn + sg, th[i][0], tl[i][0]);
        split_pair(fmaf(2.f, sg, mn), fmaf(3.f, sg, mn), th[i][1], tl[i][1]);
      }
      // coordinates u and u + NU/2 of the run, stored as (h, u) and
      // (h, u + NU/2)
#pragma unroll
      for (int j = 0; j < GJ; ++j) {
        const int u = (wave * GJ + j) % (NU / 2);
        v4u ah0, al0, ah1, al1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ia = 2 * e, ib = 2 * e + 1;
          const uint32_t sa = pair_selector<NU>(run[ia][0], u);
          const uint32_t sb = pair_selector<NU>(run[ib][0], u);
          const uint32_t xa = perm(th[ia][1], th[ia][0], sa), xb = perm(th[ib][1], th[ib][0], sb);
          const uint32_t ya = perm(tl[ia][1], tl[ia][0], sa), yb = perm(tl[ib][1], tl[ib][0], sb);
          ah0[e] = perm(xb, xa, 0x05040100u);
          ah1[e] = perm(xb, xa, 0x07060302u);
          al0[e] = perm(yb, ya, 0x05040100u);
          al1[e] = perm(yb, ya, 0x07060302u);
        }
        vop[((vh * NU + u) * 2 + 0) * 64 + lane] = ah0;
        vop[((vh * NU + u) * 2 + 1) * 64 + lane] = al0;
        vop[((vh * NU + u + NU / 2) * 2 + 0) * 64 + lane] = ah1;
        vop[((vh * NU + u + NU / 2) * 2 + 1) * 64 + lane] = al1;
      }
    } else if constexpr (V3) {
      // slot m's code at step u (coord3) from its group's words, as an LDS
      // byte offset (4 x the code) into the centroid table; u is the same on
      // every lane of the wave
      const uint32_t kb = 8u * (uint32_t)(m & 3);
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        const int u = vu0 + j;
        const bool g1 = D == 256 && u >= 8;  // a head_dim-256 lane's second group
        v4u ah, al;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t* xa = run[2 * e];
          const uint32_t* xc = run[2 * e + 1];
          uint32_t a0 = xa[0], a1 = xa[1], a2 = xa[2], c0 = xc[0], c1 = xc[1], c2 = xc[2];
          if constexpr (D == 256) {
            a0 = g1 ? xa[3] : a0;
            a1 = g1 ? xa[4] : a1;
            a2 = g1 ? xa[5] : a2;
            c0 = g1 ? xc[3] : c0;
            c1 = g1 ? xc[4] : c1;
            c2 = g1 ? xc[5] : c2;
          }
          const uint32_t oa = code3x4(a0, a1, a2, u % 8, kb);
          const uint32_t oc = code3x4(c0, c1, c2, u % 8, kb);
          const uint32_t ta = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oa);
          const uint32_t tc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oc);
          ah[e] = perm(tc, ta, 0x05040100u);
          al[e] = perm(tc, ta, 0x07060302u);
        }
        vop[((vh * NU + u) * 2 + 0) * 64 + lane] = ah;
        vop[((vh * NU + u) * 2 + 1) * 64 + lane] = al;
      }
    } else {
      constexpr int TPB = 8 / VB;
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        const int u = vu0 + j;
        constexpr int kBitsPerWord = 32;
        const int bit = u * VB, w = bit / kBitsPerWord, byte = (bit % kBitsPerWord) / 8;
        const int t = u % TPB;
        const int sh = 2 - VB * t;
        v4u ah, al;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // LDS byte offsets of the two tokens' codes (4 x the code), byte
          // `byte` zero-extended (selector 0x0c gives a zero byte)
          const uint32_t xa = run[2 * e][w], xc = run[2 * e + 1][w];
          const uint32_t va = (sh >= 0 ? (xa << sh) : (xa >> -sh)) & (0x01010101u * (VMASK << 2));
          const uint32_t vc = (sh >= 0 ? (xc << sh) : (xc >> -sh)) & (0x01010101u * (VMASK << 2));
          const uint32_t bsel = 0x0c0c0c00u + (uint32_t)byte;
          const uint32_t oa = perm(0u, va, bsel), oc = perm(0u, vc, bsel);
          const uint32_t ta = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oa);
          const uint32_t tc = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(s_vt) + oc);
          ah[e] = perm(tc, ta, 0x05040100u);
          al[e] = perm(tc, ta, 0x07060302u);
        }
        vop[((vh * NU + u) * 2 + 0) * 64 + lane] = ah;
        vop[((vh * NU + u) * 2 + 1) * 64 + lane] = al;
      }
    }
    if (wave == 0 && lane < kTile) {
      fld[lane] = rfk;
      fld[kTile + lane] = rfq;
      fld[2 * kTile + lane] = rfv;
    }
  };

  // ---- the rows' operands (registers): int8 digits of q_rot row rl, and the
  // QJL pieces of (S q_rot) row rl, in the decode kernel's lane layout
  v4i qa[KS8], qb[KS8], qc[KS8];
  v4u qh[KS], ql[KS];
  float rowc;
  {
    const size_t qoff = ((size_t)bg * rows + (rok ? rl : 0)) * D + LC * g;
    float qv[LC];
#pragma unroll
    for (int c = 0; c < LC; c += 4) {
      const v4f x = rok ? *reinterpret_cast<const v4f*>(p.qrot + qoff + c) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) qv[c + t] = x[t];
    }
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < LC; ++c) mx = fmaxf(mx, fabsf(qv[c]));
    mx = rowmax4(mx);
    const float sc = mx > 0.f ? kQMax / mx : 0.f;
    rowc = mx > 0.f ? p.scale * kLog2e * 256.f * exp2f(-(float)p.kgrid) / sc : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS8; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t u[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // the product may round one past the bound: clamp so the top digit fits
          const float x = fminf(fmaxf(rintf(qv[kstep_coord<KB>(ks, e, bb)] * sc), -kQMax), kQMax);
          u[bb] = (uint32_t)((int)x + 0x808080);  // bytes 2, 1, 0: a, b, c, each + 128
        }
        const uint32_t lo01 = perm(u[1], u[0], 0x05010400u);
        const uint32_t lo23 = perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = perm(u[1], u[0], 0x0c0c0602u);
        const uint32_t hi23 = perm(u[3], u[2], 0x0c0c0602u);
        qa[ks][e] = (int)(perm(hi23, hi01, 0x05040100u) ^ 0x80808080u);
        qb[ks][e] = (int)(perm(lo23, lo01, 0x07060302u) ^ 0x80808080u);
        qc[ks][e] = (int)(perm(lo23, lo01, 0x05040100u) ^ 0x80808080u);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qh[s] = v4u{0u, 0u, 0u, 0u};
      ql[s] = v4u{0u, 0u, 0u, 0u};
      if constexpr (PROD) {
        const float* qsr = p.qs + qoff + 32 * (s >> 2) + 4 * (s & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t h, l;
          split_pair(rok ? qsr[e] : 0.f, rok ? qsr[e + 16] : 0.f, h, l);
          qh[s][e] = h;
          ql[s][e] = l;
        }
      }
    }
  }

  if (ntok > 0) {
    stage_load(0);
    __syncthreads();  // s_vt
    stage_expand(0);
    stage_load(kTile);
  }
  float m_ref = -1e30f, l_run = 0.f;
  v4f acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int T0 = 0; T0 < ntok; T0 += kTile) {
    const uint8_t* buf = s_buf + ((T0 / kTile) & 1) * kBuf;
    const v4i* kop = reinterpret_cast<const v4i*>(buf);
    const v4u* qop = reinterpret_cast<const v4u*>(buf + Lay::kKey);
    const v4u* vop = reinterpret_cast<const v4u*>(buf + Lay::kKey + Lay::kQjl);
    const float* fld = reinterpret_cast<const float*>(buf + Lay::kKey + Lay::kQjl + Lay::kVal);
    __syncthreads();

    // the next tile's share, into the other buffer (every wave finished with
    // it before this tile's barrier), and the loads of the one after.  With
    // eight waves, half expand before their products and half after them, so
    // that the two waves sharing a SIMD (w and w + 4) tend to run matrix-core
    // and VALU phases side by side rather than in step after the barrier;
    // with four (one per SIMD) every wave expands between its score and
    // value products.
    const bool more = T0 + kTile < ntok;
    if (early && more) {
      stage_expand(T0 + kTile);
      stage_load(T0 + 2 * kTile);
    }

    // ---- scores of this wave's rows: MSE term on the int8 matrix cores, QJL
    // term on the bf16 ones (lane (m, g) ends with row m's scores of tokens
    // 16 tg + 4 g + r)
    v4f sm[TG], sq[TG];
    {
      v4i t24[TG], t16[TG], t8[TG];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) t24[tg] = t16[tg] = t8[tg] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          const v4i ah = kop[((tg * KS8 + ks) * 2 + 0) * 64 + lane];
          const v4i al = kop[((tg * KS8 + ks) * 2 + 1) * 64 + lane];
          t24[tg] = mfma8(ah, qa[ks], t24[tg]);
          t16[tg] = mfma8(al, qa[ks], t16[tg]);
          t8[tg] = mfma8(al, qb[ks], t8[tg]);
          t16[tg] = mfma8(ah, qb[ks], t16[tg]);
          t8[tg] = mfma8(ah, qc[ks], t8[tg]);
        }
      }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lo = (int)(((uint32_t)t16[tg][i] << 8) + (uint32_t)t8[tg][i]);
          sm[tg][i] = rowc * fmaf(65536.f, (float)t24[tg][i], (float)lo);
        }
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) sq[tg] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (PROD) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          const v4u as = qop[(tg * KS + s) * 64 + lane];
          sq[tg] = mfma(as, qh[s], sq[tg]);
          sq[tg] = mfma(as, ql[s], sq[tg]);
        }
    }
    if (!early && !late && more) {
      stage_expand(T0 + kTile);
      stage_load(T0 + 2 * kTile);
    }

    // ---- online softmax of row m over this lane's NT tokens
    float sc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int ti = 16 * (i >> 2) + 4 * g + (i & 3);
      const float kn = fld[ti], kq = fld[kTile + ti];
      sc[i] = PROD ? fmaf(kn, sm[i >> 2][i & 3], kq * sq[i >> 2][i & 3]) : kn * sm[i >> 2][i & 3];
    }
    if (!(T0 + kTile <= ntok && T0 + kTile <= lim_all)) {
      // masked tokens (the chunk's end, the causal edge) behind a
      // wave-uniform branch, kept there by the empty asm statement
      asm volatile("");
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int tk = T0 + 16 * (i >> 2) + 4 * g + (i & 3);
        if (!(tk < ntok && tk < lim)) sc[i] = -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) tmax = fmaxf(tmax, sc[i]);
    tmax = rowmax4(tmax);
    if (__ballot(tmax > m_ref + kFlushGap) != 0) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] *= alpha;
      l_run *= alpha;
      m_ref = m_new;
    }
    float pv[NT];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      // the hardware exp2: arguments are at most kFlushGap, or -inf (masked)
      const float pr = __builtin_amdgcn_exp2f(sc[i] - m_ref);
      psum += pr;
      pv[i] = VGROUP ? pr : pr * fld[2 * kTile + 16 * (i >> 2) + 4 * g + (i & 3)];
    }
    l_run += psum;

    // ---- values: half h takes the lane's tokens i = 8 h .. 8 h + 7
#pragma unroll
    for (int h = 0; h < TG / 2; ++h) {
      v4u bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = __float_as_uint(pv[8 * h + 2 * e]), c = __float_as_uint(pv[8 * h + 2 * e + 1]);
        bh[e] = perm(c, a, 0x07060302u);
        const float ra = pv[8 * h + 2 * e] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[8 * h + 2 * e + 1] - __uint_as_float(c & 0xffff0000u);
        bl[e] = perm(__float_as_uint(rc), __float_as_uint(ra), 0x07060302u);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const v4u ah = vop[((h * NU + u) * 2 + 0) * 64 + lane];
        const v4u al = vop[((h * NU + u) * 2 + 1) * 64 + lane];
        acc[u] = mfma(ah, bh, acc[u]);
        acc[u] = mfma(ah, bl, acc[u]);
        acc[u] = mfma(al, bh, acc[u]);
      }
    }
    if (late && more) {
      stage_expand(T0 + kTile);
      stage_load(T0 + 2 * kTile);
    }
  }

  // ---- this wave's rows' partial for the chunk
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (rok) {
    const size_t slot = ((size_t)bg * p.n_chunks + chunk_id) * rows + rl;
    float* po = p.part_o + slot * D;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) po[V3 ? coord3<D>(4 * g + r, u) : (4 * g + r) * NU + u] = acc[u][r];
    if (g == 0) {
      p.part_ml[2 * slot] = m_ref;
      p.part_ml[2 * slot + 1] = l_run;
    }
  }
}

template <int D, int KB, bool PROD>
hipError_t launch_pb_vb(const DecodeParams& p, hipStream_t stream) {
  const int64_t n_rg = (p.rows + PbShape<D>::kRows - 1) / PbShape<D>::kRows;
  if ((int64_t)p.n_chunks * n_rg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.n_chunks * n_rg), p.hkv, p.batch);
  const dim3 block(PbShape<D>::kWaves * 64);
  if (p.vmode == TQ_MODE_GROUP) {
    if (p.vbits != 2) return hipErrorInvalidValue;
    prefill_bf16_kernel<D, KB, 2, PROD, true><<<grid, block, 0, stream>>>(p);
    return hipGetLastError();
  }
  switch (p.vbits) {
    case 1: prefill_bf16_kernel<D, KB, 1, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 2: prefill_bf16_kernel<D, KB, 2, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 3: prefill_bf16_kernel<D, KB, 3, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 4: prefill_bf16_kernel<D, KB, 4, PROD, false><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_pb_d(const DecodeParams& p, hipStream_t stream) {
  const bool prod = p.kmode == TQ_MODE_PROD;
  if (p.kbits == 1) return prod ? launch_pb_vb<D, 1, true>(p, stream) : launch_pb_vb<D, 1, false>(p, stream);
  if (p.kbits == 3) return prod ? launch_pb_vb<D, 3, true>(p, stream) : launch_pb_vb<D, 3, false>(p, stream);
  return prod ? launch_pb_vb<D, 2, true>(p, stream) : launch_pb_vb<D, 2, false>(p, stream);
}

template <int D, int KB, bool PROD>
hipError_t launch_vb(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (p.vmode == TQ_MODE_GROUP) {
    if (p.vbits != 2) return hipErrorInvalidValue;
    decode_bf16_kernel<D, KB, 2, PROD, true><<<grid, block, 0, stream>>>(p);
    return hipGetLastError();
  }
  switch (p.vbits) {
    case 1: decode_bf16_kernel<D, KB, 1, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 2: decode_bf16_kernel<D, KB, 2, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 3: decode_bf16_kernel<D, KB, 3, PROD, false><<<grid, block, 0, stream>>>(p); break;
    case 4: decode_bf16_kernel<D, KB, 4, PROD, false><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  const bool prod = p.kmode == TQ_MODE_PROD;
  if (p.kbits == 1) return prod ? launch_vb<D, 1, true>(p, grid, stream) : launch_vb<D, 1, false>(p, grid, stream);
  if (p.kbits == 3) return prod ? launch_vb<D, 3, true>(p, grid, stream) : launch_vb<D, 3, false>(p, grid, stream);
  return prod ? launch_vb<D, 2, true>(p, grid, stream) : launch_vb<D, 2, false>(p, grid, stream);
}

}  // namespace

// qprep_kernel (the rotated rows), prefill_bf16_kernel over row groups (128
// rows at head_dim 128, 64 at 256) and chunks of the plan, merge_kernel; the
// codecs bf16_decode_supported accepts.  Token indices inside a chunk use
// 24-bit products: chunks hold at most 2^24 tokens.
hipError_t launch_prefill_bf16(const DecodeParams& p, hipStream_t stream) {
  if (!bf16_prefill_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits) || p.rows < 1 || p.n_chunks < 1 ||
      p.chunk % 64 || p.chunk > (1 << 24) || p.hkv > 65535 || p.batch > 65535)
    return hipErrorInvalidValue;
  hipError_t e = launch_qprep(p, stream);
  if (e != hipSuccess) return e;
  e = p.d == 128 ? launch_pb_d<128>(p, stream) : launch_pb_d<256>(p, stream);
  if (e != hipSuccess) return e;
  return launch_merge(p, stream);
}

// The decode kernel of this file for a launch that bf16_decode_supported
// accepts; the query prologue and the merge are the caller's.  Token indices
// inside a chunk use 24-bit products: chunks hold at most 2^24 tokens.
hipError_t launch_decode_bf16_kernel(const DecodeParams& p, const dim3 grid, hipStream_t stream) {
  if (!bf16_decode_supported(p.d, p.kmode, p.kbits, p.vmode, p.vbits, p.rows) || p.chunk % kStep ||
      p.chunk > (1 << 24))
    return hipErrorInvalidValue;
  return p.d == 128 ? launch_d<128>(p, grid, stream) : launch_d<256>(p, grid, stream);
}

}  // namespace tq
