// Decode attention over the compressed cache on the gfx950 matrix cores.
//
// Covers head_dim 128 with 3-bit MSE keys and values and up to 16 query rows
// per KV head (the 256k-context MTP-verify workload: 8 query heads per KV head
// x 2 new tokens).  Same split over the token axis as the general kernel, with
// the cross-chunk merge as a second, stream-ordered kernel (a device-wide fence
// per workgroup would write back and invalidate the L2 of every XCD); the
// per-token work is reorganised so that both products run as exact int8
// matrix-core operations:
//
//   scores  S^T[token][row] = C_k[token][coord] . Q^T[coord][row]
//   values  O^T[coord][row] = V^T[coord][token] . P'^T[token][row]
//
// * Centroids are integers on the codec's dyadic grid (|c| 2^E <= 16256), so
//   each is exactly hi*256 + lo with int8 pieces.  The rotated queries and the
//   probabilities p*n_v are quantised to 24 bits (three balanced base-256 int8
//   digits, 2^-23 of the row maximum / the value-norm reference), so that the
//   rounding noise summed over many small probabilities stays far below the
//   output of a sharp softmax.  The int8 v_mfma_i32_16x16x64_i8 products of
//   the digits accumulate exactly in int32: five per K-step of the scores and
//   five per tile of the values (every digit pair above 2^-24 of a product).
// * Packed indices become int8 operands with no per-coordinate loop: the 3-bit
//   byte-lane layout yields four indices per shift-and-mask ("selector"
//   dwords), and v_perm_b32 looks four of them up at once in 8-byte tables.
// * Keys are used token-major (one lane per token and 32-coordinate group).
//   Values must enter the matrix core coordinate-major: each wave writes its
//   tile's value selectors to LDS as [token][coordinate] bytes and reads them
//   back transposed with ds_read_b64_tr_b8 (lane j of a 16-lane group gets,
//   as byte i, column j%8 of the row addressed by lane 2i + j/8).
// * The score tile's token order is permuted so that a lane's score
//   accumulators are exactly the 16 consecutive tokens the value product needs
//   from it: the probabilities never move between lanes.
// * Online softmax per row in the log2 domain; the int32 value accumulators
//   are flushed to float only when a row maximum or the value-norm reference
//   grows (rare after the first tile of a wave).
// * The query is rotated once per workgroup inside the kernel (fp32 matrix
//   cores) while the first two tiles of every wave are already in flight, and
//   each workgroup's buffer resources end at its chunk, so no byte outside the
//   chunk is fetched.
#include "chunk_order.h"
#include "codes3.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v3u __attribute__((ext_vector_type(3)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kTile = 64;              // tokens per wave iteration
constexpr int kWaves = 8;              // 512-thread workgroups, one per compute unit
constexpr int kThreads = kWaves * 64;
constexpr int kStep = kWaves * kTile;  // tokens per workgroup iteration
constexpr int kMaxChunks = 128;        // merge weights kept in LDS
constexpr int kMaxChunk = 1 << 19;     // tokens per chunk (int32 accumulator bound, see the launcher)
constexpr int kRow = kD + 16;          // LDS bytes per token row of value selectors
constexpr int kSelLds = kTile * kRow + 448;       // value selectors of the tile (+ row-group offsets)
constexpr int kNormLds = 2 * kTile * 4;            // key and value norms of the tile
constexpr int kAccRow = kD / 4 + 1;               // 16-byte slots per accumulator row (one of padding)
constexpr int kAccLds = 16 * kAccRow * 16;         // float output accumulator [row][coord]
constexpr int kWaveLds = kSelLds + kNormLds + kAccLds;
constexpr int kLds = kWaves * kWaveLds;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQMax = 8355711.f;    // three-digit operand bound (2^23 - 0x8081)
// 0x808080 = 2^23 + 0x8080: for 0 <= q <= kQMax the float q + 0x808080 lies in
// [2^23, 2^24), where floats are the integers, and its mantissa is q + 0x8080:
// byte 2 is the top digit a >= 0, bytes 1 and 0 are the balanced digits + 128
constexpr float kDigitBias = 8421504.f;
constexpr int kBufWord3 = 0x00020000;     // raw buffer resource, gfx9 data format
constexpr float kFlushGap = 4.f;          // log2 headroom: p may reach 2^4 between flushes
// p n_v sig <= 2^kFlushGap * 1.001 * nref * sig = kQMax: the 0.1% margin covers
// exp2 and product rounding
constexpr float kProbBound = 16.f * 1.001f;
constexpr float kNormHeadroom = 2.f;      // value-norm reference: twice the largest norm seen

// Byte offset of row group q (rows 16q .. 16q+15) of a wave's value-selector
// tile.  LDS has 64 four-byte banks (bank = byte address / 4 mod 64) and
// serves a 16-byte store for 16 lanes at a time; offsets of 0, 128, 64 and 192
// bytes mod 256 make the sixteen rows one store touches (4 per group) fill
// all 64 banks, and put the two 16-lane halves of a transposing 8-byte read
// 32 banks apart.  The offsets grow with q (+256 where needed) so that no
// group overlaps the next.
__device__ __forceinline__ int sel_group_offset(int q) { return 128 * (q & 1) + 320 * (q >> 1); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// int8 pieces of sixteen codes (four selector dwords) from an 8-entry table.
__device__ __forceinline__ v4i lookup(const uint32_t* s, uint32_t t_hi, uint32_t t_lo) {
  v4i r;
  r.x = (int)perm(t_hi, t_lo, s[0]);
  r.y = (int)perm(t_hi, t_lo, s[1]);
  r.z = (int)perm(t_hi, t_lo, s[2]);
  r.w = (int)perm(t_hi, t_lo, s[3]);
  return r;
}

__device__ __forceinline__ v2i read_tr8(const uint8_t* a) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(a));
}

// (2^24 t24 + 2^16 t16 + 2^8 t8) / 256 in float: the digit accumulators of a
// value product in units of 256 (the kappa factor carries the rest)
__device__ __forceinline__ float flushed(int t24, int t16, int t8) {
  return fmaf(fmaf((float)t24, 256.f, (float)t16), 256.f, (float)t8);
}

// maximum over the four 16-lane rows (lanes n, n+16, n+32, n+48): the two
// lane-swap instructions exchange whole rows, so the union of their two
// results always holds both rows of each pair
__device__ __forceinline__ float rowmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// ---- query prologue ----------------------------------------------------------
//
// The rotated query rows of (b, g) as int8 operand digits, computed by the
// whole workgroup.  Operand order (matches the key selectors): K-step ks,
// digit (0 = most significant), lane l (row l%16, group h = l/16), byte s of
// the 16-byte fragment = coordinate 32h + 16ks + s.  Q = 65536 a + 256 b + c
// with balanced digits a, b, c in [-128, 127].
struct QueryOps {
  v4i a0, b0, c0, a1, b1, c1;
  float rowc;  // score (log2 units) per unit of the digit product, >= 1e-30
};

// Operands of q_rot^T = Pi_k q^T on v_mfma_f32_16x16x4f32, wave w computing
// output coordinates 16w .. 16w+15.  In K-step s (0..31) lane l supplies the
// term j = 32 (l/16) + s, i.e. A = Pi[16w + l%16][32 (l/16) + s], read from
// the transposed table Pi^T[j][16w + l%16] (for each s the 64 lanes read four
// 64-byte runs), and B = q[row l%16][32 (l/16) + s] from LDS.  The query rows
// are staged once per workgroup: thread t loads four consecutive elements of
// row t/32 (16-byte or 8-byte loads, coalesced).  All of these loads are
// issued before the tiles, so that waiting for them leaves the tile loads in
// flight.
constexpr int kQRow = kD + 4;  // LDS floats per staged query row (16-byte reads without bank conflicts)

struct QueryLoads {
  float pit[32];
  v4f qs;
};

__device__ __forceinline__ void query_loads(const DecodeParams& p, int b, int g, QueryLoads& ql) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const float* pt = p.k_pit + (size_t)(32 * kq) * kD + 16 * wave + r;
#pragma unroll
  for (int s = 0; s < 32; ++s) ql.pit[s] = pt[(size_t)s * kD];
  const int t = threadIdx.x, qr = t >> 5, qc = (t & 31) * 4;
  // the rows of KV head g are contiguous in q (query heads g*group ..
  // g*group+group-1, q_len rows each): the buffer starts at this launch's
  // first row, so 32-bit offsets cover any query tensor
  const int rr = qr < p.rows ? qr : 0;
  const uint32_t esize = p.q_bf16 ? 2u : 4u;
  const char* qbase = static_cast<const char*>(p.q) +
                      ((((int64_t)b * p.hq + (int64_t)g * p.group) * p.q_len + p.row0) * kD) * esize;
  const uint32_t qoff = (uint32_t)((rr * kD + qc) * esize);
  const __amdgpu_buffer_rsrc_t rq = rsrc(qbase, (uint32_t)(p.rows * kD) * esize);
  if (p.q_bf16) {
    const v2i w = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rq, qoff, 0, 0));
    ql.qs = v4f{__uint_as_float((uint32_t)w.x << 16), __uint_as_float((uint32_t)w.x & 0xffff0000u),
                __uint_as_float((uint32_t)w.y << 16), __uint_as_float((uint32_t)w.y & 0xffff0000u)};
  } else {
    ql.qs = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, 0, 0));
  }
  if (qr >= p.rows) ql.qs = v4f{0.f, 0.f, 0.f, 0.f};
}

// s_q: [16 rows][kQRow] staged query rows; s_max: [8 waves][16 rows] partial
// row maxima; s_op: [2 ks][3 digits][64 lanes][4 dwords] operand dwords.  None
// is touched after the prologue.
__device__ __forceinline__ void query_operands(const DecodeParams& p, const QueryLoads& ql, float* s_q,
                                               float* s_max, uint32_t* s_op, QueryOps& qo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  {
    const int t = threadIdx.x;
    *reinterpret_cast<v4f*>(s_q + (t >> 5) * kQRow + (t & 31) * 4) = ql.qs;
  }
  __syncthreads();
  v4f qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = *reinterpret_cast<const v4f*>(s_q + r * kQRow + 32 * kq + 4 * i);
  // lane l ends with q_rot[row r][16 wave + 4 kq + i], i = 0..3 (four
  // independent accumulation chains)
  v4f part[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) part[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 32; ++s)
    part[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(ql.pit[s], qv[s >> 2][s & 3], part[s & 3], 0, 0, 0);
  const v4f acc = (part[0] + part[1]) + (part[2] + part[3]);
  const float m4 = rowmax4(fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3]))));
  if (kq == 0) s_max[wave * 16 + r] = m4;
  __syncthreads();
  float mx = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_max[w * 16 + r]);
  const float sc = mx > 0.f ? kQMax / mx : 0.f;
  // coordinates 16 wave + 4 kq + i are operand K-step wave & 1, lane
  // r + 16 (wave >> 1), dword kq
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the product may round one past the bound: clamp so the top digit fits int8
    const float x = fminf(fmaxf(rintf(acc[i] * sc), -kQMax), kQMax);
    u[i] = (uint32_t)((int)x + 0x808080);  // bytes: a+128, b+128, c+128
  }
  const uint32_t lo01 = perm(u[1], u[0], 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
  const uint32_t lo23 = perm(u[3], u[2], 0x05010400u);
  const uint32_t hi01 = perm(u[1], u[0], 0x0c0c0602u);  // u0.b2 u1.b2 0 0
  const uint32_t hi23 = perm(u[3], u[2], 0x0c0c0602u);
  uint32_t* o = s_op + ((wave & 1) * 3 * 64 + r + 16 * (wave >> 1)) * 4 + kq;
  o[0] = perm(hi23, hi01, 0x05040100u) ^ 0x80808080u;
  o[64 * 4] = perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
  o[128 * 4] = perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
  __syncthreads();
  const v4i* op = reinterpret_cast<const v4i*>(s_op) + lane;
  qo.a0 = op[0];
  qo.b0 = op[64];
  qo.c0 = op[128];
  qo.a1 = op[192];
  qo.b1 = op[256];
  qo.c1 = op[320];
  // this lane's operand row is r as well
  // score = sum_j Q_j C_j / (sc 2^E) = 256 [(256 t24 + t16) 256 + t8] / (sc 2^E)
  qo.rowc = sc > 0.f ? 256.f * p.scale * kLog2e * exp2f(-(float)p.kgrid) / sc : 0.f;
  qo.rowc = fmaxf(qo.rowc, 1e-30f);  // keeps -inf * rowc = -inf for a zero query row
}

// One 64-token tile of this wave: the three key and value words of one token
// and 32-coordinate group per score tile st (token order 16(m/4) + 4st + m%4),
// and one key and one value norm per lane (token T0 + lane).  Offsets are
// per-lane so that the buffer range check covers every token: reads past the
// chunk return zeros and fetch nothing.
struct Tile {
  v3u kw[4], vw[4];
  float kn, vn;
};

__device__ __forceinline__ void load_keys(Tile& t, __amdgpu_buffer_rsrc_t rk, const uint32_t* lw, uint32_t T0) {
#pragma unroll
  for (int st = 0; st < 4; ++st) t.kw[st] = __builtin_amdgcn_raw_buffer_load_b96(rk, lw[st] + T0 * 48u, 0, 0);
}

__device__ __forceinline__ void load_values(Tile& t, __amdgpu_buffer_rsrc_t rv, const uint32_t* lw, uint32_t T0) {
#pragma unroll
  for (int st = 0; st < 4; ++st) t.vw[st] = __builtin_amdgcn_raw_buffer_load_b96(rv, lw[st] + T0 * 48u, 0, 0);
}

__device__ __forceinline__ void load_norms(Tile& t, __amdgpu_buffer_rsrc_t rkn, __amdgpu_buffer_rsrc_t rvn,
                                           uint32_t ln4, uint32_t T0) {
  t.kn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn, ln4 + T0 * 4u, 0, 0));
  t.vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn, ln4 + T0 * 4u, 0, 0));
}

__device__ __forceinline__ void load_tile(Tile& t, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          __amdgpu_buffer_rsrc_t rkn, __amdgpu_buffer_rsrc_t rvn,
                                          const uint32_t* lw, uint32_t ln4, uint32_t T0) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    t.kw[st] = __builtin_amdgcn_raw_buffer_load_b96(rk, lw[st] + T0 * 48u, 0, 0);
    t.vw[st] = __builtin_amdgcn_raw_buffer_load_b96(rv, lw[st] + T0 * 48u, 0, 0);
  }
  t.kn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn, ln4 + T0 * 4u, 0, 0));
  t.vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn, ln4 + T0 * 4u, 0, 0));
}

__global__ __launch_bounds__(kThreads, 1) void decode_fast_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kLds];
  __shared__ __attribute__((aligned(16))) uint32_t s_op[2 * 3 * 64 * 4];
  __shared__ float s_max[kWaves * 16];

  // the wave index is uniform: a scalar register keeps the tile loop uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, h = lane >> 4;  // query row, lane group
  const int chunk_id = rotated_chunk(blockIdx.x, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g;
  const int rows = p.rows;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  // this workgroup's tokens c0 .. c0 + ntok - 1; token indices below are
  // relative to c0
  const int c0 = chunk_id * p.chunk;
  const int c1 = c0 + p.chunk < len ? c0 + p.chunk : len;
  const uint32_t ntok = c1 > c0 ? (uint32_t)(c1 - c0) : 0u;
  // the causal rule counts the q_len new tokens from the sequence's whole
  // length, which a hybrid cache passes apart (its recent tokens are not in
  // this cache)
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;
  const int lim = lenm - p.q_len + ((p.row0 + n) % p.q_len) + 1 - c0;  // row n sees tokens < lim
  const int lim_all = lenm - p.q_len + 1 - c0;              // tokens every row sees

  // ---- loads: the query prologue's first, then the first two tiles
  QueryLoads ql;
  query_loads(p, b, g, ql);
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)(ntok > 0 ? c0 : 0);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rkn = rsrc(p.k_norm + base, ntok * 4u);
  const __amdgpu_buffer_rsrc_t rvn = rsrc(p.v_norm + base, ntok * 4u);
  uint32_t lw[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) lw[st] = (uint32_t)(16 * (n >> 2) + 4 * st + (n & 3)) * 48u + 12u * h;
  const uint32_t ln4 = (uint32_t)lane * 4u;
  const uint32_t t_first = (uint32_t)(wave * kTile);
  Tile ta, tb;
  // issue order matters: the loop waits on the first tile's loads with the
  // second tile's still in flight, which the wait counter can express only if
  // every load of the first tile precedes every load of the second
  load_tile(ta, rk, rv, rkn, rvn, lw, ln4, t_first);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(tb, rk, rv, rkn, rvn, lw, ln4, t_first + kStep);
  // nothing that waits for the query loads may move above the tile loads
  __builtin_amdgcn_sched_barrier(0);

  QueryOps qo;
  // the staged query rows occupy the start of s_buf until the prologue's
  // last barrier; the waves' tile areas are written only after it
  query_operands(p, ql, reinterpret_cast<float*>(s_buf), s_max, s_op, qo);
  const float rowc = qo.rowc;
  const uint32_t kh1 = p.klut[1], kh0 = p.klut[0], kl1 = p.klut[3], kl0 = p.klut[2];
  const uint32_t vh1 = p.vlut[1], vh0 = p.vlut[0], vl1 = p.vlut[3], vl0 = p.vlut[2];
  const float kappa = 256.f * exp2f(-(float)p.vgrid);

  uint8_t* sb = s_buf + wave * kWaveLds;
  float* sn = reinterpret_cast<float*>(sb + kSelLds);            // [2][64] norms of the tile
  v4f* so = reinterpret_cast<v4f*>(sb + kSelLds + kNormLds);     // [16 rows][kAccRow] x 4 coords
  // float output of row n, coordinates 16u + 4h .. +3, lives in LDS: it is
  // touched only when the int32 accumulators are flushed
  // (rows kAccRow slots apart: a 16-lane group's 16-byte accesses, one row
  // each, cover all 64 banks)
  auto oref = [&](int u) -> v4f& { return so[n * kAccRow + 4 * u + h]; };
#pragma unroll
  for (int u = 0; u < 8; ++u) oref(u) = v4f{0.f, 0.f, 0.f, 0.f};

  // running maximum of the row (log2 domain); a finite "minus infinity" so that
  // masked scores (-inf) give exp2 = 0 and an empty row never forms inf - inf
  float m_ref = -1e30f, l_run = 0.f;
  // value-norm reference: probabilities enter the digits as p n_v sig with
  // sig = kQMax / (kProbBound nref), so p n_v sig <= kQMax while n_v <= nref;
  // lsig = log2 sig is folded into the exponent, kflush = kappa / sig
  float nref = 0.f, lsig = 0.f, isig = 1.f, kflush = kappa;
  bool empty = true;  // accumulators untouched so far (wave-uniform)
  v4i ahh[8], ax[8], all[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    ahh[u] = v4i{0, 0, 0, 0};
    ax[u] = v4i{0, 0, 0, 0};
    all[u] = v4i{0, 0, 0, 0};
  }

  auto process = [&](Tile& cur, const uint32_t T0, const uint32_t Tn) {
    // ---- scores on the matrix cores, with the value selectors of the same
    // score tile computed while its ten products run (the scheduling groups
    // put two VALU instructions behind each MFMA)
    float sc[16];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint32_t s8[8];
      selectors3(cur.kw[st].x, cur.kw[st].y, cur.kw[st].z, s8);
      const v4i ah0 = lookup(s8, kh1, kh0), al0 = lookup(s8, kl1, kl0);
      const v4i ah1 = lookup(s8 + 4, kh1, kh0), al1 = lookup(s8 + 4, kl1, kl0);
      __builtin_amdgcn_sched_barrier(0);
      // Q C = 2^24 a Ch + 2^16 (a Cl + b Ch) + 2^8 (b Cl + c Ch) [+ c Cl, below
      // 2^-23 of the product]
      v4i t24 = v4i{0, 0, 0, 0}, t16 = v4i{0, 0, 0, 0}, t8 = v4i{0, 0, 0, 0};
      t24 = mfma(ah0, qo.a0, t24);
      t16 = mfma(al0, qo.a0, t16);
      t8 = mfma(al0, qo.b0, t8);
      t16 = mfma(ah0, qo.b0, t16);
      t8 = mfma(ah0, qo.c0, t8);
      t24 = mfma(ah1, qo.a1, t24);
      t16 = mfma(al1, qo.a1, t16);
      t8 = mfma(al1, qo.b1, t8);
      t16 = mfma(ah1, qo.b1, t16);
      t8 = mfma(ah1, qo.c1, t8);
      {
        uint32_t v8[8];
        selectors3(cur.vw[st].x, cur.vw[st].y, cur.vw[st].z, v8);
        const int tt = 16 * (n >> 2) + 4 * st + (n & 3);
        v4u* dst = reinterpret_cast<v4u*>(sb + tt * kRow + sel_group_offset(n >> 2) + 32 * h);
        dst[0] = v4u{v8[0], v8[1], v8[2], v8[3]};
        dst[1] = v4u{v8[4], v8[5], v8[6], v8[7]};
      }
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);    // the two LDS stores
      // 256 t24 + t16 is exact in int32; then one float rounding (2^-24)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * st + i] = fmaf((float)(t24[i] * 256 + t16[i]), 256.f, (float)t8[i]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // the key words are consumed: the next tile of this buffer is loaded now
    load_keys(cur, rk, lw, Tn);
    sn[lane] = cur.kn;
    sn[kTile + lane] = cur.vn;
    load_values(cur, rv, lw, Tn);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- online softmax for row n over tokens tb .. tb+15 held by this lane
    const int tb = (int)T0 + 16 * h;
    const v4f* snk = reinterpret_cast<const v4f*>(sn + 16 * h);
    const v4f* snv = reinterpret_cast<const v4f*>(sn + kTile + 16 * h);
    float s[16], wv[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v4f nk4 = snk[c], nv4 = snv[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[4 * c + i] = sc[4 * c + i] * nk4[i];  // score / rowc
        wv[4 * c + i] = nv4[i];
      }
    }
    const bool full = T0 + kTile <= ntok && (int)T0 + kTile <= lim_all;  // no token of the tile is masked
    if (!full) {
      // (an empty asm statement keeps the selects behind the wave-uniform
      // branch: only the last tiles of a chunk take them)
      asm volatile("");
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tok = tb + j;
        if (!(tok < (int)ntok && tok < lim)) s[j] = -INFINITY;
      }
    }
    float tmax = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) tmax = fmaxf(fmaxf(tmax, s[j]), s[j + 1]);
    tmax = fmaxf(tmax, s[15]);
    tmax = rowmax4(tmax) * rowc;
    const bool grow = tmax > m_ref + kFlushGap;
    const bool vgrow = cur.vn > nref;
    if (__ballot(grow || vgrow) != 0) {
      // the tile's largest value norm from this lane's sixteen, then across
      // the four lane groups (every lane holds the same maximum: the
      // reference stays wave-uniform)
      float vmax = fmaxf(fmaxf(wv[0], wv[1]), wv[2]);
#pragma unroll
      for (int j = 3; j < 15; j += 2) vmax = fmaxf(fmaxf(vmax, wv[j]), wv[j + 1]);
      vmax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, rowmax4(fmaxf(vmax, wv[15])))));
      const float nnew = vmax > nref ? kNormHeadroom * vmax : nref;
      const float m_new = grow ? tmax : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      if (!empty) {  // nothing to move before the wave's first tile
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v4f o = oref(u);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = fmaf(flushed(ahh[u][i], ax[u][i], all[u][i]), kflush, o[i]) * alpha;
          oref(u) = o;
          ahh[u] = v4i{0, 0, 0, 0};
          ax[u] = v4i{0, 0, 0, 0};
          all[u] = v4i{0, 0, 0, 0};
        }
      }
      l_run *= alpha;
      m_ref = m_new;
      if (nnew > nref) {
        nref = nnew;
        const float sig = kQMax / (nref * kProbBound);
        lsig = __log2f(sig);
        isig = 1.f / sig;
        kflush = kappa * isig;
      }
    }
    // p sig = exp2(s - m_ref + lsig); the digits carry p n_v sig
    const float off = lsig - m_ref;
    float psum = 0.f;
    uint32_t qv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[j], rowc, off));
      psum += pr;
      qv[j] = __float_as_uint(fmaf(pr, wv[j], kDigitBias));
    }
    l_run = fmaf(psum, isig, l_run);
    empty = false;
    v4i ba, bb, bc;  // digits of 2^16, 2^8 and 1
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t a01 = perm(qv[4 * c + 1], qv[4 * c], 0x05010400u);  // q0.b0 q1.b0 q0.b1 q1.b1
      const uint32_t a23 = perm(qv[4 * c + 3], qv[4 * c + 2], 0x05010400u);
      const uint32_t b01 = perm(qv[4 * c + 1], qv[4 * c], 0x0c0c0602u);  // q0.b2 q1.b2 0 0
      const uint32_t b23 = perm(qv[4 * c + 3], qv[4 * c + 2], 0x0c0c0602u);
      bc[c] = (int)(perm(a23, a01, 0x05040100u) ^ 0x80808080u);
      bb[c] = (int)(perm(a23, a01, 0x07060302u) ^ 0x80808080u);
      ba[c] = (int)perm(b23, b01, 0x05040100u);
    }

    // ---- values on the matrix cores: coordinates 16u + n of tokens tb..tb+15
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint8_t* a0 = sb + (16 * h + (n >> 1)) * kRow + sel_group_offset(h) + 16 * u + 8 * (n & 1);
      const v2i r0 = read_tr8(a0);
      const v2i r1 = read_tr8(a0 + 8 * kRow);
      const uint32_t sv[4] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r1.x, (uint32_t)r1.y};
      const v4i vh = lookup(sv, vh1, vh0), vl = lookup(sv, vl1, vl0);
      // P' V = 2^24 a Vh + 2^16 (a Vl + b Vh) + 2^8 (b Vl + c Vh) [+ c Vl]
      ahh[u] = mfma(vh, ba, ahh[u]);
      ax[u] = mfma(vl, ba, ax[u]);
      ax[u] = mfma(vh, bb, ax[u]);
      all[u] = mfma(vl, bb, all[u]);
      all[u] = mfma(vh, bc, all[u]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // two tile buffers in turn: a tile's successor is in flight while it is
  // processed, and a buffer's next tile (two steps ahead) is requested as
  // soon as its words are consumed: the key words after the scores, the value
  // words once their selectors are in LDS, the norms after the tile.  The
  // loads are unconditional: past the chunk they read zeros without touching
  // memory, so the number of loads in flight is the same on every path and
  // the waits stay partial.
  for (uint32_t T0 = t_first; T0 < ntok; T0 += 2 * kStep) {
    process(ta, T0, T0 + 2 * kStep);
    if (T0 + kStep >= ntok) break;
    load_norms(ta, rkn, rvn, ln4, T0 + 2 * kStep);
    process(tb, T0 + kStep, T0 + 3 * kStep);
    load_norms(tb, rkn, rvn, ln4, T0 + 3 * kStep);
  }

  v4f of[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    of[u] = oref(u);
#pragma unroll
    for (int i = 0; i < 4; ++i) of[u][i] = fmaf(flushed(ahh[u][i], ax[u][i], all[u][i]), kflush, of[u][i]);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // ---- merge the waves' partials of this chunk in LDS: each wave's block
  // holds its 16 rows (padded to kMoRow floats, so that a 16-lane group of
  // 16-byte stores covers all 64 banks) and its (m, l); the per-(wave, row)
  // weights 2^(m_w - M) are formed once
  constexpr int kMoRow = kD + 4, kMoBlock = 16 * kMoRow + 32;
  __syncthreads();
  float* cw = reinterpret_cast<float*>(s_buf);
  float* s_wt = cw + kWaves * kMoBlock;  // [kWaves][16] weights, then [16] M, [16] L
  {
    float* mo = cw + wave * kMoBlock;
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<v4f*>(mo + n * kMoRow + 16 * u + 4 * h) = of[u];
    if (h == 0) {
      mo[16 * kMoRow + n] = m_ref;
      mo[16 * kMoRow + 16 + n] = l_run;
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int r = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cw[w * kMoBlock + 16 * kMoRow + r]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = cw[w * kMoBlock + 16 * kMoRow + r];
      const float wt = (M == -INFINITY || mw == -INFINITY) ? 0.f : exp2f(mw - M);
      s_wt[w * 16 + r] = wt;
      L = fmaf(wt, cw[w * kMoBlock + 16 * kMoRow + 16 + r], L);
    }
    s_wt[kWaves * 16 + r] = M;
    s_wt[kWaves * 16 + 16 + r] = L;
  }
  __syncthreads();
  float* po = p.part_o + ((size_t)bg * p.n_chunks + chunk_id) * rows * kD;
  float* pml = p.part_ml + ((size_t)bg * p.n_chunks + chunk_id) * rows * 2;
  for (int e = threadIdx.x; e < rows * kD; e += kThreads) {
    const int r = e / kD, c = e % kD;
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) O = fmaf(s_wt[w * 16 + r], cw[w * kMoBlock + r * kMoRow + c], O);
    po[e] = O;
  }
  if (threadIdx.x < rows) {
    pml[2 * threadIdx.x] = s_wt[kWaves * 16 + threadIdx.x];
    pml[2 * threadIdx.x + 1] = s_wt[kWaves * 16 + 16 + threadIdx.x];
  }
}

// Cross-chunk merge, one workgroup of kD threads per (query row, KV head,
// sequence), stream-ordered after the decode kernel: weights 2^(m_c - M) / L
// from every chunk's (m, l), the merged rotated row o = sum_c w_c o_c (thread
// j -> coordinate j), and the single inverse rotation out = Pi_v^T o, in row
// form out_j = sum_i o_i Pi_v[i][j].
__global__ __launch_bounds__(kD) void merge_fast_kernel(DecodeParams p) {
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_o[kD];
  __shared__ float s_red[4];
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g, j = threadIdx.x, lane = j & 63, wave = j >> 6;
  const int nch = p.n_chunks, rows = p.rows;
  const float* pml = p.part_ml + (size_t)bg * nch * rows * 2;
  const float* po = p.part_o + (size_t)bg * nch * rows * kD;
  // every load is independent of the weights: (m, l), the first 32 partial
  // rows and column j of Pi_v are all in flight before any is used
  float mc = -INFINITY, lc = 0.f;
  if (j < nch) {
    mc = pml[((size_t)j * rows + r) * 2];
    lc = pml[((size_t)j * rows + r) * 2 + 1];
  }
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = k < nch ? po[((size_t)k * rows + r) * kD + j] : 0.f;
  float pv[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) pv[i] = p.v_pi[i * kD + j];
  float M = wave_max(mc);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(s_red[0], s_red[1]);
  const float w = (j < nch && M != -INFINITY && mc != -INFINITY) ? exp2f(mc - M) : 0.f;
  float L = w * lc;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  if (lane == 0) s_red[2 + wave] = L;
  if (j < kMaxChunks) s_w[j] = w;
  __syncthreads();
  L = s_red[2] + s_red[3];
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) o = fmaf(s_w[k], v[k], o);  // s_w is 0 past the last chunk
  for (int c = 32; c < nch; ++c) o = fmaf(s_w[c], po[((size_t)c * rows + r) * kD + j], o);
  s_o[j] = L > 0.f ? o / L : 0.f;
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) acc = fmaf(s_o[i], pv[i], acc);
  const int R = p.row0 + r;
  const int h = g * p.group + R / p.q_len, qi = R % p.q_len;
  const int64_t orow = ((int64_t)b * p.hq + h) * p.q_len + qi;
  p.out[orow * kD + j] = acc;
  if (p.row_ml && j == 0) {  // the row's softmax reference and sum (log2 domain), for a later combine
    p.row_ml[2 * orow] = M;
    p.row_ml[2 * orow + 1] = L;
  }
}

// ---- prefill: many query rows over shared tiles ------------------------------
//
// A launch with more query rows per KV head than one decode workgroup takes
// (prefill, long q_len) would read the state and expand its codes once per 16
// rows.  Here the eight waves of a workgroup each own 16 rows of the same KV
// head and walk the chunk's tiles together.  Per tile, wave w expands one
// eighth of the shared operands into LDS -- the int8 key pieces of score tile
// w/2, K-step w%2 (the selectors and look-ups a decode wave does for a whole
// tile), half of each of its tokens' value selectors, and eight tokens'
// norms -- and after one barrier every wave runs its own rows' score and value
// products over all of them, as the decode kernel does.  Two LDS buffers
// alternate: a wave that reaches the barrier of tile t has finished reading
// tile t-1's buffer, and the next write to that buffer (tile t+1) comes after
// the barrier of tile t, so one barrier per tile suffices.  The rotated query
// rows come from qprep_kernel; every wave writes its own rows' partial (m, l,
// o) for the chunk, merged by merge_fast_kernel.
constexpr int kPfRowsWave = 16;
constexpr int kPfRows = kWaves * kPfRowsWave;           // rows per workgroup
constexpr int kPfKeyLds = 4 * 2 * 2 * 64 * 16;          // [score tile][K-step][hi, lo][lane] int8 pieces
// one tile's shared operands: key pieces, value hi pieces (in the decode
// kernel's selector layout), norms, value lo pieces (the same layout)
constexpr int kPfLoOff = kSelLds + kNormLds;  // lo pieces, from the hi pieces' start
constexpr int kPfBuf = kPfKeyLds + 2 * kSelLds + kNormLds;
constexpr int kPfLds = 2 * kPfBuf + kWaves * kAccLds;
// every wave takes every tile of its chunk: at most 1024 tiles between
// flushes of its int32 value accumulators (the decode kernel's bound)
constexpr int kPfMaxChunk = 1 << 16;

__global__ __launch_bounds__(kThreads, 1) void prefill_fast_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kPfLds];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, h = lane >> 4;  // query row of the wave, lane group
  const int chunk_id = rotated_chunk(blockIdx.x % p.n_chunks, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int rg = blockIdx.x / p.n_chunks;
  const int g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.hkv + g;
  const int rows = p.rows;
  const int rl = rg * kPfRows + wave * kPfRowsWave + n;  // this lane's row among the launch's rows
  const bool rok = rl < rows;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int c1 = c0 + p.chunk < len ? c0 + p.chunk : len;
  const uint32_t ntok = c1 > c0 ? (uint32_t)(c1 - c0) : 0u;
  const int lenm = p.len_mask ? (p.len_mask[b] < 0 ? 0 : p.len_mask[b]) : len;
  const int lim = lenm - p.q_len + ((p.row0 + rl) % p.q_len) + 1 - c0;  // row rl sees tokens < lim
  const int lim_all = lenm - p.q_len + 1 - c0;                        // tokens every row sees

  // ---- this wave's share of each tile: lane (n, h) holds the key and value
  // words of token tt, 32-coordinate group h (score tile pst = wave/2, whose
  // token order puts a lane's scores on 16 consecutive tokens), and lanes
  // 0..7 the norms of tokens 8 wave .. 8 wave + 7
  const int pst = wave >> 1, pks = wave & 1;
  const uint32_t tt = (uint32_t)(16 * (n >> 2) + 4 * pst + (n & 3));
  const uint32_t lwo = tt * 48u + 12u * (uint32_t)h;
  const uint32_t ln4 = (uint32_t)(8 * wave + (lane & 7)) * 4u;
  const size_t base = (size_t)bg * (size_t)p.cap + (size_t)(ntok > 0 ? c0 : 0);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rkn = rsrc(p.k_norm + base, ntok * 4u);
  const __amdgpu_buffer_rsrc_t rvn = rsrc(p.v_norm + base, ntok * 4u);
  // the first tile's words are requested before the query row (loads
  // complete in order: the digits below wait for them too, which the
  // prologue's own latency covers)
  v3u kw = __builtin_amdgcn_raw_buffer_load_b96(rk, lwo, 0, 0);
  v3u vw = __builtin_amdgcn_raw_buffer_load_b96(rv, lwo, 0, 0);
  float kn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn, ln4, 0, 0));
  float vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn, ln4, 0, 0));

  // ---- query digits of row rl (zero for rows past the launch's): lane
  // (n, h) holds coordinates 32 h .. 32 h + 31, the B operand of K-step ks is
  // coordinates 32 h + 16 ks + s (byte s of the fragment); q = 65536 a + 256 b + c
  v4i qa[2], qb[2], qc[2];
  float rowc;
  {
    const float* qr = p.qrot + ((size_t)bg * rows + (rok ? rl : 0)) * kD + 32 * h;
    v4f x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = rok ? *reinterpret_cast<const v4f*>(qr + 4 * i) : v4f{0.f, 0.f, 0.f, 0.f};
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x[i][0]), fabsf(x[i][1])), fmaxf(fabsf(x[i][2]), fabsf(x[i][3]))));
    mx = rowmax4(mx);
    const float sc = mx > 0.f ? kQMax / mx : 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the product may round one past the bound: clamp so the top digit fits
          const float v = fminf(fmaxf(rintf(x[4 * ks + e][i] * sc), -kQMax), kQMax);
          u[i] = (uint32_t)((int)v + 0x808080);  // bytes 2, 1, 0: a, b, c, each + 128
        }
        const uint32_t lo01 = perm(u[1], u[0], 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
        const uint32_t lo23 = perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = perm(u[1], u[0], 0x0c0c0602u);  // u0.b2 u1.b2 0 0
        const uint32_t hi23 = perm(u[3], u[2], 0x0c0c0602u);
        qa[ks][e] = (int)(perm(hi23, hi01, 0x05040100u) ^ 0x80808080u);
        qb[ks][e] = (int)(perm(lo23, lo01, 0x07060302u) ^ 0x80808080u);
        qc[ks][e] = (int)(perm(lo23, lo01, 0x05040100u) ^ 0x80808080u);
      }
    // score = sum_j Q_j C_j / (sc 2^E) = 256 [(256 t24 + t16) 256 + t8] / (sc 2^E)
    rowc = sc > 0.f ? 256.f * p.scale * kLog2e * exp2f(-(float)p.kgrid) / sc : 0.f;
    rowc = fmaxf(rowc, 1e-30f);  // keeps -inf * rowc = -inf for a zero query row
  }
  const uint32_t kh1 = p.klut[1], kh0 = p.klut[0], kl1 = p.klut[3], kl0 = p.klut[2];
  const uint32_t vh1 = p.vlut[1], vh0 = p.vlut[0], vl1 = p.vlut[3], vl0 = p.vlut[2];
  const float kappa = 256.f * exp2f(-(float)p.vgrid);

  v4f* so = reinterpret_cast<v4f*>(s_buf + 2 * kPfBuf + wave * kAccLds);  // [16 rows][kAccRow] x 4 coords
  auto oref = [&](int u) -> v4f& { return so[n * kAccRow + 4 * u + h]; };
#pragma unroll
  for (int u = 0; u < 8; ++u) oref(u) = v4f{0.f, 0.f, 0.f, 0.f};

  float m_ref = -1e30f, l_run = 0.f;
  float nref = 0.f, lsig = 0.f, isig = 1.f, kflush = kappa;
  bool empty = true;
  v4i ahh[8], ax[8], all[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) ahh[u] = ax[u] = all[u] = v4i{0, 0, 0, 0};

  // ---- stage A: this wave's share of tile T's operands into its buffer,
  // then the request for the words of the tile after it (past the chunk the
  // loads read zeros, fetching nothing, and the expanded operands are never read)
  auto stage_a = [&](uint32_t T) {
    uint8_t* buf = s_buf + ((T / kTile) & 1u) * kPfBuf;
    v4i* kk = reinterpret_cast<v4i*>(buf);
    uint8_t* sb = buf + kPfKeyLds;
    float* sn = reinterpret_cast<float*>(sb + kSelLds);
    // (the K-step half is picked with selects: a register array takes no
    // run-time index)
    uint32_t s8[8], k4[4];
    selectors3(kw.x, kw.y, kw.z, s8);
#pragma unroll
    for (int i = 0; i < 4; ++i) k4[i] = pks ? s8[4 + i] : s8[i];
    kk[((2 * pst + pks) * 2 + 0) * 64 + lane] = lookup(k4, kh1, kh0);
    kk[((2 * pst + pks) * 2 + 1) * 64 + lane] = lookup(k4, kl1, kl0);
    // the value codes' int8 hi and lo pieces, looked up once per tile for
    // every wave
    uint32_t v8[8], v4s[4];
    selectors3(vw.x, vw.y, vw.z, v8);
#pragma unroll
    for (int i = 0; i < 4; ++i) v4s[i] = pks ? v8[4 + i] : v8[i];
    uint8_t* dst = sb + tt * kRow + sel_group_offset((int)(tt >> 4)) + 32 * h + 16 * pks;
    *reinterpret_cast<v4i*>(dst) = lookup(v4s, vh1, vh0);
    *reinterpret_cast<v4i*>(dst + kPfLoOff) = lookup(v4s, vl1, vl0);
    if (lane < 8) {
      sn[8 * wave + lane] = kn;
      sn[kTile + 8 * wave + lane] = vn;
    }
    const uint32_t Tn = T + kTile;
    kw = __builtin_amdgcn_raw_buffer_load_b96(rk, lwo + Tn * 48u, 0, 0);
    vw = __builtin_amdgcn_raw_buffer_load_b96(rv, lwo + Tn * 48u, 0, 0);
    kn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn, ln4 + Tn * 4u, 0, 0));
    vn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn, ln4 + Tn * 4u, 0, 0));
  };
  if (ntok > 0) stage_a(0);

  // Tile T's buffer was written by stage A of the previous iteration (the
  // barrier completes it); stage A of tile T + 64 runs between the score and
  // the value products of tile T, into the other buffer, whose last reader
  // (tile T - 64) every wave finished before the barrier.
  for (uint32_t T0 = 0; T0 < ntok; T0 += kTile) {
    uint8_t* buf = s_buf + ((T0 / kTile) & 1u) * kPfBuf;
    const v4i* kk = reinterpret_cast<const v4i*>(buf);  // [tile st][K-step][hi, lo][lane]
    const uint8_t* sb = buf + kPfKeyLds;                // value hi pieces [token][coordinate], lo at kPfLoOff
    const float* sn = reinterpret_cast<const float*>(sb + kSelLds);  // key norms [64], value norms [64]
    __syncthreads();

    // ---- stage B: this wave's rows.  Scores: lane (n, h) ends with row n's
    // scores of tokens 16 h + 4 st + i
    float sc[16];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      v4i t24 = v4i{0, 0, 0, 0}, t16 = v4i{0, 0, 0, 0}, t8 = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v4i ah = kk[((2 * st + ks) * 2 + 0) * 64 + lane];
        const v4i al = kk[((2 * st + ks) * 2 + 1) * 64 + lane];
        // Q C = 2^24 a Ch + 2^16 (a Cl + b Ch) + 2^8 (b Cl + c Ch) [+ c Cl, below 2^-23 of the product]
        t24 = mfma(ah, qa[ks], t24);
        t16 = mfma(al, qa[ks], t16);
        t8 = mfma(al, qb[ks], t8);
        t16 = mfma(ah, qb[ks], t16);
        t8 = mfma(ah, qc[ks], t8);
      }
      // 256 t24 + t16 is exact in int32; then one float rounding (2^-24)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * st + i] = fmaf((float)(t24[i] * 256 + t16[i]), 256.f, (float)t8[i]);
    }
    stage_a(T0 + kTile);

    // ---- online softmax for row n over tokens tb .. tb+15 held by this lane
    const int tb = (int)T0 + 16 * h;
    const v4f* snk = reinterpret_cast<const v4f*>(sn + 16 * h);
    const v4f* snv = reinterpret_cast<const v4f*>(sn + kTile + 16 * h);
    float s[16], wv[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v4f nk4 = snk[c], nv4 = snv[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[4 * c + i] = sc[4 * c + i] * nk4[i];  // score / rowc
        wv[4 * c + i] = nv4[i];
      }
    }
    const bool full = T0 + kTile <= ntok && (int)T0 + kTile <= lim_all;  // no token of the tile is masked
    if (!full) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tok = tb + j;
        if (!(tok < (int)ntok && tok < lim)) s[j] = -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, s[j]);
    tmax = rowmax4(tmax) * rowc;
    float vmax = wv[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) vmax = fmaxf(vmax, wv[j]);
    const bool grow = tmax > m_ref + kFlushGap;
    const bool vgrow = vmax > nref;
    if (__ballot(grow || vgrow) != 0) {
      const float nnew = __ballot(vgrow) != 0 ? kNormHeadroom * wave_max(vmax) : nref;
      const float m_new = grow ? tmax : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      if (!empty) {  // nothing to move before the wave's first tile
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v4f o = oref(u);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = fmaf(flushed(ahh[u][i], ax[u][i], all[u][i]), kflush, o[i]) * alpha;
          oref(u) = o;
          ahh[u] = v4i{0, 0, 0, 0};
          ax[u] = v4i{0, 0, 0, 0};
          all[u] = v4i{0, 0, 0, 0};
        }
      }
      l_run *= alpha;
      m_ref = m_new;
      if (nnew > nref) {
        nref = nnew;
        const float sig = kQMax / (nref * kProbBound);
        lsig = __log2f(sig);
        isig = 1.f / sig;
        kflush = kappa * isig;
      }
    }
    // p sig = exp2(s - m_ref + lsig); the digits carry p n_v sig
    const float off = lsig - m_ref;
    float psum = 0.f;
    uint32_t qv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[j], rowc, off));
      psum += pr;
      qv[j] = __float_as_uint(fmaf(pr, wv[j], kDigitBias));
    }
    l_run = fmaf(psum, isig, l_run);
    empty = false;
    v4i ba, bb, bc;  // digits of 2^16, 2^8 and 1
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t a01 = perm(qv[4 * c + 1], qv[4 * c], 0x05010400u);  // q0.b0 q1.b0 q0.b1 q1.b1
      const uint32_t a23 = perm(qv[4 * c + 3], qv[4 * c + 2], 0x05010400u);
      const uint32_t b01 = perm(qv[4 * c + 1], qv[4 * c], 0x0c0c0602u);  // q0.b2 q1.b2 0 0
      const uint32_t b23 = perm(qv[4 * c + 3], qv[4 * c + 2], 0x0c0c0602u);
      bc[c] = (int)(perm(a23, a01, 0x05040100u) ^ 0x80808080u);
      bb[c] = (int)(perm(a23, a01, 0x07060302u) ^ 0x80808080u);
      ba[c] = (int)perm(b23, b01, 0x05040100u);
    }

    // ---- values on the matrix cores: coordinates 16u + n of tokens tb..tb+15
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint8_t* a0 = sb + (16 * h + (n >> 1)) * kRow + sel_group_offset(h) + 16 * u + 8 * (n & 1);
      // the pieces, transposed as the decode kernel transposes its selectors
      // (a byte-wise look-up commutes with the transposition)
      const v2i h0 = read_tr8(a0), h1 = read_tr8(a0 + 8 * kRow);
      const v2i l0 = read_tr8(a0 + kPfLoOff), l1 = read_tr8(a0 + kPfLoOff + 8 * kRow);
      const v4i vh = v4i{h0.x, h0.y, h1.x, h1.y}, vl = v4i{l0.x, l0.y, l1.x, l1.y};
      // P' V = 2^24 a Vh + 2^16 (a Vl + b Vh) + 2^8 (b Vl + c Vh) [+ c Vl]
      ahh[u] = mfma(vh, ba, ahh[u]);
      ax[u] = mfma(vl, ba, ax[u]);
      ax[u] = mfma(vh, bb, ax[u]);
      all[u] = mfma(vl, bb, all[u]);
      all[u] = mfma(vh, bc, all[u]);
    }
  }

  // ---- this wave's rows' partial for the chunk
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (rok) {
    float* po = p.part_o + (((size_t)bg * p.n_chunks + chunk_id) * rows + rl) * kD;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v4f o = oref(u);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(flushed(ahh[u][i], ax[u][i], all[u][i]), kflush, o[i]);
      *reinterpret_cast<v4f*>(po + 16 * u + 4 * h) = o;
    }
    if (h == 0) {
      float* pml = p.part_ml + (((size_t)bg * p.n_chunks + chunk_id) * rows + rl) * 2;
      pml[0] = m_ref;
      pml[1] = l_run;
    }
  }
}

// ---- measurement: the decode kernel's reads alone ----------------------------
//
// The same grid, chunks, per-wave tiles, load instructions and two tiles in
// flight per wave as decode_fast_kernel, reading the packed state of every
// sequence once and folding the words instead of computing attention: the
// rate the decode kernel's own access pattern reaches with no arithmetic.
__global__ __launch_bounds__(kThreads, 1) void decode_read_kernel(DecodeParams p, uint32_t* sink, uint32_t sink_words) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, h = lane >> 4;
  const int chunk_id = rotated_chunk(blockIdx.x, blockIdx.y, blockIdx.z, p.hkv, p.n_chunks);
  const int g = blockIdx.y, b = blockIdx.z;
  int64_t len64 = p.len[b];
  len64 = len64 < 0 ? 0 : (len64 > p.cap ? p.cap : len64);
  const int len = (int)len64;
  const int c0 = chunk_id * p.chunk;
  const int c1 = c0 + p.chunk < len ? c0 + p.chunk : len;
  const uint32_t ntok = c1 > c0 ? (uint32_t)(c1 - c0) : 0u;
  const size_t base = (size_t)(b * p.hkv + g) * (size_t)p.cap + (size_t)(ntok > 0 ? c0 : 0);
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v_idx + base * 12, ntok * 48u);
  const __amdgpu_buffer_rsrc_t rkn = rsrc(p.k_norm + base, ntok * 4u);
  const __amdgpu_buffer_rsrc_t rvn = rsrc(p.v_norm + base, ntok * 4u);
  uint32_t lw[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) lw[st] = (uint32_t)(16 * (n >> 2) + 4 * st + (n & 3)) * 48u + 12u * h;
  const uint32_t ln4 = (uint32_t)lane * 4u;
  const uint32_t t_first = (uint32_t)(wave * kTile);
  Tile ta, tb;
  load_tile(ta, rk, rv, rkn, rvn, lw, ln4, t_first);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(tb, rk, rv, rkn, rvn, lw, ln4, t_first + kStep);
  uint32_t acc = 0;
  auto fold = [&](const Tile& t) {
    uint32_t x = __float_as_uint(t.kn) ^ __float_as_uint(t.vn);
#pragma unroll
    for (int st = 0; st < 4; ++st) x ^= t.kw[st].x ^ t.kw[st].y ^ t.kw[st].z ^ t.vw[st].x ^ t.vw[st].y ^ t.vw[st].z;
    acc = acc * 31u + x;
  };
  for (uint32_t T0 = t_first; T0 < ntok; T0 += 2 * kStep) {
    fold(ta);
    load_tile(ta, rk, rv, rkn, rvn, lw, ln4, T0 + 2 * kStep);
    if (T0 + kStep >= ntok) break;
    fold(tb);
    load_tile(tb, rk, rv, rkn, rvn, lw, ln4, T0 + 3 * kStep);
  }
  if (acc == 0x9E3779B9u) sink[((((size_t)b * p.hkv + g) * gridDim.x + chunk_id) * kThreads + threadIdx.x) % sink_words] = acc;
}

}  // namespace

hipError_t launch_decode_read(const DecodeParams& p, uint32_t* sink, uint32_t sink_words, hipStream_t stream) {
  if (p.n_chunks < 1 || p.hkv > 65535 || p.batch > 65535 || p.d != kD || p.chunk < 1 || sink_words < 1)
    return hipErrorInvalidValue;
  decode_read_kernel<<<dim3(p.n_chunks, p.hkv, p.batch), dim3(kThreads), 0, stream>>>(p, sink, sink_words);
  return hipGetLastError();
}

hipError_t launch_decode_fast(const DecodeParams& p, hipStream_t stream) {
  // each wave takes at most chunk / 512 tiles between flushes of its int32
  // value accumulators; one tile adds at most 64 (128*127 + 64*128) < 2^21 to
  // an element, so chunks of at most 2^19 tokens (1024 tiles) stay below 2^31
  if (p.n_chunks < 1 || p.n_chunks > kMaxChunks || p.hkv > 65535 || p.batch > 65535 || p.d != kD ||
      p.rows > 16 || p.chunk > kMaxChunk)
    return hipErrorInvalidValue;
  decode_fast_kernel<<<dim3(p.n_chunks, p.hkv, p.batch), dim3(kThreads), 0, stream>>>(p);
  merge_fast_kernel<<<dim3(p.rows, p.hkv, p.batch), dim3(kD), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill_fast(const DecodeParams& p, hipStream_t stream) {
  const int n_rg = (p.rows + kPfRows - 1) / kPfRows;
  if (p.n_chunks < 1 || p.n_chunks > kMaxChunks || p.hkv > 65535 || p.batch > 65535 || p.d != kD || p.rows < 1 ||
      p.chunk > kPfMaxChunk || p.chunk % kTile || (int64_t)p.n_chunks * n_rg > 65535 || !p.qrot)
    return hipErrorInvalidValue;
  hipError_t e = launch_qprep(p, stream);
  if (e != hipSuccess) return e;
  prefill_fast_kernel<<<dim3(p.n_chunks * n_rg, p.hkv, p.batch), dim3(kThreads), 0, stream>>>(p);
  merge_fast_kernel<<<dim3(p.rows, p.hkv, p.batch), dim3(kD), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace tq
