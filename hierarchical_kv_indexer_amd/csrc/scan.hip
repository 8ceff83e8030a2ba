// Indexer scoring on gfx950: the Full scan over every visible position and the Reindex
// scoring of pool positions.
//
// Score of position p for one query (blog.4sapi.com sec.4, readance.app sec.4.2/4.3, with
// the score form this library fixes): s[p] = sum_h w[h] * ReLU(q8[h] . k[p]), 32 heads,
// 128-dim E4M3 keys shared by the heads, q8 = the bf16 query rounded to E4M3.
//
// The contraction runs on bf16 MFMA (16x16x32).  E4M3 values are exact in bf16 and their
// products are exact in fp32, so each head's dot product is an fp32 sum of exact terms.  The
// fp8 MFMA of gfx950 was measured to drop low-order product bits relative to the largest
// product of a group, so it is not used for scoring.
//
// Tile = 16 positions x 32 heads x 128 channels.  Lane l (column j = l % 16, k-group
// g = l / 16) loads 32 bytes of row j: bytes [16g, 16g+16) and [64+16g, 64+16g+16), so one
// 16-byte load instruction of the wave covers 16 whole 64-byte half rows.  The channel
// order inside an MFMA does not matter as long as the query operands use the same order,
// which they do (both are read with the same byte offsets).
//
// FP4 indexer (the V4 indexer stored its queries and keys in FP4; animattoys.com, FP4 section):
// a position's key is 64 bytes of E2M1 codes (channel 2i in the low nibble of byte i) and 8 E4M3
// scales, one per 16 channels, stored as two arrays.  With such keys the query is rounded to the
// same format (per head and 16 channels: scale E4M3(amax/6), codes E2M1), instead of to E4M3.
// Both code x scale values are exact in fp16, so that contraction runs on the fp16 MFMA, again
// with exact products.  Lane (j, g) then takes channels [32g, 32g+32) of row j: its 16 code
// bytes and the row's 8 scale bytes (two of which it uses), and MFMA chunk c covers its
// channels 32g + 8c .. +7 on both operands.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

// ---------------------------------------------------------------------------- query prep

__global__ void k_quantize_query(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                                 int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)f32_to_e4m3(bf16_bits_to_f32(in[i]));
}

hipError_t launch_quantize_query(const uint16_t* in, uint8_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_quantize_query, dim3((unsigned)blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

// Two bf16 query values (low half first) rounded to E4M3 (nearest, ties to even, saturating at
// +-448) and returned as a bf16 pair (E4M3 values are exact in bf16): clamp, the hardware
// conversion to E4M3 bytes, and its exact conversion back.
__device__ __forceinline__ uint32_t q8_pair(uint32_t w) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const float lo = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w & 0xffffu), -448.f, 448.f);
  const float hi = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w >> 16), -448.f, 448.f);
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, lo, hi, 1.0f, false));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false));
}

// FP4 rounding of the query for FP4 keys, in the keys' own format: per head and 16-channel
// group, scale = E4M3(amax / 6) with a binary32 division, each value E2M1(x / scale) (nearest,
// ties to the even code, saturating at 6, sign kept), all zero when the scale is 0.  The code is
// the number of decision points passed (see e2m1_mag_code), compared with the group's exact
// products t * scale; the value code x scale is exact in fp16 (at most 6 significant bits within
// [2^-10, 2688]).
struct Q4Group {
  float lim[7];   // decision points x scale: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (ties down / up)
  float val[7];   // magnitudes x scale above each point: 0.5, 1, 1.5, 2, 3, 4, 6
};
__device__ __forceinline__ Q4Group q4_group(uint32_t amax_bits) {
  const float s = e4m3_to_f32(f32_to_e4m3(bf16_bits_to_f32(amax_bits) / 6.0f));
  constexpr float kLim[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  constexpr float kVal[7] = {0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  Q4Group g;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    g.lim[i] = s > 0.f ? kLim[i] * s : INFINITY;     // a zero scale keeps every value at 0
    g.val[i] = kVal[i] * s;
  }
  return g;
}
// Two bf16 query values (low half first) of one group -> fp16 pair of code x scale.
__device__ __forceinline__ uint32_t q4_pair(uint32_t w, const Q4Group& g) {
  auto one = [&](uint32_t b) {
    const float a = fabsf(bf16_bits_to_f32(b));
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 7; ++i) v = ((i & 1) ? a >= g.lim[i] : a > g.lim[i]) ? g.val[i] : v;
    return (b & 0x8000u) ? -v : v;
  };
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(one(w & 0xffffu), one(w >> 16)));
}
// Largest magnitude bit pattern of the bf16 pair w (patterns order like magnitudes).
__device__ __forceinline__ uint32_t amax_bits2(uint32_t w) { return max(w & 0x7fffu, (w >> 16) & 0x7fffu); }

// The 32x128 query of one indexer head set, held in LDS as MFMA operands: rounded to E4M3 and held
// as bf16 for E4M3 keys; rounded to FP4 (q4_group) and held as fp16 for FP4 keys.
// NT threads, 4096/NT consecutive values each, loaded with 16-byte (or 8-byte) loads; for FP4 keys
// each thread loads the whole 16-channel group its values belong to.
template <int NT, bool kFp4 = false>
__device__ __forceinline__ void stage_query(const uint16_t* __restrict__ q, uint16_t* qlds) {
  constexpr int kPer = kIdxHeads * kIdxDim / NT;      // values per thread (16 or 4)
  static_assert(kPer == 16 || kPer == 4, "query staging assumes 256 or 1024 threads");
  const int base = threadIdx.x * kPer;
  uint32_t w[kPer / 2];
  if constexpr (kPer == 16) {
    const u32x4 a = *(const u32x4*)(q + base);
    const u32x4 b = *(const u32x4*)(q + base + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
    const u32x2 a = *(const u32x2*)(q + base);
    w[0] = a.x; w[1] = a.y;
  }
  uint32_t o[kPer / 2];
  if constexpr (kFp4) {
    // a group is this thread's 16 values, or those of 4 consecutive lanes (amax over the quad)
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i) m = max(m, amax_bits2(w[i]));
    if constexpr (kPer == 4) {
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
      m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    }
    const Q4Group g = q4_group(m);
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i) o[i] = q4_pair(w[i], g);
  } else {
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i) o[i] = q8_pair(w[i]);
  }
  if constexpr (kPer == 16) {
    *(u32x4*)(qlds + base) = u32x4{o[0], o[1], o[2], o[3]};
    *(u32x4*)(qlds + base + 8) = u32x4{o[4], o[5], o[6], o[7]};
  } else {
    *(u32x2*)(qlds + base) = u32x2{o[0], o[1]};
  }
}

// Per-wave state for scoring tiles: the query as MFMA A operands and this lane's head weights.
struct TileCtx {
  u32x4 qa[2][4];   // [head half][channel chunk]
  float w[8];       // heads 4g+v (v<4) and 16+4g+v
};

// Channel offset of chunk c (0..3) for k-group g: chunks 0/1 come from the first 64 bytes of a
// row, chunks 2/3 from the last 64.
__device__ __forceinline__ int chunk_base(int c, int g) { return (c >> 1) * 64 + 16 * g + (c & 1) * 8; }

__device__ __forceinline__ void load_ctx(TileCtx& cx, const uint16_t* qlds, const float* __restrict__ w) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      cx.qa[hh][c] = *(const u32x4*)(qlds + (16 * hh + j) * kIdxDim + chunk_base(c, g));
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    cx.w[v] = w[4 * g + v];
    cx.w[4 + v] = w[16 + 4 * g + v];
  }
}

// ReLU on the bit pattern: a negative float (sign bit set) is a negative int, so an integer max
// with 0 maps it to +0 and leaves non-negative values unchanged (one instruction, no NaN
// canonicalisation).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Score of this lane's row from the key operands b[c] (bf16, or fp16 with kF16), laid out as the
// query operands.  The 8 heads of a lane are summed in a fixed order, then the four k-groups are
// combined as (g0 + g1) + (g2 + g3), identically on every lane.
template <bool kF16>
__device__ __forceinline__ float operand_score(const TileCtx& cx, const u32x4 (&b)[4]) {
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (kF16) {
      a0 = mfma16x16x32_f16(cx.qa[0][c], b[c], a0);
      a1 = mfma16x16x32_f16(cx.qa[1][c], b[c], a1);
    } else {
      a0 = mfma16x16x32(cx.qa[0][c], b[c], a0);
      a1 = mfma16x16x32(cx.qa[1][c], b[c], a1);
    }
  }
  float p = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[v], relu_bits(a0[v]), p);
#pragma unroll
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[4 + v], relu_bits(a1[v]), p);
  return sum_xor32(sum_xor16(p));
}

// E4M3 key bytes of a lane (two 16-byte pieces of its row) as bf16 operands (exact).
__device__ __forceinline__ void e4m3_operands(u32x4 lo, u32x4 hi, u32x4 (&b)[4]) {
  b[0] = e4m3x8_to_bf16x8(lo.x, lo.y);
  b[1] = e4m3x8_to_bf16x8(lo.z, lo.w);
  b[2] = e4m3x8_to_bf16x8(hi.x, hi.y);
  b[3] = e4m3x8_to_bf16x8(hi.z, hi.w);
}

// Score of this lane's row (column j of the tile); every lane of a column gets the same value.
__device__ __forceinline__ float tile_score(const TileCtx& cx, u32x4 lo, u32x4 hi) {
  u32x4 b[4];
  e4m3_operands(lo, hi, b);
  return operand_score<false>(cx, b);
}

__device__ __forceinline__ void load_row(const uint8_t* __restrict__ row, int g, u32x4& lo, u32x4& hi) {
  lo = *(const u32x4*)(row + 16 * g);
  hi = *(const u32x4*)(row + 64 + 16 * g);
}

// The raw bytes of one tile row as one lane holds them: E4M3 keys, the lane's two 16-byte pieces;
// FP4 keys, its 16 code bytes and the two scale bytes of its channels (groups 2g and 2g+1).
template <bool kFp4> struct TileRaw;
template <> struct TileRaw<false> { u32x4 lo, hi; };
template <> struct TileRaw<true> { u32x4 codes; uint32_t sc; };

__device__ __forceinline__ void load_row_fp4(const uint8_t* __restrict__ codes_row,
                                             const uint8_t* __restrict__ scales_row, int g, TileRaw<true>& r) {
  r.codes = *(const u32x4*)(codes_row + 16 * g);
  r.sc = *(const uint16_t*)(scales_row + 2 * g);
}

// Query operands in the FP4 channel order (chunk c of lane group g: channels 32g + 8c .. +7).
__device__ __forceinline__ void load_ctx_fp4(TileCtx& cx, const uint16_t* qlds, const float* __restrict__ w) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      cx.qa[hh][c] = *(const u32x4*)(qlds + (16 * hh + j) * kIdxDim + 32 * g + 8 * c);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    cx.w[v] = w[4 * g + v];
    cx.w[4 + v] = w[16 + 4 * g + v];
  }
}

// FP4 keys (same head sum as tile_score): the keys are decoded to fp16 (E2M1 by the hardware
// conversion, times the E4M3 scale in packed fp16: every product has at most 6 significant bits
// within [2^-10, 2688], so it is exact) and the query operands are fp16 too, so the contraction
// runs on the fp16 MFMA with exact products.
// 16 code bytes (channels 32g .. 32g+31) and the two scale bytes of their groups -> fp16 operands.
__device__ __forceinline__ void fp4_operands(u32x4 codes, uint32_t sc2, u32x4 (&b)[4]) {
  const h2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc2, 1.0f, false);   // groups 2g, 2g+1 (exact)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const h2 s = c < 2 ? h2{sc.x, sc.x} : h2{sc.y, sc.y};
    b[c] = u32x4{e2m1x2_scaled_to_f16x2<0>(codes[c], s), e2m1x2_scaled_to_f16x2<1>(codes[c], s),
                 e2m1x2_scaled_to_f16x2<2>(codes[c], s), e2m1x2_scaled_to_f16x2<3>(codes[c], s)};
  }
}
__device__ __forceinline__ float tile_score_fp4(const TileCtx& cx, const TileRaw<true>& r) {
  u32x4 b[4];
  fp4_operands(r.codes, r.sc, b);
  return operand_score<true>(cx, b);
}

// One tile row of either key format.
template <bool kFp4>
__device__ __forceinline__ void load_key(const uint8_t* __restrict__ kseq, const uint8_t* __restrict__ sseq,
                                         int64_t p, int g, TileRaw<kFp4>& r) {
  if constexpr (kFp4) load_row_fp4(kseq + p * (kIdxDim / 2), sseq + p * (kIdxDim / 16), g, r);
  else load_row(kseq + p * kIdxDim, g, r.lo, r.hi);
}
template <bool kFp4>
__device__ __forceinline__ float key_score(const TileCtx& cx, const TileRaw<kFp4>& r) {
  if constexpr (kFp4) return tile_score_fp4(cx, r);
  else return tile_score(cx, r.lo, r.hi);
}
template <bool kFp4>
__device__ __forceinline__ void key_ctx(TileCtx& cx, const uint16_t* qlds, const float* __restrict__ w) {
  if constexpr (kFp4) load_ctx_fp4(cx, qlds, w);
  else load_ctx(cx, qlds, w);
}

// ---------------------------------------------------------------------------- block scores

// Block score variants for the candidate pool (the order key of one block of 8 positions, held by
// an aligned group of 8 lanes, each with one position's score and whether it is visible):
//   kBlockMax   the largest visible score (the pool's block score);
//   kBlockSum   the sum of the visible scores (fp32, pairwise in a fixed order);
//   kBlockTop2  the mean of the two largest visible scores (one visible score: that score).
// A block with no visible position gets key 0.  Every lane of the group returns the same key.
// Called by whole waves (the top-2 variant counts with ballots).
__device__ __forceinline__ float max8_f32(float x) {
  x = fmaxf(x, __uint_as_float(dpp_mov<0xB1>(__float_as_uint(x))));    // quad_perm [1,0,3,2]
  x = fmaxf(x, __uint_as_float(dpp_mov<0x4E>(__float_as_uint(x))));    // quad_perm [2,3,0,1]
  x = fmaxf(x, __uint_as_float(dpp_mov<0x141>(__float_as_uint(x))));   // row_half_mirror
  return x;
}
__device__ __forceinline__ float sum8_f32(float x) {
  x += __uint_as_float(dpp_mov<0xB1>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<0x4E>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<0x141>(__float_as_uint(x)));
  return x;
}
template <int kBS>
__device__ __forceinline__ uint32_t block_key(float sc, bool valid) {
  if constexpr (kBS == kBlockMax) {
    return max8_u32(valid ? score_key(sc) : 0u);
  } else if constexpr (kBS == kBlockSum) {
    const uint64_t group = 0xffull << (threadIdx.x & 56);
    const bool any = (__ballot(valid) & group) != 0;
    const float sum = sum8_f32(valid ? sc : 0.f);
    return any ? score_key(sum) : 0u;
  } else {
    const uint64_t group = 0xffull << (threadIdx.x & 56);
    const int nvalid = __popcll(__ballot(valid) & group);
    const float x = valid ? sc : -INFINITY;
    const float m1 = max8_f32(x);
    const int n_m1 = __popcll(__ballot(valid && x == m1) & group);
    const float second = max8_f32(x == m1 ? -INFINITY : x);
    const float m2 = n_m1 >= 2 ? m1 : second;
    return nvalid == 0 ? 0u : score_key(nvalid >= 2 ? (m1 + m2) * 0.5f : m1);
  }
}

// ---------------------------------------------------------------------------- 32-row FP4 tiles

// The one-query scan over FP4 keys scores 32 rows per tile with 32x32x16 fp16 MFMAs (32 heads x
// 32 rows x 16 channels): lane l takes row l % 32 and the half h = l / 32 of its channels,
// [64h, 64h + 64), so its 32 code bytes and the 4 scale bytes of its groups are contiguous, and
// K-step c covers channels 64h + 8c .. +7 (the query operands follow the same order).  Each lane
// then holds 16 heads of its row, so the head sum is 16 fused multiply-adds and one exchange with
// lane l ^ 32.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
struct TileRaw32 {
  u32x4 c0, c1;          // code bytes 32h .. 32h+31 of the row
  uint32_t sc;           // scale bytes 4h .. 4h+3
};
struct Ctx32f {
  u32x4 qa[8];           // fp16 query operands: head l % 32, channels 64h + 8c .. +7 in qa[c]
  float w[16];           // weights of the heads output v holds: 8(v/4) + 4h + v%4
};
__device__ __forceinline__ void load_row32(const uint8_t* __restrict__ kseq, const uint8_t* __restrict__ sseq,
                                           int64_t p, TileRaw32& r) {
  const int h = (threadIdx.x >> 5) & 1;
  const u32x4* cp = (const u32x4*)(kseq + p * (kIdxDim / 2) + 32 * h);
  r.c0 = cp[0];
  r.c1 = cp[1];
  r.sc = *(const uint32_t*)(sseq + p * (kIdxDim / 16) + 4 * h);
}
__device__ __forceinline__ void load_ctx32f(Ctx32f& cx, const uint16_t* qlds, const float* __restrict__ w) {
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) cx.qa[c] = *(const u32x4*)(qlds + r * kIdxDim + 64 * h + 8 * c);
#pragma unroll
  for (int v = 0; v < 16; ++v) cx.w[v] = w[8 * (v >> 2) + 4 * h + (v & 3)];
}
__device__ __forceinline__ float score32f(const Ctx32f& cx, const TileRaw32& r) {
  const h2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sc, 1.0f, false);   // groups 4h, 4h+1
  const h2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sc, 1.0f, true);    // groups 4h+2, 4h+3
  const uint32_t wd[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
  f32x16_t a;
#pragma unroll
  for (int v = 0; v < 16; ++v) a[v] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {                       // word c: channels 64h + 8c .. +7
    const _Float16 sv = c < 2 ? s01.x : (c < 4 ? s01.y : (c < 6 ? s23.x : s23.y));
    const h2 sc = h2{sv, sv};
    const u32x4 bk = {e2m1x2_scaled_to_f16x2<0>(wd[c], sc), e2m1x2_scaled_to_f16x2<1>(wd[c], sc),
                      e2m1x2_scaled_to_f16x2<2>(wd[c], sc), e2m1x2_scaled_to_f16x2<3>(wd[c], sc)};
    a = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, cx.qa[c]), __builtin_bit_cast(h8, bk), a,
                                                0, 0, 0);
  }
  float p = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) p = fmaf(cx.w[v], relu_bits(a[v]), p);
  return sum_xor32(p);
}

// ---------------------------------------------------------------------------- Full scan

// Tiles per pipeline stage of a wave: 3 tiles of 16 rows for E4M3 keys, 2 of 32 rows for FP4 keys
// (the register budget of 16 waves per workgroup).
template <bool kFp4> constexpr int kScanU = kFp4 ? 2 : 3;
constexpr int kFullWaves = kFullThreads / 64;   // 16
constexpr int kMaxScanChunk = 8192;             // positions of a one-query scan workgroup (LDS staging)
static_assert(kFullWaves == kScanUnitsPerWg, "each wave lists the units of its own range");

// LDS of k_idx_scan: the query (bf16), the chunk's scores and block keys, the stage counter, and
// the five largest packed blocks of each of the workgroup's units (for its chunk list).
size_t scan_lds_bytes(int chunk) {
  return (size_t)kIdxHeads * kIdxDim * 2 + (size_t)chunk * 4 + (size_t)(chunk / kBlock) * 4 + 16 +
         (size_t)kScanUnitsPerWg * 5 * 4;
}

// Best ranking key (score key, block) of a wave's blocks (one per lane), removed from the
// set.  Entries are (key, block) with key 0 / block 0xffffffff meaning "none"; returns
// rank_key or 0.
// Max / min over aligned groups of LANES lanes (8, 16, 32 or 64); every lane of a group gets
// its group's value.
template <int LANES>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t x) {
  if constexpr (LANES == 64) return wave_max_u32(x);
  x = max(x, dpp_mov<0xB1>(x));                          // quad_perm [1,0,3,2]
  x = max(x, dpp_mov<0x4E>(x));                          // quad_perm [2,3,0,1]
  x = max(x, dpp_mov<0x141>(x));                         // row_half_mirror
  if constexpr (LANES >= 16) x = max(x, dpp_mov<0x140>(x));   // row_mirror
  if constexpr (LANES >= 32) x = max(x, swap16(x));
  return x;
}
template <int LANES>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t x) {
  if constexpr (LANES == 64) return wave_min_u32(x);
  x = min(x, dpp_mov<0xB1>(x));
  x = min(x, dpp_mov<0x4E>(x));
  x = min(x, dpp_mov<0x141>(x));
  if constexpr (LANES >= 16) x = min(x, dpp_mov<0x140>(x));
  if constexpr (LANES >= 32) x = min(x, swap16(x));
  return x;
}

// Best ranking key (score key, block) of a group's blocks (one per lane), removed from the
// set.  Entries are (key, block) with key 0 / block 0xffffffff meaning "none"; returns
// rank_key or 0.
template <int LANES>
__device__ __forceinline__ uint64_t group_pop_best(uint32_t& key, uint32_t& blk) {
  const uint32_t m = group_max_u32<LANES>(key);
  const uint32_t jm = group_min_u32<LANES>(key == m ? blk : 0xffffffffu);
  if (key == m && blk == jm) { key = 0u; blk = 0xffffffffu; }
  return (m == 0u && jm == 0xffffffffu) ? 0ull : rank_key(m, jm);
}

// The five best blocks of the aligned group of LANES lanes holding this lane (lane i of a group
// holds one block), as ranking keys (0 = none), the same in every lane of the group.
template <int LANES>
__device__ __forceinline__ void unit_best(uint32_t key, uint32_t blk, uint64_t (&best)[5]) {
#pragma unroll
  for (int r = 0; r < 5; ++r) best[r] = group_pop_best<LANES>(key, blk);
}

// Value of lane ^ J for J in {1, 2, 4, 8, 16, 32}.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return dpp_mov<0xB1>(v);                       // quad_perm [1,0,3,2]
  else if constexpr (J == 2) return dpp_mov<0x4E>(v);                  // quad_perm [2,3,0,1]
  else if constexpr (J == 4 || J == 8) {
    // row_shl:J into the lanes whose bit J is clear (banks 0, 2 for J = 4; 0, 1 for J = 8), then
    // row_shr:J into the others
    constexpr int kLo = J == 4 ? 0x5 : 0x3;
    const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x100 | J, 0xF, kLo, false);
    return (uint32_t)__builtin_amdgcn_update_dpp((int)t, (int)v, 0x110 | J, 0xF, 0xF ^ kLo, false);
  }
  else if constexpr (J == 16) return swap16(v);
  else return swap32(v);
}
// One compare-exchange stage of a bitonic network over the lanes of a wave (block size K,
// distance J): the lower lane of each pair keeps the larger value where its K-block sorts
// descending, else the smaller.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t x) {
  const int lane = threadIdx.x & 63;
  const uint32_t y = lane_xor<J>(x);
  return (((lane & J) == 0) == ((lane & K) == 0)) ? max(x, y) : min(x, y);
}
// Sorts x descending over each aligned group of N lanes (N = 16 or 64).
template <int N>
__device__ __forceinline__ uint32_t bitonic_sort(uint32_t x) {
#define CSA2_BSTEP(K, J) if constexpr ((K) <= N) x = bitonic_step<K, J>(x);
  CSA2_BSTEP(2, 1)
  CSA2_BSTEP(4, 2) CSA2_BSTEP(4, 1)
  CSA2_BSTEP(8, 4) CSA2_BSTEP(8, 2) CSA2_BSTEP(8, 1)
  CSA2_BSTEP(16, 8) CSA2_BSTEP(16, 4) CSA2_BSTEP(16, 2) CSA2_BSTEP(16, 1)
  CSA2_BSTEP(32, 16) CSA2_BSTEP(32, 8) CSA2_BSTEP(32, 4) CSA2_BSTEP(32, 2) CSA2_BSTEP(32, 1)
  CSA2_BSTEP(64, 32) CSA2_BSTEP(64, 16) CSA2_BSTEP(64, 8) CSA2_BSTEP(64, 4) CSA2_BSTEP(64, 2) CSA2_BSTEP(64, 1)
#undef CSA2_BSTEP
  return x;
}

// Chunk lists work on packed block keys: a block at offset o of a chunk of 2^ob blocks with key
// k > 0 packs to max(1, (k >> ob) << ob | (2^ob - 1 - o)), an empty block to 0.  Packed values of
// non-empty blocks are distinct and order blocks by their truncated key, then by block (lower
// block first), so a packed bound c bounds the exact ranking key of every block whose packed
// value is at most c by unpack_cut(c).
__device__ __forceinline__ uint32_t pack_block(uint32_t key, int off, int ob) {
  if (key == 0u) return 0u;
  const uint32_t m = (1u << ob) - 1u;
  return max(1u, (key & ~m) | (m - (uint32_t)off));
}
__device__ __forceinline__ uint64_t unpack_cut(uint32_t c, int ob) {
  return c == 0u ? 0ull : ((uint64_t)(c | ((1u << ob) - 1u)) << 32) | 0xffffffffull;
}

// The chunk list, computed by wave 0 from the five best packed blocks of each of the chunk's 16
// units in LDS (u5[5u + r], r < 4 the four best, r = 4 the fifth): of the 64 listed values and
// the largest fifth mc, the values above mc among the 16 largest, in block order, as `entry` of
// lanes 0..15 (exact ranking keys read from the chunk's block keys; 0 padded), and the cut
// unpack_cut(max(mc, the 17th largest listed value)).  Every block of the chunk that is not in its
// list is bounded by that cut: a block outside its unit's four packs at or below the unit's fifth,
// and a listed value left out is at or below mc or the 17th.  The 64 values are sorted by a
// bitonic network across the wave, the kept ones then by block.
__device__ __forceinline__ void wave_chunk_list(const uint32_t* u5, const uint32_t* wkeys, uint32_t blk0, int ob,
                                                uint64_t& entry, uint64_t& cut) {
  const int lane = threadIdx.x & 63;
  uint32_t x = u5[5 * (lane >> 2) + (lane & 3)];
  const uint32_t mc = wave_max_u32(lane < kFullWaves ? u5[5 * lane + 4] : 0u);
  x = bitonic_sort<64>(x);                                      // lane i: the i-th largest
  const uint32_t c17 = (uint32_t)__builtin_amdgcn_readlane((int)x, kListLen);
  const uint32_t m = (1u << ob) - 1u;
  const bool keep = lane < kListLen && x > mc;
  // kept values by block: 1 + (2^ob - 1 - offset), descending
  const uint32_t z = bitonic_sort<16>(keep ? (x & m) + 1u : 0u);
  const bool listed = lane < kListLen && z != 0u;
  const int off = listed ? (int)(m - (z - 1u)) : 0;
  entry = listed ? rank_key(wkeys[off], blk0 + (uint32_t)off) : 0ull;
  cut = unpack_cut(max(mc, c17), ob);
}

// grid (n_wg, Q), one workgroup of 16 waves per chunk of positions (sized so the grid is about
// one workgroup per CU).  The waves take pipeline stages of kScanU tiles from an LDS counter,
// so a wave that the CU's arbitration favours simply takes more stages and all waves finish
// together.  Each wave keeps one stage of loads in flight while it scores the previous one;
// the loop issues no global stores (scores and block keys are staged in LDS and stored once
// every tile is done).
//
// Writes scores[q][p] for p < n_visible and, when `blkkey` is non-null, the order key of
// each block's max score.  When `lists` is non-null, each of the chunk's 16*upw units (equal,
// contiguous ranges of chunk/(16*upw) positions) writes its five best blocks as ranking keys
// (score key << 32 | ~block): lists[q][unit][0..3] = the four best (0 = none) and
// cuts[q][unit] = the fifth best (0 = none), so every block of the unit that is not listed
// ranks at or below cuts[q][unit].  With `clists` non-null (one unit per wave) the chunk's list
// replaces them: clists[q][chunk][0..15] and ccuts[q][chunk] as wave_chunk_list states.  Requires
// chunk a power of two from 1024 to 8192.
template <bool kFp4, int kBS>
__global__ __launch_bounds__(kFullThreads) void k_idx_scan(
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_ks, int64_t k_rows,
    const uint16_t* __restrict__ idx_q,
    const float* __restrict__ head_w, const int32_t* __restrict__ n_visible, int T, int n_max,
    int chunk, float* __restrict__ scores, uint32_t* __restrict__ blkkey, int nb_max,
    uint64_t* __restrict__ lists, uint64_t* __restrict__ cuts, int upw, uint64_t* __restrict__ clists,
    uint64_t* __restrict__ ccuts) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  uint16_t* qlds = (uint16_t*)lds;
  float* sbuf = (float*)(lds + kIdxHeads * kIdxDim * 2);
  uint32_t* wkeys = (uint32_t*)(lds + kIdxHeads * kIdxDim * 2 + chunk * 4);
  int* ctr = (int*)(lds + kIdxHeads * kIdxDim * 2 + chunk * 4 + (chunk / kBlock) * 4);
  uint32_t* u5 = (uint32_t*)(lds + kIdxHeads * kIdxDim * 2 + chunk * 4 + (chunk / kBlock) * 4 + 16);
  const int q = blockIdx.y, b = q / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int p_begin = blockIdx.x * chunk;
  const int p_end = min(p_begin + chunk, nv);
  const int npos = max(0, p_end - p_begin);
  constexpr int kTR = kFp4 ? 32 : 16;             // rows per tile
  const int trow = kFp4 ? (lane & 31) : j;         // this lane's row of a tile
  const int ntiles = (npos + kTR - 1) / kTR;
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * (kFp4 ? kIdxDim / 2 : kIdxDim);
  const uint8_t* sseq = kFp4 ? idx_ks + (size_t)b * (size_t)k_rows * (kIdxDim / 16) : nullptr;
  const int plast = npos > 0 ? p_end - 1 : 0;
  // Workgroups start at different tiles of their chunk and wrap around, so workgroups that
  // stream in lockstep touch different address offsets at a time.
  const int rot = ntiles > 0 ? (int)((blockIdx.x * 5u + blockIdx.y) % (unsigned)ntiles) : 0;
  auto phys = [&](int t) { return t + rot < ntiles ? t + rot : t + rot - ntiles; };

  // Rows of tiles past the chunk are clamped to its last row, so every stage loads and
  // computes unconditionally; results of such tiles are never stored.  (Skipping the loads of a
  // stage past the chunk would make the loop's load waits count conservatively across the skip,
  // so each stage would wait for the next one's loads.)
  constexpr int kU = kScanU<kFp4>;
  using Raw = typename std::conditional<kFp4, TileRaw32, TileRaw<false>>::type;
  Raw rA[kU], rB[kU];
  auto load_stage = [&](Raw(&r)[kU], int t0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = t0 + u;
      const int p = min(p_begin + kTR * (t < ntiles ? phys(t) : t) + trow, plast);
      if constexpr (kFp4) load_row32(kseq, sseq, p, r[u]);
      else load_key<false>(kseq, sseq, p, g, r[u]);
    }
  };
  int tA = wave * kU;                              // first stage of each wave: static
  if (tA < ntiles) load_stage(rA, tA);             // in flight during the query prep

  if (ntiles > 0) {
    stage_query<kFullThreads, kFp4>(idx_q + (size_t)q * kIdxHeads * kIdxDim, qlds);
    if (threadIdx.x == 0) *ctr = kFullWaves * kU;
    lds_barrier();
    using Ctx = typename std::conditional<kFp4, Ctx32f, TileCtx>::type;
    Ctx cx;
    if constexpr (kFp4) load_ctx32f(cx, qlds, head_w + (size_t)q * kIdxHeads);
    else key_ctx<false>(cx, qlds, head_w + (size_t)q * kIdxHeads);
    auto grab = [&]() {                            // next stage of this wave (monotonic)
      int v = 0;
      if (lane == 0) v = atomicAdd(ctr, kU);
      return __builtin_amdgcn_readfirstlane(v);
    };
    auto compute_stage = [&](const Raw(&r)[kU], int t0) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int t = t0 + u;
        float sc;
        if constexpr (kFp4) sc = score32f(cx, r[u]);
        else sc = key_score<false>(cx, r[u]);
        if (t < ntiles) {
          const int tp = phys(t);
          const bool valid = kTR * tp + trow < npos;
          const uint32_t key = block_key<kBS>(sc, valid);
          if constexpr (kFp4) {
            if (lane < 32) sbuf[32 * tp + trow] = sc;
            if ((lane & 0x27) == 0) wkeys[4 * tp + (lane >> 3)] = key;   // lanes 0, 8, 16, 24
          } else {
            if (g == 0) sbuf[16 * tp + j] = sc;
            if ((lane & 0x37) == 0) wkeys[2 * tp + (lane >> 3)] = key;   // lanes 0, 8
          }
        }
      }
    };
    int tB = grab();
    while (tA < ntiles) {
      load_stage(rB, tB);
      compute_stage(rA, tA);
      tA = grab();
      if (tB >= ntiles) break;                     // later grabs only go further
      load_stage(rA, tA);
      compute_stage(rB, tB);
      tB = grab();
    }
  }
  lds_barrier();
  // The lists are computed before any store of the epilogue is issued: a register rewritten after
  // a store makes the wave wait for that store to complete, which takes microseconds while the
  // other workgroups stream keys.
  const int nblk = (npos + kBlock - 1) / kBlock;
  // the wave's blocks (bpu <= 64: one per lane), split into upw units of bpu/upw blocks; each
  // unit lists its five best
  const int bpu = chunk / (kBlock * kFullWaves), lanes = bpu / upw;
  const int ub = wave * bpu;
  const bool ok = lane < bpu && ub + lane < nblk;
  const uint32_t key = ok ? wkeys[ub + lane] : 0u;
  uint64_t best[5] = {0ull, 0ull, 0ull, 0ull, 0ull};
  uint64_t centry = 0ull, ccut = 0ull;
  if (clists) {
    // one unit per wave: its five largest packed blocks, then wave 0 merges the 16 units
    const int ob = 31 - __builtin_clz((unsigned)(chunk / kBlock));
    uint32_t pk = ok ? pack_block(key, ub + lane, ob) : 0u;
    uint32_t top[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      top[r] = wave_max_u32(pk);
      if (pk == top[r]) pk = 0u;
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < 5; ++r) u5[5 * wave + r] = top[r];
    }
    lds_barrier();
    if (wave == 0) wave_chunk_list(u5, wkeys, (uint32_t)(p_begin / kBlock), ob, centry, ccut);
  } else if (lists) {
    const uint32_t blk = ok ? (uint32_t)(p_begin / kBlock + ub + lane) : 0xffffffffu;
    switch (lanes) {
      case 8: unit_best<8>(key, blk, best); break;
      case 16: unit_best<16>(key, blk, best); break;
      case 32: unit_best<32>(key, blk, best); break;
      default: unit_best<64>(key, blk, best); break;
    }
  }
  // stores: the chunk's scores and block keys (coalesced), its unit lists and its chunk list
  constexpr int kSt = kMaxScanChunk / kFullThreads;
  const int nsc = scores ? npos : 0;              // scores == nullptr: block keys and lists only
  float* srow = scores + (size_t)q * n_max + p_begin;
  float sv[kSt];
#pragma unroll
  for (int u = 0; u < kSt; ++u) {
    const int i = u * kFullThreads + threadIdx.x;
    sv[u] = i < nsc ? sbuf[i] : 0.f;
  }
  const uint32_t bk = (int)threadIdx.x < nblk ? wkeys[threadIdx.x] : 0u;
#pragma unroll
  for (int u = 0; u < kSt; ++u) {
    const int i = u * kFullThreads + threadIdx.x;
    if (i < nsc) srow[i] = sv[u];
  }
  if (blkkey && (int)threadIdx.x < nblk) blkkey[(size_t)q * nb_max + p_begin / kBlock + threadIdx.x] = bk;
  if (!clists && lists && lane % lanes == 0 && lane / lanes < upw) {
    const size_t unit = (((size_t)q * gridDim.x + blockIdx.x) * kFullWaves + wave) * upw + lane / lanes;
    u32x4* lp = (u32x4*)(lists + unit * 4);
    lp[0] = u32x4{(uint32_t)best[0], (uint32_t)(best[0] >> 32), (uint32_t)best[1], (uint32_t)(best[1] >> 32)};
    lp[1] = u32x4{(uint32_t)best[2], (uint32_t)(best[2] >> 32), (uint32_t)best[3], (uint32_t)(best[3] >> 32)};
    cuts[unit] = best[4];
  }
  if (clists && wave == 0) {
    const size_t ch = (size_t)q * gridDim.x + blockIdx.x;
    if (lane < kListLen) clists[ch * kListLen + lane] = centry;
    if (lane == 0) ccuts[ch] = ccut;
  }
}

// ---------------------------------------------------------------------------- multi-query Full scan

// When many queries of one sequence scan the same keys (a prefill chunk), a workgroup scores a
// chunk of positions for 16 consecutive queries of the sequence, two per wave.  Each step stages
// 128 key rows in LDS already converted to MFMA operands (bf16 for E4M3 keys, fp16 for FP4 keys,
// both exact, channels in their natural order), so the key stream is read and converted once per
// 16 queries.  A wave scores 32 positions at a time with 32x32x16 MFMAs (32 heads x 32 positions):
// each lane then holds 16 heads of one position, so the head sum is 16 fused multiply-adds and
// one exchange with lane l ^ 32, and the block maxima of the 32 positions come from one 8-lane
// reduction.  Products are exact and accumulated in fp32, as in k_idx_scan, though in a different
// order.  Outputs are those of k_idx_scan for every query of the group (unit u of a chunk covers
// its positions [u*chunk/(16*upw), (u+1)*chunk/(16*upw))).
constexpr int kMqQueries = 16;                // queries per workgroup
constexpr int kMqRows = 128;                  // key rows per staged step
constexpr int kMqStride = 2 * kIdxDim + 16;   // LDS bytes per staged row: 128 16-bit operands + pad
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool kF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// A wave's query for 32x32x16 MFMAs: lane l holds head l % 32, channels 16c + 8(l/32) .. +7 in
// qa[c] (rounded to E4M3 as bf16 for E4M3 keys, to FP4 as fp16 for FP4 keys), and the weights
// of the heads its outputs hold:
// output v of lane l is head 8(v/4) + 4(l/32) + v%4.
struct Ctx32 {
  u32x4 qa[8];
  float w[16];
};

template <bool kF16>
__device__ __forceinline__ void load_ctx32(Ctx32& cx, const uint16_t* __restrict__ q, const float* __restrict__ w) {
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4 v = *(const u32x4*)(q + r * kIdxDim + 16 * c + 8 * h);
    if constexpr (kF16) {          // FP4 keys: group c of head r is split between lanes l and l ^ 32
      uint32_t m = max(max(amax_bits2(v.x), amax_bits2(v.y)), max(amax_bits2(v.z), amax_bits2(v.w)));
      const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
      m = max(sw[0], sw[1]);
      const Q4Group g = q4_group(m);
      cx.qa[c] = u32x4{q4_pair(v.x, g), q4_pair(v.y, g), q4_pair(v.z, g), q4_pair(v.w, g)};
    } else {
      cx.qa[c] = u32x4{q8_pair(v.x), q8_pair(v.y), q8_pair(v.z), q8_pair(v.w)};
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) cx.w[v] = w[8 * (v >> 2) + 4 * h + (v & 3)];
}

// This lane's key operands of a 32-row group of the staged step (row pointer `row`: this lane's
// row, l % 32): channels 16c + 8(l/32) .. +7 in bk[c].
__device__ __forceinline__ void load_bk32(const unsigned char* row, u32x4 (&bk)[8]) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int c = 0; c < 8; ++c) bk[c] = *(const u32x4*)(row + 32 * c + 16 * h);
}

// Two queries' MFMA chains over the same key operands of a 32-row group: a0/a1 receive the
// per-head logits of position l % 32 (heads as in Ctx32::w).
template <bool kF16>
__device__ __forceinline__ void mfma_chains32(const Ctx32& c0, const Ctx32& c1, const u32x4 (&bk)[8], f32x16& a0,
                                              f32x16& a1) {
#pragma unroll
  for (int v = 0; v < 16; ++v) a0[v] = a1[v] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    a0 = mfma32x32x16<kF16>(c0.qa[c], bk[c], a0);
    a1 = mfma32x32x16<kF16>(c1.qa[c], bk[c], a1);
  }
}

// Score of position l % 32 from its logits: sum over heads of w * relu(logit); lanes l and l ^ 32
// return the same value.
__device__ __forceinline__ float reduce32(const Ctx32& cx, const f32x16& a) {
  float p = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) p = fmaf(cx.w[v], relu_bits(a[v]), p);
  return sum_xor32(p);
}

// grid (n_wg, B * ceil(T/16)), 8 waves; wave w scores queries 2w and 2w+1 of the group, so each
// key operand read from LDS feeds two queries' MFMAs.  Step s of the chunk stages key rows
// p_begin + 128s .. +127 (rows past the group's last visible position are clamped to it and never
// scored), double-buffered: step s+1 is converted into the other buffer while step s is scored,
// and the loads of step s+2 are then in flight.  Staging: E4M3, thread t converts bytes
// 16*(t%8) .. +15 of rows t/8 and t/8 + 64 (channels 16*(t%8) .. +15); FP4, the 16 code bytes of
// row t/4 holding channels 32*(t%4) .. +31 and the two scales of their groups.
constexpr int kMqThreads = 512;
constexpr int kMqWaves = kMqThreads / 64;
constexpr int kMqPerWave = kMqQueries / kMqWaves;     // 2 queries per wave
static_assert(kMqPerWave == 2, "the step loop scores two queries per wave (mfma_chains32)");
template <bool kFp4, int kBS>
__global__ __launch_bounds__(kMqThreads) void k_idx_scan_mq(
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_ks, int64_t k_rows,
    const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w, const int32_t* __restrict__ n_visible,
    int T, int n_max, int chunk, float* __restrict__ scores, uint32_t* __restrict__ blkkey, int nb_max,
    uint64_t* __restrict__ lists, uint64_t* __restrict__ cuts, int upw) {
  __shared__ __attribute__((aligned(16))) unsigned char stage[2][kMqRows * kMqStride];
  __shared__ __attribute__((aligned(16))) float sstage[2][kMqQueries][kMqRows];   // scores of a step
  __shared__ uint32_t wkeys[kMqQueries][kMqMaxChunk / kBlock];
  const int groups = (T + kMqQueries - 1) / kMqQueries;
  const int b = blockIdx.y / groups, t0 = (blockIdx.y % groups) * kMqQueries;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = min(kMqQueries, T - t0);
  const int p_begin = blockIdx.x * chunk;
  auto visible = [&](int i) {                 // clamped n_visible of query t0 + i of the group
    const int v = n_visible[b * T + t0 + i];
    return v < 0 ? 0 : (v > n_max ? n_max : v);
  };
  int nv_max = 0;                             // the group's visible range
  for (int i = 0; i < nq; ++i) nv_max = max(nv_max, visible(i));
  bool has_q[kMqPerWave];
  int q[kMqPerWave], p_end_q[kMqPerWave];
#pragma unroll
  for (int i = 0; i < kMqPerWave; ++i) {
    const int qi = kMqPerWave * wave + i;
    has_q[i] = qi < nq;
    q[i] = b * T + t0 + (has_q[i] ? qi : 0);
    p_end_q[i] = has_q[i] ? min(p_begin + chunk, visible(qi)) : p_begin;
  }
  const int p_end = min(p_begin + chunk, nv_max);
  const int npos = max(0, p_end - p_begin);
  const int nsteps = (npos + kMqRows - 1) / kMqRows;
  const int nblk_g = (npos + kBlock - 1) / kBlock;                          // the group's blocks
  const int plast = p_end > p_begin ? p_end - 1 : 0;
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * (kFp4 ? kIdxDim / 2 : kIdxDim);
  const uint8_t* sseq = kFp4 ? idx_ks + (size_t)b * (size_t)k_rows * (kIdxDim / 16) : nullptr;

  constexpr int kReps = kFp4 ? 1 : 2;          // staged pieces per thread
  const int srow = kFp4 ? tid >> 2 : tid >> 3, piece = kFp4 ? tid & 3 : tid & 7;
  u32x4 pre[kReps];
  uint32_t pre_sc = 0u;
  auto load_step = [&](int st) {
#pragma unroll
    for (int rep = 0; rep < kReps; ++rep) {
      const int64_t p = min(p_begin + kMqRows * st + srow + 64 * rep, plast);
      if constexpr (kFp4) {
        pre[rep] = *(const u32x4*)(kseq + p * (kIdxDim / 2) + 16 * piece);
        pre_sc = *(const uint16_t*)(sseq + p * (kIdxDim / 16) + 2 * piece);
      } else {
        pre[rep] = *(const u32x4*)(kseq + p * kIdxDim + 16 * piece);
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int rep = 0; rep < kReps; ++rep) {
      unsigned char* d = stage[buf] + (srow + 64 * rep) * kMqStride;
      if constexpr (kFp4) {
        u32x4 o[4];
        fp4_operands(pre[rep], pre_sc, o);
#pragma unroll
        for (int c = 0; c < 4; ++c) *(u32x4*)(d + 64 * piece + 16 * c) = o[c];
      } else {
        *(u32x4*)(d + 32 * piece) = e4m3x8_to_bf16x8(pre[rep].x, pre[rep].y);
        *(u32x4*)(d + 32 * piece + 16) = e4m3x8_to_bf16x8(pre[rep].z, pre[rep].w);
      }
    }
  };

  // Scores of step s go to sstage[s & 1] and are written to global memory, coalesced, during step
  // s+1 (by every thread: query tid / 32, four positions each), so the stores have a whole step to
  // complete before the next wait on the staged key loads.
  const int oq = tid >> 5, opos = 4 * (tid & 31);
  const int oq_end = oq < nq ? min(p_begin + chunk, visible(oq)) : p_begin;
  float* oscores = scores + (size_t)(b * T + t0 + (oq < nq ? oq : 0)) * n_max;
  const bool rows16 = (n_max & 3) == 0;       // score rows 16-byte aligned (p is a multiple of 4)
  auto flush_scores = [&](int st) {
    const int p = p_begin + kMqRows * st + opos;
    const f32x4 v = *(const f32x4*)&sstage[st & 1][oq][opos];
    if (rows16 && p + 3 < oq_end) {
      __builtin_nontemporal_store(v, (f32x4*)(oscores + p));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p + e < oq_end) __builtin_nontemporal_store(v[e], oscores + p + e);
    }
  };
  if (nsteps > 0) {
    // The query operands are loaded before the first keys, so waiting for those keys also covers
    // them and no wait for an operand load is left inside the step loop.
    Ctx32 cx[kMqPerWave];
#pragma unroll
    for (int i = 0; i < kMqPerWave; ++i)      // a missing query scores the group's first one
      load_ctx32<kFp4>(cx[i], idx_q + (size_t)q[i] * kIdxHeads * kIdxDim, head_w + (size_t)q[i] * kIdxHeads);
    load_step(0);
    store_step(0);
    if (nsteps > 1) load_step(1);
    lds_barrier();
    const int r32 = lane & 31;
    for (int st = 0; st < nsteps; ++st) {
      if (st > 0) flush_scores(st - 1);
      const unsigned char* d = stage[st & 1] + r32 * kMqStride;
      bool act[kMqPerWave];
#pragma unroll
      for (int i = 0; i < kMqPerWave; ++i) act[i] = has_q[i] && p_begin + kMqRows * st < p_end_q[i];
      if (act[0] || act[1]) {
        // Software-pipelined over the step's 32-row groups: the MFMAs of group m+1 are issued
        // before the reductions of group m, so the two overlap within the wave.  Both queries are
        // scored; the LDS scores and keys of an inactive one lie past its visible range, where they
        // are never read.
        f32x16 acc[2][kMqPerWave];
        auto issue = [&](int m, f32x16 (&a)[kMqPerWave]) {
          u32x4 bk[8];
          load_bk32(d + 32 * m * kMqStride, bk);
          mfma_chains32<kFp4>(cx[0], cx[1], bk, a[0], a[1]);
        };
        auto finish = [&](int m, const f32x16 (&a)[kMqPerWave]) {
          const int pl = kMqRows * st + 32 * m + r32;               // position within the chunk
          float sc[kMqPerWave];
          uint32_t key[kMqPerWave];
#pragma unroll
          for (int i = 0; i < kMqPerWave; ++i) {
            sc[i] = reduce32(cx[i], a[i]);
            key[i] = block_key<kBS>(sc[i], p_begin + pl < p_end_q[i]);
          }
#pragma unroll
          for (int i = 0; i < kMqPerWave; ++i) {
            const int qi = kMqPerWave * wave + i;
            if (lane < 32) sstage[st & 1][qi][32 * m + r32] = sc[i];
            if ((lane & 0x27) == 0 && pl < 8 * nblk_g) wkeys[qi][pl >> 3] = key[i];   // lanes 0, 8, 16, 24
          }
        };
        issue(0, acc[0]);
#pragma unroll
        for (int m = 0; m < kMqRows / 32; ++m) {
          if (m + 1 < kMqRows / 32) issue(m + 1, acc[(m + 1) & 1]);
          finish(m, acc[m & 1]);
        }
      }
      if (st + 1 < nsteps) {
        store_step((st + 1) & 1);          // that buffer was last read before the previous barrier
        if (st + 2 < nsteps) load_step(st + 2);
      }
      lds_barrier();
    }
    flush_scores(nsteps - 1);
  }
  // block keys and unit lists of this wave's queries (its own LDS keys: no barrier needed)
  const int bpu = chunk / (kBlock * kScanUnitsPerWg * upw);
#pragma unroll 1
  for (int i = 0; i < kMqPerWave; ++i) {
    const int qi = kMqPerWave * wave + i;     // (recomputed: no dynamically indexed register arrays)
    if (qi >= nq) break;
    const int qg = b * T + t0 + qi;
    const uint32_t* wk = wkeys[qi];
    const int nblk = (max(0, min(p_begin + chunk, visible(qi)) - p_begin) + kBlock - 1) / kBlock;
    if (blkkey) {
      uint32_t* brow = blkkey + (size_t)qg * nb_max + p_begin / kBlock;
      for (int e = lane; e < nblk; e += 64) brow[e] = wk[e];
    }
    if (!lists) continue;
    // lane u < 16*upw keeps the five best ranking keys of unit u (bpu blocks), inserted one block
    // at a time (the keys are distinct, so the visiting order does not matter; it is rotated per
    // lane to spread the LDS reads over the banks)
    if (lane < kScanUnitsPerWg * upw) {
      const int ub = lane * bpu;
      uint64_t best[5] = {0ull, 0ull, 0ull, 0ull, 0ull};
      const int rot = lane % bpu;
      for (int e = 0; e < bpu; ++e) {
        const int o = e + rot < bpu ? e + rot : e + rot - bpu;
        uint64_t x = ub + o < nblk ? rank_key(wk[ub + o], (uint32_t)(p_begin / kBlock + ub + o)) : 0ull;
#pragma unroll
        for (int r = 0; r < 5; ++r) {
          const uint64_t hi = x > best[r] ? x : best[r];
          x = x > best[r] ? best[r] : x;
          best[r] = hi;
        }
      }
      const size_t unit = ((size_t)qg * gridDim.x + blockIdx.x) * kScanUnitsPerWg * upw + lane;
      u32x4* lp = (u32x4*)(lists + unit * 4);
      lp[0] = u32x4{(uint32_t)best[0], (uint32_t)(best[0] >> 32), (uint32_t)best[1], (uint32_t)(best[1] >> 32)};
      lp[1] = u32x4{(uint32_t)best[2], (uint32_t)(best[2] >> 32), (uint32_t)best[3], (uint32_t)(best[3] >> 32)};
      cuts[unit] = best[4];
    }
  }
}

bool scan_multi_query(int T, int n_max) { return T >= kScanMqMinT && n_max <= kMqMaxPositions; }

int scan_mq_chunk(int n_max, int B, int T) {
  // 4096 positions, or fewer (down to 1024) while the grid is under ~1024 workgroups, as long as
  // a query's positions stay within 256 chunks (the pool takes at most 4096 units)
  const long long groups = (long long)B * ((T + kMqQueries - 1) / kMqQueries);
  int c = kMqMaxChunk;
  while (c > 1024 && ((long long)n_max + c / 2 - 1) / (c / 2) <= 256 &&
         (long long)((n_max + c - 1) / c) * groups < 1024)
    c /= 2;
  return c;
}

int scan_chunk_positions(int n_max, int queries) {
  // about one workgroup per CU (256) over all queries, at most 256 workgroups per query (the
  // pool takes at most 4096 units); a power of two from 1024 to 8192 positions (LDS staging),
  // so that each wave's share of blocks splits into power-of-two units
  long long total = (long long)n_max * (queries > 0 ? queries : 1);
  long long c = (total + 255) / 256;
  long long per_query = ((long long)n_max + 255) / 256;
  if (c < per_query) c = per_query;
  long long p = 1024;
  while (p < c && p < kMaxScanChunk) p *= 2;
  return (int)p;
}

template <bool kFp4, int kBS>
static void launch_scan_variant(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows, const uint16_t* idx_q,
                                const float* head_w, const int32_t* n_visible, int Q, int T, int n_max, float* scores,
                                uint32_t* blkkey, int nb_max, uint64_t* lists, uint64_t* cuts, int chunk, int n_wg,
                                bool multi_query, int upw, uint64_t* clists, uint64_t* ccuts, hipStream_t s) {
  if (multi_query) {
    const int groups = (Q / T) * ((T + kMqQueries - 1) / kMqQueries);
    hipLaunchKernelGGL((k_idx_scan_mq<kFp4, kBS>), dim3(n_wg, groups), dim3(kMqThreads), 0, s, idx_k, idx_ks, k_rows,
                       idx_q, head_w, n_visible, T, n_max, chunk, scores, blkkey, nb_max, lists, cuts, upw);
  } else {
    hipLaunchKernelGGL((k_idx_scan<kFp4, kBS>), dim3(n_wg, Q), dim3(kFullThreads), scan_lds_bytes(chunk), s, idx_k,
                       idx_ks, k_rows, idx_q, head_w, n_visible, T, n_max, chunk, scores, blkkey, nb_max, lists,
                       cuts, upw, clists, ccuts);
  }
}

template <bool kFp4>
static void launch_scan_format(int block_score, const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows,
                               const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int Q, int T,
                               int n_max, float* scores, uint32_t* blkkey, int nb_max, uint64_t* lists,
                               uint64_t* cuts, int chunk, int n_wg, bool multi_query, int upw, uint64_t* clists,
                               uint64_t* ccuts, hipStream_t s) {
  if (block_score == kBlockSum)
    launch_scan_variant<kFp4, kBlockSum>(idx_k, idx_ks, k_rows, idx_q, head_w, n_visible, Q, T, n_max, scores, blkkey,
                                         nb_max, lists, cuts, chunk, n_wg, multi_query, upw, clists, ccuts, s);
  else if (block_score == kBlockTop2)
    launch_scan_variant<kFp4, kBlockTop2>(idx_k, idx_ks, k_rows, idx_q, head_w, n_visible, Q, T, n_max, scores,
                                          blkkey, nb_max, lists, cuts, chunk, n_wg, multi_query, upw, clists, ccuts, s);
  else
    launch_scan_variant<kFp4, kBlockMax>(idx_k, idx_ks, k_rows, idx_q, head_w, n_visible, Q, T, n_max, scores, blkkey,
                                         nb_max, lists, cuts, chunk, n_wg, multi_query, upw, clists, ccuts, s);
}

hipError_t launch_idx_scan(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* n_visible, int Q, int T, int n_max,
                           float* scores, uint32_t* blkkey, int nb_max, uint64_t* lists,
                           uint64_t* cuts, int chunk, int n_wg, bool multi_query, int block_score, int upw,
                           uint64_t* clists, uint64_t* ccuts, hipStream_t s) {
  if (block_score < kBlockMax || block_score > kBlockTop2) return hipErrorInvalidValue;
  const int bpw = chunk / (kBlock * kFullWaves);       // blocks per wave
  if (upw < 1 || bpw % upw != 0 || bpw / upw < 8 || (bpw / upw & (bpw / upw - 1)) != 0) return hipErrorInvalidValue;
  if (multi_query && (chunk % 1024 != 0 || chunk > kMqMaxChunk || Q % T != 0)) return hipErrorInvalidValue;
  if (!multi_query && (chunk < 1024 || chunk > kMaxScanChunk || (chunk & (chunk - 1)) != 0)) return hipErrorInvalidValue;
  if (clists && (multi_query || upw != 1 || !ccuts)) return hipErrorInvalidValue;   // one unit per wave
  if (idx_ks)
    launch_scan_format<true>(block_score, idx_k, idx_ks, k_rows, idx_q, head_w, n_visible, Q, T, n_max, scores, blkkey,
                             nb_max, lists, cuts, chunk, n_wg, multi_query, upw, clists, ccuts, s);
  else
    launch_scan_format<false>(block_score, idx_k, idx_ks, k_rows, idx_q, head_w, n_visible, Q, T, n_max, scores,
                              blkkey, nb_max, lists, cuts, chunk, n_wg, multi_query, upw, clists, ccuts, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- Reindex scoring

constexpr int kRiTilesPerWave = 2;
static_assert(kScanThreads / 64 * kRiTilesPerWave * 16 == kRiChunk, "a workgroup scores one chunk of slots");

// grid (n_chunks, items): item it scores pool slots [x*kRiChunk, (x+1)*kRiChunk) of its query.
//   it <  full_items  the Full layer of query q = it: the slot's key scored with the Full layer's
//                     query full_q[q] and weights full_w[q] (the arithmetic of k_idx_scan, so the
//                     scan's own score);
//   it >= full_items  Reindex layer r / Q of query q = r % Q (r = it - full_items): the slot's
//                     indexer key scored with that layer's query idx_q[r] and weights head_w[r].
// Writes slot_scores[it][slot] for slots < pool_len holding a position in [0, k_rows) (others are
// not written).  Wave w takes slots 32w .. 32w+31 of the chunk as two tiles of 16.  Eight waves per
// SIMD fit (64 registers): with many short workgroups the rate follows the waves in flight.
template <bool kFp4>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_ri_score(
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_ks, int64_t k_rows,
    const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w, int full_items,
    const uint16_t* __restrict__ full_q, const float* __restrict__ full_w,
    const int32_t* __restrict__ pool_pos, const int32_t* __restrict__ pool_len, int cap, int Q, int T,
    float* __restrict__ slot_scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kIdxHeads * kIdxDim];
  const int it = blockIdx.y;
  const bool full = it < full_items;
  const int r = it - full_items, q = full ? it : r % Q, b = q / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  // The pool length, the slots' positions and what they index are loaded without waiting for
  // one another (a position is used only if it lies in range); slots at or past the length are
  // dropped afterwards.
  const int len_raw = pool_len[q];
  const int s_begin = blockIdx.x * kRiChunk;
  const int32_t* pp = pool_pos + (size_t)q * cap;
  const int sw = s_begin + 16 * kRiTilesPerWave * wave;          // first slot of this wave
  int pos[kRiTilesPerWave];
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) {
    const int slot = sw + 16 * u + j;
    pos[u] = slot < cap ? pp[slot] : -1;
  }
  stage_query<kScanThreads, kFp4>(full ? full_q + (size_t)q * kIdxHeads * kIdxDim
                                       : idx_q + (size_t)r * kIdxHeads * kIdxDim, qlds);
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * (kFp4 ? kIdxDim / 2 : kIdxDim);
  const uint8_t* sseq = kFp4 ? idx_ks + (size_t)b * (size_t)k_rows * (kIdxDim / 16) : nullptr;
  TileRaw<kFp4> raw[kRiTilesPerWave];
  bool ok[kRiTilesPerWave];
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) {
    ok[u] = pos[u] >= 0 && (int64_t)pos[u] < k_rows;
    load_key<kFp4>(kseq, sseq, ok[u] ? pos[u] : 0, g, raw[u]);
  }
  const int len = len_raw < 0 ? 0 : (len_raw > cap ? cap : len_raw);
  const int s_end = min(s_begin + kRiChunk, len);
  if (s_end <= s_begin) return;                   // uniform across the workgroup
  lds_barrier();
  TileCtx cx;
  key_ctx<kFp4>(cx, qlds, full ? full_w + (size_t)q * kIdxHeads : head_w + (size_t)r * kIdxHeads);
  float sc[kRiTilesPerWave];
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) sc[u] = key_score<kFp4>(cx, raw[u]);
  // every lane of column j holds row j's score; lane group g < 2 stores tile g's
  if (g < kRiTilesPerWave) {
    const int slot = sw + 16 * g + j;
    if ((g == 0 ? ok[0] : ok[1]) && slot < s_end) slot_scores[(size_t)it * cap + slot] = g == 0 ? sc[0] : sc[1];
  }
}

hipError_t launch_ri_score(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, int full_items, const uint16_t* full_q, const float* full_w,
                           const int32_t* pool_pos, const int32_t* pool_len, int pool_cap, int L, int Q, int T,
                           float* slot_scores, hipStream_t s) {
  const int n_chunks = ri_chunks(pool_cap);
  const int items = full_items + L * Q;
  if (items == 0) return hipSuccess;
  if (full_items > 0 && (!full_q || !full_w)) return hipErrorInvalidValue;
  if (idx_ks)
    hipLaunchKernelGGL(k_ri_score<true>, dim3(n_chunks, items), dim3(kScanThreads), 0, s, idx_k, idx_ks, k_rows,
                       idx_q, head_w, full_items, full_q, full_w, pool_pos, pool_len, pool_cap, Q, T, slot_scores);
  else
    hipLaunchKernelGGL(k_ri_score<false>, dim3(n_chunks, items), dim3(kScanThreads), 0, s, idx_k, idx_ks, k_rows,
                       idx_q, head_w, full_items, full_q, full_w, pool_pos, pool_len, pool_cap, Q, T, slot_scores);
  return hipGetLastError();
}

}  // namespace csa2
