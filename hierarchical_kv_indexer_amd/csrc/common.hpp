// Device-side building blocks shared by the CSA2 kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kKvDim = 512;
constexpr int kKvCodeBytes = 256;
constexpr int kKvScaleBytes = 32;
constexpr int kBlock = 8;          // positions per pool block
constexpr int kMaxPool = 16384;    // largest pool (2048 blocks x 8 positions)
constexpr int kMaxTopK = 2048;
constexpr int kDensePoolBlocks = kMaxPool;   // block keys a dense pool selection holds (16 per thread)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.
// Lane l holds A row (l % 16), k = 8*(l/16) .. +7; B column (l % 16), same k;
// C column (l % 16), rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
// The same product with fp16 inputs.
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// Two E2M1 codes (byte SEL of `w`, low nibble first) times a scale held twice in `s` -> two fp16.
// With an E4M3 scale the product has at most 6 significant bits within [2^-10, 2688]: exact.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_to_f16x2(uint32_t w, h2 s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL) * s);
}
// Two E4M3 bytes (the low or high 16 bits of `w`) -> two fp16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
// 8 E4M3 bytes (two dwords) -> 8 fp16, byte order preserved.
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8(uint32_t d0, uint32_t d1) {
  return u32x4{e4m3x2_to_f16x2<false>(d0), e4m3x2_to_f16x2<true>(d0), e4m3x2_to_f16x2<false>(d1),
               e4m3x2_to_f16x2<true>(d1)};
}

// Two E4M3 bytes (the low or high 16 bits of `w`) -> two bf16 (exact: E4M3 has 4 significant
// bits and its exponent range lies inside bf16's).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 E4M3 bytes (two dwords) -> 8 bf16 (one MFMA operand), byte order preserved.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  u32x4 r;
  r.x = e4m3x2_to_bf16x2<false>(d0);
  r.y = e4m3x2_to_bf16x2<true>(d0);
  r.z = e4m3x2_to_bf16x2<false>(d1);
  r.w = e4m3x2_to_bf16x2<true>(d1);
  return r;
}

// Two E2M1 codes (byte SEL of `w`, low nibble first) times an E4M3 scale -> two bf16.
// The hardware conversion is used with a unit scale only: its scale operand contributes just
// its power-of-two exponent.  The fp32 product code * scale is exact (at most 6 significant
// bits, magnitude within [2^-10, 2688]), so its upper 16 bits are the exact bf16 value.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_to_bf16x2(uint32_t w, float scale) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const uint32_t a = __float_as_uint(v.x * scale), b = __float_as_uint(v.y * scale);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);          // upper halves of a (low) and b (high)
}

// E4M3 byte -> float, exact (software decode; used for scales and the query path).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;                 // m/8 * 2^-6 = m * 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1 + m/8) * 2^(e-7)
  if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  return s ? -v : v;
}

// float -> E4M3 byte: round to nearest even, saturate to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                       // NaN
  float fa = __uint_as_float(a);
  if (fa >= 448.0f) return sign | 0x7eu;                    // saturate (includes +-inf)
  if (fa < 0.015625f) {                                     // below 2^-6: subnormal grid 2^-9
    float q = __builtin_rintf(fa * 512.0f);                 // exact scaling, round half even
    return sign | (uint32_t)q;                              // q == 8 is the code of 2^-6
  }
  uint32_t exp = (a >> 23) - 127u + 7u;                     // E4M3 exponent field (1..15)
  uint32_t mant = a & 0x7fffffu;
  uint32_t m3 = mant >> 20, rem = mant & 0xfffffu;
  uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (m3 & 1u));
  uint32_t code = (exp << 3) + m3 + up;                     // a carry moves into the exponent
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// E2M1 magnitude code (0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6) of |x| / s for an E4M3 scale s > 0:
// the number of decision points passed, 0.25, 1.25, 2.5 and 5 strictly (their ties go down to
// the even code) and 0.75, 1.75 and 3.5 inclusively (their ties go up), compared with the exact
// products t * s.  For a bf16 |x| this equals nearest-even rounding of the binary32 quotient:
// x has 8 significant bits and t * s at most 7, so when |x| != t * s they differ by at least
// ~2^-9 relative, far more than the quotient's rounding.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a, float s) {
  return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
         (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
         (uint32_t)(a > 5.0f * s);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving 32-bit key of a float score (larger score -> larger key; -0 counts as +0).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Ranking key of (score key, index): larger key first, then smaller index first.
__device__ __forceinline__ uint64_t rank_key(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t rank_key_index(uint64_t rk) {
  return 0xffffffffu - (uint32_t)(rk & 0xffffffffu);
}

__device__ __forceinline__ int bitlen64(uint64_t x) { return x ? 64 - __clzll(x) : 0; }

// ---- cross-lane helpers (wave64)

// Sum of x over lane pairs l, l^16, combined in the same order on both lanes.
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum of x over lane pairs l, l^32, combined in the same order on both lanes.
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max of x over the aligned group of 8 lanes containing this lane (result in every lane).
__device__ __forceinline__ uint32_t max8_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  return x;
}
// Workgroup barrier that orders LDS only.  __syncthreads also orders global memory, so each
// wave first waits for every global load and store it has in flight (a prefetch, or stores of
// results, which take microseconds to complete while the GPU streams from HBM); kernels whose
// waves share data only through LDS use this instead.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// DPP wave64 primitives (no LDS traffic).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t swap16(uint32_t x) {   // value of lane l ^ 16
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t swap32(uint32_t x) {   // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
}
// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += dpp_or_zero<0x111>(x);          // row_shr:1
  x += dpp_or_zero<0x112>(x);          // row_shr:2
  x += dpp_or_zero<0x114>(x);          // row_shr:4
  x += dpp_or_zero<0x118>(x);          // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);     // row_bcast:15 into rows 1, 3
  x += dpp_or_zero<0x143, 0xc>(x);     // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_mov<0xB1>(x));        // quad_perm [1,0,3,2]
  x = max(x, dpp_mov<0x4E>(x));        // quad_perm [2,3,0,1]
  x = max(x, dpp_mov<0x141>(x));       // row_half_mirror
  x = max(x, dpp_mov<0x140>(x));       // row_mirror
  x = max(x, swap16(x));
  x = max(x, swap32(x));
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_mov<0xB1>(x));
  x = min(x, dpp_mov<0x4E>(x));
  x = min(x, dpp_mov<0x141>(x));
  x = min(x, dpp_mov<0x140>(x));
  x = min(x, swap16(x));
  x = min(x, swap32(x));
  return x;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  x += swap16(x);
  x += swap32(x);
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t w = shfl_xor_u64(v, o);
    v = w > v ? w : v;
  }
  return v;
}

}  // namespace csa2
