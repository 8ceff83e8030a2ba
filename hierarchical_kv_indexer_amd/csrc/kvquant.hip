// FP4 main-KV quantisation (gfx950): the producer of the cache that the sparse attention reads.
//
// Format (blog.4sapi.com sec.5 "FP4 KV"; animattoys.com, FP4 section): the rotated 512-wide
// latent is stored as E2M1 codes with one E4M3 scale per 16 channels and no second-level scale.
// The pages do not give the rule that picks a scale; this library takes, per group of 16
// channels,
//   scale  = E4M3(amax / 6)        amax = max |x_c|, 6 = the largest E2M1 magnitude
//   code_c = E2M1(x_c / scale)     nearest, ties to the even code, saturating at +-6, sign kept
// with both quotients rounded to binary32 (IEEE division) before the conversion, and all
// codes 0 when the scale byte is 0.  Codes are packed two per byte, channel 2i in the low
// nibble of byte i.
//
// How the kernel decides the codes without dividing:
//  * The E2M1 code of q = x / s is the number of decision points q passes: 0.25, 1.25, 2.5 and
//    5 strictly (their ties go down to the even code) and 0.75, 1.75 and 3.5 inclusively (their
//    ties go up).  Comparing |x| with the exact products t*s gives the same decisions as
//    comparing the binary32 quotient with t: x is bf16 (8 significant bits) and t*s has at most
//    7, so when |x| != t*s they differ by at least ~2^-9 relative, far more than the quotient's
//    rounding.
//  * Every E4M3 scale (subnormal ones included) is s = (1 + m/8) * 2^E with m in 0..7.  The
//    decisions depend on |x| / s only, so in bf16 bit patterns they depend on m and on
//    i = bits(|x|) - bits(s/4) alone: one table per m (768 entries, built in LDS by each
//    workgroup) maps i to the code; i <= 0 is |x| <= s/4 (code 0) and the last entry lies far
//    above 5s (code 7).
//
// A thread converts whole 16-channel groups (32 bytes of bf16 in, 8 code bytes and one scale
// byte out); consecutive threads take consecutive groups, so a wave reads two whole rows with
// contiguous 16-byte loads.  The grid is capped and strides over the groups.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kLutN = 768;

// Code magnitude of the bf16 magnitude pattern `bits` for the scale 1 + m/8 (exponent 0), from
// the decision points (exact products).
__device__ __forceinline__ uint32_t e2m1_code_at(uint32_t bits, int m) {
  return e2m1_mag_code(bf16_bits_to_f32(bits), 1.0f + 0.125f * (float)m);
}

constexpr int kQuantThreads = 256;
constexpr int kQuantGroupsPerIter = 1;   // groups a thread loads before converting them

__global__ __launch_bounds__(kQuantThreads) void k_quantize_kv(const uint16_t* __restrict__ x, int64_t rows,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  __shared__ uint8_t lut[8 * kLutN];
  for (int e = threadIdx.x; e < 8 * kLutN; e += kQuantThreads) {
    const int m = e / kLutN, i = e - m * kLutN;
    lut[e] = (uint8_t)e2m1_code_at(0x3f80u + ((uint32_t)m << 4) - 256u + (uint32_t)i, m);
  }
  __syncthreads();
  const int64_t groups = rows * 32;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  const u16x2 top2 = {(unsigned short)(kLutN - 1), (unsigned short)(kLutN - 1)};
  for (int64_t g0 = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; g0 < groups;
       g0 += stride * kQuantGroupsPerIter) {
    u32x4 ld[kQuantGroupsPerIter][2];
#pragma unroll
    for (int u = 0; u < kQuantGroupsPerIter; ++u) {
      const int64_t g = g0 + u * stride;
      const uint16_t* src = x + (g < groups ? g : g0) * 16;   // group g: row g/32, channels 16*(g%32)
      ld[u][0] = *(const u32x4*)src;
      ld[u][1] = *(const u32x4*)(src + 8);
    }
#pragma unroll
    for (int u = 0; u < kQuantGroupsPerIter; ++u) {
      const int64_t g = g0 + u * stride;
      if (g >= groups) break;
      const uint32_t w[8] = {ld[u][0].x, ld[u][0].y, ld[u][0].z, ld[u][0].w,
                             ld[u][1].x, ld[u][1].y, ld[u][1].z, ld[u][1].w};
      // amax on bit patterns (they order like the magnitudes)
      u16x2 m2 = __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu);
#pragma unroll
      for (int i = 1; i < 8; ++i) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
      const float amax = bf16_bits_to_f32(m2.x > m2.y ? m2.x : m2.y);
      const uint32_t sb = f32_to_e4m3(amax / 6.0f);
      const float s = e4m3_to_f32(sb);
      const uint32_t sbits = __float_as_uint(s) >> 16;           // bf16 pattern of s (exact)
      const unsigned short base = (unsigned short)(sbits - 256u); // pattern of s/4
      const uint8_t* tab = lut + ((sbits >> 4) & 7u) * kLutN;
      const u16x2 base2 = {base, base};
      uint32_t pk[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u16x2 a = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
        const u16x2 d = __builtin_elementwise_min(__builtin_elementwise_max(a, base2) - base2, top2);
        const uint32_t c = (uint32_t)tab[d.x] | ((uint32_t)tab[d.y] << 4) | ((w[i] >> 12) & 0x8u) |
                           ((w[i] >> 24) & 0x80u);
        pk[i >> 2] |= c << (8 * (i & 3));
      }
      if (!(s > 0.f)) pk[0] = pk[1] = 0u;        // a zero scale stores code 0 throughout
      *(u32x2*)(codes + g * 8) = u32x2{pk[0], pk[1]};
      scales[g] = (uint8_t)sb;
    }
  }
}

hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t groups = rows * 32;
  int64_t blocks = (groups + kQuantThreads * 16 - 1) / (kQuantThreads * 16);   // >= 16 groups a thread
  // short appends (a few hundred rows) are latency-bound: spread them to one group per thread
  // over up to 256 workgroups instead of looping in a few
  const int64_t spread = std::min<int64_t>(256, (groups + kQuantThreads - 1) / kQuantThreads);
  if (blocks < spread) blocks = spread;
  if (blocks > 1024) blocks = 1024;         // 4 per CU: measured best between 256 and 8192
  hipLaunchKernelGGL(k_quantize_kv, dim3((unsigned)blocks), dim3(kQuantThreads), 0, s, x, rows, codes, scales);
  return hipGetLastError();
}

}  // namespace csa2
