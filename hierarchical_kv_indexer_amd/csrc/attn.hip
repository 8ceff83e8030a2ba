// Sparse attention over gathered FP4 main-KV rows merged with the FP8 sliding window (gfx950).
//
// For layer l, query q and head h (blog.4sapi.com sec.2 and sec.5; alphalab.site sec."3. FP4"):
//   rows  = { dequant(main KV row p) : p in idx_sets[layer_set[l]][q] } followed by
//           { SWA row r of layer l : r in [max(0, swa_end - window), swa_end) }
//   o_h   = sum_r softmax_r(scale * q_h . x_r) x_r      (keys = values: one shared latent)
// A main row is 256 bytes of E2M1 codes plus 32 E4M3 scales (one per 16 channels); the
// dequantised value code * scale is exact in bf16, and so is an E4M3 SWA value.
//
// One workgroup (4 waves) handles 16 heads of one (layer, query) and streams the rows in
// chunks of 64: rows are gathered and dequantised into LDS as bf16, S = Q X^T and O += P X run
// on bf16 MFMA (16x16x32) with an online softmax in fp32; the next chunk's raw bytes are
// loaded into registers while the current chunk is computed.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

constexpr int kRows = 64;                    // rows per chunk
constexpr int kXStride = kKvDim + 8;         // bf16 elements per LDS row (pad: 16 bytes)
constexpr int kPStride = kRows + 8;          // bf16 elements per P row

struct RawRow {          // this thread's quarter (128 channels) of one chunk row
  u32x4 d[8];            // main: d[0..3] = 64 code bytes; SWA: d[0..7] = 128 E4M3 bytes
  u32x2 sc;              // main: 8 scale bytes
  int kind;              // 0 empty, 1 main, 2 SWA
};

__device__ __forceinline__ void load_raw(RawRow& r, int slot, int k, const int32_t* __restrict__ idx,
                                         int64_t kv_rows, const uint8_t* __restrict__ codes_seq,
                                         const uint8_t* __restrict__ scales_seq,
                                         const uint8_t* __restrict__ swa_seq, int ws, int we,
                                         int quarter) {
  r.kind = 0;
  if (slot < k) {
    const int pos = idx[slot];
    if (pos >= 0 && (int64_t)pos < kv_rows) {
      const u32x4* c = (const u32x4*)(codes_seq + (size_t)pos * kKvCodeBytes + 64 * quarter);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.d[i] = c[i];
      r.sc = *(const u32x2*)(scales_seq + (size_t)pos * kKvScaleBytes + 8 * quarter);
      r.kind = 1;
    }
  } else {
    const int row = ws + (slot - k);
    if (row < we) {
      const u32x4* c = (const u32x4*)(swa_seq + (size_t)row * kKvDim + 128 * quarter);
#pragma unroll
      for (int i = 0; i < 8; ++i) r.d[i] = c[i];
      r.kind = 2;
    }
  }
}

// Dequantise this thread's quarter row into LDS (128 bf16 = 16 x 16 bytes).
__device__ __forceinline__ void store_row(const RawRow& r, uint16_t* xrow, int quarter) {
  u32x4* dst = (u32x4*)(xrow + 128 * quarter);
  if (r.kind == 1) {
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[2 * i] = e4m3_to_f32((r.sc[i >> 1] >> (16 * (i & 1))) & 0xffu);
      s[2 * i + 1] = e4m3_to_f32((r.sc[i >> 1] >> (16 * (i & 1) + 8)) & 0xffu);
    }
    // 64 code bytes: bytes 8i .. 8i+7 hold channels 16i .. 16i+15 (scale s[i])
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = r.d[i >> 1][(i & 1) * 2], w1 = r.d[i >> 1][(i & 1) * 2 + 1];
      u32x4 o0, o1;
      o0.x = e2m1x2_scaled_to_bf16x2<0>(w0, s[i]);
      o0.y = e2m1x2_scaled_to_bf16x2<1>(w0, s[i]);
      o0.z = e2m1x2_scaled_to_bf16x2<2>(w0, s[i]);
      o0.w = e2m1x2_scaled_to_bf16x2<3>(w0, s[i]);
      o1.x = e2m1x2_scaled_to_bf16x2<0>(w1, s[i]);
      o1.y = e2m1x2_scaled_to_bf16x2<1>(w1, s[i]);
      o1.z = e2m1x2_scaled_to_bf16x2<2>(w1, s[i]);
      o1.w = e2m1x2_scaled_to_bf16x2<3>(w1, s[i]);
      dst[2 * i] = o0;
      dst[2 * i + 1] = o1;
    }
  } else if (r.kind == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dst[2 * i] = e4m3x8_to_bf16x8(r.d[i].x, r.d[i].y);
      dst[2 * i + 1] = e4m3x8_to_bf16x8(r.d[i].z, r.d[i].w);
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = z;
  }
}

// grid (H/16, L*Q), 256 threads.
__global__ __launch_bounds__(kAttnThreads) void k_sparse_attn(
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t kv_rows,
    const uint16_t* __restrict__ qg, const int32_t* __restrict__ idx_sets, LayerSets sets,
    const uint8_t* __restrict__ swa, int swa_rows, const int32_t* __restrict__ swa_end, int window,
    int Q, int B, int T, int H, int k, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t X[kRows * kXStride];
  __shared__ __attribute__((aligned(16))) uint16_t P[16 * kPStride];
  __shared__ float red[4][16];

  const int hg = blockIdx.x, lq = blockIdx.y;
  const int l = lq / Q, q = lq % Q, b = q / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int32_t* idx = idx_sets + ((size_t)sets.set[l] * Q + q) * k;
  int we = swa_end[q];
  we = we < 0 ? 0 : (we > swa_rows ? swa_rows : we);
  const int ws = max(0, we - window);
  const int nslots = k + (we - ws);
  const int nchunks = (nslots + kRows - 1) / kRows;
  const uint8_t* codes_seq = kv_codes + (size_t)b * kv_rows * kKvCodeBytes;
  const uint8_t* scales_seq = kv_scales + (size_t)b * kv_rows * kKvScaleBytes;
  const uint8_t* swa_seq = swa + ((size_t)l * B + b) * (size_t)swa_rows * kKvDim;

  // query of 16 heads as MFMA A operands: head j, channels 32c + 8g .. +7
  const uint16_t* qh = qg + (((size_t)l * Q + q) * H + 16 * hg) * kKvDim;
  u32x4 qa[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qa[c] = *(const u32x4*)(qh + (size_t)j * kKvDim + 32 * c + 8 * g);

  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_run[v] = -INFINITY; l_run[v] = 0.f; }

  const int my_row = tid >> 2, quarter = tid & 3;
  RawRow raw;
  load_raw(raw, my_row, k, idx, kv_rows, codes_seq, scales_seq, swa_seq, ws, we, quarter);

  for (int c = 0; c < nchunks; ++c) {
    store_row(raw, X + my_row * kXStride, quarter);
    __syncthreads();
    if (c + 1 < nchunks)
      load_raw(raw, (c + 1) * kRows + my_row, k, idx, kv_rows, codes_seq, scales_seq, swa_seq, ws,
               we, quarter);

    // S[head 4g+v][row 16*wave + j]
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xr = X + (16 * wave + j) * kXStride + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) s = mfma16x16x32(qa[cc], *(const u32x4*)(xr + 32 * cc), s);
    const int slot = c * kRows + 16 * wave + j;
    bool row_ok;
    if (slot < k) {
      const int pos = idx[slot];
      row_ok = pos >= 0 && (int64_t)pos < kv_rows;
    } else {
      row_ok = slot < nslots;
    }
    float sv[4], mx[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = row_ok ? s[v] * scale_log2 : -INFINITY;
      mx[v] = sv[v];
    }
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], o2));
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][4 * g + v] = mx[v];
    }
    __syncthreads();
    float alpha[4], mnew[4], psum[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      float mc = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
      mnew[v] = fmaxf(m_run[v], mc);
      alpha[v] = mnew[v] == -INFINITY ? 1.f : exp2f(m_run[v] - mnew[v]);
      const float p = mnew[v] == -INFINITY ? 0.f : exp2f(sv[v] - mnew[v]);
      const uint32_t pb = f32_to_bf16_rne(p);
      P[h * kPStride + 16 * wave + j] = (uint16_t)pb;
      psum[v] = bf16_bits_to_f32(pb);
    }
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1)
#pragma unroll
      for (int v = 0; v < 4; ++v) psum[v] += __shfl_xor(psum[v], o2);
    __syncthreads();   // red[] reads done, P written
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][4 * g + v] = psum[v];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const float ps = (red[0][h] + red[1][h]) + (red[2][h] + red[3][h]);
      l_run[v] = l_run[v] * alpha[v] + ps;
      m_run[v] = mnew[v];
    }
    // O[head 4g+v][dim 128*wave + 16t + j] = alpha * O + sum_r P[head][r] X[r][dim]
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[t][v] *= alpha[v];
#pragma unroll
    for (int kk = 0; kk < kRows / 32; ++kk) {
      const u32x4 pa = *(const u32x4*)(P + j * kPStride + 32 * kk + 8 * g);
      const uint16_t* xc = X + (32 * kk + 8 * g) * kXStride + 128 * wave + j;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x4 xb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = xc[(2 * e) * kXStride + 16 * t];
          const uint32_t hi = xc[(2 * e + 1) * kXStride + 16 * t];
          xb[e] = lo | (hi << 16);
        }
        o[t] = mfma16x16x32(pa, xb, o[t]);
      }
    }
    __syncthreads();   // X, P and red[] are rewritten by the next chunk
  }

  // out[l][q][16*hg + 4g+v][dim], lse
  uint16_t* oh = out + (((size_t)l * Q + q) * H + 16 * hg) * kKvDim;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * g + v;
    const float inv = l_run[v] > 0.f ? 1.f / l_run[v] : 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) oh[(size_t)h * kKvDim + 128 * wave + 16 * t + j] = (uint16_t)f32_to_bf16_rne(o[t][v] * inv);
    if (lse && wave == 0 && j == 0) {
      lse[((size_t)l * Q + q) * H + 16 * hg + h] =
          l_run[v] > 0.f ? (m_run[v] + log2f(l_run[v])) * 0.69314718055994531f : -INFINITY;
    }
  }
}

hipError_t launch_sparse_attn(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t kv_rows,
                              const uint16_t* q, const int32_t* idx_sets, const LayerSets& sets,
                              const uint8_t* swa, int swa_rows, const int32_t* swa_end, int window,
                              int L, int B, int T, int H, int k, float scale, uint16_t* out,
                              float* lse, hipStream_t s) {
  const int Q = B * T;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(k_sparse_attn, dim3(H / 16, L * Q), dim3(kAttnThreads), 0, s, kv_codes,
                     kv_scales, kv_rows, q, idx_sets, sets, swa, swa_rows, swa_end, window, Q, B, T,
                     H, k, scale_log2, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
