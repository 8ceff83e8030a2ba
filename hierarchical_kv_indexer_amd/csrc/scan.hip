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

// The 32x128 query of one indexer head set, rounded to E4M3 and held as bf16 in LDS.
__device__ __forceinline__ void stage_query(const uint16_t* __restrict__ q, uint16_t* qlds) {
  for (int i = threadIdx.x; i < kIdxHeads * kIdxDim; i += blockDim.x) {
    float v = e4m3_to_f32(f32_to_e4m3(bf16_bits_to_f32(q[i])));
    qlds[i] = (uint16_t)(__float_as_uint(v) >> 16);
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

// Score of this lane's row (column j of the tile); every lane of a column gets the same value.
__device__ __forceinline__ float tile_score(const TileCtx& cx, u32x4 lo, u32x4 hi) {
  u32x4 b[4];
  b[0] = e4m3x8_to_bf16x8(lo.x, lo.y);
  b[1] = e4m3x8_to_bf16x8(lo.z, lo.w);
  b[2] = e4m3x8_to_bf16x8(hi.x, hi.y);
  b[3] = e4m3x8_to_bf16x8(hi.z, hi.w);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a0 = mfma16x16x32(cx.qa[0][c], b[c], a0);
    a1 = mfma16x16x32(cx.qa[1][c], b[c], a1);
  }
  float p = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[v], fmaxf(a0[v], 0.f), p);
#pragma unroll
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[4 + v], fmaxf(a1[v], 0.f), p);
  p += __shfl_xor(p, 16);
  p += __shfl_xor(p, 32);
  return p;
}

__device__ __forceinline__ void load_row(const uint8_t* __restrict__ row, int g, u32x4& lo, u32x4& hi) {
  lo = *(const u32x4*)(row + 16 * g);
  hi = *(const u32x4*)(row + 64 + 16 * g);
}

// ---------------------------------------------------------------------------- Full scan

constexpr int kScanU = 4;   // tiles in flight per wave

// grid (n_wg, Q).  WG x covers positions [x*chunk, (x+1)*chunk) of query q = b*T + t.
// Writes scores[q][p] for p < n_visible, the order key of each block's max score, and the
// min / max block key of the WG (0xffffffff / 0 when it has no block); blkkey and wg_minmax
// may be null (scores only).
__global__ __launch_bounds__(kScanThreads) void k_idx_scan(
    const uint8_t* __restrict__ idx_k, int64_t k_rows, const uint16_t* __restrict__ idx_q,
    const float* __restrict__ head_w, const int32_t* __restrict__ n_visible, int T, int n_max,
    int chunk, float* __restrict__ scores, uint32_t* __restrict__ blkkey, int nb_max,
    uint32_t* __restrict__ wg_minmax) {
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kIdxHeads * kIdxDim];
  __shared__ uint32_t red[2][kScanThreads / 64];
  const int q = blockIdx.y, b = q / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int p_begin = blockIdx.x * chunk;
  const int p_end = min(p_begin + chunk, nv);
  const int ntiles = p_end > p_begin ? (p_end - p_begin + 15) >> 4 : 0;

  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (ntiles > 0) {
    stage_query(idx_q + (size_t)q * kIdxHeads * kIdxDim, qlds);
    __syncthreads();
    TileCtx cx;
    load_ctx(cx, qlds, head_w + (size_t)q * kIdxHeads);
    const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * kIdxDim;
    float* srow = scores + (size_t)q * n_max;
    uint32_t* brow = blkkey ? blkkey + (size_t)q * nb_max : nullptr;
    for (int t0 = wave * kScanU; t0 < ntiles; t0 += (kScanThreads / 64) * kScanU) {
      u32x4 lo[kScanU], hi[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        if (t0 + u < ntiles) {
          int p = p_begin + 16 * (t0 + u) + j;
          p = p < nv ? p : nv - 1;
          load_row(kseq + (size_t)p * kIdxDim, g, lo[u], hi[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        if (t0 + u < ntiles) {
          const float s = tile_score(cx, lo[u], hi[u]);
          const int p = p_begin + 16 * (t0 + u) + j;
          const bool valid = p < p_end;
          if (g == 0 && valid) srow[p] = s;
          uint32_t key = valid ? score_key(s) : 0u;
          key = max(key, (uint32_t)__shfl_xor((int)key, 1));
          key = max(key, (uint32_t)__shfl_xor((int)key, 2));
          key = max(key, (uint32_t)__shfl_xor((int)key, 4));
          if (g == 0 && (j & 7) == 0 && valid) {
            if (brow) brow[p >> 3] = key;
            kmin = min(kmin, key);
            kmax = max(kmax, key);
          }
        }
      }
    }
  }
  // WG min / max of the block keys
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) { red[0][wave] = kmin; red[1][wave] = kmax; }
  __syncthreads();
  if (threadIdx.x == 0 && wg_minmax) {
    for (int w = 1; w < kScanThreads / 64; ++w) { kmin = min(kmin, red[0][w]); kmax = max(kmax, red[1][w]); }
    wg_minmax[((size_t)q * gridDim.x + blockIdx.x) * 2 + 0] = kmin;
    wg_minmax[((size_t)q * gridDim.x + blockIdx.x) * 2 + 1] = kmax;
  }
}

int scan_chunk_positions(int n_max, int queries) {
  // aim for >= ~1024 workgroups in total, chunks of 256 .. 4096 positions (multiples of 256)
  long long total = (long long)n_max * (queries > 0 ? queries : 1);
  long long c = total / 1024;
  c = (c + 255) / 256 * 256;
  if (c < 256) c = 256;
  if (c > 4096) c = 4096;
  return (int)c;
}

hipError_t launch_idx_scan(const uint8_t* idx_k, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* n_visible, int Q, int T, int n_max,
                           float* scores, uint32_t* blkkey, int nb_max, uint32_t* wg_minmax,
                           int chunk, int n_wg, hipStream_t s) {
  hipLaunchKernelGGL(k_idx_scan, dim3(n_wg, Q), dim3(kScanThreads), 0, s, idx_k, k_rows, idx_q,
                     head_w, n_visible, T, n_max, chunk, scores, blkkey, nb_max, wg_minmax);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- Reindex scoring

// grid (n_chunks, L*Q).  Item it = l*Q + q scores pool slots [x*chunk, (x+1)*chunk) of query
// q with layer l's query and weights.  Slots beyond pool_len or holding positions outside
// [0, k_rows) are not written.
__global__ __launch_bounds__(kScanThreads) void k_ri_score(
    const uint8_t* __restrict__ idx_k, int64_t k_rows, const uint16_t* __restrict__ idx_q,
    const float* __restrict__ head_w, const int32_t* __restrict__ pool_pos,
    const int32_t* __restrict__ pool_len, int cap, int Q, int T, int chunk,
    float* __restrict__ ri_scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kIdxHeads * kIdxDim];
  const int it = blockIdx.y, q = it % Q, b = q / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  int len = pool_len[q];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int s_begin = blockIdx.x * chunk;
  const int s_end = min(s_begin + chunk, len);
  const int ntiles = s_end > s_begin ? (s_end - s_begin + 15) >> 4 : 0;
  if (ntiles == 0) return;
  stage_query(idx_q + (size_t)it * kIdxHeads * kIdxDim, qlds);
  __syncthreads();
  TileCtx cx;
  load_ctx(cx, qlds, head_w + (size_t)it * kIdxHeads);
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * kIdxDim;
  const int32_t* pp = pool_pos + (size_t)q * cap;
  float* out = ri_scores + (size_t)it * cap;
  for (int t0 = wave * kScanU; t0 < ntiles; t0 += (kScanThreads / 64) * kScanU) {
    u32x4 lo[kScanU], hi[kScanU];
    bool ok[kScanU];
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      ok[u] = false;
      if (t0 + u < ntiles) {
        const int slot = s_begin + 16 * (t0 + u) + j;
        int pos = slot < s_end ? pp[slot] : -1;
        ok[u] = pos >= 0 && (int64_t)pos < k_rows;
        load_row(kseq + (size_t)(ok[u] ? pos : 0) * kIdxDim, g, lo[u], hi[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      if (t0 + u < ntiles) {
        const float s = tile_score(cx, lo[u], hi[u]);
        const int slot = s_begin + 16 * (t0 + u) + j;
        if (g == 0 && ok[u]) out[slot] = s;
      }
    }
  }
}

int ri_chunk_slots(int pool_cap, int items) {
  long long total = (long long)pool_cap * (items > 0 ? items : 1);
  long long c = total / 1024;
  c = (c + 255) / 256 * 256;
  if (c < 256) c = 256;
  if (c > 4096) c = 4096;
  return (int)c;
}

hipError_t launch_ri_score(const uint8_t* idx_k, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* pool_pos, const int32_t* pool_len,
                           int pool_cap, int L, int Q, int T, float* ri_scores, int chunk,
                           hipStream_t s) {
  const int n_chunks = (pool_cap + chunk - 1) / chunk;
  hipLaunchKernelGGL(k_ri_score, dim3(n_chunks, L * Q), dim3(kScanThreads), 0, s, idx_k, k_rows,
                     idx_q, head_w, pool_pos, pool_len, pool_cap, Q, T, chunk, ri_scores);
  return hipGetLastError();
}

}  // namespace csa2
