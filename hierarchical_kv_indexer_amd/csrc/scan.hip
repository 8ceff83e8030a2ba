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
// 256 threads, 16 consecutive values each: two 16-byte loads issued together.
__device__ __forceinline__ void stage_query(const uint16_t* __restrict__ q, uint16_t* qlds) {
  static_assert(kIdxHeads * kIdxDim == kScanThreads * 16, "query staging assumes 256 threads");
  const int base = threadIdx.x * 16;
  const u32x4 a = *(const u32x4*)(q + base);
  const u32x4 b = *(const u32x4*)(q + base + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float lo = e4m3_to_f32(f32_to_e4m3(bf16_bits_to_f32(w[i] & 0xffffu)));
    const float hi = e4m3_to_f32(f32_to_e4m3(bf16_bits_to_f32(w[i] >> 16)));
    o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  *(u32x4*)(qlds + base) = u32x4{o[0], o[1], o[2], o[3]};
  *(u32x4*)(qlds + base + 8) = u32x4{o[4], o[5], o[6], o[7]};
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

// Score of this lane's row (column j of the tile); every lane of a column gets the same value.
// The 8 heads of a lane are summed in a fixed order, then the four k-groups are combined as
// (g0 + g1) + (g2 + g3), identically on every lane.
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
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[v], relu_bits(a0[v]), p);
#pragma unroll
  for (int v = 0; v < 4; ++v) p = fmaf(cx.w[4 + v], relu_bits(a1[v]), p);
  return sum_xor32(sum_xor16(p));
}

__device__ __forceinline__ void load_row(const uint8_t* __restrict__ row, int g, u32x4& lo, u32x4& hi) {
  lo = *(const u32x4*)(row + 16 * g);
  hi = *(const u32x4*)(row + 64 + 16 * g);
}

// ---------------------------------------------------------------------------- Full scan

constexpr int kScanU = 3;                       // tiles per pipeline stage of a wave
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kMaxBlocksPerWave = 256;          // chunk <= 8192 positions per WG

size_t scan_lds_bytes(int chunk) {
  const int tpw = chunk >> 6;
  return (size_t)kIdxHeads * kIdxDim * 2 + (size_t)kScanWaves * tpw * 16 * 4 + (size_t)kScanWaves * 2 * tpw * 4;
}

// Best ranking key (score key, block) of a wave's blocks, removed from the set.  Entries are
// (key, block) with key 0 / block 0xffffffff meaning "none"; returns rank_key or 0.
template <int E>
__device__ __forceinline__ uint64_t wave_pop_best(uint32_t (&key)[E], uint32_t (&blk)[E]) {
  uint32_t bk = 0u, bj = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] > bk || (key[e] == bk && blk[e] < bj)) { bk = key[e]; bj = blk[e]; }
  const uint32_t m = wave_max_u32(bk);
  const uint32_t jm = wave_min_u32(bk == m ? bj : 0xffffffffu);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] == m && blk[e] == jm) { key[e] = 0u; blk[e] = 0xffffffffu; }
  return (m == 0u && jm == 0xffffffffu) ? 0ull : rank_key(m, jm);
}

// grid (n_wg, Q).  WG x covers positions [x*chunk, (x+1)*chunk) of query q = b*T + t; wave v
// covers the contiguous tiles [v*tpw, (v+1)*tpw) of that range (a "unit").  Loads run one
// pipeline stage (kScanU tiles) ahead of the MFMA work; the loop issues no global stores, so
// its loads stay in flight: scores and block keys are staged in LDS and stored afterwards.
//
// Writes scores[q][p] for p < n_visible and, when `blkkey` is non-null, the order key of
// each block's max score.  When `lists` is non-null, each unit also writes its five best
// blocks as ranking keys (score key << 32 | ~block): lists[q][unit][0..3] = the four best
// (0 = none) and cuts[q][unit] = the fifth best (0 = none), so every block of the unit that
// is not listed ranks at or below cuts[q][unit].
__global__ __launch_bounds__(kScanThreads, 4) void k_idx_scan(
    const uint8_t* __restrict__ idx_k, int64_t k_rows, const uint16_t* __restrict__ idx_q,
    const float* __restrict__ head_w, const int32_t* __restrict__ n_visible, int T, int n_max,
    int chunk, float* __restrict__ scores, uint32_t* __restrict__ blkkey, int nb_max,
    uint64_t* __restrict__ lists, uint64_t* __restrict__ cuts) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tpw = chunk >> 6;                     // tiles per wave (chunk is a multiple of 256)
  uint16_t* qlds = (uint16_t*)lds;
  const int q = blockIdx.y, b = q / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  float* sbuf = (float*)(lds + kIdxHeads * kIdxDim * 2) + wave * tpw * 16;
  uint32_t* wkeys = (uint32_t*)(lds + kIdxHeads * kIdxDim * 2 + kScanWaves * tpw * 16 * 4) + wave * 2 * tpw;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int p_begin = blockIdx.x * chunk;
  const int p_end = min(p_begin + chunk, nv);
  const int ntiles = p_end > p_begin ? (p_end - p_begin + 15) >> 4 : 0;
  const int tb = wave * tpw;
  const int nt = max(0, min(tpw, ntiles - tb));   // tiles of this wave
  const int pw = p_begin + 16 * tb;               // first position of this wave
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * kIdxDim;

  // Rows past this wave's range are clamped to its last row, so every stage loads and computes
  // unconditionally (no branch around a load keeps the compiler's wait counts exact and the
  // next stage's loads in flight); results of such padding tiles are never stored.
  const int plast = min(p_end, pw + 16 * nt) - 1;
  u32x4 lo0[kScanU], hi0[kScanU], lo1[kScanU], hi1[kScanU];
  auto load_stage = [&](u32x4(&lo)[kScanU], u32x4(&hi)[kScanU], int st) {
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
      const int p = min(pw + 16 * (st * kScanU + u) + j, plast);
      load_row(kseq + (size_t)p * kIdxDim, g, lo[u], hi[u]);
    }
  };
  const int ns = (nt + kScanU - 1) / kScanU;
  if (nt > 0) load_stage(lo0, hi0, 0);            // first rows in flight before the query prep

  if (ntiles > 0) {
    stage_query(idx_q + (size_t)q * kIdxHeads * kIdxDim, qlds);
    __syncthreads();
    TileCtx cx;
    load_ctx(cx, qlds, head_w + (size_t)q * kIdxHeads);
    auto compute_stage = [&](const u32x4(&lo)[kScanU], const u32x4(&hi)[kScanU], int st) {
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        const int t = st * kScanU + u;
        const float sc = tile_score(cx, lo[u], hi[u]);
        const bool valid = pw + 16 * t + j < p_end;
        const uint32_t key = max8_u32(valid ? score_key(sc) : 0u);
        if (t < nt) {
          if (g == 0) sbuf[16 * t + j] = sc;
          if ((lane & 0x37) == 0) wkeys[2 * t + (lane >> 3)] = key;   // lanes 0, 8
        }
      }
    };
    for (int st = 0; st < ns; st += 2) {
      load_stage(lo1, hi1, st + 1);
      compute_stage(lo0, hi0, st);
      load_stage(lo0, hi0, st + 2);
      compute_stage(lo1, hi1, st + 1);
    }
    // coalesced stores of this wave's scores and block keys
    const int nsw = p_end > pw ? min(16 * tpw, p_end - pw) : 0;
    float* srow = scores + (size_t)q * n_max + pw;
    for (int i = lane; i < nsw; i += 64) srow[i] = sbuf[i];
    if (blkkey) {
      const int nbw = (nsw + 7) >> 3;
      uint32_t* brow = blkkey + (size_t)q * nb_max + (pw >> 3);
      for (int i = lane; i < nbw; i += 64) brow[i] = wkeys[i];
    }
  }
  if (!lists) return;
  // five best blocks of this wave's unit
  const int nblk = p_end > pw ? min(2 * tpw, (p_end - pw + 7) >> 3) : 0;
  const uint32_t jb0 = (uint32_t)(pw >> 3);
  constexpr int E = kMaxBlocksPerWave / 64;
  uint32_t key[E], blk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;
    const bool ok = i < nblk;
    key[e] = ok ? wkeys[i] : 0u;
    blk[e] = ok ? jb0 + (uint32_t)i : 0xffffffffu;
  }
  const size_t unit = ((size_t)q * gridDim.x + blockIdx.x) * kScanWaves + wave;
  uint64_t best[5];
#pragma unroll
  for (int r = 0; r < 5; ++r) best[r] = wave_pop_best(key, blk);
  if (lane == 0) {
    u32x4* lp = (u32x4*)(lists + unit * 4);
    lp[0] = u32x4{(uint32_t)best[0], (uint32_t)(best[0] >> 32), (uint32_t)best[1], (uint32_t)(best[1] >> 32)};
    lp[1] = u32x4{(uint32_t)best[2], (uint32_t)(best[2] >> 32), (uint32_t)best[3], (uint32_t)(best[3] >> 32)};
    cuts[unit] = best[4];
  }
}

int scan_chunk_positions(int n_max, int queries) {
  // >= ~1024 workgroups in total and at most 1024 per query; chunks are multiples of 256
  // positions and at most 8192 (the per-wave block list holds 256 blocks)
  long long total = (long long)n_max * (queries > 0 ? queries : 1);
  long long c = total / 1024;
  long long per_query = ((long long)n_max + 1023) / 1024;
  if (c < per_query) c = per_query;
  c = (c + 255) / 256 * 256;
  if (c < 256) c = 256;
  if (c > 8192) c = 8192;
  return (int)c;
}

hipError_t launch_idx_scan(const uint8_t* idx_k, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* n_visible, int Q, int T, int n_max,
                           float* scores, uint32_t* blkkey, int nb_max, uint64_t* lists,
                           uint64_t* cuts, int chunk, int n_wg, hipStream_t s) {
  hipLaunchKernelGGL(k_idx_scan, dim3(n_wg, Q), dim3(kScanThreads), scan_lds_bytes(chunk), s, idx_k, k_rows,
                     idx_q, head_w, n_visible, T, n_max, chunk, scores, blkkey, nb_max, lists, cuts);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- Reindex scoring

constexpr int kRiTilesPerWave = 2;

// grid (n_chunks, L*Q).  Item it = l*Q + q scores pool slots [x*chunk, (x+1)*chunk) of query
// q (chunk = 64 * kRiTilesPerWave) with layer l's query and weights.  Slots beyond pool_len or
// holding positions outside [0, k_rows) are not written.
__global__ __launch_bounds__(kScanThreads) void k_ri_score(
    const uint8_t* __restrict__ idx_k, int64_t k_rows, const uint16_t* __restrict__ idx_q,
    const float* __restrict__ head_w, const int32_t* __restrict__ pool_pos,
    const int32_t* __restrict__ pool_len, int cap, int Q, int T, float* __restrict__ ri_scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kIdxHeads * kIdxDim];
  __shared__ float sbuf[kScanThreads / 64][kRiTilesPerWave * 16];
  const int it = blockIdx.y, q = it % Q, b = q / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  int len = pool_len[q];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int chunk = 64 * kRiTilesPerWave;
  const int s_begin = blockIdx.x * chunk;
  const int s_end = min(s_begin + chunk, len);
  if (s_end <= s_begin) return;
  const int sw = s_begin + 16 * kRiTilesPerWave * wave;          // first slot of this wave
  const int32_t* pp = pool_pos + (size_t)q * cap;
  int pos[kRiTilesPerWave];
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) {
    const int slot = sw + 16 * u + j;
    pos[u] = slot < s_end ? pp[slot] : -1;
  }
  stage_query(idx_q + (size_t)it * kIdxHeads * kIdxDim, qlds);
  const uint8_t* kseq = idx_k + (size_t)b * (size_t)k_rows * kIdxDim;
  u32x4 lo[kRiTilesPerWave], hi[kRiTilesPerWave];
  bool ok[kRiTilesPerWave];
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) {
    ok[u] = pos[u] >= 0 && (int64_t)pos[u] < k_rows;
    load_row(kseq + (size_t)(ok[u] ? pos[u] : 0) * kIdxDim, g, lo[u], hi[u]);
  }
  __syncthreads();
  TileCtx cx;
  load_ctx(cx, qlds, head_w + (size_t)it * kIdxHeads);
#pragma unroll
  for (int u = 0; u < kRiTilesPerWave; ++u) {
    const float sc = tile_score(cx, lo[u], hi[u]);
    if (g == 0) sbuf[wave][16 * u + j] = sc;
  }
  float* out = ri_scores + (size_t)it * cap;
  if (g == 0) {
#pragma unroll
    for (int u = 0; u < kRiTilesPerWave; ++u)
      if (ok[u]) out[sw + 16 * u + j] = sbuf[wave][16 * u + j];
  }
}

hipError_t launch_ri_score(const uint8_t* idx_k, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* pool_pos, const int32_t* pool_len,
                           int pool_cap, int L, int Q, int T, float* ri_scores, hipStream_t s) {
  const int chunk = 64 * kRiTilesPerWave;
  const int n_chunks = (pool_cap + chunk - 1) / chunk;
  hipLaunchKernelGGL(k_ri_score, dim3(n_chunks, L * Q), dim3(kScanThreads), 0, s, idx_k, k_rows,
                     idx_q, head_w, pool_pos, pool_len, pool_cap, Q, T, ri_scores);
  return hipGetLastError();
}

}  // namespace csa2
