// Sparse attention over gathered FP4 main-KV rows merged with the FP8 sliding window (gfx950).
//
// For layer l, query q and head h (blog.4sapi.com sec.2 and sec.5; alphalab.site sec."3. FP4"):
//   rows  = { dequant(main KV row p) : p in idx_sets[layer_set[l]][q] } followed by
//           { SWA row r of layer l : r in [max(0, swa_end - window), swa_end) }
//   o_h   = sum_r softmax_r(scale * q_h . x_r) x_r      (keys = values: one shared latent)
// A main row is 256 bytes of E2M1 codes plus 32 E4M3 scales (one per 16 channels); the
// dequantised value code * scale is exact in bf16, and so is an E4M3 SWA value.
//
// A workgroup (4 waves) handles 16 heads of one (layer, query) over one split of its rows and
// streams them in chunks of 64: rows are gathered and dequantised into LDS as bf16, S = Q X^T
// and O += P X run on bf16 MFMA (16x16x32) with an online softmax in fp32, and the next chunk's
// raw bytes are loaded into registers while the current chunk is computed.  When the (layer,
// query, head group) count alone cannot fill the GPU, the rows are split across workgroups and
// k_attn_combine merges the partial softmax states (max, sum, weighted rows).  With H a multiple
// of 64, k_sparse_attn_wide covers 64 heads of a (layer, query) per workgroup instead, so each
// gathered row is dequantised once for all of them.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

constexpr int kRows = 64;                    // rows per chunk
constexpr int kXStride = kKvDim + 16;        // bf16 elements per LDS row (pad: 32 bytes; measured
                                             // against 16: faster S = Q X^T reads, slower stores)
constexpr int kPStride = kRows + 8;          // bf16 elements per P row
constexpr int kMaxSplitRows = 4096 + kMaxTopK;   // a split never exceeds k + window rows
constexpr float kLazyLog2 = 8.f;             // slack of the softmax reference point (log2 units)

// Two floats -> fp16 pair (round to nearest even), low half first.  Partial rows are stored
// normalised by their own softmax sums, so they lie within the rows' range (|x| <= 2688).
__device__ __forceinline__ uint32_t f16x2_rne(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, h2{(_Float16)lo, (_Float16)hi});
}

// Max / sum over the 16 lanes of a DPP row; every lane of the row gets the same value (the
// pairwise steps are symmetric, so the sum is rounded identically in each lane).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __uint_as_float(dpp_mov<0xB1>(__float_as_uint(x))));    // quad_perm [1,0,3,2]
  x = fmaxf(x, __uint_as_float(dpp_mov<0x4E>(__float_as_uint(x))));    // quad_perm [2,3,0,1]
  x = fmaxf(x, __uint_as_float(dpp_mov<0x141>(__float_as_uint(x))));   // row_half_mirror
  x = fmaxf(x, __uint_as_float(dpp_mov<0x140>(__float_as_uint(x))));   // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __uint_as_float(dpp_mov<0xB1>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<0x4E>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<0x141>(__float_as_uint(x)));
  x += __uint_as_float(dpp_mov<0x140>(__float_as_uint(x)));
  return x;
}

// Two floats to bf16 with one round-to-nearest-even conversion (low half first).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// gfx950 LDS transpose read of 16-bit elements: within each 16-lane group, lane 4a+b receives
// element b of the 8 bytes addressed by lanes a, a+4, a+8 and a+12 (in that order).
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(u32x2, r);
}

struct RawRow {          // this thread's quarter (128 channels) of one chunk row
  u32x4 d[8];            // main: d[0..3] = 64 code bytes; SWA: d[0..7] = 128 E4M3 bytes
  u32x2 sc;              // main: 8 scale bytes
  int kind;              // 0 empty, 1 main, 2 SWA
};

// Dequantise this thread's quarter row into LDS (128 bf16 = 16 x 16 bytes).
__device__ __forceinline__ void store_row(const RawRow& r, uint16_t* xrow, int quarter) {
  u32x4* dst = (u32x4*)(xrow + 128 * quarter);
  if (r.kind == 1) {
    // the eight scale bytes through the hardware E4M3 conversion (exact), two per instruction
    float s[8];
    const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc[0], 1.0f, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc[0], 1.0f, true);
    const f32x2 s45 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc[1], 1.0f, false);
    const f32x2 s67 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc[1], 1.0f, true);
    s[0] = s01.x; s[1] = s01.y; s[2] = s23.x; s[3] = s23.y;
    s[4] = s45.x; s[5] = s45.y; s[6] = s67.x; s[7] = s67.y;
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

// Rows of a (layer, query) are numbered: main slots 0 .. k-1 (index set order), then the window's
// SWA rows.  grid (n_splits, H/16, L*Q): split s covers row slots [s*split_rows, (s+1)*split_rows)
// for 16 heads.  With one split the normalised bf16 output and lse are written directly;
// otherwise the split writes its partial state (running max m in log2 units and sum l in fp32,
// and its output row sum(p*x) / l in fp16) for k_attn_combine.
__global__ __launch_bounds__(kAttnThreads) void k_sparse_attn(
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t kv_rows,
    const uint16_t* __restrict__ qg, const int32_t* __restrict__ idx_sets, LayerSets sets,
    const uint8_t* __restrict__ swa, int swa_rows, const int32_t* __restrict__ swa_end, int window,
    int Q, int B, int T, int H, int k, float scale_log2, int split_rows, int n_splits,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t X[kRows * kXStride];
  __shared__ __attribute__((aligned(16))) uint16_t P[16 * kPStride];
  __shared__ float red_m[4][16], red_l[4][16];
  __shared__ int32_t rowok[kRows];

  const int split = blockIdx.x, hg = blockIdx.y, lq = blockIdx.z;
  const int l = lq / Q, q = lq % Q, b = q / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int32_t* idx = idx_sets + ((size_t)sets.set[l] * Q + q) * k;
  int we = swa_end[q];
  we = we < 0 ? 0 : (we > swa_rows ? swa_rows : we);
  const int ws = max(0, we - window);
  const int nslots = k + (we - ws);
  const int s0 = split * split_rows, s1 = min(nslots, s0 + split_rows);
  const int nchunks = s1 > s0 ? (s1 - s0 + kRows - 1) / kRows : 0;
  const uint8_t* codes_seq = kv_codes + (size_t)b * kv_rows * kKvCodeBytes;
  const uint8_t* scales_seq = kv_scales + (size_t)b * kv_rows * kKvScaleBytes;
  const uint8_t* swa_seq = swa + ((size_t)l * B + b) * (size_t)swa_rows * kKvDim;

  // lane l of wave w takes row 16w + l % 16, quarter l / 16: the 16 lanes of each LDS write pass
  // then hold 16 different rows (one 16-byte slot each), which keeps the dequantised stores free
  // of bank conflicts (with four quarters of one row per pass they conflict four ways)
  const int my_row = 16 * (tid >> 6) + (tid & 15), quarter = (tid >> 4) & 3;
  // index-set entry of this thread's row in chunk c (-1: none), prefetched one chunk ahead and
  // checked only where its row is loaded, so nothing waits for it in between
  auto row_index = [&](int c) {
    const int slot = s0 + c * kRows + my_row;
    return (slot < s1 && slot < k) ? idx[slot] : -1;
  };
  int pos_cur = nchunks > 0 ? row_index(0) : -1;
  int pos_next = nchunks > 1 ? row_index(1) : -1;

  // query of 16 heads as MFMA A operands: head j, channels 32c + 8g .. +7
  const uint16_t* qh = qg + (((size_t)l * Q + q) * H + 16 * hg) * kKvDim;
  u32x4 qa[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qa[c] = *(const u32x4*)(qh + (size_t)j * kKvDim + 32 * c + 8 * g);

  f32x4 o[8];                                       // MFMA-initialised, as in k_sparse_attn_wide
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = mfma16x16x32(z, z, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  float m_run[4], l_run[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_run[v] = -INFINITY; l_run[v] = 0.f; }

  auto load_chunk = [&](RawRow& r, int c, int pos) {
    const int slot = s0 + c * kRows + my_row;
    r.kind = 0;
    if (slot < s1) {
      if (slot < k) {
        if (pos >= 0 && (int64_t)pos < kv_rows) {
          const u32x4* cp = (const u32x4*)(codes_seq + (size_t)pos * kKvCodeBytes + 64 * quarter);
#pragma unroll
          for (int i = 0; i < 4; ++i) r.d[i] = cp[i];
          r.sc = *(const u32x2*)(scales_seq + (size_t)pos * kKvScaleBytes + 8 * quarter);
          r.kind = 1;
        }
      } else {
        const u32x4* cp = (const u32x4*)(swa_seq + (size_t)(ws + slot - k) * kKvDim + 128 * quarter);
#pragma unroll
        for (int i = 0; i < 8; ++i) r.d[i] = cp[i];
        r.kind = 2;
      }
    }
  };
  RawRow raw;
  if (nchunks > 0) load_chunk(raw, 0, pos_cur);

  for (int c = 0; c < nchunks; ++c) {
    store_row(raw, X + my_row * kXStride, quarter);
    if (quarter == 0) rowok[my_row] = raw.kind != 0;
    lds_barrier();
    if (c + 1 < nchunks) {
      load_chunk(raw, c + 1, pos_next);
      pos_next = c + 2 < nchunks ? row_index(c + 2) : -1;
    }

    // S[head 4g+v][row 16*wave + j]
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xr = X + (16 * wave + j) * kXStride + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) s = mfma16x16x32(qa[cc], *(const u32x4*)(xr + 32 * cc), s);
    const bool row_ok = rowok[16 * wave + j] != 0;
    float sv[4], mx[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = row_ok ? s[v] * scale_log2 : -INFINITY;
      mx[v] = row16_max(sv[v]);
    }
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red_m[wave][4 * g + v] = mx[v];
    }
    lds_barrier();
    float alpha[4], mnew[4], psum[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const float mc = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
      mnew[v] = fmaxf(m_run[v], mc);
      alpha[v] = mnew[v] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[v] - mnew[v]);
      const float p = mnew[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[v] - mnew[v]);
      const uint32_t pb = f32_to_bf16_rne(p);
      P[h * kPStride + 16 * wave + j] = (uint16_t)pb;
      psum[v] = row16_sum(bf16_bits_to_f32(pb));
    }
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red_l[wave][4 * g + v] = psum[v];
    }
    lds_barrier();   // P and red_l written
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const float ps = (red_l[0][h] + red_l[1][h]) + (red_l[2][h] + red_l[3][h]);
      l_run[v] = l_run[v] * alpha[v] + ps;
      m_run[v] = mnew[v];
    }
    // O[head 4g+v][dim 128*wave + 8j + t] = alpha * O + sum_r P[head][r] X[r][dim].  The B operand
    // of tile t needs rows 8g .. 8g+7 of one dim; a lane reads its 8 dims of each row in one
    // 16-byte LDS access and pairs the halves of two rows with byte permutes.
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[t][v] *= alpha[v];
#pragma unroll
    for (int kk = 0; kk < kRows / 32; ++kk) {
      const u32x4 pa = *(const u32x4*)(P + j * kPStride + 32 * kk + 8 * g);
      const uint16_t* xc = X + (32 * kk + 8 * g) * kXStride + 128 * wave + 8 * j;
      u32x4 xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = *(const u32x4*)(xc + e * kXStride);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = __builtin_amdgcn_perm(xv[2 * e + 1][i], xv[2 * e][i], 0x05040100u);
          hi[e] = __builtin_amdgcn_perm(xv[2 * e + 1][i], xv[2 * e][i], 0x07060302u);
        }
        o[2 * i] = mfma16x16x32(pa, lo, o[2 * i]);
        o[2 * i + 1] = mfma16x16x32(pa, hi, o[2 * i + 1]);
      }
    }
    if (c + 1 < nchunks) lds_barrier();   // X, P, red_m and red_l are rewritten by the next chunk
  }

  const size_t hrow = (size_t)lq * H + 16 * hg;      // (layer, query, first head of the group)
  if (n_splits == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const float inv = l_run[v] > 0.f ? 1.f / l_run[v] : 0.f;
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = f32_to_bf16_rne(o[2 * i][v] * inv) | (f32_to_bf16_rne(o[2 * i + 1][v] * inv) << 16);
      *(u32x4*)(out + (hrow + h) * kKvDim + 128 * wave + 8 * j) = pk;
      if (lse && wave == 0 && j == 0)
        lse[hrow + h] = l_run[v] > 0.f ? (m_run[v] + log2f(l_run[v])) * 0.69314718055994531f : -INFINITY;
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const size_t pr = (hrow + h) * n_splits + split;
      const float inv = l_run[v] > 0.f ? 1.f / l_run[v] : 0.f;
      *(u32x4*)(part_o + pr * kKvDim + 128 * wave + 8 * j) =
          u32x4{f16x2_rne(o[0][v] * inv, o[1][v] * inv), f16x2_rne(o[2][v] * inv, o[3][v] * inv),
                f16x2_rne(o[4][v] * inv, o[5][v] * inv), f16x2_rne(o[6][v] * inv, o[7][v] * inv)};
      if (wave == 0 && j == 0) {
        part_ml[pr * 2] = m_run[v];
        part_ml[pr * 2 + 1] = l_run[v];
      }
    }
  }
}

// 64 heads per workgroup (H % 64 == 0), 8 waves, X double-buffered.  Wave w owns head group hg = w % 4 (heads
// 64*blockIdx.y + 16*hg .. +15) and half hf = w / 4: for the scores it takes rows 32*hf .. +31 of
// each 64-row chunk, for O += P X it accumulates dims 256*hf .. +255 over all 64 rows.  The scores
// are computed as S^T = X Q^T (X rows as the A operand, the query as B), so lane (j, g) holds head j
// and rows 4g .. 4g+3 of each 16-row tile: the softmax reductions of a head run inside the lane and
// across its four 16-lane groups.  The two waves of a head group exchange their row maxima, sums
// and P tiles through LDS, so each gathered row is dequantised once for all 64 heads and a wave
// holds 16 heads x 256 dims of accumulators (two waves per SIMD fit).  grid (n_splits, H/64, L*Q);
// outputs as k_sparse_attn.
constexpr int kWideThreads = 512;

struct RawRow8 {         // this thread's eighth (64 channels) of one chunk row
  u32x4 d[4];            // main: d[0..1] = 32 code bytes; SWA: d[0..3] = 64 E4M3 bytes
  uint32_t sc;           // main: 4 scale bytes
  int kind;              // 0 empty, 1 main, 2 SWA
};

// Dequantise this thread's eighth row into LDS (64 bf16 = 8 x 16 bytes).
__device__ __forceinline__ void store_row8(const RawRow8& r, uint16_t* xrow, int eighth) {
  u32x4* dst = (u32x4*)(xrow + 64 * eighth);
  if (r.kind == 1) {
    // the four scale bytes through the hardware E4M3 conversion (exact), two per instruction
    const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc, 1.0f, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.sc, 1.0f, true);
#pragma unroll
    for (int i = 0; i < 4; ++i) {                      // scale group i: 8 code bytes, 16 channels
      const float s = i == 0 ? s01.x : (i == 1 ? s01.y : (i == 2 ? s23.x : s23.y));
      const uint32_t w0 = r.d[i >> 1][(i & 1) * 2], w1 = r.d[i >> 1][(i & 1) * 2 + 1];
      dst[2 * i] = u32x4{e2m1x2_scaled_to_bf16x2<0>(w0, s), e2m1x2_scaled_to_bf16x2<1>(w0, s),
                         e2m1x2_scaled_to_bf16x2<2>(w0, s), e2m1x2_scaled_to_bf16x2<3>(w0, s)};
      dst[2 * i + 1] = u32x4{e2m1x2_scaled_to_bf16x2<0>(w1, s), e2m1x2_scaled_to_bf16x2<1>(w1, s),
                             e2m1x2_scaled_to_bf16x2<2>(w1, s), e2m1x2_scaled_to_bf16x2<3>(w1, s)};
    }
  } else if (r.kind == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[2 * i] = e4m3x8_to_bf16x8(r.d[i].x, r.d[i].y);
      dst[2 * i + 1] = e4m3x8_to_bf16x8(r.d[i].z, r.d[i].w);
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = z;
  }
}

__global__ __launch_bounds__(kWideThreads) void k_sparse_attn_wide(
    const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales, int64_t kv_rows,
    const uint16_t* __restrict__ qg, const int32_t* __restrict__ idx_sets, LayerSets sets,
    const uint8_t* __restrict__ swa, int swa_rows, const int32_t* __restrict__ swa_end, int window,
    int Q, int B, int T, int H, int k, float scale_log2, int split_rows, int n_splits,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t X[2][kRows * kXStride];   // chunk c in X[c & 1]
  __shared__ __attribute__((aligned(16))) uint16_t P[4 * 16 * kPStride];
  __shared__ float red_m[2][64], red_l[2][64];           // [half][16 * head group + head]
  __shared__ float alpha_s[64];                          // rescale factor of each head (rare use)
  __shared__ __attribute__((aligned(16))) int32_t rowok[2][kRows];

  const int split = blockIdx.x, hq = blockIdx.y, lq = blockIdx.z;
  const int l = lq / Q, q = lq % Q, b = q / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave & 3, hf = wave >> 2;
  const int j = lane & 15, g = lane >> 4;
  const int32_t* idx = idx_sets + ((size_t)sets.set[l] * Q + q) * k;
  int we = swa_end[q];
  we = we < 0 ? 0 : (we > swa_rows ? swa_rows : we);
  const int ws = max(0, we - window);
  const int nslots = k + (we - ws);
  const int s0 = split * split_rows, s1 = min(nslots, s0 + split_rows);
  const int nchunks = s1 > s0 ? (s1 - s0 + kRows - 1) / kRows : 0;
  const uint8_t* codes_seq = kv_codes + (size_t)b * kv_rows * kKvCodeBytes;
  const uint8_t* scales_seq = kv_scales + (size_t)b * kv_rows * kKvScaleBytes;
  const uint8_t* swa_seq = swa + ((size_t)l * B + b) * (size_t)swa_rows * kKvDim;

  // lane l of wave w takes row 8w + l % 8, eighth l / 8 (rows differ within each LDS write pass;
  // see k_sparse_attn)
  const int my_row = 8 * (tid >> 6) + (tid & 7), eighth = (tid >> 3) & 7;
  auto row_index = [&](int c) {
    const int slot = s0 + c * kRows + my_row;
    return (slot < s1 && slot < k) ? idx[slot] : -1;
  };
  int pos_a = nchunks > 0 ? row_index(0) : -1;
  int pos_b = nchunks > 1 ? row_index(1) : -1;

  const int hbase = 64 * hq + 16 * hg;              // this wave's first head
  const uint16_t* qh = qg + (((size_t)l * Q + q) * H + hbase) * kKvDim;
  u32x4 qa[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qa[c] = *(const u32x4*)(qh + (size_t)j * kKvDim + 32 * c + 8 * g);

  // Accumulators start as MFMA results (of zero operands), so the compiler keeps them in the
  // accumulation registers across the loop.
  f32x4 o[16];                                       // tile u: dims 256*hf + 16u + j
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 16; ++t) o[t] = mfma16x16x32(z, z, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  float m_run = -INFINITY, l_run = 0.f;             // head j of the group (both halves agree)
  uint16_t* Pg = P + hg * 16 * kPStride;

  auto load_chunk = [&](RawRow8& r, int c, int pos) {
    const int slot = s0 + c * kRows + my_row;
    r.kind = 0;
    if (slot < s1) {
      if (slot < k) {
        if (pos >= 0 && (int64_t)pos < kv_rows) {
          const u32x4* cp = (const u32x4*)(codes_seq + (size_t)pos * kKvCodeBytes + 32 * eighth);
          r.d[0] = cp[0];
          r.d[1] = cp[1];
          r.sc = *(const uint32_t*)(scales_seq + (size_t)pos * kKvScaleBytes + 4 * eighth);
          r.kind = 1;
        }
      } else {
        const u32x4* cp = (const u32x4*)(swa_seq + (size_t)(ws + slot - k) * kKvDim + 64 * eighth);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.d[i] = cp[i];
        r.kind = 2;
      }
    }
  };
  // Pipeline: chunk c is scored from X[c & 1] while chunk c+1 is dequantised into the other buffer
  // (between the softmax and O += P X of chunk c) and the raw rows of chunk c+2 are in flight.
  RawRow8 raw;
  if (nchunks > 0) {
    load_chunk(raw, 0, pos_a);
    store_row8(raw, X[0] + my_row * kXStride, eighth);
    if (eighth == 0) rowok[0][my_row] = raw.kind != 0;
  }
  if (nchunks > 1) load_chunk(raw, 1, pos_b);
  int pos_c = nchunks > 2 ? row_index(2) : -1;
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const uint16_t* Xc = X[c & 1];
    // S^T[row 32*hf + 16r + 4g + v][head j]
    f32x4 s[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) s[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        s[r] = mfma16x16x32(*(const u32x4*)(Xc + (32 * hf + 16 * r + j) * kXStride + 32 * cc + 8 * g), qa[cc], s[r]);
    float sv[2][4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int4 ok = *(const int4*)&rowok[c & 1][32 * hf + 16 * r + 4 * g];
      const int okv[4] = {ok.x, ok.y, ok.z, ok.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[r][v] = okv[v] != 0 ? s[r][v] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[r][v]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) red_m[hf][16 * hg + j] = mx;
    lds_barrier();                                 // both halves' maxima
    // The reference point of a head moves only when the chunk's max exceeds it by more than
    // kLazyLog2, so P <= 2^kLazyLog2 and O is rescaled only on such a move.  Both waves of a head
    // group take identical decisions (same maxima, same order).
    const float m = fmaxf(red_m[0][16 * hg + j], red_m[1][16 * hg + j]);
    const bool mv = m > m_run + kLazyLog2;           // true from -inf to finite
    const float mnew = mv ? m : m_run;
    const bool moved = mv && m_run != -INFINITY;
    const float alpha = moved ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
    // exponents are at most kLazyLog2 (no overflow); results below 2^-126 may flush to zero, far
    // below the rounding of the weights that matter.  P[head j][rows 32hf + 16r + 4g .. +3] as bf16,
    // and the sum of the rounded weights.
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t pk[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float p0 = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r][2 * e] - mnew);
        const float p1 = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r][2 * e + 1] - mnew);
        pk[e] = bf16x2_rne(p0, p1);
        ps += __uint_as_float(pk[e] << 16);
        ps += __uint_as_float(pk[e] & 0xffff0000u);
      }
      *(u32x2*)(Pg + j * kPStride + 32 * hf + 16 * r + 4 * g) = u32x2{pk[0], pk[1]};
    }
    ps += __shfl_xor(ps, 16);                        // the same sum in all four groups
    ps += __shfl_xor(ps, 32);
    if (g == 0) {
      red_l[hf][16 * hg + j] = ps;
      if (hf == 0) alpha_s[16 * hg + j] = alpha;
    }
    m_run = mnew;
    lds_barrier();                                 // P tiles, both halves' sums, the factors
    l_run = l_run * alpha + (red_l[0][16 * hg + j] + red_l[1][16 * hg + j]);
    if (__ballot(moved) != 0) {                      // wave-uniform, rare
      float a4[4];                                   // O holds heads 4g .. 4g+3 in a lane
#pragma unroll
      for (int v = 0; v < 4; ++v) a4[v] = alpha_s[16 * hg + 4 * g + v];
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[t][v] *= a4[v];
    }
    // the next chunk into the other buffer (last read before the previous barrier), then the
    // raw rows of the chunk after it
    auto dequant_next = [&]() {
      if (c + 1 < nchunks) {
        store_row8(raw, X[(c + 1) & 1] + my_row * kXStride, eighth);
        if (eighth == 0) rowok[(c + 1) & 1][my_row] = raw.kind != 0;
        if (c + 2 < nchunks) {
          load_chunk(raw, c + 2, pos_c);
          pos_c = c + 3 < nchunks ? row_index(c + 3) : -1;
        }
      }
    };
    // O[head 4g+v][dim 256*hf + 16*u + j] += sum_r P[head][r] X[r][dim].  The B operand of tile u
    // (rows 32kk + 8g .. +7 of dim 256hf + 16u + j in lane (j, g)) comes straight from row-major X
    // by two LDS transpose reads: in each 16-lane group, lane 4a+b receives element b of the
    // 8 bytes addressed by lanes a, a+4, a+8 and a+12, so lane j = 4a+i addresses row
    // 32kk + 8g + i (+4 for the second read), dims 256hf + 16u + 4a .. +3.
    auto accumulate = [&]() {
#pragma unroll
      for (int kk = 0; kk < kRows / 32; ++kk) {
        const u32x4 pa = *(const u32x4*)(Pg + j * kPStride + 32 * kk + 8 * g);
        const uint16_t* xt = Xc + (32 * kk + 8 * g + (j >> 2)) * kXStride + 256 * hf + 4 * (j & 3);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const u32x2 lo = ds_read_tr16(xt + 16 * u);
          const u32x2 hi = ds_read_tr16(xt + 4 * kXStride + 16 * u);
          o[u] = mfma16x16x32(pa, u32x4{lo.x, lo.y, hi.x, hi.y}, o[u]);
        }
      }
    };
    // Waves w and w + 4 share a SIMD (one of each half): one dequantises while the other runs its
    // MFMAs, then they swap, so the VALU and matrix work of the pair overlap.
    if (hf == 0) {
      accumulate();
      dequant_next();
    } else {
      dequant_next();
      accumulate();
    }
    if (c + 1 < nchunks) lds_barrier();            // next chunk's X and rowok written; P, red_* free
  }

  // O leaves through LDS (the chunk tiles are free once every wave has finished its last
  // O += P X): tile u of a lane holds dims 256hf + 16u + j, and each lane then stores four
  // consecutive dims of one head at a time.
  constexpr int kOStride = kKvDim + 4;                // floats per staged head row
  static_assert(64 * kOStride * 4 <= (int)sizeof(X), "the staged output fits in the chunk tiles");
  float* Os = reinterpret_cast<float*>(&X[0][0]);
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 16; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) Os[(16 * hg + 4 * g + v) * kOStride + 256 * hf + 16 * u + j] = o[u][v];
  if (hf == 0 && g == 0) {
    red_m[0][16 * hg + j] = m_run;
    red_l[0][16 * hg + j] = l_run;
  }
  lds_barrier();
  const size_t hrow = (size_t)lq * H;
  for (int hh = 0; hh < 16; ++hh) {
    const int head = 16 * hg + hh, h = 64 * hq + head;
    const f32x4 ov = *(const f32x4*)(Os + head * kOStride + 256 * hf + 4 * lane);
    const float mh = red_m[0][head], lh = red_l[0][head];
    if (n_splits == 1) {
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      const u32x2 pk = {f32_to_bf16_rne(ov.x * inv) | (f32_to_bf16_rne(ov.y * inv) << 16),
                        f32_to_bf16_rne(ov.z * inv) | (f32_to_bf16_rne(ov.w * inv) << 16)};
      *(u32x2*)(out + (hrow + h) * kKvDim + 256 * hf + 4 * lane) = pk;
      if (lse && hf == 0 && lane == 0) lse[hrow + h] = lh > 0.f ? (mh + log2f(lh)) * 0.69314718055994531f : -INFINITY;
    } else {
      const size_t pr = (hrow + h) * n_splits + split;
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      *(u32x2*)(part_o + pr * kKvDim + 256 * hf + 4 * lane) =
          u32x2{f16x2_rne(ov.x * inv, ov.y * inv), f16x2_rne(ov.z * inv, ov.w * inv)};
      if (hf == 0 && lane == 0) {
        part_ml[pr * 2] = mh;
        part_ml[pr * 2 + 1] = lh;
      }
    }
  }
}

// grid (H, L*Q), one wave per head: lane i merges dims 8i .. 8i+7 over the head's n_splits
// partial states.  Every split slot up to kMax (a bound on n_splits chosen at launch) is
// loaded up front (indices past n_splits clamp to the last split and get weight zero), so the
// loads of a lane are all in flight together.
constexpr int kMaxSplits = 16;
template <int kMax>
__global__ __launch_bounds__(64) void k_attn_combine(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml, int n_splits, int H,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const size_t hrow = (size_t)blockIdx.y * H + blockIdx.x;
  const int lane = threadIdx.x;
  const float* ml = part_ml + hrow * n_splits * 2;
  float m[kMax], l[kMax];
  u32x4 a[kMax];                               // 8 fp16 dims of the split's normalised row
#pragma unroll
  for (int s = 0; s < kMax; ++s) {
    const int sc = s < n_splits ? s : n_splits - 1;
    m[s] = ml[2 * sc];
    l[s] = ml[2 * sc + 1];
    a[s] = *(const u32x4*)(part_o + (hrow * n_splits + sc) * kKvDim + 8 * lane);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMax; ++s) M = fmaxf(M, s < n_splits ? m[s] : -INFINITY);
  // split s holds O_s / l_s, so it enters with weight 2^(m_s - M) * l_s
  float L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMax; ++s) {
    const float w = (s < n_splits && m[s] != -INFINITY) ? exp2f(m[s] - M) * l[s] : 0.f;
    L += w;
    const h8 v = __builtin_bit_cast(h8, a[s]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += w * (float)v[i];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = f32_to_bf16_rne(acc[2 * i] * inv) | (f32_to_bf16_rne(acc[2 * i + 1] * inv) << 16);
  *(u32x4*)(out + hrow * kKvDim + 8 * lane) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  if (lse && lane == 0) lse[hrow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

AttnPlan plan_attn(int L, int B, int T, int H, int k, int window) {
  AttnPlan p;
  p.heads_per_wg = H % 64 == 0 ? 64 : 16;
  const long long groups = (long long)L * B * T * (H / p.heads_per_wg);
  const int rows_max = k + window;
  const int max_chunks = (rows_max + kRows - 1) / kRows;
  // splits to reach ~512 workgroups of the 16-head kernel (two fit on a CU); the 64-head kernel
  // fits one workgroup per CU, so its splits stop at one round of ~256 workgroups: a second,
  // partial round costs more than the longer splits (measured on the batch-8 and caller-pool
  // workloads: 41.9 and 39.5 us with ~400 and 320 workgroups)
  long long want = p.heads_per_wg == 64 ? std::max(1LL, 256 / groups) : (512 + groups - 1) / groups;
  int splits = (int)(want < max_chunks ? want : max_chunks);
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  int chunks_per = (max_chunks + splits - 1) / splits;
  p.split_rows = chunks_per * kRows;
  if (p.split_rows > kMaxSplitRows) p.split_rows = kMaxSplitRows;
  p.n_splits = (rows_max + p.split_rows - 1) / p.split_rows;
  if (p.n_splits < 1) p.n_splits = 1;
  const size_t heads = (size_t)L * B * T * H;
  p.ws_bytes = p.n_splits > 1 ? heads * p.n_splits * (kKvDim * sizeof(uint16_t) + 2 * sizeof(float)) : 0;
  return p;
}

hipError_t launch_sparse_attn(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t kv_rows,
                              const uint16_t* q, const int32_t* idx_sets, const LayerSets& sets,
                              const uint8_t* swa, int swa_rows, const int32_t* swa_end, int window,
                              int L, int B, int T, int H, int k, float scale, uint16_t* out,
                              float* lse, void* workspace, hipStream_t s) {
  const int Q = B * T;
  const float scale_log2 = scale * 1.4426950408889634f;
  const AttnPlan p = plan_attn(L, B, T, H, k, window);
  uint16_t* part_o = (uint16_t*)workspace;          // fp16 normalised rows, then fp32 (m, l) pairs
  float* part_ml = part_o ? (float*)(part_o + (size_t)L * Q * H * p.n_splits * kKvDim) : nullptr;
  if (p.heads_per_wg == 64)
    hipLaunchKernelGGL(k_sparse_attn_wide, dim3(p.n_splits, H / 64, L * Q), dim3(kWideThreads), 0, s,
                       kv_codes, kv_scales, kv_rows, q, idx_sets, sets, swa, swa_rows, swa_end, window, Q,
                       B, T, H, k, scale_log2, p.split_rows, p.n_splits, part_o, part_ml, out, lse);
  else
    hipLaunchKernelGGL(k_sparse_attn, dim3(p.n_splits, H / 16, L * Q), dim3(kAttnThreads), 0, s, kv_codes,
                       kv_scales, kv_rows, q, idx_sets, sets, swa, swa_rows, swa_end, window, Q, B, T, H, k,
                       scale_log2, p.split_rows, p.n_splits, part_o, part_ml, out, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const dim3 cg(H, L * Q);
  if (p.n_splits <= 4)
    hipLaunchKernelGGL(k_attn_combine<4>, cg, dim3(64), 0, s, part_o, part_ml, p.n_splits, H, out, lse);
  else if (p.n_splits <= 8)
    hipLaunchKernelGGL(k_attn_combine<8>, cg, dim3(64), 0, s, part_o, part_ml, p.n_splits, H, out, lse);
  else if (p.n_splits <= 12)
    hipLaunchKernelGGL(k_attn_combine<12>, cg, dim3(64), 0, s, part_o, part_ml, p.n_splits, H, out, lse);
  else
    hipLaunchKernelGGL(k_attn_combine<kMaxSplits>, cg, dim3(64), 0, s, part_o, part_ml, p.n_splits, H, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
