// Candidate-pool and Top-K selection (gfx950).
//
// Both selections rank 64-bit keys (score order key << 32 | ~index), so "larger score first,
// then lower index first" is a plain descending order of distinct keys
// (blog.4sapi.com sec.4 and readance.app sec.4.3: Top-K inside the candidate pool; ties go to
// the lower index, a reading this library fixes).  The k-th largest key is found by a radix
// select whose digit width adapts to the live key range: each pass histograms the keys inside
// [lo, hi] into at most 4096 bins of width 2^shift, keeps the bin holding the k-th key, and
// repeats until the bin is a single key.  Selected elements are then written in ascending
// index order with a block-wide prefix count.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

constexpr int kBins = 4096;
constexpr int kNT = kSelectThreads;      // 1024 threads
constexpr int kWaves = kNT / 64;
constexpr int kCandCap = 8192;           // keys kept in LDS once a bin is small enough

struct SelectSmem {
  uint32_t hist[kBins];
  uint32_t wsum[kWaves];
  uint64_t w64a[kWaves];
  uint64_t w64b[kWaves];
  uint32_t found_bin, found_above, found_cnt, ncand;
};

// ------------------------------------------------------------------ block-wide helpers

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t n = (uint32_t)__shfl_up((int)v, o);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over the block (thread order); also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, SelectSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sm.wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    uint32_t s = sm.wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int o) {
  uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
  uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void block_minmax64(uint64_t& mn, uint64_t& mx, SelectSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t a = shfl_xor64(mn, o), b = shfl_xor64(mx, o);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) { sm.w64a[wave] = mn; sm.w64b[wave] = mx; }
  __syncthreads();
  mn = ~0ull; mx = 0ull;
  for (int w = 0; w < kWaves; ++w) {
    mn = sm.w64a[w] < mn ? sm.w64a[w] : mn;
    mx = sm.w64b[w] > mx ? sm.w64b[w] : mx;
  }
  __syncthreads();
}

// Among the histogram bins, find b with above(b) < need <= above(b) + hist[b], where above(b)
// counts the keys in bins > b.  Result in sm.found_*.
__device__ __forceinline__ void find_bin(int nbins, uint32_t need, SelectSmem& sm) {
  const int t = threadIdx.x;
  uint32_t h[4], mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int bin = 4 * t + i;
    h[i] = bin < nbins ? sm.hist[bin] : 0u;
    mine += h[i];
  }
  uint32_t total;
  uint32_t below = block_excl_scan(mine, total, sm);
  uint32_t above = total - below - mine;           // keys in bins of higher threads
  if (above < need && need <= above + mine) {
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (above < need && need <= above + h[i]) {
        sm.found_bin = 4 * t + i;
        sm.found_above = above;
        sm.found_cnt = h[i];
      }
      above += h[i];
    }
  }
  __syncthreads();
}

// The need-th largest of a set of distinct 64-bit keys, all inside [lo, hi] (need >= 1 and at
// least `need` keys in range).  for_each(f) calls f(key) for every key this thread holds; keys
// outside [lo, hi] are skipped.  When `cand` is non-null, keys are copied into it once the
// surviving bin holds at most kCandCap of them, and later passes read only the copy.
template <class ForEach>
__device__ uint64_t select_kth(ForEach for_each, uint32_t need, uint64_t lo, uint64_t hi,
                               SelectSmem& sm, uint64_t* cand) {
  bool use_cand = false;
  while (true) {
    const uint64_t range = hi - lo;
    if (range == 0) return lo;
    const int shift = max(0, bitlen64(range) - 12);
    const int nbins = (int)(range >> shift) + 1;
    for (int i = threadIdx.x; i < nbins; i += kNT) sm.hist[i] = 0u;
    __syncthreads();
    auto count = [&](uint64_t k) {
      if (k >= lo && k <= hi) atomicAdd(&sm.hist[(uint32_t)((k - lo) >> shift)], 1u);
    };
    if (use_cand) {
      const uint32_t n = sm.ncand;
      for (uint32_t i = threadIdx.x; i < n; i += kNT) count(cand[i]);
    } else {
      for_each(count);
    }
    __syncthreads();
    find_bin(nbins, need, sm);
    const uint32_t bin = sm.found_bin, above = sm.found_above, cnt = sm.found_cnt;
    need -= above;
    const uint64_t nlo = lo + ((uint64_t)bin << shift);
    const uint64_t nhi = shift == 0 ? nlo : min(hi, nlo + (((uint64_t)1 << shift) - 1));
    lo = nlo;
    hi = nhi;
    if (shift == 0) return lo;
    if (cand && !use_cand && cnt <= (uint32_t)kCandCap) {
      if (threadIdx.x == 0) sm.ncand = 0;
      __syncthreads();
      for_each([&](uint64_t k) {
        if (k >= lo && k <= hi) cand[atomicAdd(&sm.ncand, 1u)] = k;
      });
      __syncthreads();
      use_cand = true;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ candidate pool

// One WG per query: keep the top `P` blocks by (block max desc, block asc) and write their
// visible positions in ascending order; a query with at most P blocks keeps all of them.
__global__ __launch_bounds__(kNT) void k_pool_select(
    const uint32_t* __restrict__ blkkey, int nb_max, const int32_t* __restrict__ n_visible,
    int n_max, int P, const uint32_t* __restrict__ wg_minmax, int n_wg,
    int32_t* __restrict__ pool_pos, int cap_out, int32_t* __restrict__ pool_len) {
  __shared__ SelectSmem sm;
  __shared__ uint64_t cand[kCandCap];
  const int q = blockIdx.x, t = threadIdx.x;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int nb = (nv + kBlock - 1) / kBlock;
  const uint32_t* keys = blkkey + (size_t)q * nb_max;
  int32_t* out = pool_pos + (size_t)q * cap_out;

  uint64_t thr = 0;   // selected: rank_key >= thr
  if (nb > P) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = t; i < n_wg; i += kNT) {
      kmin = min(kmin, wg_minmax[((size_t)q * n_wg + i) * 2]);
      kmax = max(kmax, wg_minmax[((size_t)q * n_wg + i) * 2 + 1]);
    }
    uint64_t mn = rank_key(kmin, (uint32_t)(nb - 1)), mx = rank_key(kmax, 0u);
    block_minmax64(mn, mx, sm);
    auto for_each = [&](auto f) {
      for (int j = t; j < nb; j += kNT) f(rank_key(keys[j], (uint32_t)j));
    };
    thr = select_kth(for_each, (uint32_t)P, mn, mx, sm, cand);
  }
  // ascending output: thread t owns blocks [j0, j1)
  const int per = (nb + kNT - 1) / kNT;
  const int j0 = min(nb, t * per), j1 = min(nb, j0 + per);
  uint32_t cnt = 0;
  for (int j = j0; j < j1; ++j)
    if (nb <= P || rank_key(keys[j], (uint32_t)j) >= thr) cnt += min(kBlock, nv - kBlock * j);
  uint32_t total;
  uint32_t off = block_excl_scan(cnt, total, sm);
  for (int j = j0; j < j1; ++j) {
    if (nb <= P || rank_key(keys[j], (uint32_t)j) >= thr) {
      const int n = min(kBlock, nv - kBlock * j);
      for (int r = 0; r < n; ++r) out[off++] = kBlock * j + r;
    }
  }
  for (int i = (int)total + t; i < cap_out; i += kNT) out[i] = -1;
  if (t == 0) pool_len[q] = (int32_t)total;
}

hipError_t launch_pool_select(const uint32_t* blkkey, int nb_max, const int32_t* n_visible,
                              int n_max, int pool_blocks, const uint32_t* wg_minmax, int n_wg,
                              int32_t* pool_pos, int pool_cap_out, int32_t* pool_len, int Q,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_pool_select, dim3(Q), dim3(kNT), 0, s, blkkey, nb_max, n_visible, n_max,
                     pool_blocks, wg_minmax, n_wg, pool_pos, pool_cap_out, pool_len);
  return hipGetLastError();
}

// ------------------------------------------------------------------ Top-K

constexpr int kTopE = kMaxPool / kNT;    // candidates per thread (16)

// One WG per item (it = l*Q + q).  Candidates: slots [0, len) of the item's query; slot i has
// position cand_pos[i] (ignored if negative or >= n_rows).  Output: the k best positions in
// ascending order with their scores, -1 / 0 padded.
__global__ __launch_bounds__(kNT) void k_topk(
    const int32_t* __restrict__ cand_pos, const int32_t* __restrict__ cand_len, int cap,
    int64_t n_rows, const float* __restrict__ scores, int64_t score_stride, int by_position,
    int Q, int k, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  __shared__ SelectSmem sm;
  const int it = blockIdx.x, q = it % Q, t = threadIdx.x;
  int len = cand_len[q];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int32_t* cp = cand_pos + (size_t)q * cap;
  const float* sc = scores + (size_t)(by_position ? q : it) * score_stride;

  uint64_t key[kTopE];
  uint32_t nvalid = 0;
  uint64_t mn = ~0ull, mx = 0ull;
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    const int slot = t * kTopE + e;
    key[e] = 0ull;
    if (slot < len) {
      const int pos = cp[slot];
      if (pos >= 0 && (int64_t)pos < n_rows) {
        const float s = sc[by_position ? pos : slot];
        key[e] = rank_key(score_key(s), (uint32_t)pos);
        ++nvalid;
        mn = key[e] < mn ? key[e] : mn;
        mx = key[e] > mx ? key[e] : mx;
      }
    }
  }
  uint32_t total_valid;
  (void)block_excl_scan(nvalid, total_valid, sm);
  uint64_t thr = 1ull;   // every valid key is >= 1
  if (total_valid > (uint32_t)k) {
    block_minmax64(mn, mx, sm);
    auto for_each = [&](auto f) {
#pragma unroll
      for (int e = 0; e < kTopE; ++e) f(key[e]);
    };
    thr = select_kth(for_each, (uint32_t)k, mn, mx, sm, nullptr);
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < kTopE; ++e) cnt += key[e] >= thr ? 1u : 0u;
  uint32_t total;
  uint32_t off = block_excl_scan(cnt, total, sm);
  int32_t* oi = out_idx + (size_t)it * k;
  float* os = out_score ? out_score + (size_t)it * k : nullptr;
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    if (key[e] >= thr) {
      oi[off] = (int32_t)rank_key_index(key[e]);
      if (os) os[off] = key_score((uint32_t)(key[e] >> 32));
      ++off;
    }
  }
  for (int i = (int)total + t; i < k; i += kNT) {
    oi[i] = -1;
    if (os) os[i] = 0.f;
  }
}

hipError_t launch_topk(const int32_t* cand_pos, const int32_t* cand_len, int cap, int64_t n_rows,
                       const float* scores, int64_t score_stride, bool by_position, int items,
                       int Q, int k, int32_t* out_idx, float* out_score, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3(items), dim3(kNT), 0, s, cand_pos, cand_len, cap, n_rows, scores,
                     score_stride, by_position ? 1 : 0, Q, k, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace csa2
