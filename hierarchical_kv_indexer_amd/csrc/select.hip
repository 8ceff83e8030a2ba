// Candidate-pool and Top-K selection (gfx950).
//
// Both selections rank 64-bit keys (score order key << 32 | ~index), so "larger score first,
// then lower index first" is a plain descending order of distinct keys
// (blog.4sapi.com sec.4 and readance.app sec.4.3: Top-K inside the candidate pool; ties go to
// the lower index, a reading this library fixes).
//
// k-th largest key: a radix select whose digit width adapts to the live key range.  Each pass
// histograms the keys inside [lo, hi] into at most 4096 bins of width 2^shift and keeps the bin
// holding the k-th key; once that bin holds at most kRankMax keys they are ranked directly.
//
// Pool selection does not revisit every block: the scan leaves, for each unit (one wave's
// contiguous range of blocks), its four best blocks and the fifth best key.  With T0 = the
// P-th best listed key (T0 <= the true P-th best key T*, the listed keys being a subset), a unit
// whose fifth best key is below T0 has no unlisted block that can be selected; only the units
// whose fifth best key reaches T0 are re-read in full.  The P best of the surviving candidates
// are exactly the P best blocks (and when no unit is re-read, T* = T0).
//
// Layout: element i of thread t is slot i*1024 + t, so every load instruction of a wave reads
// consecutive addresses; outputs keep slot order through per-(element, wave) ballot counts.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

constexpr int kBins = 4096;
constexpr int kNT = kSelectThreads;      // 1024 threads
constexpr int kWaves = kNT / 64;
constexpr int kRankMax = 256;            // bins this small are resolved by direct ranking
constexpr int kCandCap = 4096;           // LDS candidates (saturated units, slow-path compaction)
constexpr int kTopE = kMaxPool / kNT;    // slots per thread (16)
constexpr int kUnitsPerThread = 4;       // units per thread in the pool kernel (<= 4096 units)

struct SelectSmem {
  uint32_t hist[kBins];
  uint64_t rankbuf[kRankMax];
  uint32_t rank[kRankMax];
  uint32_t wsum[2][kWaves];
  uint32_t wmin[2][kWaves];
  uint32_t wmax[2][kWaves];
  uint32_t ecnt[kTopE * kWaves];
  uint64_t result;
  uint32_t found_bin, found_above, found_cnt, ncand, nrank, nsat;
};

// Block-wide collectives.  Each alternates between two LDS buffers, so one barrier per call
// suffices: a buffer is rewritten only after the next call's barrier.
struct Block {
  SelectSmem& sm;
  int parity = 0;

  // Exclusive prefix sum in thread order; also returns the total.
  __device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_sum(v);
    if (lane == 63) sm.wsum[parity][wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t s = sm.wsum[parity][w];
      before += w < wave ? s : 0u;
      tot += s;
    }
    parity ^= 1;
    total = tot;
    return before + inc - v;
  }
  __device__ __forceinline__ uint32_t sum(uint32_t v) {
    uint32_t total;
    (void)excl_scan(v, total);
    return total;
  }
  __device__ __forceinline__ void minmax(uint32_t& mn, uint32_t& mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) { sm.wmin[parity][wave] = mn; sm.wmax[parity][wave] = mx; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mn = min(mn, sm.wmin[parity][w]);
      mx = max(mx, sm.wmax[parity][w]);
    }
    parity ^= 1;
  }
};

// Find b with above(b) < need <= above(b) + hist[b] (above(b): keys in bins > b).
__device__ __forceinline__ void find_bin(int nbins, uint32_t need, Block& bk) {
  SelectSmem& sm = bk.sm;
  const int t = threadIdx.x;
  uint32_t h[4], mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bin = 4 * t + i;
    h[i] = bin < nbins ? sm.hist[bin] : 0u;
    mine += h[i];
  }
  uint32_t total;
  const uint32_t below = bk.excl_scan(mine, total);
  uint32_t above = total - below - mine;
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

// Bounds [lo, hi] on ranking keys whose score keys lie in [mn32, mx32].
__device__ __forceinline__ uint64_t key_lo(uint32_t mn32) { return (uint64_t)mn32 << 32; }
__device__ __forceinline__ uint64_t key_hi(uint32_t mx32) { return ((uint64_t)mx32 << 32) | 0xffffffffull; }

// The need-th largest of a set of distinct 64-bit keys, all inside [lo, hi] (1 <= need <= the
// number of keys).  for_each(f) calls f(key) for every key this thread holds (keys outside
// [lo, hi], e.g. 0 for "none", are ignored).  If `cand` is non-null, the keys of a bin with at
// most kCandCap keys are copied there once and later passes read only the copy.
template <class ForEach>
__device__ uint64_t select_kth(ForEach for_each, uint32_t need, uint64_t lo, uint64_t hi, Block& bk,
                               uint64_t* cand) {
  SelectSmem& sm = bk.sm;
  bool use_cand = false;
  while (true) {
    if (lo == hi) return lo;
    const int shift = max(0, bitlen64(hi - lo) - 12);
    const int nbins = (int)((hi - lo) >> shift) + 1;
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
    find_bin(nbins, need, bk);
    const uint32_t bin = sm.found_bin, above = sm.found_above, cnt = sm.found_cnt;
    need -= above;
    const uint64_t nlo = lo + ((uint64_t)bin << shift);
    const uint64_t nhi = shift == 0 ? nlo : min(hi, nlo + (((uint64_t)1 << shift) - 1));
    lo = nlo;
    hi = nhi;
    if (shift == 0) return lo;
    if (cnt <= (uint32_t)kRankMax) {
      // rank the few keys of the bin directly
      if (threadIdx.x == 0) sm.nrank = 0;
      __syncthreads();
      auto collect = [&](uint64_t k) {
        if (k >= lo && k <= hi) sm.rankbuf[atomicAdd(&sm.nrank, 1u)] = k;
      };
      if (use_cand) {
        const uint32_t n = sm.ncand;
        for (uint32_t i = threadIdx.x; i < n; i += kNT) collect(cand[i]);
      } else {
        for_each(collect);
      }
      if (threadIdx.x < kRankMax) sm.rank[threadIdx.x] = 0u;
      __syncthreads();
      {
        // key i = t % kRankMax is compared with a quarter of the bin by each of 4 threads
        const uint32_t i = threadIdx.x % kRankMax, part = threadIdx.x / kRankMax;
        if (i < cnt) {
          const uint64_t x = sm.rankbuf[i];
          const uint32_t b0 = part * (kRankMax / 4), b1 = min(cnt, b0 + kRankMax / 4);
          uint32_t r = 0;
          for (uint32_t m = b0; m < b1; ++m) r += sm.rankbuf[m] > x ? 1u : 0u;
          if (r) atomicAdd(&sm.rank[i], r);
        }
      }
      __syncthreads();
      if (threadIdx.x < cnt && sm.rank[threadIdx.x] == need - 1) sm.result = sm.rankbuf[threadIdx.x];
      __syncthreads();
      return sm.result;
    }
    if (cand && !use_cand && cnt <= (uint32_t)kCandCap) {
      if (threadIdx.x == 0) sm.ncand = 0;
      __syncthreads();
      for_each([&](uint64_t k) {
        if (k >= lo && k <= hi) cand[atomicAdd(&sm.ncand, 1u)] = k;
      });
      use_cand = true;
    }
    __syncthreads();
  }
}

// Offsets that keep slot order (slot = i*kNT + t) for per-slot counts c[i]: returns in off[i]
// the number of counted items in all earlier slots; total = their sum.  N <= kTopE.
template <int N>
__device__ __forceinline__ uint32_t ordered_offsets(const uint32_t (&c)[N], uint32_t (&off)[N], Block& bk) {
  SelectSmem& sm = bk.sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    incl[i] = wave_incl_sum(c[i]);
    if (lane == 63) sm.ecnt[i * kWaves + wave] = incl[i];
  }
  __syncthreads();
  // exclusive scan of the N*kWaves wave totals, in (i, wave) order
  const uint32_t v = threadIdx.x < N * kWaves ? sm.ecnt[threadIdx.x] : 0u;
  uint32_t total;
  const uint32_t pre = bk.excl_scan(v, total);
  __syncthreads();
  if (threadIdx.x < N * kWaves) sm.ecnt[threadIdx.x] = pre;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) off[i] = sm.ecnt[i * kWaves + wave] + incl[i] - c[i];
  return total;
}

// ------------------------------------------------------------------ pool + Full Top-K

constexpr int kBitmapBlocks = 1 << 18;   // contexts up to 2M positions rank blocks with an LDS bitmap

// One WG per query.  Keeps the top P blocks by (block max desc, block asc) as the pool
// (positions ascending; all blocks if there are at most P), then takes the Top-K positions of
// the pool by (score desc, position asc), written in ascending order.
// lists/cuts: per-unit five best blocks from the scan (see k_idx_scan), n_units <= 4096 with
// blocks_per_unit blocks each.  blkkey rows are nb_max entries apart.
// pool_pos / pool_len may be null (no pool output).
__global__ __launch_bounds__(kNT) void k_pool_topk(
    const uint64_t* __restrict__ lists, const uint64_t* __restrict__ cuts, int n_units,
    int blocks_per_unit, const uint32_t* __restrict__ blkkey, int nb_max,
    const int32_t* __restrict__ n_visible, int n_max, const float* __restrict__ scores, int P, int K,
    int32_t* __restrict__ pool_pos, int cap_out, int32_t* __restrict__ pool_len,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelectSmem sm;
  __shared__ union {
    uint64_t cand[kCandCap];                  // blocks of re-read units (before the pool is known)
    uint32_t bitmap[kBitmapBlocks / 32];      // selected blocks (afterwards)
  } u1;
  __shared__ uint16_t wpre[kBitmapBlocks / 32];
  __shared__ uint32_t sel[kMaxTopK];         // selected blocks, any order
  __shared__ uint32_t byrank[kMaxTopK];      // selected blocks, ascending
  __shared__ uint16_t satlist[kUnitsPerThread * kNT];
  Block bk{sm};
  const int q = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int nb = (nv + kBlock - 1) / kBlock;
  const uint32_t* keys = blkkey + (size_t)q * nb_max;
  uint64_t* cand = u1.cand;

  const bool all = nb <= P;
  uint32_t nsel = 0;
  if (!all) {
    uint64_t e[kUnitsPerThread][4];
    uint64_t cut[kUnitsPerThread];
    bool sat[kUnitsPerThread];
    uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      const int u = i * kNT + t;
      const bool ok = u < n_units;
      const size_t base = (size_t)q * n_units + (ok ? u : 0);
      const u32x4 a = *(const u32x4*)(lists + base * 4);
      const u32x4 c = *(const u32x4*)(lists + base * 4 + 2);
      cut[i] = ok ? cuts[base] : 0ull;
      e[i][0] = ok ? ((uint64_t)a.y << 32 | a.x) : 0ull;
      e[i][1] = ok ? ((uint64_t)a.w << 32 | a.z) : 0ull;
      e[i][2] = ok ? ((uint64_t)c.y << 32 | c.x) : 0ull;
      e[i][3] = ok ? ((uint64_t)c.w << 32 | c.z) : 0ull;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (e[i][r]) {
          ++nvalid;
          mn = min(mn, (uint32_t)(e[i][r] >> 32));
          mx = max(mx, (uint32_t)(e[i][r] >> 32));
        }
    }
    auto for_each_e = [&](auto f) {
#pragma unroll
      for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) f(e[i][r]);
    };
    uint64_t t0 = 1ull;
    const uint32_t n_listed = bk.sum(nvalid);
    bk.minmax(mn, mx);
    if (n_listed >= (uint32_t)P) t0 = select_kth(for_each_e, (uint32_t)P, key_lo(mn), key_hi(mx), bk, nullptr);
    // units that may hold unlisted blocks >= t0: re-read them (one wave per unit)
    if (t == 0) { sm.nsat = 0; sm.ncand = 0; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      sat[i] = cut[i] != 0ull && cut[i] >= t0;
      if (sat[i]) satlist[atomicAdd(&sm.nsat, 1u)] = (uint16_t)(i * kNT + t);
    }
    __syncthreads();
    const uint32_t nsat = sm.nsat;
    for (uint32_t si = wave; si < nsat; si += kWaves) {
      const int jb = satlist[si] * blocks_per_unit, je = min(nb, jb + blocks_per_unit);
      for (int jj = jb + lane; jj < je; jj += 64) {
        const uint64_t k = rank_key(keys[jj], (uint32_t)jj);
        if (k >= t0) {
          const uint32_t idx = atomicAdd(&sm.ncand, 1u);
          if (idx < (uint32_t)kCandCap) cand[idx] = k;
        }
      }
    }
    __syncthreads();
    const uint32_t ncand = sm.ncand;
    const bool slow = ncand > (uint32_t)kCandCap;
    uint64_t tstar;
    // candidates: listed keys >= t0 of units not re-read, plus the re-read units' blocks >= t0
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (sat[i] || e[i][r] < t0) e[i][r] = 0ull;
    if (nsat == 0) {
      tstar = t0;                    // every block >= t0 is listed
    } else if (!slow) {
      mn = 0xffffffffu;
      mx = 0u;
#pragma unroll
      for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e[i][r]) { mn = min(mn, (uint32_t)(e[i][r] >> 32)); mx = max(mx, (uint32_t)(e[i][r] >> 32)); }
      for (uint32_t i = t; i < ncand; i += kNT) {
        mn = min(mn, (uint32_t)(cand[i] >> 32));
        mx = max(mx, (uint32_t)(cand[i] >> 32));
      }
      bk.minmax(mn, mx);
      auto for_each_c = [&](auto f) {
#pragma unroll
        for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) f(e[i][r]);
        for (uint32_t i = threadIdx.x; i < ncand; i += kNT) f(cand[i]);
      };
      tstar = select_kth(for_each_c, (uint32_t)P, key_lo(mn), key_hi(mx), bk, nullptr);
    } else {
      // many units re-read (heavy ties): select over every block directly
      mn = 0xffffffffu;
      mx = 0u;
      for (int jj = t; jj < nb; jj += kNT) { mn = min(mn, keys[jj]); mx = max(mx, keys[jj]); }
      bk.minmax(mn, mx);
      tstar = select_kth(
          [&](auto f) {
            constexpr int kB = 8;
            for (int base = t; base < nb; base += kNT * kB) {
              uint32_t kk[kB];
#pragma unroll
              for (int u = 0; u < kB; ++u) {
                const int jj = base + u * kNT;
                kk[u] = keys[jj < nb ? jj : 0];
              }
#pragma unroll
              for (int u = 0; u < kB; ++u) {
                const int jj = base + u * kNT;
                if (jj < nb) f(rank_key(kk[u], (uint32_t)jj));
              }
            }
          },
          (uint32_t)P, key_lo(mn), key_hi(mx), bk, cand);
    }
    // the selected blocks, in any order
    if (t == 0) sm.nrank = 0;
    __syncthreads();
    if (!slow) {
#pragma unroll
      for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e[i][r] && e[i][r] >= tstar) sel[atomicAdd(&sm.nrank, 1u)] = rank_key_index(e[i][r]);
      for (uint32_t i = t; i < ncand; i += kNT)
        if (cand[i] >= tstar) sel[atomicAdd(&sm.nrank, 1u)] = rank_key_index(cand[i]);
    } else {
      for (int jj = t; jj < nb; jj += kNT)
        if (rank_key(keys[jj], (uint32_t)jj) >= tstar) sel[atomicAdd(&sm.nrank, 1u)] = (uint32_t)jj;
    }
    __syncthreads();
    nsel = min(sm.nrank, (uint32_t)P);
    // ascending order of the selected blocks
    if (nb <= kBitmapBlocks) {
      const int nw = (nb + 31) >> 5;
      for (int w = t; w < nw; w += kNT) u1.bitmap[w] = 0u;
      __syncthreads();
      for (uint32_t i = t; i < nsel; i += kNT) atomicOr(&u1.bitmap[sel[i] >> 5], 1u << (sel[i] & 31));
      __syncthreads();
      constexpr int kWpt = kBitmapBlocks / 32 / kNT;   // words per thread (8)
      uint32_t wc[kWpt], mine = 0;
#pragma unroll
      for (int i = 0; i < kWpt; ++i) {
        const int w = kWpt * t + i;
        wc[i] = w < nw ? (uint32_t)__popc(u1.bitmap[w]) : 0u;
        mine += wc[i];
      }
      uint32_t tot;
      uint32_t pre = bk.excl_scan(mine, tot);
#pragma unroll
      for (int i = 0; i < kWpt; ++i) {
        const int w = kWpt * t + i;
        if (w < nw) wpre[w] = (uint16_t)pre;
        pre += wc[i];
      }
      __syncthreads();
      for (uint32_t i = t; i < nsel; i += kNT) {
        const uint32_t jj = sel[i];
        const uint32_t rk = wpre[jj >> 5] + (uint32_t)__popc(u1.bitmap[jj >> 5] & ((1u << (jj & 31)) - 1u));
        byrank[rk] = jj;
      }
    } else {
      // bitonic sort of the (padded) selection
      constexpr int kS = kMaxTopK;
      for (int i = t; i < kS; i += kNT) byrank[i] = i < (int)nsel ? sel[i] : 0xffffffffu;
      __syncthreads();
      for (int k2 = 2; k2 <= kS; k2 <<= 1)
        for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
          for (int i = t; i < kS; i += kNT) {
            const int x = i ^ j2;
            if (x > i) {
              const uint32_t a = byrank[i], c = byrank[x];
              const bool up = (i & k2) == 0;
              if ((a > c) == up) { byrank[i] = c; byrank[x] = a; }
            }
          }
          __syncthreads();
        }
    }
    __syncthreads();
  }

  // ---- pool positions: slot s holds block byrank[s / 8], or position s when all blocks are kept
  int total;
  if (all) {
    total = nv;
  } else {
    total = 8 * (int)nsel;
    if (nsel > 0 && (int)byrank[nsel - 1] == nb - 1) total -= kBlock - (nv - kBlock * (nb - 1));
  }
  auto slot_pos = [&](int sl) { return all ? sl : kBlock * (int)byrank[sl >> 3] + (sl & 7); };
  if (pool_pos) {
    int32_t* gp = pool_pos + (size_t)q * cap_out;
    for (int sl = t; sl < cap_out; sl += kNT) gp[sl] = sl < total ? slot_pos(sl) : -1;
  }
  if (pool_len && t == 0) pool_len[q] = total;

  // ---- Top-K of the pool (slot = i*kNT + t)
  const float* sc = scores + (size_t)q * n_max;
  int32_t ps[kTopE];
  float sv[kTopE];
#pragma unroll
  for (int i = 0; i < kTopE; ++i) {
    const int sl = i * kNT + t;
    ps[i] = sl < total ? slot_pos(sl) : -1;
  }
#pragma unroll
  for (int i = 0; i < kTopE; ++i) sv[i] = sc[ps[i] >= 0 ? ps[i] : 0];
  uint64_t key[kTopE];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kTopE; ++i) {
    const uint32_t k32 = score_key(sv[i]);
    key[i] = ps[i] >= 0 ? rank_key(k32, (uint32_t)ps[i]) : 0ull;
    if (ps[i] >= 0) { mn = min(mn, k32); mx = max(mx, k32); }
  }
  uint64_t thr = 1ull;
  if (total > K) {
    bk.minmax(mn, mx);
    auto for_each_k = [&](auto f) {
#pragma unroll
      for (int i = 0; i < kTopE; ++i) f(key[i]);
    };
    thr = select_kth(for_each_k, (uint32_t)K, key_lo(mn), key_hi(mx), bk, nullptr);
  }
  uint32_t c2[kTopE], o2[kTopE];
#pragma unroll
  for (int i = 0; i < kTopE; ++i) c2[i] = key[i] >= thr ? 1u : 0u;
  const uint32_t tot2 = ordered_offsets(c2, o2, bk);
  int32_t* oi = topk_idx + (size_t)q * K;
  float* os = topk_score ? topk_score + (size_t)q * K : nullptr;
#pragma unroll
  for (int i = 0; i < kTopE; ++i) {
    if (c2[i] && o2[i] < (uint32_t)K) {
      oi[o2[i]] = ps[i];
      if (os) os[o2[i]] = key_score((uint32_t)(key[i] >> 32));
    }
  }
  for (int i = (int)min(tot2, (uint32_t)K) + t; i < K; i += kNT) {
    oi[i] = -1;
    if (os) os[i] = 0.f;
  }
}

hipError_t launch_pool_topk(const uint64_t* lists, const uint64_t* cuts, int n_units, int blocks_per_unit,
                            const uint32_t* blkkey, int nb_max, const int32_t* n_visible, int n_max,
                            const float* scores, int P, int K, int32_t* pool_pos, int cap_out,
                            int32_t* pool_len, int32_t* topk_idx, float* topk_score, int Q, hipStream_t s) {
  hipLaunchKernelGGL(k_pool_topk, dim3(Q), dim3(kNT), 0, s, lists, cuts, n_units, blocks_per_unit, blkkey,
                     nb_max, n_visible, n_max, scores, P, K, pool_pos, cap_out, pool_len, topk_idx, topk_score);
  return hipGetLastError();
}

// ------------------------------------------------------------------ Top-K over given pools

// One WG per item (it = l*Q + q).  Candidates: slots [0, len) of the item's query; slot i has
// position cand_pos[i] (ignored if negative or >= n_rows).  by_position: its score is
// scores[q*score_stride + pos], otherwise scores[it*score_stride + slot].  Output: the k best
// positions in slot order (ascending positions for an ascending pool) with their scores,
// -1 / 0 padded.
__global__ __launch_bounds__(kNT) void k_topk(
    const int32_t* __restrict__ cand_pos, const int32_t* __restrict__ cand_len, int cap,
    int64_t n_rows, const float* __restrict__ scores, int64_t score_stride, int by_position,
    int Q, int k, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  __shared__ SelectSmem sm;
  Block bk{sm};
  const int it = blockIdx.x, q = it % Q, t = threadIdx.x;
  int len = cand_len[q];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int32_t* cp = cand_pos + (size_t)q * cap;
  const float* sc = scores + (size_t)(by_position ? q : it) * score_stride;

  int32_t pos[kTopE];
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    const int slot = e * kNT + t;
    pos[e] = cp[slot < len ? slot : 0];
  }
  bool ok[kTopE];
  float s[kTopE];
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    const int slot = e * kNT + t;
    ok[e] = slot < len && pos[e] >= 0 && (int64_t)pos[e] < n_rows;
    s[e] = sc[by_position ? (ok[e] ? pos[e] : 0) : (slot < len ? slot : 0)];
  }
  uint64_t key[kTopE];
  uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    const uint32_t k32 = score_key(s[e]);
    key[e] = ok[e] ? rank_key(k32, (uint32_t)pos[e]) : 0ull;
    nvalid += ok[e] ? 1u : 0u;
    if (ok[e]) { mn = min(mn, k32); mx = max(mx, k32); }
  }
  uint64_t thr = 1ull;
  const uint32_t n_valid = bk.sum(nvalid);
  if (n_valid > (uint32_t)k) {
    bk.minmax(mn, mx);
    auto for_each = [&](auto f) {
#pragma unroll
      for (int e = 0; e < kTopE; ++e) f(key[e]);
    };
    thr = select_kth(for_each, (uint32_t)k, key_lo(mn), key_hi(mx), bk, nullptr);
  }
  uint32_t c[kTopE], off[kTopE];
#pragma unroll
  for (int e = 0; e < kTopE; ++e) c[e] = key[e] >= thr ? 1u : 0u;
  const uint32_t total = ordered_offsets(c, off, bk);
  int32_t* oi = out_idx + (size_t)it * k;
  float* os = out_score ? out_score + (size_t)it * k : nullptr;
#pragma unroll
  for (int e = 0; e < kTopE; ++e) {
    if (c[e] && off[e] < (uint32_t)k) {   // duplicate positions in a caller pool can tie
      oi[off[e]] = pos[e];
      if (os) os[off[e]] = key_score((uint32_t)(key[e] >> 32));
    }
  }
  for (int i = (int)min(total, (uint32_t)k) + t; i < k; i += kNT) {
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
