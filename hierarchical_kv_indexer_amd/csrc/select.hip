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
// While the digit lies in the upper (score) half of the key, a pass works on 32-bit values and
// sends out-of-range keys to spare bins instead of branching.
//
// Pool selection does not revisit every block: the scan leaves, for each unit (one wave's
// contiguous range of blocks), its four best blocks and the fifth best key.  With T0 = the
// P-th best listed key (T0 <= the true P-th best key T*, the listed keys being a subset), a unit
// whose fifth best key is below T0 has no unlisted block that can be selected; only the units
// whose fifth best key reaches T0 are re-read in full.  The P best of the surviving candidates
// are exactly the P best blocks (and when no unit is re-read, T* = T0).
//
// A workgroup is 1024 threads (16 waves on one CU), so every per-thread instruction costs
// about 16 cycles: the code keeps per-key work small.  Element i of thread t is slot i*1024 + t,
// so every load instruction of a wave reads consecutive addresses; output in slot order takes
// in-wave prefixes from ballots and one barrier for the per-wave totals.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

constexpr int kBins = 4096;
constexpr int kNT = kSelectThreads;      // 1024 threads
constexpr int kWaves = kNT / 64;
constexpr int kRankMax = 256;            // bins this small are resolved by direct ranking
constexpr int kCandCap = 4096;           // LDS candidates (re-read units, slow-path compaction)
constexpr int kE = kMaxPool / kNT;       // slots per thread (16): slot i*kNT + t for i < kE
static_assert(kDensePoolBlocks <= kE * kNT, "a dense pool holds every block key in registers");
constexpr int kUnitsPerThread = 4;       // units per thread in the pool kernel (<= 4096 units)
static_assert(kBins == 4 * kNT, "find_bin gives each thread four bins");
static_assert(kNT == 4 * kRankMax, "ranking splits the bin into four quarters");
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

struct __attribute__((aligned(16))) SelectSmem {
  uint32_t hist[kBins + 64];             // all zero between passes; bins kBins.. take strays
  uint64_t rankbuf[kRankMax];
  uint32_t rankpart[3][kRankMax];        // partial ranks from quarters 1..3
  uint32_t eqpart[3][kRankMax];          // partial counts of equal keys from quarters 1..3
  u32x4 wred[2][kWaves];                 // per-wave partials of block reductions
  uint32_t ecnt[2][kE * kWaves];         // per-(element, wave) totals of ordered_offsets
  uint64_t result;
  uint32_t found_bin, found_above, found_cnt, ncand, nrank, nsat;
};

// Clears the histogram and counters; the kernel's first barrier publishes it.
__device__ __forceinline__ void smem_init(SelectSmem& sm) {
  *(u32x4*)&sm.hist[4 * threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x == 0) { sm.nrank = 0; sm.ncand = 0; sm.nsat = 0; }
}

// Block-wide collectives with one barrier each.  Their LDS buffers alternate, so a buffer is
// rewritten only after the next collective's barrier.
struct Block {
  SelectSmem& sm;
  int parity = 0;

  // Exclusive prefix sum in thread order; also returns the total.
  __device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_sum(v);
    if (lane == 63) sm.wred[parity][wave].x = inc;
    lds_barrier();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t s = sm.wred[parity][w].x;
      before += w < wave ? s : 0u;
      tot += s;
    }
    parity ^= 1;
    total = tot;
    return before + inc - v;
  }
  // Block sum of cnt, min of mn and max of mx.
  __device__ __forceinline__ void reduce(uint32_t& cnt, uint32_t& mn, uint32_t& mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    cnt = wave_sum_u32(cnt);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) sm.wred[parity][wave] = u32x4{cnt, mn, mx, 0u};
    lds_barrier();
    cnt = 0u;
    mn = 0xffffffffu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const u32x4 r = sm.wred[parity][w];
      cnt += r.x;
      mn = min(mn, r.y);
      mx = max(mx, r.z);
    }
    parity ^= 1;
  }
};

// Offsets that keep slot order (slot = i*kNT + t): off[i] = the sum of the counts c of every
// earlier slot; returns the total.  Each element's in-wave prefix comes from a ballot (counts
// 0/1, FLAGS) or a DPP scan (any counts); one barrier exchanges the per-(element, wave) totals,
// and lane i of each wave then prefixes element i over the waves.  N <= kE.
template <bool FLAGS, int N>
__device__ __forceinline__ uint32_t ordered_offsets(const uint32_t (&c)[N], uint32_t (&off)[N], Block& bk) {
  SelectSmem& sm = bk.sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* ec = sm.ecnt[bk.parity];
  bk.parity ^= 1;
  uint32_t pre[N], mine = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (FLAGS) {
      const uint64_t m = __ballot(c[i] != 0u);
      pre[i] = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (lane == i) mine = (uint32_t)__popcll(m);
    } else {
      const uint32_t inc = wave_incl_sum(c[i]);
      pre[i] = inc - c[i];
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      if (lane == i) mine = tot;
    }
  }
  if (lane < N) ec[lane * kWaves + wave] = mine;
  lds_barrier();
  uint32_t tot_i = 0u, pre_w = 0u;
  if (lane < N) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t v = ec[lane * kWaves + w];
      tot_i += v;
      pre_w += w < wave ? v : 0u;
    }
  }
  const uint32_t inc_t = wave_incl_sum(tot_i);
  const uint32_t base = inc_t - tot_i + pre_w;
#pragma unroll
  for (int i = 0; i < N; ++i) off[i] = (uint32_t)__builtin_amdgcn_readlane((int)base, i) + pre[i];
  return (uint32_t)__builtin_amdgcn_readlane((int)inc_t, N - 1);
}

// Find b with above(b) < need <= above(b) + hist[b] (above(b): keys in bins > b) and clear the
// histogram.  Thread t owns bins 4t .. 4t+3.
__device__ __forceinline__ void find_bin(uint32_t need, Block& bk) {
  SelectSmem& sm = bk.sm;
  const int t = threadIdx.x;
  u32x4* hp = (u32x4*)&sm.hist[4 * t];
  const u32x4 h = *hp;
  *hp = u32x4{0u, 0u, 0u, 0u};
  const uint32_t mine = h.x + h.y + h.z + h.w;
  uint32_t total;
  const uint32_t below = bk.excl_scan(mine, total);
  uint32_t above = total - below - mine;
  if (above < need && need <= above + mine) {
    const uint32_t hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (above < need && need <= above + hv[i]) {
        sm.found_bin = 4 * t + i;
        sm.found_above = above;
        sm.found_cnt = hv[i];
      }
      above += hv[i];
    }
    sm.nrank = 0u;
  }
  lds_barrier();
}

// Bounds [lo, hi] on ranking keys whose score keys lie in [mn32, mx32].
__device__ __forceinline__ uint64_t key_lo(uint32_t mn32) { return (uint64_t)mn32 << 32; }
__device__ __forceinline__ uint64_t key_hi(uint32_t mx32) { return ((uint64_t)mx32 << 32) | 0xffffffffull; }

// The need-th largest of the cnt keys in sm.rankbuf (1 <= need <= cnt <= kRankMax), collected
// before the caller's barrier: thread t compares key t % 256 with one quarter of the keys (the
// quarter is the same for a whole wave, so every LDS read is a broadcast).
__device__ __forceinline__ uint64_t rank_collected(uint32_t cnt, uint32_t need, Block& bk) {
  SelectSmem& sm = bk.sm;
  constexpr uint32_t kPart = kRankMax / 4;
  const uint32_t i = threadIdx.x % kRankMax, part = threadIdx.x / kRankMax;
  const uint64_t x = sm.rankbuf[i];
  const uint32_t m0 = part * kPart, m1 = min(cnt, m0 + kPart);
  uint32_t r = 0, eq = 0, m = m0;
  for (; m + 2 <= m1; m += 2) {
    const u64x2 v = *(const u64x2*)(sm.rankbuf + m);
    r += (v.x > x ? 1u : 0u) + (v.y > x ? 1u : 0u);
    eq += (v.x == x ? 1u : 0u) + (v.y == x ? 1u : 0u);
  }
  if (m < m1) {
    r += sm.rankbuf[m] > x ? 1u : 0u;
    eq += sm.rankbuf[m] == x ? 1u : 0u;
  }
  if (part) {
    sm.rankpart[part - 1][i] = r;
    sm.eqpart[part - 1][i] = eq;
  }
  lds_barrier();
  if (part == 0 && i < cnt) {
    r += sm.rankpart[0][i] + sm.rankpart[1][i] + sm.rankpart[2][i];
    eq += sm.eqpart[0][i] + sm.eqpart[1][i] + sm.eqpart[2][i];
    // fewer than need keys above x, at least need at or above it (every copy of x agrees)
    if (r < need && need <= r + eq) sm.result = x;
  }
  lds_barrier();
  return sm.result;
}

// The first pass of a selection, kept for a later one over a related set (see k_pool).
struct FirstPass {
  uint64_t lo, hi;
  int shift;
  bool wide;
  uint32_t bin, above;                   // the bin that held the result, keys in bins above it
  bool valid;
};

// Bin of key k (lo <= k <= hi) in that pass; a key outside the range would go to a spare bin.
__device__ __forceinline__ uint32_t first_pass_bin(const FirstPass& fp, uint64_t k) {
  const uint64_t b = fp.wide ? (uint64_t)(((uint32_t)(k >> 32) - (uint32_t)(fp.lo >> 32)) >> (fp.shift - 32))
                             : (k - fp.lo) >> fp.shift;
  return k >= fp.lo && k <= fp.hi && b < (uint64_t)kBins ? (uint32_t)b : (uint32_t)kBins + (threadIdx.x & 63);
}

// The need-th largest of a set of 64-bit keys, counted with repeats, all inside [lo, hi]
// (1 <= need <= the number of keys).  Keys are distinct except when a caller's pool lists a
// position more than once.  for_each(f) calls f(key) for every key this thread holds (0 = none; keys
// outside [lo, hi] are ignored).  If `cand` is non-null, the keys of a bin with at most
// kCandCap keys are copied there once and later passes read only the copy.  If `save` is
// non-null, the first pass's histogram (kBins counts) is copied there and its range, digit and
// outcome into *fp (fp->valid is false if no pass ran).
// Requires a clear histogram (smem_init); leaves it clear.
template <class ForEach>
__device__ uint64_t select_kth(ForEach for_each, uint32_t need, uint64_t lo, uint64_t hi, Block& bk,
                               uint64_t* cand, uint32_t* save = nullptr, FirstPass* fp = nullptr) {
  SelectSmem& sm = bk.sm;
  bool use_cand = false, first = true;
  if (fp) fp->valid = false;
  if (lo == 0ull) lo = 1ull;             // 0 marks "no key"
  const uint32_t stray = (uint32_t)kBins + (threadIdx.x & 63);
  while (true) {
    if (lo >= hi) return lo;
    const int shift = max(0, bitlen64(hi - lo) - 12);
    // With the digit in the upper half and lo's lower half zero (hi's is then all ones), a key
    // is in range iff its upper half is: one 32-bit subtract and compare per key.
    const bool wide = shift >= 32 && (uint32_t)lo == 0u && !use_cand;
    if (wide) {
      const uint32_t lo32 = (uint32_t)(lo >> 32), span = (uint32_t)((hi - lo) >> 32);
      const uint32_t sh = (uint32_t)(shift - 32);
      for_each([&](uint64_t k) {
        const uint32_t d = (uint32_t)(k >> 32) - lo32;
        atomicAdd(&sm.hist[d <= span ? (d >> sh) : stray], 1u);
      });
    } else {
      auto count = [&](uint64_t k) {
        if (k >= lo && k <= hi) atomicAdd(&sm.hist[(uint32_t)((k - lo) >> shift)], 1u);
      };
      if (use_cand) {
        const uint32_t n = sm.ncand;
        for (uint32_t i = threadIdx.x; i < n; i += kNT) count(cand[i]);
      } else {
        for_each(count);
      }
    }
    lds_barrier();
    if (save && first) *(u32x4*)&save[4 * threadIdx.x] = *(const u32x4*)&sm.hist[4 * threadIdx.x];
    find_bin(need, bk);
    const uint32_t bin = sm.found_bin, above = sm.found_above, cnt = sm.found_cnt;
    if (fp && first) *fp = FirstPass{lo, hi, shift, wide, bin, above, true};
    first = false;
    need -= above;
    const uint64_t nlo = lo + ((uint64_t)bin << shift);
    const uint64_t nhi = shift == 0 ? nlo : min(hi, nlo + (((uint64_t)1 << shift) - 1));
    lo = nlo;
    hi = nhi;
    if (shift == 0) return lo;
    if (cnt <= (uint32_t)kRankMax) {
      // rank the few keys of the bin directly: thread t compares key t % 256 with one quarter of
      // the bin (the quarter is the same for a whole wave, so every LDS read is a broadcast)
      if (wide) {
        const uint32_t lo32 = (uint32_t)(lo >> 32), span = (uint32_t)((hi - lo) >> 32);
        for_each([&](uint64_t k) {
          if ((uint32_t)(k >> 32) - lo32 <= span) sm.rankbuf[atomicAdd(&sm.nrank, 1u)] = k;
        });
      } else {
        auto collect = [&](uint64_t k) {
          if (k >= lo && k <= hi) sm.rankbuf[atomicAdd(&sm.nrank, 1u)] = k;
        };
        if (use_cand) {
          const uint32_t n = sm.ncand;
          for (uint32_t i = threadIdx.x; i < n; i += kNT) collect(cand[i]);
        } else {
          for_each(collect);
        }
      }
      lds_barrier();
      return rank_collected(cnt, need, bk);
    }
    if (cand && !use_cand && cnt <= (uint32_t)kCandCap) {
      if (threadIdx.x == 0) sm.ncand = 0;
      lds_barrier();
      for_each([&](uint64_t k) {
        if (k >= lo && k <= hi) cand[atomicAdd(&sm.ncand, 1u)] = k;
      });
      use_cand = true;
      lds_barrier();
    }
  }
}

// Top-K of a slot array (slot = e*kNT + t, keys 0 = none): the k best keys written in slot
// order as indices (and scores), -1 / 0 padded.
__device__ __forceinline__ void topk_out(const uint64_t (&key)[kE], uint32_t nvalid, uint32_t mn, uint32_t mx,
                                         int k, int32_t* __restrict__ oi, float* __restrict__ os, Block& bk) {
  bk.reduce(nvalid, mn, mx);
  uint64_t thr = 1ull;
  if (nvalid > (uint32_t)k) {
    auto for_each = [&](auto f) {
#pragma unroll
      for (int e = 0; e < kE; ++e) f(key[e]);
    };
    thr = select_kth(for_each, (uint32_t)k, key_lo(mn), key_hi(mx), bk, nullptr);
  }
  uint32_t c[kE], off[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) c[e] = key[e] >= thr ? 1u : 0u;
  uint32_t total = ordered_offsets<true>(c, off, bk);
  if (total > (uint32_t)k) {
    // a position listed more than once ties with itself at the threshold: every key above thr
    // stays, and copies of thr fill the remaining places in slot order
    uint32_t g[kE], goff[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) g[e] = key[e] == thr ? 1u : 0u;
    const uint32_t n_eq = ordered_offsets<true>(g, goff, bk);
    const uint32_t room = (uint32_t)k - (total - n_eq);
#pragma unroll
    for (int e = 0; e < kE; ++e) c[e] = (key[e] > thr || (g[e] && goff[e] < room)) ? 1u : 0u;
    total = ordered_offsets<true>(c, off, bk);
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    if (c[e] && off[e] < (uint32_t)k) {
      oi[off[e]] = (int32_t)rank_key_index(key[e]);
      if (os) os[off[e]] = key_score((uint32_t)(key[e] >> 32));
    }
  }
  for (int i = (int)min(total, (uint32_t)k) + (int)threadIdx.x; i < k; i += kNT) {
    oi[i] = -1;
    if (os) os[i] = 0.f;
  }
}

// ------------------------------------------------------------------ pool + Full Top-K

// Sort four block indices ascending (0xffffffff = none sorts last).
__device__ __forceinline__ void sort4(uint32_t (&v)[4]) {
  auto cx = [&](int a, int b) {
    const uint32_t x = min(v[a], v[b]), y = max(v[a], v[b]);
    v[a] = x;
    v[b] = y;
  };
  cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
}

// The pool's output, shared by both pool kernels: slot s holds block byrank[s / 8] (position s
// when all blocks are kept, `all`), ascending, -1 padded to cap_out; pool_len the count.  With
// K > 0 it goes on to the Top-K positions of the pool by (score desc, position asc) from the scan's
// scores of this query, written in slot (= position) order.
__device__ __forceinline__ void pool_out(bool all, int nv, int nb, uint32_t nsel, const uint32_t* byrank,
                                         int32_t* __restrict__ gp, int cap_out, int32_t* __restrict__ len_out,
                                         const float* __restrict__ sc, int K, int32_t* __restrict__ oi,
                                         float* __restrict__ os, Block& bk) {
  const int t = threadIdx.x;
  int total;
  if (all) {
    total = nv;
  } else {
    total = 8 * (int)nsel;
    if (nsel > 0 && (int)byrank[nsel - 1] == nb - 1) total -= kBlock - (nv - kBlock * (nb - 1));
  }
  int32_t ps[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int sl = i * kNT + t;
    ps[i] = sl < total ? (all ? sl : kBlock * (int)byrank[sl >> 3] + (sl & 7)) : -1;
  }
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int sl = i * kNT + t;
    if (sl < cap_out) gp[sl] = ps[i];
  }
  if (t == 0) *len_out = total;
  if (K == 0) return;
  float sv[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) sv[i] = sc[ps[i] >= 0 ? ps[i] : 0];
  uint64_t key[kE];
  uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const uint32_t k32 = score_key(sv[i]);
    key[i] = ps[i] >= 0 ? rank_key(k32, (uint32_t)ps[i]) : 0ull;
    nvalid += ps[i] >= 0 ? 1u : 0u;
    if (ps[i] >= 0) { mn = min(mn, k32); mx = max(mx, k32); }
  }
  topk_out(key, nvalid, mn, mx, K, oi, os, bk);
}

// One WG per query: keeps the top P blocks by (block max desc, block asc) as the pool, written
// as positions in ascending order (all blocks if there are at most P), -1 padded to cap_out
// (a multiple of 8).  With K > 0 it goes on to the Top-K positions of the pool by (score desc,
// position asc), written in ascending order (-1 padded), from the pool it holds.
// lists/cuts: per-unit five best blocks from the scan (see k_idx_scan); unit u covers blocks
// [u*bpu, (u+1)*bpu), n_units <= 4096.  blkkey rows are nb_max entries apart.
//
// Pool order: thread t owns units i*kNT + t (i < 4).  Once the P-th best block key T* is known,
// the selected blocks of a unit that was not re-read are its listed keys >= T*, sorted by index;
// a re-read unit is counted and written by one wave, in index order, with ballots.  Unit order
// is block order, so ordered_offsets over the units' counts places every unit.
__global__ __launch_bounds__(kNT) void k_pool(
    const uint64_t* __restrict__ lists, const uint64_t* __restrict__ cuts, int n_units,
    int bpu, const uint32_t* __restrict__ blkkey, int nb_max,
    const int32_t* __restrict__ n_visible, int n_max, int P,
    int32_t* __restrict__ pool_pos, int cap_out, int32_t* __restrict__ pool_len,
    const float* __restrict__ scores, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelectSmem sm;
  __shared__ uint64_t cand[kCandCap];        // re-read units, bpu keys each (0 = below T0)
  __shared__ uint32_t byrank[kMaxTopK];      // selected blocks, ascending
  __shared__ uint16_t satunit[kUnitsPerThread * kNT];   // unit of each re-read slot
  __shared__ uint32_t satcnt[kUnitsPerThread * kNT];    // its count, then its output offset
  __shared__ uint32_t hsave[kBins];          // T0's first histogram pass
  Block bk{sm};
  const int q = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int nb = (nv + kBlock - 1) / kBlock;
  const uint32_t* keys = blkkey + (size_t)q * nb_max;
  smem_init(sm);

  const bool all = nb <= P;
  uint32_t nsel = 0;
  if (!all) {
    uint64_t e[kUnitsPerThread][4];
    uint64_t cut[kUnitsPerThread];
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
    bk.reduce(nvalid, mn, mx);
    uint64_t t0 = 1ull;                       // T0 <= T*: the P-th best listed key
    FirstPass fp;
    fp.valid = false;
    if (nvalid >= (uint32_t)P)
      t0 = select_kth(for_each_e, (uint32_t)P, key_lo(mn), key_hi(mx), bk, nullptr, hsave, &fp);

    // The candidates for T* are the blocks >= T0; all lie in T0's first-pass range (a unit's
    // unlisted blocks are below its listed ones).  Their histogram over that pass's bins is the
    // saved one with: bins below T0's bin empty; T0's bin holding the listed keys >= T0, of which
    // there are P - (keys in bins above); re-read units' listed keys >= T0 taken out and their
    // blocks >= T0 put in.  Restored here into the (clear) histogram, and cleared again below if
    // no unit is re-read or the re-read keys do not fit in LDS.
    if (fp.valid) {
      const uint32_t b0 = 4u * (uint32_t)t;
      u32x4 h = *(const u32x4*)&hsave[b0];
      h.x = b0 + 0 < fp.bin ? 0u : (b0 + 0 == fp.bin ? (uint32_t)P - fp.above : h.x);
      h.y = b0 + 1 < fp.bin ? 0u : (b0 + 1 == fp.bin ? (uint32_t)P - fp.above : h.y);
      h.z = b0 + 2 < fp.bin ? 0u : (b0 + 2 == fp.bin ? (uint32_t)P - fp.above : h.z);
      h.w = b0 + 3 < fp.bin ? 0u : (b0 + 3 == fp.bin ? (uint32_t)P - fp.above : h.w);
      *(u32x4*)&sm.hist[b0] = h;
    }

    // units that may hold unlisted blocks >= T0 are re-read; sidx = their slot
    int sidx[kUnitsPerThread];
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      const bool sat = cut[i] != 0ull && cut[i] >= t0;
      sidx[i] = sat ? (int)atomicAdd(&sm.nsat, 1u) : -1;
      if (sat) satunit[sidx[i]] = (uint16_t)(i * kNT + t);
    }
    lds_barrier();
    const uint32_t nsat = sm.nsat;
    const bool dense = nsat * (uint32_t)bpu <= (uint32_t)kCandCap;   // re-read keys fit in LDS
    const bool from_first = fp.valid && nsat > 0 && dense;
    if (fp.valid && !from_first) *(u32x4*)&sm.hist[4 * t] = u32x4{0u, 0u, 0u, 0u};
    auto unit_key = [&](uint32_t si, int o) -> uint64_t {   // key of block o of re-read slot si
      const int jj = satunit[si] * bpu + o;
      return jj < nb ? rank_key(keys[jj], (uint32_t)jj) : 0ull;
    };
    if (dense) {
      for (uint32_t si = wave; si < nsat; si += kWaves)
        for (int o = lane; o < bpu; o += 64) {
          const uint64_t k = unit_key(si, o);
          cand[si * bpu + o] = k >= t0 ? k : 0ull;
          if (from_first && k >= t0) atomicAdd(&sm.hist[first_pass_bin(fp, k)], 1u);
        }
    }
    auto sat_key = [&](uint32_t si, int o) -> uint64_t {
      return dense ? cand[si * bpu + o] : unit_key(si, o);
    };
    // listed keys that stay candidates: >= T0, in units that were not re-read
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (from_first && sidx[i] >= 0 && e[i][r] >= t0) atomicSub(&sm.hist[first_pass_bin(fp, e[i][r])], 1u);
        if (sidx[i] >= 0 || e[i][r] < t0) e[i][r] = 0ull;
      }
    lds_barrier();

    uint64_t tstar = t0;                      // no unit re-read: every block >= T0 is listed
    if (nsat > 0) {
      uint32_t dummy = 0;
      mn = 0xffffffffu;
      mx = 0u;
      if (dense) {
        const uint32_t nc = nsat * (uint32_t)bpu;
        auto for_each_c = [&](auto f) {
#pragma unroll
          for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) f(e[i][r]);
          for (uint32_t i = threadIdx.x; i < nc; i += kNT) f(cand[i]);
        };
        if (from_first) {
          // the candidates' histogram is in place: find T*'s bin, then rank it or narrow it
          find_bin((uint32_t)P, bk);
          const uint32_t above = sm.found_above, cnt = sm.found_cnt;
          const uint64_t blo = fp.lo + ((uint64_t)sm.found_bin << fp.shift);
          const uint64_t bhi = fp.shift == 0 ? blo : min(fp.hi, blo + (((uint64_t)1 << fp.shift) - 1));
          if (fp.shift == 0) {
            tstar = blo;
          } else if (cnt <= (uint32_t)kRankMax) {
            for_each_c([&](uint64_t k) {
              if (k >= blo && k <= bhi) {
                const uint32_t a = atomicAdd(&sm.nrank, 1u);
                if (a < (uint32_t)kRankMax) sm.rankbuf[a] = k;
              }
            });
            lds_barrier();
            tstar = rank_collected(cnt, (uint32_t)P - above, bk);
          } else {
            tstar = select_kth(for_each_c, (uint32_t)P - above, blo, bhi, bk, nullptr);
          }
        } else {
#pragma unroll
          for (int i = 0; i < kUnitsPerThread; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (e[i][r]) { mn = min(mn, (uint32_t)(e[i][r] >> 32)); mx = max(mx, (uint32_t)(e[i][r] >> 32)); }
          for (uint32_t i = t; i < nc; i += kNT)
            if (cand[i]) { mn = min(mn, (uint32_t)(cand[i] >> 32)); mx = max(mx, (uint32_t)(cand[i] >> 32)); }
          bk.reduce(dummy, mn, mx);
          tstar = select_kth(for_each_c, (uint32_t)P, key_lo(mn), key_hi(mx), bk, nullptr);
        }
      } else {
        // many units re-read (heavy ties): select over every block directly
        for (int jj = t; jj < nb; jj += kNT) { mn = min(mn, keys[jj]); mx = max(mx, keys[jj]); }
        bk.reduce(dummy, mn, mx);
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
    }

    // selected blocks of each re-read unit, counted by one wave
    for (uint32_t si = wave; si < nsat; si += kWaves) {
      uint32_t c = 0;
      for (int o0 = 0; o0 < bpu; o0 += 64) {
        const int o = o0 + lane;
        c += (uint32_t)__popcll(__ballot(o < bpu && sat_key(si, o) >= tstar));
      }
      if (lane == 0) satcnt[si] = c;
    }
    lds_barrier();
    uint32_t lb[kUnitsPerThread][4], cnt[kUnitsPerThread], off[kUnitsPerThread];
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      cnt[i] = 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) lb[i][r] = 0xffffffffu;
      if (sidx[i] < 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e[i][r] >= tstar) { lb[i][r] = rank_key_index(e[i][r]); ++cnt[i]; }
        sort4(lb[i]);
      } else {
        cnt[i] = satcnt[sidx[i]];
      }
    }
    nsel = min(ordered_offsets<false>(cnt, off, bk), (uint32_t)P);
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
      if (sidx[i] < 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((uint32_t)r < cnt[i] && off[i] + r < (uint32_t)P) byrank[off[i] + r] = lb[i][r];
      } else {
        satcnt[sidx[i]] = off[i];
      }
    }
    lds_barrier();
    for (uint32_t si = wave; si < nsat; si += kWaves) {
      uint32_t n = satcnt[si];
      const int jb = satunit[si] * bpu;
      for (int o0 = 0; o0 < bpu; o0 += 64) {
        const int o = o0 + lane;
        const bool sel = o < bpu && sat_key(si, o) >= tstar;
        const uint64_t m = __ballot(sel);
        const uint32_t at = n + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
        if (sel && at < (uint32_t)P) byrank[at] = (uint32_t)(jb + o);
        n += (uint32_t)__popcll(m);
      }
    }
    lds_barrier();
  }

  pool_out(all, nv, nb, nsel, byrank, pool_pos + (size_t)q * cap_out, cap_out, pool_len + q,
           scores + (size_t)q * n_max, K, topk_idx + (size_t)q * K, topk_score ? topk_score + (size_t)q * K : nullptr,
           bk);
}

// ------------------------------------------------------------------ list selection, 512 threads
//
// The pool's selection from the scan's chunk lists takes few block-wide steps, and each step of a
// workgroup costs about the same however little data it touches, so it runs 512 threads (two
// waves per SIMD): measured on this part, a scan step with a barrier takes ~0.33 us at 512
// threads against ~0.60 us at 1024.
//
// Lists: group g (a chunk of the scan) lists its best keys in member
// order, and its cut bounds every member it does not list.  Let T0' be the lower edge of the
// first-pass histogram bin that holds the P-th best listed key: T0' <= T0 <= T*, where T0 is that
// key and T* the true P-th best of all members.  A group whose cut is below T0' has no unlisted
// member that can be selected; the groups whose cut reaches T0' are re-read.  T*'s histogram is
// the first pass's (left uncleared: bins below T0's bin only add to the counts below it) with the
// re-read groups' listed keys taken out and all their members >= T0' put in.
namespace ls {

constexpr int NT = 512;
constexpr int W = NT / 64;
constexpr int BINS = 4096;
constexpr int BPT = BINS / NT;              // bins per thread (8)
constexpr int RANK_MAX = 64;                // bins this small are ranked by one wave
constexpr int MAX_SAT = 128;                // re-read groups
constexpr int MAX_GROUPS = NT;              // group t's cut is held by thread t
static_assert(BPT == 8, "find_bin reads two 16-byte bin quads per thread");

struct __attribute__((aligned(16))) Smem {
  uint32_t hist[BINS + 64];                 // bins BINS.. take out-of-range keys and are never read
  u32x4 wred[2][W];
  uint32_t ecnt[2][64 * W];                 // ordered(): per-(element, wave) totals; rank_small: partials
  uint64_t rk[RANK_MAX];
  uint16_t satgroup[MAX_SAT];               // re-read slot -> group
  uint32_t gstart[MAX_SAT + 1];             // selected members of re-read slots before this one
  uint32_t satoff[MAX_SAT];                 // output offset of a re-read group
  uint16_t satof[MAX_GROUPS];               // group -> 1 + its re-read slot (0: not re-read)
  uint64_t result;
  uint32_t bin, above, cnt, nrk, nsat;
};

__device__ __forceinline__ void init(Smem& sm) {
  for (int i = threadIdx.x; i < BINS / 4; i += NT) *(u32x4*)&sm.hist[4 * i] = u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x == 0) { sm.nsat = 0; sm.nrk = 0; }
}

struct Blk {
  Smem& sm;
  int parity = 0;
  __device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_sum(v);
    if (lane == 63) sm.wred[parity][wave].x = inc;
    lds_barrier();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t s = sm.wred[parity][w].x;
      before += w < wave ? s : 0u;
      tot += s;
    }
    parity ^= 1;
    total = tot;
    return before + inc - v;
  }
  __device__ __forceinline__ void reduce(uint32_t& cnt, uint32_t& mn, uint32_t& mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    cnt = wave_sum_u32(cnt);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) sm.wred[parity][wave] = u32x4{cnt, mn, mx, 0u};
    lds_barrier();
    cnt = 0u;
    mn = 0xffffffffu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const u32x4 r = sm.wred[parity][w];
      cnt += r.x;
      mn = min(mn, r.y);
      mx = max(mx, r.z);
    }
    parity ^= 1;
  }
};

// Offsets in element-major order (element i of thread t is item i*NT + t), as ordered_offsets.
template <bool FLAGS, int N>
__device__ __forceinline__ uint32_t ordered(const uint32_t (&c)[N], uint32_t (&off)[N], Blk& bk) {
  static_assert(N <= 16, "per-(element, wave) totals hold 16 elements");
  Smem& sm = bk.sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* ec = sm.ecnt[bk.parity];
  bk.parity ^= 1;
  uint32_t pre[N], mine = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (FLAGS) {
      const uint64_t m = __ballot(c[i] != 0u);
      pre[i] = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (lane == i) mine = (uint32_t)__popcll(m);
    } else {
      const uint32_t inc = wave_incl_sum(c[i]);
      pre[i] = inc - c[i];
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      if (lane == i) mine = tot;
    }
  }
  if (lane < N) ec[lane * W + wave] = mine;
  lds_barrier();
  uint32_t tot_i = 0u, pre_w = 0u;
  if (lane < N) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t v = ec[lane * W + w];
      tot_i += v;
      pre_w += w < wave ? v : 0u;
    }
  }
  const uint32_t inc_t = wave_incl_sum(tot_i);
  const uint32_t base = inc_t - tot_i + pre_w;
#pragma unroll
  for (int i = 0; i < N; ++i) off[i] = (uint32_t)__builtin_amdgcn_readlane((int)base, i) + pre[i];
  return (uint32_t)__builtin_amdgcn_readlane((int)inc_t, N - 1);
}

// The bin b with above(b) < need <= above(b) + hist[b] (above(b): counts of bins > b) into sm.bin,
// sm.above, sm.cnt; with `clear` the histogram is cleared as it is read.  Thread t owns bins
// 8t .. 8t+7.  need >= 1 and at most the histogram's total.
__device__ __forceinline__ void find_bin(uint32_t need, bool clear, Blk& bk) {
  Smem& sm = bk.sm;
  const int t = threadIdx.x;
  u32x4* hp = (u32x4*)&sm.hist[BPT * t];
  const u32x4 h0 = hp[0], h1 = hp[1];
  if (clear) hp[0] = hp[1] = u32x4{0u, 0u, 0u, 0u};
  const uint32_t hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mine += hv[i];
  uint32_t total;
  const uint32_t below = bk.excl_scan(mine, total);
  uint32_t above = total - below - mine;
  if (above < need && need <= above + mine) {
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < need && need <= above + hv[i]) {
        sm.bin = BPT * t + i;
        sm.above = above;
        sm.cnt = hv[i];
      }
      above += hv[i];
    }
    sm.nrk = 0u;
  }
  lds_barrier();
}

// Histogram binning of one pass: keys in [lo, hi] into BINS bins of width 2^shift; while the
// digit lies in the score half of the key (wide), on the upper 32 bits only.
struct Pass {
  uint64_t lo, hi;
  int shift;
  bool wide;
  __device__ __forceinline__ void make(uint64_t l, uint64_t h) {
    lo = l;
    hi = h;
    shift = max(0, bitlen64(hi - lo) - 12);
    wide = shift >= 32 && (uint32_t)lo == 0u;
  }
  // bin of k, or BINS + lane when k lies outside [lo, hi]
  __device__ __forceinline__ uint32_t bin(uint64_t k) const {
    const uint32_t stray = (uint32_t)BINS + (threadIdx.x & 63);
    if (wide) {
      const uint32_t d = (uint32_t)(k >> 32) - (uint32_t)(lo >> 32), span = (uint32_t)((hi - lo) >> 32);
      return d <= span ? (d >> (shift - 32)) : stray;
    }
    return (k >= lo && k <= hi) ? (uint32_t)((k - lo) >> shift) : stray;
  }
  __device__ __forceinline__ uint64_t bin_lo(uint32_t b) const { return lo + ((uint64_t)b << shift); }
  __device__ __forceinline__ uint64_t bin_hi(uint32_t b) const {
    return shift == 0 ? bin_lo(b) : min(hi, bin_lo(b) + (((uint64_t)1 << shift) - 1));
  }
};

// The need-th largest key held in sm.rk (n <= RANK_MAX, counted with repeats): thread t compares
// key t % 64 with keys 8w .. 8w+7 (w = t / 64; the eight keys are the same for a whole wave, so
// the reads broadcast), and wave 0 adds the eight partial counts.
__device__ __forceinline__ uint64_t rank_small(uint32_t n, uint32_t need, Blk& bk) {
  Smem& sm = bk.sm;
  static_assert(RANK_MAX == 8 * W, "eight keys per wave");
  const int t = threadIdx.x, i = t & 63, w = t >> 6;
  const uint64_t x = i < (int)n ? sm.rk[i] : 0ull;
  uint32_t r = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = 8 * w + j;
    const uint64_t y = sm.rk[m];
    r += (m < (int)n && y > x) ? 1u : 0u;
    eq += (m < (int)n && y == x) ? 1u : 0u;
  }
  sm.ecnt[bk.parity][w * 64 + i] = r | (eq << 16);
  lds_barrier();
  if (t < 64) {
    uint32_t rt = 0, et = 0;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const uint32_t v = sm.ecnt[bk.parity][ww * 64 + t];
      rt += v & 0xffffu;
      et += v >> 16;
    }
    if (t < (int)n && rt < need && need <= rt + et) sm.result = x;
  }
  bk.parity ^= 1;
  lds_barrier();
  return sm.result;
}

// The need-th largest of a set of keys (counted with repeats) inside [lo, hi]; for_each(f) calls
// f(key) for every key this thread holds (0 and keys outside the range are ignored).  Requires
// a clear histogram; leaves it clear.
template <class ForEach>
__device__ uint64_t select_kth(ForEach for_each, uint32_t need, uint64_t lo, uint64_t hi, Blk& bk) {
  Smem& sm = bk.sm;
  if (lo == 0ull) lo = 1ull;
  while (true) {
    if (lo >= hi) return lo;
    Pass ps;
    ps.make(lo, hi);
    for_each([&](uint64_t k) { atomicAdd(&sm.hist[ps.bin(k)], 1u); });
    lds_barrier();
    find_bin(need, true, bk);
    const uint32_t b = sm.bin, cnt = sm.cnt;
    need -= sm.above;
    lo = ps.bin_lo(b);
    hi = ps.bin_hi(b);
    if (ps.shift == 0) return lo;
    if (cnt <= (uint32_t)RANK_MAX) {
      for_each([&](uint64_t k) {
        if (k >= lo && k <= hi) sm.rk[atomicAdd(&sm.nrk, 1u)] = k;
      });
      lds_barrier();
      return rank_small(cnt, need, bk);
    }
  }
}

// One list selection (see the section comment).  key[e]: element e of this thread, list entry
// g = e*NT + t of group g / L (0 = none); cut: the cut of group t (t < n_groups, else 0); gsize (a
// power of two): members per group.  reread(grp, o) -> key of member o < gsize of group grp (0 =
// none); emit(off, key, grp, o) writes output place `off` (o = -1 for a listed entry).  Entries of
// a group and members are in output order; groups follow each other.  The members of re-read
// groups are held in registers, MPT per thread (member o of re-read slot s is item s*gsize + o,
// item i*NT + t in thread t's element i).  Returns the number emitted (<= P), or -1 (nothing
// emitted) when more than MPT*NT members or MAX_SAT groups would be re-read, or when copies of
// one key straddle the P-th place: the caller then selects densely.
template <int L, int LPT, int MPT, class Reread, class Emit>
__device__ int list_select(uint64_t (&key)[LPT], uint64_t cut, int n_groups, int gsize, uint32_t P,
                           Reread reread, Emit emit, Blk& bk) {
  Smem& sm = bk.sm;
  const int t = threadIdx.x;
  uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < LPT; ++e)
    if (key[e]) {
      ++nvalid;
      mn = min(mn, (uint32_t)(key[e] >> 32));
      mx = max(mx, (uint32_t)(key[e] >> 32));
    }
  bk.reduce(nvalid, mn, mx);
  // T0': the lower edge of the first-pass bin of the P-th best listed key (1 when there are at
  // most P listed keys: every group with a cut is then re-read)
  Pass p0;
  p0.make(key_lo(mn), key_hi(mx));
  const bool hist = nvalid > P;
  uint64_t t0 = 1ull;
  if (hist) {
#pragma unroll
    for (int e = 0; e < LPT; ++e) atomicAdd(&sm.hist[p0.bin(key[e])], 1u);
    lds_barrier();
    find_bin(P, false, bk);
    t0 = p0.bin_lo(sm.bin);
  }
  const int gshift = __builtin_ctz((unsigned)gsize);
  const int max_sat = min(MAX_SAT, (MPT * NT) >> gshift);
  {
    const bool sat = t < n_groups && cut != 0ull && cut >= t0;
    uint32_t si = 0;
    if (sat) {
      si = atomicAdd(&sm.nsat, 1u);
      if (si < (uint32_t)max_sat) sm.satgroup[si] = (uint16_t)t;
    }
    sm.satof[t] = (sat && si < (uint32_t)max_sat) ? (uint16_t)(si + 1) : (uint16_t)0;
  }
  lds_barrier();
  const uint32_t nsat = sm.nsat;
  if (nsat > (uint32_t)max_sat) {
    if (hist) find_bin(1, true, bk);          // clear the histogram for the caller's dense path
    return -1;
  }
  // re-read members, all loads issued before any is used; those below T0' drop out
  const uint32_t nc = nsat << gshift;
  const uint32_t omask = (uint32_t)gsize - 1u;
  uint64_t m[MPT];
#pragma unroll
  for (int i = 0; i < MPT; ++i) {
    const uint32_t idx = (uint32_t)(i * NT + t);
    m[i] = idx < nc ? reread((int)sm.satgroup[idx >> gshift], (int)(idx & omask)) : 0ull;
  }
#pragma unroll
  for (int i = 0; i < MPT; ++i) {
    if (m[i] < t0) m[i] = 0ull;
    else if (hist) atomicAdd(&sm.hist[p0.bin(m[i])], 1u);
  }
  // listed keys that stay candidates: >= T0', in groups that were not re-read
#pragma unroll
  for (int e = 0; e < LPT; ++e) {
    const int grp = (e * NT + t) / L;
    const bool gone = grp < n_groups && sm.satof[grp];
    if (hist && gone && key[e] >= t0) atomicSub(&sm.hist[p0.bin(key[e])], 1u);
    if (gone || key[e] < t0) key[e] = 0ull;
  }
  lds_barrier();
  auto each = [&](auto f) {
#pragma unroll
    for (int e = 0; e < LPT; ++e) f(key[e]);
#pragma unroll
    for (int i = 0; i < MPT; ++i) f(m[i]);
  };
  uint64_t thr;
  if (hist) {
    // T*: its bin in the adjusted first-pass histogram, then ranked or narrowed
    find_bin(P, true, bk);
    const uint32_t b = sm.bin, cnt = sm.cnt, need = P - sm.above;
    const uint64_t lo = p0.bin_lo(b), hi = p0.bin_hi(b);
    if (p0.shift == 0) {
      thr = lo;
    } else if (cnt <= (uint32_t)RANK_MAX) {
      each([&](uint64_t k) {
        if (k >= lo && k <= hi) sm.rk[atomicAdd(&sm.nrk, 1u)] = k;
      });
      lds_barrier();
      thr = rank_small(cnt, need, bk);
    } else {
      thr = select_kth(each, need, lo, hi, bk);
    }
  } else {
    uint32_t n = 0, cmn = 0xffffffffu, cmx = 0u;
    each([&](uint64_t k) {
      if (k) {
        ++n;
        cmn = min(cmn, (uint32_t)(k >> 32));
        cmx = max(cmx, (uint32_t)(k >> 32));
      }
    });
    bk.reduce(n, cmn, cmx);
    thr = n > P ? select_kth(each, P, key_lo(cmn), key_hi(cmx), bk) : 1ull;
  }
  // selected members: their places in item order, and each re-read slot's first place
  uint32_t msel[MPT], moff[MPT];
#pragma unroll
  for (int i = 0; i < MPT; ++i) msel[i] = (m[i] && m[i] >= thr) ? 1u : 0u;
  const uint32_t mtotal = ordered<true, MPT>(msel, moff, bk);
#pragma unroll
  for (int i = 0; i < MPT; ++i) {
    const uint32_t idx = (uint32_t)(i * NT + t);
    if (idx < nc && (idx & omask) == 0u) sm.gstart[idx >> gshift] = moff[i];
  }
  if (t == 0) sm.gstart[nsat] = mtotal;
  lds_barrier();
  // output places: a re-read group takes its selected members at its first list entry
  uint32_t cnt[LPT], off[LPT];
#pragma unroll
  for (int e = 0; e < LPT; ++e) {
    const int g = e * NT + t, grp = g / L;
    const uint32_t so = grp < n_groups ? sm.satof[grp] : 0u;
    cnt[e] = so ? ((g % L == 0) ? sm.gstart[so] - sm.gstart[so - 1] : 0u) : (key[e] >= thr && key[e] ? 1u : 0u);
  }
  const uint32_t total = ordered<false, LPT>(cnt, off, bk);
  if (total > P) return -1;                  // copies of one key at the P-th place
#pragma unroll
  for (int e = 0; e < LPT; ++e) {
    const int g = e * NT + t, grp = g / L;
    const uint32_t so = grp < n_groups ? sm.satof[grp] : 0u;
    if (so) {
      if (g % L == 0) sm.satoff[so - 1] = off[e];
    } else if (cnt[e]) {
      emit(off[e], key[e], grp, -1);
    }
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < MPT; ++i) {
    if (msel[i]) {
      const uint32_t idx = (uint32_t)(i * NT + t), si = idx >> gshift;
      emit(sm.satoff[si] + moff[i] - sm.gstart[si], m[i], (int)sm.satgroup[si], (int)(idx & omask));
    }
  }
  lds_barrier();
  return (int)total;
}

// The P best of n keys read from global memory (key_at(j), 0 = none), emitted in index order:
// every key above the P-th, then copies of it in index order while places remain.  Returns the
// number emitted.  Requires a clear histogram.
template <class KeyAt, class Emit>
__device__ uint32_t dense_select(KeyAt key_at, int n, uint32_t P, Emit emit, Blk& bk) {
  constexpr int kB = 16;                     // keys per thread per batch
  const int t = threadIdx.x;
  uint32_t nv = 0, mn = 0xffffffffu, mx = 0u;
  for (int j = t; j < n; j += NT) {
    const uint64_t k = key_at(j);
    if (k) {
      ++nv;
      mn = min(mn, (uint32_t)(k >> 32));
      mx = max(mx, (uint32_t)(k >> 32));
    }
  }
  bk.reduce(nv, mn, mx);
  auto each = [&](auto f) {
    for (int base = t; base < n; base += NT * kB) {
      uint64_t kk[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) kk[u] = base + u * NT < n ? key_at(base + u * NT) : 0ull;
#pragma unroll
      for (int u = 0; u < kB; ++u) f(kk[u]);
    }
  };
  const uint64_t thr = nv > P ? select_kth(each, P, key_lo(mn), key_hi(mx), bk) : 1ull;
  // keys above thr, then copies of thr in index order while places remain
  uint32_t n_gt = 0, d0 = 0, d1 = 0;
  for (int j = t; j < n; j += NT) n_gt += key_at(j) > thr ? 1u : 0u;
  bk.reduce(n_gt, d0, d1);
  const uint32_t room = P > n_gt ? P - n_gt : 0u;
  uint32_t done = 0, eq_done = 0;
  for (int base = 0; base < n; base += NT * kB) {
    uint64_t kk[kB];
    uint32_t ceq[kB], oeq[kB], sel[kB], osel[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = base + u * NT + t;
      kk[u] = j < n ? key_at(j) : 0ull;
      ceq[u] = (kk[u] && kk[u] == thr) ? 1u : 0u;
    }
    const uint32_t neq = ordered<true, kB>(ceq, oeq, bk);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      sel[u] = (kk[u] && (kk[u] > thr || (ceq[u] && eq_done + oeq[u] < room))) ? 1u : 0u;
    const uint32_t ns = ordered<true, kB>(sel, osel, bk);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (sel[u] && done + osel[u] < P) emit(done + osel[u], kk[u], base + u * NT + t);
    done += ns;
    eq_done += neq;
  }
  lds_barrier();
  return min(done, P);
}

}  // namespace ls

// Pool from the scan's chunk lists (k_idx_scan: per chunk of bpc blocks, up to 16 listed blocks in
// block order and a cut), one WG of 512 threads per query; outputs as k_pool with K = 0.  Falls
// back to a selection over every block key when too many chunks would be re-read.
constexpr int kPoolChunks = 256;
constexpr int kPLE = kPoolChunks * kListLen / ls::NT;   // listed keys per thread (8)
constexpr int kPLM = 8;                                    // re-read blocks per thread

__global__ __launch_bounds__(ls::NT) void k_pool_chunks(
    const uint64_t* __restrict__ clists, const uint64_t* __restrict__ ccuts, int n_chunks, int bpc,
    const uint32_t* __restrict__ blkkey, int nb_max, const int32_t* __restrict__ n_visible, int n_max, int P,
    int32_t* __restrict__ pool_pos, int cap_out, int32_t* __restrict__ pool_len) {
  __shared__ ls::Smem sm;
  __shared__ uint32_t byrank[kMaxTopK];      // selected blocks, ascending
  ls::Blk bk{sm};
  const int q = blockIdx.x, t = threadIdx.x;
  // every load of the selection's first steps is issued here, before any is used
  const int nv_raw = n_visible[q];
  const uint64_t* cl = clists + (size_t)q * n_chunks * kListLen;
  uint64_t key[kPLE];
#pragma unroll
  for (int e = 0; e < kPLE; ++e) {
    const int g = e * ls::NT + t;
    key[e] = g < n_chunks * kListLen ? cl[g] : 0ull;
  }
  const uint64_t cut = t < n_chunks ? ccuts[(size_t)q * n_chunks + t] : 0ull;
  ls::init(sm);
  const int nv = nv_raw < 0 ? 0 : (nv_raw > n_max ? n_max : nv_raw);
  const int nb = (nv + kBlock - 1) / kBlock;
  const uint32_t* keys = blkkey + (size_t)q * nb_max;
  lds_barrier();
  const bool all = nb <= P;
  uint32_t nsel = 0;
  if (!all) {
    auto reread = [&](int grp, int o) -> uint64_t {
      const int j = grp * bpc + o;
      return j < nb ? rank_key(keys[j], (uint32_t)j) : 0ull;
    };
    auto emit = [&](uint32_t off, uint64_t k, int grp, int o) {
      byrank[off] = o < 0 ? rank_key_index(k) : (uint32_t)(grp * bpc + o);
    };
    const int r = ls::list_select<kListLen, kPLE, kPLM>(key, cut, n_chunks, bpc, (uint32_t)P, reread, emit, bk);
    if (r >= 0) {
      nsel = (uint32_t)r;
    } else {
      nsel = ls::dense_select([&](int j) -> uint64_t { return rank_key(keys[j], (uint32_t)j); }, nb, (uint32_t)P,
                              [&](uint32_t off, uint64_t, int j) { byrank[off] = (uint32_t)j; }, bk);
    }
  }
  // slot s holds block byrank[s / 8] (position s when every block is kept), -1 padded
  int total;
  if (all) {
    total = nv;
  } else {
    total = 8 * (int)nsel;
    if (nsel > 0 && (int)byrank[nsel - 1] == nb - 1) total -= kBlock - (nv - kBlock * (nb - 1));
  }
  // 4 slots (half a block) per 16-byte store, kMaxPool / (4 * 512) = 8 stores per thread; every
  // byrank read is issued before the stores
  int32_t* gp = pool_pos + (size_t)q * cap_out;
  constexpr int kSt = kMaxPool / (4 * ls::NT);
  uint32_t blk[kSt];
#pragma unroll
  for (int i = 0; i < kSt; ++i) {
    const int s4 = 4 * (i * ls::NT + t);
    blk[i] = (!all && s4 < total) ? byrank[s4 >> 3] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kSt; ++i) {
    const int s4 = 4 * (i * ls::NT + t);
    if (s4 < cap_out) {
      int32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sl = s4 + e;
        v[e] = sl < total ? (all ? sl : kBlock * (int)blk[i] + (sl & 7)) : -1;
      }
      *(u32x4*)(gp + s4) = u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
    }
  }
  if (t == 0) pool_len[q] = total;
}


// Pool over every block key when a query has at most kDensePoolBlocks blocks (16 per thread:
// block j = e*kNT + t): the P best by (key desc, block asc), then the pool and its Top-K as k_pool
// writes them.  Block keys are distinct as ranking keys (the block index is part of the key),
// so exactly P blocks pass the P-th best.
__global__ __launch_bounds__(kNT) void k_pool_dense(
    const uint32_t* __restrict__ blkkey, int nb_max, const int32_t* __restrict__ n_visible, int n_max, int P,
    int32_t* __restrict__ pool_pos, int cap_out, int32_t* __restrict__ pool_len,
    const float* __restrict__ scores, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelectSmem sm;
  __shared__ uint32_t byrank[kMaxTopK];      // selected blocks, ascending
  Block bk{sm};
  const int q = blockIdx.x, t = threadIdx.x;
  int nv = n_visible[q];
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int nb = (nv + kBlock - 1) / kBlock;
  const uint32_t* keys = blkkey + (size_t)q * nb_max;
  smem_init(sm);
  const bool all = nb <= P;
  uint32_t nsel = 0;
  if (!all) {
    uint32_t k32[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int jb = e * kNT + t;
      k32[e] = jb < nb ? keys[jb] : 0u;
    }
    uint64_t key[kE];
    uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int jb = e * kNT + t;
      const bool ok = jb < nb;
      key[e] = ok ? rank_key(k32[e], (uint32_t)jb) : 0ull;
      nvalid += ok ? 1u : 0u;
      if (ok) { mn = min(mn, k32[e]); mx = max(mx, k32[e]); }
    }
    bk.reduce(nvalid, mn, mx);
    auto for_each = [&](auto f) {
#pragma unroll
      for (int e = 0; e < kE; ++e) f(key[e]);
    };
    const uint64_t thr = select_kth(for_each, (uint32_t)P, key_lo(mn), key_hi(mx), bk, nullptr);
    uint32_t c[kE], off[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) c[e] = key[e] >= thr ? 1u : 0u;
    nsel = min(ordered_offsets<true>(c, off, bk), (uint32_t)P);
#pragma unroll
    for (int e = 0; e < kE; ++e)
      if (c[e] && off[e] < (uint32_t)P) byrank[off[e]] = (uint32_t)(e * kNT + t);
    lds_barrier();
  }
  pool_out(all, nv, nb, nsel, byrank, pool_pos + (size_t)q * cap_out, cap_out, pool_len + q,
           scores + (size_t)q * n_max, K, topk_idx + (size_t)q * K, topk_score ? topk_score + (size_t)q * K : nullptr,
           bk);
}

hipError_t launch_pool(const uint64_t* lists, const uint64_t* cuts, int n_units, int blocks_per_unit,
                       const uint64_t* clists, const uint64_t* ccuts, int n_chunks, int blocks_per_chunk,
                       const uint32_t* blkkey, int nb_max, const int32_t* n_visible, int n_max, int P,
                       int32_t* pool_pos, int cap_out, int32_t* pool_len, const float* scores, int K,
                       int32_t* topk_idx, float* topk_score, int Q, hipStream_t s) {
  if (clists) {
    // the chunk-list pool writes the pool only; a Top-K of it is one more launch
    if (n_chunks > kPoolChunks || blocks_per_chunk < 64 || blocks_per_chunk > 1024 ||
        (blocks_per_chunk & (blocks_per_chunk - 1)) != 0 || !ccuts || cap_out > kMaxPool)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_pool_chunks, dim3(Q), dim3(ls::NT), 0, s, clists, ccuts, n_chunks, blocks_per_chunk, blkkey,
                       nb_max, n_visible, n_max, P, pool_pos, cap_out, pool_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || K == 0) return e;
    TopkJob j{};
    j.scores = scores;
    j.score_stride = n_max;
    j.n_rows = n_max > 0 ? n_max : 1;
    j.by_position = 1;
    j.items = Q;
    j.out_idx = topk_idx;
    j.out_score = topk_score;
    return launch_topk(pool_pos, pool_len, cap_out, Q, K, j, TopkJob{}, s);
  }
  if (cap_out > kMaxPool) return hipErrorInvalidValue;
  if (nb_max <= kDensePoolBlocks) {
    hipLaunchKernelGGL(k_pool_dense, dim3(Q), dim3(kNT), 0, s, blkkey, nb_max, n_visible, n_max, P, pool_pos,
                       cap_out, pool_len, scores, K, topk_idx, topk_score);
    return hipGetLastError();
  }
  if (n_units > kUnitsPerThread * kNT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_pool, dim3(Q), dim3(kNT), 0, s, lists, cuts, n_units, blocks_per_unit, blkkey, nb_max,
                     n_visible, n_max, P, pool_pos, cap_out, pool_len, scores, K, topk_idx, topk_score);
  return hipGetLastError();
}

// ------------------------------------------------------------------ Top-K over given pools

// Top-K of one item over all its slots (slot i*kNT + t belongs to thread t, so each load
// instruction reads consecutive slots): slot i < len has position cp[i] (ignored if negative or
// >= n_rows); its score is sc[position] (by_position) or sc[i].  Output as topk_out.  Requires a
// clear histogram (smem_init).
__device__ __forceinline__ void topk_dense(const int32_t* __restrict__ cp, int len, const float* __restrict__ sc,
                                           bool by_position, int64_t n_rows, int k, int32_t* __restrict__ oi,
                                           float* __restrict__ os, Block& bk) {
  const int t = threadIdx.x;
  int32_t pos[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int slot = i * kNT + t;
    pos[i] = cp[slot < len ? slot : 0];
  }
  bool ok[kE];
  float s[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int slot = i * kNT + t;
    ok[i] = slot < len && pos[i] >= 0 && (int64_t)pos[i] < n_rows;
    s[i] = sc[by_position ? (ok[i] ? pos[i] : 0) : (slot < len ? slot : 0)];
  }
  uint64_t key[kE];
  uint32_t nvalid = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const uint32_t k32 = score_key(s[i]);
    key[i] = ok[i] ? rank_key(k32, (uint32_t)pos[i]) : 0ull;
    nvalid += ok[i] ? 1u : 0u;
    if (ok[i]) { mn = min(mn, k32); mx = max(mx, k32); }
  }
  topk_out(key, nvalid, mn, mx, k, oi, os, bk);
}

// One WG per item: the items of job a, then those of job b (it = l*Q + q within its job).
// Candidates: slots [0, len) of the item's query; slot i has position cand_pos[i] (ignored if
// negative or >= the job's n_rows); its score as TopkJob states.  Output: the k best positions
// in slot order (ascending positions for an ascending pool) with their scores, -1 / 0 padded.
__global__ __launch_bounds__(kNT) void k_topk(const int32_t* __restrict__ cand_pos,
                                              const int32_t* __restrict__ cand_len, int cap, int Q, int k,
                                              TopkJob a, TopkJob b) {
  __shared__ SelectSmem sm;
  Block bk{sm};
  const bool in_a = (int)blockIdx.x < a.items;
  const TopkJob& job = in_a ? a : b;
  const int it = in_a ? (int)blockIdx.x : (int)blockIdx.x - a.items;
  const int q = it % Q;
  smem_init(sm);
  int len = cand_len[q];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const bool by_position = job.by_position != 0;
  const float* sc = job.scores + (size_t)(by_position ? q : it) * job.score_stride;
  topk_dense(cand_pos + (size_t)q * cap, len, sc, by_position, job.n_rows, k, job.out_idx + (size_t)it * k,
             job.out_score ? job.out_score + (size_t)it * k : nullptr, bk);
}

hipError_t launch_topk(const int32_t* cand_pos, const int32_t* cand_len, int cap, int Q, int k,
                       const TopkJob& a, const TopkJob& b, hipStream_t s) {
  const int items = a.items + b.items;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3(items), dim3(kNT), 0, s, cand_pos, cand_len, cap, Q, k, a, b);
  return hipGetLastError();
}

}  // namespace csa2
