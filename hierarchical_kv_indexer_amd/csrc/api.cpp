// C ABI of the CSA2 hot path: argument checks, workspace carving and kernel dispatch.
// The operations and their readings are documented in include/csa2.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "api_internal.hpp"
#include "csa2.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

csa2_status fail(csa2_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
csa2_status fail(csa2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

csa2_status ok() {
  g_err.clear();
  return CSA2_OK;
}

}  // namespace

csa2_status csa2::api_fail(csa2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

namespace {

csa2_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CSA2_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, st, ...) \
  do {                          \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p) \
  REQUIRE((p) != nullptr && aligned16(p), CSA2_ERR_INVALID_ARG, "%s must be a non-null 16-byte aligned device pointer", #p)

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace carving: a running offset, 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

struct FullPlan {
  int Q, nb_max, nb_stride, chunk, n_wg, upw, n_units, blocks_per_unit, P, cap;
  bool internal_pool, multi_query;
  bool chunk_lists;   // the scan also leaves chunk lists and the pool selects from them first
  bool unit_lists;    // the scan leaves unit lists for the pool (neither chunk lists nor a dense pool)
};

constexpr int kMaxPositions = 1 << 23;   // scores only: 1024 chunks of 8192 positions per query

FullPlan plan_full(int B, int T, int n_max, int pool_blocks, int top_k) {
  FullPlan p;
  p.Q = B * T;
  p.nb_max = (n_max + csa2::kBlock - 1) / csa2::kBlock;
  p.nb_stride = (p.nb_max + 63) / 64 * 64;                 // 256-byte rows of block keys
  p.multi_query = csa2::scan_multi_query(T, n_max);
  p.chunk = p.multi_query ? csa2::scan_mq_chunk(n_max, B, T) : csa2::scan_chunk_positions(n_max, p.Q);
  p.n_wg = n_max > 0 ? (n_max + p.chunk - 1) / p.chunk : 1;
  // Each wave of the scan lists the five best blocks of upw units of its range.  Units are made as
  // small as the pool takes (at most 4096 units of at least 8 blocks): with a pool holding a large
  // share of the blocks, big units often have more than four selected blocks and must be re-read.
  const int bpw = p.chunk / (csa2::kBlock * csa2::kScanUnitsPerWg);
  p.upw = 1;
  while (bpw / (2 * p.upw) >= 8 && (int64_t)p.n_wg * csa2::kScanUnitsPerWg * 2 * p.upw <= 4096 &&
         (!p.multi_query || 2 * p.upw <= 4))
    p.upw *= 2;
  p.n_units = p.n_wg * csa2::kScanUnitsPerWg * p.upw;
  p.blocks_per_unit = bpw / p.upw;
  p.internal_pool = pool_blocks == 0;
  p.P = p.internal_pool ? top_k : pool_blocks;
  p.cap = p.P * csa2::kBlock;
  // Chunk lists (16 blocks and a cut per chunk of the one-query scan) pay off when a chunk is
  // expected to hold few pool blocks: at most 8 on average, so that few chunks have more than 16
  // and must be re-read.  The 1M decode (chunks of 512 blocks, 1/64 of the blocks pooled) expects 8.
  const int bpc = p.chunk / csa2::kBlock;
  p.chunk_lists = !p.multi_query && p.upw == 1 && p.n_wg <= 256 && p.nb_max > p.P &&
                  (int64_t)p.P * bpc <= (int64_t)8 * p.nb_max;
  // Otherwise queries of at most kDensePoolBlocks blocks are pooled over every block key, and
  // longer ones from the scan's unit lists.
  p.unit_lists = !p.chunk_lists && p.nb_stride > csa2::kDensePoolBlocks;
  return p;
}

// Pieces of the Full-layer workspace, in order.
struct FullWs {
  float* scores;
  uint32_t* blkkey;
  uint64_t* lists;
  uint64_t* cuts;
  uint64_t* clists;    // chunk lists (chunk_lists only)
  uint64_t* ccuts;
  int32_t* pool_pos;   // internal pool (pool_blocks == 0 only)
  int32_t* pool_len;
};

size_t carve_full(void* ws, const FullPlan& p, int n_max, FullWs* out) {
  Carver c{(char*)ws};
  FullWs w;
  w.scores = c.take<float>((size_t)p.Q * (n_max > 0 ? n_max : 1));
  w.blkkey = c.take<uint32_t>((size_t)p.Q * p.nb_stride + 64);   // + tail read by unit batches
  w.lists = p.unit_lists ? c.take<uint64_t>((size_t)p.Q * p.n_units * 4) : nullptr;
  w.cuts = p.unit_lists ? c.take<uint64_t>((size_t)p.Q * p.n_units) : nullptr;
  w.clists = p.chunk_lists ? c.take<uint64_t>((size_t)p.Q * p.n_wg * csa2::kListLen) : nullptr;
  w.ccuts = p.chunk_lists ? c.take<uint64_t>((size_t)p.Q * p.n_wg) : nullptr;
  w.pool_pos = p.internal_pool ? c.take<int32_t>((size_t)p.Q * p.cap) : nullptr;
  w.pool_len = p.internal_pool ? c.take<int32_t>((size_t)p.Q) : nullptr;
  if (out) *out = w;
  return c.off;
}

// csa2_index_full runs the scan and the selection over batches of queries, reusing one batch's
// workspace for its intermediate data (scores, block keys, lists, internal pool): batches of tb
// consecutive queries of one sequence when a sequence holds more than 16 queries, else of bb whole
// sequences.  The caller's workspace decides the batches: every query at once when it holds them
// all (fastest: the most parallel launches), else the largest batches it holds.  The smallest
// workspace the call accepts (csa2_index_full_workspace) holds batches of kFullBatchQueries
// queries (one selection workgroup per CU keeps the GPU busy), or everything when that is at most
// kFullBatchBytes; past kFullSpillCap it holds 16 queries (the multi-query scan's group).
constexpr size_t kFullBatchBytes = (size_t)64 << 20;
constexpr size_t kFullSpillCap = (size_t)1 << 30;
constexpr int kFullBatchQueries = 256;

struct FullBatches {
  bool by_seq;     // batches of bb whole sequences (else tb queries of one sequence)
  int bb, tb;
  size_t ws_bytes; // the largest batch's workspace
};

// Batches that fit `budget` bytes (ws_bytes > budget when not even the smallest batch fits).
FullBatches plan_full_batches(int B, int T, int n_max, int pool_blocks, int top_k, size_t budget) {
  auto need = [&](int b, int t) { return carve_full(nullptr, plan_full(b, t, n_max, pool_blocks, top_k), n_max, nullptr); };
  FullBatches fb;
  fb.by_seq = true;
  fb.bb = B;
  fb.tb = T;
  fb.ws_bytes = need(B, T);
  if (fb.ws_bytes <= budget) return fb;
  if (T > 16) {
    // a multiple of 16 queries of one sequence, as many as fit (need grows with the batch)
    int lo = 1, hi = (T + 15) / 16;            // batches of 16*k queries, k in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (need(1, std::min(T, 16 * mid)) <= budget) lo = mid; else hi = mid - 1;
    }
    fb.by_seq = false;
    fb.bb = 1;
    fb.tb = std::min(T, 16 * lo);
    fb.ws_bytes = need(1, fb.tb);
    if (T % fb.tb) fb.ws_bytes = std::max(fb.ws_bytes, need(1, T % fb.tb));
  } else {
    int lo = 1, hi = B;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (need(mid, T) <= budget) lo = mid; else hi = mid - 1;
    }
    fb.bb = lo;
    fb.ws_bytes = need(lo, T);
    if (B % lo) fb.ws_bytes = std::max(fb.ws_bytes, need(B % lo, T));
  }
  return fb;
}

// The smallest workspace csa2_index_full accepts (see above).
size_t full_min_workspace(int B, int T, int n_max, int pool_blocks, int top_k) {
  auto need = [&](int b, int t) { return carve_full(nullptr, plan_full(b, t, n_max, pool_blocks, top_k), n_max, nullptr); };
  const size_t all = need(B, T);
  if (all <= kFullBatchBytes) return all;
  size_t busy;                                 // batches of about kFullBatchQueries queries
  if (T > 16) {
    const int tb = std::min(T, kFullBatchQueries);
    busy = need(1, tb);
    if (T % tb) busy = std::max(busy, need(1, T % tb));
  } else {
    const int bb = std::min(B, (kFullBatchQueries + T - 1) / T);
    busy = need(bb, T);
    if (B % bb) busy = std::max(busy, need(B % bb, T));
  }
  busy = std::min(busy, all);
  if (busy <= kFullSpillCap) return busy;
  return plan_full_batches(B, T, n_max, pool_blocks, top_k, 0).ws_bytes;   // the smallest batches
}

}  // namespace

extern "C" {

const char* csa2_last_error(void) { return g_err.c_str(); }

csa2_status csa2_quantize_query(const uint16_t* in_bf16, uint8_t* out_e4m3, int64_t n, void* stream) {
  REQUIRE(n >= 0, CSA2_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  REQUIRE(in_bf16 != nullptr && out_e4m3 != nullptr, CSA2_ERR_INVALID_ARG, "null pointer");
  csa2_status st = hip_check(csa2::launch_quantize_query(in_bf16, out_e4m3, n, (hipStream_t)stream),
                             "quantize_query launch");
  return st == CSA2_OK ? ok() : st;
}

csa2_status csa2_quantize_kv_fp4(const uint16_t* latent_bf16, int64_t rows, uint8_t* kv_codes, uint8_t* kv_scales,
                                 void* stream) {
  REQUIRE(rows >= 0 && rows <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG, "rows must be in [0, 2^31]");
  if (rows == 0) return ok();
  REQUIRE_PTR(latent_bf16);
  REQUIRE_PTR(kv_codes);
  REQUIRE_PTR(kv_scales);
  csa2_status st = hip_check(csa2::launch_quantize_kv(latent_bf16, rows, kv_codes, kv_scales, (hipStream_t)stream),
                             "quantize_kv launch");
  return st == CSA2_OK ? ok() : st;
}

static csa2_status check_index_common(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows,
                                      const uint16_t* idx_q,
                                      const float* head_w, const int32_t* n_visible, int B, int T,
                                      int n_max) {
  REQUIRE(B >= 1 && T >= 1, CSA2_ERR_INVALID_ARG, "B and T must be >= 1 (got %d, %d)", B, T);
  REQUIRE((int64_t)B * T <= 65535, CSA2_ERR_UNSUPPORTED, "B*T must be <= 65535");
  REQUIRE(n_max >= 0, CSA2_ERR_INVALID_ARG, "n_max must be >= 0");
  REQUIRE(n_max <= kMaxPositions, CSA2_ERR_UNSUPPORTED, "n_max must be <= %d", kMaxPositions);
  REQUIRE(k_rows >= n_max && k_rows < ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "need n_max <= k_rows_per_seq < 2^31 (n_max %d, k_rows %lld)", n_max, (long long)k_rows);
  REQUIRE_PTR(idx_k);
  REQUIRE(idx_ks == nullptr || aligned16(idx_ks), CSA2_ERR_INVALID_ARG, "idx_k_scales must be 16-byte aligned");
  REQUIRE_PTR(idx_q);
  REQUIRE_PTR(head_w);
  REQUIRE_PTR(n_visible);
  return CSA2_OK;
}

csa2_status csa2_index_scores(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                              const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                              float* scores, void* stream) {
  csa2_status st = check_index_common(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max);
  if (st != CSA2_OK) return st;
  REQUIRE_PTR(scores);
  if (n_max == 0) return ok();
  const FullPlan p = plan_full(B, T, n_max, 1, 1);
  st = hip_check(csa2::launch_idx_scan(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, p.Q, T, n_max,
                                       scores, nullptr, p.nb_max, nullptr, nullptr, p.chunk, p.n_wg, p.multi_query,
                                       csa2::kBlockMax, p.upw, nullptr, nullptr, (hipStream_t)stream),
                 "index scan launch");
  return st == CSA2_OK ? ok() : st;
}

size_t csa2_index_stages_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k) {
  (void)block_size;
  if (B < 1 || T < 1 || n_max < 0 || pool_blocks < 0 || top_k < 1) return 0;
  return carve_full(nullptr, plan_full(B, T, n_max, pool_blocks, top_k), n_max, nullptr);
}

size_t csa2_index_full_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k) {
  (void)block_size;
  if (B < 1 || T < 1 || n_max < 0 || pool_blocks < 0 || top_k < 1) return 0;
  return full_min_workspace(B, T, n_max, pool_blocks, top_k);
}

static csa2_status check_full_shape(int B, int T, int n_max, int block_size, int pool_blocks, int top_k) {
  REQUIRE(B >= 1 && T >= 1, CSA2_ERR_INVALID_ARG, "B and T must be >= 1 (got %d, %d)", B, T);
  REQUIRE((int64_t)B * T <= 65535, CSA2_ERR_UNSUPPORTED, "B*T must be <= 65535");
  REQUIRE(n_max >= 0, CSA2_ERR_INVALID_ARG, "n_max must be >= 0");
  REQUIRE(block_size == csa2::kBlock, CSA2_ERR_UNSUPPORTED, "block_size must be 8 (got %d)", block_size);
  REQUIRE(top_k >= 1 && top_k <= csa2::kMaxTopK, CSA2_ERR_UNSUPPORTED, "top_k must be in [1, %d]", csa2::kMaxTopK);
  REQUIRE(pool_blocks >= 0 && (int64_t)pool_blocks * block_size <= csa2::kMaxPool, CSA2_ERR_UNSUPPORTED,
          "pool_blocks * block_size must be <= %d", csa2::kMaxPool);
  REQUIRE(pool_blocks == 0 || top_k <= pool_blocks * block_size, CSA2_ERR_INVALID_ARG,
          "top_k (%d) exceeds the pool capacity (%d)", top_k, pool_blocks * block_size);
  REQUIRE(n_max <= csa2::kMaxFullPositions, CSA2_ERR_UNSUPPORTED, "n_max must be <= %d for the Full layer",
          csa2::kMaxFullPositions);
  return CSA2_OK;
}

static csa2_status check_workspace(const FullPlan& p, int n_max, void* workspace, size_t ws_bytes) {
  const size_t need = carve_full(nullptr, p, n_max, nullptr);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= need, CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  return CSA2_OK;
}

static csa2_status index_scan(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq,
                              const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int B, int T,
                              int n_max, int block_size, int pool_blocks, int top_k, int block_score,
                              void* workspace, size_t ws_bytes, void* stream) {
  csa2_status st = check_index_common(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max);
  if (st != CSA2_OK) return st;
  if ((st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k)) != CSA2_OK) return st;
  REQUIRE(block_score >= csa2::kBlockMax && block_score <= csa2::kBlockTop2, CSA2_ERR_INVALID_ARG,
          "block_score must be 0 (max), 1 (sum) or 2 (top-2 mean); got %d", block_score);
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_workspace(p, n_max, workspace, ws_bytes)) != CSA2_OK) return st;
  FullWs w;
  carve_full(workspace, p, n_max, &w);
  if (n_max > 0) {
    st = hip_check(csa2::launch_idx_scan(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, p.Q, T, n_max,
                                         w.scores, w.blkkey, p.nb_stride, w.lists, w.cuts, p.chunk, p.n_wg,
                                         p.multi_query, block_score, p.upw, w.clists, w.ccuts, (hipStream_t)stream),
                   "index scan launch");
    if (st != CSA2_OK) return st;
  }
  return ok();
}

csa2_status csa2_index_scan(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                            const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                            int block_size, int pool_blocks, int top_k, void* workspace, size_t ws_bytes,
                            void* stream) {
  return index_scan(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max, block_size,
                    pool_blocks, top_k, csa2::kBlockMax, workspace, ws_bytes, stream);
}

csa2_status csa2_index_scan_blocks(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq,
                                   const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int B,
                                   int T, int n_max, int block_size, int pool_blocks, int top_k, int block_score,
                                   void* workspace, size_t ws_bytes, void* stream) {
  return index_scan(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max, block_size,
                    pool_blocks, top_k, block_score, workspace, ws_bytes, stream);
}

static csa2_status check_pool_args(const FullPlan& p, int32_t* pool_pos, int32_t* pool_len) {
  if (!p.internal_pool) {
    REQUIRE_PTR(pool_pos);
    REQUIRE_PTR(pool_len);
  }
  return CSA2_OK;
}

static csa2_status check_topk_args(int32_t* topk_idx, float* topk_score) {
  REQUIRE_PTR(topk_idx);
  REQUIRE(topk_score == nullptr || aligned16(topk_score), CSA2_ERR_INVALID_ARG, "topk_score must be 16-byte aligned");
  return CSA2_OK;
}

// The pool; with topk_idx non-null the same kernel also takes the Top-K of the pool.
static csa2_status launch_pool_stage(const FullPlan& p, const FullWs& w, const int32_t* n_visible, int n_max,
                                     int32_t* pool_pos, int32_t* pool_len, int top_k, int32_t* topk_idx,
                                     float* topk_score, hipStream_t s) {
  return hip_check(csa2::launch_pool(w.lists, w.cuts, p.n_units, p.blocks_per_unit, w.clists, w.ccuts, p.n_wg,
                                     p.chunk / csa2::kBlock, w.blkkey, p.nb_stride,
                                     n_visible, n_max, p.P, p.internal_pool ? w.pool_pos : pool_pos, p.cap,
                                     p.internal_pool ? w.pool_len : pool_len, w.scores, topk_idx ? top_k : 0,
                                     topk_idx, topk_score, p.Q, s),
                   "pool launch");
}

// The Full layer's Top-K over its pool, by position in the scan's scores.
static csa2::TopkJob full_topk_job(const FullPlan& p, const FullWs& w, int n_max, int32_t* topk_idx,
                                   float* topk_score) {
  csa2::TopkJob j{};
  j.scores = w.scores;
  j.score_stride = n_max;
  j.n_rows = n_max > 0 ? n_max : 1;
  j.by_position = 1;
  j.items = p.Q;
  j.out_idx = topk_idx;
  j.out_score = topk_score;
  return j;
}

static csa2_status launch_topk_stage(const FullPlan& p, const FullWs& w, int n_max, const int32_t* pool_pos,
                                     const int32_t* pool_len, int top_k, int32_t* topk_idx, float* topk_score,
                                     hipStream_t s) {
  return hip_check(csa2::launch_topk(p.internal_pool ? w.pool_pos : pool_pos,
                                     p.internal_pool ? w.pool_len : pool_len, p.cap, p.Q, top_k,
                                     full_topk_job(p, w, n_max, topk_idx, topk_score), csa2::TopkJob{}, s),
                   "top-k launch");
}

csa2_status csa2_index_pool(const int32_t* n_visible, int B, int T, int n_max, int block_size, int pool_blocks,
                            int top_k, int32_t* pool_pos, int32_t* pool_len, void* workspace, size_t ws_bytes,
                            void* stream) {
  csa2_status st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k);
  if (st != CSA2_OK) return st;
  REQUIRE_PTR(n_visible);
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_pool_args(p, pool_pos, pool_len)) != CSA2_OK) return st;
  if ((st = check_workspace(p, n_max, workspace, ws_bytes)) != CSA2_OK) return st;
  FullWs w;
  carve_full(workspace, p, n_max, &w);
  st = launch_pool_stage(p, w, n_visible, n_max, pool_pos, pool_len, top_k, nullptr, nullptr, (hipStream_t)stream);
  return st == CSA2_OK ? ok() : st;
}

csa2_status csa2_index_topk(int B, int T, int n_max, int block_size, int pool_blocks, int top_k,
                            const int32_t* pool_pos, const int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                            void* workspace, size_t ws_bytes, void* stream) {
  csa2_status st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k);
  if (st != CSA2_OK) return st;
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_pool_args(p, (int32_t*)pool_pos, (int32_t*)pool_len)) != CSA2_OK) return st;
  if ((st = check_topk_args(topk_idx, topk_score)) != CSA2_OK) return st;
  if ((st = check_workspace(p, n_max, workspace, ws_bytes)) != CSA2_OK) return st;
  FullWs w;
  carve_full(workspace, p, n_max, &w);
  st = launch_topk_stage(p, w, n_max, pool_pos, pool_len, top_k, topk_idx, topk_score, (hipStream_t)stream);
  return st == CSA2_OK ? ok() : st;
}

csa2_status csa2_index_select(const int32_t* n_visible, int B, int T, int n_max, int block_size,
                              int pool_blocks, int top_k, int32_t* pool_pos, int32_t* pool_len,
                              int32_t* topk_idx, float* topk_score, void* workspace, size_t ws_bytes,
                              void* stream) {
  csa2_status st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k);
  if (st != CSA2_OK) return st;
  REQUIRE_PTR(n_visible);
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_pool_args(p, pool_pos, pool_len)) != CSA2_OK) return st;
  if ((st = check_topk_args(topk_idx, topk_score)) != CSA2_OK) return st;
  if ((st = check_workspace(p, n_max, workspace, ws_bytes)) != CSA2_OK) return st;
  FullWs w;
  carve_full(workspace, p, n_max, &w);
  st = launch_pool_stage(p, w, n_visible, n_max, pool_pos, pool_len, top_k, topk_idx, topk_score,
                         (hipStream_t)stream);
  return st == CSA2_OK ? ok() : st;
}

csa2_status csa2_index_full(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                            const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                            int block_size, int pool_blocks, int top_k, int32_t* pool_pos,
                            int32_t* pool_len, int32_t* topk_idx, float* topk_score, void* workspace,
                            size_t ws_bytes, void* stream) {
  // check everything before enqueueing anything
  csa2_status st = check_index_common(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max);
  if (st != CSA2_OK) return st;
  if ((st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k)) != CSA2_OK) return st;
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_pool_args(p, pool_pos, pool_len)) != CSA2_OK) return st;
  if ((st = check_topk_args(topk_idx, topk_score)) != CSA2_OK) return st;
  const size_t min_ws = full_min_workspace(B, T, n_max, pool_blocks, top_k);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= min_ws, CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", min_ws, ws_bytes);
  const FullBatches fb = plan_full_batches(B, T, n_max, pool_blocks, top_k, ws_bytes);
  REQUIRE(fb.ws_bytes <= ws_bytes, CSA2_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", fb.ws_bytes,
          ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  const size_t krow = idx_k_scales ? csa2::kIdxDim / 2 : csa2::kIdxDim;   // key bytes per row
  const size_t srow = csa2::kIdxDim / 16;                                  // FP4 scale bytes per row
  // one batch: queries q0 .. q0 + bb*tb - 1 (bb sequences from b0, tb queries each)
  auto run = [&](int b0, int q0, int bb, int tb) -> csa2_status {
    const FullPlan bp = plan_full(bb, tb, n_max, pool_blocks, top_k);
    FullWs w;
    carve_full(workspace, bp, n_max, &w);
    const uint8_t* kb = idx_k + (size_t)b0 * (size_t)k_rows_per_seq * krow;
    const uint8_t* ksb = idx_k_scales ? idx_k_scales + (size_t)b0 * (size_t)k_rows_per_seq * srow : nullptr;
    const int32_t* nv = n_visible + q0;
    csa2_status r = CSA2_OK;
    if (n_max > 0) {
      r = hip_check(csa2::launch_idx_scan(kb, ksb, k_rows_per_seq, idx_q + (size_t)q0 * csa2::kIdxHeads * csa2::kIdxDim,
                                          head_w + (size_t)q0 * csa2::kIdxHeads, nv, bp.Q, tb, n_max, w.scores,
                                          w.blkkey, bp.nb_stride, w.lists, w.cuts, bp.chunk, bp.n_wg, bp.multi_query,
                                          csa2::kBlockMax, bp.upw, w.clists, w.ccuts, s),
                    "index scan launch");
      if (r != CSA2_OK) return r;
    }
    return launch_pool_stage(bp, w, nv, n_max, pool_pos ? pool_pos + (size_t)q0 * bp.cap : nullptr,
                             pool_len ? pool_len + q0 : nullptr, top_k, topk_idx + (size_t)q0 * top_k,
                             topk_score ? topk_score + (size_t)q0 * top_k : nullptr, s);
  };
  if (fb.by_seq) {
    for (int b0 = 0; b0 < B; b0 += fb.bb)
      if ((st = run(b0, b0 * T, std::min(fb.bb, B - b0), T)) != CSA2_OK) return st;
  } else {
    for (int b = 0; b < B; ++b)
      for (int t0 = 0; t0 < T; t0 += fb.tb)
        if ((st = run(b, b * T + t0, 1, std::min(fb.tb, T - t0))) != CSA2_OK) return st;
  }
  return ok();
}

}  // extern "C"

namespace {

// Scores by slot of `items` scored pools (see k_ri_score).
size_t carve_slot_scores(void* ws, int items, int cap, float** out) {
  Carver c{(char*)ws};
  float* sc = c.take<float>((size_t)items * cap);
  if (out) *out = sc;
  return c.off;
}

}  // namespace

extern "C" {

size_t csa2_reindex_workspace(int L, int B, int T, int pool_cap, int top_k) {
  (void)top_k;
  if (L < 1 || B < 1 || T < 1 || pool_cap < 1 || pool_cap > csa2::kMaxPool) return 0;
  return carve_slot_scores(nullptr, L * B * T, pool_cap, nullptr);
}

csa2_status csa2_reindex(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                         const float* head_w, const int32_t* pool_pos, const int32_t* pool_len,
                         int pool_cap, int L, int B, int T, int top_k, int32_t* topk_idx,
                         float* topk_score, void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(L >= 1 && B >= 1 && T >= 1, CSA2_ERR_INVALID_ARG, "L, B and T must be >= 1");
  REQUIRE((int64_t)L * B * T <= 65535, CSA2_ERR_UNSUPPORTED, "L*B*T must be <= 65535");
  REQUIRE(k_rows_per_seq >= 1 && k_rows_per_seq < ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "k_rows_per_seq must be in [1, 2^31)");
  REQUIRE(pool_cap >= 1 && pool_cap <= csa2::kMaxPool, CSA2_ERR_UNSUPPORTED, "pool_cap must be in [1, %d]", csa2::kMaxPool);
  REQUIRE(top_k >= 1 && top_k <= csa2::kMaxTopK, CSA2_ERR_UNSUPPORTED, "top_k must be in [1, %d]", csa2::kMaxTopK);
  REQUIRE(top_k <= pool_cap, CSA2_ERR_INVALID_ARG, "top_k (%d) exceeds pool_cap (%d)", top_k, pool_cap);
  REQUIRE_PTR(idx_k);
  REQUIRE(idx_k_scales == nullptr || aligned16(idx_k_scales), CSA2_ERR_INVALID_ARG,
          "idx_k_scales must be 16-byte aligned");
  REQUIRE_PTR(idx_q);
  REQUIRE_PTR(head_w);
  REQUIRE_PTR(pool_pos);
  REQUIRE_PTR(pool_len);
  REQUIRE_PTR(topk_idx);
  REQUIRE(topk_score == nullptr || aligned16(topk_score), CSA2_ERR_INVALID_ARG, "topk_score must be 16-byte aligned");
  const size_t need = csa2_reindex_workspace(L, B, T, pool_cap, top_k);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= need, CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  const int Q = B * T;
  hipStream_t s = (hipStream_t)stream;
  float* slot_scores = nullptr;
  carve_slot_scores(workspace, L * Q, pool_cap, &slot_scores);
  csa2_status st = hip_check(csa2::launch_ri_score(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, 0, nullptr,
                                                   nullptr, pool_pos, pool_len, pool_cap, L, Q, T, slot_scores, s),
                             "reindex score launch");
  if (st != CSA2_OK) return st;
  // every item's Top-K over its scored slots, one workgroup per item
  csa2::TopkJob jb{};
  jb.scores = slot_scores;
  jb.score_stride = pool_cap;
  jb.n_rows = k_rows_per_seq;
  jb.by_position = 0;
  jb.items = L * Q;
  jb.out_idx = topk_idx;
  jb.out_score = topk_score;
  st = hip_check(csa2::launch_topk(pool_pos, pool_len, pool_cap, Q, top_k, csa2::TopkJob{}, jb, s), "top-k launch");
  return st == CSA2_OK ? ok() : st;
}

}  // extern "C"

namespace {

// Full layer plus L Reindex layers over its pool: the Full workspace, then the slot scores of
// the Full layer's pool (when it is scored again from its keys) and of the L Reindex items.
size_t carve_chain(void* ws, const FullPlan& p, int n_max, int L, FullWs* fw, float** slot_scores) {
  const size_t full = carve_full(ws, p, n_max, fw);
  return full + carve_slot_scores(ws ? (char*)ws + full : nullptr, (L + 1) * p.Q, p.cap, slot_scores);
}

}  // namespace

extern "C" {

size_t csa2_index_chain_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k, int L) {
  (void)block_size;
  if (B < 1 || T < 1 || n_max < 0 || pool_blocks < 1 || top_k < 1 || L < 0) return 0;
  return carve_chain(nullptr, plan_full(B, T, n_max, pool_blocks, top_k), n_max, L, nullptr, nullptr);
}

static csa2_status index_chain(bool do_scan, const uint8_t* idx_k, const uint8_t* idx_k_scales,
                               int64_t k_rows_per_seq, const uint16_t* idx_q,
                               const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                               int block_size, int pool_blocks, int top_k, const uint16_t* ri_q,
                               const float* ri_w, int L, int32_t* pool_pos, int32_t* pool_len,
                               int32_t* topk_idx, float* topk_score, int32_t* ri_topk_idx,
                               float* ri_topk_score, void* workspace, size_t ws_bytes, void* stream) {
  csa2_status st;
  if (do_scan) {
    st = check_index_common(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max);
    if (st != CSA2_OK) return st;
  } else {
    REQUIRE(k_rows_per_seq >= n_max && k_rows_per_seq < ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
            "need n_max <= k_rows_per_seq < 2^31");
    REQUIRE_PTR(idx_k);
    REQUIRE(idx_k_scales == nullptr || aligned16(idx_k_scales), CSA2_ERR_INVALID_ARG,
            "idx_k_scales must be 16-byte aligned");
    REQUIRE_PTR(n_visible);
  }
  if ((st = check_full_shape(B, T, n_max, block_size, pool_blocks, top_k)) != CSA2_OK) return st;
  REQUIRE(pool_blocks >= 1, CSA2_ERR_INVALID_ARG, "the chain needs a pool (pool_blocks >= 1)");
  REQUIRE(L >= 0 && (int64_t)(L + 1) * B * T <= 65535, CSA2_ERR_UNSUPPORTED, "need L >= 0 and (L+1)*B*T <= 65535");
  const FullPlan p = plan_full(B, T, n_max, pool_blocks, top_k);
  if ((st = check_pool_args(p, pool_pos, pool_len)) != CSA2_OK) return st;
  if ((st = check_topk_args(topk_idx, topk_score)) != CSA2_OK) return st;
  if (L > 0) {
    REQUIRE_PTR(ri_q);
    REQUIRE_PTR(ri_w);
    if ((st = check_topk_args(ri_topk_idx, ri_topk_score)) != CSA2_OK) return st;
  }
  const size_t need = carve_chain(nullptr, p, n_max, L, nullptr, nullptr);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= need, CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  FullWs w;
  float* slot_scores = nullptr;
  carve_chain(workspace, p, n_max, L, &w, &slot_scores);
  hipStream_t s = (hipStream_t)stream;
  // With the one-query scan over E4M3 keys in the same call, the Full layer's pool slots are
  // scored again from their keys (the scan's own arithmetic, so the same scores) instead of
  // storing every position's score; the split calls, FP4 keys (the scan sums 32-row tiles) and
  // the multi-query scan (other summation orders) keep the stored scores.
  const bool rescore = do_scan && !p.multi_query && idx_k_scales == nullptr;
  if (do_scan && n_max > 0) {
    st = hip_check(csa2::launch_idx_scan(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, p.Q, T, n_max,
                                         rescore ? nullptr : w.scores, w.blkkey, p.nb_stride, w.lists, w.cuts, p.chunk,
                                         p.n_wg, p.multi_query, csa2::kBlockMax, p.upw, w.clists, w.ccuts, s),
                   "index scan launch");
    if (st != CSA2_OK) return st;
  }
  st = launch_pool_stage(p, w, n_visible, n_max, pool_pos, pool_len, top_k, nullptr, nullptr, s);
  if (st != CSA2_OK) return st;
  // the Reindex layers' scores of the pool's slots (and, when rescoring, the Full layer's); then
  // every layer's Top-K in one launch, one workgroup per item: the Full items read their scores
  // by slot, or by position from the scan's scores
  const int fi = rescore ? p.Q : 0;
  st = hip_check(csa2::launch_ri_score(idx_k, idx_k_scales, k_rows_per_seq, L ? ri_q : nullptr, L ? ri_w : nullptr,
                                       fi, idx_q, head_w, pool_pos, pool_len, p.cap, L, p.Q, T, slot_scores, s),
                 "pool scoring launch");
  if (st != CSA2_OK) return st;
  csa2::TopkJob ja{}, jb{};
  ja.scores = rescore ? slot_scores : w.scores;
  ja.score_stride = rescore ? p.cap : n_max;
  ja.n_rows = n_max > 0 ? n_max : 1;
  ja.by_position = rescore ? 0 : 1;
  ja.items = p.Q;
  ja.out_idx = topk_idx;
  ja.out_score = topk_score;
  jb.scores = slot_scores + (size_t)fi * p.cap;
  jb.score_stride = p.cap;
  jb.n_rows = k_rows_per_seq;
  jb.by_position = 0;
  jb.items = L * p.Q;
  jb.out_idx = ri_topk_idx;
  jb.out_score = ri_topk_score;
  st = hip_check(csa2::launch_topk(pool_pos, pool_len, p.cap, p.Q, top_k, ja, jb, s), "top-k launch");
  return st == CSA2_OK ? ok() : st;
}

csa2_status csa2_index_chain(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                             const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                             int block_size, int pool_blocks, int top_k, const uint16_t* ri_q, const float* ri_w,
                             int L, int32_t* pool_pos, int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                             int32_t* ri_topk_idx, float* ri_topk_score, void* workspace, size_t ws_bytes,
                             void* stream) {
  return index_chain(true, idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max, block_size, pool_blocks,
                     top_k, ri_q, ri_w, L, pool_pos, pool_len, topk_idx, topk_score, ri_topk_idx, ri_topk_score,
                     workspace, ws_bytes, stream);
}

csa2_status csa2_index_select_reindex(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const int32_t* n_visible,
                                      int B, int T, int n_max, int block_size, int pool_blocks, int top_k,
                                      const uint16_t* ri_q, const float* ri_w, int L, int32_t* pool_pos,
                                      int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                                      int32_t* ri_topk_idx, float* ri_topk_score, void* workspace,
                                      size_t ws_bytes, void* stream) {
  return index_chain(false, idx_k, idx_k_scales, k_rows_per_seq, nullptr, nullptr, n_visible, B, T, n_max, block_size,
                     pool_blocks, top_k, ri_q, ri_w, L, pool_pos, pool_len, topk_idx, topk_score, ri_topk_idx,
                     ri_topk_score, workspace, ws_bytes, stream);
}

size_t csa2_sparse_attn_workspace(int L, int B, int T, int H, int top_k, int swa_window) {
  if (L < 1 || B < 1 || T < 1 || H < 16 || H % 16 != 0 || top_k < 1 || swa_window < 0) return 0;
  return csa2::plan_attn(L, B, T, H, top_k, swa_window).ws_bytes;
}

csa2_status csa2_sparse_attn(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t kv_rows_per_seq,
                             const uint16_t* q, const int32_t* idx_sets, const int32_t* layer_set, int S,
                             const uint8_t* swa_kv, int swa_rows, const int32_t* swa_end, int swa_window,
                             int L, int B, int T, int H, int top_k, float softmax_scale, uint16_t* out,
                             float* lse, void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(L >= 1 && L <= csa2::kMaxLayers, CSA2_ERR_UNSUPPORTED, "L must be in [1, %d]", csa2::kMaxLayers);
  REQUIRE(B >= 1 && T >= 1, CSA2_ERR_INVALID_ARG, "B and T must be >= 1");
  REQUIRE((int64_t)L * B * T <= 65535, CSA2_ERR_UNSUPPORTED, "L*B*T must be <= 65535");
  REQUIRE(H >= 16 && H % 16 == 0 && H <= 1024, CSA2_ERR_UNSUPPORTED, "H must be a multiple of 16 in [16, 1024]");
  REQUIRE(top_k >= 1 && top_k <= csa2::kMaxTopK, CSA2_ERR_UNSUPPORTED, "top_k must be in [1, %d]", csa2::kMaxTopK);
  REQUIRE(S >= 1, CSA2_ERR_INVALID_ARG, "S must be >= 1");
  REQUIRE(swa_window >= 0 && swa_window <= 4096, CSA2_ERR_UNSUPPORTED, "swa_window must be in [0, 4096]");
  REQUIRE(swa_rows >= 0, CSA2_ERR_INVALID_ARG, "swa_rows must be >= 0");
  REQUIRE(kv_rows_per_seq >= 1, CSA2_ERR_INVALID_ARG, "kv_rows_per_seq must be >= 1");
  REQUIRE(layer_set != nullptr, CSA2_ERR_INVALID_ARG, "layer_set (host array) must be non-null");
  REQUIRE(softmax_scale > 0.f, CSA2_ERR_INVALID_ARG, "softmax_scale must be > 0");
  REQUIRE_PTR(kv_codes);
  REQUIRE_PTR(kv_scales);
  REQUIRE_PTR(q);
  REQUIRE_PTR(idx_sets);
  REQUIRE_PTR(swa_end);
  REQUIRE_PTR(out);
  REQUIRE(swa_rows == 0 || (swa_kv != nullptr && aligned16(swa_kv)), CSA2_ERR_INVALID_ARG,
          "swa_kv must be a 16-byte aligned device pointer");
  REQUIRE(lse == nullptr || aligned16(lse), CSA2_ERR_INVALID_ARG, "lse must be 16-byte aligned");
  csa2::LayerSets sets;
  for (int l = 0; l < L; ++l) {
    REQUIRE(layer_set[l] >= 0 && layer_set[l] < S, CSA2_ERR_INVALID_ARG, "layer_set[%d] = %d is not in [0, %d)",
            l, layer_set[l], S);
    sets.set[l] = layer_set[l];
  }
  const size_t need = csa2_sparse_attn_workspace(L, B, T, H, top_k, swa_window);
  REQUIRE(need == 0 || (workspace != nullptr && aligned16(workspace) && ws_bytes >= need), CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  csa2_status st = hip_check(csa2::launch_sparse_attn(kv_codes, kv_scales, kv_rows_per_seq, q, idx_sets, sets,
                                                      swa_rows ? swa_kv : kv_codes, swa_rows, swa_end,
                                                      swa_window, L, B, T, H, top_k, softmax_scale, out, lse,
                                                      need ? workspace : nullptr, (hipStream_t)stream),
                             "sparse attention launch");
  return st == CSA2_OK ? ok() : st;
}

// ---------------------------------------------------------------------------- encoder chunk

namespace {

struct EncoderWs {
  void* full;          // csa2_index_full workspace (no pool), sized for k_rows entries
  size_t full_bytes;
  int32_t* topk;       // [B][T][top_k] index set of the current group (when the caller keeps none)
  int32_t* n_visible;  // [B][T]
  int32_t* swa_end;    // [B][T]
  void* attn;          // csa2_sparse_attn workspace
  size_t attn_bytes;
};

size_t carve_encoder(void* ws, int B, int T, int64_t k_rows, int layers, int H, int top_k, int swa_window,
                     EncoderWs* out) {
  Carver c{(char*)ws};
  EncoderWs w;
  w.full_bytes = csa2_index_full_workspace(B, T, (int)k_rows, csa2::kBlock, 0, top_k);
  w.full = c.take<char>(w.full_bytes);
  w.topk = c.take<int32_t>((size_t)B * T * top_k);
  w.n_visible = c.take<int32_t>((size_t)B * T);
  w.swa_end = c.take<int32_t>((size_t)B * T);
  w.attn_bytes = csa2_sparse_attn_workspace(layers, B, T, H, top_k, swa_window);
  w.attn = c.take<char>(w.attn_bytes);
  if (out) *out = w;
  return c.off;
}

}  // namespace

size_t csa2_encoder_chunk_workspace(int B, int T, int64_t k_rows, int layers, int H, int top_k, int swa_window) {
  if (B < 1 || T < 1 || T > 65535 || k_rows < 0 || k_rows > csa2::kMaxFullPositions || layers < 1 ||
      layers > csa2::kMaxLayers || H < 16 || H % 16 != 0 || top_k < 1 || top_k > csa2::kMaxTopK || swa_window < 0)
    return 0;
  // enough for every chunk of at most T tokens: the attention's split plan, and so its partial
  // states, does not grow monotonically with T
  size_t need = 0;
  for (int t = 1; t <= T; ++t) need = std::max(need, carve_encoder(nullptr, B, t, k_rows, layers, H, top_k, swa_window, nullptr));
  return need;
}

csa2_status csa2_encoder_chunk(int G, int layers, const uint16_t* new_idx_k, const uint16_t* new_latent,
                               uint8_t* idx_k, uint8_t* kv_codes, uint8_t* kv_scales, int64_t k_rows,
                               const uint16_t* idx_q, const float* head_w, const uint16_t* q,
                               const uint8_t* swa_kv, int swa_rows, int B, int T, int64_t p0, int m, int H,
                               int top_k, int swa_window, float softmax_scale, uint16_t* out, int32_t* topk_idx,
                               void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(G >= 1, CSA2_ERR_INVALID_ARG, "G must be >= 1");
  REQUIRE(layers >= 1 && layers <= csa2::kMaxLayers, CSA2_ERR_UNSUPPORTED, "layers must be in [1, %d]",
          csa2::kMaxLayers);
  REQUIRE(B >= 1 && T >= 1, CSA2_ERR_INVALID_ARG, "B and T must be >= 1");
  REQUIRE((int64_t)B * T <= 65535 && (int64_t)layers * B * T <= 65535, CSA2_ERR_UNSUPPORTED,
          "B*T and layers*B*T must be <= 65535");
  REQUIRE(m >= 1, CSA2_ERR_INVALID_ARG, "m must be >= 1");
  REQUIRE(p0 >= 0, CSA2_ERR_INVALID_ARG, "p0 must be >= 0");
  REQUIRE(swa_window >= 0 && swa_window <= 4096, CSA2_ERR_UNSUPPORTED, "swa_window must be in [0, 4096]");
  REQUIRE(k_rows >= 1 && k_rows <= csa2::kMaxFullPositions, CSA2_ERR_UNSUPPORTED, "k_rows must be in [1, %d]",
          csa2::kMaxFullPositions);
  const int64_t n_before = p0 / m, n_after = (p0 + T) / m;
  REQUIRE(n_after <= k_rows, CSA2_ERR_INVALID_ARG, "the chunk completes entries up to %lld > k_rows %lld",
          (long long)n_after, (long long)k_rows);
  const int hist = (int)std::min<int64_t>(p0, swa_window > 0 ? swa_window - 1 : 0);
  REQUIRE(swa_rows == hist + T, CSA2_ERR_INVALID_ARG, "swa_rows must be min(p0, swa_window - 1) + T = %d (got %d)",
          hist + T, swa_rows);
  REQUIRE_PTR(idx_k);
  REQUIRE_PTR(kv_codes);
  REQUIRE_PTR(kv_scales);
  REQUIRE_PTR(swa_kv);
  REQUIRE(new_latent == nullptr || aligned16(new_latent), CSA2_ERR_INVALID_ARG, "new_latent must be 16-byte aligned");
  REQUIRE(new_idx_k == nullptr || aligned16(new_idx_k), CSA2_ERR_INVALID_ARG, "new_idx_k must be 16-byte aligned");
  // everything the nested Full-layer and attention calls check, before the appends modify the
  // caches: a call that fails here has enqueued nothing
  REQUIRE_PTR(idx_q);
  REQUIRE_PTR(head_w);
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  REQUIRE(topk_idx == nullptr || aligned16(topk_idx), CSA2_ERR_INVALID_ARG, "topk_idx must be 16-byte aligned");
  REQUIRE(H >= 16 && H % 16 == 0 && H <= 1024, CSA2_ERR_UNSUPPORTED, "H must be a multiple of 16 in [16, 1024]");
  REQUIRE(top_k >= 1 && top_k <= csa2::kMaxTopK, CSA2_ERR_UNSUPPORTED, "top_k must be in [1, %d]", csa2::kMaxTopK);
  REQUIRE(softmax_scale > 0.f, CSA2_ERR_INVALID_ARG, "softmax_scale must be > 0");
  const size_t need = carve_encoder(nullptr, B, T, k_rows, layers, H, top_k, swa_window, nullptr);
  REQUIRE(workspace != nullptr && aligned16(workspace) && ws_bytes >= need, CSA2_ERR_WORKSPACE,
          "workspace of %zu bytes required (got %zu)", need, ws_bytes);
  EncoderWs w;
  carve_encoder(workspace, B, T, k_rows, layers, H, top_k, swa_window, &w);
  hipStream_t s = (hipStream_t)stream;
  csa2_status st = hip_check(csa2::launch_causal_visibility(B, T, p0, m, hist, w.n_visible, w.swa_end, s),
                             "visibility launch");
  if (st != CSA2_OK) return st;
  const int64_t n_new = n_after - n_before;
  int32_t layer_set[csa2::kMaxLayers] = {0};
  for (int g = 0; g < G; ++g) {
    const size_t gb = (size_t)g * B;
    for (int b = 0; b < B && n_new > 0; ++b) {
      const size_t row0 = (gb + b) * (size_t)k_rows + (size_t)n_before;   // first appended cache row
      const size_t src = (gb + b) * (size_t)n_new;                          // its entry in the new arrays
      if (new_idx_k) {
        st = hip_check(csa2::launch_quantize_query(new_idx_k + src * csa2::kIdxDim, idx_k + row0 * csa2::kIdxDim,
                                                   n_new * csa2::kIdxDim, s),
                       "indexer-key append launch");
        if (st != CSA2_OK) return st;
      }
      if (new_latent) {
        st = hip_check(csa2::launch_quantize_kv(new_latent + src * csa2::kKvDim, n_new,
                                                kv_codes + row0 * csa2::kKvCodeBytes,
                                                kv_scales + row0 * csa2::kKvScaleBytes, s),
                       "main-KV append launch");
        if (st != CSA2_OK) return st;
      }
    }
    int32_t* topk = topk_idx ? topk_idx + gb * T * top_k : w.topk;
    st = csa2_index_full(idx_k + gb * (size_t)k_rows * csa2::kIdxDim, nullptr, k_rows,
                         idx_q ? idx_q + gb * T * csa2::kIdxHeads * csa2::kIdxDim : nullptr,
                         head_w ? head_w + gb * T * csa2::kIdxHeads : nullptr, w.n_visible, B, T, (int)n_after,
                         csa2::kBlock, 0, top_k, nullptr, nullptr, topk, nullptr, w.full, w.full_bytes, stream);
    if (st != CSA2_OK) return st;
    const size_t lb = (size_t)g * layers * B;
    st = csa2_sparse_attn(kv_codes + gb * (size_t)k_rows * csa2::kKvCodeBytes,
                          kv_scales + gb * (size_t)k_rows * csa2::kKvScaleBytes, k_rows,
                          q ? q + lb * T * H * csa2::kKvDim : nullptr, topk, layer_set, 1,
                          swa_kv + lb * (size_t)swa_rows * csa2::kKvDim, swa_rows, w.swa_end, swa_window, layers, B,
                          T, H, top_k, softmax_scale, out ? out + lb * T * H * csa2::kKvDim : nullptr, nullptr,
                          w.attn_bytes ? w.attn : nullptr, w.attn_bytes, stream);
    if (st != CSA2_OK) return st;
  }
  return ok();
}

}  // extern "C"
