// Host-side launchers of the CSA2 kernels (each defined next to its kernel).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kScanThreads = 256;      // Reindex scoring
constexpr int kFullThreads = 1024;     // Full scan: one workgroup of 16 waves per chunk
constexpr int kSelectThreads = 1024;
constexpr int kAttnThreads = 256;
constexpr int kMaxLayers = 64;
constexpr int kListLen = 16;           // keys of a chunk list (pool scan chunks, scored pool chunks)

struct LayerSets { int32_t set[kMaxLayers]; };

// scan.hip
hipError_t launch_quantize_query(const uint16_t* in, uint8_t* out, int64_t n, hipStream_t s);
int scan_chunk_positions(int n_max, int queries);
// Block score of the pool (see block_key in scan.hip).
constexpr int kBlockMax = 0, kBlockSum = 1, kBlockTop2 = 2;
// Sequences with at least kScanMqMinT queries and at most kMqMaxPositions positions share key
// tiles between 16 queries per workgroup (k_idx_scan_mq), in chunks of at most kMqMaxChunk.
constexpr int kScanMqMinT = 8;
constexpr int kMqMaxChunk = 4096;
constexpr int kMqMaxPositions = 256 * kMqMaxChunk;   // 4096 units per query
bool scan_multi_query(int T, int n_max);
int scan_mq_chunk(int n_max, int B, int T);
constexpr int kScanUnitsPerWg = kFullThreads / 64;   // 16 waves per chunk, each with upw units of the
                                                     // pool's unit lists (chunk/(16*upw) positions each)
constexpr int kMaxFullPositions = 1 << 21;           // 256 chunks of 8192 per query: 4096 units
// Indexer keys: idx_ks == null: E4M3 idx_k [rows][128]; otherwise FP4 codes idx_k [rows][64] and
// E4M3 scales idx_ks [rows][8] (one per 16 channels).
// With clists non-null (one-query scan, one unit per wave) each chunk also leaves its 16 best
// blocks and a cut (k_idx_scan's chunk list) in clists[q][chunk][16] and ccuts[q][chunk].
hipError_t launch_idx_scan(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, const int32_t* n_visible, int Q, int T, int n_max,
                           float* scores, uint32_t* blkkey, int nb_max, uint64_t* lists,
                           uint64_t* cuts, int chunk, int n_wg, bool multi_query, int block_score, int upw,
                           uint64_t* clists, uint64_t* ccuts, hipStream_t s);
// Reindex scoring of pool slots in chunks of kRiChunk (and, for the first full_items items, the
// Full layer's query over the same slots); scores by slot (see k_ri_score).
constexpr int kRiChunk = 128;
__host__ __device__ inline int ri_chunks(int pool_cap) { return (pool_cap + kRiChunk - 1) / kRiChunk; }
hipError_t launch_ri_score(const uint8_t* idx_k, const uint8_t* idx_ks, int64_t k_rows, const uint16_t* idx_q,
                           const float* head_w, int full_items, const uint16_t* full_q, const float* full_w,
                           const int32_t* pool_pos, const int32_t* pool_len, int pool_cap, int L, int Q, int T,
                           float* slot_scores, hipStream_t s);

// select.hip
// Pool of the top P blocks (positions ascending, -1 padded to cap_out), one WG per query.
// Without chunk lists, queries whose block-key rows (nb_max) hold at most kDensePoolBlocks keys are
// pooled over every block key; longer ones from the unit lists.
// With K > 0 the same WG then takes the Top-K of the pool from the scan's scores.
// With clists non-null the pool is selected from the scan's chunk lists (n_chunks chunks of
// blocks_per_chunk blocks per query), and over every block key when too many chunks would have
// to be re-read; a Top-K with K > 0 then follows as a second launch.
hipError_t launch_pool(const uint64_t* lists, const uint64_t* cuts, int n_units, int blocks_per_unit,
                       const uint64_t* clists, const uint64_t* ccuts, int n_chunks, int blocks_per_chunk,
                       const uint32_t* blkkey, int nb_max, const int32_t* n_visible, int n_max, int P,
                       int32_t* pool_pos, int cap_out, int32_t* pool_len, const float* scores, int K,
                       int32_t* topk_idx, float* topk_score, int Q, hipStream_t s);
// Top-K over candidate lists.  Candidate slot i of item it has position cand_pos[(it % Q)*cap + i]
// (slots >= cand_len[it % Q] are empty).  One kind of Top-K item: `items` items (it = l*Q + q);
// by position, the score of a candidate at position p is scores[q*score_stride + p], otherwise
// that of slot i is scores[it*score_stride + i]; positions >= n_rows are ignored.
struct TopkJob {
  const float* scores;
  int64_t score_stride, n_rows;
  int by_position, items;
  int32_t* out_idx;      // [items][k]
  float* out_score;      // [items][k] or null
};
// Items of job a, then items of job b (b.items may be 0), in one launch.
hipError_t launch_topk(const int32_t* cand_pos, const int32_t* cand_len, int cap, int Q, int k,
                       const TopkJob& a, const TopkJob& b, hipStream_t s);

// encoder.hip
// n_visible[b][t] = floor((p0 + t + 1) / m), swa_end[b][t] = hist + t + 1.
hipError_t launch_causal_visibility(int B, int T, int64_t p0, int m, int hist, int32_t* n_visible,
                                    int32_t* swa_end, hipStream_t s);

// kvquant.hip
hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales, hipStream_t s);

// attn.hip
struct AttnPlan {
  int heads_per_wg;    // 64 (k_sparse_attn_wide) when H % 64 == 0, else 16
  int split_rows, n_splits;
  size_t ws_bytes;     // partial states when the rows are split over several workgroups
};
AttnPlan plan_attn(int L, int B, int T, int H, int k, int window);
hipError_t launch_sparse_attn(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t kv_rows,
                              const uint16_t* q, const int32_t* idx_sets, const LayerSets& sets,
                              const uint8_t* swa, int swa_rows, const int32_t* swa_end, int window,
                              int L, int B, int T, int H, int k, float scale, uint16_t* out,
                              float* lse, void* workspace, hipStream_t s);

}  // namespace csa2
