/*
 * csa2.h -- C ABI of the CSA2 decode hot path on MI355X (gfx950).
 *
 * The operations follow the DeepSeek-V4.1-Flash pages:
 *   - blog.4sapi.com, section 2 "CSA2" and its mode table: a Full layer computes its own
 *     indexer scores and Top-K; a Reindex layer reuses the Full layer's indexer K and main KV
 *     but re-scores with its own indexer query; a Reuse layer inherits the Top-K indices
 *     (so it has no entry point here: the caller passes its leader's index set).
 *   - readance.app, section 4.3, and blog.4sapi.com, section 4 "Hierarchical Sparse Indexer":
 *     the first Full indexer scans every visible position, filters by block into a shared
 *     candidate pool (2048 blocks x 8 positions = 16384), Reindex layers pick their Top-512
 *     inside the pool; the indexer has 32 query heads of dim 128.
 *   - blog.4sapi.com, section 5 "FP4 KV", and the animattoys.com FP4 section: the main KV is
 *     FP4 E2M1 with one E4M3 scale per 16 channels and no second-level scale; the sliding
 *     window (SWA) KV stays FP8.
 *
 * Readings fixed by this library where the pages are silent:
 *   - indexer score s[p] = sum_h w[h] * ReLU(q8[h] . k[p]), one 128-dim E4M3 key per position
 *     shared by the 32 heads; q8 = the bf16 query rounded to E4M3 (nearest even, saturating
 *     to +-448, unit scale);
 *   - block = 8 consecutive positions aligned at 0 (the last may be partial), block score =
 *     max of its scores; ranking ties go to the lower block / position index; scores rank as
 *     float32 with -0 equal to +0;
 *   - index outputs list positions in ascending order with -1 padding;
 *   - attention: one softmax over the selected main-KV rows and the window's SWA rows,
 *     keys = values (a shared 512-wide latent), no sink, no bias.
 *
 * Indexer keys, in every call that reads them (idx_k, idx_k_scales):
 *   - idx_k_scales == NULL: idx_k is [B][k_rows_per_seq][128] E4M3 bytes;
 *   - otherwise the FP4 variant (animattoys.com, FP4 section: the V4 indexer kept its queries
 *     and keys in FP4): idx_k is [B][k_rows_per_seq][64] E2M1 code bytes (channel 2i in the
 *     low nibble of byte i) and idx_k_scales [B][k_rows_per_seq][8] E4M3 scales, scale g
 *     covering channels 16g..16g+15; a key is code x scale (exact), 72 bytes per position
 *     instead of 128.  With FP4 keys the bf16 indexer query is rounded to FP4 in the same
 *     format instead of to E4M3: per head and 16-channel group, scale = E4M3(amax / 6) and
 *     code = E2M1(x / scale) (the rule of csa2_quantize_kv_fp4).
 *
 * Conventions for every call:
 *   - tensor arguments are DEVICE pointers owned by the caller (except where marked host),
 *     row-major and contiguous; they must be 16-byte aligned;
 *   - bf16 tensors are passed as uint16_t bit patterns;
 *   - `stream` is a hipStream_t (NULL = the default stream); work is enqueued asynchronously;
 *   - argument checks run on the host, never read device memory, and return
 *     CSA2_ERR_INVALID_ARG / CSA2_ERR_UNSUPPORTED / CSA2_ERR_WORKSPACE before anything is
 *     enqueued; a failed launch returns CSA2_ERR_HIP; csa2_last_error() then describes it;
 *   - the library keeps no state between calls; concurrent calls need distinct workspaces;
 *   - device-side data outside its documented range (n_visible beyond n_max, positions
 *     outside the cache, NaN codes) is clamped or ignored, never read out of bounds, and
 *     otherwise gives unspecified results.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misaligned pointer */
  CSA2_ERR_UNSUPPORTED = 2,   /* a shape this build does not implement */
  CSA2_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace() size */
  CSA2_ERR_HIP = 4            /* a HIP launch failed */
} csa2_status;

#define CSA2_IDX_HEADS 32   /* indexer query heads */
#define CSA2_IDX_DIM 128    /* indexer head dim = indexer-K row bytes (E4M3) */
#define CSA2_KV_DIM 512     /* main-KV latent width (keys = values) */
#define CSA2_KV_CODE_BYTES 256
#define CSA2_KV_SCALE_BYTES 32

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char* csa2_last_error(void);

/* Indexer query preparation on its own. in_bf16[n] -> out_e4m3[n], round to nearest even,
 * saturating to +-448, NaN -> 0x7F. csa2_index_full / csa2_reindex apply the same rounding
 * internally; this entry exists to verify it and for callers that keep E4M3 queries. */
csa2_status csa2_quantize_query(const uint16_t* in_bf16, uint8_t* out_e4m3, int64_t n, void* stream);

/* Main-KV quantisation, the producer of the cache csa2_sparse_attn reads (blog.4sapi.com sec.5
 * "FP4 KV"; animattoys.com FP4 section: E2M1 codes with one E4M3 scale per 16 channels, applied
 * to the latent after rotation, no second-level scale).  The scale rule is this library's
 * reading (the pages give none): per group of 16 channels, scale = E4M3(amax / 6) and
 * code = E2M1(x / scale), both quotients rounded to binary32 first, nearest-even and saturating
 * conversions, the sign kept (-0 gives the negative-zero code); a group whose scale byte is 0
 * stores code 0 throughout.
 *   latent_bf16 [rows][512] bf16 (rotated latent rows)
 *   kv_codes    [rows][256] uint8 out, channel 2i in the low nibble of byte i
 *   kv_scales   [rows][32]  uint8 out (E4M3), scale g covers channels 16g..16g+15
 * To append to a cache, pass kv_codes / kv_scales offset to the first row to write.
 * NaN inputs give unspecified bytes.  Supported: 0 <= rows <= 2^31. */
csa2_status csa2_quantize_kv_fp4(const uint16_t* latent_bf16, int64_t rows, uint8_t* kv_codes, uint8_t* kv_scales,
                                 void* stream);

/* Query preparation and the Full scan on their own: every visible position's score, no selection.
 *   idx_k, idx_k_scales  indexer keys, E4M3 or FP4 (see above)
 *   idx_q      [B][T][32][128] bf16 indexer queries
 *   head_w     [B][T][32] float head weights
 *   n_visible  [B][T] int32 visible positions of each query (clamped to [0, n_max])
 *   scores     [B][T][n_max] float out; entries at or beyond n_visible are left untouched
 * Requires n_max <= k_rows_per_seq. */
csa2_status csa2_index_scores(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                              const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                              float* scores, void* stream);

/* Full layer (blog.4sapi.com sec.4; readance.app sec.4.2/4.3): score every visible position,
 * keep the top `pool_blocks` blocks of `block_size` positions by block score as the candidate
 * pool, and take the Top-`top_k` positions of the pool.  With pool_blocks == 0 there is no
 * pool and the Top-K runs over every visible position (an encoder Full layer).
 *   pool_pos   [B][T][pool_blocks*block_size] int32 out (ascending, -1 after pool_len), or NULL
 *              when pool_blocks == 0
 *   pool_len   [B][T] int32 out (pool entries), or NULL when pool_blocks == 0
 *   topk_idx   [B][T][top_k] int32 out (ascending positions, -1 padded)
 *   topk_score [B][T][top_k] float out aligned with topk_idx (0 for padding), or NULL
 *   workspace  device scratch of at least csa2_index_full_workspace(...) bytes
 * Supported: block_size == 8, 1 <= top_k <= 2048, top_k <= pool_blocks*block_size when
 * pool_blocks > 0, pool_blocks*block_size <= 16384, n_max <= 2^21 (2^23 for csa2_index_scores),
 * n_max <= k_rows_per_seq.
 * csa2_index_full works through the queries in batches whose scores, block keys and lists fit in
 * about 48 MiB (runs of a multiple of 16 queries of one sequence, or whole sequences), reusing
 * one batch's workspace, so its workspace does not grow with the number of queries beyond one
 * batch; the results are those of one pass over every query. */
size_t csa2_index_full_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k);
/* Workspace of the separate stages below, which carry every query's scores and block keys from
 * one call to the next (the unbatched intermediates of csa2_index_full). */
size_t csa2_index_stages_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k);

/* The stages of csa2_index_full as separate calls.  They take the same arguments and the same
 * workspace of csa2_index_stages_workspace(...) bytes, which carries the scan's scores and block
 * keys (and, with pool_blocks == 0, the internal pool) from one stage to the next; enqueue them in
 * this order with identical shape arguments.  csa2_index_pool and csa2_index_topk may run on different streams as long as
 * each starts after the previous stage has finished (e.g. the Top-K of the Full layer on one
 * stream while csa2_reindex scores the same pool on another).
 *   csa2_index_scan:   query preparation, the scan and the block maxima
 *                      (reads idx_k, idx_q, head_w, n_visible)
 *   csa2_index_pool:   the candidate pool (reads n_visible and the workspace; writes pool_pos
 *                      and pool_len, which may be NULL only when pool_blocks == 0)
 *   csa2_index_topk:   the Top-K over the pool (reads the workspace and the pool)
 *   csa2_index_select: the pool and its Top-K in one pass (same results as csa2_index_pool
 *                      followed by csa2_index_topk) */
csa2_status csa2_index_scan(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                            const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                            int block_size, int pool_blocks, int top_k,
                            void* workspace, size_t ws_bytes, void* stream);

/* csa2_index_scan with another block score for the pool (the block-score variants a study of
 * the hierarchical indexer's recall compares; alphalab.site sec."2. CSA2" names pool misses,
 * the candidates the first Full layer's pool leaves out, as the method's risk).  block_score:
 * 0 = the largest visible score of the block (csa2_index_scan), 1 = the sum of its visible
 * scores, 2 = the mean of its two largest visible scores (one visible position: that score).
 * The later stages (csa2_index_pool, csa2_index_select, csa2_index_select_reindex) rank blocks by
 * whichever score the scan left in the workspace.  With 1 or 2 the Full layer's Top-K over the
 * pool need not equal its Top-K over every position. */
csa2_status csa2_index_scan_blocks(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq,
                                   const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int B,
                                   int T, int n_max, int block_size, int pool_blocks, int top_k, int block_score,
                                   void* workspace, size_t ws_bytes, void* stream);
csa2_status csa2_index_pool(const int32_t* n_visible, int B, int T, int n_max,
                            int block_size, int pool_blocks, int top_k,
                            int32_t* pool_pos, int32_t* pool_len,
                            void* workspace, size_t ws_bytes, void* stream);
csa2_status csa2_index_topk(int B, int T, int n_max, int block_size, int pool_blocks, int top_k,
                            const int32_t* pool_pos, const int32_t* pool_len,
                            int32_t* topk_idx, float* topk_score,
                            void* workspace, size_t ws_bytes, void* stream);
csa2_status csa2_index_select(const int32_t* n_visible, int B, int T, int n_max,
                              int block_size, int pool_blocks, int top_k,
                              int32_t* pool_pos, int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                              void* workspace, size_t ws_bytes, void* stream);

csa2_status csa2_index_full(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                            const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                            int block_size, int pool_blocks, int top_k,
                            int32_t* pool_pos, int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                            void* workspace, size_t ws_bytes, void* stream);

/* Reindex layers (blog.4sapi.com sec.2 mode table and sec.4; alphalab.site sec."2. CSA2"):
 * for each of L layers, re-score only the pool positions with the layer's own indexer query
 * and weights, then take its own Top-`top_k`.  Positions outside the pool are never picked.
 *   idx_q      [L][B][T][32][128] bf16;  head_w [L][B][T][32] float
 *   pool_pos   [B][T][pool_cap] int32 distinct positions in ascending order (as csa2_index_full
 *              writes them; the Top-K output keeps the pool's order); entries >= pool_len and
 *              negative or out-of-range entries are ignored; a position listed more than once
 *              ranks with its copies counted, so it can be selected more than once (copies at
 *              the top_k-th place fill the remaining places in slot order); pool_len [B][T] int32
 *   topk_idx   [L][B][T][top_k] int32 out; topk_score [L][B][T][top_k] float out or NULL
 * Supported: 1 <= top_k <= 2048, top_k <= pool_cap <= 16384. */
size_t csa2_reindex_workspace(int L, int B, int T, int pool_cap, int top_k);
csa2_status csa2_reindex(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                         const float* head_w, const int32_t* pool_pos, const int32_t* pool_len,
                         int pool_cap, int L, int B, int T, int top_k,
                         int32_t* topk_idx, float* topk_score,
                         void* workspace, size_t ws_bytes, void* stream);

/* The indexer of one decode step (blog.4sapi.com sec.2 mode table and sec.4; readance.app
 * sec.4.2/4.3): the Full layer (scan, candidate pool, its Top-K) followed by L Reindex layers over
 * that pool, with the results csa2_index_full followed by csa2_reindex on its pool would give.
 * The Full layer's Top-K is taken in the same launch as the Reindex layers' Top-K, since both
 * only need the pool.  Arguments as for csa2_index_full and csa2_reindex:
 *   idx_q, head_w        the Full layer's indexer query [B][T][32][128] bf16 and weights [B][T][32]
 *   ri_q, ri_w           [L][B][T][32][128] bf16 and [L][B][T][32] float (unused when L == 0)
 *   pool_pos, pool_len   the pool, out ([B][T][pool_blocks*8] and [B][T])
 *   topk_idx, topk_score the Full layer's Top-K, out ([B][T][top_k]; topk_score may be NULL)
 *   ri_topk_idx, ri_topk_score  the Reindex layers' Top-K, out ([L][B][T][top_k]; score may be NULL)
 *   workspace            at least csa2_index_chain_workspace(...) bytes; it starts with the
 *                        csa2_index_full workspace, so csa2_index_scan accepts it too
 * csa2_index_select_reindex is csa2_index_chain without the scan: call it after csa2_index_scan
 * on the same workspace (it reads the scan's results from there).
 * Supported: as csa2_index_full with pool_blocks >= 1, L >= 0 and (L+1)*B*T <= 65535. */
size_t csa2_index_chain_workspace(int B, int T, int n_max, int block_size, int pool_blocks, int top_k, int L);
csa2_status csa2_index_chain(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const uint16_t* idx_q,
                             const float* head_w, const int32_t* n_visible, int B, int T, int n_max,
                             int block_size, int pool_blocks, int top_k, const uint16_t* ri_q, const float* ri_w,
                             int L, int32_t* pool_pos, int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                             int32_t* ri_topk_idx, float* ri_topk_score, void* workspace, size_t ws_bytes,
                             void* stream);
csa2_status csa2_index_select_reindex(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq, const int32_t* n_visible,
                                      int B, int T, int n_max, int block_size, int pool_blocks, int top_k,
                                      const uint16_t* ri_q, const float* ri_w, int L, int32_t* pool_pos,
                                      int32_t* pool_len, int32_t* topk_idx, float* topk_score,
                                      int32_t* ri_topk_idx, float* ri_topk_score, void* workspace,
                                      size_t ws_bytes, void* stream);

/* csa2_index_chain for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops and harnesses that forbid hipMalloc.  The same arguments and
 * results as csa2_index_chain without the workspace: its scratch is a fixed array of this library
 * in device memory, CSA2_NOALLOC_SCRATCH_BYTES (16 MiB) on every GPU it runs on, held until the
 * process ends; the call itself allocates nothing (the first call on a device looks up the
 * address of that device's array; callers that capture graphs make one call before capturing).
 *   - a shape whose csa2_index_chain_workspace(...) exceeds CSA2_NOALLOC_SCRATCH_BYTES returns
 *     CSA2_ERR_UNSUPPORTED before anything is enqueued (the 1M-position decode of one query and
 *     8 queries over 128K positions, each with 4 Reindex layers, need about 5 and 7 MiB);
 *   - argument errors are those of csa2_index_chain;
 *   - every call on one GPU uses that GPU's one array, so calls that may overlap on a GPU
 *     (another stream, another thread) race on it and must be serialised by the caller.
 * csa2_noalloc_scratch_bytes() returns CSA2_NOALLOC_SCRATCH_BYTES. */
#define CSA2_NOALLOC_SCRATCH_BYTES (16u << 20)
size_t csa2_noalloc_scratch_bytes(void);
csa2_status csa2_index_chain_noalloc(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq,
                                     const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int B,
                                     int T, int n_max, int block_size, int pool_blocks, int top_k,
                                     const uint16_t* ri_q, const float* ri_w, int L, int32_t* pool_pos,
                                     int32_t* pool_len, int32_t* topk_idx, float* topk_score, int32_t* ri_topk_idx,
                                     float* ri_topk_score, void* stream);

/* Sparse attention of L layers (blog.4sapi.com sec.2 and sec.5; alphalab.site sec."3. FP4"):
 * layer l attends, per query and head, over the main-KV rows of index set layer_set[l]
 * (FP4 E2M1 codes x E4M3 per-16-channel scales, dequantised exactly) followed by its own SWA
 * rows [max(0, swa_end - swa_window), swa_end), with one softmax over both segments.
 *   kv_codes   [B][kv_rows_per_seq][256] uint8, channel 2i in the low nibble of byte i
 *   kv_scales  [B][kv_rows_per_seq][32]  uint8 E4M3, scale g covers channels 16g..16g+15
 *   q          [L][B][T][H][512] bf16 (already rotated)
 *   idx_sets   [S][B][T][top_k] int32 positions (negative / out-of-range entries are empty)
 *   layer_set  HOST [L] int32 set id of each layer (a Reuse layer names its leader's set)
 *   swa_kv     [L][B][swa_rows][512] E4M3 (unit scale)
 *   swa_end    [B][T] int32 exclusive end row of each query's window (clamped to [0, swa_rows])
 *   out        [L][B][T][H][512] bf16 out;  lse [L][B][T][H] float out (natural log) or NULL;
 *              a query with no rows at all gets out = 0 and lse = -inf
 *   workspace  device scratch of csa2_sparse_attn_workspace(...) bytes (may be 0: then NULL is fine)
 * Supported: H % 16 == 0, 1 <= top_k <= 2048, 0 <= swa_window <= 4096, L <= 64. */
size_t csa2_sparse_attn_workspace(int L, int B, int T, int H, int top_k, int swa_window);
csa2_status csa2_sparse_attn(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t kv_rows_per_seq,
                             const uint16_t* q, const int32_t* idx_sets, const int32_t* layer_set, int S,
                             const uint8_t* swa_kv, int swa_rows, const int32_t* swa_end, int swa_window,
                             int L, int B, int T, int H, int top_k, float softmax_scale,
                             uint16_t* out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* One chunk of an encoder prefill through the encoder's CSA2 groups (blog.4sapi.com sec.3, the
 * encoder's layers 3-20: three groups of six, one Full layer and five Reuse layers, over a
 * sequence compressed m = 2 tokens per entry; animattoys.com, the mode configuration of the
 * encoder and decoder; alphalab.site sec."2. CSA2": the hierarchical indexer is decoder-only, so
 * an encoder Full layer ranks every visible entry).  The chunk holds the tokens at positions
 * p0 .. p0+T-1 of B sequences.  For each group g in turn it
 *   1. appends the entries the chunk completes, cache rows [floor(p0/m), floor((p0+T)/m)): the
 *      indexer keys rounded to E4M3 (as csa2_quantize_query) and the main KV quantised to FP4 (as
 *      csa2_quantize_kv_fp4);
 *   2. runs the Full layer: token t scores the floor((p0+t+1)/m) entries visible to it (an entry
 *      is visible once all m of its tokens are at or before the token) and keeps its Top-top_k,
 *      as csa2_index_full with pool_blocks == 0;
 *   3. runs the attention of the group's `layers` layers, which all use that index set (the Full
 *      layer and its Reuse layers), each with its own sliding window, as csa2_sparse_attn.
 * Arguments (n_new = floor((p0+T)/m) - floor(p0/m) entries per sequence and group):
 *   new_idx_k   [G][B][n_new][128] bf16 new indexer-key entries, or NULL (caches already hold them)
 *   new_latent  [G][B][n_new][512] bf16 new main-KV entries (rotated), 16-byte aligned, or NULL
 *   idx_k       [G][B][k_rows][128] E4M3 indexer-key caches, appended in place
 *   kv_codes    [G][B][k_rows][256], kv_scales [G][B][k_rows][32] main-KV caches, appended in place
 *   idx_q       [G][B][T][32][128] bf16 indexer queries;  head_w [G][B][T][32] float
 *   q           [G][layers][B][T][H][512] bf16 attention queries
 *   swa_kv      [G][layers][B][swa_rows][512] E4M3 window rows: row r holds the token at position
 *               p0 - hist + r, hist = min(p0, swa_window - 1), swa_rows = hist + T
 *   out         [G][layers][B][T][H][512] bf16 out
 *   topk_idx    [G][B][T][top_k] int32 out (each group's index set, ascending, -1 padded) or NULL
 *   workspace   device scratch of csa2_encoder_chunk_workspace(...) bytes, 16-byte aligned; a size
 *               queried for T tokens serves every chunk of at most T tokens
 * Work is enqueued on `stream` in group order; the caches must not be read or written by other
 * work in the meantime.  Supported: m >= 1, floor((p0+T)/m) <= k_rows <= 2^21,
 * layers*B*T <= 65535, H % 16 == 0, 1 <= top_k <= 2048, 0 <= swa_window <= 4096. */
size_t csa2_encoder_chunk_workspace(int B, int T, int64_t k_rows, int layers, int H, int top_k, int swa_window);
csa2_status csa2_encoder_chunk(int G, int layers, const uint16_t* new_idx_k, const uint16_t* new_latent,
                               uint8_t* idx_k, uint8_t* kv_codes, uint8_t* kv_scales, int64_t k_rows,
                               const uint16_t* idx_q, const float* head_w, const uint16_t* q,
                               const uint8_t* swa_kv, int swa_rows, int B, int T, int64_t p0, int m, int H,
                               int top_k, int swa_window, float softmax_scale, uint16_t* out, int32_t* topk_idx,
                               void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
