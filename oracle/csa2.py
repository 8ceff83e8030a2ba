"""Plain CPU reference of the CSA2 hot path (Full indexer, candidate pool, Top-K,
Reindex, Reuse, sparse attention with the sliding-window segment).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library.

Sources (DeepSeek-V4.1-Flash pages):
  [p1 4.2]  readance.app, section 4.2 "Full / Reindex / Reuse": per-layer static modes.
  [p1 4.3]  readance.app, section 4.3 "Hierarchical Sparse Indexer".
  [p2 2]    blog.4sapi.com, section 2 "CSA2" and its mode table (Main KV / Indexer K / Top-K).
  [p2 4]    blog.4sapi.com, section 4 "Hierarchical Sparse Indexer": the first Full indexer
            scans the visible context, filters positions by block into a shared pool; Reindex
            layers pick their own Top-512 inside it; 32 query heads, head dim 128.
  [p3 CSA2] animattoys.com, CSA2 section: pool example of 2048 blocks x 8 positions = 16384.
  [p5 2]    alphalab.site, section "2. CSA2": only the decoder's first Full layer builds the pool.
  [p2 5]    blog.4sapi.com, section 5 "FP4 KV": main KV in E2M1 with one E4M3 scale per 16
            channels, SWA KV in FP8.
  [p2 3]    blog.4sapi.com, section 3 (how CSA2 is laid out): the encoder's layers 3-20 form three
            groups of six, one Full and five Reuse layers, over a sequence compressed m = 2
            tokens per entry.
  [p3 FP4]  animattoys.com, FP4 section: V4 already stored the indexer's queries and keys in
            FP4; the main KV now too, as E2M1 with one E4M3 scale per 16 channels.
  [p3 modes] animattoys.com, the mode configuration: encoder groups of one Full then five Reuse
            layers; decoder groups with Reindex layers.

Readings where the pages are silent (each one is listed in the design notes):
  * indexer score  s[p] = sum_h w_h * ReLU(q_h . k_p), with one 128-dim key per position
    shared by the 32 query heads, and the query rounded to E4M3 (round to nearest even,
    saturating, unit scale) before the product; with FP4 keys the query is rounded to FP4 in
    the keys' format instead (E2M1 codes, one E4M3 scale per 16 channels);
  * block score = max of the block's scores; blocks are 8 consecutive positions aligned
    at 0, the last one may be partial;
  * ranking ties: (score descending, index ascending), for blocks and for positions;
  * the ranking decision is taken on the score rounded to float32 (the precision the
    GPU kernels rank in); -0 counts as +0;
  * outputs list positions in ascending order, padded with -1;
  * attention: one softmax over the selected main-KV rows and the window's SWA rows,
    keys equal values (one shared 512-wide latent), scale 1/sqrt(512), no sink or bias;
    an empty row set gives a zero output.

Floating point: dot products of E4M3 values are exact in float64 (every product is an
integer multiple of 2^-18 below 2^36 * 2^-18, and a 128-term sum stays below 2^43 of
those units), so the only roundings are in the head-weighted sum (float64) and in
the final cast to float32 used for ranking.  Attention is computed in float64.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .formats import bf16_value, e4m3_from_value, e4m3_value, kv_quantize_rows, kv_row_values

IDX_HEADS = 32
IDX_DIM = 128
KV_DIM = 512


# ---------------------------------------------------------------- indexer (Full / Reindex)

def quantize_query(q_bf16: np.ndarray) -> np.ndarray:
    """Indexer query prep: bf16 [32][128] -> E4M3 bytes [32][128] (RNE, saturate, unit scale)."""
    return e4m3_from_value(bf16_value(q_bf16))


def quantize_query_fp4(q_bf16: np.ndarray):
    """Indexer query prep for FP4 keys ([p3 FP4]: the V4 indexer kept its queries and keys in
    FP4): bf16 [..., 32, 128] -> (E2M1 codes [..., 32, 64], E4M3 scales [..., 32, 8]) in the
    keys' format, each head's 16-channel group quantised as a main-KV group is (scale
    E4M3(amax/6), codes E2M1 of x/scale; `formats.kv_quantize_rows`)."""
    bits = np.asarray(q_bf16, dtype=np.uint16)
    lead = bits.shape[:-2]
    rows = bits.reshape(lead + (IDX_HEADS * IDX_DIM // KV_DIM, KV_DIM))   # 4 heads per 512-wide row
    codes, scales = kv_quantize_rows(rows)
    return (codes.reshape(lead + (IDX_HEADS, IDX_DIM // 2)), scales.reshape(lead + (IDX_HEADS, IDX_DIM // 16)))


def query_for_keys(q_bf16: np.ndarray, k):
    """The query prep that goes with the indexer K's storage form: E4M3 bytes for E4M3 keys, the
    FP4 pair for FP4 keys (see k_values)."""
    return quantize_query_fp4(q_bf16) if isinstance(k, tuple) else quantize_query(q_bf16)


def query_values(q8) -> np.ndarray:
    """Prepared query -> float64 [32][128]: E4M3 bytes, or the FP4 pair (code x scale, exact)."""
    if isinstance(q8, tuple):
        return kv_row_values(q8[0], q8[1])
    return e4m3_value(q8)


def k_rows(k, sel):
    """Rows `sel` (a slice or index array) of an indexer K in either storage form: E4M3 bytes
    [n][128], or the FP4 variant (codes [n][64], scales [n][8])."""
    if isinstance(k, tuple):
        return (k[0][sel], k[1][sel])
    return k[sel]


def k_count(k) -> int:
    return (k[0] if isinstance(k, tuple) else k).shape[0]


def k_values(k) -> np.ndarray:
    """Indexer K rows -> float64 [n][128].  E4M3 bytes decode directly.  The FP4 variant
    ([p2 4]: the V4 indexer used FP4 keys; stored like the main KV, E2M1 codes with one E4M3
    scale per 16 channels, channel 2i in the low nibble of byte i) decodes to code x scale,
    exact in float64."""
    if isinstance(k, tuple):
        return kv_row_values(k[0], k[1])
    return e4m3_value(k)


def indexer_scores(k8, q8: np.ndarray, w: np.ndarray) -> np.ndarray:
    """s[p] = sum_h w[h] * max(0, q8[h] . k[p])  in float64, for every row p of k.

    k: indexer K rows, E4M3 bytes [n][128] or the FP4 pair (see k_values); q8 the prepared
    query (query_values: E4M3 bytes [32][128] or the FP4 pair), w [32] head weights.  [p1 4.2],
    [p2 2]: Full and Reindex layers score indexer K with their own indexer Q.  Rows are
    processed in independent chunks only to bound memory.  Every product q8 * k is exact in
    float64 (at most 12 significant bits) and so is the 128-term sum.
    """
    qv = query_values(q8)                                 # [32][128] float64
    wv = np.asarray(w, dtype=np.float32).astype(np.float64)
    n = k_count(k8)
    out = np.empty(n, np.float64)
    step = 1 << 16
    for r0 in range(0, n, step):
        kv = k_values(k_rows(k8, slice(r0, r0 + step)))   # [n][128] float64
        d = kv @ qv.T                                     # [n][32], exact
        out[r0:r0 + step] = np.maximum(d, 0.0) @ wv
    return out


def ranking_scores(s: np.ndarray) -> np.ndarray:
    """The value the selection ranks by: the score rounded to float32, with -0 made +0."""
    return np.asarray(s, dtype=np.float64).astype(np.float32) + np.float32(0.0)


BLOCK_SCORES = ("max", "sum", "top2")


def block_scores(s32: np.ndarray, n_vis: int, block: int, mode: str = "max") -> np.ndarray:
    """blk[j] over the scores of block j = positions [j*block, min((j+1)*block, n_vis)):
      max   the largest (the pool's block score, reading S4);
      sum   the sum of the block's scores;
      top2  the mean of its two largest scores (the score itself for a one-position block).
    The sum and the mean are taken in float64 and rounded to float32, the ranking precision (R1).
    The last two are variants for the recall study of the hierarchical indexer ([p5 2]: the
    pool's misses are the method's risk)."""
    nb = -(-n_vis // block)
    blk = np.empty(nb, np.float32)
    for j in range(nb):
        v = s32[j * block:min((j + 1) * block, n_vis)].astype(np.float64)
        if mode == "max":
            blk[j] = v.max()
        elif mode == "sum":
            blk[j] = np.float32(v.sum())
        elif mode == "top2":
            t = np.sort(v)[::-1][:2]
            blk[j] = np.float32(t.mean())
        else:
            raise ValueError(mode)
    return blk


def rank_order(keys: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Indices that order (keys descending, ids ascending)."""
    return np.lexsort((ids, -np.asarray(keys, dtype=np.float64)))


def candidate_pool(blk: np.ndarray, n_vis: int, block: int, pool_blocks: int) -> np.ndarray:
    """[p2 4], [p3 CSA2], [p5 2]: keep at most pool_blocks blocks, ranked by block score
    (ties: lower block first); the pool is their visible positions in ascending order."""
    nb = blk.shape[0]
    if nb <= pool_blocks:
        chosen = np.arange(nb)
    else:
        chosen = np.sort(rank_order(blk, np.arange(nb))[:pool_blocks])
    pos = [np.arange(j * block, min((j + 1) * block, n_vis)) for j in chosen]
    return (np.concatenate(pos) if pos else np.zeros(0, np.int64)).astype(np.int32)


def top_k(cand: np.ndarray, s32_cand: np.ndarray, k: int) -> np.ndarray:
    """Top-k candidate positions by (score descending, position ascending), listed in
    ascending position order and padded with -1 to length k."""
    cand = np.asarray(cand, dtype=np.int64)
    sel = np.sort(cand[rank_order(s32_cand, cand)[:k]])
    out = np.full(k, -1, np.int32)
    out[:sel.shape[0]] = sel
    return out


def full_layer(k8_seq: np.ndarray, q_bf16: np.ndarray, w: np.ndarray, n_vis: int,
               block: int, pool_blocks: int, k: int, block_score: str = "max") -> Dict[str, np.ndarray]:
    """One query of a Full layer: score every visible position, build the block pool
    (pool_blocks > 0) and take the Top-k over the pool ([p1 4.2], [p2 4]).  With
    pool_blocks == 0 there is no pool and the Top-k runs over every visible position."""
    q8 = query_for_keys(q_bf16, k8_seq)
    s = indexer_scores(k_rows(k8_seq, slice(0, n_vis)), q8, w)
    s32 = ranking_scores(s)
    if pool_blocks > 0:
        pool = candidate_pool(block_scores(s32, n_vis, block, block_score), n_vis, block, pool_blocks)
        cand = pool
    else:
        pool = None
        cand = np.arange(n_vis, dtype=np.int32)
    idx = top_k(cand, s32[cand], k)
    sel = idx[idx >= 0]
    return {"scores": s, "scores32": s32, "pool": pool, "topk": idx,
            "topk_score": np.concatenate([s[sel], np.zeros(k - sel.shape[0])])}


def reindex_layer(k8_seq: np.ndarray, q_bf16: np.ndarray, w: np.ndarray,
                  pool: np.ndarray, k: int) -> Dict[str, np.ndarray]:
    """One query of a Reindex layer: re-score only the pool positions with the layer's own
    indexer query and weights, then take its own Top-k ([p1 4.2], [p2 4], [p5 2])."""
    pool = np.asarray(pool, dtype=np.int64)
    q8 = query_for_keys(q_bf16, k8_seq)
    s = indexer_scores(k_rows(k8_seq, pool), q8, w)
    s32 = ranking_scores(s)
    idx = top_k(pool, s32, k)
    pos_to_score = dict(zip(pool.tolist(), s.tolist()))
    sc = np.array([pos_to_score[p] if p >= 0 else 0.0 for p in idx.tolist()])
    return {"scores": s, "topk": idx, "topk_score": sc}


# ---------------------------------------------------------------- sparse attention

def attention_rows(kv_codes_seq: np.ndarray, kv_scales_seq: np.ndarray, idx: np.ndarray,
                   swa_layer_seq: np.ndarray, swa_end: int, window: int) -> np.ndarray:
    """The row set one query attends over: the selected main-KV rows (FP4, exact dequant)
    followed by the SWA rows [max(0, swa_end - window), swa_end) of the layer ([p2 5])."""
    idx = np.asarray(idx, dtype=np.int64)
    idx = idx[idx >= 0]
    main = kv_row_values(kv_codes_seq[idx], kv_scales_seq[idx])
    swa = e4m3_value(swa_layer_seq[max(0, swa_end - window):swa_end])
    return np.concatenate([main, swa], axis=0)


def attention(q_bf16: np.ndarray, rows: np.ndarray, scale: float):
    """o_h = sum_r softmax_r(scale * q_h . x_r) x_r over the rows (keys = values), float64.

    q_bf16 [H][512] bf16 bits, rows [n][512] float64.  Returns (o [H][512], lse [H]);
    with no rows, o = 0 and lse = -inf."""
    q = bf16_value(q_bf16)
    H = q.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, KV_DIM)), np.full(H, -np.inf)
    z = scale * (q @ rows.T)                            # [H][n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e / l) @ rows
    return o, (m + np.log(l))[:, 0]


# ---------------------------------------------------------------- one query through the chain

def query_chain(inp: Dict[str, np.ndarray], w, b: int, t: int,
                layers: Optional[List[int]] = None,
                idx_sets_override: Optional[np.ndarray] = None,
                pool_override: Optional[np.ndarray] = None,
                with_attention: bool = True) -> Dict[str, object]:
    """Run the whole hot path for query (b, t) of a workload ``w`` (see ``workloads``).

    Index set 0 is the Full layer's Top-k (when the workload has a Full layer), then one set
    per Reindex layer; a Reuse layer reads the set ``w.layer_set`` maps it to ([p1 4.2]).
    ``pool_override`` replaces the Full layer's pool for the Reindex layers and
    ``idx_sets_override`` [S][k] replaces the index sets used by attention (stage-wise
    checks feed the GPU's own intermediate results here)."""
    n_vis = int(inp["n_visible"][b, t])
    k8 = inp["idx_k"][b] if "idx_k" in inp else (inp["idx_k_codes"][b], inp["idx_k_scales"][b])
    out: Dict[str, object] = {}
    sets = []
    if w.has_full:
        f = full_layer(k8, inp["idx_q"][b, t], inp["head_w"][b, t], n_vis,
                       w.block, w.pool_blocks, w.top_k)
        out["full"] = f
        sets.append(f["topk"])
        pool = f["pool"]
    else:
        pool = inp["pool_pos"][b, t, :int(inp["pool_len"][b, t])]
    if pool_override is not None:
        pool = pool_override
    out["reindex"] = []
    for r in range(w.n_reindex):
        ri = reindex_layer(k8, inp["ri_q"][r, b, t], inp["ri_w"][r, b, t], pool, w.top_k)
        out["reindex"].append(ri)
        sets.append(ri["topk"])
    out["sets"] = np.stack(sets) if sets else np.zeros((0, w.top_k), np.int32)
    if not with_attention:
        return out
    use_sets = out["sets"] if idx_sets_override is None else idx_sets_override
    scale = 1.0 / np.sqrt(KV_DIM)
    o_all, lse_all = {}, {}
    for l in (range(w.L) if layers is None else layers):
        rows = attention_rows(inp["kv_codes"][b], inp["kv_scales"][b], use_sets[w.layer_set[l]],
                              inp["swa"][l, b], int(inp["swa_end"][b, t]), w.swa_window)
        o_all[l], lse_all[l] = attention(inp["q"][l, b, t], rows, scale)
    out["attn_out"] = o_all
    out["attn_lse"] = lse_all
    return out


# ---------------------------------------------------------------- encoder prefill, chunk by chunk

def visible_entries(p: int, m: int) -> int:
    """Compressed entries visible to the token at absolute position p ([p2 3], m tokens per
    entry): entry j covers tokens [j*m, (j+1)*m) and is visible once all of them are at or
    before p, i.e. (j+1)*m <= p+1 (a reading: the pages do not say how a partial entry is
    treated).  The count is floor((p+1)/m)."""
    return (p + 1) // m


def encoder_chunk(idx_k: np.ndarray, kv_codes: np.ndarray, kv_scales: np.ndarray,
                  new_idx_k: Optional[np.ndarray], new_latent: Optional[np.ndarray],
                  idx_q: np.ndarray, head_w: np.ndarray, q: np.ndarray, swa: np.ndarray,
                  p0: int, m: int, top_k: int, window: int) -> Dict[str, np.ndarray]:
    """One chunk of an encoder prefill through its CSA2 groups ([p2 3], [p3 modes]; [p5 2]: the
    hierarchical indexer is decoder-only, so an encoder Full layer ranks every visible entry).

    The chunk holds the tokens at positions p0 .. p0+T-1 of B sequences.  Per group g: the
    entries the chunk completes (rows floor(p0/m) .. floor((p0+T)/m) - 1) are appended to the
    group's caches (indexer keys rounded to E4M3, main KV quantised to FP4), in place; each
    token's Full layer ranks the entries visible to it and keeps its Top-k; every layer of the
    group (the Full layer and its Reuse layers) attends over that index set and its own window.

    idx_k [G][B][k_rows][128] E4M3, kv_codes [G][B][k_rows][256], kv_scales [G][B][k_rows][32]
    (caches, modified); new_idx_k [G][B][n_new][128] / new_latent [G][B][n_new][512] bf16 or
    None; idx_q [G][B][T][32][128]; head_w [G][B][T][32]; q [G][Lg][B][T][H][512];
    swa [G][Lg][B][hist+T][512] E4M3 with row r = token p0 - hist + r, hist = min(p0, window-1).
    Returns out [G][Lg][B][T][H][512] float64 and topk [G][B][T][top_k]."""
    G, B, T = idx_q.shape[:3]
    Lg, H = q.shape[1], q.shape[4]
    n_before, n_after = p0 // m, (p0 + T) // m
    hist = min(p0, window - 1) if window > 0 else 0
    assert swa.shape[3] == hist + T
    scale = 1.0 / np.sqrt(KV_DIM)
    out = np.zeros((G, Lg, B, T, H, KV_DIM))
    topk = np.full((G, B, T, top_k), -1, np.int32)
    for g in range(G):
        for b in range(B):
            if new_idx_k is not None:
                idx_k[g, b, n_before:n_after] = e4m3_from_value(bf16_value(new_idx_k[g, b]))
            if new_latent is not None:
                kv_codes[g, b, n_before:n_after], kv_scales[g, b, n_before:n_after] = \
                    kv_quantize_rows(new_latent[g, b])
            for t in range(T):
                n_vis = visible_entries(p0 + t, m)
                f = full_layer(idx_k[g, b], idx_q[g, b, t], head_w[g, b, t], n_vis, 8, 0, top_k)
                topk[g, b, t] = f["topk"]
                for l in range(Lg):
                    rows = attention_rows(kv_codes[g, b], kv_scales[g, b], f["topk"], swa[g, l, b],
                                          hist + t + 1, window)
                    out[g, l, b, t] = attention(q[g, l, b, t], rows, scale)[0]
    return {"out": out, "topk": topk}
