"""Helpers for the GPU tests: run the HIP library through its C ABI on workload inputs and
compare with the oracle under the tolerance rules of the hot path.

Tolerances (the floating-point rules the library states):
  * scores: |s_gpu - s_ref| <= 1e-5 * A, where A = sum_h |w_h| sum_c |q8_hc k_pc| is the
    absolute-value sum of the terms.  Every product is exact in fp32; the fp32 sums of 128
    products per head and of 32 weighted heads, in any order, stay within
    n*u/(1-n*u) * A with n = 162 terms-deep and u = 2^-24, i.e. below 9.7e-6 * A.
  * Top-K / pool: identical sets, except that a position (block) may be swapped only with
    another whose oracle score (block score) lies within 1e-3 * |s_K| of the K-th (P-th) one.
  * attention: per (layer, query, head) max|o_gpu - o_ref| <= 2e-2 * max|o_ref|.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import hierarchical_kv_indexer_amd as H
from oracle import csa2 as O
from oracle import formats as F

DEV = "cuda:0"
SCORE_REL = 1e-5
TIE_REL = 1e-3
ATTN_REL = 2e-2


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if t.dtype == torch.int16 else a


def empty(shape, dtype) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=DEV)


# ------------------------------------------------------------------ library calls

def keys(inp):
    """Indexer keys on the device as the C ABI takes them: (idx_k, idx_k_scales or None, rows)."""
    if "idx_k" in inp:
        return dev(inp["idx_k"]), None, inp["idx_k"].shape[1]
    return dev(inp["idx_k_codes"]), dev(inp["idx_k_scales"]), inp["idx_k_codes"].shape[1]


def gpu_index_scores(inp, B, T, n_max):
    out = torch.full((B, T, max(n_max, 1)), float("nan"), dtype=torch.float32, device=DEV)
    k, ks, rows = keys(inp)
    H.csa2_index_scores(k, ks, rows, dev(inp["idx_q"]), dev(inp["head_w"]),
                        dev(inp["n_visible"]), B, T, n_max, out)
    return host(out)


def gpu_index_full(inp, B, T, n_max, pool_blocks, top_k, block=8):
    cap = max(pool_blocks * block, 1)
    pool_pos = empty((B, T, cap), torch.int32) if pool_blocks else None
    pool_len = empty((B, T), torch.int32) if pool_blocks else None
    idx = empty((B, T, top_k), torch.int32)
    sc = empty((B, T, top_k), torch.float32)
    ws_bytes = H.csa2_index_full_workspace(B, T, n_max, block, pool_blocks, top_k)
    ws = empty((ws_bytes,), torch.uint8)
    k, ks, rows = keys(inp)
    H.csa2_index_full(k, ks, rows, dev(inp["idx_q"]), dev(inp["head_w"]),
                      dev(inp["n_visible"]), B, T, n_max, block, pool_blocks, top_k, pool_pos,
                      pool_len, idx, sc, ws, ws_bytes)
    out = {"topk": host(idx), "topk_score": host(sc)}
    if pool_blocks:
        out["pool_pos"], out["pool_len"] = host(pool_pos), host(pool_len)
    return out


def gpu_index_full_blocks(inp, B, T, n_max, pool_blocks, top_k, block_score, block=8):
    """csa2_index_scan_blocks (the given block score) followed by csa2_index_select."""
    cap = pool_blocks * block
    pool_pos, pool_len = empty((B, T, cap), torch.int32), empty((B, T), torch.int32)
    idx, sc = empty((B, T, top_k), torch.int32), empty((B, T, top_k), torch.float32)
    ws_bytes = H.csa2_index_stages_workspace(B, T, n_max, block, pool_blocks, top_k)
    ws = empty((ws_bytes,), torch.uint8)
    k, ks, rows = keys(inp)
    nv = dev(inp["n_visible"])
    H.csa2_index_scan_blocks(k, ks, rows, dev(inp["idx_q"]), dev(inp["head_w"]), nv, B, T, n_max, block,
                             pool_blocks, top_k, block_score, ws, ws_bytes)
    H.csa2_index_select(nv, B, T, n_max, block, pool_blocks, top_k, pool_pos, pool_len, idx, sc, ws, ws_bytes)
    return {"topk": host(idx), "topk_score": host(sc), "pool_pos": host(pool_pos), "pool_len": host(pool_len)}


def gpu_reindex(inp, B, T, pool_pos, pool_len, top_k, L=None):
    L = inp["ri_q"].shape[0] if L is None else L
    cap = pool_pos.shape[-1]
    idx = empty((L, B, T, top_k), torch.int32)
    sc = empty((L, B, T, top_k), torch.float32)
    ws_bytes = H.csa2_reindex_workspace(L, B, T, cap, top_k)
    ws = empty((ws_bytes,), torch.uint8)
    k, ks, rows = keys(inp)
    H.csa2_reindex(k, ks, rows, dev(inp["ri_q"][:L]), dev(inp["ri_w"][:L]),
                   dev(pool_pos), dev(pool_len), cap, L, B, T, top_k, idx, sc, ws, ws_bytes)
    return {"topk": host(idx), "topk_score": host(sc)}


def gpu_index_chain(inp, B, T, n_max, pool_blocks, top_k, L, split=False, block=8):
    """csa2_index_chain (or csa2_index_scan + csa2_index_select_reindex with split=True)."""
    cap = pool_blocks * block
    pool_pos, pool_len = empty((B, T, cap), torch.int32), empty((B, T), torch.int32)
    idx, sc = empty((B, T, top_k), torch.int32), empty((B, T, top_k), torch.float32)
    ri_idx = empty((max(L, 1), B, T, top_k), torch.int32)
    ri_sc = empty((max(L, 1), B, T, top_k), torch.float32)
    ws_bytes = H.csa2_index_chain_workspace(B, T, n_max, block, pool_blocks, top_k, L)
    ws = empty((ws_bytes,), torch.uint8)
    k, ks, rows = keys(inp)
    q, hw, nv = dev(inp["idx_q"]), dev(inp["head_w"]), dev(inp["n_visible"])
    rq = dev(inp["ri_q"][:L]) if L else None
    rw = dev(inp["ri_w"][:L]) if L else None
    if split:
        H.csa2_index_scan(k, ks, rows, q, hw, nv, B, T, n_max, block, pool_blocks, top_k, ws, ws_bytes)
        H.csa2_index_select_reindex(k, ks, rows, nv, B, T, n_max, block, pool_blocks, top_k, rq, rw, L, pool_pos,
                                    pool_len, idx, sc, ri_idx if L else None, ri_sc if L else None, ws, ws_bytes)
    else:
        H.csa2_index_chain(k, ks, rows, q, hw, nv, B, T, n_max, block, pool_blocks, top_k, rq, rw, L, pool_pos,
                           pool_len, idx, sc, ri_idx if L else None, ri_sc if L else None, ws, ws_bytes)
    out = {"topk": host(idx), "topk_score": host(sc), "pool_pos": host(pool_pos), "pool_len": host(pool_len)}
    if L:
        out["ri_topk"], out["ri_topk_score"] = host(ri_idx), host(ri_sc)
    return out


def gpu_attention(inp, w, idx_sets: np.ndarray, layers: Optional[Sequence[int]] = None):
    """idx_sets [S][B][T][k]; returns out [L][B][T][H][512] (bf16 bits) and lse."""
    L, B, T, Hh = w.L, w.B, w.T, w.H
    S, k = idx_sets.shape[0], idx_sets.shape[-1]
    out = empty((L, B, T, Hh, 512), torch.int16)
    lse = empty((L, B, T, Hh), torch.float32)
    ws_bytes = H.csa2_sparse_attn_workspace(L, B, T, Hh, k, w.swa_window)
    ws = empty((max(ws_bytes, 1),), torch.uint8)
    swa = inp["swa"]
    H.csa2_sparse_attn(dev(inp["kv_codes"]), dev(inp["kv_scales"]), inp["kv_codes"].shape[1], dev(inp["q"]),
                       dev(idx_sets), list(w.layer_set), S, dev(swa), swa.shape[2], dev(inp["swa_end"]),
                       w.swa_window, L, B, T, Hh, k, 1.0 / math.sqrt(512), out, lse, ws, ws_bytes)
    return host(out), host(lse)


# ------------------------------------------------------------------ comparisons

def host_keys(inp, b):
    """Indexer keys of sequence b as the oracle takes them (E4M3 bytes or the FP4 pair)."""
    if "idx_k" in inp:
        return inp["idx_k"][b]
    return (inp["idx_k_codes"][b], inp["idx_k_scales"][b])


def score_abs_bound(k8_rows, q_bf16: np.ndarray, w: np.ndarray) -> np.ndarray:
    """A = sum_h |w_h| sum_c |q8_hc| |k_pc| for each row (keys in either storage form)."""
    qa = np.abs(O.query_values(O.query_for_keys(q_bf16, k8_rows)))
    ka = np.abs(O.k_values(k8_rows))
    return ka @ qa.T @ np.abs(w.astype(np.float64))


def assert_scores_close(s_gpu, s_ref, bound, what=""):
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    lim = SCORE_REL * bound + 1e-30
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} scores outside 1e-5*A; worst ratio "
                           f"{(err / lim).max():.3g}")
    return float((err / np.maximum(np.abs(s_ref), 1e-30)).max()) if len(err) else 0.0


def assert_topk_equiv(gpu_idx, ref_idx, ref_score_at, what=""):
    """gpu_idx / ref_idx: [k] ascending, -1 padded.  ref_score_at(pos) -> oracle score."""
    g = np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    gv, rv = g[g >= 0], r[r >= 0]
    assert np.all(g[len(gv):] == -1) and np.all(np.diff(gv) > 0), f"{what}: GPU output not ascending/padded"
    assert len(gv) == len(rv), f"{what}: {len(gv)} selected vs {len(rv)}"
    diff = set(gv.tolist()) ^ set(rv.tolist())
    if diff:
        sK = min(ref_score_at(p) for p in rv.tolist())
        for p in diff:
            assert abs(ref_score_at(p) - sK) <= TIE_REL * abs(sK), (
                f"{what}: position {p} (score {ref_score_at(p)}) differs beyond the tie band of s_K={sK}")
    return len(diff)


def assert_topk_multiset_equiv(gpu_idx, ref_idx, ref_score_at, what=""):
    """As assert_topk_equiv, for pools that list a position more than once: outputs are
    non-decreasing, and copies count (multiset comparison)."""
    from collections import Counter
    g = np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    gv, rv = g[g >= 0], r[r >= 0]
    assert np.all(g[len(gv):] == -1) and np.all(np.diff(gv) >= 0), f"{what}: GPU output not sorted/padded"
    assert len(gv) == len(rv), f"{what}: {len(gv)} selected vs {len(rv)}"
    cg, cr = Counter(gv.tolist()), Counter(rv.tolist())
    diff = list((cg - cr).elements()) + list((cr - cg).elements())
    if diff:
        sK = min(ref_score_at(p) for p in rv.tolist())
        for p in diff:
            assert abs(ref_score_at(p) - sK) <= TIE_REL * abs(sK), (
                f"{what}: position {p} (score {ref_score_at(p)}) differs beyond the tie band of s_K={sK}")
    return len(diff)


def assert_pool_equiv(gpu_pool, gpu_len, ref_pool, ref_s32, n_vis, block, P, what="", mode="max"):
    gp = np.asarray(gpu_pool[:gpu_len])
    assert gpu_len == len(ref_pool), f"{what}: pool length {gpu_len} vs {len(ref_pool)}"
    assert np.all(np.asarray(gpu_pool[gpu_len:]) == -1), f"{what}: pool padding"
    assert np.all(np.diff(gp) > 0), f"{what}: pool not ascending"
    gb = set((gp // block).tolist())
    rb = set((np.asarray(ref_pool) // block).tolist())
    # whole blocks: every position of a chosen block is present
    for j in gb:
        n = min(block, n_vis - block * j)
        assert np.count_nonzero(gp // block == j) == n, f"{what}: block {j} incomplete"
    diff = gb ^ rb
    if diff:
        blk = O.block_scores(ref_s32, n_vis, block, mode)
        sP = min(blk[j] for j in rb)
        for j in diff:
            assert abs(float(blk[j]) - float(sP)) <= TIE_REL * abs(float(sP)), (
                f"{what}: block {j} differs beyond the tie band")
    return len(diff)


def assert_attention_close(o_gpu_bits, o_ref, what=""):
    """o_gpu_bits [H][512] bf16 bits, o_ref [H][512] float64.  Returns the max relative error."""
    og = F.bf16_value(o_gpu_bits)
    worst = 0.0
    for h in range(o_ref.shape[0]):
        denom = np.abs(o_ref[h]).max()
        err = np.abs(og[h] - o_ref[h]).max()
        if denom == 0:
            assert err == 0, f"{what}: head {h} should be zero"
            continue
        rel = err / denom
        worst = max(worst, rel)
        assert rel <= ATTN_REL, f"{what}: head {h} max rel err {rel:.3g}"
    return worst


# ---------------------------------------------------------------- encoder prefill

class GpuEncoder:
    """Device caches and workspace of an encoder prefill run chunk by chunk through
    csa2_encoder_chunk."""

    def __init__(self, w, max_T: int):
        self.w = w
        n = max(w.prompt // w.m, 1)
        self.idx_k = torch.zeros((w.G, w.B, n, 128), dtype=torch.uint8, device=DEV)
        self.kv_codes = torch.zeros((w.G, w.B, n, 256), dtype=torch.uint8, device=DEV)
        self.kv_scales = torch.zeros((w.G, w.B, n, 32), dtype=torch.uint8, device=DEV)
        self.k_rows = n
        self.ws_bytes = H.csa2_encoder_chunk_workspace(w.B, max_T, n, w.layers, w.H, w.top_k, w.swa_window)
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=DEV)

    def load_caches(self, idx_k, kv_codes, kv_scales):
        self.idx_k.copy_(torch.from_numpy(idx_k))
        self.kv_codes.copy_(torch.from_numpy(kv_codes))
        self.kv_scales.copy_(torch.from_numpy(kv_scales))

    def chunk(self, a: Dict[str, np.ndarray], p0: int, T: int):
        """Runs one chunk; returns (out [G][layers][B][T][H][512] bf16 bits, topk [G][B][T][k])."""
        w = self.w
        out = empty((w.G, w.layers, w.B, T, w.H, 512), torch.int16)
        topk = empty((w.G, w.B, T, w.top_k), torch.int32)
        nn = a["new_idx_k"].shape[2]
        H.csa2_encoder_chunk(w.G, w.layers, dev(a["new_idx_k"]) if nn else None,
                             dev(a["new_latent"]) if nn else None, self.idx_k, self.kv_codes,
                             self.kv_scales, self.k_rows, dev(a["idx_q"]), dev(a["head_w"]), dev(a["q"]),
                             dev(a["swa"]), a["swa"].shape[3], w.B, T, p0, w.m, w.H, w.top_k,
                             w.swa_window, 1.0 / math.sqrt(512), out, topk, self.ws, self.ws_bytes)
        return host(out), host(topk)
