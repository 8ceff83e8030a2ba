"""GPU parity at the full workload sizes, in the launch configuration the benchmark times (the
chain entries where there is a pool): the whole chain runs for every query of the workload; the
oracle checks sampled queries.

  decode_1m        batch 1, 1M-entry context, Full + 4 Reindex + 15 Reuse (20 attention layers)
  decode_1m_fp4k   the same with FP4 indexer keys
  decode_b8_128k   batch 8, 128K entries each, Full + 4 Reindex + 5 Reuse, 64 heads
  reindex_pool_256k  64 queries with their own 16384-position pools over a 256K context
  prefill_4k_64k   4096 causal queries over 32768 entries, Full + 5 Reuse, 64 heads
  encoder_1m       the last 256-token chunk of a 1M-token prompt (512K entries) through 3 encoder
                   groups of Full + 5 Reuse, 64 heads (csa2_encoder_chunk)
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import csa2 as O
from tests import gpu_chain as G
from tests.test_gpu_parity import check_full, run_chain_and_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import hierarchical_kv_indexer_amd as H
    H.lib()


def _announce(name, queries):
    print(f"\n[full-size] {name}: checking queries {queries}", flush=True)


def test_decode_1m_whole_chain():
    w = workloads.WORKLOADS["decode_1m"]
    inp = workloads.make_inputs(w)
    _announce(w.name, [(0, 0)])
    run_chain_and_check(w, inp, [(0, 0)])
    g = G.gpu_index_full(inp, 1, 1, w.N, w.pool_blocks, w.top_k)
    assert np.isin(inp["planted_pos"], g["topk"][0, 0]).all(), "planted cluster not recalled"
    c = G.gpu_index_chain(inp, 1, 1, w.N, w.pool_blocks, w.top_k, w.n_reindex, split=True)
    assert np.array_equal(c["topk"], g["topk"]) and np.array_equal(c["pool_pos"], g["pool_pos"])


def test_decode_1m_fp4_keys_whole_chain():
    """The 1M decode with the FP4 indexer-K variant (72 B per position)."""
    w = workloads.WORKLOADS["decode_1m_fp4k"]
    inp = workloads.make_inputs(w)
    _announce(w.name, [(0, 0)])
    run_chain_and_check(w, inp, [(0, 0)])
    g = G.gpu_index_full(inp, 1, 1, w.N, w.pool_blocks, w.top_k)
    assert np.isin(inp["planted_pos"], g["topk"][0, 0]).all(), "planted cluster not recalled"


def test_decode_b8_128k_sampled():
    w = workloads.WORKLOADS["decode_b8_128k"]
    inp = workloads.make_inputs(w)
    queries = [(b, 0) for b in range(w.B)]                     # every query of the batch
    _announce(w.name, queries)
    run_chain_and_check(w, inp, queries)


def test_reindex_pool_256k_sampled():
    w = workloads.WORKLOADS["reindex_pool_256k"]
    inp = workloads.make_inputs(w)
    queries = [(0, t) for t in list(range(0, 64, 4)) + [17, 63]]   # 18 of the 64 caller pools
    _announce(w.name, queries)
    run_chain_and_check(w, inp, queries)


def test_prefill_4k_64k_sampled():
    w = workloads.WORKLOADS["prefill_4k_64k"]
    inp = workloads.make_inputs(w)
    # 32 tokens over the causal ramp: both ends of 16 multi-query groups of 16 tokens spread from
    # the first to the last (t = 16g and 16g + 15), so each group's largest and smallest visible
    # range is checked
    groups = np.linspace(0, w.T // 16 - 1, 16).round().astype(int)
    queries = sorted({(0, int(16 * g + d)) for g in groups for d in (0, 15)})
    assert len(queries) == 32
    _announce(w.name, queries)
    run_chain_and_check(w, inp, queries)


def test_decode_1m_all_keys_equal():
    """Every indexer key equal: all scores tie, so ranking falls to position order.  The pool is
    the first P blocks, every Top-K (Full and Reindex) the first K positions.  Every unit of the
    scan holds more than four pool blocks, so the whole-context selection path runs."""
    w = workloads.small_variant(workloads.WORKLOADS["decode_1m"], seed=97)
    inp = workloads.make_inputs(w, with_attention=False)
    inp["idx_k"][0, :] = inp["idx_k"][0, 12345]
    _announce("decode_1m, all keys equal", [(0, 0)])
    g = G.gpu_index_full(inp, 1, 1, w.N, w.pool_blocks, w.top_k)
    cap = w.pool_cap
    assert int(g["pool_len"][0, 0]) == cap
    assert np.array_equal(g["pool_pos"][0, 0], np.arange(cap, dtype=np.int32))
    assert np.array_equal(g["topk"][0, 0], np.arange(w.top_k, dtype=np.int32))
    assert np.all(g["topk_score"][0, 0] == g["topk_score"][0, 0, 0])
    ri = G.gpu_reindex(inp, 1, 1, g["pool_pos"], g["pool_len"], w.top_k)
    for r in range(w.n_reindex):
        assert np.array_equal(ri["topk"][r, 0, 0], np.arange(w.top_k, dtype=np.int32))


def test_encoder_1m_chunk_sampled():
    """The encoder chunk at 1M tokens as the benchmark launches it: the appended cache rows equal
    the oracle's quantisers' bytes, and sampled tokens' index sets and attention outputs (first
    and last layer of every group) match the oracle over the oracle's own caches."""
    from oracle import csa2 as O
    from oracle import formats as F
    w = workloads.ENCODER_WORKLOADS["encoder_1m"]
    inp = workloads.make_encoder_chunk(w)
    p0, T, m = w.p0, w.T, w.m
    n0, n1 = p0 // m, (p0 + T) // m
    gpu = G.GpuEncoder(w, T)
    gpu.load_caches(inp["idx_k"], inp["kv_codes"], inp["kv_scales"])
    out, topk = gpu.chunk(inp, p0, T)
    # the oracle's caches: the generated rows plus the chunk's entries appended by its quantisers
    idx_k, codes, scales = inp["idx_k"], inp["kv_codes"], inp["kv_scales"]
    idx_k[:, :, n0:n1] = F.e4m3_from_value(F.bf16_value(inp["new_idx_k"]))
    codes[:, :, n0:n1], scales[:, :, n0:n1] = F.kv_quantize_rows(inp["new_latent"])
    assert np.array_equal(G.host(gpu.idx_k[:, :, n0:n1]), idx_k[:, :, n0:n1])
    assert np.array_equal(G.host(gpu.kv_codes[:, :, n0:n1]), codes[:, :, n0:n1])
    assert np.array_equal(G.host(gpu.kv_scales[:, :, n0:n1]), scales[:, :, n0:n1])
    h = w.hist(p0)
    for g, t in [(0, 0), (1, 127), (2, T - 1)]:
        _announce(w.name, [(g, t)])
        n_vis = O.visible_entries(p0 + t, m)
        f = O.full_layer(idx_k[g, 0], inp["idx_q"][g, 0, t], inp["head_w"][g, 0, t], n_vis, 8, 0, w.top_k)
        G.assert_topk_equiv(topk[g, 0, t], f["topk"], lambda p: f["scores"][p], f"encoder g{g} t{t}")
        for l in (0, w.layers - 1):
            rows = O.attention_rows(codes[g, 0], scales[g, 0], topk[g, 0, t], inp["swa"][g, l, 0], h + t + 1,
                                    w.swa_window)
            o, _ = O.attention(inp["q"][g, l, 0, t], rows, 1.0 / math.sqrt(512))
            G.assert_attention_close(out[g, l, 0, t], o, f"encoder g{g} l{l} t{t}")


def test_index_chain_at_the_largest_full_context():
    """The Full layer at its largest context, 2^21 positions (256 chunks of 8192 positions: the
    largest LDS staging, and units of 64 blocks), through the chain entries: pool, Full Top-K and
    the 4 Reindex Top-Ks against the oracle, and the planted cluster recalled."""
    w = dataclasses.replace(workloads.WORKLOADS["decode_1m"], name="decode_2m", N=1 << 21, seed=1011)
    inp = workloads.make_inputs(w, with_attention=False)
    _announce(w.name, [(0, 0)])
    c = G.gpu_index_chain(inp, 1, 1, w.N, w.pool_blocks, w.top_k, w.n_reindex, split=True)
    check_full(w, inp, c, 0, 0)
    assert np.isin(inp["planted_pos"], c["topk"][0, 0]).all(), "planted cluster not recalled"
    pool = c["pool_pos"][0, 0, :c["pool_len"][0, 0]]
    for r in range(w.n_reindex):
        ref = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][r, 0, 0], inp["ri_w"][r, 0, 0], pool, w.top_k)
        sc = dict(zip(pool.tolist(), ref["scores"].tolist()))
        G.assert_topk_equiv(c["ri_topk"][r, 0, 0], ref["topk"], lambda p: sc[p], f"ri{r}")


@pytest.mark.parametrize("T,N", [(1, 1 << 23), (16, 1 << 20)])
def test_index_scores_at_the_largest_context(T, N):
    """Scores at the largest contexts the scans take: 2^23 positions for one query (1024
    workgroups of 8192 positions) and 2^20 positions for 16 queries of one sequence in the
    multi-query scan (its limit), with the last queries' visibility ragged.  Keys are random
    E4M3 codes (every finite value); sampled positions (both ends, every chunk boundary, random
    ones) against the oracle, and nothing written past a query's visible range."""
    rng = np.random.default_rng(1013 + T)
    k8 = rng.integers(0, 256, size=(1, N, 128), dtype=np.uint8)
    k8[(k8 & 0x7F) == 0x7F] ^= 1                                  # no NaN codes
    inp = {"idx_k": k8,
           "idx_q": workloads.to_bf16_bits(rng.standard_normal((1, T, 32, 128), dtype=np.float32)),
           "head_w": rng.random((1, T, 32), dtype=np.float32),
           "n_visible": np.array([[N - 3 * t for t in range(T)]], np.int32)}
    _announce(f"scores over {N} positions", [(0, t) for t in range(T)])
    s = G.gpu_index_scores(inp, 1, T, N)
    edges = np.arange(1024, N, 1024)                               # every chunk boundary
    for t in sorted({0, T - 1, T // 2}):
        n = int(inp["n_visible"][0, t])
        pos = np.unique(np.concatenate([np.arange(2048), np.arange(n - 2048, n), edges - 1, edges,
                                        rng.integers(0, n, 4096)]))
        pos = pos[pos < n]
        keys = O.k_rows(k8[0], pos)
        q8 = O.query_for_keys(inp["idx_q"][0, t], keys)
        ref = O.indexer_scores(keys, q8, inp["head_w"][0, t])
        bound = G.score_abs_bound(keys, inp["idx_q"][0, t], inp["head_w"][0, t])
        G.assert_scores_close(s[0, t, pos], ref, bound, f"t{t}")
        assert np.all(np.isnan(s[0, t, n:])), "scores beyond n_visible must be untouched"
