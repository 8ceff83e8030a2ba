"""GPU parity of the HIP library (through its C ABI) against the CPU oracle, stage by stage,
on seeded inputs that span several tiles with ragged tails, plus exhaustive format checks
and edge cases."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import csa2 as O
from oracle import formats as F
from tests import gpu_chain as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import hierarchical_kv_indexer_amd as H
    H.lib()


def small(name="tiny_4k", **kw):
    return workloads.small_variant(workloads.WORKLOADS[name], **kw)


# ------------------------------------------------------------------ formats

def test_quantize_query_all_bf16_bit_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = G.empty((65536,), torch.uint8)
    import hierarchical_kv_indexer_amd as H
    H.csa2_quantize_query(G.dev(bits), out, 65536)
    got = G.host(out)
    ref = F.e4m3_from_value(F.bf16_value(bits))
    nan = np.isnan(F.bf16_value(bits))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F) == 0x7F)


def test_scan_every_e4m3_code_exact():
    # rows r = 0..255 hold code r in channel 0; query t=0 has +1 and t=1 has -1 there (head 0)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    k8 = np.zeros((1, 256, 128), np.uint8)
    k8[0, :, 0] = codes
    qf = np.zeros((1, 2, 32, 128), np.float32)
    qf[0, 0, 0, 0], qf[0, 1, 0, 0] = 1.0, -1.0
    w = np.zeros((1, 2, 32), np.float32)
    w[:, :, 0] = 1.0
    inp = {"idx_k": k8, "idx_q": workloads.to_bf16_bits(qf), "head_w": w,
           "n_visible": np.full((1, 2), 256, np.int32)}
    s = G.gpu_index_scores(inp, 1, 2, 256)
    v = F.e4m3_value(codes)
    assert np.array_equal(s[0, 0], np.maximum(v, 0).astype(np.float32))
    assert np.array_equal(s[0, 1], np.maximum(-v, 0).astype(np.float32))


def test_scan_every_fp4_key_code_and_scale_exact():
    """FP4 keys: row r holds code r % 16 in channel c(r) with scale byte r // 16 in that channel's
    group (every code x every finite positive scale, channels spread over all lanes and groups);
    queries +1.5 / -1.5 on that channel (exact in FP4: code 6 x scale 0.25) give
    ReLU(+-1.5 x code x scale) exactly."""
    sc_bytes = np.arange(1, 127, dtype=np.uint8)                 # every finite positive E4M3 scale
    n = 16 * len(sc_bytes)
    codes = np.zeros((1, n, 64), np.uint8)
    scales = np.zeros((1, n, 8), np.uint8)
    r = np.arange(n)
    code, sb = (r % 16).astype(np.uint8), sc_bytes[r // 16]
    ch = (r * 37) % 128
    codes[0, r, ch // 2] = code << (4 * (ch & 1))
    scales[0, r, ch // 16] = sb
    rows_by_ch = {}
    for i, c in enumerate(ch):
        rows_by_ch.setdefault(int(c), []).append(i)
    for c, rows in sorted(rows_by_ch.items())[:128]:
        qf = np.zeros((1, 2, 32, 128), np.float32)
        qf[0, 0, 0, c], qf[0, 1, 0, c] = 1.5, -1.5
        assert O.query_values(O.quantize_query_fp4(workloads.to_bf16_bits(qf[0, 0])))[0, c] == 1.5
        w = np.zeros((1, 2, 32), np.float32)
        w[:, :, 0] = 1.0
        sel = np.array(rows)
        inp = {"idx_k_codes": codes[:, sel], "idx_k_scales": scales[:, sel], "idx_q": workloads.to_bf16_bits(qf),
               "head_w": w, "n_visible": np.full((1, 2), len(sel), np.int32)}
        s = G.gpu_index_scores(inp, 1, 2, len(sel))
        v = 1.5 * F.e2m1_value(code[sel]) * F.e4m3_value(sb[sel])
        assert np.array_equal(s[0, 0], np.maximum(v, 0).astype(np.float32)), c
        assert np.array_equal(s[0, 1], np.maximum(-v, 0).astype(np.float32)), c


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("multi_query", [False, True])
def test_scan_query_rounding_every_bf16(multi_query, fp4):
    """The scans' rounding of the query, for every bf16 pattern, in both scan kernels (one query
    per workgroup, and 16 queries of a sequence per workgroup): to E4M3 for E4M3 keys, to FP4 per
    16-channel group for FP4 keys (each group holds 16 consecutive patterns).  Key rows 2c / 2c+1
    hold +1 / -1 in channel c and query t weights only head t % 32, so its scores are
    ReLU(+-q[t % 32][c]) exactly: 512 queries reveal all 65536 rounded values."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits[np.isnan(F.bf16_value(bits))] = 0
    vals = bits.reshape(16, 32, 128)
    q = np.repeat(vals, 32, axis=0)                                  # query t: group t // 32
    w = np.zeros((512, 32), np.float32)
    w[np.arange(512), np.arange(512) % 32] = 1.0
    ch = np.arange(128)
    if fp4:
        codes = np.zeros((256, 64), np.uint8)
        codes[2 * ch, ch // 2] = np.uint8(0x2) << (4 * (ch & 1))     # E2M1 +1.0
        codes[2 * ch + 1, ch // 2] = np.uint8(0xA) << (4 * (ch & 1)) # E2M1 -1.0
        keys = {"idx_k_codes": codes, "idx_k_scales": np.full((256, 8), 0x38, np.uint8)}
    else:
        k8 = np.zeros((256, 128), np.uint8)
        k8[2 * ch, ch], k8[2 * ch + 1, ch] = 0x38, 0xB8               # E4M3 +1.0 / -1.0
        keys = {"idx_k": k8}
    B, T = (1, 512) if multi_query else (512, 1)
    inp = {kk: np.broadcast_to(v, (B,) + v.shape).copy() for kk, v in keys.items()}
    inp.update(idx_q=q.reshape(B, T, 32, 128), head_w=w.reshape(B, T, 32),
               n_visible=np.full((B, T), 256, np.int32))
    s = G.gpu_index_scores(inp, B, T, 256).reshape(512, 256)
    if fp4:
        qv = O.query_values(O.quantize_query_fp4(vals))              # [16][32][128]
    else:
        qv = F.e4m3_value(O.quantize_query(bits)).reshape(16, 32, 128)
    ref = qv[np.arange(512) // 32, np.arange(512) % 32]             # [512][128]
    assert np.array_equal(s[:, 0::2], np.maximum(ref, 0).astype(np.float32))
    assert np.array_equal(s[:, 1::2], np.maximum(-ref, 0).astype(np.float32))


@pytest.mark.parametrize("H", [16, 64])
def test_fp4_dequant_every_code_and_scale_exact(H):
    # one main row per query, no window: the output is the dequantised row itself (H = 16: the
    # 16-head kernel, H = 64: the 64-head kernel)
    rows = 8
    codes = np.zeros((1, rows, 256), np.uint8)
    ch = np.arange(512)
    nib = (ch % 16).astype(np.uint8)
    codes[0, :] = nib[0::2] | (nib[1::2] << 4)
    sc = (np.arange(rows * 32) % 256).astype(np.uint8).reshape(1, rows, 32)
    sc[(sc & 0x7F) == 0x7F] = 0x38
    w = workloads.Workload("dq", 1, B=1, T=rows, N=rows, H=H, layer_set=(0,), n_reindex=0,
                           top_k=1, swa_window=0)
    inp = {"kv_codes": codes, "kv_scales": sc,
           "q": workloads.to_bf16_bits(np.random.default_rng(0).standard_normal((1, 1, rows, H, 512), dtype=np.float32)),
           "swa": np.zeros((1, 1, 1, 512), np.uint8), "swa_end": np.zeros((1, rows), np.int32)}
    idx = np.arange(rows, dtype=np.int32).reshape(1, 1, rows, 1)
    out, lse = G.gpu_attention(inp, w, idx)
    ref = F.kv_row_values(codes[0], sc[0])
    got = F.bf16_value(out[0, 0])          # [rows][H][512]
    for r in range(rows):
        assert np.array_equal(got[r], np.broadcast_to(ref[r], (H, 512))), f"row {r}"


# ------------------------------------------------------------------ indexer stages

def ragged_visibility(B, T, N, seed):
    """Per-query visible counts for multi-query scans: a causal ramp ending at N with a few
    empty, tiny and chunk-straddling counts mixed in."""
    rng = np.random.default_rng(seed)
    nv = np.minimum(N, N - T + 1 + np.arange(T))[None, :].repeat(B, 0)
    special = [0, 1, 7, 8, 17, 1023, 1024, 1025, 4095, 4097]
    pick = rng.choice(B * T, size=min(len(special), B * T), replace=False)
    nv.reshape(-1)[pick] = np.minimum(special[:len(pick)], N)
    return nv.astype(np.int32)


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("B,T,N,nv", [(1, 1, 4096, None), (2, 3, 4093, [4093, 4000, 17, 0, 8, 1]),
                                      (2, 37, 9000, "ragged"), (1, 20, 9003, "ragged")])
def test_index_scores_parity(B, T, N, nv, fp4):
    """Scores of every visible position, E4M3 keys and FP4 keys; T = 37 runs the multi-query scan
    (groups of 16, 16 and 5 queries) over ragged causal visibility, and T = 20 over score rows
    that are not 16-byte aligned (N = 9003)."""
    w = small(B=B, T=T, N=N, seed=2000 + N, idx_k_fp4=fp4)
    inp = workloads.make_inputs(w, with_attention=False)
    if isinstance(nv, str):
        inp["n_visible"] = ragged_visibility(B, T, N, 7)
    elif nv is not None:
        inp["n_visible"] = np.array(nv, np.int32).reshape(B, T)
    s = G.gpu_index_scores(inp, B, T, N)
    for b in range(B):
        for t in range(T):
            n = int(inp["n_visible"][b, t])
            keys = O.k_rows(G.host_keys(inp, b), slice(0, n))
            q8 = O.query_for_keys(inp["idx_q"][b, t], keys)
            ref = O.indexer_scores(keys, q8, inp["head_w"][b, t])
            bound = G.score_abs_bound(keys, inp["idx_q"][b, t], inp["head_w"][b, t])
            G.assert_scores_close(s[b, t, :n], ref, bound, f"b{b} t{t}")
            assert np.all(np.isnan(s[b, t, n:])), "scores beyond n_visible must be untouched"


def check_full(w, inp, gpu, b, t):
    n = int(inp["n_visible"][b, t])
    keys = G.host_keys(inp, b)
    ref = O.full_layer(keys, inp["idx_q"][b, t], inp["head_w"][b, t], n, w.block,
                       w.pool_blocks, w.top_k)
    s = ref["scores"]
    nd = 0
    if w.pool_blocks:
        nd += G.assert_pool_equiv(gpu["pool_pos"][b, t], int(gpu["pool_len"][b, t]), ref["pool"],
                                  ref["scores32"], n, w.block, w.pool_blocks, f"pool b{b} t{t}")
    nd += G.assert_topk_equiv(gpu["topk"][b, t], ref["topk"], lambda p: s[p], f"topk b{b} t{t}")
    g = gpu["topk"][b, t]
    sel = g[g >= 0]
    bound = G.score_abs_bound(O.k_rows(keys, sel), inp["idx_q"][b, t], inp["head_w"][b, t])
    G.assert_scores_close(gpu["topk_score"][b, t][:len(sel)], s[sel], bound, "topk_score")
    assert np.all(gpu["topk_score"][b, t][len(sel):] == 0)
    return ref, nd


@pytest.mark.parametrize("N,P,K,nv", [
    (4096, 64, 64, None),            # tiny decode workload
    (20003, 128, 256, None),         # ragged, several scan WGs
    (5000, 64, 512, [5000, 300, 511, 0]),   # n_vis < K, n_vis = 0, pool larger than nb
    (9000, 128, 256, 20),            # multi-query scan: 20 queries, ragged causal visibility
    (270000, 0, 512, 16),            # one group of 16 queries over more than 256 chunks of 1024
    (131072, 2048, 512, [131072, 100003, 16389]),   # 16384 blocks: the pool over every block key
    (131080, 2048, 512, [131080, 100003, 16389]),   # 16385 blocks: the unit-list pool
])
def test_index_full_parity(N, P, K, nv):
    T = 1 if nv is None else (nv if isinstance(nv, int) else len(nv))
    w = small(T=T, N=N, pool_blocks=P, top_k=K, seed=3000 + N)
    inp = workloads.make_inputs(w, with_attention=False)
    if isinstance(nv, int):
        inp["n_visible"] = ragged_visibility(1, T, N, 11)
    elif nv is not None:
        inp["n_visible"] = np.array(nv, np.int32).reshape(1, T)
    gpu = G.gpu_index_full(inp, 1, T, N, P, K)
    for t in range(T):
        check_full(w, inp, gpu, 0, t)


def test_index_full_batches_match_one_pass():
    """csa2_index_full in its smallest workspace (512 causal queries over 65536 entries, no pool,
    Top-512: two batches of 256 queries) equals the same call with room for every query at once,
    output for output; sampled queries on both sides of the batch boundary against the oracle."""
    import hierarchical_kv_indexer_amd as H
    N, T, K = 65536, 512, 512
    w = small(T=T, N=N, pool_blocks=0, top_k=K, seed=3800)
    inp = workloads.make_inputs(w, with_attention=False)
    inp["n_visible"] = ragged_visibility(1, T, N, 13)
    k, ks, rows = G.keys(inp)
    q, hw, nv = G.dev(inp["idx_q"]), G.dev(inp["head_w"]), G.dev(inp["n_visible"])
    small_ws = H.csa2_index_full_workspace(1, T, N, 8, 0, K)
    big_ws = H.csa2_index_stages_workspace(1, T, N, 8, 0, K)
    assert small_ws < big_ws
    outs = []
    for wsb in (small_ws, big_ws):
        ws = G.empty((wsb,), torch.uint8)
        idx = G.empty((1, T, K), torch.int32)
        sc = G.empty((1, T, K), torch.float32)
        H.csa2_index_full(k, ks, rows, q, hw, nv, 1, T, N, 8, 0, K, None, None, idx, sc, ws, wsb)
        outs.append((G.host(idx), G.host(sc)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    gpu = {"topk": outs[0][0], "topk_score": outs[0][1]}
    for t in (0, 255, 256, 511):
        check_full(w, inp, gpu, 0, t)


@pytest.mark.parametrize("P,run", [(64, (1600, 3200)), (128, (4000, 4400)), (256, (8000, 8008))])
def test_pool_with_runs_of_high_blocks(P, run):
    """Runs of consecutive high-scoring blocks (200, 50 and 1 blocks against P = 64, 128, 256).
    P = 64, 128: the chunk holding a run has more pool blocks than its chunk list of 16, so it is
    re-read, and the P-th best block is found among the listed blocks above T0 and the re-read
    ones.  P = 256: too large a share of the 2500 blocks for chunk lists, so the pool is selected
    over every block key.  Run rows repeat the 64 best rows of the random keys."""
    N, K = 20000, 256
    w = small(N=N, pool_blocks=P, top_k=K, seed=3400 + P)
    inp = workloads.make_inputs(w, with_attention=False)
    k = inp["idx_k"]
    s = O.indexer_scores(k[0], O.query_for_keys(inp["idx_q"][0, 0], k[0]), inp["head_w"][0, 0])
    best = np.argsort(s, kind="stable")[-64:]
    a, b = run
    k[0, a:b] = k[0, best[np.arange(b - a) % 64]]
    gpu = G.gpu_index_full(inp, 1, 1, N, P, K)
    check_full(w, inp, gpu, 0, 0)


@pytest.mark.parametrize("N", [131072, 200000])
def test_pool_tied_candidates_beyond_direct_ranking(N):
    """A 2048-block pool with the P-th best block inside a group of about 600 blocks of exactly
    equal score, one per unit of 8 blocks: more than 256 candidates share T*'s histogram bin, so
    that bin is narrowed by further passes instead of ranked directly.  N = 131072 (16384 blocks)
    runs the dense pool over every block key; N = 200000 (25000 blocks) the unit-list pool, where
    a run of 6 high blocks inside one unit makes that unit re-read, so T*'s histogram is the one
    derived from T0's first pass.  Equal blocks rank by index on both sides: the pool and Top-K
    equal the oracle's exactly."""
    P, K = 2048, 512
    w = small(N=N, pool_blocks=P, top_k=K, n_reindex=1, seed=3500)
    inp = workloads.make_inputs(w, with_attention=False)
    k = inp["idx_k"]
    q8 = O.query_for_keys(inp["idx_q"][0, 0], k[0])
    s = O.ranking_scores(O.indexer_scores(k[0], q8, inp["head_w"][0, 0]))
    blk = O.block_scores(s, N, 8)
    target = int(np.argsort(-blk, kind="stable")[1800])        # the block ranked 1801st
    r0 = 8 * target + int(np.argmax(s[8 * target:8 * target + 8]))
    unit_max = blk.reshape(-1, 8).max(1)                        # units of 8 blocks (64 positions)
    low = np.flatnonzero(unit_max < s[r0])
    pick = low[np.linspace(2, len(low) - 1, 600).astype(int)]
    k[0, 64 * pick] = k[0, r0]                                  # 600 blocks of score exactly s[r0]
    run_unit = int(low[0])
    k[0, 64 * run_unit + 8 * np.arange(6)] = k[0, int(np.argmax(s))]
    got = G.gpu_index_chain(inp, 1, 1, N, P, K, 1, split=True)
    ref, nd = check_full(w, inp, got, 0, 0)
    assert nd == 0
    gp = got["pool_pos"][0, 0, :got["pool_len"][0, 0]]
    assert np.array_equal(gp, ref["pool"])


def test_chain_top2048_over_a_full_pool():
    """Top-2048 of a 16384-position pool: the chunk lists then hold exactly k keys, every chunk's cut
    reaches T0 and the Top-K of the Full layer and of 2 Reindex layers is taken over every slot (the
    lists' fallback); against the oracle."""
    N, P, K, L = 131072, 2048, 2048, 2
    w = small(N=N, pool_blocks=P, top_k=K, n_reindex=L, seed=3600)
    inp = workloads.make_inputs(w, with_attention=False)
    got = G.gpu_index_chain(inp, 1, 1, N, P, K, L, split=True)
    check_full(w, inp, got, 0, 0)
    pool = got["pool_pos"][0, 0, :got["pool_len"][0, 0]]
    for r in range(L):
        ref = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][r, 0, 0], inp["ri_w"][r, 0, 0], pool, K)
        sc = dict(zip(pool.tolist(), ref["scores"].tolist()))
        G.assert_topk_equiv(got["ri_topk"][r, 0, 0], ref["topk"], lambda p: sc[p], f"ri{r}")


def test_chain_chunk_lists_over_rounded_chunks():
    """A 600000-position context with a 256-block pool: the scan's chunk of positions rounds up to
    4096 (147 chunks, the last one ragged), so the pool is taken from chunk lists of 512 blocks;
    pool, Top-K and one Reindex layer against the oracle."""
    N, P, K, L = 600000, 256, 512, 1
    w = small(N=N, pool_blocks=P, top_k=K, n_reindex=L, seed=3700)
    inp = workloads.make_inputs(w, with_attention=False)
    got = G.gpu_index_chain(inp, 1, 1, N, P, K, L, split=False)
    check_full(w, inp, got, 0, 0)
    pool = got["pool_pos"][0, 0, :got["pool_len"][0, 0]]
    ref = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][0, 0, 0], inp["ri_w"][0, 0, 0], pool, K)
    sc = dict(zip(pool.tolist(), ref["scores"].tolist()))
    G.assert_topk_equiv(got["ri_topk"][0, 0, 0], ref["topk"], lambda p: sc[p], "ri0")


@pytest.mark.parametrize("T", [2, 9])
@pytest.mark.parametrize("mode", [1, 2])
def test_pool_block_score_variants(mode, T):
    """The pool and its Top-K with the sum (1) and top-2 mean (2) block scores, against the oracle
    with the same block score; T = 9 runs the multi-query scan."""
    name = {1: "sum", 2: "top2"}[mode]
    N, P, K = 20003, 128, 256
    w = small(T=T, N=N, pool_blocks=P, top_k=K, seed=3300 + 10 * mode + T)
    inp = workloads.make_inputs(w, with_attention=False)
    inp["n_visible"] = np.array([N - 3 * t for t in range(T)], np.int32).reshape(1, T)
    gpu = G.gpu_index_full_blocks(inp, 1, T, N, P, K, mode)
    for t in range(T):
        n = int(inp["n_visible"][0, t])
        ref = O.full_layer(G.host_keys(inp, 0), inp["idx_q"][0, t], inp["head_w"][0, t], n, 8, P, K, name)
        G.assert_pool_equiv(gpu["pool_pos"][0, t], int(gpu["pool_len"][0, t]), ref["pool"], ref["scores32"], n, 8, P,
                            f"{name} pool t{t}", mode=name)
        G.assert_topk_equiv(gpu["topk"][0, t], ref["topk"], lambda p: ref["scores"][p], f"{name} topk t{t}")


@pytest.mark.parametrize("P", [256, 0])
def test_stage_entries_match_index_full(P):
    """scan, pool and Top-K called as separate stages (the Top-K on a second stream) give the
    same bits as csa2_index_full."""
    import hierarchical_kv_indexer_amd as H
    N, K, T = 20000, 300, 2
    w = small(T=T, N=N, pool_blocks=P, top_k=K, seed=3100 + P)
    inp = workloads.make_inputs(w, with_attention=False)
    ref = G.gpu_index_full(inp, 1, T, N, P, K)
    cap = max(P * 8, 1)
    pool_pos = G.empty((1, T, cap), torch.int32) if P else None
    pool_len = G.empty((1, T), torch.int32) if P else None
    idx = G.empty((1, T, K), torch.int32)
    sc = G.empty((1, T, K), torch.float32)
    wsb = H.csa2_index_stages_workspace(1, T, N, 8, P, K)
    ws = G.empty((wsb,), torch.uint8)
    k, q, hw, nv = G.dev(inp["idx_k"]), G.dev(inp["idx_q"]), G.dev(inp["head_w"]), G.dev(inp["n_visible"])
    H.csa2_index_scan(k, None, N, q, hw, nv, 1, T, N, 8, P, K, ws, wsb)
    H.csa2_index_pool(nv, 1, T, N, 8, P, K, pool_pos, pool_len, ws, wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        H.csa2_index_topk(1, T, N, 8, P, K, pool_pos, pool_len, idx, sc, ws, wsb)
    torch.cuda.current_stream().wait_stream(side)
    assert np.array_equal(G.host(idx), ref["topk"])
    assert np.array_equal(G.host(sc).view(np.uint32), ref["topk_score"].view(np.uint32))
    if P:
        assert np.array_equal(G.host(pool_pos), ref["pool_pos"])
        assert np.array_equal(G.host(pool_len), ref["pool_len"])


@pytest.mark.parametrize("L,split,fp4", [(2, False, False), (2, True, False), (0, False, False), (2, True, True)])
def test_index_chain_matches_full_then_reindex(L, split, fp4):
    """The one-call indexer (Full Top-K launched with the Reindex Top-K) gives the same bits as
    csa2_index_full followed by csa2_reindex on its pool; ragged n_visible per query."""
    B, T, N, P, K = 2, 2, 20000, 256, 300
    w = small(B=B, T=T, N=N, pool_blocks=P, top_k=K, n_reindex=max(L, 1), seed=3200 + L, idx_k_fp4=fp4)
    inp = workloads.make_inputs(w, with_attention=False)
    inp["n_visible"] = np.array([[20000, 13001], [2047, 19999]], np.int32)
    ref = G.gpu_index_full(inp, B, T, N, P, K)
    got = G.gpu_index_chain(inp, B, T, N, P, K, L, split=split)
    for key in ("topk", "pool_pos", "pool_len"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(got["topk_score"].view(np.uint32), ref["topk_score"].view(np.uint32))
    if L:
        ri = G.gpu_reindex(inp, B, T, ref["pool_pos"], ref["pool_len"], K, L=L)
        assert np.array_equal(got["ri_topk"], ri["topk"])
        assert np.array_equal(got["ri_topk_score"].view(np.uint32), ri["topk_score"].view(np.uint32))
    check_full(w, inp, got, 1, 1)


def test_index_full_no_pool_dense_topk():
    w = small(T=3, N=9000, pool_blocks=0, top_k=200, seed=31)
    inp = workloads.make_inputs(w, with_attention=False)
    inp["n_visible"] = np.array([[9000, 4321, 100]], np.int32)
    gpu = G.gpu_index_full(inp, 1, 3, 9000, 0, 200)
    for t in range(3):
        check_full(w, inp, gpu, 0, t)


def test_index_full_ties():
    # many equal keys: identical rows -> identical scores; ranking must fall back to index order
    w = small(N=3000, pool_blocks=40, top_k=100, seed=41)
    inp = workloads.make_inputs(w, with_attention=False)
    k = inp["idx_k"]
    k[0, 1000:2000] = k[0, 5]            # 1000 identical keys
    gpu = G.gpu_index_full(inp, 1, 1, 3000, 40, 100)
    ref, nd = check_full(w, inp, gpu, 0, 0)
    assert np.array_equal(gpu["topk"][0, 0], ref["topk"])   # exact ties resolve identically


def test_reindex_parity_on_oracle_pool():
    w = small(T=2, N=30000, pool_blocks=256, top_k=300, n_reindex=3, seed=51)
    inp = workloads.make_inputs(w, with_attention=False)
    cap = w.pool_cap
    pool_pos = np.full((1, 2, cap), -1, np.int32)
    pool_len = np.zeros((1, 2), np.int32)
    refs = []
    for t in range(2):
        f = O.full_layer(inp["idx_k"][0], inp["idx_q"][0, t], inp["head_w"][0, t], w.N, w.block,
                         w.pool_blocks, w.top_k)
        pool_pos[0, t, :len(f["pool"])] = f["pool"]
        pool_len[0, t] = len(f["pool"])
        refs.append(f["pool"])
    gpu = G.gpu_reindex(inp, 1, 2, pool_pos, pool_len, w.top_k)
    for l in range(3):
        for t in range(2):
            r = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][l, 0, t], inp["ri_w"][l, 0, t], refs[t], w.top_k)
            sc = dict(zip(refs[t].tolist(), r["scores"].tolist()))
            G.assert_topk_equiv(gpu["topk"][l, 0, t], r["topk"], lambda p: sc[p], f"ri l{l} t{t}")
            sel = gpu["topk"][l, 0, t]
            assert set(sel[sel >= 0].tolist()) <= set(refs[t].tolist())


def test_reindex_user_pools_with_invalid_entries():
    w = small("reindex_pool_256k", T=4, N=50000, user_pool=3000, top_k=512, seed=61)
    inp = workloads.make_inputs(w, with_attention=False)
    pp = inp["pool_pos"].copy()
    pl = inp["pool_len"].copy()
    pp[0, 1, 10] = -5
    pp[0, 1, 11] = 10 ** 7            # out of range: ignored
    pl[0, 2] = 400                    # fewer than top_k
    pl[0, 3] = 0
    gpu = G.gpu_reindex(inp, 1, 4, pp, pl, 512)
    for t in range(4):
        pool = pp[0, t, :pl[0, t]]
        pool = pool[(pool >= 0) & (pool < w.N)]
        r = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][0, 0, t], inp["ri_w"][0, 0, t], pool, 512)
        sc = dict(zip(pool.tolist(), r["scores"].tolist()))
        G.assert_topk_equiv(gpu["topk"][0, 0, t], r["topk"], lambda p: sc[p], f"user pool t{t}")


def test_reindex_user_pool_of_odd_capacity():
    """A caller pool of 1001 slots (rows not 16-byte aligned, a last unit of 9 slots) with
    lengths that end inside, at and before that unit; against the oracle."""
    w = small("reindex_pool_256k", T=3, N=30000, user_pool=1001, top_k=256, seed=67)
    inp = workloads.make_inputs(w, with_attention=False)
    pp = inp["pool_pos"].copy()
    pl = inp["pool_len"].copy()
    pl[0, :] = [1001, 995, 990]
    gpu = G.gpu_reindex(inp, 1, 3, pp, pl, 256)
    for t in range(3):
        pool = pp[0, t, :pl[0, t]]
        pool = pool[(pool >= 0) & (pool < w.N)]
        r = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][0, 0, t], inp["ri_w"][0, 0, t], pool, 256)
        sc = dict(zip(pool.tolist(), r["scores"].tolist()))
        G.assert_topk_equiv(gpu["topk"][0, 0, t], r["topk"], lambda p: sc[p], f"odd pool t{t}")


@pytest.mark.parametrize("fp4", [False, True])
def test_reindex_many_caller_pools_ragged_lengths(fp4):
    """40 caller pools of 16384 slots (5120 scoring workgroups, several rounds of the chip) with
    lengths that end inside a unit, at unit and workgroup boundaries, at zero and at the
    capacity; E4M3 and FP4 keys, against the oracle."""
    T, K, cap = 40, 512, 16384
    w = small("reindex_pool_256k", T=T, N=40000, user_pool=cap, top_k=K, seed=69, idx_k_fp4=fp4)
    inp = workloads.make_inputs(w, with_attention=False)
    pp = inp["pool_pos"].copy()
    pl = inp["pool_len"].copy()
    lens = [cap, 0, 1, 127, 128, 129, 6 * 128, 6 * 128 + 1, 12 * 128 - 1, 5000, cap - 1, 513]
    for t, n in enumerate(lens):
        pl[0, t] = n
    gpu = G.gpu_reindex(inp, 1, T, pp, pl, K)
    for t in list(range(len(lens))) + [20, 39]:
        pool = pp[0, t, :pl[0, t]]
        pool = pool[(pool >= 0) & (pool < w.N)]
        r = O.reindex_layer(G.host_keys(inp, 0), inp["ri_q"][0, 0, t], inp["ri_w"][0, 0, t], pool, K)
        sc = dict(zip(pool.tolist(), r["scores"].tolist()))
        G.assert_topk_equiv(gpu["topk"][0, 0, t], r["topk"], lambda p: sc[p], f"runs t{t} len {pl[0, t]}")


def test_reindex_user_pool_with_repeated_positions():
    """A caller pool listing some positions two or three times: copies rank like the position
    (score desc, position asc, counted with repeats), as the oracle's stable ranking orders them,
    including copies that straddle the K-th place."""
    K = 512
    w = small("reindex_pool_256k", T=2, N=50000, user_pool=3000, top_k=K, seed=67)
    inp = workloads.make_inputs(w, with_attention=False)
    pp = inp["pool_pos"].copy()
    pl = inp["pool_len"].copy()
    for t in range(2):
        pool = pp[0, t, :pl[0, t]].astype(np.int64)
        base = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][0, 0, t], inp["ri_w"][0, 0, t], pool, len(pool))
        order = O.rank_order(O.ranking_scores(base["scores"]), pool)
        picks = pool[order[[0, 10, 508, 509, 510, 511, 700]]]
        extra = np.concatenate([picks, picks[[1, 4]]])        # two positions three times
        keep = np.setdiff1d(pool, pool[order[-len(extra):]])   # drop the lowest-ranked to fit
        new = np.sort(np.concatenate([keep, extra]))
        assert len(new) == pl[0, t]
        pp[0, t, :len(new)] = new
    gpu = G.gpu_reindex(inp, 1, 2, pp, pl, K)
    for t in range(2):
        pool = pp[0, t, :pl[0, t]]
        r = O.reindex_layer(inp["idx_k"][0], inp["ri_q"][0, 0, t], inp["ri_w"][0, 0, t], pool, K)
        assert len(r["topk"][r["topk"] >= 0]) != len(set(r["topk"][r["topk"] >= 0].tolist()))  # repeats kept
        sc = dict(zip(pool.tolist(), r["scores"].tolist()))
        G.assert_topk_multiset_equiv(gpu["topk"][0, 0, t], r["topk"], lambda p: sc[p], f"repeated t{t}")


# ------------------------------------------------------------------ attention

@pytest.mark.parametrize("H", [32, 64, 128])
def test_attention_parity_on_oracle_sets(H):
    """H = 32 runs 16 heads per workgroup; H = 64 and 128 run 64 heads per workgroup."""
    w = small(B=2, T=2, N=3000, H=H, layer_set=(0, 0, 1), n_reindex=1, pool_blocks=64, top_k=200, seed=71)
    inp = workloads.make_inputs(w)
    sets = np.full((2, 2, 2, 200), -1, np.int32)
    rng = np.random.default_rng(5)
    for s in range(2):
        for b in range(2):
            for t in range(2):
                n = [200, 137, 0, 64][(s + 2 * b + t) % 4]     # ragged and empty sets
                sets[s, b, t, :n] = np.sort(rng.choice(w.N, n, replace=False))
    inp["swa_end"] = np.array([[128, 50], [0, 128]], np.int32)   # partial and empty windows
    out, lse = G.gpu_attention(inp, w, sets)
    worst = 0.0
    for l in range(w.L):
        for b in range(2):
            for t in range(2):
                rows = O.attention_rows(inp["kv_codes"][b], inp["kv_scales"][b], sets[w.layer_set[l], b, t],
                                        inp["swa"][l, b], int(inp["swa_end"][b, t]), w.swa_window)
                o, ls = O.attention(inp["q"][l, b, t], rows, 1 / math.sqrt(512))
                worst = max(worst, G.assert_attention_close(out[l, b, t], o, f"l{l} b{b} t{t}"))
                if rows.shape[0] == 0:
                    assert np.all(np.isneginf(lse[l, b, t]))
                else:
                    assert np.allclose(lse[l, b, t], ls, rtol=1e-3, atol=1e-3)
    print(f"attention worst rel err {worst:.3g}")
    assert worst < 1e-2


@pytest.mark.parametrize("H,Bq", [(16, 1), (16, 2), (64, 1), (64, 2)])
def test_attention_skips_out_of_range_entries(H, Bq):
    """Index-set entries past the cache's rows or negative (not only -1) are empty slots, in both
    attention kernels, with row splits (one query per sequence) and without (two)."""
    w = small(B=Bq, T=2, N=3000, H=H, layer_set=(0, 1), n_reindex=1, pool_blocks=64, top_k=256, seed=91)
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(11)
    sets = np.full((2, Bq, 2, 256), -1, np.int32)
    for s in range(2):
        for b in range(Bq):
            for t in range(2):
                e = rng.choice(w.N, 256, replace=False).astype(np.int64)
                bad = rng.random(256) < 0.3
                e[bad] = rng.choice([w.N, w.N + 1, 10 ** 9, -2, -(2 ** 31)], bad.sum())
                sets[s, b, t] = e.astype(np.int32)
    out, lse = G.gpu_attention(inp, w, sets)
    worst = 0.0
    for l in range(w.L):
        for b in range(Bq):
            for t in range(2):
                e = sets[w.layer_set[l], b, t].astype(np.int64)
                kept = np.where((e >= 0) & (e < w.N), e, -1)       # the header's empty slots
                rows = O.attention_rows(inp["kv_codes"][b], inp["kv_scales"][b], kept,
                                        inp["swa"][l, b], int(inp["swa_end"][b, t]), w.swa_window)
                o, ls = O.attention(inp["q"][l, b, t], rows, 1 / math.sqrt(512))
                worst = max(worst, G.assert_attention_close(out[l, b, t], o, f"l{l} b{b} t{t}"))
                assert np.allclose(lse[l, b, t], ls, rtol=1e-3, atol=1e-3)
    print(f"attention worst rel err {worst:.3g}")


@pytest.mark.parametrize("NH", [16, 64])
def test_attention_rescales_when_logits_grow_by_chunk(NH):
    """Every 64-row chunk's logits exceed the previous chunk's by more than 2^8 (log2 units), so
    the running max moves (and the output is rescaled) at every chunk of a workgroup; 512
    (layer, query, head group) items keep the rows in one split per item."""
    L, T, K, N = 8, 64, 512, 640
    w = small(B=1, T=T, N=N, H=NH, layer_set=tuple(range(L)), n_reindex=0, pool_blocks=0, top_k=K, seed=99)
    inp = workloads.make_inputs(w)
    # main row p: every channel E2M1 1.0 x scale 0.5 + 0.25 * (p // 64) (exact in E4M3)
    sc = 0.5 + 0.25 * (np.arange(N) // 64)
    inp["kv_codes"][:] = 0x22
    inp["kv_scales"][:] = workloads.to_e4m3_bytes(np.repeat(sc[None, :, None], 32, axis=2).astype(np.float32))
    inp["q"][:] = workloads.to_bf16_bits(np.ones(inp["q"].shape, np.float32))
    sets = np.tile(np.arange(K, dtype=np.int32), (L, 1, T, 1))
    out, lse = G.gpu_attention(inp, w, sets)
    for (l, t) in [(0, 0), (3, T // 2), (L - 1, T - 1)]:
        rows = O.attention_rows(inp["kv_codes"][0], inp["kv_scales"][0], sets[l, 0, t], inp["swa"][l, 0],
                                int(inp["swa_end"][0, t]), w.swa_window)
        o, ls = O.attention(inp["q"][l, 0, t], rows, 1 / math.sqrt(512))
        G.assert_attention_close(out[l, 0, t], o, f"l{l} t{t}")
        assert np.allclose(lse[l, 0, t], ls, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("H", [16, 64])
def test_attention_at_the_largest_sets_and_window(H):
    """The attention's limits: Top-2048 index sets merged with a 4096-row window (6144 rows, split
    over the most workgroups the plan takes), positions up to the last main-KV row; one query with
    full sets and window, one with a partial set and window."""
    K, W, N = 2048, 4096, 9000
    w = small(B=1, T=2, N=N, H=H, layer_set=(0,), n_reindex=0, pool_blocks=0, top_k=K, swa_window=W,
              seed=107 + H)
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(11)
    sets = np.full((1, 1, 2, K), -1, np.int32)
    sets[0, 0, 0] = np.sort(np.concatenate([rng.choice(N - 1, K - 1, replace=False), [N - 1]]))
    sets[0, 0, 1, :1500] = np.sort(rng.choice(N, 1500, replace=False))
    inp["swa_end"] = np.array([[W, 1000]], np.int32)
    out, lse = G.gpu_attention(inp, w, sets)
    for t in range(2):
        rows = O.attention_rows(inp["kv_codes"][0], inp["kv_scales"][0], sets[0, 0, t], inp["swa"][0, 0],
                                int(inp["swa_end"][0, t]), W)
        o, ls = O.attention(inp["q"][0, 0, t], rows, 1 / math.sqrt(512))
        G.assert_attention_close(out[0, 0, t], o, f"t{t}")
        assert np.allclose(lse[0, 0, t], ls, rtol=1e-3, atol=1e-3)


# ------------------------------------------------------------------ whole chain

def run_chain_and_check(w, inp, queries):
    """The path as the benchmark runs it: with a Full layer and a pool, csa2_index_chain_scan then
    csa2_index_select_reindex; otherwise csa2_index_full and/or csa2_reindex.  Then attention."""
    B, T = w.B, w.T
    gpu_ri = None
    if w.has_full and w.pool_blocks:
        gpu_full = G.gpu_index_chain(inp, B, T, w.N, w.pool_blocks, w.top_k, w.n_reindex, split=True)
        pool_pos, pool_len = gpu_full["pool_pos"], gpu_full["pool_len"]
        if w.n_reindex:
            gpu_ri = {"topk": gpu_full["ri_topk"]}
    else:
        gpu_full = G.gpu_index_full(inp, B, T, w.N, w.pool_blocks, w.top_k) if w.has_full else None
        if not w.has_full:
            pool_pos, pool_len = inp["pool_pos"], inp["pool_len"]
        else:
            pool_pos = pool_len = None
        gpu_ri = G.gpu_reindex(inp, B, T, pool_pos, pool_len, w.top_k) if w.n_reindex else None
    sets = []
    if w.has_full:
        sets.append(gpu_full["topk"])
    if w.n_reindex:
        sets += [gpu_ri["topk"][r] for r in range(w.n_reindex)]
    sets = np.stack(sets)
    out, lse = G.gpu_attention(inp, w, sets)
    for (b, t) in queries:
        if w.has_full:
            check_full(w, inp, gpu_full, b, t)
        gp = pool_pos[b, t, :pool_len[b, t]] if pool_pos is not None else None
        ref = O.query_chain(inp, w, b, t, pool_override=gp, idx_sets_override=sets[:, b, t])
        for r in range(w.n_reindex):
            sc = dict(zip(gp.tolist(), ref["reindex"][r]["scores"].tolist()))
            G.assert_topk_equiv(gpu_ri["topk"][r, b, t], ref["reindex"][r]["topk"], lambda p: sc[p], f"ri{r}")
        for l in range(w.L):
            G.assert_attention_close(out[l, b, t], ref["attn_out"][l], f"attn l{l} b{b} t{t}")
    return out


def test_chain_tiny_decode():
    w = workloads.WORKLOADS["tiny_4k"]
    inp = workloads.make_inputs(w)
    run_chain_and_check(w, inp, [(0, 0)])


def test_chain_planted_64k():
    w = small("decode_1m", N=65536, seed=81)
    inp = workloads.make_inputs(w)
    run_chain_and_check(w, inp, [(0, 0)])
    g = G.gpu_index_full(inp, 1, 1, w.N, w.pool_blocks, w.top_k)
    assert np.isin(inp["planted_pos"], g["topk"][0, 0]).all()


def test_chain_planted_64k_fp4_keys():
    """The whole chain with FP4 indexer keys: Full layer, pool, Reindex, attention."""
    w = small("decode_1m_fp4k", N=65536, seed=83)
    inp = workloads.make_inputs(w)
    run_chain_and_check(w, inp, [(0, 0)])
    g = G.gpu_index_full(inp, 1, 1, w.N, w.pool_blocks, w.top_k)
    assert np.isin(inp["planted_pos"], g["topk"][0, 0]).all()


def test_chain_prefill_small():
    w = small("prefill_4k_64k", T=64, N=4096, prefill_tokens=8192, seed=91)
    inp = workloads.make_inputs(w)
    run_chain_and_check(w, inp, [(0, 0), (0, 31), (0, 63)])


@pytest.mark.parametrize("NH", [16, 64])
def test_attention_split_merge_repeats_and_graph_replays(NH):
    """Rows split over workgroups leave partial softmax states in the workspace for the merge.
    Repeated calls on one workspace (starting from arbitrary bytes), and replays of a captured
    call with other work in between, must all give the eager result."""
    import hierarchical_kv_indexer_amd as H
    w = small(B=1, T=1, N=5000, H=NH, layer_set=(0, 0, 1, 1), n_reindex=1, pool_blocks=64, top_k=512, seed=77)
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(9)
    sets = np.stack([np.sort(rng.choice(w.N, 512, replace=False)).astype(np.int32) for _ in range(2)]).reshape(2, 1, 1, 512)
    L, K = w.L, 512
    assert H.csa2_sparse_attn_workspace(L, 1, 1, NH, K, w.swa_window) > 0, "expected split rows"
    out_ref, _ = G.gpu_attention(inp, w, sets)
    args = dict(codes=G.dev(inp["kv_codes"]), scales=G.dev(inp["kv_scales"]), q=G.dev(inp["q"]), sets=G.dev(sets),
                swa=G.dev(inp["swa"]), end=G.dev(inp["swa_end"]))
    out = G.empty((L, 1, 1, NH, 512), torch.int16)
    wsb = H.csa2_sparse_attn_workspace(L, 1, 1, NH, K, w.swa_window)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=G.DEV)     # arbitrary initial bytes

    def call():
        H.csa2_sparse_attn(args["codes"], args["scales"], w.N, args["q"], args["sets"], list(w.layer_set), 2,
                           args["swa"], w.swa_rows, args["end"], w.swa_window, L, 1, 1, NH, K,
                           1.0 / math.sqrt(512), out, None, ws, wsb)

    for _ in range(3):
        out.zero_()
        call()
        assert np.array_equal(G.host(out), out_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(G.host(out), out_ref), f"replay {i}"
        call()                                                            # eager work between replays
        assert np.array_equal(G.host(out), out_ref)


def test_index_chain_graph_replays_and_concurrent_streams():
    """The decode indexer (csa2_index_chain: scan, pool, Full and Reindex Top-K) captured in a HIP
    graph replays to the eager result, with other eager calls on the same workspace in between and
    the workspace starting from arbitrary bytes; and two chains on two streams at once, each with
    its own workspace and outputs, give their serial results (the calls hold no global state)."""
    import hierarchical_kv_indexer_amd as H
    N, P, K, L = 30000, 128, 256, 2

    class Chain:
        def __init__(self, seed):
            w = small(N=N, pool_blocks=P, top_k=K, n_reindex=L, seed=seed)
            self.inp = workloads.make_inputs(w, with_attention=False)
            self.ref = G.gpu_index_chain(self.inp, 1, 1, N, P, K, L)
            self.k, self.ks, self.rows = G.keys(self.inp)
            self.q, self.hw, self.nv = (G.dev(self.inp[n]) for n in ("idx_q", "head_w", "n_visible"))
            self.rq, self.rw = G.dev(self.inp["ri_q"][:L]), G.dev(self.inp["ri_w"][:L])
            self.pool_pos, self.pool_len = G.empty((1, 1, P * 8), torch.int32), G.empty((1, 1), torch.int32)
            self.idx, self.ri_idx = G.empty((1, 1, K), torch.int32), G.empty((L, 1, 1, K), torch.int32)
            self.wsb = H.csa2_index_chain_workspace(1, 1, N, 8, P, K, L)
            self.ws = torch.full((self.wsb,), 0xA5, dtype=torch.uint8, device=G.DEV)

        def call(self, stream=None):
            H.csa2_index_chain(self.k, self.ks, self.rows, self.q, self.hw, self.nv, 1, 1, N, 8, P, K, self.rq,
                               self.rw, L, self.pool_pos, self.pool_len, self.idx, None, self.ri_idx, None, self.ws,
                               self.wsb, stream)

        def check(self, what):
            assert np.array_equal(G.host(self.idx), self.ref["topk"]), what
            assert np.array_equal(G.host(self.ri_idx), self.ref["ri_topk"]), what
            assert np.array_equal(G.host(self.pool_pos), self.ref["pool_pos"]), what
            assert np.array_equal(G.host(self.pool_len), self.ref["pool_len"]), what

        def clear(self):
            for t in (self.idx, self.ri_idx, self.pool_pos, self.pool_len):
                t.fill_(-7)

    a, b = Chain(3401), Chain(3402)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        a.call(s)
    torch.cuda.synchronize()
    for i in range(4):
        a.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a.check(f"replay {i}")
        a.clear()
        a.call()                                                          # eager, same workspace
        a.check(f"eager after replay {i}")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(3):
        a.clear()
        b.clear()
        torch.cuda.synchronize()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        a.call(s1)
        b.call(s2)
        torch.cuda.synchronize()
        a.check(f"stream 1, round {i}")
        b.check(f"stream 2, round {i}")


def test_chain_over_allocated_caches():
    """Caches with more rows per sequence than the visible range (k_rows_per_seq = kv_rows = 6000,
    n_max = 5000, n_visible 5000 and 4321 for two sequences): the per-sequence row strides are
    the allocation's, and nothing past a query's visible range is scored or gathered."""
    import dataclasses
    w_alloc = small("decode_1m", B=2, N=6000, pool_blocks=64, top_k=128, seed=3501)
    inp = workloads.make_inputs(w_alloc)
    inp["n_visible"] = np.array([[5000], [4321]], np.int32)
    w = dataclasses.replace(w_alloc, N=5000)
    out = run_chain_and_check(w, inp, [(0, 0), (1, 0)])
    assert out.shape[1] == 2


def test_attention_at_the_most_layers():
    """64 attention layers (the limit) over 3 index sets in a Reuse pattern, two queries: every
    layer reads its own set, query and window."""
    L = 64
    layer_set = tuple((l // 3) % 3 for l in range(L))
    w = small(B=1, T=2, N=3000, H=16, layer_set=layer_set, n_reindex=2, pool_blocks=64, top_k=96, seed=109)
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(13)
    sets = np.stack([np.stack([np.sort(rng.choice(w.N, 96, replace=False)) for _ in range(2)])
                     for _ in range(3)]).astype(np.int32).reshape(3, 1, 2, 96)
    out, lse = G.gpu_attention(inp, w, sets)
    for l in (0, 1, 31, 62, 63):
        for t in range(2):
            rows = O.attention_rows(inp["kv_codes"][0], inp["kv_scales"][0], sets[layer_set[l], 0, t],
                                    inp["swa"][l, 0], int(inp["swa_end"][0, t]), w.swa_window)
            o, ls = O.attention(inp["q"][l, 0, t], rows, 1 / math.sqrt(512))
            G.assert_attention_close(out[l, 0, t], o, f"l{l} t{t}")
            assert np.allclose(lse[l, 0, t], ls, rtol=1e-3, atol=1e-3)
