"""Pins of the oracle's indexer, pool and Top-K steps.

Each pin rests on something other than the oracle's own code: exact integer
arithmetic on E4M3 values decoded by PyTorch, a hand-worked example
(tests/golden/worked_scores.txt), the ordering characterisation of a Top-k set,
a different sorting routine (Python's ``sorted``), the block-prefilter lemma,
and the invariants the pages state (Reindex picks inside the pool; a position
outside the pool cannot be picked by a Reindex layer)."""
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import csa2 as O
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_int(codes):
    """E4M3 bytes -> exact integers in units of 2^-9 (decoded by PyTorch)."""
    v = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    x = v.to(torch.float64).numpy() * 512.0
    assert np.all(x == np.round(x))
    return x.astype(np.int64)


def torch_q8(q_bf16):
    t = torch.from_numpy(np.ascontiguousarray(q_bf16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def rand_case(rng, n=300):
    k8 = workloads.to_e4m3_bytes(rng.standard_normal((n, 128), dtype=np.float32))
    q = workloads.to_bf16_bits(rng.standard_normal((32, 128), dtype=np.float32))
    return k8, q


def test_worked_example_scores():
    rows = []
    with open(os.path.join(GOLDEN, "worked_scores.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                r, c0, c1, s = line.split()
                rows.append((int(r), int(c0, 16), int(c1, 16), float(s)))
    k8 = np.zeros((len(rows), 128), np.uint8)
    for r, c0, c1, _ in rows:
        k8[r, 0], k8[r, 1] = c0, c1
    qf = np.zeros((32, 128), np.float32)
    qf[0, 0], qf[1, 1] = 1.0, 2.0
    w = np.ones(32, np.float32)
    w[0], w[1] = 0.5, 0.25
    s = O.indexer_scores(k8, O.quantize_query(workloads.to_bf16_bits(qf)), w)
    assert list(s) == [r[3] for r in rows]


def test_quantize_query_matches_torch():
    rng = np.random.default_rng(1)
    q = workloads.to_bf16_bits(rng.standard_normal((32, 128), dtype=np.float32) * 3)
    assert np.array_equal(O.quantize_query(q), torch_q8(q))


@pytest.mark.parametrize("h", [0, 7, 31])
def test_single_head_score_is_exact_integer_dot(h):
    rng = np.random.default_rng(10 + h)
    k8, q = rand_case(rng)
    w = np.zeros(32, np.float32)
    w[h] = 1.0
    s = O.indexer_scores(k8, O.quantize_query(q), w)
    d = torch_e4m3_int(k8) @ torch_e4m3_int(torch_q8(q))[h]   # exact, units of 2^-18
    expect = np.maximum(d, 0).astype(np.float64) * 2.0 ** -18
    assert np.array_equal(s, expect)
    assert (d < 0).any() and (d > 0).any()


def test_two_head_weighted_sum_exact():
    rng = np.random.default_rng(3)
    k8, q = rand_case(rng)
    w = np.zeros(32, np.float32)
    w[4], w[19] = 0.5, 0.25
    s = O.indexer_scores(k8, O.quantize_query(q), w)
    qi = torch_e4m3_int(torch_q8(q))
    ki = torch_e4m3_int(k8)
    d4, d19 = ki @ qi[4], ki @ qi[19]
    expect = (2 * np.maximum(d4, 0) + np.maximum(d19, 0)).astype(np.float64) * 2.0 ** -20
    assert np.array_equal(s, expect)


def test_head_permutation_and_weight_scaling():
    rng = np.random.default_rng(4)
    k8, q = rand_case(rng)
    w = rng.random(32, dtype=np.float32)
    s = O.indexer_scores(k8, O.quantize_query(q), w)
    perm = rng.permutation(32)
    sp = O.indexer_scores(k8, O.quantize_query(q[perm]), w[perm])
    assert np.allclose(s, sp, rtol=1e-14, atol=0)
    s2 = O.indexer_scores(k8, O.quantize_query(q), 2 * w)
    assert np.array_equal(s2, 2 * s)
    assert np.all(s >= 0)


def topk_by_sorted(keys, ids, k):
    """Reference ranking with Python's sorted on (-key, id) tuples."""
    order = sorted(zip((-float(x) for x in keys), (int(i) for i in ids)))
    return sorted(i for _, i in order[:k])


def check_topk_characterisation(cand, s, k, sel):
    sel = [int(x) for x in sel if x >= 0]
    assert len(sel) == min(k, len(cand))
    assert sel == sorted(sel)
    sc = dict(zip([int(c) for c in cand], [float(x) for x in s]))
    chosen = set(sel)
    rest = [int(p) for p in cand if int(p) not in chosen]
    if chosen and rest:
        # every chosen (score, position) ranks before every unchosen one
        assert max((-sc[c], c) for c in chosen) < min((-sc[p], p) for p in rest)


@pytest.mark.parametrize("seed", range(5))
def test_topk_selection_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    cand = np.sort(rng.choice(1000, size=n, replace=False)).astype(np.int32)
    s = rng.integers(0, 6, size=n).astype(np.float32)      # heavy ties
    k = int(rng.integers(1, 80))
    got = O.top_k(cand, s, k)
    assert got.shape == (k,)
    assert np.all(got[min(k, n):] == -1)
    assert list(got[got >= 0]) == topk_by_sorted(s, cand, k)
    check_topk_characterisation(cand, s, k, got)


def brute_pool(blk, n_vis, block, P):
    nb = len(blk)
    order = sorted(range(nb), key=lambda j: (-float(blk[j]), j))
    chosen = sorted(order[:P])
    return [p for j in chosen for p in range(j * block, min((j + 1) * block, n_vis))]


@pytest.mark.parametrize("seed", range(6))
def test_pool_is_top_blocks_and_contains_dense_topk(seed):
    rng = np.random.default_rng(100 + seed)
    n_vis = int(rng.integers(1, 700))
    block = 8
    s32 = rng.integers(0, 9, size=n_vis).astype(np.float32)   # ties within and across blocks
    P = int(rng.integers(1, 40))
    k = int(rng.integers(1, P * block + 1))
    blk = O.block_scores(s32, n_vis, block)
    nb = -(-n_vis // block)
    assert len(blk) == nb
    for j in range(nb):
        assert blk[j] == s32[j * block:(j + 1) * block].max()
    pool = O.candidate_pool(blk, n_vis, block, P)
    assert list(pool) == brute_pool(blk, n_vis, block, P)
    # whole blocks, ascending, min(P, nb) of them
    blocks = sorted(set(int(p) // block for p in pool))
    assert len(blocks) == min(P, nb)
    assert list(pool) == sorted(pool)
    # lemma: the dense Top-k (every visible position) lies inside the pool, so the
    # Top-k over the pool equals the dense Top-k, tie-breaks included (k <= P*block)
    k = min(k, P)
    dense = topk_by_sorted(s32, np.arange(n_vis), k)
    assert set(dense) <= set(int(p) for p in pool)
    assert list(O.top_k(pool, s32[pool], k)[:len(dense)]) == dense


def test_full_layer_no_pool_and_degenerate_visibility():
    rng = np.random.default_rng(7)
    k8 = workloads.to_e4m3_bytes(rng.standard_normal((50, 128), dtype=np.float32))
    q = workloads.to_bf16_bits(rng.standard_normal((32, 128), dtype=np.float32))
    w = rng.random(32, dtype=np.float32)
    # n_vis = 0: empty pool, all -1
    f0 = O.full_layer(k8, q, w, 0, 8, 4, 16)
    assert f0["pool"].shape == (0,) and np.all(f0["topk"] == -1)
    # n_vis < k: every visible position selected, ragged last block
    f1 = O.full_layer(k8, q, w, 13, 8, 4, 16)
    assert list(f1["pool"]) == list(range(13))
    assert list(f1["topk"][:13]) == list(range(13)) and np.all(f1["topk"][13:] == -1)
    # no pool: dense Top-k
    f2 = O.full_layer(k8, q, w, 50, 8, 0, 10)
    assert f2["pool"] is None
    assert list(f2["topk"]) == topk_by_sorted(f2["scores32"], np.arange(50), 10)


def small_decode(seed=5, N=2000, P=16, k=32):
    return workloads.Workload("t", seed, B=1, T=1, N=N, H=4, layer_set=(0, 1, 1, 2),
                              n_reindex=2, pool_blocks=P, top_k=k)


def test_reindex_inside_pool_and_reproduces_full():
    w = small_decode()
    inp = workloads.make_inputs(w, with_attention=False)
    out = O.query_chain(inp, w, 0, 0, with_attention=False)
    pool = set(int(p) for p in out["full"]["pool"])
    for ri in out["reindex"]:
        sel = [int(p) for p in ri["topk"] if p >= 0]
        assert len(sel) == w.top_k and set(sel) <= pool
    # a Reindex layer given the Full layer's own query and weights picks the Full Top-k
    same = O.reindex_layer(inp["idx_k"][0], inp["idx_q"][0, 0], inp["head_w"][0, 0],
                           out["full"]["pool"], w.top_k)
    assert np.array_equal(same["topk"], out["full"]["topk"])
    assert np.array_equal(same["topk_score"], out["full"]["topk_score"])
    # a position outside the pool cannot be picked, even if it scores highest
    outside = next(p for p in range(w.N) if p not in pool)
    s_all = O.indexer_scores(inp["idx_k"][0], O.quantize_query(inp["ri_q"][0, 0, 0]), inp["ri_w"][0, 0, 0])
    assert outside not in set(out["reindex"][0]["topk"].tolist())
    assert s_all.shape == (w.N,)


def test_prefill_visibility_readings():
    w = workloads.WORKLOADS["prefill_4k_64k"]
    nv = w.n_visible()
    # the chunk is the last 4096 tokens of 65536 (p = 61440 .. 65535), m = 2 tokens per entry,
    # only complete entries are visible
    assert nv[0, 0] == 30720 and nv[0, -1] == 32768 and nv[0, 1] == 30721 and nv[0, 2] == 30721
    se = w.swa_end()
    assert se[0, 0] == 128 and se[0, -1] == 4096 + 127 and w.swa_rows == 4223


def test_planted_cluster_recall_small():
    w = workloads.small_variant(workloads.WORKLOADS["decode_1m"], N=65536, seed=77)
    inp = workloads.make_inputs(w, with_attention=False)
    out = O.query_chain(inp, w, 0, 0, with_attention=False)
    assert np.isin(inp["planted_pos"], out["full"]["topk"]).all()


def test_workload_shapes_match_page_figures():
    from tests.test_oracle_formats import page_figures
    figs = page_figures()
    for name in ("decode_b8_128k", "decode_1m"):
        w = workloads.WORKLOADS[name]
        assert w.pool_blocks == figs["pool_blocks"] and w.block == figs["pool_block_size"]
        assert w.pool_cap == figs["pool_positions"] and w.top_k == figs["top_k"]
    assert workloads.IDX_HEADS == figs["indexer_heads"] and workloads.IDX_DIM == figs["indexer_head_dim"]
    assert workloads.KV_DIM // workloads.KV_SCALE_BYTES == figs["scale_group"]


# ------------------------------------------------------------------ FP4 indexer K (variant)

def _e4m3_bytes_of(values: np.ndarray) -> np.ndarray:
    """Exactly representable values -> E4M3 bytes, through torch's cast (checked exact)."""
    t = torch.from_numpy(np.asarray(values, np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(t.to(torch.float64).numpy(), np.asarray(values, np.float64))
    return t.view(torch.uint8).numpy()


def test_fp4_keys_at_unit_scale_score_like_the_same_e4m3_keys():
    """With every scale 1, FP4 key values are E2M1 values, all exact in E4M3: the FP4 path must
    give exactly the E4M3 path's scores on the same values (that path is pinned above)."""
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 256, size=(300, 64), dtype=np.uint8)
    scales = np.full((300, 8), 0x38, np.uint8)                       # 1.0
    vals = F.kv_row_values(codes, scales)                            # [300][128]
    k8 = _e4m3_bytes_of(vals)
    q = workloads.to_bf16_bits(rng.standard_normal((32, 128)).astype(np.float32))
    w = rng.random(32, dtype=np.float32)
    q8 = O.quantize_query(q)
    assert np.array_equal(O.indexer_scores((codes, scales), q8, w), O.indexer_scores(k8, q8, w))


def test_fp4_key_channel_order_and_scale_groups():
    """A key with one non-zero channel c (code 1.0) and scale group g = c // 16 set to 2^(g-3):
    the one-head score with q = e_c is w * 2^(g-3), so channel c decodes at c (even channels in
    the low nibble) with its own group's scale."""
    q = np.zeros((32, 128), np.float32)
    w = np.zeros(32, np.float32)
    w[0] = 1.0
    scales = np.array([[0x38 + 8 * (g - 3) for g in range(8)]], np.uint8)   # 2^(g-3)
    for c in (0, 1, 14, 15, 16, 17, 63, 64, 126, 127):
        codes = np.zeros((1, 64), np.uint8)
        codes[0, c // 2] = 0x2 << (4 * (c & 1))                       # E2M1 1.0
        qq = q.copy()
        qq[0, c] = 1.0
        s = O.indexer_scores((codes, scales), O.quantize_query(workloads.to_bf16_bits(qq)), w)
        assert s[0] == 2.0 ** (c // 16 - 3), c


def test_fp4_key_scores_are_homogeneous_in_the_scales():
    """Doubling every scale (E4M3 exponent + 1) doubles every score exactly."""
    rng = np.random.default_rng(42)
    codes = rng.integers(0, 256, size=(200, 64), dtype=np.uint8)
    scales = rng.integers(0x20, 0x70, size=(200, 8), dtype=np.uint8)
    q8 = O.quantize_query(workloads.to_bf16_bits(rng.standard_normal((32, 128)).astype(np.float32)))
    w = rng.random(32, dtype=np.float32)
    s1 = O.indexer_scores((codes, scales), q8, w)
    s2 = O.indexer_scores((codes, scales + 8), q8, w)
    assert np.array_equal(s2, 2 * s1)


def test_fp4_key_workload_chain_selection_properties():
    """The tiny workload with FP4 keys: the pool holds the dense Top-K (lemma S6 on the FP4
    scores) and the planted cluster of a small planted variant is recalled."""
    w = workloads.small_variant(workloads.WORKLOADS["decode_1m_fp4k"], N=65536, seed=4301)
    inp = workloads.make_inputs(w, with_attention=False)
    assert inp["idx_k_codes"].shape == (1, 65536, 64) and inp["idx_k_scales"].shape == (1, 65536, 8)
    r = O.query_chain(inp, w, 0, 0, with_attention=False)
    f = r["full"]
    dense = O.top_k(np.arange(w.N, dtype=np.int32), f["scores32"], w.top_k)
    assert np.array_equal(f["topk"], dense)
    assert np.isin(inp["planted_pos"], f["topk"]).all()


# ---------------------------------------------------------------- block-score variants (recall study)

def test_block_score_variants_by_hand():
    s32 = np.array([1, 5, 3, 5, 2, 0, 4, 1, 7, 6, -1, 2, 9], np.float32)   # blocks of 4: 3 full + 1 partial
    assert O.block_scores(s32, 13, 4, "max").tolist() == [5, 4, 7, 9]
    assert O.block_scores(s32, 13, 4, "sum").tolist() == [14, 7, 14, 9]
    assert O.block_scores(s32, 13, 4, "top2").tolist() == [5, 3, 6.5, 9]    # ties count twice; one position
    assert O.block_scores(s32, 12, 4, "top2").tolist() == [5, 3, 6.5]


def test_block_score_variants_brute_force():
    rng = np.random.default_rng(12)
    for n in (1, 7, 8, 9, 63):
        s32 = rng.standard_normal(n).astype(np.float32)
        for j, (mx, sm, t2) in enumerate(zip(O.block_scores(s32, n, 8, "max"), O.block_scores(s32, n, 8, "sum"),
                                              O.block_scores(s32, n, 8, "top2"))):
            blk = sorted((float(x) for x in s32[8 * j:8 * j + 8]), reverse=True)
            assert mx == np.float32(blk[0])
            assert sm == np.float32(sum(blk))
            assert t2 == np.float32((blk[0] + blk[1]) / 2 if len(blk) > 1 else blk[0])


def test_only_the_max_block_score_keeps_an_isolated_needle():
    """One very high score alone in its block against dense blocks of moderate scores: the max
    block score keeps the needle's block in a one-block pool (so the dense Top-1 is in the pool,
    lemma S6), while the sum and the top-2 mean prefer a dense block and lose it."""
    s32 = np.full(64, 1.0, np.float32)
    s32[0:8] = 0.0
    s32[3] = 5.0                      # the needle
    s32[40:48] = 3.0                  # a dense block
    for mode, keeps in (("max", True), ("sum", False), ("top2", False)):
        pool = O.candidate_pool(O.block_scores(s32, 64, 8, mode), 64, 8, 1)
        assert (3 in pool.tolist()) == keeps, mode


# ------------------------------------------------------------------ FP4 query (with FP4 keys)

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _fp4_group_brute_force(x: np.ndarray) -> np.ndarray:
    """One 16-value group rounded to FP4 by brute force, independently of the oracle's codecs:
    scale = torch's E4M3 cast of float32(amax / 6); each |x| / scale goes to the nearest E2M1
    magnitude (exact rational distances, ties to the even code), saturating at 6."""
    from fractions import Fraction
    amax = np.float32(np.max(np.abs(x)))
    s32 = np.float32(amax / np.float32(6.0))
    s = float(torch.tensor(s32).to(torch.float8_e4m3fn).to(torch.float64))
    out = np.zeros(16)
    if s == 0.0:
        return out
    for i, v in enumerate(x.astype(np.float64)):
        q = Fraction(abs(v)) / Fraction(s)
        d = [abs(q - Fraction(m)) for m in E2M1_MAGS]
        best = min(range(8), key=lambda c: (d[c], c % 2))            # ties: even code
        out[i] = np.copysign(E2M1_MAGS[best] * s, v)
    return out


def test_fp4_query_matches_a_brute_force_per_head_group():
    """[p3 FP4]: with FP4 keys the query is rounded to FP4 per head and 16-channel group.  Random
    queries of several magnitudes (and one group of zeros) against a brute force over each group."""
    rng = np.random.default_rng(71)
    for scale in (1.0, 1e-3, 37.0):
        qf = (rng.standard_normal((32, 128)) * scale).astype(np.float32)
        qf[5, 32:48] = 0.0
        q = workloads.to_bf16_bits(qf)
        got = O.query_values(O.quantize_query_fp4(q))
        x = F.bf16_value(q)
        for h in range(32):
            for g in range(8):
                ref = _fp4_group_brute_force(x[h, 16 * g:16 * g + 16])
                assert np.array_equal(got[h, 16 * g:16 * g + 16], ref), (scale, h, g)


def test_fp4_query_round_trips_fp4_values_and_groups_are_independent():
    """A query whose every group is code x scale with a +-6 code already is returned unchanged; a
    change inside one group leaves every other group's values alone."""
    rng = np.random.default_rng(72)
    codes = rng.integers(0, 16, size=(32, 128))
    codes[:, ::16] = rng.choice([7, 15], size=(32, 8))                # a +-6 code in every group
    sc = 2.0 ** rng.integers(-6, 4, size=(32, 8)) * (1 + rng.integers(0, 8, size=(32, 8)) / 8)
    vals = np.where(codes >= 8, -1, 1) * E2M1_MAGS[codes % 8] * np.repeat(sc, 16, axis=1)
    q = workloads.to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(F.bf16_value(q), vals)                      # exact in bf16
    v1 = O.query_values(O.quantize_query_fp4(q))
    assert np.array_equal(v1, vals)
    q2 = q.copy()
    q2[3, 20] = workloads.to_bf16_bits(np.float32([1000.0]))[0]       # group (3, 1) only
    v2 = O.query_values(O.quantize_query_fp4(q2))
    mask = np.ones((32, 128), bool)
    mask[3, 16:32] = False
    assert np.array_equal(v2[mask], v1[mask]) and not np.array_equal(v2[3, 16:32], v1[3, 16:32])


def test_fp4_keys_score_with_the_fp4_query():
    """The Full layer with FP4 keys scores with the FP4 query: its scores equal indexer_scores with
    that query, and a one-hot key reads back one rounded query value."""
    rng = np.random.default_rng(73)
    codes = rng.integers(0, 256, size=(100, 64), dtype=np.uint8)
    scales = rng.integers(0x30, 0x48, size=(100, 8), dtype=np.uint8)
    q = workloads.to_bf16_bits(rng.standard_normal((32, 128)).astype(np.float32))
    w = rng.random(32, dtype=np.float32)
    r = O.full_layer((codes, scales), q, w, 100, 8, 0, 10)
    assert np.array_equal(r["scores"], O.indexer_scores((codes, scales), O.quantize_query_fp4(q), w))
    one = np.zeros((1, 64), np.uint8)
    one[0, 9] = 0x2 << 4                                              # channel 19: E2M1 1.0
    w1 = np.zeros(32, np.float32)
    w1[7] = 1.0
    s = O.indexer_scores((one, np.full((1, 8), 0x38, np.uint8)), O.quantize_query_fp4(q), w1)
    assert s[0] == max(0.0, O.query_values(O.quantize_query_fp4(q))[7, 19])
