"""CPU checks of the C ABI: the library loads, exports every entry point include/csa2.h
declares, and rejects bad arguments on the host before anything is enqueued."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def H():
    import hierarchical_kv_indexer_amd as H
    if not os.path.exists(H.LIB_PATH):
        from hierarchical_kv_indexer_amd import build
        build.build()
    H.lib()
    return H


def declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(H):
    names = declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(H.lib(), n), n
    assert set(names) == {e[0] for e in H.EXPORTS}


def test_workspace_sizes(H):
    assert H.csa2_index_full_workspace(1, 1, 1 << 20, 8, 2048, 512) >= (1 << 20) * 4 + (1 << 17) * 4
    assert H.csa2_reindex_workspace(4, 1, 1, 16384, 512) >= 4 * 16384 * 4
    assert H.csa2_index_full_workspace(0, 1, 10, 8, 4, 4) == 0
    full = H.csa2_index_stages_workspace(1, 1, 1 << 20, 8, 2048, 512)
    assert H.csa2_index_full_workspace(1, 1, 1 << 20, 8, 2048, 512) == full   # one batch
    # the chain adds, after the Full workspace, the slot scores of the Full layer's Top-K item and
    # of each Reindex layer (16384 fp32 scores each)
    per_item = 16384 * 4
    assert H.csa2_index_chain_workspace(1, 1, 1 << 20, 8, 2048, 512, 0) >= full + per_item
    assert H.csa2_index_chain_workspace(1, 1, 1 << 20, 8, 2048, 512, 4) >= full + 5 * per_item
    assert H.csa2_index_chain_workspace(1, 1, 1 << 20, 8, 0, 512, 4) == 0     # the chain needs a pool


def test_full_workspace_is_batched(H):
    """csa2_index_full works through the queries in batches: 4096 causal queries over 32768
    entries (Top-512, no pool) run as 16 batches of 256 queries (one per CU) in under 64 MiB,
    where the separate stages, which keep every query's scores, need over 512 MiB.  Batches too
    small to fill the GPU are used only past the spill cap (1 GiB)."""
    MiB = 1 << 20
    assert H.csa2_index_full_workspace(1, 4096, 32768, 8, 0, 512) <= 64 * MiB
    assert H.csa2_index_stages_workspace(1, 4096, 32768, 8, 0, 512) >= 512 * MiB
    # 256 queries at 2^19 entries: batches of 16 would leave most CUs idle, so one batch
    assert H.csa2_index_full_workspace(1, 256, 1 << 19, 8, 0, 512) == H.csa2_index_stages_workspace(1, 256, 1 << 19, 8, 0, 512)
    # many short sequences: batches of whole sequences, at least 256 queries each
    assert H.csa2_index_full_workspace(64, 8, 131072, 8, 2048, 512) < 0.6 * H.csa2_index_stages_workspace(64, 8, 131072, 8, 2048, 512)
    # past the spill cap (2048 queries at 2^20 entries: 8 GiB of scores) batches of 16 queries
    assert H.csa2_index_full_workspace(1, 2048, 1 << 20, 8, 0, 512) <= 96 * MiB
    # small shapes: one batch, the stages' workspace
    assert H.csa2_index_full_workspace(2, 3, 5000, 8, 64, 256) == H.csa2_index_stages_workspace(2, 3, 5000, 8, 64, 256)


FAKE = 1 << 20   # a 16-byte aligned non-null value; validation fails before it is used


def expect(H, status, fn, *args):
    with pytest.raises(H.Csa2Error) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)


def test_index_full_rejects(H):
    ok = [FAKE, None, 4096, FAKE, FAKE, FAKE, 1, 1, 4096, 8, 64, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30]
    def call(**ch):
        a = list(ok)
        names = ["idx_k", "idx_ks", "k_rows", "idx_q", "head_w", "nvis", "B", "T", "n_max", "block", "P", "K",
                 "pool_pos", "pool_len", "topk_idx", "topk_score", "ws", "ws_bytes"]
        for k, v in ch.items():
            a[names.index(k)] = v
        return lambda: H.csa2_index_full(*a)
    expect(H, 1, call(idx_k=None))
    expect(H, 1, call(idx_q=FAKE + 4))                 # misaligned
    expect(H, 1, call(idx_ks=FAKE + 8))                # misaligned FP4 key scales
    expect(H, 2, call(block=16))
    expect(H, 1, call(K=600))                          # top_k > pool capacity
    expect(H, 2, call(K=4096))
    expect(H, 2, call(P=4096))                         # pool > 16384 positions
    expect(H, 1, call(n_max=5000))                     # n_max > k_rows
    expect(H, 3, call(ws_bytes=16))
    expect(H, 3, call(ws=None))
    expect(H, 1, call(B=0))


def test_reindex_and_attention_reject(H):
    expect(H, 1, lambda: H.csa2_reindex(FAKE, None, 100, FAKE, FAKE, FAKE, FAKE, 512, 1, 1, 1, 1024, FAKE, None, FAKE, 1 << 30))
    expect(H, 2, lambda: H.csa2_reindex(FAKE, None, 100, FAKE, FAKE, FAKE, FAKE, 20000, 1, 1, 1, 512, FAKE, None, FAKE, 1 << 30))
    expect(H, 3, lambda: H.csa2_reindex(FAKE, None, 100, FAKE, FAKE, FAKE, FAKE, 1024, 1, 1, 1, 512, FAKE, None, FAKE, 8))
    base = [FAKE, FAKE, 100, FAKE, FAKE, [0, 0], 1, FAKE, 128, FAKE, 128, 2, 1, 1, 16, 512, 0.04, FAKE, None, None, 0]
    a = list(base); a[14] = 24                                       # H not a multiple of 16
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[5] = [0, 3]                                    # layer_set out of range
    expect(H, 1, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[16] = 0.0
    expect(H, 1, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[11] = 65; a[5] = [0] * 65
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[19] = None; a[20] = 0                          # split rows need a workspace
    expect(H, 3, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[10] = 4097                                     # window beyond 4096
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[15] = 2049                                     # top_k beyond 2048
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[14] = 1040                                     # more than 1024 heads
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[12] = 65536                                    # L*B*T beyond 65535
    expect(H, 2, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[18] = FAKE + 4                                 # lse not 16-byte aligned
    expect(H, 1, lambda: H.csa2_sparse_attn(*a))
    a = list(base); a[2] = 0                                         # no main-KV rows
    expect(H, 1, lambda: H.csa2_sparse_attn(*a))


def test_stage_entries_reject(H):
    # pool stage: a caller pool is required when pool_blocks > 0
    expect(H, 1, lambda: H.csa2_index_pool(FAKE, 1, 1, 4096, 8, 64, 64, None, FAKE, FAKE, 1 << 30))
    expect(H, 2, lambda: H.csa2_index_pool(FAKE, 1, 1, 4096, 16, 64, 64, FAKE, FAKE, FAKE, 1 << 30))
    expect(H, 3, lambda: H.csa2_index_pool(FAKE, 1, 1, 4096, 8, 64, 64, FAKE, FAKE, FAKE, 64))
    # top-k stage: output required, internal pool allowed when pool_blocks == 0
    expect(H, 1, lambda: H.csa2_index_topk(1, 1, 4096, 8, 64, 64, FAKE, FAKE, None, None, FAKE, 1 << 30))
    expect(H, 1, lambda: H.csa2_index_topk(1, 1, 4096, 8, 0, 64, None, None, FAKE, FAKE + 4, FAKE, 1 << 30))
    expect(H, 3, lambda: H.csa2_index_topk(1, 1, 4096, 8, 0, 64, None, None, FAKE, None, FAKE, 8))


def test_chain_entries_reject(H):
    ws = H.csa2_index_chain_workspace(1, 1, 4096, 8, 64, 64, 2)
    ok = dict(pool_pos=FAKE, pool_len=FAKE, topk_idx=FAKE, topk_score=None, ri_topk_idx=FAKE, ri_topk_score=None)

    def chain(pool_blocks=64, L=2, ri_q=FAKE, ws_bytes=ws, **kw):
        a = dict(ok, **kw)
        H.csa2_index_chain(FAKE, None, 4096, FAKE, FAKE, FAKE, 1, 1, 4096, 8, pool_blocks, 64, ri_q, FAKE, L,
                           a["pool_pos"], a["pool_len"], a["topk_idx"], a["topk_score"], a["ri_topk_idx"],
                           a["ri_topk_score"], FAKE, ws_bytes)

    expect(H, 1, lambda: chain(pool_blocks=0))                 # no pool
    expect(H, 1, lambda: chain(ri_q=None))                     # Reindex query missing
    expect(H, 1, lambda: chain(ri_topk_idx=None))              # Reindex output missing
    expect(H, 1, lambda: chain(pool_len=None))
    expect(H, 2, lambda: chain(L=70000))
    expect(H, 3, lambda: chain(ws_bytes=ws - 256))
    # without the scan: the Full query is not needed, the keys and the pool still are
    expect(H, 1, lambda: H.csa2_index_select_reindex(None, None, 4096, FAKE, 1, 1, 4096, 8, 64, 64, FAKE, FAKE, 2, FAKE,
                                                     FAKE, FAKE, None, FAKE, None, FAKE, ws))
    expect(H, 3, lambda: H.csa2_index_select_reindex(FAKE, None, 4096, FAKE, 1, 1, 4096, 8, 64, 64, None, None, 0, FAKE,
                                                     FAKE, FAKE, None, None, None, FAKE, 64))


def test_quantize_kv_rejects(H):
    H.csa2_quantize_kv_fp4(None, 0, None, None)                          # no rows: nothing to check
    expect(H, 1, lambda: H.csa2_quantize_kv_fp4(FAKE, -1, FAKE, FAKE))
    expect(H, 1, lambda: H.csa2_quantize_kv_fp4(FAKE, 4, None, FAKE))
    expect(H, 1, lambda: H.csa2_quantize_kv_fp4(FAKE, 4, FAKE, FAKE + 8))  # misaligned scales


def test_encoder_chunk_rejects(H):
    assert H.csa2_encoder_chunk_workspace(1, 256, 1 << 19, 6, 64, 512, 128) > 256 * (1 << 19) * 4
    assert H.csa2_encoder_chunk_workspace(1, 256, 1 << 22, 6, 64, 512, 128) == 0      # k_rows beyond 2^21
    assert H.csa2_encoder_chunk_workspace(1, 256, 1 << 19, 6, 24, 512, 128) == 0      # H % 16 != 0
    ws = H.csa2_encoder_chunk_workspace(1, 128, 4096, 6, 64, 512, 128)
    # G, layers, new_idx_k, new_latent, idx_k, kv_codes, kv_scales, k_rows, idx_q, head_w, q, swa, swa_rows,
    # B, T, p0, m, H, top_k, window, scale, out, topk, ws, ws_bytes
    ok = [3, 6, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, 127 + 128, 1, 128, 1024, 2, 64, 512,
          128, 0.044, FAKE, None, FAKE, ws]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return lambda: H.csa2_encoder_chunk(*a)
    expect(H, 1, call(0, 0))                    # G
    expect(H, 2, call(1, 65))                   # layers
    expect(H, 1, call(16, 0))                   # m
    expect(H, 1, call(15, 8192))                # entries beyond k_rows
    expect(H, 1, call(12, 128))                 # swa_rows != min(p0, window - 1) + T
    expect(H, 1, call(4, None))                 # idx_k
    expect(H, 1, call(3, FAKE + 2))             # new_latent alignment
    expect(H, 3, call(24, 64))                  # workspace
    a = list(ok)
    a[15], a[12] = 0, 128                       # first chunk: no history rows
    a[24] = 8
    expect(H, 3, lambda: H.csa2_encoder_chunk(*a))
    # pointers only the nested Full-layer and attention calls use are checked before the cache
    # appends: without a GPU any launch would fail with CSA2_ERR_HIP, so an argument error here
    # means nothing was enqueued (the caches stay untouched)
    for i in (8, 9, 10, 21):                    # idx_q, head_w, q, out
        expect(H, 1, call(i, None))
    expect(H, 1, call(22, FAKE + 4))            # topk_idx alignment
    expect(H, 2, call(17, 40))                  # H
    expect(H, 2, call(18, 4096))                # top_k


def test_noalloc_chain_rejects(H):
    """csa2_index_chain_noalloc: the chain's argument errors, then shapes beyond its fixed scratch,
    all before anything is enqueued (without a GPU a launch or the scratch lookup would fail with
    CSA2_ERR_HIP)."""
    cap = H.csa2_noalloc_scratch_bytes()
    assert cap == 16 << 20
    for B, N in ((1, 1 << 20), (8, 131072), (1, 1 << 21)):
        assert H.csa2_index_chain_workspace(B, 1, N, 8, 2048, 512, 4) <= cap, (B, N)
    assert H.csa2_index_chain_workspace(16, 1, 1 << 21, 8, 2048, 512, 4) > cap
    # idx_k, ks, rows, idx_q, head_w, nvis, B, T, n_max, block, P, K, ri_q, ri_w, L, pool_pos, pool_len,
    # topk_idx, topk_score, ri_topk_idx, ri_topk_score
    ok = [FAKE, None, 1 << 21, FAKE, FAKE, FAKE, 16, 1, 1 << 21, 8, 2048, 512, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None,
          FAKE, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return lambda: H.csa2_index_chain_noalloc(*a)
    expect(H, 2, call(6, 16))                   # 16 queries at 2^21 positions: beyond the scratch
    expect(H, 1, call(6, 0))                    # B
    expect(H, 1, call(3, None))                 # idx_q
    expect(H, 2, call(10, 4096))                # pool beyond 16384 positions
    expect(H, 1, call(12, None))                # ri_q with L > 0


def test_scan_blocks_rejects_unknown_block_score(H):
    ws = H.csa2_index_stages_workspace(1, 1, 4096, 8, 64, 64)
    expect(H, 1, lambda: H.csa2_index_scan_blocks(FAKE, None, 4096, FAKE, FAKE, FAKE, 1, 1, 4096, 8, 64, 64, 3,
                                                  FAKE, ws))
