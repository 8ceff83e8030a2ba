"""GPU check of csa2_index_chain_noalloc (the indexer chain with the library's own scratch, for
callers that cannot allocate): its outputs equal those of csa2_index_chain with a caller
workspace, bit for bit, on two calls in a row where the second is smaller (the scratch keeps the
first call's bytes), and the shared scratch is not reported as a caller workspace."""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_chain as G

pytestmark = pytest.mark.gpu


def _case(B, T, N, P, K, L, seed, fp4=False, nv=None):
    w = workloads.small_variant(workloads.WORKLOADS["tiny_4k"], B=B, T=T, N=N, pool_blocks=P, top_k=K,
                                n_reindex=max(L, 1), seed=seed, idx_k_fp4=fp4)
    inp = workloads.make_inputs(w, with_attention=False)
    if nv is not None:
        inp["n_visible"] = np.asarray(nv, np.int32).reshape(B, T)
    return inp


def _noalloc(inp, B, T, N, P, K, L):
    import hierarchical_kv_indexer_amd as H
    cap = P * 8
    pool_pos = torch.full((B, T, cap), 7, dtype=torch.int32, device=G.DEV)
    pool_len = torch.full((B, T), 7, dtype=torch.int32, device=G.DEV)
    idx = torch.full((B, T, K), 7, dtype=torch.int32, device=G.DEV)
    sc = torch.full((B, T, K), 7.0, dtype=torch.float32, device=G.DEV)
    ri_idx = torch.full((max(L, 1), B, T, K), 7, dtype=torch.int32, device=G.DEV)
    ri_sc = torch.full((max(L, 1), B, T, K), 7.0, dtype=torch.float32, device=G.DEV)
    k, ks, rows = G.keys(inp)
    H.csa2_index_chain_noalloc(k, ks, rows, G.dev(inp["idx_q"]), G.dev(inp["head_w"]), G.dev(inp["n_visible"]),
                               B, T, N, 8, P, K, G.dev(inp["ri_q"][:L]) if L else None,
                               G.dev(inp["ri_w"][:L]) if L else None, L, pool_pos, pool_len, idx, sc,
                               ri_idx if L else None, ri_sc if L else None)
    out = {"topk": G.host(idx), "topk_score": G.host(sc), "pool_pos": G.host(pool_pos),
           "pool_len": G.host(pool_len)}
    if L:
        out["ri_topk"], out["ri_topk_score"] = G.host(ri_idx), G.host(ri_sc)
    return out


def _same(got, ref):
    for key in ref:
        a, b = got[key], ref[key]
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert np.array_equal(a, b), key


@pytest.mark.parametrize("fp4", [False, True])
def test_noalloc_chain_equals_chain_with_workspace_twice(fp4):
    assert torch.cuda.is_available()
    big = dict(B=2, T=2, N=40000, P=512, K=384, L=3)
    small = dict(B=1, T=1, N=6000, P=64, K=100, L=1)
    inp_big = _case(seed=7100 + fp4, fp4=fp4, nv=[40000, 31007, 9999, 40000], **{k: big[k] for k in "BTN"},
                    P=big["P"], K=big["K"], L=big["L"])
    inp_small = _case(seed=7200 + fp4, fp4=fp4, nv=[5993], **{k: small[k] for k in "BTN"}, P=small["P"],
                      K=small["K"], L=small["L"])
    for inp, s in ((inp_big, big), (inp_small, small)):
        print(f"noalloc chain fp4={fp4} shape={s}", flush=True)
        got = _noalloc(inp, s["B"], s["T"], s["N"], s["P"], s["K"], s["L"])
        ref = G.gpu_index_chain(inp, s["B"], s["T"], s["N"], s["P"], s["K"], s["L"])
        _same(got, ref)


def test_noalloc_rejects_beyond_its_scratch():
    import hierarchical_kv_indexer_amd as H
    cap = H.csa2_noalloc_scratch_bytes()
    assert cap == 16 << 20
    assert H.csa2_index_chain_workspace(1, 1, 1 << 21, 8, 2048, 512, 4) <= cap
    assert H.csa2_index_chain_workspace(16, 1, 1 << 21, 8, 2048, 512, 4) > cap
    F = 1 << 20
    with pytest.raises(H.Csa2Error) as e:
        H.csa2_index_chain_noalloc(F, None, 1 << 21, F, F, F, 16, 1, 1 << 21, 8, 2048, 512, F, F, 4, F, F, F, None,
                                   F, None)
    assert e.value.status == 2 and "scratch" in str(e.value)
