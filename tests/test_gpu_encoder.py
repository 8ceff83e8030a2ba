"""GPU parity of the encoder prefill entry (csa2_encoder_chunk) against the oracle: a prompt run
chunk by chunk from empty caches through groups of one Full and several Reuse layers."""
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


def enc(**kw):
    base = dict(name="enc_gpu", seed=78, B=1, G=2, layers=3, H=64, prompt=512, T=128, m=2, top_k=64,
                swa_window=32)
    base.update(kw)
    return workloads.EncoderPrefill(**base)


def oracle_run(w, prompt, chunks):
    """The oracle over the prompt in the given chunks; returns per-chunk results and the caches."""
    n = max(w.prompt // w.m, 1)
    caches = (np.zeros((w.G, w.B, n, 128), np.uint8), np.zeros((w.G, w.B, n, 256), np.uint8),
              np.zeros((w.G, w.B, n, 32), np.uint8))
    res = []
    for p0, T in chunks:
        a = workloads.encoder_chunk_args(w, prompt, p0, T)
        res.append(O.encoder_chunk(*caches, a["new_idx_k"], a["new_latent"], a["idx_q"], a["head_w"], a["q"],
                                   a["swa"], p0, w.m, w.top_k, w.swa_window))
    return res, caches


def chunk_list(prompt, sizes):
    out, p0, i = [], 0, 0
    while p0 < prompt:
        T = min(sizes[i % len(sizes)], prompt - p0)
        out.append((p0, T))
        p0 += T
        i += 1
    return out


def check_chunk(w, prompt, gpu_out, gpu_topk, ref, caches_after, p0, T, what):
    """GPU outputs of one chunk against the oracle: index sets by the tie rule, attention over the
    GPU's own index sets (so a tie swap does not change the reference)."""
    idx_k, kv_codes, kv_scales = caches_after
    a = workloads.encoder_chunk_args(w, prompt, p0, T)
    h = w.hist(p0)
    for g in range(w.G):
        for b in range(w.B):
            for t in range(T):
                n_vis = O.visible_entries(p0 + t, w.m)
                q8 = O.quantize_query(a["idx_q"][g, b, t])
                s = O.indexer_scores(idx_k[g, b, :n_vis], q8, a["head_w"][g, b, t])
                G.assert_topk_equiv(gpu_topk[g, b, t], ref["topk"][g, b, t], lambda p: s[p],
                                    f"{what} g{g} b{b} t{t}")
                for l in range(w.layers):
                    rows = O.attention_rows(kv_codes[g, b], kv_scales[g, b], gpu_topk[g, b, t], a["swa"][g, l, b],
                                            h + t + 1, w.swa_window)
                    o, _ = O.attention(a["q"][g, l, b, t], rows, 1.0 / math.sqrt(512))
                    G.assert_attention_close(gpu_out[g, l, b, t], o, f"{what} g{g} l{l} t{t}")


@pytest.mark.parametrize("sizes,m,B", [((128,), 2, 1), ((33, 64, 95), 3, 1), ((96, 160), 2, 2)])
def test_encoder_chunks_match_oracle(sizes, m, B):
    """Every chunk of a 512-token prompt: index sets, attention of every layer, and the caches
    the chunks append (bytes equal to the oracle's).  Ragged chunk sizes with m = 3 put entry
    boundaries inside chunks; B = 2 runs two prompts side by side."""
    w = enc(m=m, B=B)
    prompt = workloads.make_encoder_prompt(w)
    chunks = chunk_list(w.prompt, sizes)
    ref, caches = oracle_run(w, prompt, chunks)
    gpu = G.GpuEncoder(w, max(T for _, T in chunks))
    for (p0, T), r in zip(chunks, ref):
        out, topk = gpu.chunk(workloads.encoder_chunk_args(w, prompt, p0, T), p0, T)
        check_chunk(w, prompt, out, topk, r, caches, p0, T, f"chunk {p0}+{T}")
    assert np.array_equal(G.host(gpu.idx_k), caches[0])
    assert np.array_equal(G.host(gpu.kv_codes), caches[1])
    assert np.array_equal(G.host(gpu.kv_scales), caches[2])


def test_encoder_chunking_does_not_change_results():
    """Causality on the GPU: chunks of 128 and of 256 tokens give the same index sets for every
    token, and attention outputs within the tolerance of each other."""
    w = enc(layers=6)
    prompt = workloads.make_encoder_prompt(w)
    res = {}
    for size in (128, 256):
        gpu = G.GpuEncoder(w, size)
        outs, topks = [], []
        for p0, T in chunk_list(w.prompt, (size,)):
            o, t = gpu.chunk(workloads.encoder_chunk_args(w, prompt, p0, T), p0, T)
            outs.append(o)
            topks.append(t)
        res[size] = (np.concatenate(outs, axis=3), np.concatenate(topks, axis=2))
    assert np.array_equal(res[128][1], res[256][1])
    a, b = F.bf16_value(res[128][0]), F.bf16_value(res[256][0])
    denom = np.abs(b).max(axis=-1, keepdims=True)
    assert np.all(np.abs(a - b) <= 2e-2 * denom)


def test_encoder_chunk_validation():
    import hierarchical_kv_indexer_amd as H
    w = enc()
    gpu = G.GpuEncoder(w, 128)
    prompt = workloads.make_encoder_prompt(w)
    a = workloads.encoder_chunk_args(w, prompt, 128, 128)
    with pytest.raises(RuntimeError, match="swa_rows"):
        H.csa2_encoder_chunk(w.G, w.layers, G.dev(a["new_idx_k"]), G.dev(a["new_latent"]), gpu.idx_k,
                             gpu.kv_codes, gpu.kv_scales, gpu.k_rows, G.dev(a["idx_q"]), G.dev(a["head_w"]),
                             G.dev(a["q"]), G.dev(a["swa"]), a["swa"].shape[3] + 1, w.B, 128, 128, w.m, w.H,
                             w.top_k, w.swa_window, 0.05, G.empty((1,), torch.int16), None, gpu.ws, gpu.ws_bytes)
    with pytest.raises(RuntimeError, match="k_rows"):
        H.csa2_encoder_chunk(w.G, w.layers, None, None, gpu.idx_k, gpu.kv_codes, gpu.kv_scales, gpu.k_rows,
                             G.dev(a["idx_q"]), G.dev(a["head_w"]), G.dev(a["q"]), G.dev(a["swa"]),
                             a["swa"].shape[3], w.B, 128, 2 * w.prompt, w.m, w.H, w.top_k, w.swa_window, 0.05,
                             G.empty((1,), torch.int16), None, gpu.ws, gpu.ws_bytes)
