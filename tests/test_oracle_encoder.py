"""Pins of the oracle's encoder prefill (a chunk of tokens through groups of one Full and
several Reuse layers over a sequence compressed m tokens per entry).

Each pin rests on something other than the formula under test: brute-force enumeration of
which entries a token sees and which entries a chunk completes, PyTorch's scaled dot-product
attention over row sets built token by token, and causality itself (a prompt run in several
chunks gives the same outputs as in one)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import csa2 as O
from oracle import formats as F


def small(**kw):
    base = dict(name="enc_small", seed=77, B=1, G=2, layers=2, H=16, prompt=48, T=48, m=2, top_k=32,
                swa_window=8)
    base.update(kw)
    return workloads.EncoderPrefill(**base)


def run_chunks(w, prompt, chunk):
    """The oracle over the whole prompt, chunk by chunk, from empty caches."""
    n = w.prompt // w.m
    caches = (np.zeros((w.G, w.B, max(n, 1), 128), np.uint8), np.zeros((w.G, w.B, max(n, 1), 256), np.uint8),
              np.zeros((w.G, w.B, max(n, 1), 32), np.uint8))
    outs, topks = [], []
    for p0 in range(0, w.prompt, chunk):
        T = min(chunk, w.prompt - p0)
        a = workloads.encoder_chunk_args(w, prompt, p0, T)
        r = O.encoder_chunk(*caches, a["new_idx_k"], a["new_latent"], a["idx_q"], a["head_w"], a["q"],
                            a["swa"], p0, w.m, w.top_k, w.swa_window)
        outs.append(r["out"])
        topks.append(r["topk"])
    return np.concatenate(outs, axis=3), np.concatenate(topks, axis=2), caches


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_visible_entries_by_enumeration(m):
    for p in range(60):
        seen = sum(1 for j in range(100) if all(tok <= p for tok in range(j * m, (j + 1) * m)))
        assert O.visible_entries(p, m) == seen


@pytest.mark.parametrize("m", [1, 2, 3])
def test_chunk_completes_exactly_the_entries_it_appends(m):
    rng = np.random.default_rng(5)
    for _ in range(200):
        p0, T = int(rng.integers(0, 200)), int(rng.integers(1, 40))
        done = [j for j in range(300) if p0 <= (j + 1) * m - 1 < p0 + T]   # last token inside the chunk
        assert done == list(range(p0 // m, (p0 + T) // m))


def test_small_context_equals_sdpa_over_visible_entries_and_window():
    """While every token sees at most top_k entries, the Top-k keeps all of them, so each layer
    is plain attention over (every visible entry) + (the token's window), built here token by
    token and evaluated with torch's SDPA in float64."""
    w = small()
    prompt = workloads.make_encoder_prompt(w)
    out, topk, _ = run_chunks(w, prompt, 16)
    codes, scales = F.kv_quantize_rows(prompt["new_latent"])          # [G][B][n][...]
    main = F.kv_row_values(codes, scales)                              # [G][B][n][512]
    swa = F.e4m3_value(prompt["swa"])                                  # [G][L][B][P][512]
    for g in range(w.G):
        for t in range(w.prompt):
            vis = [j for j in range(w.prompt // w.m) if (j + 1) * w.m <= t + 1]
            assert sorted(topk[g, 0, t][topk[g, 0, t] >= 0].tolist()) == vis
            win = list(range(max(0, t - w.swa_window + 1), t + 1))
            for l in range(w.layers):
                rows = np.concatenate([main[g, 0, vis], swa[g, l, 0, win]], axis=0)
                q = torch.from_numpy(F.bf16_value(prompt["q"][g, l, 0, t]))[None, :, None, :]   # [1][H][1][512]
                kv = torch.from_numpy(rows)[None, None].expand(1, w.H, -1, -1)
                ref = torch.nn.functional.scaled_dot_product_attention(q, kv, kv)[0, :, 0].numpy()
                np.testing.assert_allclose(out[g, l, 0, t], ref, rtol=1e-9, atol=1e-12)


def test_chunking_does_not_change_outputs():
    """Causality: the same prompt in chunks of 16, 40 and 64 tokens gives the same index sets
    and outputs for every token, and the same caches (selection active: top_k < entries)."""
    w = small(prompt=64, T=64, top_k=8)
    prompt = workloads.make_encoder_prompt(w)
    ref_out, ref_topk, ref_caches = run_chunks(w, prompt, 64)
    for chunk in (16, 40):
        out, topk, caches = run_chunks(w, prompt, chunk)
        assert np.array_equal(topk, ref_topk)
        np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
        for a, b in zip(caches, ref_caches):
            assert np.array_equal(a, b)


def test_index_sets_are_dense_top_k_of_visible_entries():
    """With selection active, each token's set is the top_k of the visible entries by
    (score desc, entry asc), checked with Python's sorted over exact scores."""
    w = small(prompt=64, T=64, top_k=8)
    prompt = workloads.make_encoder_prompt(w)
    _, topk, caches = run_chunks(w, prompt, 32)
    idx_k = caches[0]
    for g in range(w.G):
        for t in range(0, w.prompt, 7):
            n = (t + 1) // w.m
            q8 = F.e4m3_value(F.e4m3_from_value(F.bf16_value(prompt["idx_q"][g, 0, t])))
            k = F.e4m3_value(idx_k[g, 0, :n])
            s = (np.maximum(q8 @ k.T, 0) * prompt["head_w"][g, 0, t][:, None].astype(np.float64)).sum(0)
            s32 = s.astype(np.float32)
            best = sorted(range(n), key=lambda j: (-s32[j], j))[:w.top_k]
            got = topk[g, 0, t]
            assert sorted(got[got >= 0].tolist()) == sorted(best)
