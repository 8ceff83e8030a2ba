"""Pins of the oracle's sparse attention: it reduces to textbook scaled dot-product
attention (PyTorch's scaled_dot_product_attention, float64) with keys equal to the
values, plus special cases with closed forms and the row-set composition
(selected main-KV rows followed by the window's SWA rows)."""
import numpy as np
import torch

import workloads
from oracle import csa2 as O
from oracle import formats as F

SCALE = 1.0 / np.sqrt(512)


def rand_q(rng, H):
    return workloads.to_bf16_bits(rng.standard_normal((H, 512), dtype=np.float32))


def test_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((37, 512)) * 1.3
    q = rand_q(rng, 4)
    o, lse = O.attention(q, rows, SCALE)
    qt = torch.from_numpy(F.bf16_value(q))[None, :, None, :]          # [1][H][1][512]
    kt = torch.from_numpy(rows)[None, None].expand(1, 4, 37, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=SCALE)[0, :, 0]
    assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    z = SCALE * (F.bf16_value(q) @ rows.T)
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(z), dim=1).numpy(), rtol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((9, 512))
    zero_q = np.zeros((2, 512), np.uint16)
    o, lse = O.attention(zero_q, rows, SCALE)
    assert np.allclose(o, rows.mean(axis=0)[None], atol=1e-14)      # q = 0: mean of the rows
    assert np.allclose(lse, np.log(9.0))
    o1, _ = O.attention(rand_q(rng, 3), rows[4:5], SCALE)
    assert np.allclose(o1, rows[4][None], atol=0)                   # one row: that row
    o0, lse0 = O.attention(rand_q(rng, 3), rows[:0], SCALE)
    assert np.all(o0 == 0) and np.all(np.isneginf(lse0))            # no rows: zero output


def test_lse_merge_equals_joint_softmax():
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((50, 512))
    q = rand_q(rng, 5)
    o, lse = O.attention(q, rows, SCALE)
    oa, la = O.attention(q, rows[:20], SCALE)
    ob, lb = O.attention(q, rows[20:], SCALE)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (oa * wa[:, None] + ob * wb[:, None]) / (wa + wb)[:, None]
    assert np.allclose(merged, o, atol=1e-12)
    assert np.allclose(m + np.log(wa + wb), lse, atol=1e-12)


def test_row_set_composition():
    rng = np.random.default_rng(3)
    N = 40
    codes = rng.integers(0, 256, size=(N, 256), dtype=np.uint8)
    scales = workloads.to_e4m3_bytes(rng.uniform(0.5, 2, size=(N, 32)).astype(np.float32))
    swa = workloads.to_e4m3_bytes(rng.standard_normal((10, 512), dtype=np.float32))
    idx = np.array([3, 17, 39, -1, -1], np.int32)
    rows = O.attention_rows(codes, scales, idx, swa, swa_end=10, window=4)
    assert rows.shape == (3 + 4, 512)
    assert np.array_equal(rows[1], F.kv_row_values(codes[17], scales[17]))
    assert np.array_equal(rows[3:], F.e4m3_value(swa[6:10]))
    # window clipped at row 0
    assert O.attention_rows(codes, scales, idx, swa, swa_end=2, window=4).shape == (3 + 2, 512)
    # no selected entries: only the window; no window: only main rows
    assert O.attention_rows(codes, scales, np.full(5, -1), swa, 10, 4).shape == (4, 512)
    assert O.attention_rows(codes, scales, idx, swa, 0, 4).shape == (3, 512)


def test_reuse_layers_share_indices_and_main_rows():
    w = workloads.Workload("t", 9, B=1, T=1, N=1500, H=4, layer_set=(0, 0, 1, 1),
                           n_reindex=1, pool_blocks=16, top_k=32)
    inp = workloads.make_inputs(w)
    out = O.query_chain(inp, w, 0, 0)
    # layers 0/1 read set 0 (Full), layers 2/3 read set 1 (Reindex); a Reuse layer with its
    # own query but its leader's indices: same main rows, different outputs
    assert out["sets"].shape == (2, 32)
    r0 = O.attention_rows(inp["kv_codes"][0], inp["kv_scales"][0], out["sets"][0], inp["swa"][1, 0], 128, 128)
    o1, _ = O.attention(inp["q"][1, 0, 0], r0, SCALE)
    assert np.array_equal(o1, out["attn_out"][1])
    assert not np.allclose(out["attn_out"][0], out["attn_out"][1])


def test_synthetic_kv_latent_norm_near_page_figure():
    # the synthetic FP4 main KV is drawn so that a row's L2 norm is near sqrt(512) ~ 22.6
    rng = np.random.default_rng(4)
    codes = workloads.draw_kv_codes(rng, 256)
    scales = workloads.to_e4m3_bytes(rng.uniform(0.5, 2, size=(256, 32)).astype(np.float32))
    norms = np.linalg.norm(F.kv_row_values(codes, scales), axis=1)
    assert 20.0 < norms.mean() < 28.0
