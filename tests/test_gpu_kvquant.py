"""GPU parity of the FP4 main-KV quantiser (csa2_quantize_kv_fp4) with the oracle: bytes must be
identical (codes and scales are integer decisions taken in binary32 on both sides)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import gpu_chain as G

pytestmark = pytest.mark.gpu


def run(bits: np.ndarray):
    import hierarchical_kv_indexer_amd as H
    rows = bits.shape[0]
    codes = G.empty((rows, 256), torch.uint8)
    scales = G.empty((rows, 32), torch.uint8)
    H.csa2_quantize_kv_fp4(G.dev(bits), rows, codes, scales)
    return G.host(codes), G.host(scales)


def latent_rows(rng, rows):
    """Latent-like rows: unit RMS (the width-512 RMSNorm output has L2 norm sqrt(512)), a few
    channels several times larger, and some rows scaled far down or up."""
    x = rng.standard_normal((rows, 512)).astype(np.float32)
    x[:, rng.integers(0, 512, 6)] *= 8.0
    x[::7] *= 1e-3
    x[::11] *= 300.0
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quantize_kv_random_rows_ragged():
    bits = latent_rows(np.random.default_rng(11), 1003)      # 1003 rows: a partial last workgroup
    c, s = run(bits)
    rc, rs = F.kv_quantize_rows(bits)
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)


@pytest.mark.parametrize("anchor", [None, 6.0, 6.0 * 1.375, 6.0 * 2.0 ** -7])
def test_quantize_kv_every_bf16_value(anchor):
    """Every finite bf16 value, either alone in its group (it sets the scale: every amax) or next
    to an anchor that sets the scale (power-of-two and inexact quotients)."""
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_value(vals)
    vals = vals[np.isfinite(v)]
    if anchor is None:
        groups = np.zeros((len(vals), 16), np.uint16)
        groups[:, 3] = vals
    else:
        per = 15
        n = (len(vals) + per - 1) // per
        pad = np.zeros(n * per, np.uint16)
        pad[:len(vals)] = vals
        a = torch.tensor([anchor], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        groups = np.empty((n, 16), np.uint16)
        groups[:, 0] = a[0]
        groups[:, 1:] = pad.reshape(n, per)
    rows = (groups.shape[0] + 31) // 32
    full = np.zeros((rows * 32, 16), np.uint16)
    full[:groups.shape[0]] = groups
    bits = full.reshape(rows, 512)
    c, s = run(bits)
    rc, rs = F.kv_quantize_rows(bits)
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)


def test_quantize_kv_2p20_rows_sampled():
    """A million rows in one launch (1 GiB of bf16 in, 288 MiB out), checked on sampled rows."""
    import hierarchical_kv_indexer_amd as H
    rows = 1 << 20
    g = torch.Generator(device=G.DEV)
    g.manual_seed(12)
    x = torch.randn((rows, 512), generator=g, device=G.DEV, dtype=torch.float32)
    x[:, 5] *= 8.0
    xb = x.to(torch.bfloat16)
    del x
    codes = G.empty((rows, 256), torch.uint8)
    scales = G.empty((rows, 32), torch.uint8)
    H.csa2_quantize_kv_fp4(xb, rows, codes, scales)
    idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(13).integers(0, rows, 4096)]))
    ti = torch.from_numpy(idx).to(G.DEV)
    bits = G.host(xb[ti].view(torch.int16))
    rc, rs = F.kv_quantize_rows(bits)
    assert np.array_equal(G.host(scales[ti]), rs)
    assert np.array_equal(G.host(codes[ti]), rc)


def test_quantize_kv_append_at_offset_and_empty():
    import hierarchical_kv_indexer_amd as H
    bits = latent_rows(np.random.default_rng(14), 9)
    cache_c = torch.full((32, 256), 0xAB, dtype=torch.uint8, device=G.DEV)
    cache_s = torch.full((32, 32), 0xCD, dtype=torch.uint8, device=G.DEV)
    H.csa2_quantize_kv_fp4(G.dev(bits), 9, cache_c[7:], cache_s[7:])
    H.csa2_quantize_kv_fp4(G.dev(bits), 0, cache_c[20:], cache_s[20:])      # no rows: no writes
    c, s = G.host(cache_c), G.host(cache_s)
    rc, rs = F.kv_quantize_rows(bits)
    assert np.array_equal(c[7:16], rc) and np.array_equal(s[7:16], rs)
    assert (c[:7] == 0xAB).all() and (c[16:] == 0xAB).all()
    assert (s[:7] == 0xCD).all() and (s[16:] == 0xCD).all()
