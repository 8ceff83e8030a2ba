"""Seeded synthetic inputs for the CSA2 decode / prefill workloads.

This module only draws random numbers and stores them in the dtypes the
library's boundary takes.  It holds none of the method's arithmetic: the
conversions to bf16 and to the OCP E4M3 byte format are done by PyTorch's own
dtype casts (``torch.bfloat16`` and ``torch.float8_e4m3fn``), and the FP4
(E2M1) codes of the main KV are drawn directly from a fixed categorical
distribution over the 16 codes.  Both the CPU oracle and the GPU path read
the bytes produced here.

Workload shapes follow the CSA2 description (DeepSeek-V4.1-Flash pages): a
Full indexer with 32 query heads of dim 128, a candidate pool of 2048 blocks x
8 positions, Top-512, Reindex layers with their own indexer query, Reuse layers
that inherit indices, and sparse attention over an FP4 main KV (one E4M3 scale
per 16 channels) merged with an FP8 sliding window.

Recipe (one ``numpy.random.SeedSequence(seed)`` per workload, one child
generator per tensor, children spawned in the order of ``STREAMS``):

  indexer K            N(0,1) float32 -> E4M3 (torch cast, values clamped to +-448 first);
                       FP4 variant (``idx_k_fp4``): the same draws -> E2M1 codes with one
                       E4M3 scale per 16 channels: amax/6 times U(1, 1.5) (stream
                       ``fp4_scale``), cast to E4M3 by torch (any mantissa), negative for
                       half the groups (sign bit drawn from the same stream); codes the
                       nearest E2M1 magnitude of |x / scale| by table lookup, sign that of
                       x / scale (this generator's own encoder; any FP4 bytes are valid
                       input), 64 code bytes + 8 scale bytes per position
  indexer Q (Full/RI)  N(0,1) float32 -> bf16 (torch cast, round to nearest even)
  head weights w       U(0,1) float32
  main-KV E2M1 codes   categorical over the 16 codes (``E2M1_MAG_WEIGHTS`` / 256 per
                       magnitude, sign uniform), two codes per byte, even channel in
                       the low nibble
  main-KV scales       U(0.5,2) float32 -> E4M3 (torch cast)
  attention q          N(0,1) float32 -> bf16
  SWA rows             N(0,1) float32 -> E4M3
  planted cluster      (1M decode only) 512 contiguous, 8-aligned positions whose keys
                       are shifted, before the E4M3 cast, by the minimum-norm vector
                       delta with  q8_h . delta = 4 * ||q8_h||  for every Full-layer head
  user pools           (pool-only workload) 16384 distinct positions per query drawn
                       uniformly without replacement from the context, sorted
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

IDX_HEADS = 32
IDX_DIM = 128
KV_DIM = 512
KV_CODE_BYTES = KV_DIM // 2
KV_SCALE_BYTES = KV_DIM // 16

STREAMS = ("idx_k", "idx_q", "head_w", "ri_q", "ri_w", "kv_codes", "kv_scales",
           "q", "swa", "planted", "user_pool", "fp4_scale")

# Relative frequencies (out of 256) of the E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
# Codes are drawn independently of the U(0.5, 2) scales (E[s^2] = 1.75); the mean
# squared code, 178.25/256 = 0.70, puts the dequantised channel RMS near 1.1, so a
# row's L2 norm is about 25, near the sqrt(512) ~ 22.6 of a unit-gain RMSNorm output.
# Every magnitude, 6 included, keeps a non-zero frequency.
E2M1_MAG_WEIGHTS = (92, 100, 43, 13, 5, 1, 1, 1)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                    # sequences
    T: int                    # query tokens per sequence
    N: int                    # compressed positions (indexer-K / main-KV rows) per sequence
    H: int                    # attention query heads
    layer_set: tuple          # attention layer -> index-set id (set 0 = first indexer output)
    n_reindex: int            # Reindex layers
    has_full: bool = True     # a Full layer runs (False: caller-provided pools)
    block: int = 8
    pool_blocks: int = 2048   # 0: no pool (Top-K over every visible position)
    top_k: int = 512
    swa_window: int = 128
    planted: bool = False
    user_pool: int = 0        # >0: caller-provided pools of this many positions
    prefill_tokens: int = 0   # >0: causal prefill over a context of this many tokens
    m: int = 2                # tokens per compressed entry (prefill visibility)
    idx_k_fp4: bool = False   # indexer K stored as FP4 (E2M1 codes + E4M3 per-16 scales)

    @property
    def L(self) -> int:
        return len(self.layer_set)

    @property
    def n_sets(self) -> int:
        return max(self.layer_set) + 1

    @property
    def pool_cap(self) -> int:
        if self.user_pool:
            return self.user_pool
        return self.pool_blocks * self.block

    @property
    def swa_rows(self) -> int:
        return self.T + self.swa_window - 1 if self.prefill_tokens else self.swa_window

    def n_visible(self) -> np.ndarray:
        """[B][T] visible compressed positions per query."""
        if not self.prefill_tokens:
            return np.full((self.B, self.T), self.N, np.int32)
        p = self.prefill_tokens - self.T + np.arange(self.T, dtype=np.int64)
        nv = np.minimum((p + 1) // self.m, self.N).astype(np.int32)
        return np.broadcast_to(nv, (self.B, self.T)).copy()

    def swa_end(self) -> np.ndarray:
        """[B][T] exclusive end row of each query's sliding window in its layer's SWA rows."""
        if not self.prefill_tokens:
            return np.full((self.B, self.T), self.swa_window, np.int32)
        e = np.arange(self.T, dtype=np.int32) + self.swa_window
        return np.broadcast_to(e, (self.B, self.T)).copy()


def _decode_sets(groups):
    out = []
    for s, n in groups:
        out += [s] * n
    return tuple(out)


WORKLOADS: Dict[str, Workload] = {
    # tiny decode: Full + Reindex + Reuse(<- Reindex)
    "tiny_4k": Workload("tiny_4k", 1001, B=1, T=1, N=4096, H=16, layer_set=(0, 1, 1),
                        n_reindex=1, pool_blocks=64, top_k=64),
    # batch-8 decode over 128K contexts: [F, RU] + 4 x [RI, RU]
    "decode_b8_128k": Workload("decode_b8_128k", 1002, B=8, T=1, N=131072, H=64,
                               layer_set=_decode_sets([(0, 2), (1, 2), (2, 2), (3, 2), (4, 2)]),
                               n_reindex=4),
    # batch-1 decode over a 1M context: [F, RU x3] + 4 x [RI, RU x3], planted cluster
    "decode_1m": Workload("decode_1m", 1003, B=1, T=1, N=1 << 20, H=16,
                          layer_set=_decode_sets([(0, 4), (1, 4), (2, 4), (3, 4), (4, 4)]),
                          n_reindex=4, planted=True),
    # the same decode with the FP4 indexer variant (keys 72 B per position instead of 128 B; the
    # query rounded to FP4 by the library)
    "decode_1m_fp4k": Workload("decode_1m_fp4k", 1006, B=1, T=1, N=1 << 20, H=16,
                               layer_set=_decode_sets([(0, 4), (1, 4), (2, 4), (3, 4), (4, 4)]),
                               n_reindex=4, planted=True, idx_k_fp4=True),
    # 64 queries of one 256K context with caller pools: 1 Reindex layer + 1 attention layer
    "reindex_pool_256k": Workload("reindex_pool_256k", 1004, B=1, T=64, N=262144, H=64,
                                  layer_set=(0,), n_reindex=1, has_full=False,
                                  pool_blocks=0, user_pool=16384),
    # causal prefill of 4096 tokens over a 64K-token context compressed m=2: Full + 5 Reuse
    "prefill_4k_64k": Workload("prefill_4k_64k", 1005, B=1, T=4096, N=32768, H=64,
                               layer_set=(0,) * 6, n_reindex=0, pool_blocks=0,
                               prefill_tokens=65536, m=2),
}


def _torch():
    import torch  # local import: only the casts below use it
    return torch


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), via torch's round-to-nearest-even cast."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3 bytes via torch's float8_e4m3fn cast (inputs clamped to +-448)."""
    torch = _torch()
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def e4m3_bytes_as_float(codes: np.ndarray) -> np.ndarray:
    """E4M3 bytes -> float32 via torch's float8_e4m3fn cast (used for the planted shift)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def bf16_bits_as_float(bits: np.ndarray) -> np.ndarray:
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).numpy()


def _e2m1_lut() -> np.ndarray:
    lut = np.zeros(256, np.uint8)
    pos = 0
    for mag, n in enumerate(E2M1_MAG_WEIGHTS):
        lut[pos:pos + n] = mag
        pos += n
    assert pos == 256
    return lut


def draw_kv_codes(rng: np.random.Generator, rows: int) -> np.ndarray:
    """[rows][256] packed E2M1 code bytes (low nibble = even channel)."""
    lut = _e2m1_lut()
    out = np.empty((rows, KV_CODE_BYTES), np.uint8)
    chunk = 16384
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        n = (r1 - r0) * KV_DIM
        raw = np.frombuffer(rng.bytes(2 * n), np.uint8).reshape(n, 2)
        nib = lut[raw[:, 0]] | ((raw[:, 1] & 1) << 3).astype(np.uint8)
        nib = nib.reshape(r1 - r0, KV_CODE_BYTES, 2)
        out[r0:r1] = nib[:, :, 0] | (nib[:, :, 1] << 4)
    return out


E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def to_fp4_keys(x: np.ndarray, rng: np.random.Generator):
    """float32 [n][d] -> (codes [n][d/2] u8, scales [n][d/16] u8): per 16 channels an E4M3 scale
    of amax/6 times U(1, 1.5) (within [2^-9, 448]; torch's E4M3 cast, so any mantissa), negated
    for a random half of the groups; each channel the nearest E2M1 magnitude of |x / scale| (a
    table lookup on the midpoints), with the sign of x / scale."""
    n, dch = x.shape
    g = x.reshape(n, dch // 16, 16).astype(np.float32)
    amax = np.abs(g).max(-1)
    jitter = rng.uniform(1.0, 1.5, size=amax.shape).astype(np.float32)
    neg = rng.random(size=amax.shape) < 0.5
    mag = np.clip(amax / 6.0 * jitter, 2.0 ** -9, 448.0).astype(np.float32)
    sbytes = to_e4m3_bytes(mag) | (neg.astype(np.uint8) << 7)
    scale = e4m3_bytes_as_float(sbytes)                     # the stored (signed) scale
    q = np.abs(g) / np.abs(scale)[..., None]
    mid = (E2M1_MAGS[1:] + E2M1_MAGS[:-1]) / 2
    code_mag = np.searchsorted(mid, q, side="left").astype(np.uint8)
    sign = np.signbit(g) ^ np.signbit(scale)[..., None]
    c = (code_mag | (sign.astype(np.uint8) << 3)).reshape(n, dch)
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return codes, sbytes


def draw_normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(w: Workload, with_attention: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one workload as numpy arrays in the boundary's layouts.

    Keys: idx_k [B][N][128] u8 (or, FP4 indexer K, idx_k_codes [B][N][64] u8 and
    idx_k_scales [B][N][8] u8), idx_q [B][T][32][128] u16 (bf16 bits), head_w [B][T][32] f32,
    n_visible [B][T] i32, ri_q [Lri][B][T][32][128] u16, ri_w [Lri][B][T][32] f32,
    kv_codes [B][N][256] u8, kv_scales [B][N][32] u8, q [L][B][T][H][512] u16,
    swa [L][B][swa_rows][512] u8, swa_end [B][T] i32, and for caller pools
    pool_pos [B][T][pool_cap] i32 / pool_len [B][T] i32; planted_pos [512] when planted.
    """
    ss = np.random.SeedSequence(w.seed)
    gens = dict(zip(STREAMS, (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(STREAMS)))))
    B, T, N = w.B, w.T, w.N
    d: Dict[str, np.ndarray] = {}

    d["idx_q"] = to_bf16_bits(draw_normal_f32(gens["idx_q"], (B, T, IDX_HEADS, IDX_DIM)))
    d["head_w"] = gens["head_w"].random(size=(B, T, IDX_HEADS), dtype=np.float32)
    d["ri_q"] = to_bf16_bits(draw_normal_f32(gens["ri_q"], (w.n_reindex, B, T, IDX_HEADS, IDX_DIM)))
    d["ri_w"] = gens["ri_w"].random(size=(w.n_reindex, B, T, IDX_HEADS), dtype=np.float32)

    if w.idx_k_fp4:
        idx_k = np.empty((B, N, IDX_DIM // 2), np.uint8)
        idx_k_scales = np.empty((B, N, IDX_DIM // 16), np.uint8)
    else:
        idx_k = np.empty((B, N, IDX_DIM), np.uint8)
    planted_pos = None
    if w.planted:
        g = gens["planted"]
        off = int(g.integers(0, (N - 512) // 8 + 1)) * 8
        planted_pos = np.arange(off, off + 512, dtype=np.int32)
        q8 = e4m3_bytes_as_float(to_e4m3_bytes(bf16_bits_as_float(d["idx_q"][0, 0])))  # [32][128]
        target = 4.0 * np.linalg.norm(q8.astype(np.float64), axis=1)
        delta = np.linalg.lstsq(q8.astype(np.float64), target, rcond=None)[0].astype(np.float32)
    chunk = 1 << 17
    for b in range(B):
        for r0 in range(0, N, chunk):
            r1 = min(N, r0 + chunk)
            x = draw_normal_f32(gens["idx_k"], (r1 - r0, IDX_DIM))
            if planted_pos is not None and b == 0:
                lo, hi = max(r0, planted_pos[0]), min(r1, planted_pos[-1] + 1)
                if lo < hi:
                    x[lo - r0:hi - r0] += delta
            if w.idx_k_fp4:
                idx_k[b, r0:r1], idx_k_scales[b, r0:r1] = to_fp4_keys(x, gens["fp4_scale"])
            else:
                idx_k[b, r0:r1] = to_e4m3_bytes(x)
    if w.idx_k_fp4:
        d["idx_k_codes"], d["idx_k_scales"] = idx_k, idx_k_scales
    else:
        d["idx_k"] = idx_k
    if planted_pos is not None:
        d["planted_pos"] = planted_pos
    d["n_visible"] = w.n_visible()

    if w.user_pool:
        g = gens["user_pool"]
        pp = np.empty((B, T, w.user_pool), np.int32)
        for b in range(B):
            for t in range(T):
                pp[b, t] = np.sort(g.choice(N, size=w.user_pool, replace=False)).astype(np.int32)
        d["pool_pos"] = pp
        d["pool_len"] = np.full((B, T), w.user_pool, np.int32)

    if with_attention:
        kv_codes = np.empty((B, N, KV_CODE_BYTES), np.uint8)
        for b in range(B):
            kv_codes[b] = draw_kv_codes(gens["kv_codes"], N)
        d["kv_codes"] = kv_codes
        d["kv_scales"] = to_e4m3_bytes(
            gens["kv_scales"].uniform(0.5, 2.0, size=(B, N, KV_SCALE_BYTES)).astype(np.float32))
        q = np.empty((w.L, B, T, w.H, KV_DIM), np.uint16)
        for l in range(w.L):
            q[l] = to_bf16_bits(draw_normal_f32(gens["q"], (B, T, w.H, KV_DIM)))
        d["q"] = q
        swa = np.empty((w.L, B, w.swa_rows, KV_DIM), np.uint8)
        for l in range(w.L):
            swa[l] = to_e4m3_bytes(draw_normal_f32(gens["swa"], (B, w.swa_rows, KV_DIM)))
        d["swa"] = swa
        d["swa_end"] = w.swa_end()
    return d


# ---------------------------------------------------------------- encoder prefill

ENC_STREAMS = ("enc_k", "enc_latent", "enc_idx_q", "enc_w", "enc_q", "enc_swa",
               "enc_cache_k", "enc_cache_codes", "enc_cache_scales")


@dataclasses.dataclass(frozen=True)
class EncoderPrefill:
    """A prompt run through the encoder's CSA2 groups in chunks of T tokens (G groups of one
    Full layer and layers-1 Reuse layers, m tokens per compressed entry).  The measured chunk
    is the last one: tokens prompt - T .. prompt - 1."""
    name: str
    seed: int
    B: int
    G: int
    layers: int
    H: int
    prompt: int
    T: int
    m: int = 2
    top_k: int = 512
    swa_window: int = 128

    @property
    def k_rows(self) -> int:
        return self.prompt // self.m

    @property
    def p0(self) -> int:
        return self.prompt - self.T

    def hist(self, p0: int) -> int:
        return min(p0, self.swa_window - 1) if self.swa_window > 0 else 0


ENCODER_WORKLOADS: Dict[str, EncoderPrefill] = {
    # the last 256-token chunk of a 1M-token prompt: 3 groups x (Full + 5 Reuse), 512K entries
    "encoder_1m": EncoderPrefill("encoder_1m", 1007, B=1, G=3, layers=6, H=64, prompt=1 << 20, T=256),
}


def _enc_gens(seed: int):
    ss = np.random.SeedSequence(seed)
    return dict(zip(ENC_STREAMS, (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(ENC_STREAMS)))))


def make_encoder_prompt(w: EncoderPrefill) -> Dict[str, np.ndarray]:
    """Every token of the prompt, for chunk-by-chunk runs from an empty cache:
    new_idx_k [G][B][n][128] and new_latent [G][B][n][512] bf16 (n = prompt // m entries, N(0,1)),
    idx_q [G][B][P][32][128] bf16, head_w [G][B][P][32] U(0,1), q [G][layers][B][P][H][512] bf16,
    swa [G][layers][B][P][512] E4M3 (row = token)."""
    g = _enc_gens(w.seed)
    G, B, P, L, H = w.G, w.B, w.prompt, w.layers, w.H
    n = P // w.m
    d: Dict[str, np.ndarray] = {}
    d["new_idx_k"] = to_bf16_bits(draw_normal_f32(g["enc_k"], (G, B, n, IDX_DIM)))
    d["new_latent"] = to_bf16_bits(draw_normal_f32(g["enc_latent"], (G, B, n, KV_DIM)))
    d["idx_q"] = to_bf16_bits(draw_normal_f32(g["enc_idx_q"], (G, B, P, IDX_HEADS, IDX_DIM)))
    d["head_w"] = g["enc_w"].random(size=(G, B, P, IDX_HEADS), dtype=np.float32)
    d["q"] = to_bf16_bits(draw_normal_f32(g["enc_q"], (G, L, B, P, H, KV_DIM)))
    d["swa"] = to_e4m3_bytes(draw_normal_f32(g["enc_swa"], (G, L, B, P, KV_DIM)))
    return d


def encoder_chunk_args(w: EncoderPrefill, prompt: Dict[str, np.ndarray], p0: int, T: int) -> Dict[str, np.ndarray]:
    """The arguments of the chunk p0 .. p0+T-1 sliced from make_encoder_prompt's arrays."""
    n0, n1 = p0 // w.m, (p0 + T) // w.m
    h = w.hist(p0)
    return {"new_idx_k": prompt["new_idx_k"][:, :, n0:n1], "new_latent": prompt["new_latent"][:, :, n0:n1],
            "idx_q": prompt["idx_q"][:, :, p0:p0 + T], "head_w": prompt["head_w"][:, :, p0:p0 + T],
            "q": prompt["q"][:, :, :, p0:p0 + T], "swa": prompt["swa"][:, :, :, p0 - h:p0 + T]}


def make_encoder_chunk(w: EncoderPrefill) -> Dict[str, np.ndarray]:
    """The last chunk of the prompt with the caches already holding every earlier entry, drawn
    directly in their storage formats (indexer keys N(0,1) -> E4M3; main KV E2M1 codes and
    U(0.5,2) -> E4M3 scales as in make_inputs): idx_k [G][B][k_rows][128], kv_codes
    [G][B][k_rows][256], kv_scales [G][B][k_rows][32] (rows at or beyond floor(p0/m) zero), and
    the chunk's arguments as encoder_chunk_args gives them."""
    g = _enc_gens(w.seed)
    G, B, L, H, T, p0 = w.G, w.B, w.layers, w.H, w.T, w.p0
    n0, n1 = p0 // w.m, (p0 + T) // w.m
    h = w.hist(p0)
    d: Dict[str, np.ndarray] = {}
    d["idx_k"] = np.zeros((G, B, w.k_rows, IDX_DIM), np.uint8)
    d["kv_codes"] = np.zeros((G, B, w.k_rows, KV_CODE_BYTES), np.uint8)
    d["kv_scales"] = np.zeros((G, B, w.k_rows, KV_SCALE_BYTES), np.uint8)
    chunk = 1 << 17
    for gi in range(G):
        for b in range(B):
            for r0 in range(0, n0, chunk):
                r1 = min(n0, r0 + chunk)
                d["idx_k"][gi, b, r0:r1] = to_e4m3_bytes(draw_normal_f32(g["enc_cache_k"], (r1 - r0, IDX_DIM)))
                d["kv_codes"][gi, b, r0:r1] = draw_kv_codes(g["enc_cache_codes"], r1 - r0)
                d["kv_scales"][gi, b, r0:r1] = to_e4m3_bytes(
                    g["enc_cache_scales"].uniform(0.5, 2.0, size=(r1 - r0, KV_SCALE_BYTES)).astype(np.float32))
    d["new_idx_k"] = to_bf16_bits(draw_normal_f32(g["enc_k"], (G, B, n1 - n0, IDX_DIM)))
    d["new_latent"] = to_bf16_bits(draw_normal_f32(g["enc_latent"], (G, B, n1 - n0, KV_DIM)))
    d["idx_q"] = to_bf16_bits(draw_normal_f32(g["enc_idx_q"], (G, B, T, IDX_HEADS, IDX_DIM)))
    d["head_w"] = g["enc_w"].random(size=(G, B, T, IDX_HEADS), dtype=np.float32)
    q = np.empty((G, L, B, T, H, KV_DIM), np.uint16)
    for gi in range(G):
        for l in range(L):
            q[gi, l] = to_bf16_bits(draw_normal_f32(g["enc_q"], (B, T, H, KV_DIM)))
    d["q"] = q
    d["swa"] = to_e4m3_bytes(draw_normal_f32(g["enc_swa"], (G, L, B, h + T, KV_DIM)))
    return d


# ---------------------------------------------------------------- recall study of the hierarchical indexer

RECALL_FAMILIES = ("full_isolated", "reindex_isolated", "shared_isolated", "full_clusters")


def make_recall_context(N: int, seed: int, n_needles: int = 32, n_clusters: int = 8,
                        sigma: float = 4.0, cluster_sigma: float = 2.0,
                        rho: Optional[float] = None) -> Dict[str, object]:
    """One decode query over N positions with planted needles for the hierarchical indexer's recall
    study (alphalab.site sec."2. CSA2": the first Full layer's pool decides what the Reindex layers
    can pick).  Keys are N(0,1) rows with, before the E4M3 cast, a shift delta added at the needle
    positions: the minimum-norm delta with q8_h . delta = s * ||q8_h|| for every head h of the
    target queries (the planted-cluster recipe of the 1M decode):
      full_isolated     n_needles single positions, target the Full query, s = sigma;
      reindex_isolated  n_needles single positions, target the Reindex query only, s = sigma;
      shared_isolated   n_needles single positions, target both queries, s = sigma;
      full_clusters     n_clusters aligned blocks of 8 positions, target the Full query,
                        s = cluster_sigma (weaker alone, dense as a block).
    The Reindex query is an independent N(0,1) draw z, or with `rho` the mix rho * q + sqrt(1 -
    rho^2) * z of the Full query q and that draw (element-wise correlation rho).
    Returns idx_k [1][N][128], idx_q / head_w (Full), ri_q [1][1][1][32][128] / ri_w (one Reindex
    layer), n_visible [1][1], and families {name: sorted positions}."""
    ss = np.random.SeedSequence(seed)
    g = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(5)]
    d: Dict[str, object] = {}
    q_full = draw_normal_f32(g[0], (1, 1, IDX_HEADS, IDX_DIM))
    d["idx_q"] = to_bf16_bits(q_full)
    d["head_w"] = g[1].random(size=(1, 1, IDX_HEADS), dtype=np.float32)
    z = draw_normal_f32(g[0], (1, 1, 1, IDX_HEADS, IDX_DIM))
    if rho is not None:
        z = (np.float32(rho) * q_full[None] + np.float32(np.sqrt(1.0 - rho * rho)) * z).astype(np.float32)
    d["ri_q"] = to_bf16_bits(z)
    d["ri_w"] = g[1].random(size=(1, 1, 1, IDX_HEADS), dtype=np.float32)
    qf = e4m3_bytes_as_float(to_e4m3_bytes(bf16_bits_as_float(d["idx_q"][0, 0]))).astype(np.float64)
    qr = e4m3_bytes_as_float(to_e4m3_bytes(bf16_bits_as_float(d["ri_q"][0, 0, 0]))).astype(np.float64)

    def shift(a, s):
        return np.linalg.lstsq(a, s * np.linalg.norm(a, axis=1), rcond=None)[0].astype(np.float32)

    deltas = {"full_isolated": shift(qf, sigma), "reindex_isolated": shift(qr, sigma),
              "shared_isolated": shift(np.concatenate([qf, qr]), sigma), "full_clusters": shift(qf, cluster_sigma)}
    nb = N // 8
    blocks = g[2].choice(nb, size=3 * n_needles + n_clusters, replace=False)
    fam: Dict[str, np.ndarray] = {}
    off = g[3].integers(0, 8, size=3 * n_needles)
    for i, name in enumerate(RECALL_FAMILIES[:3]):
        b = blocks[i * n_needles:(i + 1) * n_needles]
        fam[name] = np.sort(8 * b + off[i * n_needles:(i + 1) * n_needles]).astype(np.int32)
    cb = blocks[3 * n_needles:]
    fam["full_clusters"] = np.sort((8 * cb[:, None] + np.arange(8)[None, :]).reshape(-1)).astype(np.int32)
    idx_k = np.empty((1, N, IDX_DIM), np.uint8)
    chunk = 1 << 17
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        x = draw_normal_f32(g[4], (r1 - r0, IDX_DIM))
        for name, pos in fam.items():
            sel = pos[(pos >= r0) & (pos < r1)] - r0
            x[sel] += deltas[name]
        idx_k[0, r0:r1] = to_e4m3_bytes(x)
    d["idx_k"] = idx_k
    d["n_visible"] = np.full((1, 1), N, np.int32)
    d["families"] = fam
    return d


def small_variant(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (for parity cases at reduced size)."""
    return dataclasses.replace(w, **changes)
