"""Python binding of libcsa2.so, the CSA2 decode hot path for MI355X (gfx950).

Argument marshalling only: every function below has the name and argument order of the C
entry point it calls (see include/csa2.h), takes torch tensors (or None) where the C call
takes pointers, and raises Csa2Error when the call returns a non-OK status.  Device tensors
must be contiguous; ``stream`` defaults to torch's current stream on the tensors' device.
The library has no CPU fallback: without the built shared object every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

STATUS = {0: "CSA2_OK", 1: "CSA2_ERR_INVALID_ARG", 2: "CSA2_ERR_UNSUPPORTED",
          3: "CSA2_ERR_WORKSPACE", 4: "CSA2_ERR_HIP"}

# (name, restype, argtypes) of every exported entry point
_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
EXPORTS = (
    ("csa2_last_error", ctypes.c_char_p, ()),
    ("csa2_quantize_query", _I, (_P, _P, _I64, _P)),
    ("csa2_quantize_kv_fp4", _I, (_P, _I64, _P, _P, _P)),
    ("csa2_index_scores", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _P, _P)),
    ("csa2_index_full_workspace", _SZ, (_I, _I, _I, _I, _I, _I)),
    ("csa2_index_stages_workspace", _SZ, (_I, _I, _I, _I, _I, _I)),
    ("csa2_index_scan", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _SZ, _P)),
    ("csa2_index_scan_blocks", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _SZ, _P)),
    ("csa2_index_pool", _I, (_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P)),
    ("csa2_index_topk", _I, (_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P)),
    ("csa2_index_select", _I, (_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P)),
    ("csa2_index_full", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P)),
    ("csa2_index_chain_workspace", _SZ, (_I, _I, _I, _I, _I, _I, _I)),
    ("csa2_index_chain", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                              _P, _SZ, _P)),
    ("csa2_index_select_reindex", _I, (_P, _P, _I64, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                                       _P, _SZ, _P)),
    ("csa2_noalloc_scratch_bytes", _SZ, ()),
    ("csa2_index_chain_noalloc", _I, (_P, _P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P,
                                      _P, _P, _P)),
    ("csa2_reindex_workspace", _SZ, (_I, _I, _I, _I, _I)),
    ("csa2_reindex", _I, (_P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P)),
    ("csa2_sparse_attn_workspace", _SZ, (_I, _I, _I, _I, _I, _I)),
    ("csa2_sparse_attn", _I, (_P, _P, _I64, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F,
                              _P, _P, _P, _SZ, _P)),
    ("csa2_encoder_chunk_workspace", _SZ, (_I, _I, _I64, _I, _I, _I, _I)),
    ("csa2_encoder_chunk", _I, (_I, _I, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _I, _I, _I, _I64, _I, _I,
                                _I, _I, _F, _P, _P, _P, _SZ, _P)),
)

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hierarchical_kv_indexer_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, res, args in EXPORTS:
            f = getattr(l, name)
            f.restype = res
            f.argtypes = list(args)
        _lib = l
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_contiguous(), "tensors passed to libcsa2 must be contiguous"
    return t.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int) -> None:
    if status != 0:
        raise Csa2Error(status, lib().csa2_last_error().decode())


def csa2_last_error() -> str:
    return lib().csa2_last_error().decode()


def csa2_quantize_query(in_bf16, out_e4m3, n: int, stream=None) -> None:
    _check(lib().csa2_quantize_query(_ptr(in_bf16), _ptr(out_e4m3), n, _stream(stream, in_bf16)))


def csa2_quantize_kv_fp4(latent_bf16, rows: int, kv_codes, kv_scales, stream=None) -> None:
    _check(lib().csa2_quantize_kv_fp4(_ptr(latent_bf16), rows, _ptr(kv_codes), _ptr(kv_scales),
                                      _stream(stream, latent_bf16)))


def csa2_index_scores(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int,
                      n_max: int, scores, stream=None) -> None:
    _check(lib().csa2_index_scores(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w),
                                   _ptr(n_visible), B, T, n_max, _ptr(scores), _stream(stream, idx_k)))


def csa2_index_full_workspace(B: int, T: int, n_max: int, block_size: int, pool_blocks: int,
                              top_k: int) -> int:
    return lib().csa2_index_full_workspace(B, T, n_max, block_size, pool_blocks, top_k)


def csa2_index_stages_workspace(B: int, T: int, n_max: int, block_size: int, pool_blocks: int,
                                top_k: int) -> int:
    return lib().csa2_index_stages_workspace(B, T, n_max, block_size, pool_blocks, top_k)


def csa2_index_full(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int,
                    n_max: int, block_size: int, pool_blocks: int, top_k: int, pool_pos, pool_len,
                    topk_idx, topk_score, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_full(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w),
                                 _ptr(n_visible), B, T, n_max, block_size, pool_blocks, top_k,
                                 _ptr(pool_pos), _ptr(pool_len), _ptr(topk_idx), _ptr(topk_score),
                                 _ptr(workspace), ws_bytes, _stream(stream, idx_k)))


def csa2_index_scan(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int,
                    n_max: int, block_size: int, pool_blocks: int, top_k: int, workspace,
                    ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_scan(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w),
                                 _ptr(n_visible), B, T, n_max, block_size, pool_blocks, top_k,
                                 _ptr(workspace), ws_bytes, _stream(stream, idx_k)))



def csa2_index_scan_blocks(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int,
                           n_max: int, block_size: int, pool_blocks: int, top_k: int, block_score: int,
                           workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_scan_blocks(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q),
                                        _ptr(head_w), _ptr(n_visible), B, T, n_max, block_size, pool_blocks,
                                        top_k, block_score, _ptr(workspace), ws_bytes, _stream(stream, idx_k)))

def csa2_index_pool(n_visible, B: int, T: int, n_max: int, block_size: int, pool_blocks: int,
                    top_k: int, pool_pos, pool_len, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_pool(_ptr(n_visible), B, T, n_max, block_size, pool_blocks, top_k,
                                 _ptr(pool_pos), _ptr(pool_len), _ptr(workspace), ws_bytes,
                                 _stream(stream, n_visible)))


def csa2_index_topk(B: int, T: int, n_max: int, block_size: int, pool_blocks: int, top_k: int,
                    pool_pos, pool_len, topk_idx, topk_score, workspace, ws_bytes: int,
                    stream=None) -> None:
    _check(lib().csa2_index_topk(B, T, n_max, block_size, pool_blocks, top_k, _ptr(pool_pos),
                                 _ptr(pool_len), _ptr(topk_idx), _ptr(topk_score), _ptr(workspace),
                                 ws_bytes, _stream(stream, topk_idx)))


def csa2_index_select(n_visible, B: int, T: int, n_max: int, block_size: int, pool_blocks: int,
                      top_k: int, pool_pos, pool_len, topk_idx, topk_score, workspace,
                      ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_select(_ptr(n_visible), B, T, n_max, block_size, pool_blocks, top_k,
                                   _ptr(pool_pos), _ptr(pool_len), _ptr(topk_idx), _ptr(topk_score),
                                   _ptr(workspace), ws_bytes, _stream(stream, n_visible)))


def csa2_index_chain_workspace(B: int, T: int, n_max: int, block_size: int, pool_blocks: int,
                               top_k: int, L: int) -> int:
    return lib().csa2_index_chain_workspace(B, T, n_max, block_size, pool_blocks, top_k, L)


def csa2_index_chain(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int, n_max: int,
                     block_size: int, pool_blocks: int, top_k: int, ri_q, ri_w, L: int, pool_pos, pool_len,
                     topk_idx, topk_score, ri_topk_idx, ri_topk_score, workspace, ws_bytes: int,
                     stream=None) -> None:
    _check(lib().csa2_index_chain(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w), _ptr(n_visible),
                                  B, T, n_max, block_size, pool_blocks, top_k, _ptr(ri_q), _ptr(ri_w), L,
                                  _ptr(pool_pos), _ptr(pool_len), _ptr(topk_idx), _ptr(topk_score),
                                  _ptr(ri_topk_idx), _ptr(ri_topk_score), _ptr(workspace), ws_bytes,
                                  _stream(stream, idx_k)))


def csa2_noalloc_scratch_bytes() -> int:
    return lib().csa2_noalloc_scratch_bytes()


def csa2_index_chain_noalloc(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, n_visible, B: int, T: int,
                             n_max: int, block_size: int, pool_blocks: int, top_k: int, ri_q, ri_w, L: int,
                             pool_pos, pool_len, topk_idx, topk_score, ri_topk_idx, ri_topk_score,
                             stream=None) -> None:
    _check(lib().csa2_index_chain_noalloc(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w),
                                          _ptr(n_visible), B, T, n_max, block_size, pool_blocks, top_k, _ptr(ri_q),
                                          _ptr(ri_w), L, _ptr(pool_pos), _ptr(pool_len), _ptr(topk_idx),
                                          _ptr(topk_score), _ptr(ri_topk_idx), _ptr(ri_topk_score),
                                          _stream(stream, idx_k)))


def csa2_index_select_reindex(idx_k, idx_k_scales, k_rows_per_seq: int, n_visible, B: int, T: int, n_max: int,
                              block_size: int, pool_blocks: int, top_k: int, ri_q, ri_w, L: int,
                              pool_pos, pool_len, topk_idx, topk_score, ri_topk_idx, ri_topk_score,
                              workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_index_select_reindex(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(n_visible), B, T, n_max,
                                           block_size, pool_blocks, top_k, _ptr(ri_q), _ptr(ri_w), L,
                                           _ptr(pool_pos), _ptr(pool_len), _ptr(topk_idx), _ptr(topk_score),
                                           _ptr(ri_topk_idx), _ptr(ri_topk_score), _ptr(workspace), ws_bytes,
                                           _stream(stream, idx_k)))


def csa2_reindex_workspace(L: int, B: int, T: int, pool_cap: int, top_k: int) -> int:
    return lib().csa2_reindex_workspace(L, B, T, pool_cap, top_k)


def csa2_reindex(idx_k, idx_k_scales, k_rows_per_seq: int, idx_q, head_w, pool_pos, pool_len, pool_cap: int,
                 L: int, B: int, T: int, top_k: int, topk_idx, topk_score, workspace,
                 ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_reindex(_ptr(idx_k), _ptr(idx_k_scales), k_rows_per_seq, _ptr(idx_q), _ptr(head_w),
                              _ptr(pool_pos), _ptr(pool_len), pool_cap, L, B, T, top_k,
                              _ptr(topk_idx), _ptr(topk_score), _ptr(workspace), ws_bytes,
                              _stream(stream, idx_k)))


def csa2_sparse_attn_workspace(L: int, B: int, T: int, H: int, top_k: int, swa_window: int) -> int:
    return lib().csa2_sparse_attn_workspace(L, B, T, H, top_k, swa_window)


def csa2_sparse_attn(kv_codes, kv_scales, kv_rows_per_seq: int, q, idx_sets,
                     layer_set: Sequence[int], S: int, swa_kv, swa_rows: int, swa_end,
                     swa_window: int, L: int, B: int, T: int, H: int, top_k: int,
                     softmax_scale: float, out, lse, workspace, ws_bytes: int,
                     stream=None) -> None:
    ls = (ctypes.c_int32 * len(layer_set))(*[int(x) for x in layer_set])
    _check(lib().csa2_sparse_attn(_ptr(kv_codes), _ptr(kv_scales), kv_rows_per_seq, _ptr(q),
                                  _ptr(idx_sets), ctypes.cast(ls, ctypes.c_void_p), S,
                                  _ptr(swa_kv), swa_rows, _ptr(swa_end), swa_window, L, B, T, H,
                                  top_k, softmax_scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                  ws_bytes, _stream(stream, kv_codes)))


def csa2_encoder_chunk_workspace(B: int, T: int, k_rows: int, layers: int, H: int, top_k: int,
                                 swa_window: int) -> int:
    return lib().csa2_encoder_chunk_workspace(B, T, k_rows, layers, H, top_k, swa_window)


def csa2_encoder_chunk(G: int, layers: int, new_idx_k, new_latent, idx_k, kv_codes, kv_scales,
                       k_rows: int, idx_q, head_w, q, swa_kv, swa_rows: int, B: int, T: int, p0: int,
                       m: int, H: int, top_k: int, swa_window: int, softmax_scale: float, out,
                       topk_idx, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().csa2_encoder_chunk(G, layers, _ptr(new_idx_k), _ptr(new_latent), _ptr(idx_k),
                                    _ptr(kv_codes), _ptr(kv_scales), k_rows, _ptr(idx_q), _ptr(head_w),
                                    _ptr(q), _ptr(swa_kv), swa_rows, B, T, p0, m, H, top_k, swa_window,
                                    softmax_scale, _ptr(out), _ptr(topk_idx), _ptr(workspace), ws_bytes,
                                    _stream(stream, idx_k)))
