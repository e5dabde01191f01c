"""Block-diffusion decoding hot path on MI355X (gfx950): Python binding of libbd.

Each function has the name of the C entry point it calls (include/bd.h) and
only marshals arguments: it reads shapes off torch tensors, allocates outputs
and workspaces with torch when the caller passes none, and launches on the
current HIP stream.  All computation happens in the library's HIP kernels;
there is no fallback path.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import (BD_BF16, BD_F32, BD_FALLBACK_NONE, BD_FALLBACK_TOP1, BdError, check, lib)

__all__ = [
    "bd_attn_fwd", "bd_attn_bwd", "bd_attn_decode_block", "bd_confidence_commit", "bd_confidence_commit_noalloc",
    "bd_confidence_commit_rowwise", "bd_lmhead_commit", "bd_lmhead_commit_workspace_size",
    "bd_confidence_commit_sampled", "bd_confidence_commit_sampled_workspace_size",
    "bd_attn_decode_block_paged", "bd_kv_append_block",
    "bd_attn_bwd_workspace_size", "bd_attn_decode_workspace_size", "bd_confidence_commit_workspace_size",
    "BdError", "BD_F32", "BD_BF16", "BD_FALLBACK_NONE", "BD_FALLBACK_TOP1", "lib",
]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BD_BF16
    if t.dtype == torch.float32:
        return BD_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _out(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> Optional[torch.Tensor]:
    """A caller-supplied output (or None): the kernels write exactly `shape` elements of `dtype` to it."""
    if t is not None:
        _need(t, name, shape, dtype, device)
    return t


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]):
    if given is not None:
        _need(given, "workspace", device=device)
        return given, given.numel() * given.element_size()
    n = max(int(nbytes), 16)
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _row_outputs(rows: int, n_seq: int, dev, want_rows: bool, conf, pred, n_committed, n_masked_left):
    """The commit's optional outputs: caller-supplied ones checked, missing ones allocated."""
    conf = _out(conf, "conf", (rows,), torch.float32, dev)
    pred = _out(pred, "pred", (rows,), torch.int32, dev)
    n_committed = _out(n_committed, "n_committed", (n_seq,), torch.int32, dev)
    n_masked_left = _out(n_masked_left, "n_masked_left", (n_seq,), torch.int32, dev)
    if want_rows:
        conf = torch.empty(rows, dtype=torch.float32, device=dev) if conf is None else conf
        pred = torch.empty(rows, dtype=torch.int32, device=dev) if pred is None else pred
    n_committed = torch.empty(n_seq, dtype=torch.int32, device=dev) if n_committed is None else n_committed
    n_masked_left = torch.empty(n_seq, dtype=torch.int32, device=dev) if n_masked_left is None else n_masked_left
    return conf, pred, n_committed, n_masked_left


# ---------------------------------------------------------------------------
def bd_attn_fwd(q, k, v, block_size: int = 32, softmax_scale: float = 0.0, o=None, lse=None,
                want_lse: bool = True, stream=None):
    """Block-causal attention forward.  q [B,L,Hq,d], k/v [B,L,Hkv,d] -> (o, lse)."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    _need(q, "q")
    _need(k, "k", (B, L, Hkv, d), q.dtype, q.device)
    _need(v, "v", (B, L, Hkv, d), q.dtype, q.device)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", q.shape, q.dtype, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", (B, Hq, L), torch.float32, q.device)
    st = lib.bd_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, L, Hq, Hkv, d, block_size,
                         float(softmax_scale), _dtype_code(q), _stream(stream))
    check(st, "bd_attn_fwd")
    return o, lse


def bd_attn_bwd_workspace_size(batch, seqlen, n_q_heads, n_kv_heads, head_dim) -> int:
    return int(lib.bd_attn_bwd_workspace_size(batch, seqlen, n_q_heads, n_kv_heads, head_dim))


def bd_attn_bwd(q, k, v, o, lse, d_o, block_size: int = 32, softmax_scale: float = 0.0, dq=None, dk=None,
                dv=None, workspace=None, stream=None):
    """Gradients of bd_attn_fwd for the loss sum(o * d_o) -> (dq, dk, dv)."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    for t, n, shp in ((q, "q", None), (k, "k", (B, L, Hkv, d)), (v, "v", (B, L, Hkv, d)), (o, "o", q.shape),
                      (d_o, "d_o", q.shape)):
        _need(t, n, shp, q.dtype, q.device)
    _need(lse, "lse", (B, Hq, L), torch.float32, q.device)
    dq = torch.empty_like(q) if dq is None else _out(dq, "dq", q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _out(dk, "dk", k.shape, k.dtype, q.device)
    dv = torch.empty_like(v) if dv is None else _out(dv, "dv", v.shape, v.dtype, q.device)
    ws, nb = _workspace(bd_attn_bwd_workspace_size(B, L, Hq, Hkv, d), q.device, workspace)
    st = lib.bd_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
                         _ptr(ws), nb, B, L, Hq, Hkv, d, block_size, float(softmax_scale), _dtype_code(q),
                         _stream(stream))
    check(st, "bd_attn_bwd")
    return dq, dk, dv


def bd_attn_decode_workspace_size(n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim) -> int:
    return int(lib.bd_attn_decode_workspace_size(n_seq, blk_len, max_prefix_len, n_q_heads, n_kv_heads, head_dim))


def bd_attn_decode_block(q_blk, k_blk, v_blk, k_cache, v_cache, prefix_start, prefix_len, max_prefix_len: int,
                         softmax_scale: float = 0.0, o=None, lse=None, want_lse: bool = True, workspace=None,
                         stream=None):
    """One block per sequence against its prefix cache -> (o, lse)."""
    n, T, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    dev = q_blk.device
    _need(q_blk, "q_blk")
    _need(k_blk, "k_blk", (n, T, Hkv, d), q_blk.dtype, dev)
    _need(v_blk, "v_blk", (n, T, Hkv, d), q_blk.dtype, dev)
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t is not None:
            _need(t, name, None, q_blk.dtype, dev)
            if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, d):
                raise ValueError(f"{name} must be [rows, {Hkv}, {d}]")
    _need(prefix_start, "prefix_start", (n,), torch.int64, dev)
    _need(prefix_len, "prefix_len", (n,), torch.int32, dev)
    o = torch.empty_like(q_blk) if o is None else _out(o, "o", q_blk.shape, q_blk.dtype, dev)
    lse = _out(lse, "lse", (n, Hq, T), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((n, Hq, T), dtype=torch.float32, device=dev)
    ws, nb = _workspace(bd_attn_decode_workspace_size(n, T, max_prefix_len, Hq, Hkv, d), q_blk.device, workspace)
    st = lib.bd_attn_decode_block(_ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(prefix_start), _ptr(prefix_len), int(max_prefix_len), _ptr(o), _ptr(lse),
                                  n, T, Hq, Hkv, d, float(softmax_scale), _dtype_code(q_blk), _ptr(ws), nb,
                                  _stream(stream))
    check(st, "bd_attn_decode_block")
    return o, lse


def bd_confidence_commit_workspace_size(n_seq, blk_len, vocab) -> int:
    return int(lib.bd_confidence_commit_workspace_size(n_seq, blk_len, vocab))


def bd_confidence_commit(logits, tokens, masked, blk_len: int, threshold, fallback: int = BD_FALLBACK_TOP1,
                         vocab: Optional[int] = None, conf=None, pred=None, n_committed=None, n_masked_left=None,
                         want_rows: bool = True, workspace=None, stream=None):
    """Threshold commit; updates ``tokens``/``masked`` in place.

    logits [rows, >= vocab] (row stride = logits.stride(0)); tokens int32 [rows];
    masked uint8 [rows]; ``threshold`` a number (every row) or a float32 device
    tensor [rows] (one per row: ``bd_confidence_commit_rowwise``).  Returns
    dict(conf, pred, n_committed, n_masked_left).
    """
    rows = logits.shape[0]
    if rows % blk_len:
        raise ValueError("logits rows must be a multiple of blk_len")
    n_seq = rows // blk_len
    V = logits.shape[1] if vocab is None else int(vocab)
    if V > logits.shape[1]:
        raise ValueError(f"vocab {V} exceeds the {logits.shape[1]} logits per row")
    if not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a device tensor with unit stride along the vocabulary")
    dev = logits.device
    _need(tokens, "tokens", (rows,), torch.int32, dev)
    _need(masked, "masked", (rows,), torch.uint8, dev)
    conf, pred, n_committed, n_masked_left = _row_outputs(rows, n_seq, dev, want_rows, conf, pred, n_committed,
                                                          n_masked_left)
    ws, nb = _workspace(bd_confidence_commit_workspace_size(n_seq, blk_len, V), dev, workspace)
    if isinstance(threshold, torch.Tensor):
        _need(threshold, "threshold", (rows,), torch.float32, dev)
        st = lib.bd_confidence_commit_rowwise(_ptr(logits), logits.stride(0), n_seq, blk_len, V, _dtype_code(logits),
                                              _ptr(threshold), int(fallback), _ptr(tokens), _ptr(masked), _ptr(conf),
                                              _ptr(pred), _ptr(n_committed), _ptr(n_masked_left), _ptr(ws), nb,
                                              _stream(stream))
        check(st, "bd_confidence_commit_rowwise")
    else:
        st = lib.bd_confidence_commit(_ptr(logits), logits.stride(0), n_seq, blk_len, V, _dtype_code(logits),
                                      float(threshold), int(fallback), _ptr(tokens), _ptr(masked), _ptr(conf),
                                      _ptr(pred), _ptr(n_committed), _ptr(n_masked_left), _ptr(ws), nb,
                                      _stream(stream))
        check(st, "bd_confidence_commit")
    return {"conf": conf, "pred": pred, "n_committed": n_committed, "n_masked_left": n_masked_left}


def bd_confidence_commit_noalloc(logits, tokens, masked, blk_len: int, threshold: float,
                                 fallback: int = BD_FALLBACK_TOP1, vocab: Optional[int] = None, conf=None, pred=None,
                                 n_committed=None, n_masked_left=None, stream=None):
    """bd_confidence_commit with the library's fixed device scratch in place of a workspace (the
    C entry point allocates nothing; outputs not passed in are allocated here).  Updates
    ``tokens``/``masked`` in place; returns dict(conf, pred, n_committed, n_masked_left)."""
    rows = logits.shape[0]
    if rows % blk_len:
        raise ValueError("logits rows must be a multiple of blk_len")
    n_seq = rows // blk_len
    V = logits.shape[1] if vocab is None else int(vocab)
    if V > logits.shape[1]:
        raise ValueError(f"vocab {V} exceeds the {logits.shape[1]} logits per row")
    if not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a device tensor with unit stride along the vocabulary")
    dev = logits.device
    _need(tokens, "tokens", (rows,), torch.int32, dev)
    _need(masked, "masked", (rows,), torch.uint8, dev)
    conf = _out(conf, "conf", (rows,), torch.float32, dev)
    pred = _out(pred, "pred", (rows,), torch.int32, dev)
    n_committed = _out(n_committed, "n_committed", (n_seq,), torch.int32, dev)
    n_masked_left = _out(n_masked_left, "n_masked_left", (n_seq,), torch.int32, dev)
    st = lib.bd_confidence_commit_noalloc(_ptr(logits), logits.stride(0), n_seq, blk_len, V, _dtype_code(logits),
                                          float(threshold), int(fallback), _ptr(tokens), _ptr(masked), _ptr(conf),
                                          _ptr(pred), _ptr(n_committed), _ptr(n_masked_left), _stream(stream))
    check(st, "bd_confidence_commit_noalloc")
    return {"conf": conf, "pred": pred, "n_committed": n_committed, "n_masked_left": n_masked_left}


def bd_lmhead_commit_workspace_size(n_seq, blk_len, vocab) -> int:
    return int(lib.bd_lmhead_commit_workspace_size(n_seq, blk_len, vocab))


def bd_lmhead_commit(hidden, weight, tokens, masked, blk_len: int, threshold: float,
                     fallback: int = BD_FALLBACK_TOP1, conf=None, pred=None, n_committed=None, n_masked_left=None,
                     want_rows: bool = True, workspace=None, stream=None):
    """Output projection fused with the threshold commit; updates ``tokens``/``masked`` in place.

    hidden bf16 [rows, H] and weight bf16 [vocab, H] (unit stride along H); tokens int32 [rows];
    masked uint8 [rows].  Returns dict(conf, pred, n_committed, n_masked_left).
    """
    rows, H = hidden.shape
    if rows % blk_len:
        raise ValueError("hidden rows must be a multiple of blk_len")
    n_seq = rows // blk_len
    V = weight.shape[0]
    for t, name in ((hidden, "hidden"), (weight, "weight")):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor with unit stride along the hidden dimension")
    if weight.shape[1] != H:
        raise ValueError("weight must be [vocab, hidden]")
    dev = hidden.device
    if weight.device != dev:
        raise ValueError(f"weight is on {weight.device}, expected {dev}")
    _need(tokens, "tokens", (rows,), torch.int32, dev)
    _need(masked, "masked", (rows,), torch.uint8, dev)
    conf, pred, n_committed, n_masked_left = _row_outputs(rows, n_seq, dev, want_rows, conf, pred, n_committed,
                                                          n_masked_left)
    ws, nb = _workspace(bd_lmhead_commit_workspace_size(n_seq, blk_len, V), dev, workspace)
    st = lib.bd_lmhead_commit(_ptr(hidden), hidden.stride(0), _ptr(weight), weight.stride(0), n_seq, blk_len, H, V,
                              float(threshold), int(fallback), _ptr(tokens), _ptr(masked), _ptr(conf), _ptr(pred),
                              _ptr(n_committed), _ptr(n_masked_left), _ptr(ws), nb, _stream(stream))
    check(st, "bd_lmhead_commit")
    return {"conf": conf, "pred": pred, "n_committed": n_committed, "n_masked_left": n_masked_left}


def bd_confidence_commit_sampled_workspace_size(n_seq, blk_len, vocab) -> int:
    return int(lib.bd_confidence_commit_sampled_workspace_size(n_seq, blk_len, vocab))


def bd_confidence_commit_sampled(logits, tokens, masked, blk_len: int, threshold: float, temperature: float = 1.0,
                                 seed: int = 0, step: int = 0, fallback: int = BD_FALLBACK_TOP1,
                                 vocab: Optional[int] = None, top_k: int = 0, top_p: float = 1.0, conf=None,
                                 pred=None, n_committed=None, n_masked_left=None, want_rows: bool = True,
                                 workspace=None, stream=None):
    """Threshold commit with sampled predictions (temperature, then top-k / top-p truncation, then
    Philox4x32-10 keyed by seed/row/step); updates ``tokens``/``masked`` in place.  Returns
    dict(conf, pred, n_committed, n_masked_left)."""
    rows = logits.shape[0]
    if rows % blk_len:
        raise ValueError("logits rows must be a multiple of blk_len")
    n_seq = rows // blk_len
    V = logits.shape[1] if vocab is None else int(vocab)
    if V > logits.shape[1]:
        raise ValueError(f"vocab {V} exceeds the {logits.shape[1]} logits per row")
    if not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a device tensor with unit stride along the vocabulary")
    dev = logits.device
    _need(tokens, "tokens", (rows,), torch.int32, dev)
    _need(masked, "masked", (rows,), torch.uint8, dev)
    conf, pred, n_committed, n_masked_left = _row_outputs(rows, n_seq, dev, want_rows, conf, pred, n_committed,
                                                          n_masked_left)
    ws, nb = _workspace(bd_confidence_commit_sampled_workspace_size(n_seq, blk_len, V), dev, workspace)
    st = lib.bd_confidence_commit_sampled(_ptr(logits), logits.stride(0), n_seq, blk_len, V, _dtype_code(logits),
                                          float(temperature), int(seed), int(step), int(top_k), float(top_p),
                                          float(threshold), int(fallback),
                                          _ptr(tokens), _ptr(masked), _ptr(conf), _ptr(pred), _ptr(n_committed),
                                          _ptr(n_masked_left), _ptr(ws), nb, _stream(stream))
    check(st, "bd_confidence_commit_sampled")
    return {"conf": conf, "pred": pred, "n_committed": n_committed, "n_masked_left": n_masked_left}


def bd_attn_decode_block_paged(q_blk, k_blk, v_blk, k_pages, v_pages, block_table, page_size: int, prefix_len,
                               max_prefix_len: int, softmax_scale: float = 0.0, o=None, lse=None, workspace=None,
                               stream=None):
    """One block against a paged prefix cache.  q_blk [n_seq, T, Hq, d], k_blk/v_blk [n_seq, T, Hkv, d],
    k_pages/v_pages [n_pages * page_size, Hkv, d] (bf16), block_table int32 [n_seq, max_pages],
    prefix_len int32 [n_seq].  Returns (o, lse)."""
    n_seq, T, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    dev = q_blk.device
    _need(q_blk, "q_blk", dtype=torch.bfloat16)
    _need(k_blk, "k_blk", (n_seq, T, Hkv, d), torch.bfloat16, dev)
    _need(v_blk, "v_blk", (n_seq, T, Hkv, d), torch.bfloat16, dev)
    for t, name in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, dtype=torch.bfloat16, device=dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, d):
            raise ValueError(f"{name} must be [n_pages * page_size, {Hkv}, {d}]")
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(prefix_len, "prefix_len", (n_seq,), torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != n_seq:
        raise ValueError("block_table must be [n_seq, max_pages]")
    o = torch.empty_like(q_blk) if o is None else _out(o, "o", q_blk.shape, torch.bfloat16, dev)
    lse = torch.empty((n_seq, Hq, T), dtype=torch.float32, device=dev) if lse is None else \
        _out(lse, "lse", (n_seq, Hq, T), torch.float32, dev)
    ws, nb = _workspace(bd_attn_decode_workspace_size(n_seq, T, max_prefix_len, Hq, Hkv, d), dev, workspace)
    st = lib.bd_attn_decode_block_paged(_ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pages), _ptr(v_pages),
                                        _ptr(block_table), block_table.shape[1], page_size, _ptr(prefix_len),
                                        max_prefix_len, _ptr(o), _ptr(lse), n_seq, T, Hq, Hkv, d,
                                        float(softmax_scale), BD_BF16, _ptr(ws), nb, _stream(stream))
    check(st, "bd_attn_decode_block_paged")
    return o, lse


def bd_kv_append_block(k_blk, v_blk, k_pages, v_pages, block_table, page_size: int, prefix_len, n_masked_left=None,
                       stream=None):
    """Append finished blocks (n_masked_left == 0, or all) to the paged cache; prefix_len grows in place."""
    n_seq, T, Hkv, d = k_blk.shape
    dev = k_blk.device
    _need(k_blk, "k_blk", dtype=torch.bfloat16)
    _need(v_blk, "v_blk", (n_seq, T, Hkv, d), torch.bfloat16, dev)
    for t, name in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, dtype=torch.bfloat16, device=dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, d):
            raise ValueError(f"{name} must be [n_pages * page_size, {Hkv}, {d}]")
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    if block_table.dim() != 2 or block_table.shape[0] != n_seq:
        raise ValueError("block_table must be [n_seq, max_pages]")
    _need(prefix_len, "prefix_len", (n_seq,), torch.int32, dev)
    if n_masked_left is not None:
        _need(n_masked_left, "n_masked_left", (n_seq,), torch.int32, dev)
    st = lib.bd_kv_append_block(_ptr(k_blk), _ptr(v_blk), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                block_table.shape[1], page_size, _ptr(prefix_len),
                                _ptr(n_masked_left) if n_masked_left is not None else None, n_seq, T, Hkv, d, BD_BF16,
                                _stream(stream))
    check(st, "bd_kv_append_block")
