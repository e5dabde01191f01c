"""Oracle: block-causal attention (TEST INFRASTRUCTURE; see ``oracle/__init__.py``).

Definition followed (digest page, method step 3; editorial page, "The idea: OCR
as inverse rendering"; blog page, Fig. 2): the output sequence is cut into
consecutive blocks of ``L'`` tokens; a token attends to every token of its own
block (both directions) and to every token of all earlier blocks, and to no
token of a later block.  So query ``i`` sees key ``j`` exactly when
``floor(j / L') <= floor(i / L')``, i.e. ``j < key_limit(i)`` with
``key_limit(i) = min(L, (floor(i / L') + 1) * L')``.

Readings where the pages are silent:

* softmax scale ``1/sqrt(d)`` unless given;
* grouped-query heads: query head ``h`` reads KV head ``h // (Hq / Hkv)``;
* layout ``[batch, seq, heads, head_dim]`` for q, k, v, o and ``[batch, heads,
  seq]`` for the natural-log log-sum-exp;
* a sequence length that is not a multiple of ``L'`` ends in a short block.

Everything is float64 on the exact input values.  The loops run over query
*blocks*: every row of one block has the same visible key range, so one matmul
per block evaluates the definition directly.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def key_limit(i: int, seqlen: int, block_size: int) -> int:
    """Number of keys visible to query ``i`` (keys ``0 .. key_limit-1``)."""
    return min(seqlen, (i // block_size + 1) * block_size)


def block_mask(seqlen: int, block_size: int) -> np.ndarray:
    """Boolean ``[L, L]`` matrix, ``True`` where query ``i`` may attend key ``j``."""
    blk = np.arange(seqlen) // block_size
    return blk[None, :] <= blk[:, None]


def _scale(head_dim: int, scale: Optional[float]) -> float:
    return 1.0 / np.sqrt(head_dim) if (scale is None or scale <= 0) else float(scale)


def _softmax_rows(s: np.ndarray):
    """Row-wise max, exp-sum and normalised weights of score matrix ``s``."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_size: int,
             scale: Optional[float] = None, q_blocks: Optional[Sequence[int]] = None,
             heads: Optional[Sequence[int]] = None, batches: Optional[Sequence[int]] = None):
    """Block-causal attention forward.

    q ``[B, L, Hq, d]``, k/v ``[B, L, Hkv, d]`` (any float dtype; computed in
    float64).  Returns ``o [B, L, Hq, d]`` and ``lse [B, Hq, L]`` (float64).
    With ``q_blocks`` / ``heads`` / ``batches`` only those query blocks, query
    heads and batch entries are computed; the other entries are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, L, Hkv, d) and v.shape == k.shape and Hq % Hkv == 0
    G = Hq // Hkv
    sc = _scale(d, scale)
    nblk = -(-L // block_size)
    o = np.full((B, L, Hq, d), np.nan)
    lse = np.full((B, Hq, L), np.nan)
    for b in (range(B) if batches is None else batches):
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            for blk in (range(nblk) if q_blocks is None else q_blocks):
                r0, r1 = blk * block_size, min(L, (blk + 1) * block_size)
                kend = key_limit(r0, L, block_size)
                s = sc * (q[b, r0:r1, h, :] @ k[b, :kend, g, :].T)
                p, lse_rows = _softmax_rows(s)
                o[b, r0:r1, h, :] = p @ v[b, :kend, g, :]
                lse[b, h, r0:r1] = lse_rows
    return o, lse


def attn_fwd_bruteforce(q, k, v, block_size: int, scale: Optional[float] = None):
    """The same definition as scalar loops (for tiny shapes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, d = q.shape
    G = Hq // k.shape[2]
    sc = _scale(d, scale)
    o = np.zeros((B, L, Hq, d))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(L):
                scores = []
                for j in range(L):
                    if (j // block_size) <= (i // block_size):
                        acc = 0.0
                        for c in range(d):
                            acc += q[b, i, h, c] * k[b, j, g, c]
                        scores.append((j, sc * acc))
                mx = max(s for _, s in scores)
                den = sum(np.exp(s - mx) for _, s in scores)
                for j, s in scores:
                    w = np.exp(s - mx) / den
                    for c in range(d):
                        o[b, i, h, c] += w * v[b, j, g, c]
                lse[b, h, i] = mx + np.log(den)
    return o, lse


def attn_bwd(q, k, v, do, block_size: int, scale: Optional[float] = None,
             q_block_start: int = 0, batches: Optional[Sequence[int]] = None,
             heads_kv: Optional[Sequence[int]] = None):
    """Gradients of block-causal attention with respect to q, k and v.

    For loss ``sum(o * do)``: with ``P`` the attention weights of a query block,
    ``D_i = sum_c do_ic * o_ic``, ``dP = do V^T``, ``dS = P * (dP - D)``:
    ``dq = scale * dS K``, ``dk += scale * dS^T q``, ``dv += P^T do``, the last two
    summed over the query heads that share a KV head.

    Only query blocks ``>= q_block_start`` are processed.  Because a key in block
    ``c`` is seen only by queries in blocks ``>= c``, the returned
    ``dk``/``dv`` rows for keys ``>= q_block_start * L'`` are complete, as are the
    ``dq`` rows for queries ``>= q_block_start * L'``.  Returns
    ``dq [B, L-s, Hq, d]``, ``dk``/``dv [B, L-s, Hkv, d]`` for those rows
    (``s = q_block_start * L'``).  ``o`` is recomputed here from the definition.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = _scale(d, scale)
    nblk = -(-L // block_size)
    s0 = q_block_start * block_size
    dq = np.zeros((B, L - s0, Hq, d))
    dk = np.zeros((B, L, Hkv, d))
    dv = np.zeros((B, L, Hkv, d))
    for b in (range(B) if batches is None else batches):
        for g in (range(Hkv) if heads_kv is None else heads_kv):
            for h in range(g * G, (g + 1) * G):
                for blk in range(q_block_start, nblk):
                    r0, r1 = blk * block_size, min(L, (blk + 1) * block_size)
                    kend = key_limit(r0, L, block_size)
                    qb, dob = q[b, r0:r1, h, :], do[b, r0:r1, h, :]
                    kb, vb = k[b, :kend, g, :], v[b, :kend, g, :]
                    p, _ = _softmax_rows(sc * (qb @ kb.T))
                    ob = p @ vb
                    D = (dob * ob).sum(axis=-1, keepdims=True)
                    dp = dob @ vb.T
                    ds = p * (dp - D)
                    dq[b, r0 - s0:r1 - s0, h, :] = sc * (ds @ kb)
                    dk[b, :kend, g, :] += sc * (ds.T @ qb)
                    dv[b, :kend, g, :] += p.T @ dob
    return dq, dk[:, s0:], dv[:, s0:]


def decode_block(q_blk, k_blk, v_blk, k_cache, v_cache, prefix_start, prefix_len,
                 scale: Optional[float] = None):
    """One block of every sequence against that sequence's cached prefix.

    The digest page (novelty paragraph) notes that the block structure lets the
    decoder reuse the KV cache of the preceding blocks.  The block being decoded
    is the last block of its sequence, so all its tokens see the whole prefix and
    every token of the block itself: keys are ``prefix[0, P) ++ block[0, L')``
    with no mask.

    q_blk ``[n, L', Hq, d]``; k_blk/v_blk ``[n, L', Hkv, d]``; k_cache/v_cache
    ``[sum P, Hkv, d]`` with sequence ``s`` at rows
    ``prefix_start[s] .. prefix_start[s] + prefix_len[s] - 1``.
    Returns ``o [n, L', Hq, d]`` and ``lse [n, Hq, L']`` in float64.
    """
    q_blk = np.asarray(q_blk, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    n, T, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    sc = _scale(d, scale)
    o = np.zeros((n, T, Hq, d))
    lse = np.zeros((n, Hq, T))
    for s in range(n):
        a, P = int(prefix_start[s]), int(prefix_len[s])
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([k_cache[a:a + P, g, :], k_blk[s, :, g, :]], axis=0)
            vals = np.concatenate([v_cache[a:a + P, g, :], v_blk[s, :, g, :]], axis=0)
            p, lse_rows = _softmax_rows(sc * (q_blk[s, :, h, :] @ keys.T))
            o[s, :, h, :] = p @ vals
            lse[s, h, :] = lse_rows
    return o, lse


def attn_flops(seqlen: int, block_size: int, n_q_heads: int, head_dim: int, batch: int = 1) -> float:
    """Algorithmic forward flops: 4*d per allowed (query, key) pair (QK^T and PV)."""
    pairs = 0
    nblk = -(-seqlen // block_size)
    for blk in range(nblk):
        rows = min(seqlen, (blk + 1) * block_size) - blk * block_size
        pairs += rows * min(seqlen, (blk + 1) * block_size)
    return 4.0 * head_dim * pairs * n_q_heads * batch
