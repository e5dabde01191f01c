"""Oracle: the prefix cache held in pages (TEST INFRASTRUCTURE; see ``oracle/__init__.py``).

What it follows: the block structure lets later blocks reuse the KV cache of the earlier ones
(digest page, novelty paragraph); the serving engines the pages name for the model (SGLang and
the Nano-vLLM adaptation: editorial page, "The model, the weights and the serving stack") keep
that cache in fixed-size pages addressed through a per-sequence page table.  The attention does
not change: decoding a block against a paged prefix is :func:`oracle.attention.decode_block` on
the prefix gathered back into order, and appending a finished block writes its rows after the
prefix.  Layout (the reading taken): pages ``[n_pages * page_size, Hkv, d]``, page p holding cache
rows p*page_size .. p*page_size + page_size - 1; ``block_table[s][i]`` is the page of prefix rows
i*page_size .. i*page_size + page_size - 1 of sequence s.
"""
from __future__ import annotations

import numpy as np

from . import attention as A


def prefix_rows(block_table: np.ndarray, s: int, P: int, page_size: int) -> np.ndarray:
    """Page-buffer row of each prefix row 0 .. P-1 of sequence s."""
    j = np.arange(P)
    return np.asarray(block_table)[s, j // page_size].astype(np.int64) * page_size + j % page_size


def gather_prefixes(pages: np.ndarray, block_table: np.ndarray, prefix_len, page_size: int):
    """The prefixes of all sequences back in order, packed: ([sum P, Hkv, d], prefix_start)."""
    prefix_len = np.asarray(prefix_len, dtype=np.int64)
    start = np.concatenate([[0], np.cumsum(prefix_len)[:-1]]).astype(np.int64)
    rows = [prefix_rows(block_table, s, int(P), page_size) for s, P in enumerate(prefix_len)]
    idx = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    return np.asarray(pages)[idx], start


def decode_block_paged(q_blk, k_blk, v_blk, k_pages, v_pages, block_table, prefix_len, page_size: int,
                       scale=None):
    """:func:`oracle.attention.decode_block` with the prefix read through the page table."""
    kc, start = gather_prefixes(k_pages, block_table, prefix_len, page_size)
    vc, _ = gather_prefixes(v_pages, block_table, prefix_len, page_size)
    return A.decode_block(q_blk, k_blk, v_blk, kc, vc, start, prefix_len, scale)


def append_block(k_pages, v_pages, block_table, prefix_len, k_blk, v_blk, page_size: int, n_masked_left=None):
    """Write each finished block (n_masked_left[s] == 0, or every block) after its prefix and grow
    the prefix; a block that would pass the sequence's last page is left out.  Returns new arrays."""
    k_pages, v_pages = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    prefix_len = np.array(prefix_len, dtype=np.int32, copy=True)
    n, T = k_blk.shape[:2]
    max_pages = np.asarray(block_table).shape[1]
    for s in range(n):
        if n_masked_left is not None and n_masked_left[s] != 0:
            continue
        P = int(prefix_len[s])
        if P + T > max_pages * page_size:
            continue
        rows = prefix_rows(block_table, s, P + T, page_size)[P:]
        k_pages[rows] = k_blk[s]
        v_pages[rows] = v_blk[s]
        prefix_len[s] = P + T
    return k_pages, v_pages, prefix_len
