"""Oracle: the LM head in front of the confidence commit (TEST INFRASTRUCTURE; see
``oracle/__init__.py``).

What it follows: the commit acts on the prediction of each masked position
(digest page, method step 4); the prediction is the decoder's distribution
over the shared vocabulary (digest page, method step 1), i.e. the softmax of
the logits that the output projection ("LM head") makes from the last hidden
state.  Fusing that projection with the confidence reduction is a "next" row of
the build (the logits are never stored); the arithmetic is unchanged:

    logits[r, v] = sum_k hidden[r, k] * weight[v, k]      (weight: [vocab, hidden])

then the commit of :mod:`oracle.commit` on those logits.  Readings: no bias and
no scaling (the pages name none); float64 on the exact bf16 input values.
"""
from __future__ import annotations

import numpy as np

from . import commit as C


def lmhead_logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """[rows, hidden] x [vocab, hidden]^T -> [rows, vocab], float64."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T


def lmhead_commit(hidden: np.ndarray, weight: np.ndarray, tokens: np.ndarray, masked: np.ndarray,
                  blk_len: int, threshold, fallback: str = C.FALLBACK_TOP1):
    """The commit step of :func:`oracle.commit.confidence_commit` on ``hidden @ weight.T``."""
    return C.confidence_commit(lmhead_logits(hidden, weight), tokens, masked, blk_len, threshold, fallback)
