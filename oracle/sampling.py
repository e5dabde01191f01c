"""Oracle: the sampling variant of the confidence commit (TEST INFRASTRUCTURE; see
``oracle/__init__.py``).

What it follows: at inference the pages decode with temperature 1.0, top-k 0 and top-p 1.0
(digest page, method step 6), i.e. tokens are drawn from the full softmax at temperature 1 with
no truncation; a masked position is confirmed when its confidence exceeds T (method step 4).
The greedy commit (:mod:`oracle.commit`) reads "temperature 1" as the argmax; this module is
the sampling reading:

* p_v = softmax(logits / tau)_v over the whole vocabulary (tau = the temperature, 1 on the
  pages; top-k and top-p stay off, as the pages set them);
* one uniform u in (0, 1) per row and step from a counter-based generator (below); the sampled
  id is the first v (in id order) whose cumulative probability sum_{w <= v} p_w exceeds u
  (inverse-CDF sampling);
* confidence = p of the sampled id; the threshold rule, the fallback and the state update are
  those of :func:`oracle.commit.confidence_commit`, with the sampled id in place of the argmax.

Truncation (the pages name the top-k and top-p knobs and switch both off; the reading below
applies when a caller turns them on), in the order the pages list the knobs -- temperature, then
top-k, then top-p:

* top-k (k >= 1): keep the ids whose logit is at least the k-th largest finite logit of the row
  (counted with multiplicity); ids with equal logits are kept or dropped together, so a tie at the
  k-th place keeps more than k ids.  k = 0, or k at least the number of finite logits, keeps all.
* top-p (nucleus sampling, Holtzman et al., "The Curious Case of Neural Text Degeneration",
  ICLR 2020), 0 < p <= 1: on the distribution left by top-k (renormalised), keep the smallest set
  of highest-probability ids whose total probability reaches p -- the ids down to the first
  logit value at which the running total, taken over distinct values in decreasing order, is at
  least p times the total; ties are again kept together.  p = 1 keeps all.
* the sampled id and its confidence then come from the kept ids only, renormalised: the first id
  (in id order) whose running weight passes u times the kept total; conf = its weight over that
  total.

Counter-based generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011), written from its published definition: a 4 x 32-bit
counter and a 2 x 32-bit key; each round multiplies words 0 and 2 of the counter by the two
round multipliers, forms the new counter from the high and low product halves xored with the
other two words and the key, and the key is bumped by the two Weyl constants between rounds.
Row r at step n draws counter (r, n mod 2^32, n >> 32, 0) under key (seed mod 2^32, seed >> 32);
u = (word 0 + 1/2) / 2^32.
"""
from __future__ import annotations

import numpy as np

from . import commit as C

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter under a 2-word key (Python ints); returns 4 words."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in ctr)
    k0, k1 = (int(x) & MASK32 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def row_uniform(seed: int, row: int, step: int) -> float:
    """The uniform u in (0, 1) of row ``row`` at step ``step`` under ``seed``."""
    w0 = philox4x32_10((row, step & MASK32, (step >> 32) & MASK32, 0), (seed & MASK32, (seed >> 32) & MASK32))[0]
    return (w0 + 0.5) / 4294967296.0


def truncation_cut(row: np.ndarray, tau: float, top_k: int = 0, top_p: float = 1.0) -> float:
    """The smallest logit value kept by top-k and then top-p (every id whose logit is at least this
    value is kept); -inf when neither cuts anything.  The row must be valid (see row_sample)."""
    assert top_k >= 0 and 0.0 < top_p <= 1.0
    x = np.asarray(row, dtype=np.float64)
    fin = x[np.isfinite(x)]
    cut = -np.inf
    if 1 <= top_k < len(fin):
        cut = float(np.sort(fin)[::-1][top_k - 1])          # the k-th largest, with multiplicity
    if top_p < 1.0:
        kept = fin[fin >= cut]
        vals, counts = np.unique(kept, return_counts=True)  # distinct values, ascending
        vals, counts = vals[::-1], counts[::-1]
        mass = counts * np.exp((vals - vals[0]) / tau)      # weight of each distinct value's ids
        cum = np.cumsum(mass)
        first = int(np.flatnonzero(cum >= top_p * cum[-1])[0])
        cut = max(cut, float(vals[first]))
    return cut


def row_sample(row: np.ndarray, tau: float, u: float, top_k: int = 0, top_p: float = 1.0):
    """(probability of the sampled id, sampled id) of one logit row at temperature tau, after the
    top-k / top-p truncation; NaN and -1 for an invalid row (NaN or +Inf anywhere, or only -Inf)."""
    x = np.asarray(row, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any():
        return float("nan"), -1
    m = x.max()
    if np.isneginf(m):
        return float("nan"), -1
    if top_k or top_p < 1.0:
        x = np.where(x >= truncation_cut(x, tau, top_k, top_p), x, -np.inf)
    w = np.exp((x - m) / tau)
    p = w / w.sum()
    cum = np.cumsum(p)
    s = int(np.flatnonzero(cum > u)[0]) if (cum > u).any() else int(np.flatnonzero(p > 0)[-1])
    return float(p[s]), s


def sampled_commit(logits: np.ndarray, tokens: np.ndarray, masked: np.ndarray, blk_len: int,
                   threshold, temperature: float, seed: int, step: int, fallback: str = C.FALLBACK_TOP1,
                   top_k: int = 0, top_p: float = 1.0):
    """One commit step with sampled predictions; same outputs as :func:`oracle.commit.confidence_commit`,
    plus ``u`` (the uniform of every row; NaN for rows not masked on entry)."""
    logits = np.asarray(logits)
    R = logits.shape[0]
    conf = np.full(R, np.nan)
    pred = np.full(R, -1, dtype=np.int32)
    us = np.full(R, np.nan)
    for r in range(R):
        if masked[r]:
            us[r] = row_uniform(seed, r, step)
            conf[r], pred[r] = row_sample(logits[r], temperature, us[r], top_k, top_p)
    out = C.decide(conf, pred, tokens, masked, blk_len, threshold, fallback)
    out["u"] = us
    return out
