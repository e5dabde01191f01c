"""Oracle: confidence-threshold token commit (TEST INFRASTRUCTURE; see ``oracle/__init__.py``).

Definition followed (digest page, method step 4 "confidence dynamic
scheduling", and method step 6 inference settings T = 0.95, top-k 0,
temperature 1.0, top-p 1.0; editorial page and blog page Fig. 1 on confirmed /
updating / masked tokens): after each denoising step, a still-masked position
whose prediction confidence exceeds the threshold T is confirmed; the others
stay masked and are predicted again at the next step.

Readings where the pages are silent or loose:

* confidence = the largest softmax probability over the whole vocabulary at
  temperature 1, i.e. ``exp(l_max - logsumexp(l)) = 1 / sum_v exp(l_v - l_max)``;
* the committed id is the argmax (greedy), lowest id on ties;
* "exceeds" is strict: ``conf > T``;
* confirmed tokens stay confirmed;
* if no masked token of a block clears T, the block commits its single most
  confident masked token (lowest row on ties) -- a stated choice, not a rule of
  the pages; ``fallback="none"`` turns it off;
* a row holding NaN or +Inf, or only -Inf, has confidence NaN: it never
  commits and never wins the fallback; -Inf entries alone are legal and add
  nothing to the sum.

A threshold per position (the digest's weaknesses, point 2: local thresholds
that follow the complexity of each region, in place of one global T) is
taken as one T_r per row: row r clears it when ``conf_r > T_r``; a NaN T_r is
never cleared.  The fallback rule is the same as with one threshold.
"""
from __future__ import annotations

import numpy as np

FALLBACK_NONE = "none"
FALLBACK_TOP1 = "top1"


def row_confidence(row: np.ndarray):
    """(confidence, argmax id) of one logit row, float64.  NaN and -1 if the row is invalid."""
    x = np.asarray(row, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any():
        return float("nan"), -1
    m = x.max()
    if np.isneginf(m):
        return float("nan"), -1
    a = int(np.flatnonzero(x == m)[0])
    s = np.exp(x - m).sum()
    return float(1.0 / s), a


def confidence_commit(logits: np.ndarray, tokens: np.ndarray, masked: np.ndarray,
                      blk_len: int, threshold, fallback: str = FALLBACK_TOP1):
    """One commit step over ``n_seq`` blocks of ``blk_len`` rows each.

    ``threshold`` is one number for every row or an array of one per row.

    ``logits [n_seq*blk_len, V]``; ``tokens`` int32 and ``masked`` uint8 (1 =
    still masked) of length ``n_seq*blk_len``.  Rows that are not masked on entry
    are neither read nor changed.  Returns a dict with the new ``tokens`` and
    ``masked``, per-row ``conf`` (float64, NaN for rows not masked on entry) and
    ``pred`` (int32, -1 for rows not masked or invalid), the per-block
    ``n_committed`` and ``n_masked_left``, and ``committed`` (bool per row).
    """
    logits = np.asarray(logits)
    R = logits.shape[0]
    conf = np.full(R, np.nan)
    pred = np.full(R, -1, dtype=np.int32)
    for r in range(R):
        if masked[r]:
            conf[r], pred[r] = row_confidence(logits[r])
    return decide(conf, pred, tokens, masked, blk_len, threshold, fallback)


def decide(conf: np.ndarray, pred: np.ndarray, tokens: np.ndarray, masked: np.ndarray,
           blk_len: int, threshold, fallback: str = FALLBACK_TOP1):
    """The threshold rule, the fallback and the state update, given each masked row's confidence
    and predicted id (NaN / -1 for invalid rows)."""
    R = len(conf)
    assert R % blk_len == 0
    n_seq = R // blk_len
    tokens = np.array(tokens, dtype=np.int32, copy=True)
    masked = np.array(masked, dtype=np.uint8, copy=True)
    conf = np.asarray(conf, dtype=np.float64)
    pred = np.asarray(pred, dtype=np.int32)
    thr = np.broadcast_to(np.asarray(threshold, dtype=np.float64), (R,))
    committed = np.zeros(R, dtype=bool)
    n_committed = np.zeros(n_seq, dtype=np.int32)
    n_left = np.zeros(n_seq, dtype=np.int32)
    for g in range(n_seq):
        rows = range(g * blk_len, (g + 1) * blk_len)
        chosen = [r for r in rows if masked[r] and not np.isnan(conf[r]) and conf[r] > thr[r]]
        if not chosen and fallback == FALLBACK_TOP1:
            best = None
            for r in rows:
                if masked[r] and not np.isnan(conf[r]) and (best is None or conf[r] > conf[best]):
                    best = r
            if best is not None:
                chosen = [best]
        for r in chosen:
            committed[r] = True
            tokens[r] = pred[r]
            masked[r] = 0
        n_committed[g] = len(chosen)
        n_left[g] = int(masked[g * blk_len:(g + 1) * blk_len].sum())
    return {"tokens": tokens, "masked": masked, "conf": conf.copy(), "pred": pred.copy(),
            "n_committed": n_committed, "n_masked_left": n_left, "committed": committed}
