"""Pins of the oracle's confidence-threshold commit and of the decode loop (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import commit as C
from oracle import decode_loop as DL


def _golden_rows(golden_dir):
    out = []
    for ln in open(os.path.join(golden_dir, "commit_rows.txt")):
        if not ln.strip() or ln.startswith("#"):
            continue
        conf, ident, row = [x.strip() for x in ln.split(";")]
        vals = []
        for tok in row.split():
            vals.append(math.log(float(tok[1:])) if tok.startswith("L") else float(tok))
        out.append((float(conf), int(ident), np.array(vals)))
    return out


def test_golden_rows(golden_dir):
    rows = _golden_rows(golden_dir)
    assert len(rows) == 6
    for conf, ident, row in rows:
        c, a = C.row_confidence(row)
        assert abs(c - conf) < 1e-15 and a == ident


@pytest.mark.parametrize("V", [2, 1000, 151936])
@pytest.mark.parametrize("T", [0.5, 0.95, 0.99])
def test_closed_form_one_peak(V, T):
    """One value a and V-1 values c: conf = 1 / (1 + (V-1) exp(c - a)).  Place conf at T +- 1e-3."""
    for delta, want in ((1e-3, True), (-1e-3, False)):
        target = T + delta
        gap = math.log((V - 1) * target / (1.0 - target))  # a - c
        if gap <= 0:  # the single value is not the maximum: the closed form does not apply
            continue
        row = np.zeros(V)
        row[V // 3] = gap
        c, a = C.row_confidence(row)
        assert abs(c - target) < 1e-12 and a == V // 3
        res = C.confidence_commit(row[None].repeat(1, 0), np.array([-1]), np.array([1], np.uint8), 1, T,
                                  C.FALLBACK_NONE)
        assert bool(res["committed"][0]) == want


def test_matches_torch_softmax():
    x = np.random.default_rng(1).standard_normal((16, 777)) * 3
    p = torch.softmax(torch.from_numpy(x), dim=-1)
    for r in range(16):
        c, a = C.row_confidence(x[r])
        assert abs(c - float(p[r].max())) < 1e-14
        assert a == int(torch.argmax(p[r]))


def _case(seed, n_seq=6, blk=8, V=50, std=2.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((n_seq * blk, V)) * std
    logits[np.arange(n_seq * blk), rng.integers(0, V, n_seq * blk)] += rng.uniform(0, 8, n_seq * blk)
    masked = (rng.random(n_seq * blk) < 0.7).astype(np.uint8)
    tokens = np.where(masked == 1, -1, rng.integers(0, V, n_seq * blk)).astype(np.int32)
    return logits, tokens, masked, blk, V


@pytest.mark.parametrize("seed", range(5))
def test_invariants(seed):
    logits, tokens, masked, blk, V = _case(seed)
    for T in (0.3, 0.6, 0.9):
        res = C.confidence_commit(logits, tokens, masked, blk, T)
        conf = res["conf"]
        m = masked == 1
        assert np.all((conf[m] >= 1.0 / V - 1e-15) & (conf[m] <= 1.0))          # (a)
        assert np.all(np.isnan(conf[~m]))
        for g in range(len(tokens) // blk):
            sl = slice(g * blk, (g + 1) * blk)
            above = m[sl] & (conf[sl] > T)
            if above.any():                                                     # (b)
                assert np.array_equal(res["committed"][sl], above)
            elif m[sl].any():
                assert res["committed"][sl].sum() == 1
                r = np.flatnonzero(res["committed"][sl])[0]
                assert conf[sl][r] == np.nanmax(np.where(m[sl], conf[sl], np.nan))
            assert res["n_committed"][g] == res["committed"][sl].sum()           # (g)
            assert res["n_masked_left"][g] == m[sl].sum() - res["n_committed"][g]
        assert np.array_equal(res["tokens"][~m], tokens[~m])                    # (f)
        assert np.array_equal(res["masked"][~m], masked[~m])
        assert np.array_equal(res["tokens"][res["committed"]], res["pred"][res["committed"]])
    lo = C.confidence_commit(logits, tokens, masked, blk, 0.4, C.FALLBACK_NONE)["committed"]
    hi = C.confidence_commit(logits, tokens, masked, blk, 0.8, C.FALLBACK_NONE)["committed"]
    assert np.all(lo | ~hi)                                                     # (c) nested


def test_threshold_extremes():
    logits, tokens, masked, blk, V = _case(7)
    res = C.confidence_commit(logits, tokens, masked, blk, 1.0)                 # (d)
    for g in range(len(tokens) // blk):
        sl = slice(g * blk, (g + 1) * blk)
        assert res["n_committed"][g] == (1 if masked[sl].any() else 0)
    res = C.confidence_commit(logits, tokens, masked, blk, 0.5 / V)             # (e)
    assert np.array_equal(res["committed"], masked == 1)
    assert not res["masked"].any()


def test_tie_breaks():
    row = np.array([1.0, 3.0, 0.0, 3.0])
    assert C.row_confidence(row)[1] == 1
    logits = np.array([[0.0, 1.0], [1.0, 0.0], [0.0, 0.5]])
    res = C.confidence_commit(logits, np.full(3, -1, np.int32), np.ones(3, np.uint8), 3, 0.99)
    assert list(res["committed"]) == [True, False, False]      # rows 0 and 1 tie: lowest row
    assert res["tokens"][0] == 1


def test_invalid_rows():
    V = 5
    rows = np.array([[0, np.nan, 1, 2, 3], [0, np.inf, 1, 2, 3], [-np.inf] * V,
                     [-np.inf, -np.inf, 2.0, -np.inf, -np.inf]])
    res = C.confidence_commit(rows, np.full(4, -1, np.int32), np.ones(4, np.uint8), 4, 0.5)
    assert np.isnan(res["conf"][:3]).all() and (res["pred"][:3] == -1).all()
    assert res["conf"][3] == 1.0 and res["pred"][3] == 2
    assert list(res["committed"]) == [False, False, False, True]
    res = C.confidence_commit(rows[:3], np.full(3, -1, np.int32), np.ones(3, np.uint8), 3, 0.5)
    assert not res["committed"].any() and res["n_masked_left"][0] == 3


def test_loop_threshold_one_is_token_level():
    """T >= 1: nothing clears the threshold, so the fallback commits one token per step and a
    block of L' tokens takes exactly L' steps (the "near token-level" end of the T knob)."""
    rng = np.random.default_rng(3)
    n, blk, V = 3, 8, 20
    res = DL.decode_loop(n, blk, lambda s: rng.standard_normal((n * blk, V)), 1.0)
    assert list(res["steps"]) == [blk] * n
    assert not res["masked"].any()
    for g in range(n):
        assert sorted(res["commit_step"][g * blk:(g + 1) * blk]) == list(range(blk))


def test_loop_low_threshold_is_one_step():
    rng = np.random.default_rng(4)
    n, blk, V = 2, 8, 20
    res = DL.decode_loop(n, blk, lambda s: rng.standard_normal((n * blk, V)), 0.5 / V)
    assert list(res["steps"]) == [1, 1]


def test_loop_scripted_schedule():
    """Scripted logits: row r becomes confident (conf 0.99) at step r // 2 and stays low before.
    Then a block of 8 commits two rows per step and finishes in 4 steps."""
    blk, V = 8, 10
    def logits(step):
        x = np.zeros((blk, V))
        for r in range(blk):
            if r // 2 <= step:
                x[r, r % V] = math.log(0.99 * (V - 1) / 0.01)
        return x
    res = DL.decode_loop(1, blk, logits, 0.95)
    assert res["steps"][0] == 4
    assert list(res["commit_step"]) == [0, 0, 1, 1, 2, 2, 3, 3]
    assert list(res["tokens"]) == [r % V for r in range(blk)]


def test_loop_with_sampled_commit():
    """The loop with the sampled commit rule in place of the greedy one.  (i) The scripted
    schedule above at temperature 0.05: a confident row's boosted id then holds all but
    e^-136 of the probability, so every draw takes it and the schedule, the commit steps and the
    tokens are those of the greedy loop.  (ii) T >= 1 stays token-level: one fallback commit per
    step whatever the rule, so a block of L' tokens takes exactly L' steps."""
    from oracle import sampling as S
    blk, V = 8, 10

    def logits(step):
        x = np.zeros((blk, V))
        for r in range(blk):
            if r // 2 <= step:
                x[r, r % V] = math.log(0.99 * (V - 1) / 0.01)
        return x

    def sampled(tau, seed):
        return lambda lg, tok, msk, b, T, fb, step: S.sampled_commit(lg, tok, msk, b, T, tau, seed, step, fb)

    res = DL.decode_loop(1, blk, logits, 0.95, commit=sampled(0.05, 11))
    assert res["steps"][0] == 4
    assert list(res["commit_step"]) == [0, 0, 1, 1, 2, 2, 3, 3]
    assert list(res["tokens"]) == [r % V for r in range(blk)]
    rng = np.random.default_rng(5)
    n = 3
    res = DL.decode_loop(n, blk, lambda s: rng.standard_normal((n * blk, V)), 1.0, commit=sampled(1.0, 12))
    assert list(res["steps"]) == [blk] * n and not res["masked"].any()
    for g in range(n):
        assert sorted(res["commit_step"][g * blk:(g + 1) * blk]) == list(range(blk))


@pytest.mark.parametrize("seed", range(3))
def test_loop_bounds(seed):
    rng = np.random.default_rng(seed)
    n, blk, V = 4, 8, 30
    def logits(step):
        x = rng.standard_normal((n * blk, V))
        x[np.arange(n * blk), rng.integers(0, V, n * blk)] += rng.uniform(0, 8, n * blk)
        return x
    res = DL.decode_loop(n, blk, logits, 0.9)
    assert np.all((res["steps"] >= 1) & (res["steps"] <= blk))
    assert not res["masked"].any() and (res["tokens"] >= 0).all()


def test_per_row_thresholds_closed_form():
    """Per-position thresholds: rows built with a known confidence (one value a, V-1 values 0:
    conf = 1 / (1 + (V-1) exp(-a))) and each row's own T placed 1e-3 above or below it; the rows
    that commit are exactly those whose T lies below, whatever the other rows' T."""
    V, blk, n_seq = 300, 6, 4
    rng = np.random.default_rng(3)
    R = n_seq * blk
    target = rng.uniform(0.2, 0.9, R)
    gap = np.log((V - 1) * target / (1.0 - target))
    logits = np.zeros((R, V))
    ids = rng.integers(0, V, R)
    logits[np.arange(R), ids] = gap
    below = rng.random(R) < 0.5
    below[:blk] = False                       # block 0: nobody clears, fallback takes the top row
    thr = np.where(below, target - 1e-3, target + 1e-3)
    thr[blk + 1] = np.nan                     # a NaN threshold is never cleared
    below[blk + 1] = False
    masked = np.ones(R, np.uint8)
    tokens = np.full(R, -1, np.int32)
    res = C.confidence_commit(logits, tokens, masked, blk, thr)
    assert np.allclose(res["conf"], target, rtol=0, atol=1e-12)
    for g in range(n_seq):
        sl = slice(g * blk, (g + 1) * blk)
        if below[sl].any():
            assert np.array_equal(res["committed"][sl], below[sl])
        else:
            assert np.flatnonzero(res["committed"][sl]).tolist() == [int(np.argmax(target[sl]))]
    assert np.array_equal(res["tokens"][res["committed"]], ids[res["committed"]])
    # a per-row array of one value decides as that single threshold
    for T in (0.3, 0.6):
        a = C.confidence_commit(logits, tokens, masked, blk, np.full(R, T))
        b = C.confidence_commit(logits, tokens, masked, blk, T)
        assert np.array_equal(a["committed"], b["committed"])
