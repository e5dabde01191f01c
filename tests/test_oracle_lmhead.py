"""Pins of oracle.lmhead (CPU only): brute force, closed forms and the boost construction."""
import math

import numpy as np

import workloads as W
from oracle import commit as C
from oracle import lmhead as LH


def test_brute_force_small():
    rng = np.random.default_rng(0)
    x, w = rng.standard_normal((3, 8)), rng.standard_normal((11, 8))
    ref = LH.lmhead_logits(x, w)
    for r in range(3):
        for v in range(11):
            s = 0.0
            for k in range(8):
                s += x[r, k] * w[v, k]
            assert abs(ref[r, v] - s) < 1e-12


def test_one_hot_hidden_selects_a_weight_column():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((50, 6))
    x = np.zeros((6, 6))
    for j in range(6):
        x[j, j] = 2.5
    lg = LH.lmhead_logits(x, w)
    assert np.array_equal(lg, 2.5 * w.T)


def test_single_aligned_row_closed_form():
    """All weight rows zero except W[t] = a x / |x|^2: logits are a at t and 0 elsewhere, so
    conf = 1 / (1 + (V - 1) e^-a), pred = t."""
    V, H = 400, 16
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, H))
    for a, t in ((3.0, 17), (9.0, 399), (-1.0, 5)):
        w = np.zeros((V, H))
        w[t] = a * x[0] / (x[0] @ x[0])
        res = LH.lmhead_commit(x, w, np.array([-1], np.int32), np.array([1], np.uint8), 1, 0.5)
        if a > 0:
            assert res["pred"][0] == t
            assert abs(res["conf"][0] - 1.0 / (1.0 + (V - 1) * math.exp(-a))) < 1e-12
        else:   # the maximum 0 is shared by every other id: the lowest id wins
            assert res["pred"][0] == (0 if t != 0 else 1)
            assert abs(res["conf"][0] - 1.0 / ((V - 1) + math.exp(a))) < 1e-12


def test_boost_construction_raises_its_logit():
    """The input recipe adds b_r X_r / |X_r|^2 to W[t_r], which raises logit (r, t_r) by b_r (up
    to the bf16 rounding of W): with b_r ~ U(8, 9) over N(0,1) logits it is the row maximum."""
    d = W.lmhead_inputs(1, 8, 64, 500, seed=3, boost=(8.0, 9.0))
    x = W.bf16_bits_to_f32(d["hidden"]).astype(np.float64)
    w = W.bf16_bits_to_f32(d["weight"]).astype(np.float64)
    lg = LH.lmhead_logits(x, w)
    ids = d["boost_ids"]
    top = lg[np.arange(8), ids]
    assert np.all(top > 4.0)
    assert np.all(np.argmax(lg, axis=1) == ids)


def test_commit_rules_carry_over():
    """The fused commit is the plain commit on the product: same sets, ids and counts."""
    d = W.lmhead_inputs(2, 16, 32, 300, seed=4, masked_frac=0.75)
    x = W.bf16_bits_to_f32(d["hidden"])
    w = W.bf16_bits_to_f32(d["weight"])
    for T in (0.3, 0.9):
        a = LH.lmhead_commit(x, w, d["tokens"], d["masked"], 16, T)
        b = C.confidence_commit(x.astype(np.float64) @ w.astype(np.float64).T, d["tokens"], d["masked"], 16, T)
        for key in ("committed", "pred", "n_committed", "n_masked_left"):
            assert np.array_equal(a[key], b[key])
