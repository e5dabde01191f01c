"""Pins of oracle.sampling (CPU only): the generator's published known-answer vectors, exact
inverse-CDF frequencies, a chi-square test of the sampled ids, closed forms and the commit rule."""
import math
import os

import numpy as np

from oracle import commit as C
from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        ctr, key, out = (tuple(int(w, 16) for w in part.split()) for part in line.split(";"))
        assert S.philox4x32_10(ctr, key) == out
        n += 1
    assert n == 3


def test_uniform_range_and_spread():
    u = np.array([S.row_uniform(123, r, s) for r in range(64) for s in range(64)])
    assert np.all((u > 0) & (u < 1))
    assert abs(u.mean() - 0.5) < 0.02 and abs(u.var() - 1 / 12) < 0.01
    # distinct counters give distinct draws; the seed matters
    assert len(np.unique(u)) == len(u)
    assert S.row_uniform(1, 0, 0) != S.row_uniform(2, 0, 0)


def test_inverse_cdf_exact_frequencies():
    """With u on an even grid the sampler returns each id exactly in proportion to p."""
    logits = np.log(np.array([1.0, 2.0, 3.0, 4.0]))          # p = 0.1, 0.2, 0.3, 0.4
    counts = np.zeros(4, int)
    N = 1000
    for i in range(N):
        _, s = S.row_sample(logits, 1.0, (i + 0.5) / N)
        counts[s] += 1
    assert counts.tolist() == [100, 200, 300, 400]


def test_chi_square_of_generated_samples():
    rng = np.random.default_rng(0)
    logits = rng.standard_normal(12) * 1.5
    p = np.exp(logits - logits.max())
    p /= p.sum()
    N = 6000
    counts = np.zeros(12, int)
    for step in range(N):
        _, s = S.row_sample(logits, 1.0, S.row_uniform(7, 3, step))
        counts[s] += 1
    chi2 = float(((counts - N * p) ** 2 / (N * p)).sum())
    assert chi2 < 35.0          # 11 degrees of freedom: p-value far below 1e-3 above this


def test_temperature_closed_forms():
    """One value a and V-1 zeros at temperature tau: p_peak = 1 / (1 + (V-1) e^(-a/tau)).
    u below p_peak with the peak first samples the peak with that confidence."""
    V = 50
    row = np.zeros(V)
    row[0] = 3.0
    for tau in (0.5, 1.0, 2.0):
        c, s = S.row_sample(row, tau, 0.01)
        assert s == 0 and abs(c - 1.0 / (1.0 + (V - 1) * math.exp(-3.0 / tau))) < 1e-14
    # a high temperature flattens towards uniform; a low one concentrates on the argmax
    c, _ = S.row_sample(row, 1e4, 0.5)
    assert abs(c - 1.0 / V) < 1e-4
    c, s = S.row_sample(row, 1e-3, 0.999)
    assert s == 0 and c > 1 - 1e-12


def test_invalid_rows_and_neg_inf():
    assert S.row_sample(np.array([0.0, np.nan]), 1.0, 0.5)[1] == -1
    assert S.row_sample(np.array([-np.inf, -np.inf]), 1.0, 0.5)[1] == -1
    # -inf entries are never sampled
    row = np.array([-np.inf, 0.0, -np.inf, 0.0, -np.inf])
    for u in (0.01, 0.49, 0.51, 0.99):
        c, s = S.row_sample(row, 1.0, u)
        assert s in (1, 3) and abs(c - 0.5) < 1e-15


def test_commit_rule_carries_over():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((3 * 8, 40)) * 2
    logits[np.arange(24), rng.integers(0, 40, 24)] += 6
    masked = (rng.random(24) < 0.8).astype(np.uint8)
    tokens = np.where(masked == 1, -1, 5).astype(np.int32)
    res = S.sampled_commit(logits, tokens, masked, 8, 0.6, 1.0, seed=11, step=4)
    again = C.decide(res["conf"], res["pred"], tokens, masked, 8, 0.6)
    for key in ("committed", "tokens", "masked", "n_committed", "n_masked_left"):
        assert np.array_equal(res[key], again[key])
    m = masked == 1
    assert np.all(res["tokens"][res["committed"]] == res["pred"][res["committed"]])
    assert np.all(np.isnan(res["u"][~m])) and np.all((res["u"][m] > 0) & (res["u"][m] < 1))
