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


# ---- top-k / top-p truncation -------------------------------------------------------------
def kept_ids(row, tau, k, p):
    row = np.asarray(row)
    return set(np.flatnonzero(np.isfinite(row) & (row >= S.truncation_cut(row, tau, k, p))).tolist())


def test_truncation_worked_example():
    """p = (0.5, 0.3, 0.2): the nucleus of mass p and top-k by hand, and top-p taken on the top-k
    distribution renormalised (0.625, 0.375)."""
    row = np.log(np.array([0.5, 0.3, 0.2]))
    assert kept_ids(row, 1.0, 0, 0.45) == {0}
    assert kept_ids(row, 1.0, 0, 0.55) == {0, 1}
    assert kept_ids(row, 1.0, 0, 0.85) == {0, 1, 2}          # 0.5 + 0.3 < 0.85
    assert kept_ids(row, 1.0, 2, 1.0) == {0, 1}
    assert kept_ids(row, 1.0, 2, 0.6) == {0}                 # 0.625 >= 0.6
    assert kept_ids(row, 1.0, 2, 0.7) == {0, 1}              # 0.625 < 0.7
    assert kept_ids(row, 1.0, 3, 1.0) == kept_ids(row, 1.0, 0, 1.0) == {0, 1, 2}
    # sampling over the kept pair: cumulative 0.625, 1.0
    c, s = S.row_sample(row, 1.0, 0.6, top_k=2)
    assert s == 0 and abs(c - 0.625) < 1e-15
    c, s = S.row_sample(row, 1.0, 0.7, top_k=2)
    assert s == 1 and abs(c - 0.375) < 1e-15
    c, s = S.row_sample(row, 1.0, 0.99, top_p=0.45)
    assert s == 0 and c == 1.0


def test_truncation_temperature_comes_first():
    """Logits (2, 1, 0): at tau = 1 the probabilities are (0.665, 0.245, 0.090), so top-p 0.7 keeps
    two ids; at tau = 0.5 they are (0.867, 0.117, 0.016) and it keeps one.  Top-k ignores tau."""
    row = np.array([2.0, 1.0, 0.0])
    assert kept_ids(row, 1.0, 0, 0.7) == {0, 1}
    assert kept_ids(row, 0.5, 0, 0.7) == {0}
    assert kept_ids(row, 0.5, 2, 1.0) == kept_ids(row, 3.0, 2, 1.0) == {0, 1}


def test_truncation_ties_are_kept_together():
    row = np.array([1.0, 1.0, 0.0, 1.0, -1.0])
    assert kept_ids(row, 1.0, 1, 1.0) == {0, 1, 3}
    assert kept_ids(row, 1.0, 3, 1.0) == {0, 1, 3}
    assert kept_ids(row, 1.0, 4, 1.0) == {0, 1, 2, 3}
    assert kept_ids(row, 1.0, 0, 0.1) == {0, 1, 3}           # one id of mass 0.3 each, kept as a group
    # -inf ids never count as kept candidates
    row = np.array([-np.inf, 2.0, -np.inf, 1.0])
    assert kept_ids(row, 1.0, 2, 1.0) == {1, 3} and S.truncation_cut(row, 1.0, 5, 1.0) == -np.inf


def test_truncation_characterised_by_brute_force():
    """On small rows with many tied values, the kept set is checked against what characterises
    it, by enumeration over the distinct values: it is closed upwards; top-k alone keeps at least
    k ids, and fewer than k without its lowest value; top-p keeps a mass of at least p times the
    top-k mass, and less without its lowest value."""
    rng = np.random.default_rng(3)
    for trial in range(400):
        n = int(rng.integers(1, 12))
        row = rng.integers(-3, 4, n).astype(np.float64) * rng.choice([0.5, 1.0, 1.7])
        row[rng.random(n) < 0.15] = -np.inf
        if not np.isfinite(row).any():
            continue
        tau = float(rng.choice([0.5, 1.0, 2.0]))
        k = int(rng.integers(0, n + 2))
        p = float(rng.choice([1.0, 0.999, 0.9, 0.5, 0.2, 1e-6]))
        fin = row[np.isfinite(row)]
        kept = kept_ids(row, tau, k, p)
        cut = S.truncation_cut(row, tau, k, p)
        assert kept == {i for i in range(n) if np.isfinite(row[i]) and row[i] >= cut}
        # top-k alone
        kk = {i for i in range(n) if np.isfinite(row[i]) and row[i] >= S.truncation_cut(row, tau, k, 1.0)}
        if 1 <= k < len(fin):
            low = min(row[i] for i in kk)
            assert len(kk) >= k and len([i for i in kk if row[i] > low]) < k
        else:
            assert len(kk) == len(fin)
        # top-p on the top-k ids
        m = fin.max()
        w = {i: math.exp((row[i] - m) / tau) for i in kk}
        zk = sum(w.values())
        assert kept <= kk
        mass = sum(w[i] for i in kept)
        low = min(row[i] for i in kept)
        above = sum(w[i] for i in kept if row[i] > low)
        if p < 1.0:
            assert mass >= p * zk * (1 - 1e-12) and above < p * zk
        else:
            assert kept == kk


def test_truncated_sampling_frequencies():
    """Draws from the generator under top-k 3 and under top-p 0.8 land only on the kept ids, with
    the renormalised frequencies (chi-square)."""
    rng = np.random.default_rng(5)
    row = rng.standard_normal(10) * 1.2
    order = np.argsort(-row)
    for k, p in ((3, 1.0), (0, 0.8)):
        kept = sorted(kept_ids(row, 1.0, k, p))
        if k:
            assert kept == sorted(order[:3].tolist())
        w = np.exp(row[kept] - row.max())
        q = w / w.sum()
        N = 4000
        counts = np.zeros(len(row), int)
        for step in range(N):
            c, s = S.row_sample(row, 1.0, S.row_uniform(11, 0, step), k, p)
            counts[s] += 1
            assert abs(c - q[kept.index(s)]) < 1e-12
        assert counts[[i for i in range(len(row)) if i not in kept]].sum() == 0
        chi2 = float(((counts[kept] - N * q) ** 2 / (N * q)).sum())
        assert chi2 < 8 + 6 * math.sqrt(2 * len(kept))


def test_no_op_truncations_equal_plain_sampling():
    rng = np.random.default_rng(8)
    row = rng.standard_normal(30)
    row[4] = -np.inf
    for u in (0.013, 0.5, 0.97):
        ref = S.row_sample(row, 1.3, u)
        for k, p in ((0, 1.0), (29, 1.0), (40, 1.0)):
            assert S.row_sample(row, 1.3, u, k, p) == ref
