"""Helpers shared by the GPU parity tests: host <-> device moves and the commit grader."""
from __future__ import annotations

import os

import numpy as np
import torch

import workloads as W


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit array (uint16) -> device bfloat16 tensor with the same values."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return dev_bf16(x) if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_vals(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values an input array stands for, in float64 (what the oracle reads)."""
    return W.bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy()


# One record per graded commit step: (test id, masked rows graded, near-T rows, ambiguous groups).
# The terminal summary of the test session (conftest.py) prints the totals.
NEAR_T_LOG: list = []


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def grade_commit(ref: dict, gpu: dict, masked_in: np.ndarray, tokens_in: np.ndarray, blk_len: int, T: float,
                 fallback_top1: bool = True, band: float = 1e-4, conf_rtol: float = 1e-5, flagged=None):
    """Compare one GPU commit step with the oracle's.

    Ids and masks must match bit for bit, except in groups where the oracle's confidence
    of some row lies within ``band`` of T (near-T rows), or where the fallback choice is
    decided by confidences within a relative ``band`` of each other; such groups are counted
    and only their validity is checked.  Returns (n_near_rows, n_ambiguous_groups); the
    indices of those groups are added to the set ``flagged`` when one is given.
    """
    m_in = masked_in.astype(bool)
    assert np.array_equal(gpu["pred"][m_in], ref["pred"][m_in]), "argmax ids differ"
    cr, cg = ref["conf"][m_in], gpu["conf"][m_in]
    assert np.array_equal(np.isnan(cr), np.isnan(cg)), "invalid-row flags differ"
    ok = ~np.isnan(cr)
    if ok.any():
        err = np.abs(cg[ok] - cr[ok])
        assert np.all(err <= conf_rtol * cr[ok] + 1e-7), f"conf max rel err {np.max(err / cr[ok])}"
    assert np.array_equal(gpu["tokens"][~m_in], tokens_in[~m_in]), "unmasked rows touched"
    assert np.array_equal(gpu["masked"][~m_in], masked_in[~m_in]), "unmasked rows touched"
    committed = m_in & (gpu["masked"] == 0)
    assert np.array_equal(gpu["tokens"][committed], gpu["pred"][committed])
    assert np.array_equal(gpu["tokens"][m_in & ~committed], tokens_in[m_in & ~committed])
    near_rows, ambiguous = 0, 0
    thr = np.broadcast_to(np.asarray(T, dtype=np.float64), masked_in.shape)   # one T, or one per row
    for g in range(len(masked_in) // blk_len):
        sl = slice(g * blk_len, (g + 1) * blk_len)
        mg, c, com_g, com_r = m_in[sl], ref["conf"][sl], committed[sl], ref["committed"][sl]
        T = thr[sl]
        valid = mg & ~np.isnan(c)
        near = valid & (np.abs(c - T) <= band)
        near_rows += int(near.sum())
        assert gpu["n_committed"][g] == com_g.sum()
        assert gpu["n_masked_left"][g] == mg.sum() - com_g.sum()
        if near.any():
            ambiguous += 1
            if flagged is not None:
                flagged.add(g)
            assert np.all(com_g[valid & (c > T + band)]), f"group {g}: a row far above T was not committed"
            if com_g.sum() > 1:
                assert not np.any(com_g & valid & (c < T - band)), f"group {g}: a row far below T was committed"
            continue
        if (valid & (c > T)).any() or not fallback_top1 or not valid.any():
            assert np.array_equal(com_g, com_r), f"group {g}: committed set differs"
            continue
        cv = np.where(valid, c, -np.inf)
        top = np.sort(cv)[::-1]
        # the GPU's confidences carry a relative error of at most conf_rtol, so the fallback's
        # choice is fixed unless the top two lie within a relative `band` (ten times that) apart
        if len(top) > 1 and top[0] - top[1] <= band * top[0]:
            ambiguous += 1
            if flagged is not None:
                flagged.add(g)
            assert com_g.sum() == 1 and cv[np.flatnonzero(com_g)[0]] >= top[0] * (1 - band)
        else:
            assert np.array_equal(com_g, com_r), f"group {g}: fallback row differs"
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    NEAR_T_LOG.append((test, int(m_in.sum()), near_rows, ambiguous))
    return near_rows, ambiguous


def grade_sampled(ref: dict, gpu: dict, x: np.ndarray, masked_in: np.ndarray, tokens_in: np.ndarray, blk_len: int,
                  T: float, tau: float, fallback_top1: bool = True, flagged=None):
    """Compare one GPU sampled-commit step with the oracle's (oracle.sampling.sampled_commit on
    the same input state, ``x`` the logits as float64 values).

    Both sides draw the same u per row and take the first id whose cumulative probability exceeds
    it; the GPU sums in fp32, the oracle in fp64.  The GPU's id equals the oracle's except where u
    lies within 2e-5 of the cumulative boundary of the two ids ("boundary" rows, each checked to
    straddle it); conf must equal the oracle's probability of the GPU's id to 1e-5 relative; the
    decision is then graded as the greedy commit's, against the oracle's rule applied to the
    GPU's (conf, id).  Groups holding a boundary row are added to ``flagged`` with those of
    grade_commit.  Returns (near-T rows, ambiguous groups, boundary rows, rows committed)."""
    from oracle import commit as C
    conf_o = np.full(len(tokens_in), np.nan)
    boundary = 0
    for r in np.flatnonzero(masked_in):
        g, o = int(gpu["pred"][r]), int(ref["pred"][r])
        assert (g < 0) == (o < 0), f"row {r}: invalid flags differ"
        if g < 0:
            continue
        row = np.asarray(x[r], dtype=np.float64)
        p = np.exp((row - row.max()) / tau)
        p /= p.sum()
        if g != o:
            cum = np.cumsum(p)
            lo, hi = (cum[g - 1] if g > 0 else 0.0), cum[g]
            u = ref["u"][r]
            assert p[g] > 0 and lo - 2e-5 <= u <= hi + 2e-5, f"row {r}: id {g} vs {o}, u={u} outside [{lo}, {hi}]"
            boundary += 1
            if flagged is not None:
                flagged.add(int(r) // blk_len)
        conf_o[r] = p[g]
        assert abs(gpu["conf"][r] - p[g]) <= 1e-5 * p[g] + 1e-9, f"row {r}: conf {gpu['conf'][r]} vs {p[g]}"
    # tail ids have probabilities ~1e-6 apart, comparable to the fp32 sums: some boundary rows are
    # expected; each one was checked above, a wholesale mismatch would not pass this
    assert boundary <= max(2, int(0.05 * masked_in.sum())), f"{boundary} boundary rows"
    rule = C.decide(conf_o, np.where(gpu["pred"] >= 0, gpu["pred"], -1).astype(np.int32), tokens_in, masked_in,
                    blk_len, T, C.FALLBACK_TOP1 if fallback_top1 else C.FALLBACK_NONE)
    near, amb = grade_commit(rule, gpu, masked_in, tokens_in, blk_len, T, fallback_top1, flagged=flagged)
    return near, amb, boundary, int(rule["committed"].sum())
