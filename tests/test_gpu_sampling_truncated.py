"""GPU parity of bd_confidence_commit_sampled with top-k / top-p truncation against oracle.sampling.

The cut (the smallest kept logit value) is exact for top-k (a count) and decided by fp32 masses
for top-p, against the oracle's fp64; so, per masked row:
  * the GPU's kept set is read back from its confidence (conf = weight / kept mass): it must be
    the oracle's, or -- only with top-p on -- the next distinct value up or down where the
    oracle's running mass at that value lies within 1e-5 (relative) of top_p times the top-k
    mass (boundary cuts, counted);
  * within that kept set the sampled id must be the oracle's inverse-CDF id for the same u,
    except where u lies within 2e-5 of a cumulative boundary (fp32 sums), and conf must equal the
    oracle's probability of the id to 1e-5 relative;
  * the commit decision is bit-exact against the oracle's rule on those (conf, id), outside the
    1e-4 near-T band.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import commit as C
from oracle import sampling as S
from gpu_util import banner, dev, grade_commit, host_vals

pytestmark = pytest.mark.gpu


def run_case(logits_np, dtype, tokens, masked, blk_len, T, tau, seed, step, top_k, top_p, fallback=True,
             stride=None, rows_checked=None):
    V = logits_np.shape[1]
    lg = dev(logits_np, dtype)
    if stride is not None:
        pad = torch.zeros((lg.shape[0], stride), dtype=lg.dtype, device=lg.device)
        pad[:, :V] = lg
        lg = pad
    tok = torch.from_numpy(tokens.copy()).cuda()
    msk = torch.from_numpy(masked.copy()).cuda()
    out = bd.bd_confidence_commit_sampled(lg, tok, msk, blk_len, T, temperature=tau, seed=seed, step=step,
                                          fallback=bd.BD_FALLBACK_TOP1 if fallback else bd.BD_FALLBACK_NONE,
                                          vocab=V, top_k=top_k, top_p=top_p)
    torch.cuda.synchronize()
    gpu = {"tokens": tok.cpu().numpy(), "masked": msk.cpu().numpy(),
           "conf": out["conf"].cpu().numpy().astype(np.float64), "pred": out["pred"].cpu().numpy(),
           "n_committed": out["n_committed"].cpu().numpy(), "n_masked_left": out["n_masked_left"].cpu().numpy()}
    x = host_vals(logits_np, dtype)[:, :V]
    conf_o = np.full(len(tokens), np.nan)
    boundary_cut = boundary_id = 0
    rows = np.flatnonzero(masked) if rows_checked is None else rows_checked
    for r in rows:
        row = np.asarray(x[r], dtype=np.float64)
        ref_c, ref_p = S.row_sample(row, tau, S.row_uniform(seed, r, step), top_k, top_p)
        g = int(gpu["pred"][r])
        assert (g < 0) == (ref_p < 0), f"row {r}: invalid flags differ"
        if g < 0:
            continue
        fin = np.isfinite(row)
        w = np.where(fin, np.exp((row - row[fin].max()) / tau), 0.0)
        vals = np.unique(row[fin])[::-1]
        cut_o = S.truncation_cut(row, tau, top_k, top_p)
        io = 0 if cut_o == -np.inf else int(np.flatnonzero(vals == cut_o)[0])
        if cut_o == -np.inf:
            io = len(vals) - 1
        mass = lambda c: float(w[fin & (row >= c)].sum())
        cg = gpu["conf"][r]
        match = None
        for d in (0, 1, -1):
            i = io + d
            if 0 <= i < len(vals) and row[g] >= vals[i]:
                z = mass(vals[i])
                if abs(cg - w[g] / z) <= 1e-5 * w[g] / z + 1e-9:
                    match = i
                    break
        assert match is not None, f"row {r}: conf {cg} fits no kept set near the oracle's cut"
        if match != io:
            assert top_p < 1.0, f"row {r}: top-k cut differs"
            zk = mass(S.truncation_cut(row, tau, top_k, 1.0)) if top_k else mass(-np.inf)
            edge = vals[min(io, match)]          # the value whose inclusion the two cuts disagree on
            assert abs(mass(edge) - top_p * zk) <= 1e-5 * zk, f"row {r}: cut {match} vs {io} not at the boundary"
            boundary_cut += 1
        kept = fin & (row >= vals[match])
        z = w[kept].sum()
        p = np.where(kept, w / z, 0.0)
        u = S.row_uniform(seed, r, step)
        cum = np.cumsum(p)
        o = int(np.flatnonzero(cum > u)[0]) if (cum > u).any() else int(np.flatnonzero(p > 0)[-1])
        if g != o:
            lo, hi = (cum[g - 1] if g > 0 else 0.0), cum[g]
            assert p[g] > 0 and lo - 2e-5 <= u <= hi + 2e-5, f"row {r}: id {g} vs {o}, u={u} outside [{lo}, {hi}]"
            boundary_id += 1
        elif match == io:
            assert g == ref_p
        conf_o[r] = p[g]
    n = len(rows)
    assert boundary_cut <= max(2, int(0.02 * n)), f"{boundary_cut} boundary cuts"
    assert boundary_id <= max(2, int(0.05 * n)), f"{boundary_id} boundary ids"
    if rows_checked is None:
        rule = C.decide(conf_o, np.where(gpu["pred"] >= 0, gpu["pred"], -1).astype(np.int32), tokens, masked,
                        blk_len, T, C.FALLBACK_TOP1 if fallback else C.FALLBACK_NONE)
        near, amb = grade_commit(rule, gpu, masked, tokens, blk_len, T, fallback)
    else:
        near = amb = -1
    print(f"  k={top_k} p={top_p} tau={tau} T={T}: rows={n} boundary cuts={boundary_cut} "
          f"boundary ids={boundary_id} near-T={near} ambiguous={amb}")
    return gpu


# (top_k, top_p); the last keeps every id (top-k beyond the vocabulary) through the truncating kernel
KP = [(1, 1.0), (5, 1.0), (50, 1.0), (0, 0.1), (0, 0.5), (0, 0.9), (50, 0.9), (1000, 0.95), (10**6, 1.0)]


@pytest.mark.parametrize("k,p", KP)
def test_tiny_f32(k, p):
    wl = W.WORKLOADS["tiny_f32"]
    banner(f"truncated sampling tiny_f32 k={k} p={p}")
    c = W.commit_inputs(1, 32, wl.vocab, "f32", wl.seed, masked_frac=0.75, logit_std=wl.logit_std)
    for tau in (1.0, 0.7):
        run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, 0.3, tau, seed=17, step=2, top_k=k, top_p=p)


@pytest.mark.parametrize("k,p", KP)
def test_decode_step_bf16(k, p):
    wl = W.WORKLOADS["decode_step_bf16"]
    banner(f"truncated sampling decode_step_bf16 k={k} p={p}")
    c = W.commit_inputs(1, 32, wl.vocab, "bf16", wl.seed, boost=wl.boost)
    gpu = run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 0.5, 1.0, seed=3, step=1, top_k=k, top_p=p)
    if k == 1:   # top-1: the argmax, with certainty (the boosted id is the unique maximum)
        x = host_vals(c["logits"], "bf16")
        assert np.array_equal(gpu["pred"], np.argmax(x, axis=1)) and np.allclose(gpu["conf"], 1.0)


def test_second_window_cuts():
    """bf16 rows whose cut lies more than 32768 order keys below the maximum (one logit at +30, the
    rest N(0,1), a high temperature): the histogram's second window places the cut."""
    banner("truncated sampling, cuts in the second key window")
    rng = np.random.default_rng(21)
    V = 5003
    x = rng.standard_normal((32, V)).astype(np.float32)
    x[np.arange(32), rng.integers(0, V, 32)] = 30.0
    bits = W.f32_to_bf16_bits(x)
    masked = np.ones(32, np.uint8)
    tokens = np.full(32, -1, np.int32)
    for k, p, tau in ((4000, 1.0, 20.0), (0, 0.97, 20.0), (4500, 0.9, 50.0), (0, 0.5, 50.0)):
        run_case(bits, "bf16", tokens, masked, 32, 0.9, tau, seed=5, step=k, top_k=k, top_p=p)


def test_ties_and_small_rows():
    """Logits with many exact ties (small integers), vocabularies smaller than one vector per
    thread and not a multiple of eight, and unaligned row strides (element loads)."""
    banner("truncated sampling ties / ragged")
    rng = np.random.default_rng(4)
    for V, stride in ((7, None), (77, None), (1000, 1003), (4099, None)):
        x = rng.integers(-4, 5, (64, V)).astype(np.float32) * 0.75
        masked = (rng.random(64) < 0.8).astype(np.uint8)
        tokens = np.where(masked == 1, -1, 2).astype(np.int32)
        for dt, arr in (("bf16", W.f32_to_bf16_bits(x)), ("f32", x)):
            for k, p in ((3, 1.0), (0, 0.6), (10, 0.8)):
                run_case(arr, dt, tokens, masked, 32, 0.4, 1.0, seed=V, step=k, top_k=k, top_p=p, stride=stride)


def test_invalid_rows_and_neg_inf():
    banner("truncated sampling invalid rows")
    rng = np.random.default_rng(9)
    V, blk = 3000, 8
    x = rng.standard_normal((2 * blk, V)).astype(np.float32)
    x[0, 17] = np.nan
    x[1, 2999] = np.inf
    x[2, :] = -np.inf
    x[3, :2500] = -np.inf
    x[4, ::2] = -np.inf
    x[5, 1:] = -np.inf
    x[6, :] = 0.0
    x[6, 5] = -0.0
    masked = np.ones(2 * blk, np.uint8)
    tokens = np.full(2 * blk, -1, np.int32)
    for dt, arr in (("bf16", W.f32_to_bf16_bits(x)), ("f32", x)):
        for k, p in ((2, 1.0), (0, 0.3), (4, 0.5)):
            gpu = run_case(arr, dt, tokens, masked, blk, 0.5, 1.0, seed=5, step=0, top_k=k, top_p=p)
            assert gpu["pred"][5] == 0 and abs(gpu["conf"][5] - 1.0) < 1e-6
            assert gpu["pred"][4] % 2 == 1 and gpu["pred"][3] >= 2500


def test_fp32_full_vocabulary():
    """fp32 logits at the largest vocabulary the register-held row allows (77824): the bisection
    path at scale."""
    banner("truncated sampling fp32 V=77824")
    c = W.commit_inputs(1, 32, 77824, "f32", seed=31, masked_frac=0.25, logit_std=1.5)
    run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, 0.5, 1.0, seed=8, step=4, top_k=200, top_p=0.9)
    run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, 0.5, 1.3, seed=8, step=5, top_k=0, top_p=0.95)


def test_bf16_full_vocabulary():
    """bf16 logits at the largest vocabulary the register-held row allows (155648 ids)."""
    banner("truncated sampling bf16 V=155648")
    c = W.commit_inputs(1, 32, 155648, "bf16", seed=33, masked_frac=0.25, logit_std=1.5)
    run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 0.5, 1.0, seed=8, step=6, top_k=200, top_p=0.9)
    run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 0.5, 0.8, seed=8, step=7, top_k=0, top_p=0.95)


def test_batched_loop_scale():
    """The 64-sequence decode step (2048 rows of 151936 bf16 logits, 60 % masked) with top-p 0.9;
    a sample of rows is checked against the oracle."""
    wl = W.WORKLOADS["decode_loop_bf16"]
    banner("truncated sampling 64 x 32 x 151936")
    rng = np.random.default_rng(wl.seed)
    bits = W.boosted_logits_bits(64 * 32, wl.vocab, wl.boost[0], wl.boost[1], rng)
    masked = (rng.random(64 * 32) < 0.6).astype(np.uint8)
    tokens = np.where(masked == 1, -1, 5).astype(np.int32)
    rows = np.flatnonzero(masked)[::24]
    run_case(bits, "bf16", tokens, masked, 32, 0.95, 1.0, seed=21, step=3, top_k=0, top_p=0.9, rows_checked=rows)
    run_case(bits, "bf16", tokens, masked, 32, 0.95, 1.0, seed=21, step=4, top_k=64, top_p=0.95, rows_checked=rows)


def test_sample_frequencies_match_the_truncated_distribution():
    """2048 rows holding the same 40 logits: the draws under top-k 5 and under top-p 0.6 land only
    on the kept ids, with the renormalised frequencies (chi-square)."""
    banner("truncated sampling frequencies")
    rng = np.random.default_rng(13)
    base = (rng.standard_normal(40) * 1.5).astype(np.float32)
    rows = 2048
    x = np.repeat(base[None], rows, axis=0)
    masked = np.ones(rows, np.uint8)
    tokens = np.full(rows, -1, np.int32)
    for k, p in ((5, 1.0), (0, 0.6)):
        lg = torch.from_numpy(x).cuda()
        out = bd.bd_confidence_commit_sampled(lg, torch.from_numpy(tokens.copy()).cuda(),
                                              torch.from_numpy(masked.copy()).cuda(), 32, 2.0, seed=99, step=7,
                                              fallback=bd.BD_FALLBACK_NONE, top_k=k, top_p=p)
        pred = out["pred"].cpu().numpy()
        row = base.astype(np.float64)
        kept = np.flatnonzero(row >= S.truncation_cut(row, 1.0, k, p))
        w = np.exp(row[kept] - row.max())
        q = w / w.sum()
        counts = np.bincount(pred, minlength=40)
        assert counts[np.setdiff1d(np.arange(40), kept)].sum() == 0
        keep = rows * q >= 5
        chi2 = float(((counts[kept][keep] - rows * q[keep]) ** 2 / (rows * q[keep])).sum())
        dof = int(keep.sum())
        print(f"  k={k} p={p}: {len(kept)} kept ids, chi2={chi2:.1f} over {dof} cells")
        assert chi2 < dof + 6 * np.sqrt(2 * dof)


def test_reproducible():
    banner("truncated sampling reproducibility")
    c = W.commit_inputs(2, 32, 20000, "bf16", seed=8, masked_frac=1.0, logit_std=1.0)
    lg = dev(c["logits"], "bf16")

    def draw(step):
        return bd.bd_confidence_commit_sampled(lg, torch.from_numpy(c["tokens"].copy()).cuda(),
                                               torch.from_numpy(c["masked"].copy()).cuda(), 32, 2.0, seed=1234,
                                               step=step, fallback=bd.BD_FALLBACK_NONE, top_k=100,
                                               top_p=0.9)["pred"].cpu().numpy()
    a, b, d = draw(4), draw(4), draw(5)
    assert np.array_equal(a, b)
    assert (a != d).mean() > 0.5
