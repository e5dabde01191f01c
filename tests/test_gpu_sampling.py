"""GPU parity of bd_confidence_commit_sampled against oracle.sampling.

Both sides draw the same uniform u per row (Philox4x32-10 of (row, step) under the seed) and take
the first id whose cumulative probability exceeds u.  The GPU sums the probabilities in fp32 (by
chunks, then within one chunk); the oracle in fp64 in id order.  So:
  * the sampled id equals the oracle's, except when u lies within 2e-5 of the cumulative boundary
    between the two ids (fp32 sums over up to 151936 terms, plus the fp32 rounding of u); such
    rows are counted and must be adjacent in that sense;
  * conf equals the oracle's probability of the GPU's id to 1e-5 relative;
  * the commit decision (threshold, fallback, state update) is then bit-exact against the oracle's
    rule applied to those (conf, id), outside the 1e-4 near-T band.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import commit as C
from oracle import sampling as S
from gpu_util import banner, dev, grade_sampled, host_vals

pytestmark = pytest.mark.gpu


def run_case(logits_np, dtype, tokens, masked, blk_len, T, tau, seed, step, fallback=True, stride=None):
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
                                          vocab=V)
    torch.cuda.synchronize()
    gpu = {"tokens": tok.cpu().numpy(), "masked": msk.cpu().numpy(),
           "conf": out["conf"].cpu().numpy().astype(np.float64), "pred": out["pred"].cpu().numpy(),
           "n_committed": out["n_committed"].cpu().numpy(), "n_masked_left": out["n_masked_left"].cpu().numpy()}
    x = host_vals(logits_np, dtype)[:, :V]
    ref = S.sampled_commit(x, tokens, masked, blk_len, T, tau, seed, step,
                           C.FALLBACK_TOP1 if fallback else C.FALLBACK_NONE)
    near, amb, boundary, n_com = grade_sampled(ref, gpu, x, masked, tokens, blk_len, T, tau, fallback)
    print(f"  tau={tau} T={T} seed={seed} step={step}: committed={n_com} "
          f"near-T={near} ambiguous={amb} boundary ids={boundary}")
    return gpu, ref


def test_tiny_f32_workload():
    wl = W.WORKLOADS["tiny_f32"]
    banner("sampled commit tiny_f32")
    c = W.commit_inputs(1, 32, wl.vocab, "f32", wl.seed, masked_frac=0.5, logit_std=wl.logit_std)
    for tau in (1.0, 0.7):
        for T in (wl.threshold, 0.3, 0.1):
            for step in (0, 1):
                run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, T, tau, seed=17, step=step)


def test_decode_step_workload():
    wl = W.WORKLOADS["decode_step_bf16"]
    banner("sampled commit decode_step_bf16")
    c = W.commit_inputs(1, 32, wl.vocab, "bf16", wl.seed, boost=wl.boost)
    for T in (0.95, 0.5):
        for seed, step in ((1, 0), (2, 5), (2**40 + 3, 2**33 + 1)):
            run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, T, 1.0, seed, step)


def test_longest_blocks():
    """Blocks of the longest length the commit takes (1024 rows)."""
    banner("sampled commit blk_len=1024")
    c = W.commit_inputs(2, 1024, 700, "bf16", seed=31, masked_frac=0.9, logit_std=3.0)
    for T in (0.5, 0.999):
        run_case(c["logits"], "bf16", c["tokens"], c["masked"], 1024, T, 1.0, seed=9, step=3)


@pytest.mark.parametrize("V,stride", [(5003, None), (5003, 5008), (4096, 4100), (77, None)])
def test_ragged_vocab_and_strides(V, stride):
    banner(f"sampled commit V={V} stride={stride}")
    c = W.commit_inputs(4, 32, V, "bf16", seed=V, masked_frac=0.75, boost=(0.0, 9.0))
    run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 0.4, 1.0, seed=3, step=9, stride=stride)
    c = W.commit_inputs(2, 32, V, "f32", seed=V + 1, masked_frac=0.75, logit_std=2.5)
    run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, 0.2, 0.8, seed=4, step=1, stride=stride)


def test_invalid_rows_and_neg_inf():
    banner("sampled commit invalid rows")
    rng = np.random.default_rng(9)
    V, blk = 3000, 8
    x = rng.standard_normal((2 * blk, V)).astype(np.float32)
    x[0, 17] = np.nan
    x[1, 2999] = np.inf
    x[2, :] = -np.inf
    x[3, :2500] = -np.inf
    x[4, ::2] = -np.inf
    x[5, 1:] = -np.inf
    masked = np.ones(2 * blk, np.uint8)
    tokens = np.full(2 * blk, -1, np.int32)
    for dt, arr in (("bf16", W.f32_to_bf16_bits(x)), ("f32", x)):
        gpu, _ = run_case(arr, dt, tokens, masked, blk, 0.5, 1.0, seed=5, step=0)
        assert gpu["pred"][5] == 0 and abs(gpu["conf"][5] - 1.0) < 1e-6
        assert gpu["pred"][4] % 2 == 1 and gpu["pred"][3] >= 2500


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batched_loop_scale(dtype):
    """64 x 32 rows of 151936 ids, bf16 and fp32 (the same values): the full-size step, with the
    target's chunk of 10240 ids rescanned as 5 vectors of 8 or 10 vectors of 4 per thread."""
    wl = W.WORKLOADS["decode_loop_bf16"]
    banner(f"sampled commit 64 x 32 x 151936 {dtype}")
    rng = np.random.default_rng(wl.seed)
    bits = W.boosted_logits_bits(64 * 32, wl.vocab, wl.boost[0], wl.boost[1], rng)
    masked = (rng.random(64 * 32) < 0.6).astype(np.uint8)
    tokens = np.where(masked == 1, -1, 5).astype(np.int32)
    logits = bits if dtype == "bf16" else W.bf16_bits_to_f32(bits)
    run_case(logits, dtype, tokens, masked, 32, 0.95, 1.0, seed=21, step=3)


def test_sample_frequencies_match_the_distribution():
    """2048 rows holding the same 40 logits draw 2048 independent samples (each row has its own
    counter): their frequencies follow softmax(logits / tau) (chi-square), at two temperatures."""
    banner("sampled commit frequencies")
    rng = np.random.default_rng(13)
    base = (rng.standard_normal(40) * 1.5).astype(np.float32)
    rows = 2048
    x = np.repeat(base[None], rows, axis=0)
    masked = np.ones(rows, np.uint8)
    tokens = np.full(rows, -1, np.int32)
    for tau in (1.0, 2.0):
        lg = torch.from_numpy(x).cuda()
        tok = torch.from_numpy(tokens.copy()).cuda()
        msk = torch.from_numpy(masked.copy()).cuda()
        out = bd.bd_confidence_commit_sampled(lg, tok, msk, 32, 2.0, temperature=tau, seed=99, step=7,
                                              fallback=bd.BD_FALLBACK_NONE)
        pred = out["pred"].cpu().numpy()
        p = np.exp((base.astype(np.float64) - base.max()) / tau)
        p /= p.sum()
        counts = np.bincount(pred, minlength=40)
        keep = rows * p >= 5
        chi2 = float(((counts[keep] - rows * p[keep]) ** 2 / (rows * p[keep])).sum()) + \
            float(((counts[~keep].sum() - rows * p[~keep].sum()) ** 2 / max(rows * p[~keep].sum(), 1e-9)))
        dof = int(keep.sum())
        print(f"  tau={tau}: chi2={chi2:.1f} over {dof} cells")
        assert chi2 < dof + 6 * np.sqrt(2 * dof)
        # nothing passes T = 2 and the fallback is off: the state is unchanged
        assert (msk.cpu().numpy() == 1).all()


def test_reproducible_and_fresh_per_step():
    banner("sampled commit reproducibility")
    c = W.commit_inputs(2, 32, 2000, "bf16", seed=8, masked_frac=1.0, logit_std=1.0)
    lg = dev(c["logits"], "bf16")

    def draw(step):
        tok = torch.from_numpy(c["tokens"].copy()).cuda()
        msk = torch.from_numpy(c["masked"].copy()).cuda()
        return bd.bd_confidence_commit_sampled(lg, tok, msk, 32, 2.0, seed=1234, step=step,
                                               fallback=bd.BD_FALLBACK_NONE)["pred"].cpu().numpy()
    a, b, d = draw(4), draw(4), draw(5)
    assert np.array_equal(a, b)
    assert (a != d).mean() > 0.5


def test_target_on_a_chunk_boundary():
    """A draw that lands on the boundary between two vocabulary chunks of the reduce.  1024 rows
    hold one logit row of 65536 ids (chunks of 4096 ids per row with the default chunking); the
    generator's steps are searched (oracle Philox4x32-10) for a row whose u lies within 5e-7 of
    the cumulative probability at a chunk boundary, where each id carries ~1.5e-5.  The sampled id
    must be one of the two ids at that boundary (rounding may pick either side, never an id far
    from it), and the whole step passes the usual sampling grade."""
    banner("sampled commit: target on a chunk boundary")
    rng = np.random.default_rng(31)
    V, chunk, n_seq, blk = 65536, 4096, 32, 32
    bits = W.f32_to_bf16_bits(rng.uniform(-1.0, 1.0, V).astype(np.float32))
    x = W.bf16_bits_to_f32(bits).astype(np.float64)
    p = np.exp(x - x.max())
    cum = np.cumsum(p / p.sum())
    bounds = cum[np.arange(1, V // chunk) * chunk - 1]     # probability of ids below each boundary
    seed, found = 91, None
    for step in range(4000):
        for r in range(n_seq * blk):
            u = S.row_uniform(seed, r, step)
            k = int(np.argmin(np.abs(bounds - u)))
            if abs(bounds[k] - u) < 5e-7:
                found = (step, r, (k + 1) * chunk)
                break
        if found:
            break
    assert found, "no draw near a boundary"
    step, r, b_id = found
    rows = np.repeat(bits[None], n_seq * blk, axis=0)
    masked = np.ones(n_seq * blk, np.uint8)
    tokens = np.full(n_seq * blk, -1, np.int32)
    gpu, ref = run_case(rows, "bf16", tokens, masked, blk, 2.0, 1.0, seed, step, fallback=False)
    print(f"  step {step} row {r}: boundary before id {b_id}, oracle id {ref['pred'][r]}, GPU id {gpu['pred'][r]}")
    assert gpu["pred"][r] in (b_id - 1, b_id), (gpu["pred"][r], b_id)
