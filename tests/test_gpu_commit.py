"""GPU parity of bd_confidence_commit against the oracle (ids and masks bit-exact outside the
near-T band; confidences to 1e-5 relative)."""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import commit as OC
from gpu_util import banner, dev, grade_commit, host_vals

pytestmark = pytest.mark.gpu


def run_case(logits_np, dtype, tokens, masked, blk_len, T, fallback=True, stride=None, vocab=None):
    """Run GPU and oracle on the same input; returns (near rows, ambiguous groups, oracle result)."""
    V = logits_np.shape[1] if vocab is None else vocab
    lg = dev(logits_np, dtype)
    if stride is not None:
        pad = torch.zeros((lg.shape[0], stride), dtype=lg.dtype, device=lg.device)
        pad[:, :lg.shape[1]] = lg
        lg = pad
    tok = torch.from_numpy(tokens.copy()).cuda()
    msk = torch.from_numpy(masked.copy()).cuda()
    thr = torch.from_numpy(np.asarray(T, np.float32)).cuda() if np.ndim(T) else T
    out = bd.bd_confidence_commit(lg, tok, msk, blk_len, thr, bd.BD_FALLBACK_TOP1 if fallback else bd.BD_FALLBACK_NONE,
                                  vocab=V)
    torch.cuda.synchronize()
    gpu = {"tokens": tok.cpu().numpy(), "masked": msk.cpu().numpy(), "conf": out["conf"].cpu().numpy().astype(np.float64),
           "pred": out["pred"].cpu().numpy(), "n_committed": out["n_committed"].cpu().numpy(),
           "n_masked_left": out["n_masked_left"].cpu().numpy()}
    ref = OC.confidence_commit(host_vals(logits_np, dtype)[:, :V], tokens, masked, blk_len, T,
                               OC.FALLBACK_TOP1 if fallback else OC.FALLBACK_NONE)
    near, amb = grade_commit(ref, gpu, masked, tokens, blk_len, T, fallback)
    return near, amb, ref


def test_tiny_f32_workload():
    wl = W.WORKLOADS["tiny_f32"]
    banner("commit tiny_f32")
    c = W.commit_inputs(1, 32, wl.vocab, "f32", wl.seed, masked_frac=0.5, logit_std=wl.logit_std)
    confs = [OC.row_confidence(c["logits"][r])[0] for r in np.flatnonzero(c["masked"])]
    for T in (wl.threshold, 0.1, float(np.median(confs)), 0.5):
        near, amb, ref = run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, T)
        print(f"  T={T:.4f} committed={int(ref['committed'].sum())} near={near} ambiguous={amb}")


def test_decode_step_workload():
    wl = W.WORKLOADS["decode_step_bf16"]
    banner("commit decode_step_bf16")
    rng = np.random.default_rng(wl.seed)
    W.decode_inputs(1, [wl.prefix_len], 32, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.seed, rng=rng)
    c = W.commit_inputs(1, 32, wl.vocab, "bf16", wl.seed, boost=wl.boost, rng=rng)
    for T in (0.95, 0.5, 0.9):
        near, amb, ref = run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, T)
        print(f"  T={T} committed={int(ref['committed'].sum())} near={near} ambiguous={amb}")


@pytest.mark.parametrize("V,stride", [(5003, None), (5003, 5008), (4096, 4100), (77, None), (8192 * 3 + 1, None)])
def test_ragged_vocab_and_strides(V, stride):
    banner(f"commit ragged V={V} stride={stride}")
    c = W.commit_inputs(6, 32, V, "bf16", seed=V, masked_frac=0.75, boost=(0.0, 9.0))
    for T in (0.3, 0.8):
        run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, T, stride=stride)
    c = W.commit_inputs(3, 32, V, "f32", seed=V + 1, masked_frac=0.75, logit_std=2.5)
    run_case(c["logits"], "f32", c["tokens"], c["masked"], 32, 0.2, stride=stride)


def test_invalid_rows_and_ties():
    banner("commit invalid rows and ties")
    rng = np.random.default_rng(5)
    V, blk = 3000, 8
    x = rng.standard_normal((4 * blk, V)).astype(np.float32)
    x[0, 17] = np.nan
    x[1, 2999] = np.inf
    x[2, :] = -np.inf
    x[3, ::2] = -np.inf
    x[4, [5, 900, 2000]] = 6.0          # tie at the maximum: lowest id wins
    x[9, 100] = x[9, 7] = 30.0          # confident row with a tie
    x[16:24] = 0.0                       # identical rows: fallback takes the lowest row
    x[16:24, 3] = 1.0
    bits = W.f32_to_bf16_bits(x)
    masked = np.ones(4 * blk, np.uint8)
    tokens = np.full(4 * blk, -1, np.int32)
    for dt, arr in (("bf16", bits), ("f32", x)):
        for T in (0.45, 0.99, 1.5):
            run_case(arr, dt, tokens, masked, blk, T)
        run_case(arr, dt, tokens, masked, blk, 0.45, fallback=False)


def test_threshold_extremes_and_partial_masks():
    banner("commit threshold extremes")
    c = W.commit_inputs(8, 32, 2000, "bf16", seed=11, masked_frac=0.4, boost=(0.0, 12.0))
    _, _, ref = run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 1.0)
    assert (ref["n_committed"] == 1).all()
    _, _, ref = run_case(c["logits"], "bf16", c["tokens"], c["masked"], 32, 1e-5)
    assert ref["committed"].sum() == c["masked"].sum()
    none = np.zeros_like(c["masked"])
    run_case(c["logits"], "bf16", c["tokens"], none, 32, 0.5)


@pytest.mark.parametrize("blk_len,dtype", [(1000, "f32"), (1024, "bf16"), (1024, "f32")])
def test_long_blocks(blk_len, dtype):
    """Blocks up to the longest the commit takes (1024 rows)."""
    banner(f"commit blk_len={blk_len} {dtype}")
    c = W.commit_inputs(2, blk_len, 700, dtype, seed=12, masked_frac=0.9, logit_std=3.0)
    for T in (0.9, 0.999):
        run_case(c["logits"], dtype, c["tokens"], c["masked"], blk_len, T)


def test_batched_loop_scale():
    """The batched-decode shape: 64 sequences x 32 rows x 151936 bf16 logits (622 MB)."""
    wl = W.WORKLOADS["decode_loop_bf16"]
    banner("commit decode_loop_bf16 scale")
    rng = np.random.default_rng(wl.seed)
    bits = W.boosted_logits_bits(64 * 32, wl.vocab, wl.boost[0], wl.boost[1], rng)
    masked = (rng.random(64 * 32) < 0.6).astype(np.uint8)
    tokens = np.where(masked == 1, -1, 5).astype(np.int32)
    for T in wl.thresholds:
        near, amb, ref = run_case(bits, "bf16", tokens, masked, 32, T)
        print(f"  T={T} committed={int(ref['committed'].sum())} near={near} ambiguous={amb}")


@pytest.mark.parametrize("n_masked", [1, 5, 37, 256])
def test_few_masked_rows_in_large_batch(n_masked):
    """A few masked rows among 256 rows of 151936 bf16 logits: the masked rows' logits are cut into
    many short ranges (up to hundreds per row) whose partials the decide step merges; also every
    row masked."""
    banner(f"commit {n_masked} masked of 256 rows, V=151936")
    rng = np.random.default_rng(100 + n_masked)
    V, rows = 151936, 256
    bits = W.boosted_logits_bits(rows, V, 2.0, 14.0, rng)
    masked = np.zeros(rows, np.uint8)
    masked[rng.choice(rows, n_masked, replace=False)] = 1
    tokens = np.where(masked == 1, -1, 3).astype(np.int32)
    for T in (0.5, 0.95):
        near, amb, ref = run_case(bits, "bf16", tokens, masked, 32, T)
        print(f"  T={T} committed={int(ref['committed'].sum())} near={near} ambiguous={amb}")


def test_neg_inf_runs():
    """-Inf logits in contiguous runs (a vocabulary mask): at the start of a row (whole load vectors
    of -Inf before any finite value), in the middle and at the end; such rows are valid."""
    banner("commit -inf runs")
    rng = np.random.default_rng(21)
    V, blk = 20011, 16
    x = rng.standard_normal((2 * blk, V)).astype(np.float32)
    x[0, :4096] = -np.inf
    x[1, :8] = -np.inf
    x[2, :7] = -np.inf
    x[3, :2051] = -np.inf
    x[4, 5000:9000] = -np.inf
    x[5, V - 3000:] = -np.inf
    x[6, :V - 1] = -np.inf               # one finite value, the last id: conf = 1
    x[7, 1:] = -np.inf                   # one finite value, the first id
    x[8, :] = -np.inf                    # all -inf: invalid
    x[9, :10000] = -np.inf
    x[9, 12345] = 9.0
    bits = W.f32_to_bf16_bits(x)
    masked = np.ones(2 * blk, np.uint8)
    tokens = np.full(2 * blk, -1, np.int32)
    for dt, arr in (("bf16", bits), ("f32", x)):
        for T in (0.3, 0.9):
            near, amb, ref = run_case(arr, dt, tokens, masked, blk, T)
            assert np.isfinite(ref["conf"][[0, 1, 2, 3, 4, 5, 6, 7, 9]]).all()


def test_per_row_thresholds():
    """One threshold per position (bd_confidence_commit_rowwise): random T_r per row, some NaN, some
    blocks where no row clears its own T (fallback), both dtypes."""
    banner("commit per-row thresholds")
    rng = np.random.default_rng(31)
    for dt, V, n_seq in (("bf16", 151936, 8), ("f32", 5003, 16)):
        c = W.commit_inputs(n_seq, 32, V, dt, seed=77 + V, masked_frac=0.8, boost=(2.0, 14.0))
        R = n_seq * 32
        thr = rng.uniform(0.3, 0.99, R)
        thr[rng.random(R) < 0.05] = np.nan
        thr[:32] = 2.0                         # block 0: nothing clears, fallback
        for fb in (True, False):
            near, amb, ref = run_case(c["logits"], dt, c["tokens"], c["masked"], 32, thr, fallback=fb)
            print(f"  {dt} fallback={fb} committed={int(ref['committed'].sum())} near={near} ambiguous={amb}")
