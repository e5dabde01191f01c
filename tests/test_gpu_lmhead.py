"""GPU parity of bd_lmhead_commit (output projection fused with the confidence commit) against
oracle.lmhead.

Tolerances follow from the arithmetic: the GPU sums the H products of each logit in fp32 (exact
bf16 x bf16 products, fp32 additions in the matrix cores' order), the oracle in fp64.
  * Worst case, each logit of row r is off by at most delta_r = H * 2^-23 * max_v sum_k
    |x_rk w_vk|.  pred must equal the oracle's argmax unless other ids lie within 2 delta_r of
    the maximum; then it must be one of those ids.
  * The rounding errors of a sum of H products of random sign add up like a random walk:
    about 2^-24 sqrt(H) |x_r| |w_v| (1e-6 .. 1e-5 on these inputs), so conf (a ratio of
    exponentials of logit differences) must agree to 1e-4 relative; the worst-case bound is
    only used to decide which ids count as tied.
  * The committed sets are bit-exact, except where a row's conf lies within that tolerance of T
    (counted as near-T) or the fallback is decided by confidences within it.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import commit as C
from oracle import lmhead as LH
from gpu_util import banner

pytestmark = pytest.mark.gpu


def run_case(d, blk_len, T, fallback=True):
    """Run the fused GPU commit and the oracle on the same inputs; check and return counts."""
    xb, wb = d["hidden"], d["weight"]
    rows, H = xb.shape
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(wb.view(np.int16)).cuda().view(torch.bfloat16)
    tok = torch.from_numpy(d["tokens"].copy()).cuda()
    msk = torch.from_numpy(d["masked"].copy()).cuda()
    out = bd.bd_lmhead_commit(x, w, tok, msk, blk_len, T, bd.BD_FALLBACK_TOP1 if fallback else bd.BD_FALLBACK_NONE)
    torch.cuda.synchronize()
    g_tok, g_msk = tok.cpu().numpy(), msk.cpu().numpy()
    g_conf = out["conf"].cpu().numpy().astype(np.float64)
    g_pred = out["pred"].cpu().numpy()
    g_ncom, g_nleft = out["n_committed"].cpu().numpy(), out["n_masked_left"].cpu().numpy()
    del x, w

    x64 = W.bf16_bits_to_f32(xb).astype(np.float64)
    w64 = W.bf16_bits_to_f32(wb).astype(np.float64)
    logits = LH.lmhead_logits(x64, w64)
    bound = np.abs(x64) @ np.abs(w64).T
    delta = H * 2.0 ** -23 * bound.max(axis=1)
    del w64, bound
    ref = C.confidence_commit(logits, d["tokens"], d["masked"], blk_len, T,
                              C.FALLBACK_TOP1 if fallback else C.FALLBACK_NONE)
    m_in = d["masked"].astype(bool)
    tol = 1e-4 * np.nan_to_num(ref["conf"], nan=0.0) + 1e-7

    # per-row ids and confidences
    ambiguous_ids = 0
    for r in np.flatnonzero(m_in):
        assert np.isnan(g_conf[r]) == np.isnan(ref["conf"][r]), f"row {r}: invalid flags differ"
        row = logits[r]
        cands = np.flatnonzero(row >= row.max() - 2 * delta[r])
        if len(cands) == 1:
            assert g_pred[r] == ref["pred"][r], f"row {r}: pred {g_pred[r]} vs {ref['pred'][r]}"
        else:
            ambiguous_ids += 1
            assert g_pred[r] in cands, f"row {r}: pred {g_pred[r]} not among near-max ids {cands}"
        assert abs(g_conf[r] - ref["conf"][r]) <= tol[r], f"row {r}: conf {g_conf[r]} vs {ref['conf'][r]}"
    assert np.array_equal(g_tok[~m_in], d["tokens"][~m_in]), "unmasked rows touched"
    assert np.array_equal(g_msk[~m_in], d["masked"][~m_in]), "unmasked rows touched"

    # committed sets per block
    committed = m_in & (g_msk == 0)
    assert np.array_equal(g_tok[committed], g_pred[committed])
    near = 0
    for g in range(rows // blk_len):
        sl = slice(g * blk_len, (g + 1) * blk_len)
        mg, c, com_g, com_r = m_in[sl], ref["conf"][sl], committed[sl], ref["committed"][sl]
        valid = mg & ~np.isnan(c)
        band = tol[sl]
        assert g_ncom[g] == com_g.sum() and g_nleft[g] == mg.sum() - com_g.sum()
        near_rows = valid & (np.abs(c - T) <= band)
        if near_rows.any():
            near += int(near_rows.sum())
            assert np.all(com_g[valid & (c > T + band)])
            continue
        if (valid & (c > T)).any() or not fallback or not valid.any():
            assert np.array_equal(com_g, com_r), f"block {g}: committed set differs"
            continue
        cv = np.where(valid, c, -np.inf)
        top = np.sort(cv)[::-1]
        if len(top) > 1 and top[0] - top[1] <= band.max():
            assert com_g.sum() == 1
        else:
            assert np.array_equal(com_g, com_r), f"block {g}: fallback row differs"
    ok = m_in & ~np.isnan(ref["conf"])
    rel = np.max(np.abs(g_conf[ok] - ref["conf"][ok]) / ref["conf"][ok]) if ok.any() else 0.0
    print(f"  T={T} committed={int(ref['committed'].sum())} near-T={near} ambiguous ids={ambiguous_ids} "
          f"worst-case logit bound={delta.max():.1e} conf max rel err={rel:.1e}")
    return ref


@pytest.mark.parametrize("H,V", [(64, 1000), (192, 5003), (128, 4099), (256, 777), (512, 20000), (1024, 6007),
                                 (2048, 3001)])
def test_shapes(H, V):
    """Every loads-in-flight variant (H/64 = 1, 3, 2, 4, 8, 16, 32 steps per block) and ragged
    vocabularies (V not a multiple of the 8-row block; fewer blocks than waves)."""
    banner(f"lmhead H={H} V={V}")
    d = W.lmhead_inputs(1, 32, H, V, seed=H + V, boost=(1.0, 10.0))
    for T in (0.3, 0.9):
        run_case(d, 32, T)


def test_several_blocks_and_partial_masks():
    """Three blocks (three row tiles; the middle one with no masked row is skipped), 40-row blocks
    (tiles straddle blocks), and the fallback switched off."""
    banner("lmhead several blocks")
    d = W.lmhead_inputs(3, 32, 512, 9000, seed=5, masked_frac=0.5)
    d["masked"][32:64] = 0
    d["tokens"][32:64] = 7
    run_case(d, 32, 0.5)
    run_case(d, 32, 0.99, fallback=False)
    d = W.lmhead_inputs(3, 40, 256, 7001, seed=6, masked_frac=0.6)
    run_case(d, 40, 0.7)


def test_decode_block_workload():
    """The full-size shape: one block of 32 hidden states of width 2048 against the
    [151936 x 2048] weight (622 MB), as timed by the benchmark."""
    wl = W.WORKLOADS["lmhead_block_bf16"]
    H = wl.n_q_heads * wl.head_dim
    banner(f"lmhead workload 32 x {H} x {wl.vocab}")
    d = W.lmhead_inputs(1, wl.block_size, H, wl.vocab, seed=wl.seed, boost=wl.boost)
    for T in (wl.threshold, 0.5):
        run_case(d, wl.block_size, T)
