"""GPU check of bd_confidence_commit_noalloc, the commit entry point that allocates nothing (its
chunk partials live in the library's fixed device scratch array).

Called through the C ABI on two inputs in a row, the second smaller than the first (so it runs
on a scratch array that still holds the first call's partials), and compared with
bd_confidence_commit with a caller workspace on identical copies of the state: the same kernels
on the same chunking, so tokens, masks, ids, counts and confidences must be bit-identical.
"""
import numpy as np
import pytest
import torch

import workloads as W
from block_diffusion_decoding_amd import _lib as L
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def call_both(logits, dtype_code, n_seq, blk, vocab, T, tokens, masked):
    """Run the no-allocation entry point and the workspace one on copies of the same state."""
    rows = n_seq * blk
    outs = []
    for noalloc in (True, False):
        tok = tokens.clone()
        msk = masked.clone()
        conf = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
        pred = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
        ncom = torch.full((n_seq,), -7, dtype=torch.int32, device="cuda")
        nleft = torch.full((n_seq,), -7, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = L.lib.bd_confidence_commit_noalloc(logits.data_ptr(), logits.stride(0), n_seq, blk, vocab, dtype_code,
                                                    T, L.BD_FALLBACK_TOP1, tok.data_ptr(), msk.data_ptr(),
                                                    conf.data_ptr(), pred.data_ptr(), ncom.data_ptr(), nleft.data_ptr(),
                                                    stream)
        else:
            nb = L.lib.bd_confidence_commit_workspace_size(n_seq, blk, vocab)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
            st = L.lib.bd_confidence_commit(logits.data_ptr(), logits.stride(0), n_seq, blk, vocab, dtype_code, T,
                                            L.BD_FALLBACK_TOP1, tok.data_ptr(), msk.data_ptr(), conf.data_ptr(),
                                            pred.data_ptr(), ncom.data_ptr(), nleft.data_ptr(), ws.data_ptr(), nb,
                                            stream)
        assert st == L.BD_OK, st
        torch.cuda.synchronize()
        outs.append({k: v.cpu().numpy() for k, v in (("tokens", tok), ("masked", msk), ("conf", conf),
                                                    ("pred", pred), ("n_committed", ncom), ("n_masked_left", nleft))})
    a, b = outs
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    return a


def test_noalloc_matches_workspace_commit_twice():
    wl = W.WORKLOADS["decode_loop_bf16"]
    # call 1: the 64-sequence step (2048 rows x 151936 bf16), 60% of the rows masked
    banner("commit noalloc: 64 x 32 x 151936 bf16, then 6 x 32 x 5003 fp32")
    rng = np.random.default_rng(wl.seed + 3)
    bits = W.boosted_logits_bits(64 * 32, wl.vocab, wl.boost[0], wl.boost[1], rng)
    msk_np = (rng.random(64 * 32) < 0.6).astype(np.uint8)
    tok_np = np.where(msk_np == 1, -1, 9).astype(np.int32)
    lg = dev(bits, "bf16")
    a = call_both(lg, L.BD_BF16, 64, 32, wl.vocab, 0.5, torch.from_numpy(tok_np).cuda(),
                  torch.from_numpy(msk_np).cuda())
    assert a["n_committed"].sum() > 0 and (a["n_masked_left"] >= 0).all()
    del lg
    # call 2: smaller, other dtype, padded rows; the scratch still holds call 1's partials
    c = W.commit_inputs(6, 32, 5003, "f32", seed=77, masked_frac=0.75, logit_std=2.5)
    pad = np.zeros((6 * 32, 5008), np.float32)
    pad[:, :5003] = c["logits"]
    lg = torch.from_numpy(pad).cuda()
    b = call_both(lg, L.BD_F32, 6, 32, 5003, 0.2, torch.from_numpy(c["tokens"]).cuda(),
                  torch.from_numpy(c["masked"]).cuda())
    assert b["n_committed"].sum() > 0
