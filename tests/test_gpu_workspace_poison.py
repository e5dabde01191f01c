"""Workspace contents on entry are ignored (include/bd.h, every entry point that takes one).

Each call runs three times on the same inputs with its workspace filled first with zero
bytes, then with 0xFF bytes (NaN as float32, -1 as int32) and then with 0x7F bytes (3.4e38
as float32): every output must be bit-identical across the three runs.  A kernel that read a
workspace word before writing it in the same call would see the poison here.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu

POISONS = (0x00, 0xFF, 0x7F)


def same_for_every_poison(nbytes, run):
    """run(ws) -> tuple of output tensors; ws is a fresh uint8 workspace of nbytes per poison."""
    outs = []
    for byte in POISONS:
        ws = torch.full((max(int(nbytes), 16),), byte, dtype=torch.uint8, device="cuda")
        res = run(ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in res])
    for byte, o in zip(POISONS[1:], outs[1:]):
        for i, (a, b) in enumerate(zip(outs[0], o)):   # bytes, so that NaN outputs compare equal too
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
                f"output {i} differs with the workspace filled with 0x{byte:02x}"


@pytest.mark.parametrize("dtype,L,Hq,Hkv,d,blk", [("bf16", 300, 4, 2, 128, 32), ("f32", 130, 4, 2, 64, 16)])
def test_backward(dtype, L, Hq, Hkv, d, blk):
    banner(f"workspace poison: backward {dtype} L={L}")
    inp = W.attention_inputs(1, L, Hq, Hkv, d, dtype, seed=L)
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = bd.bd_attn_fwd(q, k, v, block_size=blk)
    d_o = dev(W.attention_inputs(1, L, Hq, Hkv, d, dtype, seed=L + 1)["q"], dtype)
    nbytes = bd.bd_attn_bwd_workspace_size(1, L, Hq, Hkv, d)
    same_for_every_poison(nbytes, lambda ws: bd.bd_attn_bwd(q, k, v, o, lse, d_o, block_size=blk, workspace=ws))


@pytest.mark.parametrize("plens", [[0, 37, 1000, 129, 5], [4096]])
def test_decode(plens):
    banner(f"workspace poison: decode plens={plens}")
    Hq, Hkv, T = 16, 8, 32
    dd = W.decode_inputs(len(plens), plens, T, Hq, Hkv, 128, "bf16", seed=sum(plens))
    t = {n: dev(dd[n], "bf16") for n in ("q_blk", "k_blk", "v_blk")}
    kc = dev(dd["k_cache"], "bf16") if dd["k_cache"].shape[0] else None
    vc = dev(dd["v_cache"], "bf16") if dd["v_cache"].shape[0] else None
    ps, pl = torch.from_numpy(dd["prefix_start"]).cuda(), torch.from_numpy(dd["prefix_len"]).cuda()
    max_p = max(plens)
    nbytes = bd.bd_attn_decode_workspace_size(len(plens), T, max_p, Hq, Hkv, 128)
    same_for_every_poison(nbytes, lambda ws: bd.bd_attn_decode_block(t["q_blk"], t["k_blk"], t["v_blk"], kc, vc, ps,
                                                                     pl, max_p, workspace=ws))

    # the same prefixes in pages of 64 rows (sequence s in pages s*mp .. s*mp + mp - 1)
    page = 64
    mp = (max_p + page - 1) // page
    kp = np.zeros((len(plens) * mp * page, Hkv, 128), np.uint16)
    vp = np.zeros_like(kp)
    for s, P in enumerate(plens):
        a = int(dd["prefix_start"][s])
        kp[s * mp * page:s * mp * page + P] = dd["k_cache"][a:a + P]
        vp[s * mp * page:s * mp * page + P] = dd["v_cache"][a:a + P]
    table = torch.arange(len(plens) * mp, dtype=torch.int32, device="cuda").view(len(plens), mp)
    kpd, vpd = dev(kp, "bf16"), dev(vp, "bf16")
    pl32 = pl.to(torch.int32)
    same_for_every_poison(nbytes, lambda ws: bd.bd_attn_decode_block_paged(t["q_blk"], t["k_blk"], t["v_blk"], kpd,
                                                                           vpd, table, page, pl32, max_p,
                                                                           workspace=ws))


def commit_state(n_seq, blk, V, dtype, seed):
    c = W.commit_inputs(n_seq, blk, V, dtype, seed, masked_frac=0.6, boost=(0.0, 9.0))
    return dev(c["logits"], dtype), c["tokens"], c["masked"]


def fresh(tokens, masked):
    """Device copies of the token state, and conf / pred outputs holding sentinels (the calls
    write them only for rows masked on entry)."""
    rows = len(tokens)
    conf = torch.full((rows,), -7.0, dtype=torch.float32, device="cuda")
    pred = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    return torch.from_numpy(tokens.copy()).cuda(), torch.from_numpy(masked.copy()).cuda(), conf, pred


@pytest.mark.parametrize("dtype,n_seq,V", [("bf16", 8, 5003), ("f32", 2, 151936), ("bf16", 64, 32768)])
def test_commit(dtype, n_seq, V):
    banner(f"workspace poison: commit {dtype} {n_seq}x32x{V}")
    lg, tokens, masked = commit_state(n_seq, 32, V, dtype, seed=V + n_seq)
    nbytes = bd.bd_confidence_commit_workspace_size(n_seq, 32, V)
    thr = torch.linspace(0.3, 0.99, n_seq * 32, device="cuda", dtype=torch.float32)

    def greedy(ws, threshold):
        tok, msk, conf, pred = fresh(tokens, masked)
        out = bd.bd_confidence_commit(lg, tok, msk, 32, threshold, conf=conf, pred=pred, workspace=ws)
        return tok, msk, out["conf"], out["pred"], out["n_committed"], out["n_masked_left"]

    same_for_every_poison(nbytes, lambda ws: greedy(ws, 0.9))
    same_for_every_poison(nbytes, lambda ws: greedy(ws, thr))

    snbytes = bd.bd_confidence_commit_sampled_workspace_size(n_seq, 32, V)
    for top_k, top_p in ((0, 1.0), (50, 1.0), (0, 0.9)):
        if (top_k or top_p < 1.0) and V > 77824 and dtype == "f32":
            continue   # truncation holds the row in registers: fp32 rows of at most 77824 ids

        def sampled(ws):
            tok, msk, conf, pred = fresh(tokens, masked)
            out = bd.bd_confidence_commit_sampled(lg, tok, msk, 32, 0.9, temperature=0.8, seed=3, step=1,
                                                  top_k=top_k, top_p=top_p, conf=conf, pred=pred, workspace=ws)
            return tok, msk, out["conf"], out["pred"], out["n_committed"], out["n_masked_left"]

        same_for_every_poison(snbytes, sampled)


def test_lmhead_commit():
    banner("workspace poison: lmhead commit 2x32x1024x20000")
    inp = W.lmhead_inputs(2, 32, 1024, 20000, seed=5, masked_frac=0.75)
    h, w = dev(inp["hidden"], "bf16"), dev(inp["weight"], "bf16")
    nbytes = bd.bd_lmhead_commit_workspace_size(2, 32, 20000)

    def run(ws):
        tok, msk, conf, pred = fresh(inp["tokens"], inp["masked"])
        out = bd.bd_lmhead_commit(h, w, tok, msk, 32, 0.9, conf=conf, pred=pred, workspace=ws)
        return tok, msk, out["conf"], out["pred"], out["n_committed"], out["n_masked_left"]

    same_for_every_poison(nbytes, run)
