"""Graph capture of the hot path: a forward, a decode step and the commit (greedy and sampled),
and the backward, captured with every buffer allocated beforehand, replayed several times with eager work and
synchronisations between the replays; every replay must reproduce the eager results bit for bit
(the kernels are deterministic and the library issues no memory fills or allocations)."""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    banner("graph capture: forward, decode step, commit, sampled commit")
    torch.cuda.synchronize()
    # forward
    a = W.attention_inputs(1, 512, 16, 8, 128, "bf16", seed=3)
    q, k, v = (dev(a[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((1, 16, 512), dtype=torch.float32, device="cuda")
    # decode step: 8 ragged sequences
    plens = [0, 31, 100, 700, 1500, 33, 4096, 2]
    d = W.decode_inputs(len(plens), plens, 32, 16, 8, 128, "bf16", seed=7)
    qb, kb, vb = (dev(d[n], "bf16") for n in ("q_blk", "k_blk", "v_blk"))
    kc, vc = dev(d["k_cache"], "bf16"), dev(d["v_cache"], "bf16")
    ps = torch.from_numpy(d["prefix_start"]).cuda()
    pl = torch.from_numpy(d["prefix_len"]).cuda()
    max_p = max(plens)
    dec_o = torch.empty_like(qb)
    dec_lse = torch.empty((len(plens), 16, 32), dtype=torch.float32, device="cuda")
    dec_ws = torch.empty(bd.bd_attn_decode_workspace_size(len(plens), 32, max_p, 16, 8, 128), dtype=torch.uint8,
                         device="cuda")
    # commit state for the 8 blocks of 32 rows
    c = W.commit_inputs(8, 32, 5003, "bf16", seed=11, masked_frac=0.7, boost=(1.0, 9.0))
    lg = dev(c["logits"], "bf16")
    tok0 = torch.from_numpy(c["tokens"].copy()).cuda()
    msk0 = torch.from_numpy(c["masked"].copy()).cuda()
    tok, msk = tok0.clone(), msk0.clone()
    outs = {n: torch.empty(256, dtype=torch.float32 if n == "conf" else torch.int32, device="cuda")
            for n in ("conf", "pred")}
    cnt = {n: torch.empty(8, dtype=torch.int32, device="cuda") for n in ("ncom", "nleft")}
    cws = torch.empty(bd.bd_confidence_commit_workspace_size(8, 32, 5003), dtype=torch.uint8, device="cuda")
    tok_s, msk_s = tok0.clone(), msk0.clone()
    outs_s = {n: torch.empty_like(t) for n, t in outs.items()}
    cnt_s = {n: torch.empty_like(t) for n, t in cnt.items()}
    sws = torch.empty(bd.bd_confidence_commit_sampled_workspace_size(8, 32, 5003), dtype=torch.uint8, device="cuda")

    def step():
        bd.bd_attn_fwd(q, k, v, 32, o=o, lse=lse)
        bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse, workspace=dec_ws)
        bd.bd_confidence_commit(lg, tok, msk, 32, 0.6, conf=outs["conf"], pred=outs["pred"],
                                n_committed=cnt["ncom"], n_masked_left=cnt["nleft"], workspace=cws)
        bd.bd_confidence_commit_sampled(lg, tok_s, msk_s, 32, 0.3, seed=5, step=2, conf=outs_s["conf"],
                                        pred=outs_s["pred"], n_committed=cnt_s["ncom"],
                                        n_masked_left=cnt_s["nleft"], workspace=sws)

    rows_in = msk0.bool()   # conf / pred are written for the rows masked on entry only

    def results():
        torch.cuda.synchronize()
        r = [o, lse, dec_o, dec_lse, tok, msk, tok_s, msk_s, *cnt.values(), *cnt_s.values()]
        r += [t[rows_in] for t in (*outs.values(), *outs_s.values())]
        return [t.clone() for t in r]

    def reset_state():
        tok.copy_(tok0)
        msk.copy_(msk0)
        tok_s.copy_(tok0)
        msk_s.copy_(msk0)

    def poison():
        for t in (o, dec_o):
            t.fill_(float("nan"))
        for t in (lse, dec_lse, outs["conf"], outs_s["conf"]):
            t.fill_(-7.0)
        for t in (outs["pred"], outs_s["pred"], *cnt.values(), *cnt_s.values()):
            t.fill_(-99)

    reset_state()
    step()
    eager = results()
    reset_state()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        reset_state()
        poison()
        torch.cuda.synchronize()
        g.replay()
        got = results()
        for i, (x, y) in enumerate(zip(eager, got)):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), f"replay {rep}: output {i} differs"
        # eager work between replays, on other buffers
        bd.bd_confidence_commit(lg, tok0.clone(), msk0.clone(), 32, 0.9, workspace=cws)
        torch.cuda.synchronize()
    print("  4 replays bit-identical to the eager step")


def test_graph_backward_replays_equal_eager():
    # 1 x 512 tokens, 16 / 8 heads: 32 dK/dV and 32 dQ items, so the backward runs as
    # one persistent launch whose work counters (in the workspace) the prep kernel
    # zeroes; the workspace is filled with 0xFF before every replay.
    banner("graph capture: backward (queued launch)")
    torch.cuda.synchronize()
    a = W.attention_inputs(1, 512, 16, 8, 128, "bf16", seed=21, with_grad=True)
    q, k, v, d_o = (dev(a[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = bd.bd_attn_fwd(q, k, v, 32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(bd.bd_attn_bwd_workspace_size(1, 512, 16, 8, 128), dtype=torch.uint8, device="cuda")

    def step():
        bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        ws.fill_(0xFF)
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(eager, (dq, dk, dv))):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"replay {rep}: gradient {i} differs"
        step()   # eager work between replays
        torch.cuda.synchronize()
    print("  4 replays bit-identical to the eager backward")
