"""Benchmark of the block-diffusion decoding hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  * block-causal attention forward and backward on the 2 x 16384-token
    workload (16 q / 8 kv heads, head_dim 128, block 32, bf16), and
  * one step of the batched decode loop (64 sequences with ragged prefixes
    U[1024, 16384]): one block against the prefix cache for every sequence,
    then the threshold commit over their [64*32 x 151936] bf16 logits and the
    read-back of the per-block counts.
`value` is the forward's TFLOP/s on the 16384-token workload, counted on the
allowed (query, key) pairs only (4 * head_dim flops per pair), from HIP events
around each forward launch.  The other rows of the metric (decode steps/s,
commit GB/s, backward TFLOP/s) are reported beside it, together with the
single-shot decode-step and commit kernels of the 4096-token workload, measured
over rotating input copies so that the 256 MB Infinity Cache does not serve
them, and the output projection fused with the commit (one block of 32 hidden
states of width 2048 against a 151936-row weight) beside the unfused path
(library GEMM to bf16 logits, then the commit).  The CPU oracle is timed on a
bounded sample on the host.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# Mean steps per block of the 64-sequence loop under its logits recipe (N(0,1) plus a U(2, 14)
# boost at one id per row, vocabulary 151936, fresh every step), by Monte Carlo of the recipe.
EXPECTED_STEPS = {0.5: 15.9, 0.95: 31.9, 0.99: 32.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run each hot-path kernel a few times plus a 1 GiB reference copy (for rocprofv3 --pmc)")
    ap.add_argument("--summarize", nargs="+", metavar="DB",
                    help="summarize rocprofv3 result databases into a text profile (see --out, --title)")
    ap.add_argument("--out", default=None)
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="", help="the command that produced the databases (recorded)")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the block-causal attention, decode and commit kernels "
              "shard without communication (see the design notes); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_decoding_amd as bd
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ------------------------------------------------------------------ inputs
    wl = W.WORKLOADS["fwdbwd_L16384_bf16"]
    B, L, Hq, Hkv, D, blk = wl.batch, wl.seqlen, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size
    inp = W.attention_inputs(B, L, Hq, Hkv, D, "bf16", wl.seed, with_grad=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bwd_ws = torch.empty(bd.bd_attn_bwd_workspace_size(B, L, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    pairs = blk * blk * (L // blk) * (L // blk + 1) // 2
    fwd_flops = 4.0 * D * pairs * Hq * B
    bwd_flops = 2.5 * fwd_flops

    have_bwd = True
    try:
        bd.bd_attn_fwd(q, k, v, blk, o=o, lse=lse)
        bd.bd_attn_bwd(q, k, v, o, lse, do, blk, dq=dq, dk=dk, dv=dv, workspace=bwd_ws)
    except bd.BdError as e:
        if e.status != 3:
            raise
        have_bwd = False

    # batched decode loop state (64 ragged sequences)
    lw = W.WORKLOADS["decode_loop_bf16"]
    rng = np.random.default_rng(lw.seed)
    plen = W.prefix_lengths(lw.n_seq, lw.prefix_range[0], lw.prefix_range[1], rng)
    dec = W.decode_inputs(lw.n_seq, plen, lw.block_size, Hq, Hkv, D, "bf16", lw.seed, rng=rng)
    kc, vc = to_dev(dec["k_cache"]), to_dev(dec["v_cache"])
    ps, pl = torch.from_numpy(dec["prefix_start"]).to(dev), torch.from_numpy(dec["prefix_len"]).to(dev)
    qb, kb, vb = (to_dev(dec[n]) for n in ("q_blk", "k_blk", "v_blk"))
    del dec
    max_p = int(plen.max())
    n_rows = lw.n_seq * lw.block_size
    V = lw.vocab
    gen = torch.Generator(device=dev)
    gen.manual_seed(lw.seed)
    # Fresh logits for every step of a loop: with the fallback a block finishes within block_size
    # steps, so one buffer per step (32 x 622 MB, resident in HBM) gives every step of every loop
    # its own draw; the generator runs before any timed region.
    n_pool = lw.block_size
    logit_pool = []
    for _ in range(n_pool):   # N(0,1) + U(2,14) at one random id per row, bf16
        x = torch.randn((n_rows, V), generator=gen, device=dev, dtype=torch.float32)
        ids = torch.randint(0, V, (n_rows,), generator=gen, device=dev)
        x[torch.arange(n_rows, device=dev), ids] += torch.empty(n_rows, device=dev).uniform_(
            lw.boost[0], lw.boost[1], generator=gen)
        logit_pool.append(x.to(torch.bfloat16))
        del x
    dec_o = torch.empty_like(qb)
    dec_lse = torch.empty((lw.n_seq, Hq, lw.block_size), dtype=torch.float32, device=dev)
    dec_ws = torch.empty(bd.bd_attn_decode_workspace_size(lw.n_seq, lw.block_size, max_p, Hq, Hkv, D),
                         dtype=torch.uint8, device=dev)
    com_ws = torch.empty(bd.bd_confidence_commit_workspace_size(lw.n_seq, lw.block_size, V), dtype=torch.uint8,
                         device=dev)
    tokens = torch.full((n_rows,), -1, dtype=torch.int32, device=dev)
    masked = torch.ones(n_rows, dtype=torch.uint8, device=dev)
    conf = torch.empty(n_rows, dtype=torch.float32, device=dev)
    pred = torch.empty(n_rows, dtype=torch.int32, device=dev)
    ncom = torch.empty(lw.n_seq, dtype=torch.int32, device=dev)
    nleft = torch.empty(lw.n_seq, dtype=torch.int32, device=dev)
    nleft_host = torch.empty(lw.n_seq, dtype=torch.int32, pin_memory=True)
    kv_bytes_loop = float((plen.astype(np.int64) + lw.block_size).sum() * Hkv * D * 2 * 2)
    T_step = 0.95
    loop_state = {"step": 0}

    if args.traffic_probe:
        # Counter runs (rocprofv3 --pmc) read per-dispatch HBM bytes of these kernels.  The
        # scale of each counter comes from a plain streaming kernel of known size that no other
        # step launches: a bitwise NOT of 2^28 int32 (1 GiB read, 1 GiB written).
        src = torch.empty(REF_COPY_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        for _ in range(3):
            bd.bd_attn_fwd(q, k, v, blk, o=o, lse=lse)
        if have_bwd:
            for _ in range(2):
                bd.bd_attn_bwd(q, k, v, o, lse, do, blk, dq=dq, dk=dk, dv=dv, workspace=bwd_ws)
        hw = W.WORKLOADS["lmhead_block_bf16"]
        H_lm = hw.n_q_heads * hw.head_dim
        d_lm = W.lmhead_inputs(1, hw.block_size, H_lm, hw.vocab, hw.seed, boost=hw.boost)
        x_lm = to_dev(d_lm["hidden"]).view(hw.block_size, H_lm)
        w_lm = to_dev(d_lm["weight"]).view(hw.vocab, H_lm)
        del d_lm
        t_lm = torch.full((hw.block_size,), -1, dtype=torch.int32, device=dev)
        m_lm = torch.ones(hw.block_size, dtype=torch.uint8, device=dev)
        for _ in range(3):
            bd.bd_lmhead_commit(x_lm, w_lm, t_lm, m_lm, hw.block_size, 2.0, fallback=bd.BD_FALLBACK_NONE)
        torch.cuda.synchronize()
        del x_lm, w_lm
        for i in range(3):
            masked.fill_(1)
            bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse, workspace=dec_ws)
            bd.bd_confidence_commit(logit_pool[i % n_pool], tokens, masked, lw.block_size, T_step, conf=conf,
                                    pred=pred, n_committed=ncom, n_masked_left=nleft, workspace=com_ws)
        for i in range(3):   # sampled commit, plain and with top-p truncation, on all-masked rows
            for k_, p_ in ((0, 1.0), (0, 0.9)):
                masked.fill_(1)
                bd.bd_confidence_commit_sampled(logit_pool[i % n_pool], tokens, masked, lw.block_size, T_step,
                                                seed=lw.seed, step=i, top_k=k_, top_p=p_)
        torch.cuda.synchronize()
        print("traffic probe done", flush=True)
        return

    def one_step(rec):
        """decode + commit for every sequence, then forward + backward; one sync at the end."""
        s = loop_state["step"]
        rec[0].record()
        bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse, workspace=dec_ws)
        rec[1].record()
        bd.bd_confidence_commit(logit_pool[s % n_pool], tokens, masked, lw.block_size, T_step, conf=conf,
                                pred=pred, n_committed=ncom, n_masked_left=nleft, workspace=com_ws)
        rec[2].record()
        bd.bd_attn_fwd(q, k, v, blk, o=o, lse=lse)
        rec[3].record()
        if have_bwd:
            bd.bd_attn_bwd(q, k, v, o, lse, do, blk, dq=dq, dk=dk, dv=dv, workspace=bwd_ws)
        rec[4].record()
        nleft_host.copy_(nleft, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        loop_state["step"] = s + 1
        if int(nleft_host.sum()) == 0:          # every block committed: the next block starts masked
            masked.fill_(1)
            tokens.fill_(-1)

    for _ in range(args.warmup):
        one_step([ev() for _ in range(5)])
    torch.cuda.synchronize()
    recs = [[ev() for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for r in recs:
        one_step(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [r[2].elapsed_time(r[3]) for r in recs]
    bwd_ms = [r[3].elapsed_time(r[4]) for r in recs]
    fwd_avg = float(np.mean(fwd_ms))
    fwd_tflops = fwd_flops / (fwd_avg * 1e-3) / 1e12

    def primed(launches, n_launch_us=60.0):
        """Per-launch GPU time of short kernels: a spin kernel holds the queue while the host
        enqueues every launch with its events, so no launch waits on the host."""
        evs = [(ev(), ev()) for _ in launches]
        spin_ms = len(launches) * n_launch_us * 1e-3
        torch.cuda._sleep(int(spin_ms * 1e-3 * sleep_hz))
        for (a, b_), fn in zip(evs, launches):
            a.record()
            fn()
            b_.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b_) * 1e3 for a, b_ in evs])

    # calibrate the spin kernel
    a0, b0 = ev(), ev()
    a0.record()
    torch.cuda._sleep(1_000_000)
    b0.record()
    torch.cuda.synchronize()
    sleep_hz = 1_000_000 / (a0.elapsed_time(b0) * 1e-3)

    # decode-loop kernels, primed: one full loop at T = 0.95 with per-launch GPU times
    masked.fill_(1)
    tokens.fill_(-1)
    dec_us, com_us, com_rows = [], [], []
    for step in range(64):
        m_rows = int(masked.sum())
        if m_rows == 0:
            break
        t_us = primed([lambda: bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse,
                                                       workspace=dec_ws),
                       lambda st=step: bd.bd_confidence_commit(logit_pool[st % n_pool], tokens, masked,
                                                               lw.block_size, T_step, conf=conf, pred=pred,
                                                               n_committed=ncom, n_masked_left=nleft,
                                                               workspace=com_ws)])
        dec_us.append(t_us[0])
        com_us.append(t_us[1])
        com_rows.append(m_rows)
    dec_ms = np.array(dec_us) * 1e-3
    com_gbs_loop = [r * V * 2 / (u * 1e-6) / 1e9 for r, u in zip(com_rows, com_us)]

    # ------------------------------------------- decode-loop steps/s per T
    def loop_record(T, steps_all, blk_steps, t_all, reps):
        """steps/s of the whole loops, and the steps each sequence's block took (mean over the
        sequences and runs, and the largest), beside the values the workload's recipe predicts."""
        bs = np.concatenate(blk_steps)
        return {"T": T, "loop_steps": steps_all[0], "steps_per_block_mean": round(float(bs.mean()), 2),
                "steps_per_block_max": int(bs.max()), "steps_per_block_expected_mean": EXPECTED_STEPS.get(T),
                "steps_per_s": round(sum(steps_all) / t_all, 1), "tokens_per_s": round(n_rows * reps / t_all, 1)}

    def block_steps(left_per_step):
        """Per sequence, the step count at which its block had no masked row left."""
        left = np.stack(left_per_step)                   # [steps, n_seq]
        return (left > 0).sum(axis=0) + 1

    def full_loop(T, reps=3):
        """Whole loops from an all-masked block until every sequence's block is committed, with
        fresh logits at every step; wall-clock steps/s including the per-step read-back of the
        block counts."""
        steps_all, blk_steps, t_all = [], [], 0.0
        for _ in range(reps):
            masked.fill_(1)
            tokens.fill_(-1)
            torch.cuda.synchronize()
            n, left = 0, []
            t0 = time.perf_counter()
            while True:
                bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse, workspace=dec_ws)
                bd.bd_confidence_commit(logit_pool[n % n_pool], tokens, masked, lw.block_size, T, conf=conf,
                                        pred=pred, n_committed=ncom, n_masked_left=nleft, workspace=com_ws)
                nleft_host.copy_(nleft, non_blocking=True)
                torch.cuda.current_stream().synchronize()
                n += 1
                left.append(nleft_host.numpy().copy())
                if int(nleft_host.sum()) == 0 or n >= n_pool:
                    break
            t_all += time.perf_counter() - t0
            steps_all.append(n)
            blk_steps.append(block_steps(left))
        return loop_record(T, steps_all, blk_steps, t_all, reps)

    loops = [full_loop(T) for T in lw.thresholds]

    def graph_loop(T, reps=3):
        """The same loop with each step (decode, commit, read-back of the block counts) replayed
        from a captured graph: one graph per step's logits buffer."""
        graphs = []
        for i in range(n_pool):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, max_p, o=dec_o, lse=dec_lse, workspace=dec_ws)
                bd.bd_confidence_commit(logit_pool[i], tokens, masked, lw.block_size, T, conf=conf, pred=pred,
                                        n_committed=ncom, n_masked_left=nleft, workspace=com_ws)
                nleft_host.copy_(nleft, non_blocking=True)
            graphs.append(g)
        steps_all, blk_steps, t_all = [], [], 0.0
        for _ in range(reps):
            masked.fill_(1)
            tokens.fill_(-1)
            torch.cuda.synchronize()
            n, left = 0, []
            t0 = time.perf_counter()
            while True:
                graphs[n % n_pool].replay()
                torch.cuda.current_stream().synchronize()
                n += 1
                left.append(nleft_host.numpy().copy())
                if int(nleft_host.sum()) == 0 or n >= n_pool:
                    break
            t_all += time.perf_counter() - t0
            steps_all.append(n)
            blk_steps.append(block_steps(left))
        del graphs
        return loop_record(T, steps_all, blk_steps, t_all, reps)

    loops_graph = [graph_loop(T) for T in lw.thresholds]

    # the same decode step with the prefix in shuffled pages of 256 rows (bd_attn_decode_block_paged)
    page = 256
    max_pages = (max_p + page - 1) // page
    pstart_np = ps.cpu().numpy()
    prng = np.random.default_rng(lw.seed + 11)
    table_np = prng.permutation(lw.n_seq * max_pages).astype(np.int32).reshape(lw.n_seq, max_pages)
    src_rows, dst_rows = [], []
    for s_ in range(lw.n_seq):
        P_ = int(plen[s_])
        j_ = np.arange(P_)
        src_rows.append(int(pstart_np[s_]) + j_)
        dst_rows.append(table_np[s_, j_ // page].astype(np.int64) * page + j_ % page)
    src_t = torch.from_numpy(np.concatenate(src_rows)).to(dev)
    dst_t = torch.from_numpy(np.concatenate(dst_rows)).to(dev)
    kpg = torch.zeros((lw.n_seq * max_pages * page, Hkv, D), dtype=torch.bfloat16, device=dev)
    vpg = torch.zeros_like(kpg)
    kpg[dst_t] = kc[src_t]
    vpg[dst_t] = vc[src_t]
    del src_t, dst_t
    table_t = torch.from_numpy(table_np).to(dev)
    pl32 = pl.to(torch.int32)
    pg_us = []
    for rnd in range(4):
        t_us = primed([lambda: bd.bd_attn_decode_block_paged(qb, kb, vb, kpg, vpg, table_t, page, pl32, max_p,
                                                             o=dec_o, lse=dec_lse, workspace=dec_ws)
                       for _ in range(8)])
        if rnd:
            pg_us.extend(t_us)
    del kpg, vpg

    # per-position thresholds (bd_confidence_commit_rowwise) on the all-masked first step
    thr_rows = torch.from_numpy(np.random.default_rng(lw.seed + 7).uniform(0.5, 0.99, n_rows)
                                .astype(np.float32)).to(dev)
    msk_rw = [torch.ones_like(masked) for _ in range(n_pool)]
    rw_us = []
    for rnd in range(4):
        for m in msk_rw:
            m.fill_(1)
        t_us = primed([lambda i=i: bd.bd_confidence_commit(logit_pool[i], tokens, msk_rw[i], lw.block_size, thr_rows,
                                                           conf=conf, pred=pred, n_committed=ncom,
                                                           n_masked_left=nleft, workspace=com_ws)
                       for i in range(n_pool)])
        if rnd:
            rw_us.extend(t_us)
    rw_bytes = n_rows * V * 2

    # sampled predictions at temperature 1 (bd_confidence_commit_sampled) on the all-masked first step
    sm_ws = torch.empty(bd.bd_confidence_commit_sampled_workspace_size(lw.n_seq, lw.block_size, V), dtype=torch.uint8,
                        device=dev)
    sm_us = []
    for rnd in range(4):
        for m in msk_rw:
            m.fill_(1)
        t_us = primed([lambda i=i: bd.bd_confidence_commit_sampled(logit_pool[i], tokens, msk_rw[i], lw.block_size,
                                                                   T_step, temperature=1.0, seed=lw.seed, step=rnd,
                                                                   conf=conf, pred=pred, n_committed=ncom,
                                                                   n_masked_left=nleft, workspace=sm_ws)
                       for i in range(n_pool)])
        if rnd:
            sm_us.extend(t_us)

    # the same step with top-k / top-p truncation (one workgroup per row, the row held in registers)
    tr_us = {}
    for k_, p_ in ((50, 1.0), (0, 0.9)):
        tr_us[(k_, p_)] = []
        for rnd in range(3):
            for m in msk_rw:
                m.fill_(1)
            t_us = primed([lambda i=i: bd.bd_confidence_commit_sampled(logit_pool[i], tokens, msk_rw[i], lw.block_size,
                                                                       T_step, temperature=1.0, seed=lw.seed,
                                                                       step=rnd, top_k=k_, top_p=p_, conf=conf,
                                                                       pred=pred, n_committed=ncom,
                                                                       n_masked_left=nleft, workspace=sm_ws)
                           for i in range(n_pool)], n_launch_us=400.0)
            if rnd:
                tr_us[(k_, p_)].extend(t_us)

    # ------------------------------- single-shot decode step / commit, 4096 prefix
    sw = W.WORKLOADS["decode_step_bf16"]
    n_copies_kv, n_copies_lg = 40, 64
    srng = np.random.default_rng(sw.seed)
    d1 = W.decode_inputs(1, [sw.prefix_len], sw.block_size, Hq, Hkv, D, "bf16", sw.seed, rng=srng)
    c1 = W.commit_inputs(1, sw.block_size, sw.vocab, "bf16", sw.seed, boost=sw.boost, rng=srng)
    kc1 = [to_dev(d1["k_cache"]) for _ in range(n_copies_kv)]
    vc1 = [to_dev(d1["v_cache"]) for _ in range(n_copies_kv)]
    qb1, kb1, vb1 = (to_dev(d1[n]) for n in ("q_blk", "k_blk", "v_blk"))
    ps1, pl1 = torch.from_numpy(d1["prefix_start"]).to(dev), torch.from_numpy(d1["prefix_len"]).to(dev)
    ws1 = torch.empty(bd.bd_attn_decode_workspace_size(1, sw.block_size, sw.prefix_len, Hq, Hkv, D),
                      dtype=torch.uint8, device=dev)
    o1 = torch.empty_like(qb1)
    lse1 = torch.empty((1, Hq, sw.block_size), dtype=torch.float32, device=dev)
    lg1 = [to_dev(c1["logits"]) for _ in range(n_copies_lg)]
    tok1 = torch.from_numpy(c1["tokens"]).to(dev)
    msk_src = torch.from_numpy(c1["masked"]).to(dev)
    msk1 = [msk_src.clone() for _ in range(n_copies_lg)]
    cws1 = torch.empty(bd.bd_confidence_commit_workspace_size(1, sw.block_size, sw.vocab), dtype=torch.uint8,
                       device=dev)
    dec1_us, com1_us = [], []
    for rnd in range(4):
        t_us = primed([lambda i=i: bd.bd_attn_decode_block(qb1, kb1, vb1, kc1[i], vc1[i], ps1, pl1, sw.prefix_len,
                                                           o=o1, lse=lse1, workspace=ws1)
                       for i in range(n_copies_kv)])
        if rnd:
            dec1_us.extend(t_us)
        for m in msk1:
            m.copy_(msk_src)
        t_us = primed([lambda i=i: bd.bd_confidence_commit(lg1[i], tok1, msk1[i], sw.block_size, sw.threshold,
                                                           want_rows=False, workspace=cws1)
                       for i in range(n_copies_lg)])
        if rnd:
            com1_us.extend(t_us)
    dec1_us, com1_us = np.array(dec1_us), np.array(com1_us)
    # floor of a call that launches two kernels: two empty kernels back to back, timed the same way
    floor_us = []
    for rnd in range(4):
        t_us = primed([lambda: (torch.cuda._sleep(0), torch.cuda._sleep(0)) for _ in range(n_copies_lg)])
        if rnd:
            floor_us.extend(t_us)
    floor_us = np.array(floor_us)
    dec1_bytes = (sw.prefix_len + sw.block_size) * Hkv * D * 2 * 2
    com1_bytes = sw.block_size * sw.vocab * 2

    # ------------------ output projection fused with the commit: one block of 32 hidden rows
    hw = W.WORKLOADS["lmhead_block_bf16"]
    H_lm = hw.n_q_heads * hw.head_dim
    d_lm = W.lmhead_inputs(1, hw.block_size, H_lm, hw.vocab, hw.seed, boost=hw.boost)
    x_lm = to_dev(d_lm["hidden"]).view(hw.block_size, H_lm)
    w_lm = [to_dev(d_lm["weight"]).view(hw.vocab, H_lm) for _ in range(2)]
    del d_lm
    wt_lm = [w.t().contiguous() for w in w_lm]      # [H, V] for the library GEMM of the unfused path
    tok_lm = torch.full((hw.block_size,), -1, dtype=torch.int32, device=dev)
    msk_lm = torch.ones(hw.block_size, dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(bd.bd_lmhead_commit_workspace_size(1, hw.block_size, hw.vocab), dtype=torch.uint8,
                        device=dev)
    lg_lm = torch.empty((hw.block_size, hw.vocab), dtype=torch.bfloat16, device=dev)
    cws_lm = torch.empty(bd.bd_confidence_commit_workspace_size(1, hw.block_size, hw.vocab), dtype=torch.uint8,
                         device=dev)

    # A threshold above 1 without fallback commits nothing, so every call does the same work.
    def lm_fused(i):
        bd.bd_lmhead_commit(x_lm, w_lm[i % 2], tok_lm, msk_lm, hw.block_size, 2.0, fallback=bd.BD_FALLBACK_NONE,
                            want_rows=False, workspace=ws_lm)

    def lm_unfused(i):   # library GEMM to bf16 logits, then the commit kernels
        torch.mm(x_lm, wt_lm[i % 2], out=lg_lm)
        bd.bd_confidence_commit(lg_lm, tok_lm, msk_lm, hw.block_size, 2.0, fallback=bd.BD_FALLBACK_NONE,
                                want_rows=False, workspace=cws_lm)

    lm_us, un_us = [], []
    for rnd in range(4):
        t_us = primed([lambda i=i: lm_fused(i) for i in range(8)], n_launch_us=150.0)
        if rnd:
            lm_us.extend(t_us)
        t_us = primed([lambda i=i: lm_unfused(i) for i in range(8)], n_launch_us=150.0)
        if rnd:
            un_us.extend(t_us)
    lm_us, un_us = np.array(lm_us), np.array(un_us)
    lm_bytes = (hw.vocab + hw.block_size) * H_lm * 2

    # ------------------------------- forward at the first training length (12288 tokens)
    w3 = W.WORKLOADS["fwd_L12288_bf16"]
    inp3 = W.attention_inputs(w3.batch, w3.seqlen, w3.n_q_heads, w3.n_kv_heads, w3.head_dim, "bf16", w3.seed)
    q3, k3, v3 = (to_dev(inp3[n]) for n in ("q", "k", "v"))
    del inp3
    o3 = torch.empty_like(q3)
    lse3 = torch.empty((w3.batch, w3.n_q_heads, w3.seqlen), dtype=torch.float32, device=dev)
    nb3 = w3.seqlen // w3.block_size
    f3_flops = 4.0 * w3.head_dim * w3.block_size ** 2 * nb3 * (nb3 + 1) / 2 * w3.n_q_heads * w3.batch
    for _ in range(5):
        bd.bd_attn_fwd(q3, k3, v3, w3.block_size, o=o3, lse=lse3)
    f3_ev = [(ev(), ev()) for _ in range(30)]
    for a, b_ in f3_ev:
        a.record()
        bd.bd_attn_fwd(q3, k3, v3, w3.block_size, o=o3, lse=lse3)
        b_.record()
    torch.cuda.synchronize()
    f3_ms = np.array([a.elapsed_time(b_) for a, b_ in f3_ev])
    del q3, k3, v3, o3, lse3

    # --------------- the tiny fp32 workload: one forward and one commit step, GPU time per launch
    w1 = W.WORKLOADS["tiny_f32"]
    inp1 = W.attention_inputs(w1.batch, w1.seqlen, w1.n_q_heads, w1.n_kv_heads, w1.head_dim, "f32", w1.seed)
    q1t, k1t, v1t = (torch.from_numpy(np.ascontiguousarray(inp1[n], dtype=np.float32)).to(dev) for n in ("q", "k", "v"))
    o1t = torch.empty_like(q1t)
    lse1t = torch.empty((w1.batch, w1.n_q_heads, w1.seqlen), dtype=torch.float32, device=dev)
    ct1 = W.commit_inputs(1, w1.block_size, w1.vocab, "f32", w1.seed, masked_frac=w1.masked_frac,
                          logit_std=w1.logit_std)
    lg1t = torch.from_numpy(np.ascontiguousarray(ct1["logits"], dtype=np.float32)).to(dev)
    n_tiny = 40      # one token state per commit launch, so every launch sees the same masked rows
    tok1t = [torch.from_numpy(ct1["tokens"].copy()).to(dev) for _ in range(n_tiny)]
    msk1t = [torch.from_numpy(ct1["masked"].copy()).to(dev) for _ in range(n_tiny)]
    cws1t = torch.empty(bd.bd_confidence_commit_workspace_size(1, w1.block_size, w1.vocab), dtype=torch.uint8,
                        device=dev)
    tok0t, msk0t = tok1t[0].clone(), msk1t[0].clone()
    conf1t = torch.empty(w1.block_size, dtype=torch.float32, device=dev)
    pred1t = torch.empty(w1.block_size, dtype=torch.int32, device=dev)
    ncom1t = torch.empty(1, dtype=torch.int32, device=dev)
    nleft1t = torch.empty(1, dtype=torch.int32, device=dev)
    tiny_fwd_us, tiny_com_us = [], []
    for rnd in range(3):   # the first round warms up and is not kept
        t_us = primed([lambda: bd.bd_attn_fwd(q1t, k1t, v1t, w1.block_size, o=o1t, lse=lse1t)] * n_tiny)
        for t_, m_ in zip(tok1t, msk1t):
            t_.copy_(tok0t)
            m_.copy_(msk0t)
        c_us = primed([lambda i=i: bd.bd_confidence_commit(lg1t, tok1t[i], msk1t[i], w1.block_size, w1.threshold,
                                                           conf=conf1t, pred=pred1t, n_committed=ncom1t,
                                                           n_masked_left=nleft1t, workspace=cws1t)
                       for i in range(n_tiny)])
        if rnd:
            tiny_fwd_us.extend(t_us)
            tiny_com_us.extend(c_us)
    del q1t, k1t, v1t, o1t, lse1t, lg1t, tok1t, msk1t

    # --------------------------------------------------------- CPU oracle sample
    cpu = None
    if not args.no_cpu:
        # the first loop step's inputs and the GPU's commit of it, for 4 of the 64 sequences
        sample_seqs = [0, 16, 32, 48]
        masked.fill_(1)
        tokens.fill_(-1)
        bd.bd_confidence_commit(logit_pool[0], tokens, masked, lw.block_size, 0.95, conf=conf, pred=pred,
                                n_committed=ncom, n_masked_left=nleft, workspace=com_ws)
        torch.cuda.synchronize()
        rows = np.concatenate([np.arange(s_ * lw.block_size, (s_ + 1) * lw.block_size) for s_ in sample_seqs])
        rows_t = torch.from_numpy(rows).to(dev)
        ps_np, pl_np = ps.cpu().numpy(), pl.cpu().numpy()

        def host_bits(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        loop_sample = {
            "seqs": sample_seqs,
            "q_blk": host_bits(qb[sample_seqs]), "k_blk": host_bits(kb[sample_seqs]), "v_blk": host_bits(vb[sample_seqs]),
            "k_cache": [host_bits(kc[int(ps_np[s_]):int(ps_np[s_]) + int(pl_np[s_])]) for s_ in sample_seqs],
            "v_cache": [host_bits(vc[int(ps_np[s_]):int(ps_np[s_]) + int(pl_np[s_])]) for s_ in sample_seqs],
            "logits": host_bits(logit_pool[0][rows_t]),
            "gpu_conf": conf[rows_t].cpu().numpy(), "gpu_pred": pred[rows_t].cpu().numpy(),
            "n_seq": lw.n_seq, "thresholds": lw.thresholds,
        }
        cfg2 = {"decode": d1, "logits": c1["logits"], "threshold": sw.threshold}
        cpu = cpu_baseline(wl, args.cpu_seconds, cfg2, loop_sample)

    ms_per_step = wall / args.steps * 1e3
    line = {
        "metric": "block-causal attn TFLOP/s (%MFMA peak) at L=16384; decode steps/s; commit GB/s",
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/dO; boosted N(0,1) logits)",
        "config": {"workload": "fwdbwd_L16384_bf16 + decode_loop_bf16 step", "batch": B, "seq_len": L,
                   "block_size": blk, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "decode_seqs": lw.n_seq, "vocab": V},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("attn_fwd_bf16_d128"), "traffic_unit": "HBM bytes per launch",
                     "kernel": "attn_fwd_bf16_d128", "flops_per_launch": fwd_flops,
                     "avg_launch_ms": round(fwd_avg, 4)},
        "cpu_baseline": cpu,
        "fwd": {"TFLOPs": round(fwd_tflops, 2), "ms_mean": round(fwd_avg, 4), "ms_min": round(min(fwd_ms), 4),
                "frac_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4)},
        "bwd": ({"TFLOPs_2.5x": round(bwd_flops / (np.mean(bwd_ms) * 1e-3) / 1e12, 2),
                 "ms_mean": round(float(np.mean(bwd_ms)), 4)} if have_bwd else None),
        "decode_loop": {"kv_GB_per_step": round(kv_bytes_loop / 1e9, 3),
                        "attn_us_median": round(float(np.median(dec_ms)) * 1e3, 1),
                        "attn_GBps": round(kv_bytes_loop / (np.median(dec_ms) * 1e-3) / 1e9, 1),
                        "attn_paged256_us_median": round(float(np.median(pg_us)), 1),
                        "attn_paged256_GBps": round(kv_bytes_loop / (np.median(pg_us) * 1e-6) / 1e9, 1),
                        "commit_GBps_first_step": round(com_gbs_loop[0], 1),
                        "commit_GBps_median": round(float(np.median(com_gbs_loop)), 1),
                        "commit_rowwise_GBps_first_step": round(rw_bytes / (np.median(rw_us) * 1e-6) / 1e9, 1),
                        "commit_sampled_GBps_first_step": round(rw_bytes / (np.median(sm_us) * 1e-6) / 1e9, 1),
                        "commit_sampled_topk50_GBps_first_step":
                            round(rw_bytes / (np.median(tr_us[(50, 1.0)]) * 1e-6) / 1e9, 1),
                        "commit_sampled_topp0.9_GBps_first_step":
                            round(rw_bytes / (np.median(tr_us[(0, 0.9)]) * 1e-6) / 1e9, 1),
                        "by_threshold": loops, "by_threshold_graph_replay": loops_graph},
        "launch_floor_two_empty_kernels_us": {"us_median": round(float(np.median(floor_us)), 2),
                                              "us_p10": round(float(np.percentile(floor_us, 10)), 2),
                                              "us_p90": round(float(np.percentile(floor_us, 90)), 2)},
        "decode_step_4096": {"bytes": dec1_bytes, "us_median": round(float(np.median(dec1_us)), 2),
                             "us_p10": round(float(np.percentile(dec1_us, 10)), 2),
                             "us_p90": round(float(np.percentile(dec1_us, 90)), 2),
                             "GBps": round(dec1_bytes / (np.median(dec1_us) * 1e-6) / 1e9, 1)},
        "lmhead_commit_32x2048x151936": {"bytes": lm_bytes, "us_median": round(float(np.median(lm_us)), 2),
                                         "us_p10": round(float(np.percentile(lm_us, 10)), 2),
                                         "us_p90": round(float(np.percentile(lm_us, 90)), 2),
                                         "GBps": round(lm_bytes / (np.median(lm_us) * 1e-6) / 1e9, 1),
                                         "unfused_us_median": round(float(np.median(un_us)), 2),
                                         "speedup_vs_unfused": round(float(np.median(un_us) / np.median(lm_us)), 3)},
        "fwd_L12288": {"flops": f3_flops, "ms_median": round(float(np.median(f3_ms)), 4),
                       "ms_p10": round(float(np.percentile(f3_ms, 10)), 4),
                       "ms_p90": round(float(np.percentile(f3_ms, 90)), 4),
                       "TFLOPs": round(f3_flops / (np.median(f3_ms) * 1e-3) / 1e12, 2),
                       "frac_peak": round(f3_flops / (np.median(f3_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "commit_32x151936": {"bytes": com1_bytes, "us_median": round(float(np.median(com1_us)), 2),
                             "us_p10": round(float(np.percentile(com1_us, 10)), 2),
                             "us_p90": round(float(np.percentile(com1_us, 90)), 2),
                             "GBps": round(com1_bytes / (np.median(com1_us) * 1e-6) / 1e9, 1)},
        "tiny_f32_latency": {"fwd_us_median": round(float(np.median(tiny_fwd_us)), 2),
                             "commit_us_median": round(float(np.median(tiny_com_us)), 2)},
    }
    print(json.dumps(line), flush=True)


KERNEL_SRC = os.path.join(ROOT, "block_diffusion_decoding_amd", "csrc")
REF_COPY_KERNEL = "bitwise_not_kernel"     # the counter-scale reference kernel of the traffic probe
REF_COPY_BYTES = 1 << 30
SIMD_NUM = 256 * 4                          # MI355X: 256 compute units of 4 SIMDs
N_XCD = 8                                   # ... in 8 XCDs
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """Hash of every kernel source: counter profiles are valid only for the sources they ran."""
    import hashlib
    h = hashlib.sha1()
    for name in sorted(os.listdir(KERNEL_SRC)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(KERNEL_SRC, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:12]


def measured_traffic(kernel: str):
    """HBM bytes (read + written) per launch of `kernel` from the committed counter profile, or None
    if there is none for the current kernel sources."""
    path = os.path.join(PROFILES, "hbm_traffic_hot_path_kernels.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash()
    for ln in open(path):
        parts = ln.split()
        if len(parts) >= 5 and parts[0] == "traffic" and parts[1] == kernel and parts[4] == f"src={want}":
            return int(float(parts[2]) + float(parts[3]))
    return None


def _short(name: str) -> str:
    n = name
    for pre in ("void ", "bd::(anonymous namespace)::", "at::native::(anonymous namespace)::", "at::native::"):
        n = n.replace(pre, "")
    return n.split("(")[0].replace(" ", "")[:60]


def summarize(args):
    """Write a short text summary of rocprofv3 result databases (kernel trace or counters)."""
    import sqlite3
    out = [f"# {args.title}".rstrip(), f"# command: {args.command}", f"# kernel sources: src={kernel_source_hash()}", ""]
    pmc, trace_us = {}, {}
    for dbp in args.summarize:
        db = sqlite3.connect(dbp)
        cur = db.cursor()
        rows = cur.execute("select count(*) from counters_collection").fetchone()[0]
        if rows:
            for kname, cname, n, avg in cur.execute(
                    "select kernel_name, counter_name, count(*), avg(value) from counters_collection "
                    "group by kernel_name, counter_name"):
                pmc.setdefault(_short(kname), {})[cname] = (n, avg)
        else:
            for kname, n, avg in cur.execute("select name, count(*), avg(end-start) from kernels group by name"):
                trace_us[_short(kname)] = avg / 1e3
            out.append(f"## kernel trace: {os.path.basename(dbp)} (one line per kernel and grid size)")
            out.append(f"{'kernel':60s} {'grid':>10s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
                       f"{'total_ms':>10s}")
            for kname, grid, n, avg, mn, mx, tot in cur.execute(
                    "select name, grid_x, count(*), avg(end-start), min(end-start), max(end-start), sum(end-start) "
                    "from kernels group by name, grid_x order by sum(end-start) desc limit 30"):
                out.append(f"{_short(kname):60s} {grid:10d} {n:6d} {avg / 1e3:10.2f} {mn / 1e3:10.2f} {mx / 1e3:10.2f} "
                           f"{tot / 1e6:10.3f}")
            out.append("")
    if pmc:
        names = sorted({c for d in pmc.values() for c in d})
        out.append("## counters (average per dispatch)")
        out.append(f"{'kernel':60s} " + " ".join(f"{c:>26s}" for c in names))
        for kname, d in sorted(pmc.items()):
            if not kname:
                continue
            out.append(f"{kname:60s} " + " ".join(f"{d[c][1]:26.6g}" if c in d else f"{'-':>26s}" for c in names))
        mf = [(k, d) for k, d in sorted(pmc.items()) if k and ("SQ_VALU_MFMA_BUSY_CYCLES" in d
                                                                or "SQ_INSTS_VALU_MFMA_MOPS_BF16" in d)]
        if mf:
            out.append("")
            out.append(f"## matrix-core use per dispatch; busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the "
                       f"{SIMD_NUM} SIMDs) / (SIMDs x active cycles), active cycles = GRBM_GUI_ACTIVE / {N_XCD} "
                       "(the counter comes back summed over the XCDs; rocprofv3's MfmaUtil takes their maximum); "
                       "bf16 flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; avg_us from the kernel trace of the same "
                       "program (another run), clk = active cycles / avg_us")
            out.append(f"{'kernel':40s} {'mfma_busy':>10s} {'cycles/XCD':>12s} {'avg_us':>10s} {'clk_MHz':>9s} "
                       f"{'bf16_TFLOP':>11s} {'TFLOP/s':>9s} {'lds_confl/inst':>15s}")
            for kname, d in mf:
                busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", (0, None))[1]
                gui = d.get("GRBM_GUI_ACTIVE", (0, None))[1]
                gui = gui / N_XCD if gui is not None else None
                mops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", (0, None))[1]
                lds = d.get("SQ_INSTS_LDS", (0, None))[1]
                confl = d.get("SQ_LDS_BANK_CONFLICT", (0, None))[1]
                us = trace_us.get(kname)
                util = busy / (gui * SIMD_NUM) if busy is not None and gui else None
                tfl = mops * 512 / 1e12 if mops is not None else None

                def fmt(x, w, f):
                    return f"{x:{w}{f}}" if x is not None else f"{'-':>{w}s}"
                out.append(f"{kname[:40]:40s} {fmt(util, 10, '.4f')} {fmt(gui, 12, '.0f')} {fmt(us, 10, '.2f')} "
                           f"{fmt(gui / us if gui and us else None, 9, '.0f')} {fmt(tfl, 11, '.4f')} "
                           f"{fmt(tfl / (us * 1e-6) if tfl is not None and us else None, 9, '.1f')} "
                           f"{fmt(confl / lds if confl is not None and lds else None, 15, '.4f')}")
        copy = next((d for k, d in pmc.items() if REF_COPY_KERNEL in k), None)
        if copy and "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
            ref_kib = REF_COPY_BYTES / 1024.0
            ff, fw = ref_kib / copy["FETCH_SIZE"][1], ref_kib / copy["WRITE_SIZE"][1]
            out.append("")
            out.append(f"## HBM bytes per launch; counter scale from the reference kernel ({REF_COPY_KERNEL}, "
                       f"{REF_COPY_BYTES} bytes read and written): FETCH x{ff:.3f}, WRITE x{fw:.3f}")
            out.append("# traffic <kernel> <read_bytes> <written_bytes> src=<kernel source hash>")
            for kname, d in sorted(pmc.items()):
                if "FETCH_SIZE" in d and "WRITE_SIZE" in d and REF_COPY_KERNEL not in kname and kname:
                    out.append(f"traffic {kname} {d['FETCH_SIZE'][1] * 1024 * ff:.0f} {d['WRITE_SIZE'][1] * 1024 * fw:.0f} "
                               f"src={kernel_source_hash()}")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def cpu_baseline(wl, budget_s: float, cfg2: dict, loop_sample: dict):
    """The oracle, as it stands, on bounded samples of the same workloads.

    Headline: the oracle forward on whole (batch, head) pairs of the 16384-token workload, one
    after another until the time budget is spent (TFLOP/s on the allowed pairs).  Beside it:
    the 4096-prefix decode step and its 32-row commit in full (GB/s of the same algorithmic
    bytes as the GPU figures), the backward on the last 1024 tokens of one (batch, KV head)
    group of the 16384-token workload (TFLOP/s, 2.5x count), and one step of the 64-sequence loop
    on 4 of its sequences (block attention + commit; steps/s scaled to 64 sequences).  The
    oracle commit of those 128 first-step rows also gives the near-T accounting of the loop's
    first step (rows whose confidence lies within 1e-4 of each T) and a spot check of the GPU's
    ids and confidences on them."""
    import workloads as W
    from oracle import attention as OA
    from oracle import commit as OC
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    rng = np.random.default_rng(wl.seed)
    L, D, blk = wl.seqlen, wl.head_dim, wl.block_size

    def draw(heads=1):
        x = rng.standard_normal((1, L, heads, D), dtype=np.float32)
        return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)).astype(np.float64)

    def f64(bits):
        return W.bf16_bits_to_f32(bits).astype(np.float64)

    flops_pair = OA.attn_flops(L, blk, 1, D)
    done, pairs = 0.0, 0
    t_work = 0.0
    while pairs < wl.batch * wl.n_q_heads and (t_work < budget_s or pairs == 0):
        q, k, v = draw(), draw(), draw()
        t0 = time.perf_counter()
        OA.attn_fwd(q, k, v, blk)
        t_work += time.perf_counter() - t0
        done += flops_pair
        pairs += 1
    legs = {}

    # the 4096-prefix decode step and the commit of its [32 x 151936] logits, in full
    d = cfg2["decode"]
    Hkv, Dd = d["k_blk"].shape[2], d["k_blk"].shape[3]
    P = int(d["prefix_len"][0])
    args_ = [f64(d[n]) for n in ("q_blk", "k_blk", "v_blk", "k_cache", "v_cache")]
    t0 = time.perf_counter()
    OA.decode_block(*args_, d["prefix_start"], d["prefix_len"])
    t_dec = time.perf_counter() - t0
    dec_bytes = (P + d["k_blk"].shape[1]) * Hkv * Dd * 2 * 2
    lg = W.bf16_bits_to_f32(cfg2["logits"])
    R = lg.shape[0]
    t0 = time.perf_counter()
    OC.confidence_commit(lg, np.full(R, -1, np.int32), np.ones(R, np.uint8), R, cfg2["threshold"])
    t_com = time.perf_counter() - t0
    legs["decode_step_4096"] = {"GBps": round(dec_bytes / t_dec / 1e9, 4), "s": round(t_dec, 3)}

    # the tiny fp32 workload in full: block attention over 128 tokens and one commit step
    w1 = W.WORKLOADS["tiny_f32"]
    i1 = W.attention_inputs(w1.batch, w1.seqlen, w1.n_q_heads, w1.n_kv_heads, w1.head_dim, "f32", w1.seed)
    c1 = W.commit_inputs(1, w1.block_size, w1.vocab, "f32", w1.seed, masked_frac=w1.masked_frac,
                         logit_std=w1.logit_std)
    t0 = time.perf_counter()
    OA.attn_fwd(*(np.asarray(i1[n], np.float64) for n in ("q", "k", "v")), w1.block_size)
    t_tf = time.perf_counter() - t0
    t0 = time.perf_counter()
    OC.confidence_commit(np.asarray(c1["logits"], np.float64), c1["tokens"], c1["masked"], w1.block_size,
                         w1.threshold)
    t_tc = time.perf_counter() - t0
    legs["tiny_f32"] = {"fwd_us": round(t_tf * 1e6, 1), "commit_us": round(t_tc * 1e6, 1)}
    legs["commit_32x151936"] = {"GBps": round(lg.size * 2 / t_com / 1e9, 4), "s": round(t_com, 3)}

    # backward on the last 1024 tokens of one group (2 query heads sharing one KV head)
    G = wl.n_q_heads // wl.n_kv_heads
    q, do = draw(G), draw(G)
    k, v = draw(), draw()
    qb0 = (L - 1024) // blk
    t0 = time.perf_counter()
    OA.attn_bwd(q, k, v, do, blk, q_block_start=qb0)
    t_bwd = time.perf_counter() - t0
    slice_pairs = sum(blk * min(L, (b + 1) * blk) for b in range(qb0, L // blk))
    bwd_flops = 2.5 * 4.0 * D * slice_pairs * G
    legs["bwd_last1024_one_group"] = {"TFLOPs_2.5x": round(bwd_flops / t_bwd / 1e12, 5), "s": round(t_bwd, 3)}

    # one loop step on 4 of the 64 sequences: block attention against each prefix, then the commit
    ls = loop_sample
    n4 = len(ls["seqs"])
    plen = np.array([c.shape[0] for c in ls["k_cache"]], np.int64)
    pstart = np.concatenate([[0], np.cumsum(plen)[:-1]])
    kcache = np.concatenate([f64(c) for c in ls["k_cache"]])
    vcache = np.concatenate([f64(c) for c in ls["v_cache"]])
    qs, ks, vs = f64(ls["q_blk"]), f64(ls["k_blk"]), f64(ls["v_blk"])
    lg = W.bf16_bits_to_f32(ls["logits"])
    Rs = lg.shape[0]
    t0 = time.perf_counter()
    OA.decode_block(qs, ks, vs, kcache, vcache, pstart, plen)
    ref = OC.confidence_commit(lg, np.full(Rs, -1, np.int32), np.ones(Rs, np.uint8), Rs // n4, 0.95)
    t_step = time.perf_counter() - t0
    legs["loop_step_4_of_64_seqs"] = {"steps_per_s_scaled_to_64": round(n4 / (ls["n_seq"] * t_step), 4),
                                      "s": round(t_step, 3)}
    # near-T accounting and spot check of the GPU's first-step commit on these rows
    c = ref["conf"]
    near = {str(T): int((np.abs(c - T) <= 1e-4).sum()) for T in ls["thresholds"]}
    valid = ~np.isnan(c)
    rel = float(np.max(np.abs(ls["gpu_conf"][valid] - c[valid]) / c[valid])) if valid.any() else 0.0
    check = {"rows": int(Rs), "band": 1e-4, "near_T_rows": near,
             "pred_equal": bool(np.array_equal(ls["gpu_pred"], ref["pred"])), "conf_max_rel_err": rel}
    return {"value": round(done / t_work / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 oracle forward over {pairs} of the {wl.batch * wl.n_q_heads} (batch, head) "
                      f"pairs of the {L}-token workload ({done / 1e9:.0f} GFLOP in {t_work:.1f} s)",
            "legs": legs, "first_loop_step_check": check}


if __name__ == "__main__":
    main()
