"""GPU parity of the paged prefix cache: bd_attn_decode_block_paged against oracle.paged (and
bit for bit against the packed-cache kernel on the same rows), bd_kv_append_block against the
oracle's append, and a decode loop that appends every finished block."""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import attention as OA
from oracle import paged as PG
from gpu_util import banner, dev, host_vals, to_np

pytestmark = pytest.mark.gpu
TOL_O, TOL_LSE = 2e-2, 1e-3


def scatter_to_pages(d, page_size, rng, spare_pages=0):
    """Pages holding the packed prefixes of d under a shuffled page table (plus spare pages per
    sequence for appends)."""
    plen = d["prefix_len"].astype(np.int64)
    n = len(plen)
    max_pages = int(max(1, (plen.max() + page_size - 1) // page_size + spare_pages))
    n_pages = n * max_pages
    table = rng.permutation(n_pages).astype(np.int32).reshape(n, max_pages)
    hkv, dim = d["k_cache"].shape[1:] if d["k_cache"].shape[0] else d["k_blk"].shape[2:]
    kp = np.zeros((n_pages * page_size, hkv, dim), d["k_blk"].dtype)
    vp = np.zeros_like(kp)
    for s in range(n):
        a, P = int(d["prefix_start"][s]), int(plen[s])
        rows = PG.prefix_rows(table, s, P, page_size)
        kp[rows] = d["k_cache"][a:a + P]
        vp[rows] = d["v_cache"][a:a + P]
    return kp, vp, table


def run_paged(d, kp, vp, table, page_size, max_p):
    t = {k: dev(d[k], "bf16") for k in ("q_blk", "k_blk", "v_blk")}
    o, lse = bd.bd_attn_decode_block_paged(t["q_blk"], t["k_blk"], t["v_blk"], dev(kp, "bf16"), dev(vp, "bf16"),
                                           torch.from_numpy(table).cuda(), page_size,
                                           torch.from_numpy(d["prefix_len"].astype(np.int32)).cuda(), max_p)
    torch.cuda.synchronize()
    return o, lse


def check_against_oracle(d, kp, vp, table, page_size, o, lse, seqs):
    f = {k: host_vals(d[k], "bf16") for k in ("q_blk", "k_blk", "v_blk")}
    go, gl = to_np(o), to_np(lse)
    eo = el = 0.0
    for s in seqs:
        P = int(d["prefix_len"][s])
        sub = table[s:s + 1]
        kc, _ = PG.gather_prefixes(host_vals(kp, "bf16"), sub, [P], page_size)
        vc, _ = PG.gather_prefixes(host_vals(vp, "bf16"), sub, [P], page_size)
        ro, rl = OA.decode_block(f["q_blk"][s:s + 1], f["k_blk"][s:s + 1], f["v_blk"][s:s + 1], kc, vc,
                                 np.zeros(1, np.int64), np.array([P], np.int32))
        eo = max(eo, float(np.max(np.abs(go[s] - ro[0]))))
        el = max(el, float(np.max(np.abs(gl[s] - rl[0]))))
    print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


@pytest.mark.parametrize("plens,page_size", [
    ([0, 1, 31, 32, 33, 100, 257], 32),
    ([4096 + 5, 77, 640], 64),
    ([3000, 1, 2048], 256),
    (list(range(0, 1500, 10)), 128),       # 150 sequences: the line scan spans several wave chunks
])
def test_paged_decode_matches_oracle_and_packed(plens, page_size):
    banner(f"paged decode page_size={page_size} plens[:8]={plens[:8]}")
    rng = np.random.default_rng(page_size + len(plens))
    d = W.decode_inputs(len(plens), plens, 32, 16, 8, 128, "bf16", seed=sum(plens) + page_size)
    kp, vp, table = scatter_to_pages(d, page_size, rng, spare_pages=1)
    max_p = max(plens)
    o, lse = run_paged(d, kp, vp, table, page_size, max_p)
    check_against_oracle(d, kp, vp, table, page_size, o, lse, range(min(len(plens), 12)))
    # the packed kernel on the same rows gives the same bits
    t = {k: dev(d[k], "bf16") for k in ("q_blk", "k_blk", "v_blk")}
    kc = dev(d["k_cache"], "bf16") if d["k_cache"].shape[0] else None
    vc = dev(d["v_cache"], "bf16") if d["v_cache"].shape[0] else None
    o2, lse2 = bd.bd_attn_decode_block(t["q_blk"], t["k_blk"], t["v_blk"], kc, vc,
                                       torch.from_numpy(d["prefix_start"]).cuda(),
                                       torch.from_numpy(d["prefix_len"]).cuda(), max_p)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_append_matches_oracle():
    banner("kv append")
    rng = np.random.default_rng(7)
    plens = [0, 30, 64, 100, 250]
    d = W.decode_inputs(len(plens), plens, 32, 16, 8, 128, "bf16", seed=77)
    ps = 64
    kp, vp, table = scatter_to_pages(d, ps, rng, spare_pages=1)
    nml = np.array([0, 3, 0, 0, 1], np.int32)            # sequences 1 and 4 are not finished
    kp_t, vp_t = dev(kp, "bf16"), dev(vp, "bf16")
    pl_t = torch.from_numpy(d["prefix_len"].astype(np.int32)).cuda()
    bd.bd_kv_append_block(dev(d["k_blk"], "bf16"), dev(d["v_blk"], "bf16"), kp_t, vp_t,
                          torch.from_numpy(table).cuda(), ps, pl_t, n_masked_left=torch.from_numpy(nml).cuda())
    torch.cuda.synchronize()
    rk, rv, rpl = PG.append_block(kp, vp, table, d["prefix_len"], d["k_blk"], d["v_blk"], ps, n_masked_left=nml)
    assert np.array_equal(pl_t.cpu().numpy(), rpl)
    assert np.array_equal(kp_t.view(torch.int16).cpu().numpy().view(np.uint16), rk)
    assert np.array_equal(vp_t.view(torch.int16).cpu().numpy().view(np.uint16), rv)


def test_decode_loop_with_appends_is_the_forward():
    """Blocks of a 4-sequence batch decoded one after another against the paged cache, each
    appended when done: every block's output equals the forward rows of that block (digest,
    method step 3: a block sees itself and every earlier block)."""
    banner("paged decode loop = forward rows")
    rng = np.random.default_rng(11)
    n, L, blk, ps = 4, 192, 32, 64
    inp = W.attention_inputs(n, L, 16, 8, 128, "bf16", seed=5)
    q = dev(inp["q"], "bf16")
    k = dev(inp["k"], "bf16")
    v = dev(inp["v"], "bf16")
    o_ref, lse_ref = bd.bd_attn_fwd(q, k, v, blk)
    max_pages = L // ps
    table = torch.from_numpy(rng.permutation(n * max_pages).astype(np.int32).reshape(n, max_pages)).cuda()
    kp = torch.zeros((n * max_pages * ps, 8, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    pl = torch.zeros(n, dtype=torch.int32, device="cuda")
    worst = 0.0
    for b in range(L // blk):
        sl = slice(b * blk, (b + 1) * blk)
        qb, kb, vb = (t[:, sl].contiguous() for t in (q, k, v))
        o, lse = bd.bd_attn_decode_block_paged(qb, kb, vb, kp, vp, table, ps, pl, b * blk)
        torch.cuda.synchronize()
        worst = max(worst, float((o.float() - o_ref[:, sl].float()).abs().max()))
        assert torch.allclose(lse, lse_ref[:, :, sl], atol=TOL_LSE, rtol=0)
        bd.bd_kv_append_block(kb, vb, kp, vp, table, ps, pl)
    torch.cuda.synchronize()
    print(f"  max|o_paged - o_forward| = {worst:.3e}")
    assert worst <= TOL_O
    assert pl.cpu().tolist() == [L] * n
