"""GPU parity of bd_attn_fwd and bd_attn_decode_block against the oracle.

Tolerances: O max-abs 2e-2 (bf16) / 1e-5 (fp32); LSE 1e-3 (bf16) / 1e-5 (fp32).
Small cases are compared element by element; the 12288- and 16384-token
workloads run in full on the GPU and are compared on sampled query blocks (all
their rows, several heads and both batch entries), which the oracle computes
one block at a time.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import attention as OA
from gpu_util import banner, dev, host_vals, to_np

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}


def gpu_fwd(inp, dtype, blk, scale=0.0):
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = bd.bd_attn_fwd(q, k, v, block_size=blk, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def check_fwd(inp, dtype, blk, o, lse, q_blocks=None, heads=None, batches=None, scale=None):
    qf, kf, vf = (host_vals(inp[n], dtype) for n in ("q", "k", "v"))
    ro, rl = OA.attn_fwd(qf, kf, vf, blk, scale, q_blocks=q_blocks, heads=heads, batches=batches)
    go, gl = to_np(o), to_np(lse)
    sel = ~np.isnan(ro)
    sel_l = ~np.isnan(rl)
    eo = np.max(np.abs(go[sel] - ro[sel]))
    el = np.max(np.abs(gl[sel_l] - rl[sel_l]))
    to, tl = TOL[dtype]
    print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= to and el <= tl, (eo, el)


def test_tiny_f32_workload():
    wl = W.WORKLOADS["tiny_f32"]
    banner("fwd tiny_f32")
    inp = W.attention_inputs(1, wl.seqlen, 1, 1, wl.head_dim, "f32", wl.seed)
    o, lse = gpu_fwd(inp, "f32", wl.block_size)
    check_fwd(inp, "f32", wl.block_size, o, lse)


@pytest.mark.parametrize("B,L,Hq,Hkv,d,blk", [(2, 300, 4, 2, 64, 32), (1, 77, 2, 2, 128, 5), (1, 50, 3, 1, 100, 1)])
def test_f32_shapes(B, L, Hq, Hkv, d, blk):
    banner(f"fwd f32 B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} blk={blk}")
    inp = W.attention_inputs(B, L, Hq, Hkv, d, "f32", seed=L)
    o, lse = gpu_fwd(inp, "f32", blk)
    check_fwd(inp, "f32", blk, o, lse)


@pytest.mark.parametrize("B,L,Hq,Hkv,blk", [
    (2, 300, 4, 2, 32),      # several 128-row tiles, ragged tail
    (1, 512, 2, 1, 32),      # aligned
    (1, 200, 2, 2, 1),       # block size 1: causal
    (1, 200, 2, 1, 200),     # block size L: full attention
    (1, 333, 4, 1, 48),      # block not dividing the 64-key tile
    (1, 1, 1, 1, 32),        # single token
    (1, 130, 2, 2, 7),
    (1, 300, 16, 1, 32),     # sixteen query heads per KV head (multi-query)
])
def test_bf16_shapes(B, L, Hq, Hkv, blk):
    banner(f"fwd bf16 B={B} L={L} Hq={Hq} Hkv={Hkv} blk={blk}")
    inp = W.attention_inputs(B, L, Hq, Hkv, 128, "bf16", seed=L + blk)
    o, lse = gpu_fwd(inp, "bf16", blk)
    check_fwd(inp, "bf16", blk, o, lse)


def test_bf16_many_query_heads():
    # ten query heads per KV head (320 query tiles, more than one per compute
    # unit), a ragged last tile and a block size that does not divide the
    # 64-key tile; every row is compared, and a second call is bit-identical
    banner("fwd bf16 B=1 L=1000 Hq=80 Hkv=8 blk=48")
    inp = W.attention_inputs(1, 1000, 80, 8, 128, "bf16", seed=77)
    o, lse = gpu_fwd(inp, "bf16", 48)
    check_fwd(inp, "bf16", 48, o, lse)
    o2, lse2 = gpu_fwd(inp, "bf16", 48)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_bf16_custom_scale():
    banner("fwd bf16 scale 0.2")
    inp = W.attention_inputs(1, 256, 2, 1, 128, "bf16", seed=3)
    o, lse = gpu_fwd(inp, "bf16", 32, scale=0.2)
    check_fwd(inp, "bf16", 32, o, lse, scale=0.2)


def test_bf16_future_blocks_bitwise_invisible():
    banner("fwd bf16 future-block invariance")
    inp = W.attention_inputs(1, 384, 2, 1, 128, "bf16", seed=9)
    o1, l1 = gpu_fwd(inp, "bf16", 32)
    cut = 160
    inp2 = {k: v.copy() for k, v in inp.items()}
    rng = np.random.default_rng(10)
    for name in ("q", "k", "v"):
        inp2[name][:, cut:] = W.f32_to_bf16_bits(rng.standard_normal(inp2[name][:, cut:].shape).astype(np.float32) * 4)
    o2, l2 = gpu_fwd(inp2, "bf16", 32)
    assert torch.equal(o1[:, :cut], o2[:, :cut]) and torch.equal(l1[..., :cut], l2[..., :cut])
    assert not torch.equal(o1[:, cut:], o2[:, cut:])


def test_bf16_deterministic():
    banner("fwd bf16 determinism")
    inp = W.attention_inputs(2, 1024, 4, 2, 128, "bf16", seed=4)
    o1, l1 = gpu_fwd(inp, "bf16", 32)
    o2, l2 = gpu_fwd(inp, "bf16", 32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["fwd_L12288_bf16", "fwdbwd_L16384_bf16"])
def test_full_size_workloads_sampled(name):
    wl = W.WORKLOADS[name]
    banner(f"fwd {name} full size, sampled rows")
    inp = W.attention_inputs(wl.batch, wl.seqlen, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.seed)
    o, lse = gpu_fwd(inp, "bf16", wl.block_size)
    nblk = wl.seqlen // wl.block_size
    q_blocks = [0, 1, 2, nblk // 3, nblk // 2 + 1, nblk - 2, nblk - 1]
    check_fwd(inp, "bf16", wl.block_size, o, lse, q_blocks=q_blocks, heads=[0, 5, 15],
              batches=list(range(wl.batch)))
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


# ---------------------------------------------------------------------------
# one block against a prefix cache
# ---------------------------------------------------------------------------
def gpu_decode(d, dtype, max_p, scale=0.0):
    t = {k: dev(d[k], dtype) for k in ("q_blk", "k_blk", "v_blk")}
    kc = dev(d["k_cache"], dtype) if d["k_cache"].shape[0] else None
    vc = dev(d["v_cache"], dtype) if d["v_cache"].shape[0] else None
    ps = torch.from_numpy(d["prefix_start"]).cuda()
    pl = torch.from_numpy(d["prefix_len"]).cuda()
    o, lse = bd.bd_attn_decode_block(t["q_blk"], t["k_blk"], t["v_blk"], kc, vc, ps, pl, max_p, scale)
    torch.cuda.synchronize()
    return o, lse


def check_decode(d, dtype, o, lse, seqs=None):
    f = {k: host_vals(d[k], dtype) for k in ("q_blk", "k_blk", "v_blk")}
    seqs = range(d["q_blk"].shape[0]) if seqs is None else seqs
    go, gl = to_np(o), to_np(lse)
    eo = el = 0.0
    for s in seqs:
        a, P = int(d["prefix_start"][s]), int(d["prefix_len"][s])
        kc = host_vals(d["k_cache"][a:a + P], dtype)
        vc = host_vals(d["v_cache"][a:a + P], dtype)
        ro, rl = OA.decode_block(f["q_blk"][s:s + 1], f["k_blk"][s:s + 1], f["v_blk"][s:s + 1], kc, vc,
                                 np.zeros(1, np.int64), np.array([P], np.int32))
        eo = max(eo, np.max(np.abs(go[s] - ro[0])))
        el = max(el, np.max(np.abs(gl[s] - rl[0])))
    to, tl = TOL[dtype]
    print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= to and el <= tl, (eo, el)


def test_decode_step_workload():
    wl = W.WORKLOADS["decode_step_bf16"]
    banner("decode decode_step_bf16")
    d = W.decode_inputs(1, [wl.prefix_len], wl.block_size, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.seed)
    o, lse = gpu_decode(d, "bf16", wl.prefix_len)
    check_decode(d, "bf16", o, lse)


@pytest.mark.parametrize("plens,T,Hq,Hkv", [
    ([0, 1, 37, 64, 1000, 129], 32, 16, 8),
    ([5, 300], 8, 4, 4),         # fewer rows than a row tile
    ([70, 2], 40, 8, 2),         # rows = 160: three row tiles
    ([4096 + 5], 32, 16, 8),
    (list(range(0, 1500, 10)), 32, 16, 8),   # 150 sequences: the line scan spans several wave chunks
    ([100, 2000, 0], 32, 16, 1),  # sixteen query heads per KV head: 512 rows, eight row tiles
])
def test_decode_ragged(plens, T, Hq, Hkv):
    banner(f"decode bf16 plens={plens} T={T} Hq={Hq} Hkv={Hkv}")
    d = W.decode_inputs(len(plens), plens, T, Hq, Hkv, 128, "bf16", seed=sum(plens) + T)
    o, lse = gpu_decode(d, "bf16", max(plens))
    check_decode(d, "bf16", o, lse)
    # a looser max_prefix_len (grid sized for longer prefixes, other split plan) still matches
    o2, lse2 = gpu_decode(d, "bf16", max(plens) + 3000)
    check_decode(d, "bf16", o2, lse2)


@pytest.mark.parametrize("plens,max_p", [
    ([600, 50], 40),                 # split planned for 6 tiles, 23 run
    ([2000, 5, 900, 70, 900, 3, 900, 900, 0, 900], 900),   # one sequence past the bound
])
def test_decode_prefix_above_bound(plens, max_p):
    banner(f"decode bf16 plens={plens} max_prefix_len={max_p}")
    d = W.decode_inputs(len(plens), plens, 32, 16, 8, 128, "bf16", seed=sum(plens) + max_p)
    o, lse = gpu_decode(d, "bf16", max_p)
    check_decode(d, "bf16", o, lse)


def test_decode_matches_forward_rows():
    """Decoding block b against the first b blocks as a cache equals the forward rows of block b."""
    banner("decode bf16 == forward rows")
    L, blk = 256, 32
    inp = W.attention_inputs(1, L, 4, 2, 128, "bf16", seed=21)
    o_f, l_f = gpu_fwd(inp, "bf16", blk)
    P = L - blk
    d = {"q_blk": inp["q"][:, P:], "k_blk": inp["k"][:, P:], "v_blk": inp["v"][:, P:],
         "k_cache": inp["k"][0, :P], "v_cache": inp["v"][0, :P],
         "prefix_start": np.zeros(1, np.int64), "prefix_len": np.array([P], np.int32)}
    o_d, l_d = gpu_decode(d, "bf16", P)
    assert torch.max(torch.abs(o_d.float() - o_f[:, P:].float())) <= 2e-2
    assert torch.max(torch.abs(l_d - l_f[..., P:])) <= 1e-3


def test_decode_f32():
    banner("decode f32")
    d = W.decode_inputs(3, [0, 33, 100], 32, 4, 2, 64, "f32", seed=7)
    o, lse = gpu_decode(d, "f32", 100)
    check_decode(d, "f32", o, lse)


def test_decode_loop_workload_sampled():
    wl = W.WORKLOADS["decode_loop_bf16"]
    banner("decode decode_loop_bf16 (64 ragged sequences), sampled sequences")
    rng = np.random.default_rng(wl.seed)
    plen = W.prefix_lengths(wl.n_seq, wl.prefix_range[0], wl.prefix_range[1], rng)
    d = W.decode_inputs(wl.n_seq, plen, wl.block_size, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.seed,
                        rng=rng)
    o, lse = gpu_decode(d, "bf16", int(plen.max()))
    check_decode(d, "bf16", o, lse, seqs=[0, 1, int(np.argmax(plen)), int(np.argmin(plen)), 63])
