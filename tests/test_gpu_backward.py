"""GPU parity of bd_attn_bwd against the oracle.

The GPU runs its own forward and then the backward (the chain a training step
uses); the oracle recomputes O from the definition.  Tolerance on dQ, dK, dV:
max-abs <= tol * max(1, max|ref|) with tol = 2e-2 for bf16 (as for the forward
output) and 2e-5 for fp32 (fp32 sums of up to L products, each within a few
ulp).  The 2 x 16384-token workload runs in full on the GPU and is compared on
its last 1024 tokens (dK/dV of those keys depend only on queries in the slice,
and dQ of those queries sees every key) and, for one (batch, KV head) group, on
every key and query: the first keys' dK/dV sum over all 16384 queries of both
query heads of the group, the longest accumulation chains of the kernel.
"""
import numpy as np
import pytest
import torch

import block_diffusion_decoding_amd as bd
import workloads as W
from oracle import attention as OA
from gpu_util import banner, dev, host_vals, to_np

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 2e-5}


def gpu_fwd_bwd(inp, dtype, blk, scale=0.0):
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = bd.bd_attn_fwd(q, k, v, block_size=blk, softmax_scale=scale)
    dq, dk, dv = bd.bd_attn_bwd(q, k, v, o, lse, do, block_size=blk, softmax_scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(name, got, ref, dtype):
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    lim = TOL[dtype] * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    rel = float(np.linalg.norm(got - ref) / max(1e-30, np.linalg.norm(ref)))
    print(f"  {name}: max|err|={err:.3e} (limit {lim:.3e}) rel-L2={rel:.3e}")
    assert err <= lim, (name, err, lim)


def check(inp, dtype, blk, grads, q_block_start=0, batches=None, scale=None):
    f = {n: host_vals(inp[n], dtype) for n in ("q", "k", "v", "do")}
    rq, rk, rv = OA.attn_bwd(f["q"], f["k"], f["v"], f["do"], blk, scale, q_block_start=q_block_start,
                             batches=batches)
    s0 = q_block_start * blk
    bsel = slice(None) if batches is None else batches
    for name, g, r in (("dq", grads[0], rq), ("dk", grads[1], rk), ("dv", grads[2], rv)):
        compare(name, to_np(g)[bsel, s0:], r[bsel], dtype)


@pytest.mark.parametrize("B,L,Hq,Hkv,blk", [
    (2, 300, 4, 2, 32),
    (1, 256, 2, 1, 32),
    (1, 200, 2, 2, 1),
    (1, 200, 2, 1, 200),
    (1, 333, 4, 1, 48),
    (1, 1, 1, 1, 32),
    (1, 130, 2, 2, 7),
    # dK/dV and dQ items counts divisible by 8: both run in one launch
    (2, 1000, 8, 2, 32),     # 32 dK/dV and 64 dQ items, ragged last tiles
    (1, 512, 16, 8, 48),     # 32 of each, block not dividing the tiles
    (2, 512, 16, 8, 32),     # two (batch, KV head) groups per XCD list, interleaved
    (1, 300, 16, 1, 32),     # sixteen query heads per KV head (multi-query)
])
def test_bf16_shapes(B, L, Hq, Hkv, blk):
    banner(f"bwd bf16 B={B} L={L} Hq={Hq} Hkv={Hkv} blk={blk}")
    inp = W.attention_inputs(B, L, Hq, Hkv, 128, "bf16", seed=7 * L + blk, with_grad=True)
    check(inp, "bf16", blk, gpu_fwd_bwd(inp, "bf16", blk))


@pytest.mark.parametrize("L", [384, 512])   # 512: dK/dV and dQ in one launch
def test_bf16_scale_and_determinism(L):
    banner(f"bwd bf16 custom scale, determinism, L={L}")
    inp = W.attention_inputs(1, L, 4, 2, 128, "bf16", seed=5, with_grad=True)
    g1 = gpu_fwd_bwd(inp, "bf16", 32, scale=0.3)
    check(inp, "bf16", 32, g1, scale=0.3)
    g2 = gpu_fwd_bwd(inp, "bf16", 32, scale=0.3)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,L,Hq,Hkv,d,blk", [(1, 128, 1, 1, 64, 32), (2, 70, 4, 2, 32, 8), (1, 40, 2, 1, 128, 1)])
def test_f32_shapes(B, L, Hq, Hkv, d, blk):
    banner(f"bwd f32 B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} blk={blk}")
    inp = W.attention_inputs(B, L, Hq, Hkv, d, "f32", seed=L + d, with_grad=True)
    check(inp, "f32", blk, gpu_fwd_bwd(inp, "f32", blk))


def test_full_size_workload_last_1024_tokens():
    wl = W.WORKLOADS["fwdbwd_L16384_bf16"]
    banner("bwd fwdbwd_L16384_bf16 full size, last 1024 tokens")
    inp = W.attention_inputs(wl.batch, wl.seqlen, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.seed,
                             with_grad=True)
    grads = gpu_fwd_bwd(inp, "bf16", wl.block_size)
    for g in grads:
        assert torch.isfinite(g.float()).all()
    check(inp, "bf16", wl.block_size, grads, q_block_start=(wl.seqlen - 1024) // wl.block_size)
    # one whole group: batch 1, KV head 5 and its query heads 10, 11, all keys and queries
    b, g = 1, 5
    G = wl.n_q_heads // wl.n_kv_heads
    hs = slice(g * G, (g + 1) * G)
    f = {n: host_vals(inp[n][b:b + 1, :, hs if n in ("q", "do") else slice(g, g + 1)], "bf16")
         for n in ("q", "k", "v", "do")}
    rq, rk, rv = OA.attn_bwd(f["q"], f["k"], f["v"], f["do"], wl.block_size)
    compare("dk group (all keys)", to_np(grads[1])[b:b + 1, :, g:g + 1], rk, "bf16")
    compare("dv group (all keys)", to_np(grads[2])[b:b + 1, :, g:g + 1], rv, "bf16")
    compare("dk keys [0, 1024)", to_np(grads[1])[b:b + 1, :1024, g:g + 1], rk[:, :1024], "bf16")
    compare("dv keys [0, 1024)", to_np(grads[2])[b:b + 1, :1024, g:g + 1], rv[:, :1024], "bf16")
    compare("dq group (all queries)", to_np(grads[0])[b:b + 1, :, hs], rq, "bf16")
