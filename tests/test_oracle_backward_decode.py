"""Pins of the oracle's attention backward and of one block against a prefix cache (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, blk, scale):
    o, _ = A.attn_fwd(q, k, v, blk, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("L,blk,Hq,Hkv", [(10, 4, 2, 1), (8, 3, 2, 2)])
def test_backward_finite_differences(L, blk, Hq, Hkv):
    d, sc = 3, 0.7
    q, k, v = _rand((1, L, Hq, d), 1), _rand((1, L, Hkv, d), 2), _rand((1, L, Hkv, d), 3)
    do = _rand((1, L, Hq, d), 4)
    dq, dk, dv = A.attn_bwd(q, k, v, do, blk, sc)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, blk, sc)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, blk, sc)) / (2 * eps)
        rel = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(num)))
        assert rel < 1e-6, (name, rel)


@pytest.mark.parametrize("blk,causal", [(1, True), (24, False)])
def test_backward_matches_autograd_in_special_cases(blk, causal):
    """Block size 1 is causal attention, block size L is full attention: torch autograd
    through SDPA in float64 gives the reference gradients."""
    B, L, Hq, Hkv, d = 1, 24, 4, 2, 8
    q, k, v = _rand((B, L, Hq, d), 5), _rand((B, L, Hkv, d), 6), _rand((B, L, Hkv, d), 7)
    do = _rand((B, L, Hq, d), 8)
    dq, dk, dv = A.attn_bwd(q, k, v, do, blk)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).clone().requires_grad_(True)
    o = F.scaled_dot_product_attention(tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1),
                                       is_causal=causal)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    assert np.max(np.abs(tq.grad.permute(0, 2, 1, 3).numpy() - dq)) < 1e-12
    assert np.max(np.abs(tk.grad.permute(0, 2, 1, 3).numpy() - dk)) < 1e-12
    assert np.max(np.abs(tv.grad.permute(0, 2, 1, 3).numpy() - dv)) < 1e-12


def test_backward_tail_slice_equals_full():
    B, L, Hq, Hkv, d, blk = 2, 20, 4, 2, 6, 4
    q, k, v = _rand((B, L, Hq, d), 9), _rand((B, L, Hkv, d), 10), _rand((B, L, Hkv, d), 11)
    do = _rand((B, L, Hq, d), 12)
    dq, dk, dv = A.attn_bwd(q, k, v, do, blk)
    dq2, dk2, dv2 = A.attn_bwd(q, k, v, do, blk, q_block_start=3)
    assert np.max(np.abs(dq[:, 12:] - dq2)) < 1e-13
    assert np.max(np.abs(dk[:, 12:] - dk2)) < 1e-13
    assert np.max(np.abs(dv[:, 12:] - dv2)) < 1e-13


def test_backward_gqa_is_sum_over_group():
    B, L, Hq, d, blk = 1, 12, 4, 5, 4
    q, k, v = _rand((B, L, Hq, d), 13), _rand((B, L, 2, d), 14), _rand((B, L, 2, d), 15)
    do = _rand((B, L, Hq, d), 16)
    dq, dk, dv = A.attn_bwd(q, k, v, do, blk)
    dq2, dk2, dv2 = A.attn_bwd(q, np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2), do, blk)
    assert np.max(np.abs(dq - dq2)) < 1e-13
    assert np.max(np.abs(dk - (dk2[:, :, 0::2] + dk2[:, :, 1::2]))) < 1e-13
    assert np.max(np.abs(dv - (dv2[:, :, 0::2] + dv2[:, :, 1::2]))) < 1e-13


def test_decode_block_equals_forward_rows():
    """A block decoded against a block-aligned prefix gives the forward rows of that block
    of the concatenated sequence: the prefix cache reuse is exact."""
    Hq, Hkv, d, blk = 4, 2, 8, 4
    plens = [8, 0, 12]
    rng = np.random.default_rng(17)
    seqs = [rng.standard_normal((p + blk, Hq + 2 * Hkv, d)) for p in plens]
    kc = np.concatenate([s[:p, Hq:Hq + Hkv] for s, p in zip(seqs, plens)])
    vc = np.concatenate([s[:p, Hq + Hkv:] for s, p in zip(seqs, plens)])
    start = np.concatenate([[0], np.cumsum(plens)[:-1]])
    q_blk = np.stack([s[p:, :Hq] for s, p in zip(seqs, plens)])
    k_blk = np.stack([s[p:, Hq:Hq + Hkv] for s, p in zip(seqs, plens)])
    v_blk = np.stack([s[p:, Hq + Hkv:] for s, p in zip(seqs, plens)])
    o, lse = A.decode_block(q_blk, k_blk, v_blk, kc, vc, start, plens)
    for n, (s, p) in enumerate(zip(seqs, plens)):
        of, lf = A.attn_fwd(s[None, :, :Hq], s[None, :, Hq:Hq + Hkv], s[None, :, Hq + Hkv:], blk)
        assert np.max(np.abs(of[0, p:] - o[n])) < 1e-12
        assert np.max(np.abs(lf[0, :, p:] - lse[n])) < 1e-12


def test_decode_block_unaligned_prefix_is_full_attention():
    """Any prefix length: every block token sees the whole prefix and the whole block
    (SDPA with no mask over the concatenated keys)."""
    Hq, Hkv, d, blk, P = 4, 2, 8, 5, 37
    rng = np.random.default_rng(18)
    q_blk = rng.standard_normal((1, blk, Hq, d))
    k_blk, v_blk = rng.standard_normal((1, blk, Hkv, d)), rng.standard_normal((1, blk, Hkv, d))
    kc, vc = rng.standard_normal((P, Hkv, d)), rng.standard_normal((P, Hkv, d))
    o, _ = A.decode_block(q_blk, k_blk, v_blk, kc, vc, [0], [P])
    keys = np.concatenate([kc, k_blk[0]])[None].transpose(0, 2, 1, 3)
    vals = np.concatenate([vc, v_blk[0]])[None].transpose(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q_blk.transpose(0, 2, 1, 3)),
                                         torch.from_numpy(keys).repeat_interleave(2, 1),
                                         torch.from_numpy(vals).repeat_interleave(2, 1))
    assert np.max(np.abs(ref.permute(0, 2, 1, 3).numpy() - o)) < 1e-12
