"""Pins of the oracle's block-causal attention forward (CPU only).

Each test ties ``oracle.attention`` to something other than itself: a library
routine in the special cases the block mask reduces to (block size 1 = causal,
block size L = full), a hand-drawn mask, closed forms, invariants the pages'
definition implies, and brute force.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in float64 on CPU; q [B,L,Hq,d], k/v [B,L,Hkv,d]."""
    G = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.permute(0, 2, 1, 3).numpy()


def _shapes():
    return [(1, 13, 2, 2, 5, 4), (2, 16, 4, 2, 8, 4), (1, 9, 3, 1, 4, 3)]


@pytest.mark.parametrize("B,L,Hq,Hkv,d,blk", _shapes())
def test_bruteforce_agrees(B, L, Hq, Hkv, d, blk):
    q, k, v = _rand((B, L, Hq, d), 1), _rand((B, L, Hkv, d), 2), _rand((B, L, Hkv, d), 3)
    o1, l1 = A.attn_fwd(q, k, v, blk)
    o2, l2 = A.attn_fwd_bruteforce(q, k, v, blk)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("B,L,Hq,Hkv,d", [(1, 37, 4, 2, 16), (2, 20, 2, 2, 8)])
def test_block_size_one_is_causal(B, L, Hq, Hkv, d):
    q, k, v = _rand((B, L, Hq, d), 4), _rand((B, L, Hkv, d), 5), _rand((B, L, Hkv, d), 6)
    o, _ = A.attn_fwd(q, k, v, 1)
    ref = _sdpa(q, k, v, causal=True)
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("blk", [37, 64])
def test_block_size_L_is_full(blk):
    B, L, Hq, Hkv, d = 1, 37, 4, 2, 16
    q, k, v = _rand((B, L, Hq, d), 7), _rand((B, L, Hkv, d), 8), _rand((B, L, Hkv, d), 9)
    o, _ = A.attn_fwd(q, k, v, blk)
    ref = _sdpa(q, k, v)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_hand_drawn_mask(golden_dir):
    rows = [ln.strip() for ln in open(os.path.join(golden_dir, "block_mask_L8_blk3.txt"))
            if ln.strip() and not ln.startswith("#")]
    mask = np.array([[c == "1" for c in r] for r in rows])
    assert mask.shape == (8, 8)
    assert np.array_equal(A.block_mask(8, 3), mask)
    for i in range(8):
        assert A.key_limit(i, 8, 3) == mask[i].sum()
    q, k, v = _rand((1, 8, 2, 4), 10), _rand((1, 8, 1, 4), 11), _rand((1, 8, 1, 4), 12)
    o, _ = A.attn_fwd(q, k, v, 3)
    ref = _sdpa(q, k, v, mask=mask)
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("L,blk", [(16, 4), (13, 5), (8, 8)])
def test_zero_query_averages_visible_values(L, blk):
    """q = 0 gives equal weights: o_i is the mean of the visible v_j and lse_i = ln(#visible)."""
    q = np.zeros((1, L, 2, 3))
    k, v = _rand((1, L, 1, 3), 13), _rand((1, L, 1, 3), 14)
    o, lse = A.attn_fwd(q, k, v, blk)
    for i in range(L):
        n = (i // blk + 1) * blk
        n = min(n, L)
        assert np.allclose(o[0, i, 0], v[0, :n, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - np.log(n)) < 1e-14


def test_future_blocks_do_not_leak():
    B, L, Hq, Hkv, d, blk = 1, 24, 2, 1, 8, 4
    q, k, v = _rand((B, L, Hq, d), 15), _rand((B, L, Hkv, d), 16), _rand((B, L, Hkv, d), 17)
    o, lse = A.attn_fwd(q, k, v, blk)
    for b in range(L // blk - 1):
        cut = (b + 1) * blk
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, cut:] += 5.0
        k2[:, cut:] *= -3.0
        v2[:, cut:] += 7.0
        o2, lse2 = A.attn_fwd(q2, k2, v2, blk)
        assert np.array_equal(o[:, :cut], o2[:, :cut])
        assert np.array_equal(lse[..., :cut], lse2[..., :cut])
        assert not np.allclose(o[:, cut:], o2[:, cut:])


def test_within_block_permutation_is_invisible_to_later_rows():
    """Bidirectional inside a block: permuting the keys/values of one block leaves every row
    that sees that block unchanged -- unlike causal attention, whose rows inside it change."""
    B, L, Hq, Hkv, d, blk = 1, 16, 2, 2, 6, 4
    q, k, v = _rand((B, L, Hq, d), 18), _rand((B, L, Hkv, d), 19), _rand((B, L, Hkv, d), 20)
    perm = np.arange(L)
    perm[4:8] = [6, 4, 7, 5]
    o, _ = A.attn_fwd(q, k, v, blk)
    o2, _ = A.attn_fwd(q, k[:, perm], v[:, perm], blk)
    assert np.max(np.abs(o[:, 4:] - o2[:, 4:])) < 1e-12
    oc, _ = A.attn_fwd(q, k, v, 1)
    oc2, _ = A.attn_fwd(q, k[:, perm], v[:, perm], 1)
    assert np.max(np.abs(oc[:, 4:8] - oc2[:, 4:8])) > 1e-3


def test_lse_normalises_visible_weights():
    B, L, Hq, Hkv, d, blk = 1, 20, 2, 1, 8, 6
    q, k, v = _rand((B, L, Hq, d), 21), _rand((B, L, Hkv, d), 22), _rand((B, L, Hkv, d), 23)
    _, lse = A.attn_fwd(q, k, v, blk, scale=0.3)
    for h in range(Hq):
        for i in range(L):
            n = A.key_limit(i, L, blk)
            s = 0.3 * (k[0, :n, 0] @ q[0, i, h])
            assert abs(np.exp(s - lse[0, h, i]).sum() - 1.0) < 1e-13


def test_gqa_equals_repeated_heads():
    B, L, Hq, Hkv, d, blk = 1, 12, 4, 2, 5, 4
    q, k, v = _rand((B, L, Hq, d), 24), _rand((B, L, Hkv, d), 25), _rand((B, L, Hkv, d), 26)
    o, lse = A.attn_fwd(q, k, v, blk)
    o2, lse2 = A.attn_fwd(q, np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2), blk)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_subset_rows_match_full():
    B, L, Hq, Hkv, d, blk = 2, 20, 4, 2, 6, 4
    q, k, v = _rand((B, L, Hq, d), 27), _rand((B, L, Hkv, d), 28), _rand((B, L, Hkv, d), 29)
    o, lse = A.attn_fwd(q, k, v, blk)
    o2, lse2 = A.attn_fwd(q, k, v, blk, q_blocks=[1, 4], heads=[3], batches=[1])
    assert np.array_equal(o[1, 4:8, 3], o2[1, 4:8, 3])
    assert np.array_equal(o[1, 16:20, 3], o2[1, 16:20, 3])
    assert np.isnan(o2[0]).all()


@pytest.mark.parametrize("L,blk", [(128, 32), (12288, 32), (16384, 32), (37, 5)])
def test_flop_count_matches_mask(L, blk):
    pairs = A.attn_flops(L, blk, 1, 1) / 4.0
    if L <= 128:
        assert pairs == A.block_mask(L, blk).sum()
    if L % blk == 0:
        nb = L // blk
        assert pairs == blk * blk * nb * (nb + 1) // 2
