"""Pins of oracle.paged (CPU only): gathering through the page table is the identity on an
identity table and a permutation otherwise; decoding against pages equals decoding against the
packed cache; appending writes the rows after the prefix; a chain of appends rebuilds the
sequence so that decoding block b equals the forward rows of block b."""
import numpy as np

from oracle import attention as A
from oracle import paged as PG


def _pages(rng, n_pages, ps, hkv=2, d=8):
    return rng.standard_normal((n_pages * ps, hkv, d)), rng.standard_normal((n_pages * ps, hkv, d))


def test_identity_table_is_slicing():
    rng = np.random.default_rng(0)
    kp, _ = _pages(rng, 6, 4)
    table = np.arange(6, dtype=np.int32).reshape(2, 3)
    kc, start = PG.gather_prefixes(kp, table, [10, 7], 4)
    assert np.array_equal(kc[:10], kp[:10]) and np.array_equal(kc[10:], kp[12:19])
    assert start.tolist() == [0, 10]


def test_permuted_pages_equal_packed_decode():
    rng = np.random.default_rng(1)
    ps, n, T, hq, hkv, d = 4, 3, 5, 4, 2, 8
    plen = np.array([9, 0, 14])
    packed_k = rng.standard_normal((plen.sum(), hkv, d))
    packed_v = rng.standard_normal((plen.sum(), hkv, d))
    start = np.concatenate([[0], np.cumsum(plen)[:-1]])
    # scatter the packed prefixes into shuffled pages
    max_pages = 4
    perm = rng.permutation(n * max_pages).astype(np.int32)
    table = perm.reshape(n, max_pages)
    kp = np.zeros((n * max_pages * ps, hkv, d))
    vp = np.zeros_like(kp)
    for s in range(n):
        rows = PG.prefix_rows(table, s, int(plen[s]), ps)
        kp[rows] = packed_k[start[s]:start[s] + plen[s]]
        vp[rows] = packed_v[start[s]:start[s] + plen[s]]
    q = rng.standard_normal((n, T, hq, d))
    kb, vb = rng.standard_normal((n, T, hkv, d)), rng.standard_normal((n, T, hkv, d))
    o1, l1 = A.decode_block(q, kb, vb, packed_k, packed_v, start, plen)
    o2, l2 = PG.decode_block_paged(q, kb, vb, kp, vp, table, plen, ps)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_append_then_decode_is_the_forward():
    """Blocks appended one after another into shuffled pages: decoding block b against the paged
    prefix of blocks 0..b-1 gives the forward rows of block b (digest, method step 3)."""
    rng = np.random.default_rng(2)
    L, blk, hq, hkv, d, ps = 20, 5, 2, 1, 8, 8
    q = rng.standard_normal((1, L, hq, d))
    k = rng.standard_normal((1, L, hkv, d))
    v = rng.standard_normal((1, L, hkv, d))
    o_ref, _ = A.attn_fwd(q, k, v, blk)
    max_pages = 3
    table = rng.permutation(max_pages).astype(np.int32)[None]
    kp = np.zeros((max_pages * ps, hkv, d))
    vp = np.zeros_like(kp)
    plen = np.array([0], np.int32)
    for b in range(L // blk):
        sl = slice(b * blk, (b + 1) * blk)
        o, _ = PG.decode_block_paged(q[:, sl], k[:, sl], v[:, sl], kp, vp, table, plen, ps)
        assert np.allclose(o[0], o_ref[0, sl], rtol=0, atol=1e-12)
        kp, vp, plen = PG.append_block(kp, vp, table, plen, k[:, sl], v[:, sl], ps)
        assert plen[0] == (b + 1) * blk
    kc, _ = PG.gather_prefixes(kp, table, plen, ps)
    assert np.array_equal(kc, k[0])


def test_append_respects_mask_and_capacity():
    rng = np.random.default_rng(3)
    kp, vp = _pages(rng, 4, 4)
    table = np.array([[0, 1], [2, 3]], np.int32)
    kb, vb = rng.standard_normal((2, 3, 2, 8)), rng.standard_normal((2, 3, 2, 8))
    k2, _, pl = PG.append_block(kp, vp, table, [2, 6], kb, vb, 4, n_masked_left=[0, 0])
    assert pl.tolist() == [5, 6]                    # sequence 1 would pass its 8 rows: left out
    assert np.array_equal(k2[2:5], kb[0]) and np.array_equal(k2[8:16], kp[8:16])
    _, _, pl = PG.append_block(kp, vp, table, [2, 1], kb, vb, 4, n_masked_left=[1, 0])
    assert pl.tolist() == [2, 4]
