"""The C-ABI library: it loads, exports every entry point include/bd.h declares, and rejects
bad arguments on the host before anything is enqueued (no GPU needed: every call below
fails validation, so no kernel is launched)."""
import math
import os
import re

import pytest

from block_diffusion_decoding_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 16-byte aligned, never dereferenced stand-in address
MIS = FAKE + 8          # misaligned stand-in


def _declared():
    text = open(os.path.join(ROOT, "include", "bd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 18, names
    for n in names:
        assert hasattr(L.lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_status_strings_and_version():
    for s in range(9):
        assert L.lib.bd_status_string(s)
    assert L.lib.bd_status_string(99) == b"unknown status"
    assert L.lib.bd_version() >= 100


def fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, S=64, Hq=2, Hkv=1, d=128, blk=32, sc=0.0, dt=L.BD_BF16):
    return L.lib.bd_attn_fwd(q, k, v, o, lse, B, S, Hq, Hkv, d, blk, sc, dt, None)


def test_fwd_validation():
    assert fwd(q=None) == L.BD_ERR_NULL
    assert fwd(o=None) == L.BD_ERR_NULL
    assert fwd(B=0) == L.BD_ERR_SHAPE
    assert fwd(S=-1) == L.BD_ERR_SHAPE
    assert fwd(blk=0) == L.BD_ERR_SHAPE
    assert fwd(Hq=3, Hkv=2) == L.BD_ERR_SHAPE
    assert fwd(d=64) == L.BD_ERR_UNSUPPORTED
    assert fwd(d=256, dt=L.BD_F32) == L.BD_ERR_UNSUPPORTED
    assert fwd(dt=7) == L.BD_ERR_UNSUPPORTED
    assert fwd(sc=math.nan) == L.BD_ERR_VALUE
    assert fwd(sc=math.inf) == L.BD_ERR_VALUE
    assert fwd(k=MIS) == L.BD_ERR_ALIGNMENT
    assert fwd(o=MIS) == L.BD_ERR_ALIGNMENT


def test_bwd_validation():
    ws = L.lib.bd_attn_bwd_workspace_size(1, 64, 2, 1, 128)
    assert ws == 1 * 2 * 64 * 8 + 64        # -D and -LSE/scale per row, then the work counters
    args = [FAKE] * 9 + [FAKE, ws, 1, 64, 2, 1, 128, 32, 0.0, L.BD_BF16, None]
    bad = list(args); bad[4] = None
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_NULL          # lse is required
    bad = list(args); bad[9] = None
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_WORKSPACE
    bad = list(args); bad[10] = ws - 8
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_WORKSPACE
    bad = list(args); bad[14] = 3
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_SHAPE
    bad = list(args); bad[5] = MIS
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_ALIGNMENT
    bad = list(args); bad[9] = MIS
    assert L.lib.bd_attn_bwd(*bad) == L.BD_ERR_ALIGNMENT     # the workspace too


def test_decode_validation():
    ws = L.lib.bd_attn_decode_workspace_size(1, 32, 4096, 16, 8, 128)
    assert ws > 0
    assert L.lib.bd_attn_decode_workspace_size(1, 32, 4096, 16, 6, 128) == 0

    def call(**kw):
        a = dict(qb=FAKE, kb=FAKE, vb=FAKE, kc=FAKE, vc=FAKE, ps=FAKE, pl=FAKE, maxp=4096, o=FAKE, lse=None,
                 n=1, T=32, Hq=16, Hkv=8, d=128, sc=0.0, dt=L.BD_BF16, ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_attn_decode_block(a["qb"], a["kb"], a["vb"], a["kc"], a["vc"], a["ps"], a["pl"], a["maxp"],
                                          a["o"], a["lse"], a["n"], a["T"], a["Hq"], a["Hkv"], a["d"], a["sc"],
                                          a["dt"], a["ws"], a["nb"], None)
    assert call(qb=None) == L.BD_ERR_NULL
    assert call(ps=None) == L.BD_ERR_NULL
    assert call(kc=None) == L.BD_ERR_NULL
    assert call(maxp=-1) == L.BD_ERR_SHAPE
    assert call(n=0) == L.BD_ERR_SHAPE
    assert call(Hkv=6) == L.BD_ERR_SHAPE
    assert call(d=96) == L.BD_ERR_UNSUPPORTED
    assert call(ws=None) == L.BD_ERR_WORKSPACE
    assert call(nb=ws - 1) == L.BD_ERR_WORKSPACE
    assert call(kc=MIS) == L.BD_ERR_ALIGNMENT
    assert call(ws=MIS) == L.BD_ERR_ALIGNMENT
    assert call(sc=math.nan) == L.BD_ERR_VALUE


def test_commit_validation():
    ws = L.lib.bd_confidence_commit_workspace_size(2, 32, 151936)
    assert ws > 0 and ws % (2 * 32 * 16) == 0     # 16-byte partials per (row, vocabulary chunk)

    def call(**kw):
        a = dict(lg=FAKE, stride=151936, n=2, T=32, V=151936, dt=L.BD_BF16, thr=0.95, fb=1, tok=FAKE, msk=FAKE,
                 ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_confidence_commit(a["lg"], a["stride"], a["n"], a["T"], a["V"], a["dt"], a["thr"], a["fb"],
                                          a["tok"], a["msk"], None, None, None, None, a["ws"], a["nb"], None)
    assert call(lg=None) == L.BD_ERR_NULL
    assert call(tok=None) == L.BD_ERR_NULL
    assert call(msk=None) == L.BD_ERR_NULL
    assert call(stride=100) == L.BD_ERR_SHAPE
    assert call(V=0) == L.BD_ERR_SHAPE
    assert call(T=2048) == L.BD_ERR_UNSUPPORTED
    assert call(dt=5) == L.BD_ERR_UNSUPPORTED
    assert call(thr=math.nan) == L.BD_ERR_VALUE
    assert call(fb=7) == L.BD_ERR_VALUE
    assert call(ws=None) == L.BD_ERR_WORKSPACE
    assert call(nb=ws - 16) == L.BD_ERR_WORKSPACE
    assert call(ws=MIS) == L.BD_ERR_ALIGNMENT

    def call_rw(**kw):
        a = dict(lg=FAKE, stride=151936, n=2, T=32, V=151936, dt=L.BD_BF16, thr=FAKE, fb=1, tok=FAKE, msk=FAKE,
                 ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_confidence_commit_rowwise(a["lg"], a["stride"], a["n"], a["T"], a["V"], a["dt"], a["thr"],
                                                  a["fb"], a["tok"], a["msk"], None, None, None, None, a["ws"],
                                                  a["nb"], None)
    assert call_rw(thr=None) == L.BD_ERR_NULL
    assert call_rw(lg=None) == L.BD_ERR_NULL
    assert call_rw(stride=100) == L.BD_ERR_SHAPE
    assert call_rw(T=2048) == L.BD_ERR_UNSUPPORTED
    assert call_rw(fb=7) == L.BD_ERR_VALUE
    assert call_rw(nb=ws - 16) == L.BD_ERR_WORKSPACE
    assert call_rw(ws=MIS) == L.BD_ERR_ALIGNMENT


def test_sampled_commit_validation():
    ws = L.lib.bd_confidence_commit_sampled_workspace_size(2, 32, 151936)
    assert ws >= L.lib.bd_confidence_commit_workspace_size(2, 32, 151936) + 64 * 8   # finer chunks, + (conf, id)

    def call(**kw):
        a = dict(lg=FAKE, stride=151936, n=2, T=32, V=151936, dt=L.BD_BF16, tau=1.0, seed=5, step=0, k=0, p=1.0,
                 thr=0.95, fb=1, tok=FAKE, msk=FAKE, ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_confidence_commit_sampled(a["lg"], a["stride"], a["n"], a["T"], a["V"], a["dt"], a["tau"],
                                                  a["seed"], a["step"], a["k"], a["p"], a["thr"], a["fb"], a["tok"],
                                                  a["msk"], None, None, None, None, a["ws"], a["nb"], None)
    assert call(lg=None) == L.BD_ERR_NULL
    assert call(stride=100) == L.BD_ERR_SHAPE
    assert call(tau=0.0) == L.BD_ERR_VALUE
    assert call(tau=-1.0) == L.BD_ERR_VALUE
    assert call(tau=math.inf) == L.BD_ERR_VALUE
    assert call(tau=math.nan) == L.BD_ERR_VALUE
    assert call(thr=math.nan) == L.BD_ERR_VALUE
    assert call(nb=ws - 1) == L.BD_ERR_WORKSPACE
    assert call(ws=MIS) == L.BD_ERR_ALIGNMENT
    assert call(seed=2**64 - 1, step=2**63, nb=0) == L.BD_ERR_WORKSPACE    # 64-bit arguments pass through
    # truncation: top_k >= 0, 0 < top_p <= 1; rows held in registers bound the vocabulary
    assert call(k=-1) == L.BD_ERR_VALUE
    assert call(p=0.0) == L.BD_ERR_VALUE
    assert call(p=1.5) == L.BD_ERR_VALUE
    assert call(p=math.nan) == L.BD_ERR_VALUE
    assert call(k=50, nb=0) == L.BD_ERR_WORKSPACE and call(p=0.9, nb=0) == L.BD_ERR_WORKSPACE
    big = L.lib.bd_confidence_commit_sampled_workspace_size(2, 32, 155649)
    assert call(V=155649, stride=155656, k=50, nb=big) == L.BD_ERR_UNSUPPORTED
    assert call(V=155649, stride=155656, nb=0) == L.BD_ERR_WORKSPACE       # no truncation: any vocabulary
    f32 = L.lib.bd_confidence_commit_sampled_workspace_size(2, 32, 77825)
    assert call(V=77825, stride=77828, dt=L.BD_F32, p=0.5, nb=f32) == L.BD_ERR_UNSUPPORTED
    assert call(V=77824, stride=77824, dt=L.BD_F32, p=0.5, nb=0) == L.BD_ERR_WORKSPACE


def test_paged_validation():
    ws = L.lib.bd_attn_decode_workspace_size(1, 32, 4096, 16, 8, 128)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, mp=64, ps=64, pl=FAKE, mpl=4096, o=FAKE, n=1,
                 T=32, hq=16, hkv=8, d=128, sc=0.0, dt=L.BD_BF16, ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_attn_decode_block_paged(a["q"], a["k"], a["v"], a["kp"], a["vp"], a["bt"], a["mp"], a["ps"],
                                                a["pl"], a["mpl"], a["o"], None, a["n"], a["T"], a["hq"], a["hkv"],
                                                a["d"], a["sc"], a["dt"], a["ws"], a["nb"], None)
    assert call(bt=None) == L.BD_ERR_NULL
    assert call(pl=None) == L.BD_ERR_NULL
    assert call(ps=48) == L.BD_ERR_UNSUPPORTED
    assert call(ps=0) == L.BD_ERR_UNSUPPORTED
    assert call(mp=63) == L.BD_ERR_SHAPE             # 63 pages of 64 rows < 4096
    assert call(dt=L.BD_F32) == L.BD_ERR_UNSUPPORTED
    assert call(kp=MIS) == L.BD_ERR_ALIGNMENT
    assert call(nb=ws - 1) == L.BD_ERR_WORKSPACE
    assert call(ws=MIS) == L.BD_ERR_ALIGNMENT

    def app(**kw):
        a = dict(k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, mp=64, ps=64, pl=FAKE, nml=None, n=1, T=32, hkv=8, d=128,
                 dt=L.BD_BF16)
        a.update(kw)
        return L.lib.bd_kv_append_block(a["k"], a["v"], a["kp"], a["vp"], a["bt"], a["mp"], a["ps"], a["pl"],
                                        a["nml"], a["n"], a["T"], a["hkv"], a["d"], a["dt"], None)
    assert app(bt=None) == L.BD_ERR_NULL
    assert app(mp=0) == L.BD_ERR_SHAPE
    assert app(ps=0) == L.BD_ERR_SHAPE
    assert app(dt=L.BD_F32) == L.BD_ERR_UNSUPPORTED
    assert app(hkv=1, d=4) == L.BD_ERR_UNSUPPORTED
    assert app(kp=MIS) == L.BD_ERR_ALIGNMENT


def test_lmhead_validation():
    ws = L.lib.bd_lmhead_commit_workspace_size(1, 32, 151936)
    assert ws == 32 * 256 * 16      # one 16-byte partial per (row, workgroup)

    def call(**kw):
        a = dict(x=FAKE, xs=2048, w=FAKE, wsd=2048, n=1, T=32, H=2048, V=151936, thr=0.95, fb=1, tok=FAKE,
                 msk=FAKE, ws=FAKE, nb=ws)
        a.update(kw)
        return L.lib.bd_lmhead_commit(a["x"], a["xs"], a["w"], a["wsd"], a["n"], a["T"], a["H"], a["V"], a["thr"],
                                      a["fb"], a["tok"], a["msk"], None, None, None, None, a["ws"], a["nb"], None)
    assert call(x=None) == L.BD_ERR_NULL
    assert call(w=None) == L.BD_ERR_NULL
    assert call(msk=None) == L.BD_ERR_NULL
    assert call(V=0) == L.BD_ERR_SHAPE
    assert call(xs=100) == L.BD_ERR_SHAPE
    assert call(H=2056, xs=2056, wsd=2056) == L.BD_ERR_UNSUPPORTED      # more than 2048
    assert call(H=96, xs=96, wsd=96) == L.BD_ERR_UNSUPPORTED            # not a multiple of 64
    assert call(x=MIS) == L.BD_ERR_ALIGNMENT
    assert call(wsd=2052) == L.BD_ERR_ALIGNMENT
    assert call(thr=math.nan) == L.BD_ERR_VALUE
    assert call(fb=3) == L.BD_ERR_VALUE
    assert call(nb=ws - 1) == L.BD_ERR_WORKSPACE
    assert call(ws=MIS) == L.BD_ERR_ALIGNMENT


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    import block_diffusion_decoding_amd as bd
    x = torch.zeros(1, 32, 1, 64)
    with pytest.raises(ValueError):
        bd.bd_attn_fwd(x, x, x)


def test_commit_noalloc_validation():
    """The no-allocation commit validates like bd_confidence_commit and refuses, before touching
    the device, a shape whose partials exceed its fixed scratch (BD_NOALLOC_SCRATCH_BYTES)."""
    def call(logits=FAKE, n_seq=1, blk=32, V=151936, dt=L.BD_BF16, T=0.95, fb=1, tok=FAKE, msk=FAKE):
        return L.lib.bd_confidence_commit_noalloc(logits, V, n_seq, blk, V, dt, T, fb, tok, msk, None, None, None,
                                                  None, None)
    assert call(logits=None) == L.BD_ERR_NULL
    assert call(tok=None) == L.BD_ERR_NULL
    assert call(n_seq=0) == L.BD_ERR_SHAPE
    assert call(blk=2048) == L.BD_ERR_UNSUPPORTED
    assert call(T=math.nan) == L.BD_ERR_VALUE
    assert call(fb=5) == L.BD_ERR_VALUE
    cap = L.BD_NOALLOC_SCRATCH_BYTES
    # the largest shapes that fit: 262144 rows at any vocabulary (one chunk per row from 8192 rows
    # on, fewer than 16384 partials below)
    for n_seq, blk, V in ((262144, 1, 151936), (8192, 32, 151936), (1, 32, 151936), (255, 32, 2**31 - 1),
                          (8191, 1, 10**9)):
        assert L.lib.bd_confidence_commit_workspace_size(n_seq, blk, V) <= cap, (n_seq, blk, V)
    assert L.lib.bd_confidence_commit_workspace_size(262145, 1, 151936) > cap
    assert call(n_seq=262145, blk=1) == L.BD_ERR_SCRATCH
    assert call(n_seq=8193, blk=32) == L.BD_ERR_SCRATCH
    assert L.lib.bd_status_string(L.BD_ERR_SCRATCH) != L.lib.bd_status_string(L.BD_ERR_WORKSPACE)
