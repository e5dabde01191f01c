"""The Python binding refuses caller-supplied outputs and workspaces that the kernels would write
past or could not address (wrong shape or dtype, host memory, a strided view) before anything is
launched, so a mistake in the caller raises ValueError instead of writing out of bounds."""
import pytest
import torch

import block_diffusion_decoding_amd as bd
from gpu_util import banner

pytestmark = pytest.mark.gpu


def _bf16(*shape):
    return torch.randn(shape, device="cuda").to(torch.bfloat16)


def test_attention_outputs_checked():
    banner("binding: attention outputs and workspaces")
    q, k, v = _bf16(1, 64, 2, 128), _bf16(1, 64, 1, 128), _bf16(1, 64, 1, 128)
    with pytest.raises(ValueError):
        bd.bd_attn_fwd(q, k, v, 32, o=_bf16(1, 32, 2, 128))
    with pytest.raises(ValueError):
        bd.bd_attn_fwd(q, k, v, 32, lse=torch.empty((1, 2, 63), device="cuda"))
    o, lse = bd.bd_attn_fwd(q, k, v, 32)
    d_o = _bf16(1, 64, 2, 128)
    with pytest.raises(ValueError):
        bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, dk=_bf16(1, 64, 2, 128))      # dk has the q heads
    with pytest.raises(ValueError):
        bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, dq=torch.empty_like(q, dtype=torch.float32))
    ws = torch.empty(bd.bd_attn_bwd_workspace_size(1, 64, 2, 1, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, workspace=ws)                  # host memory
    wsd = torch.empty(2 * ws.numel(), dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError):
        bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, workspace=wsd)                 # strided view
    dq, dk, dv = bd.bd_attn_bwd(q, k, v, o, lse, d_o, 32, workspace=ws.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


def test_decode_and_cache_shapes_checked():
    banner("binding: decode outputs and cache shapes")
    n, T, Hq, Hkv, d = 2, 32, 4, 2, 128
    qb, kb, vb = _bf16(n, T, Hq, d), _bf16(n, T, Hkv, d), _bf16(n, T, Hkv, d)
    kc, vc = _bf16(100, Hkv, d), _bf16(100, Hkv, d)
    ps = torch.tensor([0, 50], dtype=torch.int64, device="cuda")
    pl = torch.tensor([50, 50], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        bd.bd_attn_decode_block(qb, kb, vb, _bf16(100, Hkv * d), vc, ps, pl, 50)     # flattened rows
    with pytest.raises(ValueError):
        bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, 50, o=_bf16(n, T, Hkv, d))
    with pytest.raises(ValueError):
        bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, 50, lse=torch.empty((n, T, Hq), device="cuda"))
    o, lse = bd.bd_attn_decode_block(qb, kb, vb, kc, vc, ps, pl, 50)
    kp, vp = _bf16(128, Hkv, d), _bf16(128, Hkv, d)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        bd.bd_attn_decode_block_paged(qb, kb, vb, _bf16(128, Hq, d), vp, bt, 32, pl, 50)
    with pytest.raises(ValueError):
        bd.bd_kv_append_block(kb, vb, kp, vp, bt[:1], 32, pl)                      # one table row for two seqs
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_commit_outputs_checked():
    banner("binding: commit outputs")
    rows, V = 64, 1000
    logits = _bf16(rows, V)
    tokens = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    masked = torch.ones(rows, dtype=torch.uint8, device="cuda")
    for kw in ({"conf": torch.empty(rows - 1, device="cuda")},
               {"pred": torch.empty(rows, dtype=torch.int64, device="cuda")},
               {"n_committed": torch.empty(rows, dtype=torch.int32, device="cuda")},
               {"n_masked_left": torch.empty(1, dtype=torch.int32, device="cuda")}):
        with pytest.raises(ValueError):
            bd.bd_confidence_commit(logits, tokens, masked, 32, 0.9, **kw)
        with pytest.raises(ValueError):
            bd.bd_confidence_commit_noalloc(logits, tokens, masked, 32, 0.9, **kw)
        with pytest.raises(ValueError):
            bd.bd_confidence_commit_sampled(logits, tokens, masked, 32, 0.9, **kw)
    with pytest.raises(ValueError):   # a vocabulary wider than the rows would read past the last row
        bd.bd_confidence_commit(logits, tokens, masked, 32, 0.9, vocab=V + 8)
    w, h = _bf16(V, 64), _bf16(rows, 64)
    with pytest.raises(ValueError):
        bd.bd_lmhead_commit(h, w, tokens, masked, 32, 0.9, conf=torch.empty(rows, dtype=torch.float64,
                                                                               device="cuda"))
    assert torch.equal(masked, torch.ones_like(masked))     # nothing ran
    out = bd.bd_confidence_commit(logits, tokens, masked, 32, 0.9)
    torch.cuda.synchronize()
    assert int(out["n_masked_left"].sum()) == int(masked.sum())
