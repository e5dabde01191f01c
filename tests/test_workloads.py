"""The seeded input generators: determinism, shapes and the bf16 storage rounding."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1e-40, -1e-40, np.inf, -np.inf, 3.4e38, 65504.0], np.float32)])
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_seeded():
    a = W.attention_inputs(1, 64, 4, 2, 16, "bf16", seed=5, with_grad=True)
    b = W.attention_inputs(1, 64, 4, 2, 16, "bf16", seed=5, with_grad=True)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (1, 64, 4, 16) and a["k"].shape == (1, 64, 2, 16) and a["q"].dtype == np.uint16


def test_decode_inputs_pack_prefixes():
    rng = np.random.default_rng(3)
    plen = W.prefix_lengths(5, 10, 20, rng)
    d = W.decode_inputs(5, plen, 4, 4, 2, 8, "f32", seed=1)
    assert d["k_cache"].shape == (int(plen.sum()), 2, 8)
    assert d["prefix_start"][0] == 0 and np.array_equal(np.diff(d["prefix_start"]), plen[:-1])
    assert ((plen >= 10) & (plen <= 20)).all()


def test_commit_inputs_masking():
    c = W.commit_inputs(3, 32, 100, "f32", seed=2, masked_frac=0.5)
    assert c["masked"].reshape(3, 32).sum(axis=1).tolist() == [16, 16, 16]
    assert (c["tokens"][c["masked"] == 1] == -1).all() and (c["tokens"][c["masked"] == 0] >= 0).all()
    b = W.commit_inputs(1, 32, 1000, "bf16", seed=2, boost=(4.0, 14.0))
    x = W.bf16_bits_to_f32(b["logits"])
    assert (x.max(axis=1) > 3.0).all()
