"""Seeded synthetic inputs for the block-diffusion decoding hot path.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It draws random numbers and lays them out; it performs none of the
method's arithmetic (no attention, no softmax, no commit rule).

The shapes follow the workloads the MinerU-Diffusion pages imply: block size 32
("Reliability / weaknesses" paragraph of the paper digest page, which notes the
fixed block size), the two training sequence lengths 12288 and 16384 (method
step 5 of the same digest), the threshold T = 0.95 (method steps 4 and 6).  The
head shapes and the vocabulary size are synthetic choices: the pages name
neither.  The public benchmarks the pages evaluate on (OmniDocBench v1.5,
CC-OCR, OCRBench v2, UniMER-Test) and the trained weights are not available, so
every input here is random and stands in for them.

Draw order inside one generator call is fixed (q, k, v, dO, then logits) and the
generator is ``numpy.random.default_rng(seed)``; the default seed of workload
``n`` is ``1000 + n``.

bf16 values are produced by drawing float32 and rounding to nearest-even on the
bit pattern; they are handed out as ``uint16`` bit arrays so that the GPU side
and the oracle side read exactly the same values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "Workload", "WORKLOADS",
    "attention_inputs", "decode_inputs", "commit_inputs", "prefix_lengths",
    "boosted_logits_bits", "loop_step_logits", "loop_step_block", "lmhead_inputs",
]


# ---------------------------------------------------------------------------
# bf16 bit handling (storage format only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as ``uint16``.  NaN stays NaN (quiet), +-Inf
    stays +-Inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # at most 0xFF807FFF for finite and infinite inputs: no 32-bit overflow
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (``uint16``) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """One synthetic workload: the shape of the hot path at one operating point."""

    wid: int
    name: str
    dtype: str                    # "f32" or "bf16"
    batch: int = 1
    seqlen: int = 0               # full-sequence attention length L (0: none)
    n_q_heads: int = 1
    n_kv_heads: int = 1
    head_dim: int = 64
    block_size: int = 32          # L' on the pages
    vocab: int = 0                # 0: no commit step
    prefix_len: int = 0           # decode: cached prefix length P
    n_seq: int = 1                # decode / commit: sequences
    threshold: float = 0.95
    thresholds: tuple = field(default_factory=tuple)
    masked_frac: float = 1.0
    logit_std: float = 1.0
    boost: Optional[tuple] = None  # (lo, hi) of the uniform boost at one id per row
    prefix_range: Optional[tuple] = None  # (lo, hi) inclusive of ragged prefix lengths

    @property
    def seed(self) -> int:
        return 1000 + self.wid


WORKLOADS = {
    # 1 seq, 1 head, d=64, L=128 in 4 blocks of 32; logits [32 x 1000] N(0, 3^2),
    # half the positions masked; T = 0.95.
    "tiny_f32": Workload(1, "tiny_f32", "f32", batch=1, seqlen=128, n_q_heads=1, n_kv_heads=1,
                         head_dim=64, block_size=32, vocab=1000, n_seq=1, threshold=0.95,
                         masked_frac=0.5, logit_std=3.0),
    # One decode step: 4096-token prefix, a block of 32, 16/8 heads, d=128;
    # logits [32 x 151936] N(0,1) + U(4,14) at one random id per row.
    "decode_step_bf16": Workload(2, "decode_step_bf16", "bf16", batch=1, n_q_heads=16, n_kv_heads=8,
                                 head_dim=128, block_size=32, vocab=151936, prefix_len=4096,
                                 n_seq=1, threshold=0.95, boost=(4.0, 14.0)),
    # Full-sequence forward at the first training length.
    "fwd_L12288_bf16": Workload(3, "fwd_L12288_bf16", "bf16", batch=1, seqlen=12288, n_q_heads=16,
                                n_kv_heads=8, head_dim=128, block_size=32),
    # Forward + backward at the second training length (the headline shape).
    "fwdbwd_L16384_bf16": Workload(4, "fwdbwd_L16384_bf16", "bf16", batch=2, seqlen=16384,
                                   n_q_heads=16, n_kv_heads=8, head_dim=128, block_size=32),
    # The LM head in front of the commit (a "next" row): one block of 32 hidden
    # states of width 2048 (= 16 heads x 128, the decoder of the 1.7B base named
    # on the digest page) against a [151936 x 2048] weight; logits never stored.
    "lmhead_block_bf16": Workload(6, "lmhead_block_bf16", "bf16", batch=1, n_q_heads=16, n_kv_heads=8,
                                  head_dim=128, block_size=32, vocab=151936, n_seq=1, threshold=0.95,
                                  boost=(2.0, 14.0)),
    # Batched decode loop: 64 sequences, ragged prefixes U[1024, 16384].
    "decode_loop_bf16": Workload(5, "decode_loop_bf16", "bf16", batch=1, n_q_heads=16, n_kv_heads=8,
                                 head_dim=128, block_size=32, vocab=151936, n_seq=64,
                                 thresholds=(0.5, 0.95, 0.99), boost=(2.0, 14.0),
                                 prefix_range=(1024, 16384)),
}


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> float32 array, or bf16 bits (uint16)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def attention_inputs(batch: int, seqlen: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                     dtype: str, seed: int, with_grad: bool = False,
                     rng: Optional[np.random.Generator] = None) -> dict:
    """q [B,L,Hq,d], k/v [B,L,Hkv,d] (and dO [B,L,Hq,d]) drawn from N(0,1)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    out = {
        "q": _as_dtype(_normal(rng, (batch, seqlen, n_q_heads, head_dim)), dtype),
        "k": _as_dtype(_normal(rng, (batch, seqlen, n_kv_heads, head_dim)), dtype),
        "v": _as_dtype(_normal(rng, (batch, seqlen, n_kv_heads, head_dim)), dtype),
    }
    if with_grad:
        out["do"] = _as_dtype(_normal(rng, (batch, seqlen, n_q_heads, head_dim)), dtype)
    return out


def prefix_lengths(n_seq: int, lo: int, hi: int, rng: np.random.Generator) -> np.ndarray:
    """Ragged prefix lengths, uniform integers in [lo, hi] (inclusive)."""
    return rng.integers(lo, hi + 1, size=n_seq).astype(np.int32)


def decode_inputs(n_seq: int, prefix_lens, blk_len: int, n_q_heads: int, n_kv_heads: int,
                  head_dim: int, dtype: str, seed: int,
                  rng: Optional[np.random.Generator] = None) -> dict:
    """One decode step: the current block's q/k/v per sequence plus a packed prefix cache.

    q_blk [n_seq, blk_len, Hq, d]; k_blk/v_blk [n_seq, blk_len, Hkv, d];
    k_cache/v_cache [sum(P), Hkv, d] with sequence n at rows
    [prefix_start[n], prefix_start[n] + prefix_len[n]).
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    plen = np.asarray(prefix_lens, dtype=np.int32).reshape(n_seq)
    start = np.zeros(n_seq, dtype=np.int64)
    if n_seq > 1:
        start[1:] = np.cumsum(plen[:-1].astype(np.int64))
    total = int(plen.astype(np.int64).sum())
    out = {
        "q_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_q_heads, head_dim)), dtype),
        "k_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_kv_heads, head_dim)), dtype),
        "v_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_kv_heads, head_dim)), dtype),
        "k_cache": _as_dtype(_normal(rng, (max(total, 0), n_kv_heads, head_dim)), dtype),
        "v_cache": _as_dtype(_normal(rng, (max(total, 0), n_kv_heads, head_dim)), dtype),
        "prefix_start": start,
        "prefix_len": plen,
    }
    return out


def boosted_logits_bits(rows: int, vocab: int, boost_lo: float, boost_hi: float,
                        rng: np.random.Generator, dtype: str = "bf16") -> np.ndarray:
    """Logits N(0,1) plus a uniform U(lo, hi) boost at one random id per row."""
    x = _normal(rng, (rows, vocab))
    ids = rng.integers(0, vocab, size=rows)
    x[np.arange(rows), ids] += rng.uniform(boost_lo, boost_hi, size=rows).astype(np.float32)
    return _as_dtype(x, dtype)


def loop_step_logits(n_seq: int, blk_len: int, vocab: int, boost: tuple, seed: int, step: int,
                     dtype: str = "bf16") -> np.ndarray:
    """Fresh logits of one step of the decode loop: ``[n_seq*blk_len, vocab]`` drawn as
    ``boosted_logits_bits`` from a generator seeded by ``(seed, step)``, so any step can be
    drawn again on its own."""
    rng = np.random.default_rng((seed, step))
    return boosted_logits_bits(n_seq * blk_len, vocab, boost[0], boost[1], rng, dtype)


def loop_step_block(n_seq: int, blk_len: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                    dtype: str, seed: int, step: int) -> dict:
    """Fresh q_blk / k_blk / v_blk of one step of the decode loop (N(0,1)), from a generator
    seeded by ``(seed, step, 1)``."""
    rng = np.random.default_rng((seed, step, 1))
    return {"q_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_q_heads, head_dim)), dtype),
            "k_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_kv_heads, head_dim)), dtype),
            "v_blk": _as_dtype(_normal(rng, (n_seq, blk_len, n_kv_heads, head_dim)), dtype)}


def commit_inputs(n_seq: int, blk_len: int, vocab: int, dtype: str, seed: int,
                  masked_frac: float = 1.0, logit_std: float = 1.0,
                  boost: Optional[tuple] = None,
                  rng: Optional[np.random.Generator] = None) -> dict:
    """Logits [n_seq*blk_len, vocab] plus the token state (tokens, masked flags).

    With ``masked_frac < 1`` exactly ``round(masked_frac * blk_len)`` positions of
    every block are masked, picked by a random permutation; the others hold an
    already-committed token id.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    rows = n_seq * blk_len
    if boost is None:
        logits = _as_dtype(_normal(rng, (rows, vocab), logit_std), dtype)
    else:
        logits = boosted_logits_bits(rows, vocab, boost[0], boost[1], rng, dtype)
    masked = np.ones(rows, dtype=np.uint8)
    if masked_frac < 1.0:
        masked[:] = 0
        k = int(round(masked_frac * blk_len))
        for s in range(n_seq):
            pos = rng.permutation(blk_len)[:k]
            masked[s * blk_len + pos] = 1
    tokens = np.where(masked == 1, -1, rng.integers(0, vocab, size=rows)).astype(np.int32)
    return {"logits": logits, "tokens": tokens, "masked": masked}


def lmhead_inputs(n_seq: int, blk_len: int, hidden: int, vocab: int, seed: int,
                  boost: tuple = (2.0, 14.0), masked_frac: float = 1.0,
                  rng: Optional[np.random.Generator] = None) -> dict:
    """Hidden states X [n_seq*blk_len, hidden] ~ N(0,1) and an LM-head weight W [vocab, hidden]
    ~ N(0, 1/hidden) (so every logit X W^T starts as roughly N(0,1)), both rounded to bf16, plus
    the token state as in ``commit_inputs``.  Each row r gets a boost b_r ~ U(lo, hi) at one id
    t_r: W[t_r] += b_r X_r / |X_r|^2 before rounding, which raises logit (r, t_r) by b_r and moves
    the other rows' logits of id t_r by b_r <X_r', X_r> / |X_r|^2 (about b_r / sqrt(hidden)).
    The recipe mirrors the boosted synthetic logits of the commit workloads."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    rows = n_seq * blk_len
    xb = f32_to_bf16_bits(_normal(rng, (rows, hidden)))
    x = bf16_bits_to_f32(xb)
    w = _normal(rng, (vocab, hidden), std=float(1.0 / np.sqrt(hidden)))
    ids = rng.integers(0, vocab, size=rows)
    b = rng.uniform(boost[0], boost[1], size=rows).astype(np.float32)
    norm2 = (x.astype(np.float64) ** 2).sum(axis=1)
    for r in range(rows):
        w[ids[r]] += (b[r] / norm2[r] * x[r]).astype(np.float32)
    wb = f32_to_bf16_bits(w)
    del w
    if masked_frac >= 1.0:
        masked = np.ones(rows, np.uint8)
    else:
        masked = np.zeros(rows, np.uint8)
        k = int(round(masked_frac * blk_len))
        for s in range(n_seq):
            masked[s * blk_len + rng.permutation(blk_len)[:k]] = 1
    tokens = np.where(masked == 1, -1, rng.integers(0, vocab, size=rows)).astype(np.int32)
    return {"hidden": xb, "weight": wb, "boost_ids": ids, "tokens": tokens, "masked": masked}
