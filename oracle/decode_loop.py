"""Oracle: the per-block denoising loop (TEST INFRASTRUCTURE; see ``oracle/__init__.py``).

Definition followed (digest page, method step 2: the posterior factorises over
blocks, each block conditioned on the earlier ones; method step 4: each step
confirms the masked tokens whose confidence exceeds T and leaves the rest for
the next step; blog page, Fig. 1).  For one block of every sequence:

1. all ``L'`` positions start masked;
2. each step produces logits for the block (here: supplied by the caller, as
   the model is not part of the path) and runs the commit rule of
   :func:`oracle.commit.confidence_commit`;
3. a sequence whose block has no masked position left is finished; its later
   steps are no-ops;
4. the loop ends when every sequence is finished.

The rule of step 2 is the greedy commit by default; ``commit`` swaps in another
per-step rule with the same outputs (the sampled commit of
:mod:`oracle.sampling`, which follows the digest's method step 6 settings
temperature / top-k / top-p), leaving the loop itself unchanged.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .commit import FALLBACK_TOP1, confidence_commit


def decode_loop(n_seq: int, blk_len: int, logits_for_step: Callable[[int], np.ndarray],
                threshold: float, fallback: str = FALLBACK_TOP1, max_steps: int = 10_000,
                commit: Optional[Callable[..., dict]] = None):
    """Run the loop; ``logits_for_step(step)`` returns ``[n_seq*blk_len, V]`` logits.

    ``commit(logits, tokens, masked, blk_len, threshold, fallback, step)`` is one
    commit step (default: :func:`oracle.commit.confidence_commit`, which takes no
    step).

    Returns ``steps`` (per sequence: the step count at which its block finished,
    or -1 if it never did), the final ``tokens`` and ``masked``, and
    ``commit_step`` (per row, the step at which it was committed).
    """
    R = n_seq * blk_len
    tokens = np.full(R, -1, dtype=np.int32)
    masked = np.ones(R, dtype=np.uint8)
    steps = np.full(n_seq, -1, dtype=np.int64)
    commit_step = np.full(R, -1, dtype=np.int64)
    step = 0
    while masked.any() and step < max_steps:
        if commit is None:
            res = confidence_commit(logits_for_step(step), tokens, masked, blk_len, threshold, fallback)
        else:
            res = commit(logits_for_step(step), tokens, masked, blk_len, threshold, fallback, step)
        commit_step[res["committed"]] = step
        tokens, masked = res["tokens"], res["masked"]
        for g in range(n_seq):
            if steps[g] < 0 and res["n_masked_left"][g] == 0:
                steps[g] = step + 1
        step += 1
    return {"steps": steps, "tokens": tokens, "masked": masked, "commit_step": commit_step,
            "total_steps": step}
