"""CPU oracle for the block-diffusion decoding hot path (TEST INFRASTRUCTURE).

This package is the plain, slow, obviously-correct definition of what the GPU
path computes, in numpy float64.  It is test infrastructure: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``block_diffusion_decoding_amd``) never imports,
calls or falls back to anything here, and nothing here imports the product path.

Sources are the five web pages about MinerU-Diffusion.  They are cited by page
title and section:

* **skill page** -- "MinerU-Diffusion: Document OCR via Diffusion Decoding"
  (skillsmp.com), section "The Swap: Diffusion Decoder with Block-Wise
  Attention" (its pseudocode is garbled; read for intent only).
* **abstract page** -- "MinerU-Diffusion: Rethinking Document OCR as Inverse
  Rendering via Diffusion Decoding" (mlsanity.com), "Abstract (arXiv)".
* **digest page** -- the paper.rainbus.top digest of the same paper: the six
  method steps (step 2 block factorisation, step 3 block attention, step 4
  confidence scheduling, step 6 inference settings), the novelty paragraph
  (KV-cache reuse, the T = 0.5 .. 0.99 knob) and the weaknesses paragraph
  (fixed block size 32).
* **editorial page** -- "MinerU-Diffusion reads documents with diffusion decoding
  instead of left to right" (hysenlabs.com), sections "The idea: OCR as inverse
  rendering" and "FAQ".
* **blog page** -- the OpenDataLab team's post on gitcode.csdn.net, Fig. 1
  (confirmed / updating / masked tokens) and Fig. 2 (block-attention mask).

Modules:

* :mod:`oracle.attention` -- block-causal attention forward and backward, and
  one block against a prefix KV cache.
* :mod:`oracle.commit` -- max-softmax confidence and the threshold commit.
* :mod:`oracle.decode_loop` -- the per-block denoising loop as a state machine.
* :mod:`oracle.lmhead` -- the output projection feeding the commit (logits =
  hidden x weight^T), for the fused projection + confidence kernel.
* :mod:`oracle.sampling` -- the commit with sampled predictions (temperature,
  inverse-CDF sampling from a counter-based generator).
* :mod:`oracle.paged` -- the prefix cache in pages (gather through the page
  table, append a finished block).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than
itself (library routines in special cases, closed forms, invariants, brute
force and finite differences).  No function here is "parity unpinned".
"""

from . import attention, commit, decode_loop, lmhead, paged, sampling  # noqa: F401
