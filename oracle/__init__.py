"""CPU oracle for block-wise video-DiT attention: TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 restatement of what the library computes, written from the
method's description and the textbook definitions it builds on.  Nothing here
is part of the product: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP path (``block_wise_long_amd``) and imports nothing from it.

Sources (cited by page title and section):
  * "Minute-Long Videos with Dual Parallelisms" (arXiv 2505.21070), Abstract:
    block-wise denoising with per-block noise levels; a per-GPU feature cache
    that stores the prior block's features and reuses them as context.
  * The pith.science verdict on arXiv 2505.21070: ``pith_extraction``
    (key_machinery, core_discovery) for the FIFO queue of blocks and the
    self-attention K/V cache of the neighbouring block; ``referee_report``
    major comment 2 (paper section 3.2) for the cache being read one
    denoising step after it was written.
  * "Attention Is All You Need" (listed by title among the works the DualParal
    page builds on) for scaled dot-product attention.
  * "Denoising Diffusion Probabilistic Models" (listed by title on the same
    page) for the linear beta schedule and "Denoising Diffusion Implicit
    Models" (listed by title on the Vchitect-2.0 page) for the deterministic
    update; both restated from the published methods.

Modules:
  numerics   exact bf16 <-> fp64 conversion (own implementation)
  attention  softmax(QK^T * scale) V over the [cache segments | text] key set,
             and the separate text cross-attention (two softmaxes) with the
             merge of two disjoint key sets' results
  ring       byte-level model of the K/V ring buffer's documented layout
  schedule   DDPM linear betas, alpha-bar table, DDIM (eta = 0) block update,
             and the flow-matching (rectified flow, Euler) variant
  queue      the single-GPU FIFO block queue: which ring slots a step writes
             and reads, and each block's timestep
  projection the fused K/V producer: QKV projection and the pair rotation
  noise      coordinated noise initialisation: shuffled assignment of a shared
             noise pool's frames to each new block (SplitMix64, partial
             Fisher-Yates) and the frame gather
"""
from . import numerics, attention, ring, schedule, queue, projection, noise  # noqa: F401
