"""Single-GPU FIFO block queue over the library's calls.

Block-wise denoising as the pith.science verdict on "Minute-Long Videos with
Dual Parallelisms" describes it (pith_extraction.key_machinery): the queued
blocks sit at decreasing noise levels from tail to head, and each step
appends a new noisy block at the tail and pops a clean one at the head.  The
bookkeeping (which ring slot each block writes and reads, each block's
timestep) is the library's ba_queue_*; every step of the data path runs in
the library's kernels: ba_cache_append_batched, ba_block_attention (one
launch over all queued blocks), ba_block_update (each block at its own t).

The model between those calls is a stand-in without trained weights.  By
default a block's latents, viewed as [tokens][heads][head_dim], are its
queries, keys and values.  With a projection layer (a weight W of
[3 heads head_dim][heads head_dim], random in the tests and the bench, and an
optional rotation table) every block's latents, viewed as [tokens][dim], go
through one ba_qkv_project_batched launch instead, which writes K and V
straight into each block's ring slot (no append) and Q to a buffer.  Either way the attention
output is the prediction the update consumes (the noise for DDIM, the
velocity for flow matching).
"""
import torch

from . import (BA_BF16, ba_block_attention, ba_block_update, ba_cache_append, ba_cache_append_batched,
               ba_noise_assign, ba_noise_block, ba_qkv_project_batched, ba_queue_advance, ba_queue_init,
               ba_queue_plan, ba_queue_ring_slots, ba_ring_init)


class FifoQueue:
    """latents: [n_queue][tokens][heads][head_dim] bf16 on the GPU, latent
    slot m holding the block at queue position m (the head first) at
    timestep (m + 1) T / n_queue.  text_k, text_v: [text_len][heads][head_dim]
    or None.  kind: "ddim" or "flow" (with shift).  noise: optional dict
    {"pool": [channels][pool_frames][...] bf16, "n_exclude": e, "seed": s}:
    a step without a new block then draws the new tail block from the pool
    (coordinated noise initialisation), its latents viewed as
    [channels][block_frames][...] with the pool's frame size.  layer:
    optional dict {"w": [3 H D][H D] bf16, "rope": [D/2][tokens][2] fp32 or
    None}: the QKV projection layer described above."""

    def __init__(self, latents, text_k=None, text_v=None, T=1000, kind="ddim", shift=1.0, workspace="auto",
                 noise=None, layer=None):
        if latents.dtype != torch.bfloat16 or latents.dim() != 4:
            raise ValueError("latents must be [n_queue][tokens][heads][head_dim] bf16")
        n, L, H, D = latents.shape
        text_len = 0 if text_k is None else int(text_k.shape[0])
        self.q = ba_queue_init(n, T, L, text_len)
        self.ring = ba_ring_init(ba_queue_ring_slots(n), L, H, D, BA_BF16, device=latents.device)
        self.text = None
        if text_len:
            self.text = ba_ring_init(1, text_len, H, D, BA_BF16, device=latents.device)
            ba_cache_append(self.text, text_k, text_v, text_len)
        self.x = latents
        self.pred = torch.empty_like(latents)
        self.T, self.kind, self.shift, self.workspace = T, kind, shift, workspace
        self.last_plan = None
        self.layer = layer
        self.qbuf = None
        if layer is not None:
            if tuple(layer["w"].shape) != (3 * H * D, H * D) or layer["w"].dtype != torch.bfloat16:
                raise ValueError("layer w must be [3 heads head_dim][heads head_dim] bf16")
            self.qbuf = torch.empty_like(latents)
        self.noise = noise
        if noise is not None:
            pool = noise["pool"]
            frame = pool[0, 0].numel()
            per_block = L * H * D
            if pool.dtype != torch.bfloat16 or per_block % (pool.shape[0] * frame):
                raise ValueError("a block's latents must be a whole number of the pool's frames per channel")
            self.block_frames = per_block // (pool.shape[0] * frame)

    @property
    def head_slot(self):
        """Latent slot of the current head block."""
        return self.q.head_id % self.q.n_queue

    def new_block_frames(self):
        """Pool frames of the block that enters at the next step."""
        nz = self.noise
        return ba_noise_assign(nz.get("seed", 0), self.q.head_id + self.q.n_queue, nz["pool"].shape[1],
                               nz.get("n_exclude", 0), self.block_frames)

    def step(self, new_block=None):
        """One queue step.  Returns the block that left the head (clean, a new
        tensor); new_block ([tokens][heads][head_dim] bf16, pure noise) takes
        its latent slot as the new tail, or, when None, the block is drawn
        from the noise pool."""
        n = self.q.n_queue
        slots, metas, t, stride = ba_queue_plan(self.q)
        self.last_plan = (slots, metas, t, stride)
        if self.layer is None:
            # keys and values are the latents themselves
            ba_cache_append_batched(self.ring, self.x, self.x, slots)
            q = self.x
        else:
            # one projection launch writes every block's K/V into its ring slot
            ba_qkv_project_batched(self.x.view(n, self.x.shape[1], -1), self.layer["w"], self.ring, slots,
                                   q=self.qbuf, rope=self.layer.get("rope"))
            q = self.qbuf
        ba_block_attention(q, self.ring, self.text, metas, out=self.pred, workspace=self.workspace)
        ba_block_update(self.x.view(n, -1), self.pred.view(n, -1), t,
                        {"kind": self.kind, "T": self.T, "stride": stride, "shift": self.shift})
        m = self.head_slot
        done = self.x[m].clone()
        if new_block is not None:
            self.x[m].copy_(new_block)
        else:
            if self.noise is None:
                raise ValueError("no new block and no noise pool")
            pool = self.noise["pool"]
            ba_noise_block(pool, self.new_block_frames(),
                           self.x[m].view(pool.shape[0], self.block_frames, *pool.shape[2:]))
        ba_queue_advance(self.q)
        return done
