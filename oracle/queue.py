"""Single-GPU FIFO block queue (oracle side; test infrastructure only).

Block-wise denoising as the pith.science verdict on "Minute-Long Videos with
Dual Parallelisms" describes it (pith_extraction.key_machinery): the queued
blocks are ordered with decreasing noise from tail to head; every step
appends a new noisy block at the tail and pops a clean block at the head.
The feature cache (the page's Abstract) lets a block reuse the K/V its
neighbour produced as attention context; in the pipelined original those
features are one step old (the verdict's referee report on its section 3.2).

Restated here as plain rules, one queue position at a time:
  * n_queue blocks; position i (0 = head) holds block id k = head_id + i,
    kept in latent slot k mod n_queue;
  * before step g block i sits at t = (i + 1) * T / n_queue and the step
    takes it one rung down (stride T / n_queue); the head leaves at t = 0;
  * at step g block k writes its K/V into ring slot 2 * (k mod n_queue) +
    g mod 2, and (for g > 0) reads the K/V of block k - 1 from step g - 1
    (slot 2 * ((k - 1) mod n_queue) + (g - 1) mod 2), then its own, then the
    text.

The stand-in layer of the queue test (no trained weights): a block's latents,
viewed as [tokens][heads][head_dim], are its queries, keys and values, and
the attention output is the model's prediction for the update.
"""


def plan(n_queue, T, block_tokens, text_len, step, head_id):
    """The step's plan by latent slot: list of dicts with keys write_slot,
    meta (q_len, segs, text_slot, text_len) and t; plus the stride."""
    stride = T // n_queue
    out = [None] * n_queue
    for i in range(n_queue):
        k = head_id + i
        write = 2 * (k % n_queue) + step % 2
        segs = []
        if step > 0:
            segs.append((2 * ((k - 1) % n_queue) + (step - 1) % 2, block_tokens))
        segs.append((write, block_tokens))
        out[k % n_queue] = {
            "write_slot": write,
            "meta": {"q_len": block_tokens, "segs": segs, "text_slot": 0, "text_len": text_len},
            "t": (i + 1) * stride,
            "block": k,
        }
    return out, stride
