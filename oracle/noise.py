"""Coordinated noise initialisation (oracle side; test infrastructure only).

"Minute-Long Videos with Dual Parallelisms", Abstract: the initial noise
patterns are shared across GPUs at no extra cost; the pith.science verdict on
it (pith_extraction.core_discovery, pith_inferences) describes the recipe as a
full noise pool, a shuffled assignment of its latents to each new block, and
the last few latents of the pool left out, so that concatenated blocks do not
repeat one noise pattern.

Reading (the pages give no formula):
  * pool: pool_frames latent frames of N(0, 1) noise, laid out
    [channels][pool_frames][frame_elems], the same on every GPU (one seed);
  * candidates: frames 0 .. m - 1 with m = pool_frames - n_exclude;
  * block b takes block_frames distinct candidates: the first block_frames
    entries of a uniformly random permutation of the candidates, drawn by a
    partial Fisher-Yates shuffle from the front (position i swaps with a
    uniform position in [i, m));
  * the random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast
    Splittable Pseudorandom Number Generators", OOPSLA 2014: a Weyl sequence
    with increment gamma = 0x9E3779B97F4A7C15, each state passed through the
    64-bit finaliser z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31).  Block b's generator starts from
    the b-th output (0-based) of the generator started from `seed`, so any
    GPU computes any block's assignment alone;
  * a uniform integer in [0, n) rejects draws below 2^64 mod n and takes the
    rest modulo n (no bias);
  * frame f of block b, channel c = pool[c][assign_b[f]].
"""
import numpy as np

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def finalise(z):
    """The SplitMix64 output function of one 64-bit state."""
    z &= MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


class SplitMix64:
    def __init__(self, seed):
        self.state = seed & MASK

    def next(self):
        self.state = (self.state + GAMMA) & MASK
        return finalise(self.state)

    def below(self, n):
        """Uniform integer in [0, n), n >= 1."""
        threshold = (1 << 64) % n
        while True:
            r = self.next()
            if r >= threshold:
                return r % n


def block_generator(seed, block_id):
    g = SplitMix64(seed)
    for _ in range(block_id):
        g.next()
    return SplitMix64(g.next())


def assign(seed, block_id, pool_frames, n_exclude, block_frames):
    """Pool frames of block block_id, in the block's frame order."""
    m = pool_frames - n_exclude
    if not (0 <= n_exclude < pool_frames and 1 <= block_frames <= m and block_id >= 0):
        raise ValueError("need 0 <= n_exclude < pool_frames, 1 <= block_frames <= pool_frames - n_exclude")
    g = block_generator(seed, block_id)
    a = list(range(m))
    for i in range(block_frames):
        j = i + g.below(m - i)
        a[i], a[j] = a[j], a[i]
    return a[:block_frames]


def noise_block_ref(pool, channels, pool_frames, frames):
    """pool: [channels][pool_frames][frame_elems] (any dtype, e.g. bf16 bit
    patterns); returns [channels][len(frames)][frame_elems]."""
    p = np.asarray(pool).reshape(channels, pool_frames, -1)
    return np.stack([np.stack([p[c, f] for f in frames]) for c in range(channels)])
