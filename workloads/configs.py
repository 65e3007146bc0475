"""The five workloads the library is measured and parity-tested on.

Shapes follow the video-DiT setting of "Minute-Long Videos with Dual
Parallelisms" (arXiv 2505.21070): a block of latent frames (4 frames of a
30x45 token grid at 480p, 5 frames of 30x52 at 720p) attends over the cached
keys/values of its neighbouring block, its own keys/values and the text keys.
The token grids, head counts and text lengths are the stated workload sizes;
the pages print none of them, they fix only 480p/720p and the block scheme.
"""
from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    dtype: str            # "f32" or "bf16"
    n_blocks: int
    heads: int
    head_dim: int
    q_len: int            # queries per block (= tokens of the current block)
    ctx_len: int          # cached keys of the neighbouring block (0: none)
    cur_len: int          # keys of the block itself
    text_len: int         # text-conditioning keys
    std: float            # inputs are N(0, 1) * std
    seed: int
    frames_per_block: int
    # Ring plan: n_slots of the ring, and per block the ordered list of
    # (slot, length) segments that make up its cached keys (ctx..., cur).
    n_slots: int = 2
    segs: Tuple[Tuple[Tuple[int, int], ...], ...] = field(default_factory=tuple)
    timesteps: Tuple[int, ...] = ()   # per-block integer timestep for the update
    full_sequence: bool = False       # config 4: queries = the whole prefix

    @property
    def key_len(self) -> int:
        return sum(l for _, l in self.segs[0]) + self.text_len

    @property
    def slot_tokens(self) -> int:
        return max(l for b in self.segs for _, l in b)

    def flops(self) -> int:
        """Algorithmic attention FLOPs: QK^T plus PV over valid keys only."""
        return 4 * self.q_len * self.key_len * self.head_dim * self.heads * self.n_blocks

    @property
    def latent_frames(self) -> int:
        return self.frames_per_block * self.n_blocks

    @property
    def update_elems(self) -> int:
        # one block of latents: frames x 16 channels x (2*grid_h) x (2*grid_w);
        # equals q_len * 64 for the 30x45 grid (2x2 patches of a 60x90 latent).
        return self.q_len * 64


def _cfg3_segs():
    # 8 queued blocks, absolute ids 13..20, generation 5, 16 slots: the
    # current block of id k sits in slot 2*(k mod 8) + (g mod 2), its context
    # (block k-1 of the previous generation) in 2*((k-1) mod 8) + ((g-1) mod 2).
    g = 5
    segs = []
    for b in range(8):
        k = 13 + b
        cur = 2 * (k % 8) + (g % 2)
        ctx = 2 * ((k - 1) % 8) + ((g - 1) % 2)
        segs.append(((ctx, 5400), (cur, 5400)))
    return tuple(segs)


CONFIGS: List[Config] = [
    Config(0, "tiny-f32", "f32", 1, 2, 64, 128, 128, 128, 16, 1.0, 20251, 2,
           n_slots=2, segs=(((0, 128), (1, 128)),), timesteps=(500,)),
    Config(1, "dit-480p-block", "bf16", 1, 24, 64, 5400, 5400, 5400, 226, 0.5, 20252, 4,
           n_slots=2, segs=(((0, 5400), (1, 5400)),), timesteps=(500,)),
    Config(2, "dit-720p-block", "bf16", 1, 40, 128, 7800, 7800, 7800, 512, 0.5, 20253, 5,
           n_slots=2, segs=(((0, 7800), (1, 7800)),), timesteps=(500,)),
    Config(3, "queued-8-blocks", "bf16", 8, 24, 64, 5400, 5400, 5400, 226, 0.5, 20254, 4,
           n_slots=16, segs=_cfg3_segs(),
           timesteps=tuple(1 + (999 * b) // 7 for b in range(8))),
    Config(4, "full-sequence-3heads", "bf16", 1, 3, 64, 43200, 0, 43200, 226, 0.5, 20255, 32,
           n_slots=8, segs=(tuple((s, 5400) for s in range(8)),), timesteps=(500,),
           full_sequence=True),
]


def config_by_index(i: int) -> Config:
    return CONFIGS[i]
