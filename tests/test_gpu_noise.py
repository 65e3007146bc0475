"""Coordinated noise initialisation through the C ABI: the block's frames
gathered from the shared pool, byte for byte against the oracle's gather of
the oracle's assignment; guard bands around the output untouched; the FIFO
queue drawing each new tail block from the pool."""
import numpy as np
import pytest

from _util import to_dev, to_host_bits
from oracle import noise as NZ
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


@pytest.mark.parametrize("C,F,E,excl,bf,dtype", [
    (16, 21, 5400, 3, 4, "bf16"),       # 480p latent frame plane (60 x 90), 4-frame block
    (16, 21, 6240, 1, 5, "bf16"),       # 720p plane (60 x 104), 5-frame block
    (3, 9, 24, 0, 9, "bf16"),           # three vectors per frame: ragged against the grid
    (1, 4, 1 << 21, 1, 3, "bf16"),      # 4 MB frames: grid-stride loop
    (2, 7, 20, 2, 5, "f32"),            # any element type
])
def test_gather_matches_oracle(C, F, E, excl, bf, dtype):
    import torch
    import block_wise_long_amd as B
    rng = _rng(C * 1000 + E)
    pool = draw(rng, (C, F, E), 1.0, dtype)
    frames = B.ba_noise_assign(20251, 17, F, excl, bf)
    assert frames == NZ.assign(20251, 17, F, excl, bf)
    dp = to_dev(pool, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    guard = 64
    buf = torch.full((C * bf * E + 2 * guard,), float("nan"), dtype=tdt, device="cuda")
    out = buf[guard:guard + C * bf * E].view(C, bf, E)
    B.ba_noise_block(dp, frames, out)
    torch.cuda.synchronize()
    ref = NZ.noise_block_ref(pool, C, F, frames)
    got = to_host_bits(out) if dtype == "bf16" else out.cpu().numpy()
    assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))
    rest = torch.cat([buf[:guard], buf[-guard:]])
    assert torch.isnan(rest).all()                      # nothing outside the block written


def test_queue_draws_new_blocks_from_the_pool():
    import torch
    from block_wise_long_amd.fifo import FifoQueue
    rng = _rng(9)
    n, L, H, D, T = 3, 120, 2, 64, 30
    C, F, excl = 4, 13, 2
    block_elems = L * H * D                      # 15360 = 4 channels x 3 frames x 1280
    E = block_elems // (C * 3)
    pool = draw(rng, (C, F, E), 1.0, "bf16")
    fq = FifoQueue(to_dev(draw(rng, (n, L, H, D), 0.5, "bf16"), "bf16"), T=T,
                   noise={"pool": to_dev(pool, "bf16"), "n_exclude": excl, "seed": 77})
    assert fq.block_frames == 3
    for g in range(2 * n + 1):
        head = fq.head_slot
        new_id = fq.q.head_id + n
        fq.step()
        torch.cuda.synchronize()
        frames = NZ.assign(77, new_id, F, excl, 3)
        ref = NZ.noise_block_ref(pool, C, F, frames)
        got = to_host_bits(fq.x)[head].reshape(C, 3, E)
        assert np.array_equal(got, ref), g


def test_gather_at_the_grid_limit():
    # channels x block_frames = 64 x 64 = 4096 grid rows, frames of one vector
    import torch
    import block_wise_long_amd as B
    rng = _rng(4096)
    C, F, E, bf = 64, 70, 8, 64
    pool = draw(rng, (C, F, E), 1.0, "bf16")
    frames = B.ba_noise_assign(9, 3, F, 6, bf)
    out = torch.empty((C, bf, E), dtype=torch.bfloat16, device="cuda")
    B.ba_noise_block(to_dev(pool, "bf16"), frames, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out), NZ.noise_block_ref(pool, C, F, frames))
