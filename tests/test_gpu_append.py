"""Cache append through the C ABI: the device ring must equal the oracle's
byte-level ring model bit for bit (FIFO wrap, ragged token counts, batched
slots, both dtypes and head dims)."""
import numpy as np
import pytest

from _util import Workload, ring_bytes
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_fifo_append_wraps_bit_exact(dtype, D):
    rng = _rng(100 + D)
    H, n_slots, slot_tokens = 3, 3, 150          # T_pad = 192: ragged slot
    w = Workload(dtype, n_slots, slot_tokens, H, D, 0)
    lens = [150, 1, 64, 65, 149, 127, 150]     # 7 appends into 3 slots
    slots = []
    for n in lens:
        k = draw(rng, (n, H, D), 1.0, dtype)
        v = draw(rng, (n, H, D), 1.0, dtype)
        slots.append(w.append(k, v))
        assert ring_bytes(w.ring) == w.oring.as_bytes()
    assert slots == [0, 1, 2, 0, 1, 2, 0]
    assert w.ring.appended == 7


def test_batched_append_parity_scheme_bit_exact():
    # 8 queued blocks into a 16-slot ring, current/context slots by generation parity
    rng = _rng(7)
    H, D, n = 2, 64, 200
    w = Workload("bf16", 16, n, H, D, 0)
    g = 5
    cur = [2 * ((13 + b) % 8) + g % 2 for b in range(8)]
    ctx = [2 * ((12 + b) % 8) + (g - 1) % 2 for b in range(8)]
    for slots in (ctx, cur):
        k = draw(rng, (8, n, H, D), 0.5, "bf16")
        v = draw(rng, (8, n, H, D), 0.5, "bf16")
        w.append_batched(k, v, slots)
    assert ring_bytes(w.ring) == w.oring.as_bytes()
    assert w.ring.appended == 0


def test_rejected_append_leaves_ring_alone():
    import block_wise_long_amd as B
    w = Workload("bf16", 2, 64, 1, 64, 0)
    k = draw(_rng(1), (65, 1, 64), 1.0, "bf16")
    from _util import to_dev
    with pytest.raises(B.BlockAttnError) as e:
        B.ba_cache_append(w.ring, to_dev(k, "bf16"), to_dev(k, "bf16"), 65)
    assert e.value.status == B.BA_ERR_OUT_OF_RANGE
    assert w.ring.appended == 0
    with pytest.raises(B.BlockAttnError):
        B.ba_cache_append_batched(w.ring, to_dev(k, "bf16"), to_dev(k, "bf16"), [1, 1])
    assert ring_bytes(w.ring) == w.oring.as_bytes()


def test_batched_append_more_slots_than_one_launch_takes():
    # 70 blocks: launches of 64 and 6 slots, bit-exact against the ring model
    rng = _rng(70)
    H, D, n, nb = 1, 64, 40, 70
    w = Workload("bf16", 80, n, H, D, 0)
    slots = [(7 * b + 3) % 80 for b in range(nb)]          # distinct, scattered
    assert len(set(slots)) == nb
    k = draw(rng, (nb, n, H, D), 0.5, "bf16")
    v = draw(rng, (nb, n, H, D), 0.5, "bf16")
    w.append_batched(k, v, slots)
    assert ring_bytes(w.ring) == w.oring.as_bytes()


@pytest.mark.parametrize("dtype,D,H,n,slot_tokens", [
    ("bf16", 64, 120, 1050, 1060),   # T_pad 1088: the last 128-token tile ends half past the slot
    ("f32", 128, 64, 2000, 2000),    # T_pad 2048
    ("bf16", 128, 40, 3333, 3400),   # ragged count, T_pad 3456 (27 tiles of 128)
])
def test_large_appends_take_long_tiles_bit_exact(dtype, D, H, n, slot_tokens):
    # enough work for the 128-token tiles (at least 1024 workgroups), with
    # ragged counts and slot strides that are not a multiple of 128
    rng = _rng(300 + D + H)
    w = Workload(dtype, 2, slot_tokens, H, D, 0)
    for m in (slot_tokens, n):
        k = draw(rng, (m, H, D), 1.0, dtype)
        v = draw(rng, (m, H, D), 1.0, dtype)
        w.append(k, v)
    assert ring_bytes(w.ring) == w.oring.as_bytes()
