"""The text K/V as plain [heads][text_cap][head_dim] arrays through the C ABI.
ba_text_ring_set must leave the text ring equal, byte for byte, to the
oracle's ring model filled with the same tokens; ba_block_attention_text_arrays
must give exactly the bits of ba_block_attention on a ring filled with the
same text, and the oracle's attention within the usual bound."""
import math

import numpy as np
import pytest
import torch

import block_wise_long_amd as B
from _util import Workload, check_contract, decode, ring_bytes, to_dev
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _token_major(a):
    """[heads][tokens][head_dim] -> [tokens][heads][head_dim] (data movement only)."""
    return np.ascontiguousarray(np.transpose(a, (1, 0, 2)))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_text_ring_set_bit_exact(dtype, D):
    # a two-slot text ring: a FIFO append into slot 0, then the arrays into
    # slot 1 (a prefix of text_cap) and again into slot 0 (a shorter text
    # over the longer one: the rest of the slot becomes zeros)
    rng = _rng(300 + D + (dtype == "f32"))
    H, S, cap = 3, 150, 170                      # T_pad = 192
    w = Workload(dtype, 2, S, H, D, 0)
    w.append(draw(rng, (S, H, D), 1.0, dtype), draw(rng, (S, H, D), 1.0, dtype))
    for slot, n in ((1, 133), (0, 65)):
        tk = draw(rng, (H, cap, D), 1.0, dtype)
        tv = draw(rng, (H, cap, D), 1.0, dtype)
        B.ba_text_ring_set(w.ring, to_dev(tk, dtype), to_dev(tv, dtype), text_len=n, slot=slot)
        w.oring.append(_token_major(tk[:, :n]), _token_major(tv[:, :n]), n, slot=slot)
        assert ring_bytes(w.ring) == w.oring.as_bytes(), (slot, n)
    assert w.ring.appended == 1


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_ws", ["ring-only", "full"])
def test_attention_with_text_arrays_same_bits_as_ring_form(D, with_ws):
    # three blocks: cache segments plus texts of different lengths (prefixes
    # of one prompt), one block without text; the arrays form against the
    # ring form on the same inputs, and both against the oracle
    rng = _rng(400 + D + (with_ws == "full"))
    H, L, cap = 4, 300, 100
    w = Workload("bf16", 3, L, H, D, cap)
    for _ in range(3):
        w.append(draw(rng, (L, H, D), 0.5, "bf16"), draw(rng, (L, H, D), 0.5, "bf16"))
    tk = draw(rng, (H, cap, D), 0.5, "bf16")
    tv = draw(rng, (H, cap, D), 0.5, "bf16")
    w.set_text(_token_major(tk), _token_major(tv))          # the ring form's text ring (and the oracle's)
    metas = [{"q_len": 300, "segs": [(0, 300), (1, 211)], "text_slot": 0, "text_len": 100},
             {"q_len": 129, "segs": [(2, 300)], "text_slot": 0, "text_len": 37},
             {"q_len": 77, "segs": [(1, 5)], "text_slot": 0, "text_len": 0}]
    q = draw(rng, (3, 300, H, D), 0.5, "bf16")
    qd = to_dev(q, "bf16")
    ring_form = torch.full_like(qd, float("nan"))
    lse_ring = torch.full((3, H, 300), float("nan"), dtype=torch.float32, device="cuda")
    B.ba_block_attention(qd, w.ring, w.text, metas, out=ring_form, lse=lse_ring, workspace=None)
    full = B.ba_attention_text_arrays_workspace_bytes(D, B.BA_BF16, 3, 300, H, cap)
    ring_only = -(-B.ba_ring_bytes(1, cap, H, D, B.BA_BF16) // 256) * 256
    nbytes = full if with_ws == "full" else ring_only
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + nbytes]
    arrays_form = torch.full_like(qd, float("nan"))
    lse_arr = torch.full((3, H, 300), float("nan"), dtype=torch.float32, device="cuda")
    B.ba_block_attention_text_arrays(qd, w.ring, to_dev(tk, "bf16"), to_dev(tv, "bf16"), metas, ws,
                                     out=arrays_form, lse=lse_arr)
    torch.cuda.synchronize()
    if with_ws == "ring-only":
        # no room for partial results: the same schedule as the ring form without a workspace
        assert torch.equal(arrays_form.view(torch.int16), ring_form.view(torch.int16))
        assert torch.equal(lse_arr.view(torch.int32), lse_ring.view(torch.int32))
    ref, ref_lse = w.oracle(q, metas)
    got = decode(arrays_form, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse_arr.cpu().numpy()[sel] - ref_lse[sel])) < 2e-3
    for b, m in enumerate(metas):
        assert np.isnan(got[b, m["q_len"]:]).all()


def test_text_arrays_with_the_480p_text_only_key_set():
    # the separate text cross-attention of a 480p block (5400 queries, 24
    # heads x 64, a 512-token prompt): the resident launch shape, whose
    # output must be the ring form's bit for bit; sampled rows against the
    # oracle
    rng = _rng(500)
    H, D, L, cap = 24, 64, 5400, 512
    w = Workload("bf16", 1, 64, H, D, cap)
    tk = draw(rng, (H, cap, D), 0.5, "bf16")
    tv = draw(rng, (H, cap, D), 0.5, "bf16")
    w.set_text(_token_major(tk), _token_major(tv))
    metas = [{"q_len": L, "segs": [], "text_slot": 0, "text_len": cap}]
    q = draw(rng, (1, L, H, D), 0.5, "bf16")
    qd = to_dev(q, "bf16")
    ring_form = B.ba_block_attention(qd, w.ring, w.text, metas, workspace=None)
    ws = torch.empty(B.ba_attention_text_arrays_workspace_bytes(D, B.BA_BF16, 1, L, H, cap) + 256,
                     dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    arrays_form = B.ba_block_attention_text_arrays(qd, w.ring, to_dev(tk, "bf16"), to_dev(tv, "bf16"), metas,
                                                   ws[off:])
    torch.cuda.synchronize()
    assert torch.equal(arrays_form.view(torch.int16), ring_form.view(torch.int16))
    heads, rows = [0, 23], list(range(0, L, 97)) + [L - 1]
    ref, _ = w.oracle(q, metas, heads=heads, rows=rows)
    got = decode(arrays_form, "bf16")
    check_contract(got[:, rows][:, :, heads], ref[:, rows][:, :, heads], "bf16", gate2=False)
