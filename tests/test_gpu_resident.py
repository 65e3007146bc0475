"""The resident-key-set attention kernel (head dim 64, key sets of at most 8
tiles of 64 keys held whole in LDS, independent 32-query units) against the
fp64 oracle: ranges of units that cross heads and blocks, ragged tiles in
the middle of a key set, a per-wave exact re-run, and bit equality with the
streaming kernel on the same block."""
import math

import numpy as np
import pytest

from _util import Workload, check_contract, decode
from oracle import numerics as N
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _resident(units):
    # the resident kernel runs when a launch has at least 12 units of 32
    # queries per CU; below that the same key sets take the narrow kernel
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if units < 12 * cus:
        pytest.skip(f"{units} units < 12 x {cus} CUs: the launch would take the narrow kernel")


def _bar(got, ref):
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms


def test_ranges_cross_heads_and_blocks():
    # 5 blocks x 16 heads, 4064 units of 32 queries over 256 workgroups: many
    # workgroups run two (block, head) phases, each with its own key set
    # copy; partial tiles at every segment end, blocks of 37, 0 and 1 queries
    import block_wise_long_amd as B
    rng = _rng(81)
    H, D = 16, 64
    w = Workload("bf16", 3, 200, H, D, 100)
    for n in (200, 37, 64):
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (100, H, D), 0.5, "bf16"), draw(rng, (100, H, D), 0.5, "bf16"))
    metas = [{"q_len": 5000, "segs": [(0, 200), (1, 37)], "text_slot": 0, "text_len": 100},   # 7 tiles
             {"q_len": 37, "segs": [(2, 64)], "text_slot": 0, "text_len": 0},                  # 1 tile
             {"q_len": 0, "segs": [(2, 64)], "text_slot": 0, "text_len": 0},
             {"q_len": 3000, "segs": [(1, 37), (0, 200), (2, 1)], "text_slot": 0, "text_len": 60},  # 7
             {"q_len": 1, "segs": [], "text_slot": 0, "text_len": 100}]                       # 2
    _resident(H * sum((m["q_len"] + 31) // 32 for m in metas))
    assert B.ba_attention_query_tile(D, B.BA_BF16, 301) == 32
    q = draw(rng, (5, 5000, H, D), 0.5, "bf16")
    out, lse = w.run(q, metas)
    heads = [0, 9, 15]
    ref, ref_lse = w.oracle(q, metas, heads=heads)
    got = decode(out, "bf16")
    _bar(got[:, :, heads], ref[:, :, heads])
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < 2e-3
    for b, m in enumerate(metas):            # rows past each q_len untouched
        assert np.isnan(got[b, m["q_len"]:]).all()


def test_many_units_per_wave():
    # 24 heads x 4200 queries over a 512-key text set: 3168 units, about 12
    # per workgroup, every head's last unit ragged (4200 = 131.25 x 32)
    rng = _rng(82)
    H, D, L, TXT = 24, 64, 4200, 512
    _resident(H * ((L + 31) // 32))
    w = Workload("bf16", 1, 64, H, D, TXT)
    w.set_text(draw(rng, (TXT, H, D), 0.5, "bf16"), draw(rng, (TXT, H, D), 0.5, "bf16"))
    metas = [{"q_len": L, "segs": [], "text_slot": 0, "text_len": TXT}]
    q = draw(rng, (1, L, H, D), 0.5, "bf16")
    out, lse = w.run(q, metas)
    heads = [0, 5, 11, 23]
    ref, ref_lse = w.oracle(q, metas, heads=heads)
    got = decode(out, "bf16")
    _bar(got[:, :, heads], ref[:, :, heads])
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < 2e-3


@pytest.mark.parametrize("growth", [6.0, 90.0, 300.0])
def test_scores_rising_along_the_keys_some_waves_rerun(growth):
    # scores rise along 500 keys by `growth` (exp2 domain) for the queries of
    # even 32-query units and by a tenth of it for the others: at 300 the
    # even units' fast pass overflows and those waves alone run their unit
    # again in the exact form, next to waves whose fast pass stands
    rng = _rng(83 + int(growth))
    H, D, L, nq = 8, 64, 500, 12320
    _resident(H * nq // 32)
    w = Workload("bf16", 1, L, H, D, 0)
    k = np.zeros((L, H, D))
    k[:, :, 0] = (growth / math.log2(math.e)) * np.arange(L)[:, None] / L
    k[:, :, 1] = N.bf16_bits_to_f64(draw(rng, (L, H), 0.25, "bf16"))
    w.append(N.f64_to_bf16_bits(k), draw(rng, (L, H, D), 1.0, "bf16"))
    q = np.zeros((1, nq, H, D))
    q[..., 0] = np.where((np.arange(nq) // 32) % 2 == 0, 1.0, 0.1)[:, None]
    q[..., 1] = N.bf16_bits_to_f64(draw(rng, (1, nq, H), 1.0, "bf16"))
    qb = N.f64_to_bf16_bits(q)
    metas = [{"q_len": nq, "segs": [(0, L)], "text_slot": 0, "text_len": 0}]
    out, lse = w.run(qb, metas, scale=1.0)
    heads = [0, 3, 7]
    rows = sorted(set(range(0, 256)) | set(range(0, nq, 61)) | set(range(nq - 64, nq)))
    ref, ref_lse = w.oracle(qb, metas, scale=1.0, heads=heads, rows=rows)
    got = decode(out, "bf16")[:, rows][:, :, heads]
    ref = ref[:, rows][:, :, heads]
    assert not np.isnan(got).any()
    assert np.max(np.abs(got - ref)) <= 2 ** -6 * max(1.0, np.max(np.abs(ref)))
    gl = lse.cpu().numpy()[:, heads][:, :, rows]
    rl = ref_lse[:, heads][:, :, rows]
    assert np.max(np.abs(gl - rl) / np.maximum(1, np.abs(rl))) < 1e-3


def test_same_bits_as_the_streaming_kernel():
    # Block 0's key set (7 tiles, 3168 units) alone takes the resident
    # kernel; beside a block of 10 tiles the same launch takes the streaming
    # (narrow) one.  Both run the same per-group arithmetic in the same
    # order, so block 0's outputs and log-sum-exps agree bit for bit.
    import torch
    import block_wise_long_amd as B
    rng = _rng(84)
    H, D, L = 24, 64, 4200
    _resident(H * ((L + 31) // 32))
    w = Workload("bf16", 3, 300, H, D, 64)
    for n in (300, 150, 290):
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (64, H, D), 0.5, "bf16"), draw(rng, (64, H, D), 0.5, "bf16"))
    m0 = {"q_len": L, "segs": [(0, 300), (1, 37)], "text_slot": 0, "text_len": 50}      # 5 + 1 + 1 tiles
    m9 = {"q_len": L, "segs": [(0, 300), (2, 290)], "text_slot": 0, "text_len": 0}      # 5 + 5
    assert B.ba_attention_query_tile(D, B.BA_BF16, 387) == 32
    q = draw(rng, (2, L, H, D), 0.5, "bf16")
    # no workspace: the streaming launch runs whole tasks (no cut, no merge)
    out_r, lse_r = w.run(q[:1], [m0], workspace=None)
    out_s, lse_s = w.run(q, [m0, m9], workspace=None)
    assert torch.equal(out_r[0].view(torch.int16), out_s[0].view(torch.int16))
    assert torch.equal(lse_r[0].view(torch.int32), lse_s[0].view(torch.int32))
    heads, rows = [0, H - 1], list(range(0, L, 37)) + [L - 1]
    ref, _ = w.oracle(q, [m0, m9], heads=heads, rows=rows)
    got = decode(out_s, "bf16")
    _bar(got[:, rows][:, :, heads], ref[:, rows][:, :, heads])


def test_eight_tiles_from_four_segments():
    # the largest resident key set, made of three cache segments and the text
    # (128 + 64 + 100 + 140 keys: 2 + 1 + 2 + 3 = 8 tiles, a partial tile
    # inside the key set and one at its end); 16 heads x 6144 queries
    import block_wise_long_amd as B
    rng = _rng(85)
    H, D, L = 16, 64, 6144
    _resident(H * L // 32)
    w = Workload("bf16", 3, 128, H, D, 140)
    for n in (128, 64, 100):
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (140, H, D), 0.5, "bf16"), draw(rng, (140, H, D), 0.5, "bf16"))
    metas = [{"q_len": L, "segs": [(0, 128), (1, 64), (2, 100)], "text_slot": 0, "text_len": 140}]
    assert B.ba_attention_query_tile(D, B.BA_BF16, 432) == 32
    q = draw(rng, (1, L, H, D), 0.5, "bf16")
    out, lse = w.run(q, metas)
    heads, rows = [0, 7, 15], sorted(set(range(0, L, 41)) | set(range(L - 40, L)))
    ref, ref_lse = w.oracle(q, metas, heads=heads, rows=rows)
    got = decode(out, "bf16")
    _bar(got[:, rows][:, :, heads], ref[:, rows][:, :, heads])
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < 2e-3


def test_eight_segments_in_one_resident_key_set():
    # the most cache segments a block takes, one of them empty, each at most
    # one tile, in an order unlike their slots', plus a text of 30 keys:
    # 7 + 1 = 8 tiles, every one of them partial but two
    import block_wise_long_amd as B
    rng = _rng(86)
    H, D, L = 16, 64, 6144
    _resident(H * L // 32)
    w = Workload("bf16", 8, 64, H, D, 30)
    lens = (64, 1, 63, 33, 64, 17, 40, 5)
    for n in lens:
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (30, H, D), 0.5, "bf16"), draw(rng, (30, H, D), 0.5, "bf16"))
    segs = [(6, 40), (0, 64), (3, 33), (7, 0), (1, 1), (5, 17), (4, 64), (2, 63)]
    assert len(segs) == B.BA_MAX_SEGS
    metas = [{"q_len": L, "segs": segs, "text_slot": 0, "text_len": 30}]
    assert B.ba_attention_query_tile(D, B.BA_BF16, sum(n for _, n in segs) + 30) == 32
    q = draw(rng, (1, L, H, D), 0.5, "bf16")
    out, lse = w.run(q, metas)
    heads, rows = [0, 8, 15], sorted(set(range(0, L, 43)) | set(range(L - 33, L)))
    ref, ref_lse = w.oracle(q, metas, heads=heads, rows=rows)
    got = decode(out, "bf16")
    _bar(got[:, rows][:, :, heads], ref[:, rows][:, :, heads])
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < 2e-3


def test_per_head_workgroups_same_bits_as_contiguous_ranges():
    # one 480p block over a 512-key text: each of its 24 heads takes whole
    # workgroups (no workgroup copies two key sets); the same block beside a
    # block of another query count is cut into contiguous ranges that cross
    # heads.  A unit's arithmetic does not depend on the workgroup that runs
    # it, so the block's outputs and log-sum-exps agree bit for bit.
    import torch
    rng = _rng(87)
    H, D, L, TXT = 24, 64, 5400, 512
    _resident(H * ((L + 31) // 32))
    w = Workload("bf16", 1, 64, H, D, TXT)
    w.set_text(draw(rng, (TXT, H, D), 0.5, "bf16"), draw(rng, (TXT, H, D), 0.5, "bf16"))
    m0 = {"q_len": L, "segs": [], "text_slot": 0, "text_len": TXT}
    m1 = {"q_len": 1000, "segs": [], "text_slot": 0, "text_len": TXT}
    q = draw(rng, (2, L, H, D), 0.5, "bf16")
    out_a, lse_a = w.run(q[:1], [m0], workspace=None)
    out_c, lse_c = w.run(q, [m0, m1], workspace=None)
    assert torch.equal(out_a[0].view(torch.int16), out_c[0].view(torch.int16))
    assert torch.equal(lse_a[0].view(torch.int32), lse_c[0].view(torch.int32))
    heads, rows = [0, 12, 23], sorted(set(range(0, L, 59)) | set(range(L - 8, L)))
    ref, _ = w.oracle(q[:1], [m0], heads=heads, rows=rows)
    got = decode(out_a, "bf16")
    _bar(got[:, rows][:, :, heads], ref[:, rows][:, :, heads])
