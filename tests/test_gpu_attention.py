"""Block attention through the C ABI against the fp64 oracle, element by
element, at sizes the oracle finishes in seconds that still span several
query and key tiles with ragged tails; plus the discriminating cases:
needles (indexing proven bit-exact through the attention kernel), V = 1,
q = 0, segment order, the lazy-maximum path and the degenerate shapes."""
import math

import numpy as np
import pytest

from _util import Workload, check_contract, decode, to_dev
from oracle import numerics as N
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _fill(w, rng, lens, H, D, dtype, std, text_len):
    for n in lens:
        w.append(draw(rng, (n, H, D), std, dtype), draw(rng, (n, H, D), std, dtype))
    if text_len:
        w.set_text(draw(rng, (text_len, H, D), std, dtype), draw(rng, (text_len, H, D), std, dtype))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("q_len,lens,text_len", [
    (300, (200, 150), 37),       # ragged everywhere: 3 query tiles, tails in every segment
    (128, (128, 128), 16),       # exact tiles
    (1, (1,), 0),                # a single query over a single key
    (257, (64, 65, 63), 64),     # tile-boundary lengths
    (300, (200, 200, 150), 37),  # 12 key tiles: past the resident limit at head dim 64
])
def test_bf16_parity_small(D, q_len, lens, text_len):
    rng = _rng(D * 1000 + q_len)
    H = 3
    w = Workload("bf16", 3, 200, H, D, 64)
    _fill(w, rng, lens, H, D, "bf16", 0.5, text_len)
    q = draw(rng, (1, q_len, H, D), 0.5, "bf16")
    metas = [{"q_len": q_len, "segs": [(i, n) for i, n in enumerate(lens)], "text_slot": 0,
              "text_len": text_len}]
    out, lse = w.run(q, metas)
    ref, ref_lse = w.oracle(q, metas)
    # outputs here are larger than at the video shapes (fewer keys), so the
    # secondary gate is scaled by the output's rms
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    mx = np.nanmax(np.abs(got - ref))
    assert mx <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms, mx
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3


@pytest.mark.parametrize("D", [64, 128])
def test_f32_parity(D):
    rng = _rng(D)
    H, q_len = 2, 130
    w = Workload("f32", 2, 140, H, D, 16)
    _fill(w, rng, (140, 77), H, D, "f32", 1.0, 16)
    q = draw(rng, (2, q_len, H, D), 1.0, "f32")
    metas = [{"q_len": 130, "segs": [(0, 140), (1, 77)], "text_slot": 0, "text_len": 16},
             {"q_len": 65, "segs": [(1, 77)], "text_slot": 0, "text_len": 5}]
    out, lse = w.run(q, metas)
    ref, ref_lse = w.oracle(q, metas)
    got = out.cpu().numpy().astype(np.float64)
    check_contract(got, ref, "f32")
    assert np.isnan(got[1, 65:]).all()       # rows past q_len are not written
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse)) < 1e-5


def test_batched_blocks_with_different_key_sets():
    rng = _rng(5)
    H, D = 4, 64
    w = Workload("bf16", 6, 300, H, D, 100)
    _fill(w, rng, (300, 250, 300, 17, 300, 299), H, D, "bf16", 0.5, 100)
    q = draw(rng, (5, 280, H, D), 0.5, "bf16")
    metas = [{"q_len": 280, "segs": [(0, 300), (1, 250)], "text_slot": 0, "text_len": 100},
             {"q_len": 129, "segs": [(2, 300)], "text_slot": 0, "text_len": 0},
             {"q_len": 0, "segs": [(3, 17)], "text_slot": 0, "text_len": 3},
             {"q_len": 200, "segs": [(3, 17), (4, 300), (5, 299), (0, 1)], "text_slot": 0, "text_len": 99},
             {"q_len": 17, "segs": [(5, 0), (1, 5)], "text_slot": 0, "text_len": 1}]
    out, lse = w.run(q, metas)
    ref, ref_lse = w.oracle(q, metas)
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    # rows past each q_len stay untouched (NaN fill)
    assert np.isnan(got[1, 129:]).all() and np.isnan(got[2]).all() and np.isnan(got[4, 17:]).all()



@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_eight_segments_per_block(D, dtype):
    # the most cache segments a block takes, in an order unlike their slots'
    # and after a FIFO wrap (11 appends into 9 slots), one of them empty,
    # lengths at and around tile edges, plus the text (13 key tiles); a
    # second block of eight one-key segments and no text (8 one-key tiles)
    import block_wise_long_amd as B
    rng = _rng(880 + D + (dtype == "f32"))
    H = 2
    std = 0.5 if dtype == "bf16" else 1.0
    w = Workload(dtype, 9, 130, H, D, 40)
    held = {}
    for n in (130, 1, 63, 64, 65, 129, 17, 100, 128, 77, 33):
        held[w.append(draw(rng, (n, H, D), std, dtype), draw(rng, (n, H, D), std, dtype))] = n
    assert held == {0: 77, 1: 33, 2: 63, 3: 64, 4: 65, 5: 129, 6: 17, 7: 100, 8: 128}
    w.set_text(draw(rng, (40, H, D), std, dtype), draw(rng, (40, H, D), std, dtype))
    segs0 = [(5, 129), (0, 77), (8, 128), (3, 64), (6, 0), (2, 63), (4, 65), (1, 33)]
    segs1 = [(s, 1) for s in (7, 0, 6, 1, 5, 2, 4, 3)]
    assert len(segs0) == len(segs1) == B.BA_MAX_SEGS
    metas = [{"q_len": 300, "segs": segs0, "text_slot": 0, "text_len": 40},
             {"q_len": 45, "segs": segs1, "text_slot": 0, "text_len": 0}]
    q = draw(rng, (2, 300, H, D), std, dtype)
    out, lse = w.run(q, metas)
    ref, ref_lse = w.oracle(q, metas)
    got = decode(out, dtype)
    check_contract(got, ref, dtype, gate2=False)
    if dtype == "bf16":
        rms = math.sqrt(np.nanmean(ref ** 2))
        assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
    sel = ~np.isnan(ref_lse)
    assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < (1e-5 if dtype == "f32" else 2e-3)
    assert np.isnan(got[1, 45:]).all()

def _needle_case(D, slot_of_needle, pos, text=False):
    """One key aligned with every query, huge gap to all others: output = that key's V."""
    H, n_slots, L = 2, 3, 150
    rng = _rng(pos + 7 * D)
    w = Workload("bf16", n_slots, L, H, D, 80)
    zeros = np.zeros((L, H, D), np.uint16)
    vals = [draw(rng, (L, H, D), 1.0, "bf16") for _ in range(5)]
    # 5 FIFO appends into 3 slots: slot 0 holds append 3, slot 1 append 4 (wrap)
    for i in range(5):
        k = zeros.copy()
        if not text and i >= 3 and (i % n_slots) == slot_of_needle:
            k[pos, :, 0] = N.f64_to_bf16_bits(np.array([128.0]))[0]
        w.append(k, vals[i])
    tv = draw(rng, (80, H, D), 1.0, "bf16")
    tk = np.zeros((80, H, D), np.uint16)
    if text:
        tk[pos, :, 0] = N.f64_to_bf16_bits(np.array([128.0]))[0]
    w.set_text(tk, tv)
    q = np.zeros((1, 200, H, D), np.uint16)
    q[..., 0] = N.f64_to_bf16_bits(np.array([16.0]))[0]
    metas = [{"q_len": 200, "segs": [(2, 150), (0, 150), (1, 150)], "text_slot": 0, "text_len": 80}]
    out, _ = w.run(q, metas, with_lse=False)
    from _util import to_host_bits
    got = to_host_bits(out)[0]
    if text:
        exp = tv[pos]
    else:
        exp = vals[3 if slot_of_needle == 0 else 4][pos]
    assert np.array_equal(got, np.broadcast_to(exp, got.shape)), (slot_of_needle, pos, text)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("slot,pos", [(0, 0), (0, 63), (0, 64), (1, 149), (1, 127), (1, 128), (0, 31), (1, 32)])
def test_needle_bit_exact(D, slot, pos):
    _needle_case(D, slot, pos)


@pytest.mark.parametrize("pos", [0, 63, 64, 79])
def test_needle_in_text_bit_exact(pos):
    _needle_case(64, 0, pos, text=True)


@pytest.mark.parametrize("D", [64, 128])
def test_v_ones_gives_exactly_one(D):
    rng = _rng(9)
    H = 2
    w = Workload("bf16", 2, 300, H, D, 50)
    one = N.f64_to_bf16_bits(np.ones((300, H, D)))
    w.append(draw(rng, (300, H, D), 1.0, "bf16"), one)
    w.append(draw(rng, (211, H, D), 1.0, "bf16"), one[:211])
    w.set_text(draw(rng, (50, H, D), 1.0, "bf16"), one[:50])
    q = draw(rng, (1, 333, H, D), 1.0, "bf16")
    out, _ = w.run(q, [{"q_len": 333, "segs": [(0, 300), (1, 211)], "text_slot": 0, "text_len": 50}])
    assert np.all(decode(out, "bf16") == 1.0)


def test_q_zero_gives_mean_of_values():
    rng = _rng(10)
    H, D = 2, 64
    w = Workload("bf16", 2, 300, H, D, 50)
    _fill(w, rng, (300, 211), H, D, "bf16", 1.0, 50)
    q = np.zeros((1, 130, H, D), np.uint16)
    metas = [{"q_len": 130, "segs": [(0, 300), (1, 211)], "text_slot": 0, "text_len": 50}]
    out, _ = w.run(q, metas)
    ref, _ = w.oracle(q, metas)
    got = decode(out, "bf16")
    # the mean is accumulated in fp32 and rounded once to bf16
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)


def test_segment_order_does_not_matter():
    # Unmasked attention does not depend on key order.  The kernel's reference
    # maximum comes from the first tile, so another order rounds the weights to
    # bf16 at other points: each result must meet the bar against the oracle,
    # and the two may differ by at most the weight-rounding bound
    # 2 * 2^-9 * max|v| (relative error 2^-9 per weight, on each side).
    rng = _rng(11)
    H, D = 2, 128
    w = Workload("bf16", 2, 300, H, D, 50)
    _fill(w, rng, (300, 211), H, D, "bf16", 0.5, 50)
    q = draw(rng, (1, 256, H, D), 0.5, "bf16")
    m1 = [{"q_len": 256, "segs": [(0, 300), (1, 211)], "text_slot": 0, "text_len": 50}]
    m2 = [{"q_len": 256, "segs": [(1, 211), (0, 300)], "text_slot": 0, "text_len": 50}]
    a, _ = w.run(q, m1)
    b, _ = w.run(q, m2)
    ref, _ = w.oracle(q, m1)
    ga, gb = decode(a, "bf16"), decode(b, "bf16")
    check_contract(ga, ref, "bf16")
    check_contract(gb, ref, "bf16")
    vmax = max(np.abs(w.oring.values(s, h, 300)).max() for s in (0, 1) for h in range(H))
    assert np.abs(ga - gb).max() <= 2 * 2 ** -9 * vmax


@pytest.mark.parametrize("D", [64, 128])
def test_growing_scores_exercise_lazy_maximum(D):
    # keys scaled up along the key sequence so later tiles keep raising the
    # maximum by more than the lazy threshold
    rng = _rng(12)
    H, L = 2, 512
    w = Workload("bf16", 2, L, H, D, 0)
    k = N.bf16_bits_to_f64(draw(rng, (L, H, D), 1.0, "bf16"))
    ramp = np.linspace(0.05, 4.0, L)[:, None, None]
    kb = N.f64_to_bf16_bits(k * ramp)
    w.append(kb, draw(rng, (L, H, D), 1.0, "bf16"))
    q = draw(rng, (1, 200, H, D), 1.0, "bf16")
    metas = [{"q_len": 200, "segs": [(0, L)], "text_slot": 0, "text_len": 0}]
    out, lse = w.run(q, metas, scale=0.5)
    ref, ref_lse = w.oracle(q, metas, scale=0.5)
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -6 * np.nanmax(np.abs(ref))
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse) / np.maximum(1, np.abs(ref_lse))) < 1e-3


@pytest.mark.parametrize("D", [64, 128])
def test_scores_far_below_zero_do_not_underflow(D):
    # every score around -1000 in the exp2 domain: the first tile sets the
    # reference maximum, so the weights stay normal
    rng = _rng(13)
    H, L = 1, 300
    w = Workload("bf16", 1, L, H, D, 0)
    k = np.zeros((L, H, D))
    k[..., 0] = -64.0
    k[..., 1] = N.bf16_bits_to_f64(draw(rng, (L, H), 1.0, "bf16"))
    w.append(N.f64_to_bf16_bits(k), draw(rng, (L, H, D), 1.0, "bf16"))
    q = np.zeros((1, 64, H, D))
    q[..., 0] = 128.0
    q[..., 1] = 1.0
    qb = N.f64_to_bf16_bits(q)
    metas = [{"q_len": 64, "segs": [(0, L)], "text_slot": 0, "text_len": 0}]
    out, _ = w.run(qb, metas, scale=1.0)
    ref, _ = w.oracle(qb, metas, scale=1.0)
    check_contract(decode(out, "bf16"), ref, "bf16", gate2=False)


@pytest.mark.parametrize("D", [64, 128])
def test_growing_scores_with_ragged_segments_and_text(D):
    # the lazy maximum is raised inside tail groups (segments of 500 and 77
    # keys, 40 text keys): masked keys must stay out of the new reference
    rng = _rng(14 + D)
    H = 2
    w = Workload("bf16", 2, 512, H, D, 64)
    for n, (lo, hi) in ((500, (0.05, 3.0)), (77, (3.0, 4.5))):
        k = N.bf16_bits_to_f64(draw(rng, (n, H, D), 1.0, "bf16"))
        kb = N.f64_to_bf16_bits(k * np.linspace(lo, hi, n)[:, None, None])
        w.append(kb, draw(rng, (n, H, D), 1.0, "bf16"))
    w.set_text(draw(rng, (40, H, D), 1.0, "bf16"), draw(rng, (40, H, D), 1.0, "bf16"))
    q = draw(rng, (1, 130, H, D), 1.0, "bf16")
    metas = [{"q_len": 130, "segs": [(0, 500), (1, 77)], "text_slot": 0, "text_len": 40}]
    out, lse = w.run(q, metas, scale=0.5)
    ref, ref_lse = w.oracle(q, metas, scale=0.5)
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -6 * np.nanmax(np.abs(ref))
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse) / np.maximum(1, np.abs(ref_lse))) < 1e-3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("growth", [6.0, 40.0, 90.0, 300.0])
def test_scores_rising_along_the_keys(D, growth):
    # scores rise linearly along the key sequence by `growth` (exp2 domain)
    # above the first group's maximum.  Head dim 64's fast form keeps its
    # first reference: at 6 the weights stay within [0, 2^6], at 40 and 90
    # they grow to 2^40 and 2^90 (sums near 2^94, below the 2^100 check); at
    # 300 they overflow fp32 and the chunk is computed again in the exact
    # form.  Head dim 128 raises its reference whenever a group's weights
    # pass 2^12.  Every case matches the oracle.
    rng = _rng(15 + D + int(growth))
    H, L = 2, 700
    w = Workload("bf16", 1, L, H, D, 0)
    k = np.zeros((L, H, D))
    k[:, :, 0] = (growth / math.log2(math.e)) * np.arange(L)[:, None] / L
    k[:, :, 1] = N.bf16_bits_to_f64(draw(rng, (L, H), 0.25, "bf16"))
    w.append(N.f64_to_bf16_bits(k), draw(rng, (L, H, D), 1.0, "bf16"))
    q = np.zeros((1, 200, H, D))
    q[..., 0] = 1.0
    q[..., 1] = N.bf16_bits_to_f64(draw(rng, (1, 200, H), 1.0, "bf16"))
    qb = N.f64_to_bf16_bits(q)
    metas = [{"q_len": 200, "segs": [(0, L)], "text_slot": 0, "text_len": 0}]
    out, lse = w.run(qb, metas, scale=1.0)
    ref, ref_lse = w.oracle(qb, metas, scale=1.0)
    got = decode(out, "bf16")
    assert not np.isnan(got).any()
    # a few dozen keys carry the weight: each output is an average of a few
    # values of |v| ~ 1, with the weights rounded to bf16
    assert np.max(np.abs(got - ref)) <= 2 ** -6 * max(1.0, np.max(np.abs(ref)))
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse) / np.maximum(1, np.abs(ref_lse))) < 1e-3


def test_in_place_output():
    import torch
    import block_wise_long_amd as B
    rng = _rng(14)
    H, D = 2, 64
    w = Workload("bf16", 2, 200, H, D, 0)
    _fill(w, rng, (200, 150), H, D, "bf16", 0.5, 0)
    q = draw(rng, (1, 300, H, D), 0.5, "bf16")
    metas = [{"q_len": 300, "segs": [(0, 200), (1, 150)]}]
    ref, _ = w.run(q, metas, with_lse=False)
    qd = to_dev(q, "bf16")
    B.ba_block_attention(qd, w.ring, None, metas, out=qd)
    torch.cuda.synchronize()
    assert torch.equal(qd.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("workspace", ["auto", None])
def test_more_blocks_than_one_launch_takes(workspace):
    # 21 blocks: the call runs as launches of 16 and 5 blocks, each with its
    # own q / out / lse offsets; every block checked against the oracle
    rng = _rng(21)
    H, D, L, nb = 2, 64, 96, 21
    w = Workload("bf16", 5, L, H, D, 24)
    _fill(w, rng, (L, 90, L, 40, L), H, D, "bf16", 0.5, 24)
    q = draw(rng, (nb, 100, H, D), 0.5, "bf16")
    metas = []
    for b in range(nb):
        segs = [((b + i) % 5, (L, 90, L, 40, L)[(b + i) % 5]) for i in range(1 + b % 3)]
        metas.append({"q_len": 100 - (b % 4) * 13, "segs": segs, "text_slot": 0, "text_len": (b * 5) % 25})
    out, lse = w.run(q, metas, workspace=workspace)
    ref, ref_lse = w.oracle(q, metas)
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3
    for b in range(nb):        # rows past each q_len untouched
        assert np.isnan(got[b, metas[b]["q_len"]:]).all()


@pytest.mark.parametrize("workspace", ["auto", None])
def test_launches_of_one_call_take_different_shapes(workspace):
    # 18 blocks at head dim 64: the first launch (16 blocks) has key sets of at
    # most 3072 keys (narrow workgroups), the second (2 blocks) one of 3300
    # (wide workgroups); one call, one workspace, every block against the oracle
    import block_wise_long_amd as B
    rng = _rng(22)
    H, D, nb = 2, 64, 18
    w = Workload("bf16", 3, 1650, H, D, 16)
    _fill(w, rng, (1650, 1422, 1650), H, D, "bf16", 0.5, 16)
    q = draw(rng, (nb, 200, H, D), 0.5, "bf16")
    metas = []
    for b in range(nb):
        segs = [(1, 1422), (2, 1650)] if b < 16 else [(0, 1650), (2, 1650)]
        metas.append({"q_len": 200 - (b % 3) * 37, "segs": segs, "text_slot": 0, "text_len": 0})
    assert B.ba_attention_query_tile(D, B.BA_BF16, 1422 + 1650) < B.ba_attention_query_tile(D, B.BA_BF16, 3300)
    out, lse = w.run(q, metas, workspace=workspace)
    ref, ref_lse = w.oracle(q, metas)
    got = decode(out, "bf16")
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
    assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3
    for b in range(nb):
        assert np.isnan(got[b, metas[b]["q_len"]:]).all()
