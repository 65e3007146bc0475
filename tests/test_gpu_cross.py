"""Separate text cross-attention (Wan-style; the alternative to the joint
key set) through the block-attention call: a block with no cache segments
attends over the text keys alone, a block with text_len = 0 over its cache
segments alone, each part with its own softmax.  Compared with the oracle's
split parts element by element at small shapes and on sampled rows at the
480p block's shape with a 512-token text; and the GPU's two parts, merged
through their log-sum-exps, meet the contract against the oracle's joint
attention."""
import math

import numpy as np
import pytest

from _util import Workload, check_contract, decode, sample_rows
from oracle import attention as A
from oracle import numerics as N
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _bar(got, ref):
    # few keys give larger outputs than the video key sets: the bar scales
    # with the output (weights carry 2^-9 relative rounding, the output 2^-9)
    check_contract(got, ref, "bf16", gate2=False)
    rms = math.sqrt(np.nanmean(ref ** 2))
    mx = np.nanmax(np.abs(got - ref))
    assert mx <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms, mx


def _setup(rng, H, D, lens, text_len, slot_tokens):
    w = Workload("bf16", len(lens), slot_tokens, H, D, text_len)
    for n in lens:
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (text_len, H, D), 0.5, "bf16"), draw(rng, (text_len, H, D), 0.5, "bf16"))
    return w


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("q_len,text_len", [(300, 37), (257, 512), (64, 1), (130, 226)])
def test_text_only_and_self_only_parity(D, q_len, text_len):
    rng = _rng(7000 + D + q_len + text_len)
    H = 3
    lens = (200, 150)
    w = _setup(rng, H, D, lens, text_len, 200)
    q = draw(rng, (1, q_len, H, D), 0.5, "bf16")
    segs = [(i, n) for i, n in enumerate(lens)]
    (ref_s, ref_ls), (ref_t, ref_lt) = A.split_text_attention_ref(
        N.decode(q, "bf16"), w.oring, w.otext, [{"q_len": q_len, "segs": segs, "text_slot": 0,
                                                  "text_len": text_len}])
    out_t, lse_t = w.run(q, [{"q_len": q_len, "segs": [], "text_slot": 0, "text_len": text_len}])
    _bar(decode(out_t, "bf16"), ref_t)
    assert np.nanmax(np.abs(lse_t.cpu().numpy() - ref_lt)) < 2e-3
    out_s, lse_s = w.run(q, [{"q_len": q_len, "segs": segs, "text_slot": 0, "text_len": 0}])
    _bar(decode(out_s, "bf16"), ref_s)
    assert np.nanmax(np.abs(lse_s.cpu().numpy() - ref_ls)) < 2e-3


def test_single_text_key_is_exact():
    # one text key: every weight is exactly 1, the output is that key's V
    rng = _rng(71)
    H, D = 2, 64
    w = _setup(rng, H, D, (64,), 1, 64)
    q = draw(rng, (1, 200, H, D), 0.5, "bf16")
    out, _ = w.run(q, [{"q_len": 200, "segs": [], "text_slot": 0, "text_len": 1}])
    got = decode(out, "bf16")
    for h in range(H):
        assert np.array_equal(got[0, :, h, :], np.broadcast_to(w.otext.values(0, h, 1)[0], (200, D)))


def test_split_parts_at_video_shape():
    # 480p block: 5400 queries, 24 heads x 64, cache [5400 | 5400], text 512
    rng = _rng(72)
    H, D, L, TXT = 24, 64, 5400, 512
    w = _setup(rng, H, D, (L, L), TXT, L)
    q = draw(rng, (1, L, H, D), 0.5, "bf16")
    segs = [(0, L), (1, L)]
    joint_m = [{"q_len": L, "segs": segs, "text_slot": 0, "text_len": TXT}]
    out_j, lse_j = w.run(q, joint_m)
    out_s, lse_s = w.run(q, [{"q_len": L, "segs": segs, "text_slot": 0, "text_len": 0}])
    out_t, lse_t = w.run(q, [{"q_len": L, "segs": [], "text_slot": 0, "text_len": TXT}])
    # the text-only call runs whole query tiles (8 key tiles per task: too
    # short to cut), the self part takes the split schedule
    import block_wise_long_amd as B
    ws = B.attention_workspace(D, B.BA_BF16, 1, L, H, "cuda")
    assert B.ba_attention_plan(L, w.ring, w.text, [{"q_len": L, "segs": [], "text_slot": 0,
                                                    "text_len": TXT}], ws.numel()) == 0
    assert B.ba_attention_plan(L, w.ring, w.text, joint_m, ws.numel()) > 0
    # edge rows of both launch shapes: the text-only call's narrow tile and
    # the self and joint calls' wide one
    rows = sorted(set(sample_rows(L, 24, seed=72, tile=B.ba_attention_query_tile(D, B.BA_BF16, TXT)))
                  | set(sample_rows(L, 0, seed=72, tile=B.ba_attention_query_tile(D, B.BA_BF16, 2 * L + TXT))))
    heads = [0, 7, 23]
    qf = N.decode(q, "bf16")
    (ref_s, ref_ls), (ref_t, ref_lt) = A.split_text_attention_ref(qf, w.oring, w.otext, joint_m,
                                                                    heads=heads, rows=rows)
    ref_j, ref_lj = A.block_attention_ref(qf, w.oring, w.otext, joint_m, heads=heads, rows=rows)
    gs, gt, gj = (decode(o, "bf16") for o in (out_s, out_t, out_j))
    check_contract(gs, ref_s, "bf16", gate2=True)      # ~11k keys: the video-shape gate
    _bar(gt, ref_t)
    check_contract(gj, ref_j, "bf16", gate2=True)
    # the GPU's parts, merged through their lse, give the joint attention
    ls = np.transpose(lse_s.cpu().numpy(), (0, 2, 1))
    lt = np.transpose(lse_t.cpu().numpy(), (0, 2, 1))
    merged, ml = A.merge_partials(gs, ls, gt, lt)
    check_contract(merged, ref_j, "bf16", gate2=True)
    sel = ~np.isnan(ref_lj)
    assert np.max(np.abs(np.transpose(ml, (0, 2, 1))[sel] - ref_lj[sel])) < 2e-3
    for lse, ref_l in ((lse_s, ref_ls), (lse_t, ref_lt), (lse_j, ref_lj)):
        sel = ~np.isnan(ref_l)
        assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_l[sel])) < 2e-3
