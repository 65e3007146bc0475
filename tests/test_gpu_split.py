"""The two work schedules of the bf16 attention kernel through the C ABI:
one workgroup per query tile (no workspace) and equal ranges of key tiles
over the resident workgroups with cut tasks merged through the workspace.
Both must meet the bar against the oracle; the split schedule must also be
deterministic, whatever the workspace held before."""
import numpy as np
import pytest

from _util import Workload, check_contract, decode, to_dev, to_host_bits
from workloads import draw

pytestmark = pytest.mark.gpu


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


# key sets of the two launch shapes at head dim 64: the longest one above
# 3072 keys (wide workgroups) or not (narrow ones)
_LENS = {"wide": ((1600, 1500, 1600, 33, 1600, 1599), 120), "narrow": ((1600, 1400, 1600, 33, 1600, 1300), 60)}


def _setup(D, seed, shape="wide"):
    # long enough key sets (25-52 tiles of 64 per task) and enough tasks
    # (12 heads: 48-84 query tiles) that the library takes the split schedule
    # with 1, 2 and 5 tail workgroups per XCD
    rng = _rng(seed)
    H = 12
    lens, txt0 = _LENS[shape]
    w = Workload("bf16", 6, 1600, H, D, 120)
    for n in lens:
        w.append(draw(rng, (n, H, D), 0.5, "bf16"), draw(rng, (n, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (120, H, D), 0.5, "bf16"), draw(rng, (120, H, D), 0.5, "bf16"))
    q = draw(rng, (4, 600, H, D), 0.5, "bf16")
    metas = [{"q_len": 600, "segs": [(0, lens[0]), (1, lens[1])], "text_slot": 0, "text_len": txt0},
             {"q_len": 257, "segs": [(2, lens[2])], "text_slot": 0, "text_len": 0},
             {"q_len": 0, "segs": [(3, lens[3])], "text_slot": 0, "text_len": 3},
             {"q_len": 333, "segs": [(3, lens[3]), (4, lens[4]), (5, lens[5])], "text_slot": 0, "text_len": 119}]
    return w, q, metas


def _max_keys(metas):
    return max(sum(n for _, n in m["segs"]) + m["text_len"] for m in metas if m["q_len"] > 0)


def _workspace(D, tail_wg, fill, max_keys):
    """A workspace with room for exactly tail_wg tail workgroups per XCD,
    pre-filled with garbage (its contents must not matter)."""
    import torch
    import block_wise_long_amd as B
    # one partial result per query of the query tile: head_dim fp32 output
    # values, and the fp32 maximum and sum of each of its two lanes
    part = 4 * B.ba_attention_query_tile(D, B.BA_BF16, max_keys) * (D + 4)
    nbytes = 16 * tail_wg * part
    ws = torch.full((nbytes + 256,), fill, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


@pytest.mark.parametrize("D,shape", [(64, "wide"), (64, "narrow"), (128, "wide")])
def test_both_schedules_meet_the_bar(D, shape):
    w, q, metas = _setup(D, 21 + D, shape)
    ref, ref_lse = w.oracle(q, metas)
    outs = []
    for ws in ("auto", None):
        out, lse = w.run(q, metas, workspace=ws)
        got = decode(out, "bf16")
        check_contract(got, ref, "bf16", gate2=False)
        assert np.nanmax(np.abs(lse.cpu().numpy() - ref_lse)) < 2e-3
        assert np.isnan(got[1, 257:]).all() and np.isnan(got[2]).all() and np.isnan(got[3, 333:]).all()
        outs.append(got)
    vmax = max(np.abs(w.oring.values(s, h, 33)).max() for s in range(6) for h in range(12))
    vmax = max(vmax, max(np.abs(w.oring.values(s, h, 1300)).max() for s in (0, 1, 2, 4, 5) for h in range(12)))
    assert np.nanmax(np.abs(outs[0] - outs[1])) <= 2 * 2 ** -9 * vmax


@pytest.mark.parametrize("D,shape", [(64, "wide"), (64, "narrow"), (128, "wide")])
@pytest.mark.parametrize("tail_wg", [1, 2, 5])
def test_few_tail_workgroups_cut_many_tasks(D, shape, tail_wg):
    # few tail workgroups: every tail range spans several tasks and blocks, and
    # most tail tasks are cut between two or more workgroups
    import block_wise_long_amd as B
    w, q, metas = _setup(D, 5 + D + tail_wg, shape)
    mk = _max_keys(metas)
    assert (mk > 3072) == (shape == "wide")
    ws = _workspace(D, tail_wg, 0x7F, mk)
    # the call does take the split schedule with this workspace
    assert B.ba_attention_plan(q.shape[1], w.ring, w.text, metas, ws.numel()) == tail_wg
    ref, _ = w.oracle(q, metas)
    out1, _ = w.run(q, metas, workspace=ws)
    out2, _ = w.run(q, metas, workspace=_workspace(D, tail_wg, 0xFF, mk))
    check_contract(decode(out1, "bf16"), ref, "bf16", gate2=False)
    assert np.array_equal(to_host_bits(out1), to_host_bits(out2))


def test_split_schedule_is_deterministic_at_video_shape():
    from _util import build_config
    from workloads import CONFIGS
    import block_wise_long_amd as B
    w, inputs, metas = build_config(CONFIGS[1])
    ws = B.attention_workspace(64, B.BA_BF16, 1, inputs["q"].shape[1], 24, "cuda")
    assert B.ba_attention_plan(inputs["q"].shape[1], w.ring, w.text, metas, ws.numel()) > 0
    a, _ = w.run(inputs["q"], metas, with_lse=False)
    b, _ = w.run(inputs["q"], metas, with_lse=False)
    assert np.array_equal(to_host_bits(a), to_host_bits(b))
