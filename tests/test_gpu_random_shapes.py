"""Block attention on seeded random shapes against the fp64 oracle: head dims
64 and 128, bf16 and fp32 rings, one to three blocks per call with their
own query counts and key sets (cache segments of random lengths, empty ones
among them, and a text of random length or none), random scales, with and
without a workspace.  Each case is small enough for the oracle to check
every output and log-sum-exp."""
import math

import numpy as np
import pytest

from _util import Workload, check_contract, decode
from workloads import draw

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.Generator(np.random.PCG64(seed))
    D = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    H = int(r.integers(1, 4))
    n_slots = int(r.integers(1, 5))
    slot_tokens = int(r.integers(1, 300))
    text_tokens = int(r.integers(0, 120))
    nb = int(r.integers(1, 4))
    q_stride = int(r.integers(1, 400))
    lens = [int(r.integers(1, slot_tokens + 1)) for _ in range(n_slots)]   # appended tokens per slot
    metas = []
    for _ in range(nb):
        n_segs = int(r.integers(0, 4))
        segs = [(int(r.integers(0, n_slots)), None) for _ in range(n_segs)]
        segs = [(s, int(r.integers(0, lens[s] + 1))) for s, _ in segs]
        text_len = int(r.integers(0, text_tokens + 1)) if text_tokens else 0
        if sum(n for _, n in segs) + text_len == 0:
            segs = segs + [(0, 1)]             # a block with queries needs a key (zero-length segments stay)
        metas.append({"q_len": int(r.integers(0, q_stride + 1)), "segs": segs, "text_slot": 0,
                      "text_len": text_len})
    scale = float(r.choice([0.0, 0.05, 0.3]))
    workspace = "auto" if r.random() < 0.5 else None
    return D, dtype, H, n_slots, slot_tokens, text_tokens, lens, q_stride, metas, scale, workspace, r


@pytest.mark.parametrize("seed", range(40))
def test_random_shape(seed):
    D, dtype, H, n_slots, slot_tokens, text_tokens, lens, q_stride, metas, scale, workspace, r = _case(9000 + seed)
    w = Workload(dtype, n_slots, slot_tokens, H, D, text_tokens)
    for n in lens:
        w.append(draw(r, (n, H, D), 0.5, dtype), draw(r, (n, H, D), 0.5, dtype), n)
    if text_tokens:
        w.set_text(draw(r, (text_tokens, H, D), 0.5, dtype), draw(r, (text_tokens, H, D), 0.5, dtype))
    q = draw(r, (len(metas), q_stride, H, D), 0.5, dtype)
    out, lse = w.run(q, metas, scale=scale, workspace=workspace)
    ref, ref_lse = w.oracle(q, metas, scale=scale if scale > 0 else None)
    got = decode(out, dtype)
    if not np.isnan(ref).all():
        check_contract(got, ref, dtype, gate2=False)
        if dtype == "bf16":
            rms = math.sqrt(np.nanmean(ref ** 2))
            assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
        sel = ~np.isnan(ref_lse)
        assert np.max(np.abs(lse.cpu().numpy()[sel] - ref_lse[sel])) < (1e-5 if dtype == "f32" else 2e-3)
    for b, m in enumerate(metas):            # rows past each q_len untouched
        assert np.isnan(got[b, m["q_len"]:]).all()
