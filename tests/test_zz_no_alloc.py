"""The entry point that allocates nothing (ba_block_attention_static): its
output equals ba_block_attention's with a workspace, bit for bit (same
kernels, same schedule), on two calls in a row, the second with a smaller
input."""
import numpy as np
import pytest

from _util import Workload, to_host_bits
from workloads import draw

pytestmark = pytest.mark.gpu


def test_static_entry_matches_workspace_entry_twice():
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(777))
    H, D, L, TXT = 24, 64, 5400, 226
    w = Workload("bf16", 2, L, H, D, TXT)
    for _ in range(2):
        w.append(draw(rng, (L, H, D), 0.5, "bf16"), draw(rng, (L, H, D), 0.5, "bf16"))
    w.set_text(draw(rng, (TXT, H, D), 0.5, "bf16"), draw(rng, (TXT, H, D), 0.5, "bf16"))
    cases = [(L, [(0, L), (1, L)], TXT), (1900, [(1, 3001)], 100)]
    ws = B.attention_workspace(D, B.BA_BF16, 1, L, H)
    for i, (q_len, segs, text_len) in enumerate(cases):
        metas = [{"q_len": q_len, "segs": segs, "text_slot": 0, "text_len": text_len}]
        if i == 0:
            # the first call takes the split schedule, so the partial results
            # go through the library's own array
            assert B.ba_attention_plan(q_len, w.ring, w.text, metas, ws.numel()) > 0
        q = torch.from_numpy(draw(rng, (1, q_len, H, D), 0.5, "bf16").view(np.int16)).view(torch.bfloat16).cuda()
        ref = torch.full_like(q, float("nan"))
        got = torch.full_like(q, float("nan"))
        lse_ref = torch.full((1, H, q_len), float("nan"), device="cuda")
        lse_got = torch.full((1, H, q_len), float("nan"), device="cuda")
        B.ba_block_attention(q, w.ring, w.text, metas, out=ref, lse=lse_ref, workspace=ws)
        B.ba_block_attention_static(q, w.ring, w.text, metas, out=got, lse=lse_got)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(got), to_host_bits(ref)), f"call {i}: outputs differ"
        assert torch.equal(lse_got, lse_ref), f"call {i}: lse differs"
        assert not torch.isnan(got.float()).any()
