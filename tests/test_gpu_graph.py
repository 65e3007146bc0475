"""The hot path recorded once in a HIP graph (torch's stream capture) and
replayed: one queue step's data path (the batched append, one attention
launch over the queued blocks, the per-block update), and the projection
layer with a text-only cross-attention.  The calls allocate nothing, set no
memory and wait on nothing, so they can be captured; between replays the
inputs are restored eagerly and the device synchronised, and every replay
must give the bytes of the eager run."""
import pytest
import torch

import block_wise_long_amd as B
from block_wise_long_amd.fifo import FifoQueue

pytestmark = pytest.mark.gpu


def _randn(gen, shape, std):
    return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _replay_matches(run, state, eager_out, replays=3):
    """Restore `state` (list of (tensor, saved copy)), capture `run` once,
    then replay it `replays` times from the restored state; each replay's
    outputs must equal eager_out bit for bit."""
    for t, saved in state:
        t.copy_(saved)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for r in range(replays):
        for t, saved in state:
            t.copy_(saved)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, (got, want) in enumerate(zip(outs, eager_out)):
            assert torch.equal(_bits(got), _bits(want)), (r, name)
        # eager work of the program's own between replays
        _ = (outs[0].float() * 2).sum().item()


def test_queue_step_in_a_graph():
    # two queued blocks of 3000 tokens (24 heads x 64) with a text: 384
    # tasks of 384 queries, 48 per XCD, whose last round leaves half of the
    # XCD's 32 slots idle, so the attention launch takes the split schedule
    # (tail workgroups and the merge kernel)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    n, L, H, D, TXT = 2, 3000, 24, 64, 226
    x0 = _randn(gen, (n, L, H, D), 0.5)
    fq = FifoQueue(x0.clone(), _randn(gen, (TXT, H, D), 0.5), _randn(gen, (TXT, H, D), 0.5))
    for _ in range(2):                         # steps with cached context behind
        fq.step(_randn(gen, (L, H, D), 0.5))
    slots, metas, t, stride = B.ba_queue_plan(fq.q)
    assert any(m.n_segs > 1 for m in metas)
    ws = B.attention_workspace(D, B.BA_BF16, n, L, H)
    assert ws is not None
    assert B.ba_attention_plan(L, fq.ring, fq.text, list(metas), ws.numel()) > 0   # split schedule
    sched = {"kind": "ddim", "T": fq.T, "stride": stride}

    def run():
        B.ba_cache_append_batched(fq.ring, fq.x, fq.x, list(slots))
        B.ba_block_attention(fq.x, fq.ring, fq.text, list(metas), out=fq.pred, workspace=ws)
        B.ba_block_update(fq.x.view(n, -1), fq.pred.view(n, -1), list(t), sched)
        return [fq.ring.buffer, fq.pred, fq.x]

    state = [(fq.ring.buffer, fq.ring.buffer.clone()), (fq.x, fq.x.clone()), (fq.pred, fq.pred.clone())]
    eager = [o.clone() for o in run()]
    torch.cuda.synchronize()
    _replay_matches(run, state, eager)


def test_projection_and_text_cross_attention_in_a_graph():
    # the fused producer writes one block's K and V into its ring slot and Q
    # to a buffer; the block's queries then attend over the text alone (the
    # resident key-set kernel: 24 heads x 5400 queries, 512 text keys)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    L, H, D, TXT = 5400, 24, 64, 512
    dim = H * D
    x = _randn(gen, (1, L, dim), 1.0)
    w = _randn(gen, (3 * H * D, dim), dim ** -0.5)
    pos = torch.arange(L, device="cuda", dtype=torch.float32)[:, None]
    freq = 10000.0 ** (-torch.arange(D // 2, device="cuda", dtype=torch.float32) * 2 / D)[None, :]
    rope = torch.stack([torch.cos((pos * freq).t()), torch.sin((pos * freq).t())], dim=-1).contiguous()
    ring = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    text = B.ba_ring_init(1, TXT, H, D, B.BA_BF16)
    B.ba_cache_append(text, _randn(gen, (TXT, H, D), 0.5), _randn(gen, (TXT, H, D), 0.5), TXT)
    q = torch.empty((1, L, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, H, L), dtype=torch.float32, device="cuda")
    metas = [{"q_len": L, "segs": [], "text_slot": 0, "text_len": TXT}]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if H * ((L + 31) // 32) < 12 * cus:
        pytest.skip("too few query units for the resident kernel on this device")
    assert B.ba_attention_query_tile(D, B.BA_BF16, TXT) == 32

    def run():
        B.ba_qkv_project_batched(x, w, ring, [1], q=q, rope=rope)
        B.ba_block_attention(q, ring, text, metas, out=out, lse=lse, workspace=None)
        return [ring.buffer, q, out, lse]

    state = [(ring.buffer, ring.buffer.clone()), (q, q.clone()), (out, out.clone()), (lse, lse.clone())]
    eager = [o.clone() for o in run()]
    torch.cuda.synchronize()
    _replay_matches(run, state, eager)


def test_static_entry_in_a_graph():
    # the entry point that allocates nothing, meant for code under capture:
    # a 480p block on the split schedule (tail workgroups, the library's own
    # scratch array, the merge kernel) recorded once and replayed
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    L, H, D, TXT = 5400, 24, 64, 226
    ring = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    text = B.ba_ring_init(1, TXT, H, D, B.BA_BF16)
    for _ in range(2):
        B.ba_cache_append(ring, _randn(gen, (L, H, D), 0.5), _randn(gen, (L, H, D), 0.5), L)
    B.ba_cache_append(text, _randn(gen, (TXT, H, D), 0.5), _randn(gen, (TXT, H, D), 0.5), TXT)
    q = _randn(gen, (1, L, H, D), 0.5)
    metas = [{"q_len": L, "segs": [(0, L), (1, L)], "text_slot": 0, "text_len": TXT}]
    out = torch.empty_like(q)
    lse = torch.empty((1, H, L), dtype=torch.float32, device="cuda")
    ws = B.attention_workspace(D, B.BA_BF16, 1, L, H)
    assert B.ba_attention_plan(L, ring, text, metas, ws.numel()) > 0      # split schedule

    def run():
        B.ba_block_attention_static(q, ring, text, metas, out=out, lse=lse)
        return [out, lse]

    eager = [o.clone() for o in run()]
    ref = B.ba_block_attention(q, ring, text, metas, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(eager[0].view(torch.int16), ref.view(torch.int16))
    state = [(out, out.clone()), (lse, lse.clone())]
    _replay_matches(run, state, eager)
