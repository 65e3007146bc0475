"""Shared helpers of the GPU parity tests: device transfer of the seeded
inputs, the HIP path through the C ABI, the oracle on the same inputs, and
the tolerance checks."""
import math

import numpy as np

from oracle import numerics as N
from oracle import ring as oring

# Tolerances of the contract: max-abs / mean-abs on bf16 inputs, and 1e-5 on
# the fp32 path.  The secondary gate is ten times above the error of an
# emulated bf16-weights / fp32-accumulation kernel at these input statistics
# and several times below the error of dropping the text segment.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5
GATE2_MAX_ABS, GATE2_MEAN_ABS = 5e-4, 5e-5


def to_dev(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host_bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def decode(t_or_arr, dtype):
    if dtype == "bf16":
        a = t_or_arr if isinstance(t_or_arr, np.ndarray) else to_host_bits(t_or_arr)
        return N.bf16_bits_to_f64(a)
    a = t_or_arr if isinstance(t_or_arr, np.ndarray) else t_or_arr.cpu().numpy()
    return a.astype(np.float64)


def ring_bytes(ring):
    return ring.buffer.cpu().numpy().tobytes()


def errors(got, ref, mask=None):
    d = np.abs(got - ref)
    if mask is not None:
        d = d[mask]
    d = d[~np.isnan(d)] if d.size else d
    return float(d.max()), float(d.mean())


def check_contract(got, ref, dtype, gate2=True):
    """The parity bar: max/mean abs error of the computed entries."""
    sel = ~np.isnan(ref)
    assert not np.isnan(got[sel]).any(), "NaN in kernel output"
    mx, mn = errors(got[sel], ref[sel])
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"fp32 max-abs {mx:.3g} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS and mn <= BF16_MEAN_ABS, f"bf16 max {mx:.3g} mean {mn:.3g}"
        if gate2:
            assert mx <= GATE2_MAX_ABS and mn <= GATE2_MEAN_ABS, f"gate2 max {mx:.3g} mean {mn:.3g}"
    return mx, mn


def sample_rows(q_len, n_random=48, seed=0, tile=128):
    """Edge rows plus random rows.  tile is the launch's query tile
    (ba_attention_query_tile): every tile boundary, and in the first and the
    last tile every 32-query wave boundary; the ragged tail; random rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = {0, 1, q_len - 1, q_len - 2}
    for t0 in range(0, q_len, tile):
        rows |= {t0 - 1, t0, t0 + 1}
    last_tile = (q_len - 1) // tile * tile
    for t0 in (0, last_tile):
        for w0 in range(t0, t0 + tile, 32):
            rows |= {w0 - 1, w0, w0 + 31}
    rows |= set(rng.integers(0, q_len, n_random).tolist())
    return sorted(r for r in rows if 0 <= r < q_len)


def cut_heads(n_blocks, heads, q_len, tile, tail_wg):
    """Heads of the tasks that the split schedule cuts into pieces, given the
    tail workgroups per XCD that ba_attention_plan reports (0: none cut).
    Tasks are (block, head, query tile), head-major within a block; XCD x owns
    tasks [x n / 8, (x + 1) n / 8); its last round, or the last two when the
    last is under a quarter full, is shared by the tail workgroups."""
    if tail_wg <= 0:
        return []
    nqt = -(-q_len // tile)
    n = n_blocks * heads * nqt
    cut = set()
    for x in range(8):
        t0, t1 = x * n // 8, (x + 1) * n // 8
        rounds = (t1 - t0) // tail_wg
        if ((t1 - t0) - rounds * tail_wg) * 4 < tail_wg and rounds > 0:
            rounds -= 1
        for t in range(t0 + rounds * tail_wg, t1):
            cut.add((t % (heads * nqt)) // nqt)
    return sorted(cut)


class Workload:
    """Device and oracle state of one attention workload built from a config
    (or from explicit arrays): rings filled the same way on both sides."""

    def __init__(self, dtype, n_slots, slot_tokens, heads, head_dim, text_tokens):
        import block_wise_long_amd as B
        self.B = B
        self.dtype = dtype
        code = B.BA_BF16 if dtype == "bf16" else B.BA_F32
        self.ring = B.ba_ring_init(n_slots, slot_tokens, heads, head_dim, code)
        self.oring = oring.RingModel(n_slots, slot_tokens, heads, head_dim, dtype)
        self.text = None
        self.otext = None
        if text_tokens:
            self.text = B.ba_ring_init(1, text_tokens, heads, head_dim, code)
            self.otext = oring.RingModel(1, text_tokens, heads, head_dim, dtype)

    def append(self, k, v, n=None):
        n = k.shape[0] if n is None else n
        s = self.B.ba_cache_append(self.ring, to_dev(k, self.dtype), to_dev(v, self.dtype), n)
        s2 = self.oring.append(k, v, n)
        assert s == s2
        return s

    def append_batched(self, k, v, slots):
        self.B.ba_cache_append_batched(self.ring, to_dev(k, self.dtype), to_dev(v, self.dtype), slots)
        for i, s in enumerate(slots):
            self.oring.append(k[i], v[i], k.shape[1], slot=s)

    def set_text(self, k, v):
        self.B.ba_cache_append(self.text, to_dev(k, self.dtype), to_dev(v, self.dtype), k.shape[0])
        self.otext.append(k, v, k.shape[0])

    def run(self, q, metas, scale=0.0, with_lse=True, workspace="auto"):
        import torch
        qd = to_dev(q, self.dtype)
        lse = None
        if with_lse:
            lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"),
                             dtype=torch.float32, device="cuda")
        out = torch.full_like(qd, float("nan"))
        self.B.ba_block_attention(qd, self.ring, self.text, metas, scale, out=out, lse=lse,
                                  workspace=workspace)
        torch.cuda.synchronize()
        return out, lse

    def oracle(self, q, metas, scale=None, heads=None, rows=None):
        from oracle import attention as A
        qf = N.decode(q, self.dtype)
        return A.block_attention_ref(qf, self.oring, self.otext, metas,
                                     scale=scale, heads=heads, rows=rows)


def build_config(cfg, inputs=None):
    """Fill rings for one of the five workloads, as the bench does."""
    from workloads import make_attention_inputs
    if inputs is None:
        inputs = make_attention_inputs(cfg)
    H, D = cfg.heads, cfg.head_dim
    w = Workload(cfg.dtype, cfg.n_slots, cfg.slot_tokens, H, D, cfg.text_len)
    if cfg.full_sequence:
        nseg = len(cfg.segs[0])
        L = cfg.segs[0][0][1]
        k = inputs["k_cur"][0].reshape(nseg, L, H, D)
        v = inputs["v_cur"][0].reshape(nseg, L, H, D)
        w.append_batched(k, v, [s for s, _ in cfg.segs[0]])
    elif cfg.n_blocks == 1:
        w.append(inputs["k_ctx"][0], inputs["v_ctx"][0])
        w.append(inputs["k_cur"][0], inputs["v_cur"][0])
    else:
        w.append_batched(inputs["k_ctx"], inputs["v_ctx"], [seg[0][0] for seg in cfg.segs])
        w.append_batched(inputs["k_cur"], inputs["v_cur"], [seg[1][0] for seg in cfg.segs])
    w.set_text(inputs["k_text"], inputs["v_text"])
    metas = [{"q_len": cfg.q_len, "segs": list(cfg.segs[b]), "text_slot": 0,
              "text_len": cfg.text_len} for b in range(cfg.n_blocks)]
    return w, inputs, metas


def default_scale(D):
    return 1.0 / math.sqrt(D)
