"""The fused K/V producer (ba_qkv_project) through the C ABI against the fp64
oracle: Q in its buffer, K and V in the ring slot in the cache's layout with
the slot's tail zeroed, every other slot untouched.

The kernel accumulates the dim products in fp32 on the matrix cores (and
rotates in fp32); the oracle rounds the exact fp64 value once.  Bar: every
element within one bf16 ulp of the exact value plus the fp32 error bound
e = 2^-21 * sum_c |x_c w_c| (covering the accumulation and the rotation),
and at least 99 % of the elements bit-exact."""
import numpy as np
import pytest

from _util import ring_bytes, to_dev, to_host_bits
from oracle import numerics as N
from oracle import projection as P
from oracle import ring as oring
from workloads import draw

pytestmark = pytest.mark.gpu


def _check(got_bits, exact, bound):
    got = N.bf16_bits_to_f64(got_bits)
    mag = np.abs(exact) + bound
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(mag, 2.0 ** -126))).astype(int) - 7)
    bad = np.abs(got - exact) > ulp + bound
    assert not bad.any(), (got[bad][:4], exact[bad][:4])
    frac = float(np.mean(got_bits == N.f64_to_bf16_bits(exact)))
    assert frac >= 0.99, f"bit-exact fraction {frac:.4f}"


def _case(L, dim, H, D, slot, n_slots, with_q, with_rope, seed):
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(seed))
    x = draw(rng, (L, dim), 1.0, "bf16")
    w = draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16")
    table = None
    if with_rope:
        ang = rng.uniform(-40.0, 40.0, (L, D // 2))
        table = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    ring = B.ba_ring_init(n_slots, L + 37, H, D, B.BA_BF16)
    q = torch.full((L, H, D), float("nan"), dtype=torch.bfloat16, device="cuda") if with_q else None
    # the library takes the table pair-major: [D/2][L][2]
    B.ba_qkv_project(to_dev(x, "bf16"), to_dev(w, "bf16"), ring, slot, q=q,
                     rope=torch.from_numpy(table.transpose(1, 0, 2).copy()).cuda() if with_rope else None)
    torch.cuda.synchronize()
    qe, ke, ve = P.qkv_project_ref(x, w, H, D, table)
    absx = np.abs(N.bf16_bits_to_f64(x))
    absw = np.abs(N.bf16_bits_to_f64(w))
    bound = (2.0 ** -21) * (absx @ absw.T)                       # [L][3HD]
    HD = H * D
    bq, bk, bv = (bound[:, j * HD:(j + 1) * HD].reshape(L, H, D) for j in range(3))
    if with_rope:   # a rotated pair mixes both members' errors
        def partner(b):
            return b.reshape(L, H, D // 2, 2)[..., ::-1].reshape(L, H, D)
        bq = bq + partner(bq)
        bk = bk + partner(bk)
    if with_q:
        _check(to_host_bits(q), qe, bq)
    # K and V read back through the ring model's documented offsets
    model = oring.RingModel(n_slots, L + 37, H, D, "bf16")
    buf = np.frombuffer(ring_bytes(ring), dtype=np.uint16)
    got_k = np.empty((L, H, D), np.uint16)
    got_v = np.empty((L, H, D), np.uint16)
    for h in range(H):
        for t in range(L):
            got_k[t, h] = buf[[model.k_offset(slot, h, t, d) for d in range(D)]]
            got_v[t, h] = buf[[model.v_offset(slot, h, t, d) for d in range(D)]]
    _check(got_k, ke, bk)
    _check(got_v, ve, bv)
    # the slot's tail is zero and no other slot was touched
    mask = np.ones(buf.size, bool)
    for h in range(H):
        for t in range(L):
            for d in range(D):
                mask[model.k_offset(slot, h, t, d)] = False
                mask[model.v_offset(slot, h, t, d)] = False
    assert not buf[mask].any()


@pytest.mark.parametrize("L,dim,H,D,with_q,with_rope", [
    (300, 128, 2, 64, True, True),      # ragged token tile, rotation
    (300, 128, 2, 64, True, False),
    (257, 192, 3, 64, True, True),      # odd heads: a channel tile spans q and k
    (200, 256, 2, 128, True, True),
    (130, 64, 1, 64, False, False),     # no q: only the k and v rows are computed
])
def test_producer_matches_oracle(L, dim, H, D, with_q, with_rope):
    _case(L, dim, H, D, slot=1, n_slots=3, with_q=with_q, with_rope=with_rope, seed=L + dim + D)


def test_producer_feeds_attention_like_append():
    # K/V produced into a slot equal, bit for bit, the same K/V appended there
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(5))
    L, dim, H, D = 190, 128, 2, 64
    x = to_dev(draw(rng, (L, dim), 1.0, "bf16"), "bf16")
    w = to_dev(draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16"), "bf16")
    r1 = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    r2 = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    q = torch.empty((L, H, D), dtype=torch.bfloat16, device="cuda")
    B.ba_qkv_project(x, w, r1, 1, q=q)
    # the same projection in three calls' worth of pieces: q from the first,
    # k and v extracted from r1 and appended into r2's slot 1 through the
    # append path; the two rings must be byte-identical
    torch.cuda.synchronize()
    model = oring.RingModel(2, L, H, D, "bf16")
    buf = np.frombuffer(ring_bytes(r1), dtype=np.uint16)
    k = np.empty((L, H, D), np.uint16)
    v = np.empty((L, H, D), np.uint16)
    for h in range(H):
        for t in range(L):
            k[t, h] = buf[[model.k_offset(1, h, t, d) for d in range(D)]]
            v[t, h] = buf[[model.v_offset(1, h, t, d) for d in range(D)]]
    B.ba_cache_append_batched(r2, to_dev(k[None], "bf16"), to_dev(v[None], "bf16"), [1])
    torch.cuda.synchronize()
    assert ring_bytes(r1) == ring_bytes(r2)


@pytest.mark.parametrize("per_block_rope", [False, True])
def test_batched_producer_equals_single_calls(per_block_rope):
    # one launch over three blocks writes, bit for bit, what three single
    # calls write; and meets the bar against the oracle block by block
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(31 + per_block_rope))
    nb, L, dim, H, D = 3, 230, 192, 1, 64
    x = draw(rng, (nb, L, dim), 1.0, "bf16")
    w = draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16")
    tabs = []
    for _ in range(nb if per_block_rope else 1):
        ang = rng.uniform(-40.0, 40.0, (L, D // 2))
        tabs.append(np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32))
    dev_tab = torch.from_numpy(np.stack([t.transpose(1, 0, 2) for t in tabs]).copy()).cuda()
    slots = [4, 0, 2]
    r1 = B.ba_ring_init(5, L + 10, H, D, B.BA_BF16)
    r2 = B.ba_ring_init(5, L + 10, H, D, B.BA_BF16)
    q1 = torch.full((nb, L, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    q2 = torch.full((nb, L, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    B.ba_qkv_project_batched(xd, wd, r1, slots, q=q1, rope=dev_tab if per_block_rope else dev_tab[0])
    for b in range(nb):
        B.ba_qkv_project(xd[b], wd, r2, slots[b], q=q2[b], rope=dev_tab[b if per_block_rope else 0])
    torch.cuda.synchronize()
    assert ring_bytes(r1) == ring_bytes(r2)
    assert np.array_equal(to_host_bits(q1), to_host_bits(q2))
    model = oring.RingModel(5, L + 10, H, D, "bf16")
    buf = np.frombuffer(ring_bytes(r1), dtype=np.uint16)
    absw = np.abs(N.bf16_bits_to_f64(w))
    for b in range(nb):
        tab = tabs[b if per_block_rope else 0]
        qe, ke, ve = P.qkv_project_ref(x[b], w, H, D, tab)
        bound = (2.0 ** -21) * (np.abs(N.bf16_bits_to_f64(x[b])) @ absw.T)
        bq, bk, bv = (bound[:, j * H * D:(j + 1) * H * D].reshape(L, H, D) for j in range(3))
        pr = lambda t: t + t.reshape(L, H, D // 2, 2)[..., ::-1].reshape(L, H, D)
        _check(to_host_bits(q1)[b], qe, pr(bq))
        got_k = np.stack([buf[[model.k_offset(slots[b], 0, t, d) for d in range(D)]] for t in range(L)])[:, None]
        got_v = np.stack([buf[[model.v_offset(slots[b], 0, t, d) for d in range(D)]] for t in range(L)])[:, None]
        _check(got_k, ke, pr(bk))
        _check(got_v, ve, bv)
    # the ring's untouched slots stay zero
    for s in (1, 3):
        assert not any(buf[model.k_offset(s, 0, t, 0)] for t in range(L))


def test_producer_at_480p_shape_sampled():
    # the bench's launch: 5400 tokens x 1536 -> 4608 rows (24 heads x 64),
    # rotation on, one block and the 8-block batch; sampled tokens (tile
    # edges, the ragged tail, random) checked in every output row
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(480))
    nb, L, H, D = 8, 5400, 24, 64
    dim = H * D
    x = draw(rng, (nb, L, dim), 1.0, "bf16")
    w = draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16")
    pos = np.arange(L, dtype=np.float64)[:, None]
    freq = 10000.0 ** (-np.arange(D // 2, dtype=np.float64) * 2 / D)[None, :]
    ang = pos * freq
    table = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)      # [L][D/2][2]
    tdev = torch.from_numpy(table.transpose(1, 0, 2).copy()).cuda()
    ring = B.ba_ring_init(nb + 1, L, H, D, B.BA_BF16)
    q1 = torch.empty((L, H, D), dtype=torch.bfloat16, device="cuda")
    qb = torch.empty((nb, L, H, D), dtype=torch.bfloat16, device="cuda")
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    B.ba_qkv_project(xd[0], wd, ring, nb, q=q1, rope=tdev)                 # one block into the last slot
    B.ba_qkv_project_batched(xd, wd, ring, list(range(nb)), q=qb, rope=tdev)
    torch.cuda.synchronize()
    toks = sorted({0, 1, 255, 256, 511, 512, 5119, 5120, 5375, 5376, 5398, 5399}
                  | set(rng.integers(0, L, 20).tolist()))
    model = oring.RingModel(nb + 1, L, H, D, "bf16")
    buf = np.frombuffer(ring_bytes(ring), dtype=np.uint16)
    absw = np.abs(N.bf16_bits_to_f64(w))
    hh, tt, dd = np.meshgrid(np.arange(H), np.array(toks), np.arange(D), indexing="ij")
    for b, slot, qt in [(0, nb, q1), (0, 0, qb[0]), (5, 5, qb[5]), (7, 7, qb[7])]:
        xs = x[b][toks]
        qe, ke, ve = P.qkv_project_ref(xs, w, H, D, table[toks])
        bound = (2.0 ** -21) * (np.abs(N.bf16_bits_to_f64(xs)) @ absw.T)
        n = len(toks)
        bq, bk, bv = (bound[:, j * dim:(j + 1) * dim].reshape(n, H, D) for j in range(3))
        pr = lambda t: t + t.reshape(n, H, D // 2, 2)[..., ::-1].reshape(n, H, D)
        _check(to_host_bits(qt)[toks], qe, pr(bq))
        got_k = buf[model.k_offset(slot, hh, tt, dd)].transpose(1, 0, 2)         # [n][H][D]
        got_v = buf[model.v_offset(slot, hh, tt, dd)].transpose(1, 0, 2)
        _check(got_k, ke, pr(bk))
        _check(got_v, ve, bv)
    # the one-block call and block 0 of the batch agree bit for bit
    assert np.array_equal(to_host_bits(q1), to_host_bits(qb[0]))


def test_batched_producer_at_the_block_limit():
    # 64 blocks (the largest batch) of a small shape: every slot written as
    # by its own single call, bit for bit
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(64))
    nb, L, dim, H, D = 64, 70, 64, 1, 64
    x = to_dev(draw(rng, (nb, L, dim), 1.0, "bf16"), "bf16")
    w = to_dev(draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16"), "bf16")
    slots = [(5 * b + 1) % nb for b in range(nb)]
    r1 = B.ba_ring_init(nb, L, H, D, B.BA_BF16)
    r2 = B.ba_ring_init(nb, L, H, D, B.BA_BF16)
    B.ba_qkv_project_batched(x, w, r1, slots)
    for b in range(nb):
        B.ba_qkv_project(x[b], w, r2, slots[b])
    torch.cuda.synchronize()
    assert ring_bytes(r1) == ring_bytes(r2)
    assert any(ring_bytes(r1))


def test_producer_at_720p_shape_sampled():
    # 7800 tokens x 5120 -> 15360 rows (40 heads x 128), rotation on, q
    # skipped (only the k and v rows computed); sampled tokens in every row
    import torch
    import block_wise_long_amd as B
    rng = np.random.Generator(np.random.PCG64(720))
    L, H, D = 7800, 40, 128
    dim = H * D
    x = draw(rng, (L, dim), 1.0, "bf16")
    w = draw(rng, (3 * H * D, dim), dim ** -0.5, "bf16")
    ang = rng.uniform(-60.0, 60.0, (L, D // 2))
    table = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    ring = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    B.ba_qkv_project(to_dev(x, "bf16"), to_dev(w, "bf16"), ring, 1,
                     rope=torch.from_numpy(table.transpose(1, 0, 2).copy()).cuda())
    torch.cuda.synchronize()
    toks = sorted({0, 255, 256, 7679, 7680, 7798, 7799} | set(rng.integers(0, L, 12).tolist()))
    n = len(toks)
    _, ke, ve = P.qkv_project_ref(x[toks], w, H, D, table[toks])
    bound = (2.0 ** -21) * (np.abs(N.bf16_bits_to_f64(x[toks])) @ np.abs(N.bf16_bits_to_f64(w)).T)
    bk, bv = (bound[:, j * dim:(j + 1) * dim].reshape(n, H, D) for j in (1, 2))
    model = oring.RingModel(2, L, H, D, "bf16")
    buf = np.frombuffer(ring_bytes(ring), dtype=np.uint16)
    hh, tt, dd = np.meshgrid(np.arange(H), np.array(toks), np.arange(D), indexing="ij")
    pr = lambda t: t + t.reshape(n, H, D // 2, 2)[..., ::-1].reshape(n, H, D)
    _check(buf[model.k_offset(1, hh, tt, dd)].transpose(1, 0, 2), ke, pr(bk))
    _check(buf[model.v_offset(1, hh, tt, dd)].transpose(1, 0, 2), ve, bv)
    # the slot's padded tail (7800 .. 7807) reads as zeros, slot 0 untouched
    tail = buf[model.k_offset(1, hh[:, :1], np.full_like(tt[:, :1], L), dd[:, :1])]
    assert not tail.any() and not buf[model.k_offset(0, hh, tt, dd)].any()
