"""Pins of the fp64 oracle against things other than itself (CPU only).

Every pin below checks the oracle against a closed form, an invariant that
the definition implies, a 60-digit brute force on tiny inputs, a library
routine used as an independent route, or a value worked by hand.  The
mutation test at the end plants plausible mistakes in the oracle and checks
that at least one pin fails for each.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as A
from oracle import noise as NZ
from oracle import numerics as N
from oracle import ring as R
from oracle import projection as P
from oracle import queue as Q
from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# attention pins
# ---------------------------------------------------------------------------

def brute_force_attention(q, K, V, scale):
    """Per-row, pure Python, 60 significant digits, no max subtraction."""
    ctx = decimal.Context(prec=60)
    out, lses = [], []
    for qi in q:
        w = []
        for kj in K:
            s = ctx.multiply(decimal.Decimal(scale),
                             sum((decimal.Decimal(a) * decimal.Decimal(b) for a, b in zip(qi, kj)),
                                 decimal.Decimal(0)))
            w.append(ctx.exp(s))
        z = sum(w, decimal.Decimal(0))
        row = []
        for d in range(len(V[0])):
            num = sum((w[j] * decimal.Decimal(V[j][d]) for j in range(len(K))), decimal.Decimal(0))
            row.append(float(ctx.divide(num, z)))
        out.append(row)
        lses.append(float(ctx.ln(z)))
    return np.array(out), np.array(lses)


def pin_brute_force():
    rng = _rng(1)
    for n, L, D in [(1, 1, 1), (3, 5, 4), (4, 9, 8), (2, 7, 3)]:
        q = rng.standard_normal((n, D))
        K = rng.standard_normal((L, D)) * 2
        V = rng.standard_normal((L, D + 1))
        sc = 1 / math.sqrt(D)
        o, l = A.softmax_attention(q, K, V, sc)
        ob, lb = brute_force_attention(q.tolist(), K.tolist(), V.tolist(), sc)
        assert np.allclose(o, ob, rtol=0, atol=1e-12), np.abs(o - ob).max()
        assert np.allclose(l, lb, rtol=0, atol=1e-12)


def pin_two_key_closed_form():
    # two keys: o = sigmoid(d) v1 + sigmoid(-d) v2 with d = scale (q.k1 - q.k2)
    rng = _rng(2)
    q = rng.standard_normal((5, 6))
    K = rng.standard_normal((2, 6))
    V = rng.standard_normal((2, 3))
    sc = 0.37
    o, lse = A.softmax_attention(q, K, V, sc)
    d = sc * (q @ K[0] - q @ K[1])
    sig = 1 / (1 + np.exp(-d))
    exp_o = sig[:, None] * V[0] + (1 - sig)[:, None] * V[1]
    assert np.allclose(o, exp_o, atol=1e-13)
    s1, s2 = sc * q @ K[0], sc * q @ K[1]
    assert np.allclose(lse, np.logaddexp(s1, s2), atol=1e-13)


def pin_weights_sum_to_one():
    # with V = identity the output rows are the weights themselves
    rng = _rng(3)
    L = 13
    q = rng.standard_normal((7, 5)) * 3
    K = rng.standard_normal((L, 5)) * 3
    o, _ = A.softmax_attention(q, K, np.eye(L), 1.0)
    assert np.all(o >= 0)
    assert np.allclose(o.sum(axis=1), 1.0, atol=1e-12)
    # and they are the softmax of the scores (library routine as the other route)
    assert np.allclose(o, scipy.special.softmax(q @ K.T, axis=1), atol=1e-12)


def pin_key_permutation_invariance():
    rng = _rng(4)
    q = rng.standard_normal((6, 8))
    K = rng.standard_normal((20, 8))
    V = rng.standard_normal((20, 8))
    perm = rng.permutation(20)
    o1, l1 = A.softmax_attention(q, K, V, 0.3)
    o2, l2 = A.softmax_attention(q, K[perm], V[perm], 0.3)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def pin_uniform_when_q_zero():
    rng = _rng(5)
    K = rng.standard_normal((11, 4))
    V = rng.standard_normal((11, 4))
    o, lse = A.softmax_attention(np.zeros((2, 4)), K, V, 1.0)
    assert np.allclose(o, V.mean(axis=0), atol=1e-13)
    assert np.allclose(lse, math.log(11), atol=1e-13)


def pin_needle():
    rng = _rng(6)
    D, L = 8, 30
    q = rng.standard_normal((1, D))
    K = rng.standard_normal((L, D)) * 0.01
    V = rng.standard_normal((L, D))
    K[17] = 500 * q[0] / np.linalg.norm(q[0])
    o, _ = A.softmax_attention(q, K, V, 1.0)
    assert np.array_equal(o[0], V[17]) or np.allclose(o[0], V[17], rtol=0, atol=1e-300)


def _tiny_ring_setup(seed=7, slot_tokens=6, lens=(6, 5, 6, 4), heads=2, D=4, text=3):
    rng = _rng(seed)
    ring = R.RingModel(n_slots=5, slot_tokens=slot_tokens, heads=heads, head_dim=D, dtype="f32")
    blocks = []
    for n in lens:
        k = rng.standard_normal((n, heads, D)).astype(np.float32)
        v = rng.standard_normal((n, heads, D)).astype(np.float32)
        ring.append(k, v, n)
        blocks.append((k, v))
    tring = R.RingModel(n_slots=1, slot_tokens=8, heads=heads, head_dim=D, dtype="f32")
    tk = rng.standard_normal((text, heads, D)).astype(np.float32)
    tv = rng.standard_normal((text, heads, D)).astype(np.float32)
    tring.append(tk, tv, text)
    return rng, ring, tring, blocks, (tk, tv)


def pin_full_prefix_equivalence():
    # A video of 4 tiny blocks; the last block's queries over the cache holding
    # the whole prefix equal plain full attention over the concatenated sequence,
    # restricted to that block's rows (computed here by the 60-digit brute force).
    rng, ring, tring, blocks, (tk, tv) = _tiny_ring_setup()
    H, D = 2, 4
    n3 = blocks[3][0].shape[0]
    q = rng.standard_normal((1, n3, H, D))
    meta = {"q_len": n3, "segs": [(0, 6), (1, 5), (2, 6), (3, 4)], "text_slot": 0, "text_len": 3}
    out, lse = A.block_attention_ref(q, ring, tring, [meta], scale=0.5)
    for h in range(H):
        Kf = np.concatenate([b[0][:, h, :] for b in blocks] + [tk[:, h, :]]).astype(np.float64)
        Vf = np.concatenate([b[1][:, h, :] for b in blocks] + [tv[:, h, :]]).astype(np.float64)
        ob, lb = brute_force_attention(q[0, :, h, :].tolist(), Kf.tolist(), Vf.tolist(), 0.5)
        assert np.allclose(out[0, :, h, :], ob, atol=1e-12)
        assert np.allclose(lse[0, h, :], lb, atol=1e-12)


def pin_key_set_order_and_lengths():
    rng, ring, tring, blocks, (tk, tv) = _tiny_ring_setup()
    meta = {"q_len": 1, "segs": [(2, 3), (0, 6)], "text_slot": 0, "text_len": 2}
    K, V = A.key_set(ring, tring, meta, 1)
    expK = np.concatenate([blocks[2][0][:3, 1], blocks[0][0][:6, 1], tk[:2, 1]])
    expV = np.concatenate([blocks[2][1][:3, 1], blocks[0][1][:6, 1], tv[:2, 1]])
    assert np.array_equal(K, expK.astype(np.float64))
    assert np.array_equal(V, expV.astype(np.float64))


def pin_tokens_past_length_ignored():
    rng, ring, tring, blocks, _ = _tiny_ring_setup()
    q = rng.standard_normal((1, 3, 2, 4))
    meta = {"q_len": 3, "segs": [(0, 2), (1, 5)], "text_slot": 0, "text_len": 1}
    o1, _ = A.block_attention_ref(q, ring, tring, [meta])
    # overwrite everything past the lengths; the result must not move
    k0 = blocks[0][0].copy(); v0 = blocks[0][1].copy()
    k0[2:] = 99.0; v0[2:] = -99.0
    ring.append(k0, v0, 6, slot=0)
    tk = np.full((3, 2, 4), 50.0, np.float32); tv = np.full((3, 2, 4), 7.0, np.float32)
    tk[0] = tring.keys(0, 0, 1)[0][None].astype(np.float32).repeat(1, 0)
    tk[0, 1] = tring.keys(0, 1, 1)[0]
    tv[0, 0] = tring.values(0, 0, 1)[0]
    tv[0, 1] = tring.values(0, 1, 1)[0]
    tring.append(tk, tv, 3, slot=0)
    o2, _ = A.block_attention_ref(q, ring, tring, [meta])
    assert np.array_equal(o1, o2)


def pin_default_scale():
    rng, ring, tring, _, _ = _tiny_ring_setup()
    q = rng.standard_normal((1, 4, 2, 4))
    meta = {"q_len": 4, "segs": [(1, 5), (3, 4)], "text_slot": 0, "text_len": 3}
    o1, l1 = A.block_attention_ref(q, ring, tring, [meta])
    o2, l2 = A.block_attention_ref(q, ring, tring, [meta], scale=0.5)  # 1/sqrt(4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, _ = A.block_attention_ref(q, ring, tring, [meta], scale=0.25)
    assert not np.allclose(o1, o3)


def pin_rows_and_heads_subset():
    rng, ring, tring, _, _ = _tiny_ring_setup()
    q = rng.standard_normal((2, 5, 2, 4))
    metas = [{"q_len": 5, "segs": [(0, 6), (1, 5)], "text_slot": 0, "text_len": 3},
             {"q_len": 3, "segs": [(2, 6)], "text_slot": 0, "text_len": 0}]
    o, l = A.block_attention_ref(q, ring, tring, metas)
    os_, ls = A.block_attention_ref(q, ring, tring, metas, heads=[1], rows=[0, 4])
    # BLAS may take another summation path for fewer rows: equal to rounding
    assert np.allclose(os_[0, [0, 4], 1], o[0, [0, 4], 1], rtol=0, atol=1e-14)
    assert np.allclose(os_[1, [0], 1], o[1, [0], 1], rtol=0, atol=1e-14)
    assert np.isnan(os_[1, 4]).all() and np.isnan(o[1, 3:]).all()
    assert np.isnan(os_[0, :, 0]).all()


def pin_lse():
    rng = _rng(9)
    q = rng.standard_normal((4, 6))
    K = rng.standard_normal((25, 6)) * 4
    V = rng.standard_normal((25, 6))
    _, lse = A.softmax_attention(q, K, V, 0.9)
    assert np.allclose(lse, scipy.special.logsumexp(0.9 * q @ K.T, axis=1), atol=1e-12)


def pin_split_text_parts_by_brute_force():
    # separate text cross-attention: the self part is the 60-digit brute force
    # over the cache segments alone, the text part over the text keys alone
    rng, ring, tring, blocks, (tk, tv) = _tiny_ring_setup(seed=11)
    H, D = 2, 4
    q = rng.standard_normal((1, 5, H, D))
    meta = {"q_len": 5, "segs": [(1, 5), (2, 6)], "text_slot": 0, "text_len": 3}
    (os_, ls), (ot, lt) = A.split_text_attention_ref(q, ring, tring, [meta], scale=0.7)
    for h in range(H):
        Ks = np.concatenate([blocks[1][0][:, h], blocks[2][0][:, h]]).astype(np.float64)
        Vs = np.concatenate([blocks[1][1][:, h], blocks[2][1][:, h]]).astype(np.float64)
        ob, lb = brute_force_attention(q[0, :, h].tolist(), Ks.tolist(), Vs.tolist(), 0.7)
        assert np.allclose(os_[0, :, h], ob, atol=1e-12) and np.allclose(ls[0, h], lb, atol=1e-12)
        ob, lb = brute_force_attention(q[0, :, h].tolist(), tk[:, h].astype(np.float64).tolist(),
                                       tv[:, h].astype(np.float64).tolist(), 0.7)
        assert np.allclose(ot[0, :, h], ob, atol=1e-12) and np.allclose(lt[0, h], lb, atol=1e-12)


def pin_split_parts_merge_to_joint():
    # the two parts, weighted by exp(lse_part - lse_union), are the joint
    # softmax over [cache | text] computed in one go; and the union's lse is
    # the joint lse
    rng, ring, tring, blocks, (tk, tv) = _tiny_ring_setup(seed=12)
    H, D = 2, 4
    q = rng.standard_normal((2, 6, H, D)) * 1.5
    metas = [{"q_len": 6, "segs": [(0, 6), (3, 4)], "text_slot": 0, "text_len": 3},
             {"q_len": 4, "segs": [(2, 6)], "text_slot": 0, "text_len": 1}]
    joint, jl = A.block_attention_ref(q, ring, tring, metas)
    (os_, ls), (ot, lt) = A.split_text_attention_ref(q, ring, tring, metas)
    lt_rows = np.transpose(lt, (0, 2, 1))               # [b][row][head]
    ls_rows = np.transpose(ls, (0, 2, 1))
    merged, ml = A.merge_partials(os_, ls_rows, ot, lt_rows)
    ok = ~np.isnan(joint)
    assert np.allclose(merged[ok], joint[ok], rtol=0, atol=1e-12)
    assert np.allclose(np.transpose(ml, (0, 2, 1))[~np.isnan(jl)], jl[~np.isnan(jl)], atol=1e-12)
    # the parts differ from the joint output (the text competes in the joint softmax)
    assert np.abs(os_[ok] - joint[ok]).max() > 1e-3


def pin_merge_partials_closed_form():
    # two single-key parts: the union is the two-key softmax, a logistic mix
    v1, v2 = np.array([1.0, -2.0]), np.array([3.0, 0.5])
    for s1, s2 in [(0.3, -1.1), (5.0, 5.0), (-40.0, 2.0)]:
        o, l = A.merge_partials(v1[None], np.array([s1]), v2[None], np.array([s2]))
        w = 1.0 / (1.0 + math.exp(s2 - s1))
        assert np.allclose(o[0], w * v1 + (1 - w) * v2, atol=1e-15)
        assert abs(l[0] - (max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-14


ATTENTION_PINS = [pin_brute_force, pin_two_key_closed_form, pin_weights_sum_to_one,
                  pin_key_permutation_invariance, pin_uniform_when_q_zero, pin_needle,
                  pin_full_prefix_equivalence, pin_key_set_order_and_lengths,
                  pin_tokens_past_length_ignored, pin_default_scale,
                  pin_rows_and_heads_subset, pin_lse, pin_split_text_parts_by_brute_force,
                  pin_split_parts_merge_to_joint, pin_merge_partials_closed_form]


# ---------------------------------------------------------------------------
# ring pins
# ---------------------------------------------------------------------------

def pin_ring_fifo_wraps():
    ring = R.RingModel(3, 4, 1, 2, "bf16")
    slots = [ring.append(np.full((4, 1, 2), i, np.uint16), np.full((4, 1, 2), i, np.uint16), 4)
             for i in range(7)]
    assert slots == [0, 1, 2, 0, 1, 2, 0] and ring.appended == 7
    assert ring.append(np.ones((4, 1, 2), np.uint16), np.ones((4, 1, 2), np.uint16), 2, slot=2) == 2
    assert ring.appended == 7


def pin_ring_layout_golden():
    with open(os.path.join(GOLDEN, "ring_layout_tiny.json")) as f:
        g = json.load(f)
    ring = R.RingModel(**g["ring"], dtype="bf16")
    assert ring.mem.size == g["total_elems"] and ring.t_pad == 64
    # write distinct codes so every element is identifiable
    H, D = g["ring"]["heads"], g["ring"]["head_dim"]
    for s in range(g["ring"]["n_slots"]):
        t = np.arange(5)[:, None, None]; h = np.arange(H)[None, :, None]; d = np.arange(D)[None, None, :]
        k = (1 + s * 1000 + t * 100 + h * 10 + d).astype(np.uint16)
        v = (20000 + s * 1000 + t * 100 + h * 10 + d).astype(np.uint16)
        ring.append(k, v, 5, slot=s)
    for e in g["k"]:
        assert ring.mem[e["offset"]] == 1 + e["s"] * 1000 + e["t"] * 100 + e["h"] * 10 + e["d"]
    for e in g["v"]:
        assert ring.mem[e["offset"]] == 20000 + e["s"] * 1000 + e["t"] * 100 + e["h"] * 10 + e["d"]


def pin_ring_roundtrip_and_zero_tail():
    rng = _rng(11)
    ring = R.RingModel(2, 70, 3, 8, "bf16")
    assert ring.t_pad == 128
    k = rng.integers(1, 60000, (70, 3, 8)).astype(np.uint16)
    v = rng.integers(1, 60000, (70, 3, 8)).astype(np.uint16)
    ring.append(k, v, 70, slot=1)
    k2 = rng.integers(1, 60000, (70, 3, 8)).astype(np.uint16)
    ring.append(k2, k2, 33, slot=1)   # shorter append: tokens 33.. become zero
    for h in range(3):
        assert np.array_equal(ring.keys(1, h, 33), N.bf16_bits_to_f64(k2[:33, h]))
        assert np.array_equal(ring.values(1, h, 33), N.bf16_bits_to_f64(k2[:33, h]))
        assert not ring.keys(1, h, 128)[33:].any() and not ring.values(1, h, 128)[33:].any()
    assert not ring.mem[: ring.mem.size // 2].any()   # slot 0 untouched


def pin_ring_loop_writer():
    # element-by-element writer in plain loops gives the same bytes
    rng = _rng(12)
    S_, T, H, D = 2, 3, 2, 2
    ring = R.RingModel(S_, T, H, D, "bf16")
    k = rng.integers(1, 999, (T, H, D)).astype(np.uint16)
    v = rng.integers(1, 999, (T, H, D)).astype(np.uint16)
    ring.append(k, v, T, slot=1)
    ref = np.zeros(S_ * 2 * H * 64 * D, np.uint16)
    for t in range(T):
        for h in range(H):
            for d in range(D):
                ref[(((1 * 2) + 0) * H + h) * 64 * D + t * D + d] = k[t, h, d]
                ref[(((1 * 2) + 1) * H + h) * 64 * D + d * 64 + t] = v[t, h, d]
    assert np.array_equal(ring.mem, ref)


RING_PINS = [pin_ring_fifo_wraps, pin_ring_layout_golden, pin_ring_roundtrip_and_zero_tail,
             pin_ring_loop_writer]


# ---------------------------------------------------------------------------
# schedule pins
# ---------------------------------------------------------------------------

def pin_alpha_bar_start_and_product():
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    assert ab[0] == 1.0 and ab[1] == 1.0 - 1e-4
    b = np.array([1e-4 + (0.02 - 1e-4) * i / 999 for i in range(1000)])
    other = np.exp(np.cumsum(np.log1p(-b)))          # a different route: sum of logs
    assert np.allclose(ab[1:], other, rtol=1e-12, atol=0)
    assert np.all(np.diff(ab) < 0)
    assert abs(ab[1000] - 4.035830e-5) < 5e-11


def pin_betas_linear():
    b = S.betas(1000, 1e-4, 0.02)
    assert b[0] == 1e-4 and abs(b[-1] - 0.02) < 1e-18
    assert np.allclose(np.diff(b), (0.02 - 1e-4) / 999, rtol=1e-9)


def pin_two_step_schedule_by_hand():
    # T = 2, betas (0.1, 0.3): abar_1 = 0.9, abar_2 = 0.63.  A step from t=2 to
    # t'=0 returns x0_hat = (x - sqrt(0.37) eps) / sqrt(0.63).
    ab = S.alpha_bar(2, 0.1, 0.3)
    assert abs(ab[1] - 0.9) < 1e-15 and abs(ab[2] - 0.63) < 1e-15
    x, e = 1.25, -0.5
    got = S.ddim_step(np.array([x]), np.array([e]), 2, 0, ab)[0]
    assert abs(got - (1.25 + 0.5 * math.sqrt(0.37)) / math.sqrt(0.63)) < 1e-14
    # t=2 -> t'=1: sqrt(0.9) x0_hat + sqrt(0.1) eps
    got = S.ddim_step(np.array([x]), np.array([e]), 2, 1, ab)[0]
    x0 = (1.25 + 0.5 * math.sqrt(0.37)) / math.sqrt(0.63)
    assert abs(got - (math.sqrt(0.9) * x0 - 0.5 * math.sqrt(0.1))) < 1e-14


def pin_ddim_consistency():
    # x on the forward-process line of (x0, eps) stays on it after a step
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    rng = _rng(13)
    x0 = rng.standard_normal(100)
    eps = rng.standard_normal(100)
    for t in [1, 20, 143, 500, 999, 1000]:
        tp = S.prev_timestep(t, 20)
        x = math.sqrt(ab[t]) * x0 + math.sqrt(1 - ab[t]) * eps
        exp = math.sqrt(ab[tp]) * x0 + math.sqrt(1 - ab[tp]) * eps
        assert np.allclose(S.ddim_step(x, eps, t, tp, ab), exp, atol=1e-10)


def pin_trajectory_recovers_x0():
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    rng = _rng(14)
    x0 = rng.standard_normal(50)
    eps = rng.standard_normal(50)
    x = math.sqrt(ab[1000]) * x0 + math.sqrt(1 - ab[1000]) * eps
    t = 1000
    while t > 0:
        tp = S.prev_timestep(t, 20)
        x = S.ddim_step(x, eps, t, tp, ab)
        t = tp
    assert np.allclose(x, x0, atol=1e-9)


def pin_identity_and_coefficients():
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    rng = _rng(15)
    x = rng.standard_normal(64)
    e = rng.standard_normal(64)
    for t in [0, 7, 500]:
        assert np.allclose(S.ddim_step(x, e, t, t, ab), x, atol=1e-14)
        c1, c2 = S.ddim_coefficients(t, t, ab)
        assert abs(c1 - 1) < 1e-15 and abs(c2) < 1e-15
    for t in [1, 143, 1000]:
        tp = S.prev_timestep(t, 20)
        c1, c2 = S.ddim_coefficients(t, tp, ab)
        assert np.allclose(c1 * x + c2 * e, S.ddim_step(x, e, t, tp, ab), atol=1e-13)
        assert c1 >= 1.0 and c2 < 0


def pin_prev_timestep():
    assert S.prev_timestep(1000, 20) == 980 and S.prev_timestep(15, 20) == 0
    assert S.prev_timestep(20, 20) == 0 and S.prev_timestep(0, 20) == 0


def pin_bf16_rounding():
    cases = {1.0: 0x3F80, 1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82,
             1 + 2 ** -8 + 2 ** -40: 0x3F81, -2.0: 0xC000, 0.0: 0x0000,
             3.5e38: 0x7F80, 2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000,
             1.5 * 2.0 ** -133: 0x0002}
    for x, bits in cases.items():
        assert int(N.f64_to_bf16_bits(np.array([x]))[0]) == bits, (x, hex(bits))
    # on fp32-representable values, single rounding equals torch's fp32 -> bf16
    x = _rng(16).standard_normal(20000).astype(np.float32) * 7
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(N.f64_to_bf16_bits(x.astype(np.float64)), tb)
    assert np.array_equal(N.bf16_bits_to_f64(tb), torch.from_numpy(tb.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def pin_block_update_rounding():
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    rng = _rng(17)
    x = N.f64_to_bf16_bits(rng.standard_normal((2, 300)))
    e = N.f64_to_bf16_bits(rng.standard_normal((2, 300)))
    out = S.block_update_ref(x, e, [500, 0])
    assert np.array_equal(out[1], x[1])    # t = 0: t' = 0, identity
    exact = S.ddim_step(N.bf16_bits_to_f64(x[0]), N.bf16_bits_to_f64(e[0]), 500, 480, ab)
    got = N.bf16_bits_to_f64(out[0])
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)


def pin_flow_sigma_by_hand():
    # linear: sigma = t / T; shift 3 at u = 1/2: 1.5 / (1 + 1) = 0.75; ends 0 and 1
    assert S.flow_sigma(250, 1000) == 0.25 and S.flow_sigma(1000, 1000) == 1.0
    assert S.flow_sigma(0, 1000, 3.0) == 0.0 and S.flow_sigma(1000, 1000, 3.0) == 1.0
    assert abs(S.flow_sigma(500, 1000, 3.0) - 0.75) < 1e-15
    # shift s maps the linear sigma u to s u / (1 + (s - 1) u): its inverse is
    # the same map with 1 / s
    for u in [0.1, 0.37, 0.9]:
        s_u = S.flow_sigma(u * 1000, 1000, 5.0)
        assert abs(S.flow_sigma(s_u * 1000, 1000, 0.2) - u) < 1e-12
    sig = [S.flow_sigma(t, 1000, 5.0) for t in range(0, 1001, 50)]
    assert np.all(np.diff(sig) > 0)


def pin_flow_consistency():
    # on the straight path x_s = (1 - s) x0 + s eps with v = eps - x0, one Euler
    # step lands exactly on the path at the next noise level
    rng = _rng(18)
    x0 = rng.standard_normal(80)
    eps = rng.standard_normal(80)
    for shift in [1.0, 3.0, 7.5]:
        for t in [1000, 733, 143, 20, 7]:
            tp = S.prev_timestep(t, 20)
            st, sp = S.flow_sigma(t, 1000, shift), S.flow_sigma(tp, 1000, shift)
            x = (1 - st) * x0 + st * eps
            assert np.allclose(S.flow_step(x, eps - x0, t, tp, 1000, shift), (1 - sp) * x0 + sp * eps,
                               atol=1e-12)


def pin_flow_trajectory_recovers_x0():
    rng = _rng(19)
    x0 = rng.standard_normal(40)
    eps = rng.standard_normal(40)
    x, t = eps.copy(), 1000          # sigma(T) = 1: pure noise
    while t > 0:
        tp = S.prev_timestep(t, 20)
        x = S.flow_step(x, eps - x0, t, tp, 1000, 3.0)
        t = tp
    assert np.allclose(x, x0, atol=1e-12)


def pin_flow_coefficients_and_update():
    for t, tp in [(1000, 980), (143, 123), (5, 0)]:
        c1, c2 = S.flow_coefficients(t, tp, 1000)
        assert c1 == 1.0 and abs(c2 - (tp - t) / 1000) < 1e-15
    rng = _rng(20)
    x = N.f64_to_bf16_bits(rng.standard_normal((2, 200)))
    v = N.f64_to_bf16_bits(rng.standard_normal((2, 200)))
    out = S.block_update_ref(x, v, [600, 0], kind="flow", shift=3.0)
    assert np.array_equal(out[1], x[1])          # t = 0: no step
    sp, st = S.flow_sigma(580, 1000, 3.0), S.flow_sigma(600, 1000, 3.0)
    exact = N.bf16_bits_to_f64(x[0]) + (sp - st) * N.bf16_bits_to_f64(v[0])
    assert np.array_equal(out[0], N.f64_to_bf16_bits(exact))


SCHEDULE_PINS = [pin_alpha_bar_start_and_product, pin_betas_linear, pin_two_step_schedule_by_hand,
                 pin_ddim_consistency, pin_trajectory_recovers_x0, pin_identity_and_coefficients,
                 pin_prev_timestep, pin_bf16_rounding, pin_block_update_rounding,
                 pin_flow_sigma_by_hand, pin_flow_consistency, pin_flow_trajectory_recovers_x0,
                 pin_flow_coefficients_and_update]

# ---------------------------------------------------------------------------
# FIFO queue pins: simulate the queue symbolically (which block wrote which
# ring slot at which step) and check the rules' consequences
# ---------------------------------------------------------------------------

def _simulate_queue(n_queue, T, steps):
    written = {}                     # ring slot -> (block, step) of its last write
    ages = {}                        # block -> list of its timesteps, step by step
    head = 0
    for g in range(steps):
        pl, stride = Q.plan(n_queue, T, 10, 3, g, head)
        assert stride * n_queue == T
        reads, writes = [], []
        for m, e in enumerate(pl):
            k = e["block"]
            assert k % n_queue == m                      # latent slot of block k
            ages.setdefault(k, []).append(e["t"])
            segs = e["meta"]["segs"]
            assert segs[-1] == (e["write_slot"], 10)     # own K/V last among the segments
            if g == 0:
                assert len(segs) == 1
            else:
                assert len(segs) == 2
                reads.append((k, segs[0][0]))
            writes.append((k, e["write_slot"]))
        ws = [w for _, w in writes]
        assert len(set(ws)) == n_queue                   # no two blocks share a slot
        assert not set(ws) & {r for _, r in reads}       # nothing read is overwritten this step
        for k, r in reads:                               # the neighbour's K/V of the previous step
            assert written[r] == (k - 1, g - 1), (g, k, r, written.get(r))
        for k, w in writes:
            written[w] = (k, g)
        head += 1
    return ages


def pin_queue_context_is_neighbour_previous_step():
    for n in [1, 2, 3, 8]:
        _simulate_queue(n, 8 * 5 * 7 * n if n > 1 else 10, 3 * n + 5)


def pin_queue_noise_staircase():
    # every block that enters at the tail passes t = T, T - s, ..., s, one rung
    # per step, and leaves right after the step at t = s
    n, T = 4, 1000
    ages = _simulate_queue(n, T, 30)
    s = T // n
    for k, ts in ages.items():
        if k >= n and len(ts) == n:                      # entered at the tail, left at the head
            assert ts == [T - j * s for j in range(n)], (k, ts)
    assert ages[0] == [s] and ages[n - 1][:2] == [T, T - s]


QUEUE_PINS = [pin_queue_context_is_neighbour_previous_step, pin_queue_noise_staircase]


# ---------------------------------------------------------------------------
# K/V producer pins
# ---------------------------------------------------------------------------

def pin_projection_brute_force():
    # the linear layer by explicit loops on a tiny shape, split into q | k | v
    rng = _rng(30)
    L, dim, H, D = 3, 5, 2, 4
    xb = N.f64_to_bf16_bits(rng.standard_normal((L, dim)))
    wb = N.f64_to_bf16_bits(rng.standard_normal((3 * H * D, dim)))
    x, w = N.bf16_bits_to_f64(xb), N.bf16_bits_to_f64(wb)
    q, k, v = P.qkv_project_ref(xb, wb, H, D)
    for t in range(L):
        for j, out in enumerate((q, k, v)):
            for h in range(H):
                for d in range(D):
                    row = j * H * D + h * D + d
                    acc = math.fsum(x[t, c] * w[row, c] for c in range(dim))
                    assert abs(out[t, h, d] - acc) < 1e-12


def pin_rotation_identity_quarter_turn_and_norm():
    rng = _rng(31)
    y = rng.standard_normal((4, 3, 8))
    ident = np.zeros((4, 4, 2)); ident[..., 0] = 1.0
    assert np.array_equal(P.rotate_pairs(y, ident), y)
    quarter = np.zeros((4, 4, 2)); quarter[..., 1] = 1.0          # multiply by i: (a, b) -> (-b, a)
    r = P.rotate_pairs(y, quarter)
    assert np.array_equal(r[..., 0::2], -y[..., 1::2]) and np.array_equal(r[..., 1::2], y[..., 0::2])
    ang = rng.uniform(-7, 7, (4, 4))
    tab = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    r = P.rotate_pairs(y, tab)
    n0 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


def pin_rotation_relative_position():
    # rotating q by angle a and k by angle b leaves <q, k> depending on a - b
    # only: the property the rotation is used for
    rng = _rng(32)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    freqs = rng.uniform(0.01, 1.0, 8)

    def rot(y, pos):
        ang = (pos * freqs)[None, :]
        return P.rotate_pairs(y, np.stack([np.cos(ang), np.sin(ang)], axis=-1))
    d1 = float(np.sum(rot(q, 17.0) * rot(k, 5.0)))
    d2 = float(np.sum(rot(q, 112.0) * rot(k, 100.0)))
    d3 = float(np.sum(rot(q, 5.0) * rot(k, 17.0)))
    assert abs(d1 - d2) < 1e-12 and abs(d1 - d3) > 1e-6


PROJECTION_PINS = [pin_projection_brute_force, pin_rotation_identity_quarter_turn_and_norm,
                   pin_rotation_relative_position]

# ---------------------------------------------------------------------------
# coordinated noise initialisation pins
# ---------------------------------------------------------------------------

def pin_noise_weyl_sequence():
    # the generator is a Weyl sequence under a fixed finaliser: its k-th
    # output is the finaliser of seed + (k + 1) gamma, whatever came before
    for seed in (0, 1, 0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF):
        g = NZ.SplitMix64(seed)
        for k in range(50):
            assert g.next() == NZ.finalise((seed + (k + 1) * NZ.GAMMA) % (1 << 64))
    # the finaliser is a bijection of 64-bit words: undo it step by step
    inv1 = pow(0xBF58476D1CE4E5B9, -1, 1 << 64)
    inv2 = pow(0x94D049BB133111EB, -1, 1 << 64)

    def unshift(z, k):
        x = z
        for _ in range(64 // k + 1):
            x = z ^ (x >> k)
        return x
    rng = _rng(60)
    for z in rng.integers(0, 1 << 63, 20, dtype=np.int64).tolist() + [0, 1, (1 << 64) - 1]:
        y = NZ.finalise(z)
        x = unshift(((unshift(y, 31) * inv2) % (1 << 64)), 27)
        x = unshift((x * inv1) % (1 << 64), 30)
        assert x == z


def pin_noise_below_rejects_the_biased_zone():
    class Feed(NZ.SplitMix64):
        def __init__(self, vals):
            self.vals = list(vals)

        def next(self):
            return self.vals.pop(0)
    n = (1 << 63) + 1                      # 2^64 mod n = 2^63 - 1: about half the words are rejected
    g = Feed([5, (1 << 63) - 2, (1 << 63) + 7])
    assert g.below(n) == ((1 << 63) + 7) % n and not g.vals
    g = Feed([0, 7])
    assert g.below(1) == 0 and g.vals == [7]   # n = 1: nothing rejected
    # range and balance of small bounds
    g = NZ.SplitMix64(61)
    draws = [g.below(3) for _ in range(30000)]
    cnt = np.bincount(draws, minlength=3)
    assert cnt.sum() == 30000 and len(cnt) == 3
    chi2 = float(((cnt - 10000.0) ** 2 / 10000.0).sum())
    assert chi2 < 30.0                      # 2 dof: p ~ 3e-7


def pin_noise_assign_distinct_excluded_deterministic():
    for seed in (0, 7, 12345):
        for pool, excl, bf in ((21, 3, 4), (21, 0, 21), (9, 8, 1), (33, 5, 8)):
            for b in range(0, 40, 7):
                a = NZ.assign(seed, b, pool, excl, bf)
                assert len(a) == bf and len(set(a)) == bf and all(0 <= f < pool - excl for f in a)
                assert NZ.assign(seed, b, pool, excl, bf) == a     # any GPU computes the same
    seqs = {tuple(NZ.assign(3, b, 21, 3, 4)) for b in range(60)}
    assert len(seqs) > 50                   # consecutive blocks do not repeat one pattern
    for bad in ((0, 0, 10, 3, 8), (0, 0, 10, 10, 1)):   # more frames than candidates; none left
        try:
            NZ.assign(*bad)
        except ValueError:
            continue
        raise AssertionError(f"assign{bad} accepted")


def pin_noise_assign_uniform():
    # every ordering of the candidates equally likely: 24 permutations of 4,
    # and the 20 ordered pairs of 5 (partial shuffle); chi-square, p ~ 1e-6
    perms = {}
    for seed in range(12000):
        for b in (0, 1):
            t = tuple(NZ.assign(seed, b, 6, 2, 4))
            perms[t] = perms.get(t, 0) + 1
    assert len(perms) == 24
    c = np.array(list(perms.values()), float)
    assert float(((c - 1000.0) ** 2 / 1000.0).sum()) < 66.0
    pairs = {}
    for seed in range(20000):
        t = tuple(NZ.assign(seed, 3, 5, 0, 2))
        pairs[t] = pairs.get(t, 0) + 1
    assert len(pairs) == 20
    c = np.array(list(pairs.values()), float)
    assert float(((c - 1000.0) ** 2 / 1000.0).sum()) < 60.0


def pin_noise_block_gather_by_hand():
    C, F, E = 3, 7, 5
    pool = np.arange(C * F * E, dtype=np.int64).reshape(C, F, E)
    frames = [6, 0, 3]
    out = NZ.noise_block_ref(pool, C, F, frames)
    assert out.shape == (C, 3, E)
    for c in range(C):
        for i, f in enumerate(frames):
            for e in range(E):
                assert out[c, i, e] == (c * F + f) * E + e


NOISE_PINS = [pin_noise_weyl_sequence, pin_noise_below_rejects_the_biased_zone,
              pin_noise_assign_distinct_excluded_deterministic, pin_noise_assign_uniform,
              pin_noise_block_gather_by_hand]

ALL_PINS = ATTENTION_PINS + RING_PINS + SCHEDULE_PINS + QUEUE_PINS + PROJECTION_PINS + NOISE_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_drop_text(orig):
    def key_set(ring, text_ring, meta, head):
        m = dict(meta); m["text_len"] = 0
        return orig(ring, text_ring, m, head)
    return key_set


def _mut_seg_off_by_one(orig):
    def key_set(ring, text_ring, meta, head):
        m = dict(meta); m["segs"] = [(s, max(n - 1, 1)) for s, n in meta["segs"]]
        return orig(ring, text_ring, m, head)
    return key_set


def _mut_values_are_keys(orig):
    def key_set(ring, text_ring, meta, head):
        K, V = orig(ring, text_ring, meta, head)
        return K, K.copy()
    return key_set


def _mut_scale(orig):
    def block_attention_ref(q, ring, text_ring, metas, scale=None, heads=None, rows=None):
        if scale is None:
            scale = 1.0 / q.shape[-1]
        return orig(q, ring, text_ring, metas, scale, heads, rows)
    return block_attention_ref


def _mut_softmax_axis(orig):
    # normalises over the queries instead of over the keys
    def softmax_attention(q, k, v, scale, chunk=256):
        s = scale * (np.asarray(q) @ np.asarray(k).T)
        e = np.exp(s - s.max(axis=0, keepdims=True))
        o = (e / e.sum(axis=0, keepdims=True)) @ np.asarray(v)
        return o, scipy.special.logsumexp(s, axis=1)
    return softmax_attention


def _mut_lse_no_max(orig):
    def softmax_attention(q, k, v, scale, chunk=256):
        o, lse = orig(q, k, v, scale, chunk)
        s = scale * (np.asarray(q) @ np.asarray(k).T)
        return o, lse - s.max(axis=1)
    return softmax_attention


def _mut_ring_v_not_transposed(orig_cls):
    class Mut(orig_cls):
        def v_offset(self, s, h, t, d):
            H, D, T = self.heads, self.head_dim, self.t_pad
            return ((s * 2 + 1) * H + h) * T * D + t * D + d
    return Mut


def _mut_ring_fifo(orig_cls):
    class Mut(orig_cls):
        def append(self, k, v, n_tokens, slot=None):
            if slot is None:
                slot = min(self.appended, self.n_slots - 1)
                self.appended += 1
            return orig_cls.append(self, k, v, n_tokens, slot)
    return Mut


def _mut_abar_index(orig):
    def alpha_bar(T, b0, b1):
        ab = orig(T, b0, b1)
        return np.concatenate([[1.0, 1.0], ab[1:-1]])
    return alpha_bar


def _mut_c2_sign(orig):
    def ddim_step(x, eps, t, t_prev, ab):
        x = np.asarray(x, dtype=np.float64); eps = np.asarray(eps, dtype=np.float64)
        x0 = (x + np.sqrt(1.0 - ab[t]) * eps) / np.sqrt(ab[t])
        return np.sqrt(ab[t_prev]) * x0 + np.sqrt(1.0 - ab[t_prev]) * eps
    return ddim_step


def _mut_no_clamp(orig):
    return lambda t, stride: int(t) - int(stride)


def _mut_round_truncate(orig):
    def f64_to_bf16_bits(x):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return f64_to_bf16_bits


def _mut_flow_sign(orig):
    def flow_step(x, v, t, t_prev, T, shift=1.0):
        x = np.asarray(x, dtype=np.float64); v = np.asarray(v, dtype=np.float64)
        return x - (S.flow_sigma(t_prev, T, shift) - S.flow_sigma(t, T, shift)) * v
    return flow_step


def _mut_flow_shift_inverted(orig):
    def flow_sigma(t, T, shift=1.0):
        u = float(t) / float(T)
        return u / (shift + (1.0 - shift) * u)
    return flow_sigma


def _mut_queue_same_step_context(orig):
    def plan(n_queue, T, block_tokens, text_len, step, head_id):
        out, stride = orig(n_queue, T, block_tokens, text_len, step, head_id)
        for e in out:
            segs = e["meta"]["segs"]
            if len(segs) == 2:                 # read the neighbour's K/V of this step instead
                segs[0] = (segs[0][0] ^ 1, segs[0][1])
        return out, stride
    return plan


def _mut_queue_single_buffer(orig):
    # one slot per block instead of two: the block entering at the tail takes
    # the slot the head still reads as its context
    def plan(n_queue, T, block_tokens, text_len, step, head_id):
        out, stride = orig(n_queue, T, block_tokens, text_len, step, head_id)
        for e in out:
            k = e["block"]
            e["write_slot"] = k % n_queue
            segs = e["meta"]["segs"]
            segs[-1] = (e["write_slot"], segs[-1][1])
            if len(segs) == 2:
                segs[0] = ((k - 1) % n_queue, segs[0][1])
        return out, stride
    return plan


def _mut_rotation_sign(orig):
    def rotate_pairs(y, table):
        c = np.asarray(table[..., 0])[:, None, :]; s_ = np.asarray(table[..., 1])[:, None, :]
        a, b = y[..., 0::2], y[..., 1::2]
        out = np.empty_like(y)
        out[..., 0::2] = a * c + b * s_
        out[..., 1::2] = a * s_ + b * c
        return out
    return rotate_pairs


def _mut_projection_weight_not_transposed(orig):
    def qkv_project_ref(x_bits, w_bits, heads, head_dim, table=None):
        X = N.bf16_bits_to_f64(x_bits); W = N.bf16_bits_to_f64(w_bits)
        Y = X @ W.reshape(W.shape[1], W.shape[0]) if W.shape[0] != W.shape[1] else X @ W
        L, HD = X.shape[0], heads * head_dim
        return tuple(Y[:, j * HD:(j + 1) * HD].reshape(L, heads, head_dim) for j in range(3))
    return qkv_project_ref


def _mut_merge_weights_swapped(orig):
    def merge_partials(o1, lse1, o2, lse2):
        l1, l2 = np.asarray(lse1, np.float64), np.asarray(lse2, np.float64)
        with np.errstate(invalid="ignore"):
            lse = np.logaddexp(l1, l2)
            return np.exp(l2 - lse)[..., None] * o1 + np.exp(l1 - lse)[..., None] * o2, lse
    return merge_partials


def _mut_split_text_keeps_cache(orig):
    def split_text_attention_ref(q, ring, text_ring, metas, scale=None, heads=None, rows=None):
        self_m = [dict(m, text_len=0) for m in metas]
        return (A.block_attention_ref(q, ring, text_ring, self_m, scale, heads, rows),
                A.block_attention_ref(q, ring, text_ring, metas, scale, heads, rows))
    return split_text_attention_ref


def _mut_noise_sattolo(orig):
    def assign(seed, block_id, pool_frames, n_exclude, block_frames):
        m = pool_frames - n_exclude
        g = NZ.block_generator(seed, block_id)
        a = list(range(m))
        for i in range(block_frames):
            if i + 1 < m:
                j = i + 1 + g.below(m - i - 1)
                a[i], a[j] = a[j], a[i]
        return a[:block_frames]
    return assign


def _mut_noise_no_exclusion(orig):
    def assign(seed, block_id, pool_frames, n_exclude, block_frames):
        return orig(seed, block_id, pool_frames, 0, block_frames)
    return assign


def _mut_noise_biased_below(orig):
    def below(self, n):
        return self.next() % n
    return below


def _mut_noise_gather_transposed(orig):
    def noise_block_ref(pool, channels, pool_frames, frames):
        p = np.asarray(pool).reshape(pool_frames, channels, -1)
        return np.stack([np.stack([p[f, c] for f in frames]) for c in range(channels)])
    return noise_block_ref


MUTATIONS = [
    (A, "key_set", _mut_drop_text),
    (A, "key_set", _mut_seg_off_by_one),
    (A, "key_set", _mut_values_are_keys),
    (A, "block_attention_ref", _mut_scale),
    (A, "softmax_attention", _mut_softmax_axis),
    (A, "softmax_attention", _mut_lse_no_max),
    (R, "RingModel", _mut_ring_v_not_transposed),
    (R, "RingModel", _mut_ring_fifo),
    (S, "alpha_bar", _mut_abar_index),
    (S, "ddim_step", _mut_c2_sign),
    (S, "prev_timestep", _mut_no_clamp),
    (N, "f64_to_bf16_bits", _mut_round_truncate),
    (S, "flow_step", _mut_flow_sign),
    (S, "flow_sigma", _mut_flow_shift_inverted),
    (Q, "plan", _mut_queue_same_step_context),
    (Q, "plan", _mut_queue_single_buffer),
    (P, "rotate_pairs", _mut_rotation_sign),
    (P, "qkv_project_ref", _mut_projection_weight_not_transposed),
    (A, "merge_partials", _mut_merge_weights_swapped),
    (A, "split_text_attention_ref", _mut_split_text_keeps_cache),
    (NZ, "assign", _mut_noise_sattolo),
    (NZ, "assign", _mut_noise_no_exclusion),
    (NZ.SplitMix64, "below", _mut_noise_biased_below),
    (NZ, "noise_block_ref", _mut_noise_gather_transposed),
]


@pytest.mark.parametrize("mod,name,mut", MUTATIONS, ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, mod, name, mut):
    monkeypatch.setattr(mod, name, mut(getattr(mod, name)))
    if mod is N:   # rounding is also imported by name into the schedule module
        monkeypatch.setattr(S, name, getattr(N, name))
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001  (a crash counts as caught, too)
            failed.append(pin.__name__)
    assert failed, f"planted mistake {mut.__name__} passed every pin"
