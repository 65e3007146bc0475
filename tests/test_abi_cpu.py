"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, sizes rings like the oracle's model,
computes the update coefficients like the oracle, and rejects bad arguments
before it would enqueue anything.  No call here reaches a kernel launch."""
import ctypes
import json
import math
import os

import numpy as np
import pytest

import block_wise_long_amd as B
from oracle import queue as oqueue
from oracle import ring as oring
from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FAKE = 0x7F0000000000        # 256-byte aligned dummy device address, never dereferenced


def test_exports_every_declared_symbol():
    names = B.header_symbols()
    assert len(names) == 25
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert B.ba_version() == 10400


@pytest.mark.parametrize("shape", [(2, 5400, 24, 64), (16, 5400, 24, 64), (2, 7800, 40, 128), (1, 226, 24, 64),
                                   (3, 1, 1, 64), (5, 65, 3, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_bytes_match_model(shape, dtype):
    code = B.BA_BF16 if dtype == "bf16" else B.BA_F32
    assert B.ba_ring_bytes(*shape, code) == oring.RingModel(*shape, dtype).nbytes()


def test_ring_bytes_rejects():
    assert B.ba_ring_bytes(0, 10, 1, 64, 0) == 0
    assert B.ba_ring_bytes(1, 10, 1, 96, 0) == 0
    assert B.ba_ring_bytes(1, 10, 1, 64, 7) == 0


def test_schedule_coefficients_match_oracle_golden():
    with open(os.path.join(GOLDEN, "ddim_coefficients.json")) as f:
        g = json.load(f)
    ts = [r["t"] for r in g["coefficients"]]
    c1, c2 = B.ba_schedule_coefficients(ts)
    for r, a, b in zip(g["coefficients"], c1, c2):
        assert a == np.float32(r["c1"]), (r["t"], a, r["c1"])
        assert abs(b - np.float32(r["c2"])) <= abs(np.spacing(np.float32(r["c2"]))), (r["t"], b, r["c2"])


def test_schedule_coefficients_custom_schedule():
    sched = {"T": 50, "stride": 3, "beta_start": 1e-3, "beta_end": 0.05}
    ab = S.alpha_bar(50, 1e-3, 0.05)
    ts = list(range(0, 51))
    c1, c2 = B.ba_schedule_coefficients(ts, sched)
    for t, a, b in zip(ts, c1, c2):
        e1, e2 = S.ddim_coefficients(t, S.prev_timestep(t, 3), ab)
        assert abs(a - e1) <= 1e-6 * abs(e1) and abs(b - e2) <= 1e-6 * abs(e2) + 1e-7


@pytest.mark.parametrize("shift", [1.0, 3.0, 5.0])
def test_flow_coefficients_match_oracle(shift):
    sched = {"kind": "flow", "T": 1000, "stride": 20, "shift": shift}
    ts = [0, 1, 7, 20, 143, 500, 999, 1000]
    c1, c2 = B.ba_schedule_coefficients(ts, sched)
    for t, a, b in zip(ts, c1, c2):
        e1, e2 = S.flow_coefficients(t, S.prev_timestep(t, 20), 1000, shift)
        assert a == 1.0 and e1 == 1.0
        assert b == np.float32(e2), (t, b, e2)     # fp64 on the host, one rounding


def test_flow_schedule_rejects():
    t = (ctypes.c_int32 * 1)(10)
    c = (ctypes.c_float * 1)()
    for shift in (0.0, -1.0, float("nan"), 2e6):
        bad = B.ba_schedule(1000, 20, 0.0, 0.0, B.BA_SCHED_FLOW, shift)
        assert B.raw.ba_schedule_coefficients(ctypes.byref(bad), t, 1, c, c) == B.BA_ERR_OUT_OF_RANGE
    bad = B.ba_schedule(1000, 20, 1e-4, 0.02, 7, 1.0)
    assert B.raw.ba_schedule_coefficients(ctypes.byref(bad), t, 1, c, c) == B.BA_ERR_INVALID_ARG
    ok = B.ba_schedule(1000, 20, 0.0, 0.0, B.BA_SCHED_FLOW, 1.0)     # betas unused by flow
    assert B.raw.ba_schedule_coefficients(ctypes.byref(ok), t, 1, c, c) == B.BA_OK


def _status(fn, *args):
    return fn(*args)


def test_schedule_rejects():
    t = (ctypes.c_int32 * 1)(1001)
    c = (ctypes.c_float * 1)()
    assert B.raw.ba_schedule_coefficients(None, t, 1, c, c) == B.BA_ERR_OUT_OF_RANGE
    assert "1001" in B.ba_last_error()
    bad = B.ba_schedule(1, 20, 1e-4, 0.02)
    assert B.raw.ba_schedule_coefficients(ctypes.byref(bad), t, 0, c, c) == B.BA_ERR_OUT_OF_RANGE
    bad = B.ba_schedule(100, 20, 0.5, 0.1)
    assert B.raw.ba_schedule_coefficients(ctypes.byref(bad), t, 0, c, c) == B.BA_ERR_OUT_OF_RANGE
    bad = B.ba_schedule(100, -1, 1e-4, 0.02)
    assert B.raw.ba_schedule_coefficients(ctypes.byref(bad), t, 0, c, c) == B.BA_ERR_OUT_OF_RANGE


def _ring(n_slots=2, slot_tokens=100, heads=2, head_dim=64, dtype=0):
    r = B.ba_ring()
    r.base = FAKE
    r.n_slots, r.slot_tokens, r.heads, r.head_dim, r.dtype = n_slots, slot_tokens, heads, head_dim, dtype
    r.slot_stride_tokens = -(-slot_tokens // 64) * 64
    r.appended = 5
    return r


def test_ring_init_rejects():
    r = B.ba_ring()
    f = B.raw.ba_ring_init
    assert f(None, FAKE, 1 << 30, 2, 10, 1, 64, 0, None) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(r), None, 1 << 30, 2, 10, 1, 64, 0, None) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(r), FAKE + 16, 1 << 30, 2, 10, 1, 64, 0, None) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(r), FAKE, 10, 2, 10, 1, 64, 0, None) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(r), FAKE, 1 << 30, 2, 10, 1, 80, 0, None) == B.BA_ERR_UNSUPPORTED
    assert f(ctypes.byref(r), FAKE, 1 << 30, 2, 10, 1, 64, 3, None) == B.BA_ERR_UNSUPPORTED
    assert r.base is None and r.n_slots == 0      # untouched on failure


def test_append_rejects_and_leaves_ring():
    r = _ring()
    slot = ctypes.c_int32(-7)
    f = B.raw.ba_cache_append
    assert f(ctypes.byref(r), FAKE, FAKE, 101, ctypes.byref(slot), None) == B.BA_ERR_OUT_OF_RANGE
    assert f(ctypes.byref(r), FAKE, FAKE, 0, ctypes.byref(slot), None) == B.BA_ERR_OUT_OF_RANGE
    assert f(ctypes.byref(r), None, FAKE, 10, ctypes.byref(slot), None) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(r), FAKE + 8, FAKE, 10, ctypes.byref(slot), None) == B.BA_ERR_INVALID_ARG
    r2 = _ring(); r2.slot_stride_tokens = 100     # not from ba_ring_init
    assert f(ctypes.byref(r2), FAKE, FAKE, 10, ctypes.byref(slot), None) == B.BA_ERR_INVALID_ARG
    assert r.appended == 5 and slot.value == -7
    fb = B.raw.ba_cache_append_batched
    slots = (ctypes.c_int32 * 3)(0, 1, 0)
    assert fb(ctypes.byref(r), FAKE, FAKE, 10, slots, 3, None) == B.BA_ERR_INVALID_ARG   # slot twice
    slots = (ctypes.c_int32 * 2)(0, 2)
    assert fb(ctypes.byref(r), FAKE, FAKE, 10, slots, 2, None) == B.BA_ERR_OUT_OF_RANGE
    assert fb(ctypes.byref(r), FAKE, FAKE, 10, None, 2, None) == B.BA_ERR_INVALID_ARG


def _meta(q_len=10, segs=((0, 50),), text_slot=0, text_len=0):
    return B.make_meta(q_len, list(segs), text_slot, text_len)


def _attn(cache, text, metas, q=FAKE, out=FAKE, q_stride=16, scale=0.0, lse=None, ws=None, ws_bytes=0):
    arr = (B.ba_block_meta * len(metas))(*metas)
    return B.raw.ba_block_attention(q, q_stride, ctypes.byref(cache) if cache is not None else None,
                                    ctypes.byref(text) if text is not None else None,
                                    arr, len(metas), scale, out, lse, ws, ws_bytes, None)


def test_attention_rejects():
    c, t = _ring(), _ring(1, 30)
    assert _attn(None, None, [_meta()]) == B.BA_ERR_INVALID_ARG
    assert _attn(c, None, [_meta(segs=((2, 5),))]) == B.BA_ERR_OUT_OF_RANGE          # slot
    assert _attn(c, None, [_meta(segs=((1, 101),))]) == B.BA_ERR_OUT_OF_RANGE        # len > slot_tokens
    assert _attn(c, None, [_meta(segs=((1, -1),))]) == B.BA_ERR_OUT_OF_RANGE
    assert _attn(c, None, [_meta(q_len=17)]) == B.BA_ERR_OUT_OF_RANGE                # q_len > q_stride
    assert _attn(c, None, [_meta(text_len=3)]) == B.BA_ERR_INVALID_ARG               # text missing
    assert _attn(c, t, [_meta(text_len=31)]) == B.BA_ERR_OUT_OF_RANGE
    assert _attn(c, t, [_meta(text_len=3, text_slot=1)]) == B.BA_ERR_OUT_OF_RANGE
    assert _attn(c, None, [_meta(segs=((0, 0),))]) == B.BA_ERR_INVALID_ARG           # queries, no keys
    assert _attn(c, None, [_meta()], q=FAKE + 2) == B.BA_ERR_INVALID_ARG
    assert _attn(c, None, [_meta()], out=None) == B.BA_ERR_INVALID_ARG
    assert _attn(c, None, [_meta()], scale=float("nan")) == B.BA_ERR_INVALID_ARG
    assert _attn(c, _ring(1, 30, heads=3), [_meta(text_len=2)]) == B.BA_ERR_INVALID_ARG
    m = _meta(); m.n_segs = 9
    assert _attn(c, None, [m]) == B.BA_ERR_OUT_OF_RANGE
    c2 = _ring(head_dim=96)
    assert _attn(c2, None, [_meta()]) == B.BA_ERR_UNSUPPORTED
    assert "head_dim" in B.ba_last_error()
    assert _attn(c, None, [_meta()], ws=FAKE + 64, ws_bytes=1 << 20) == B.BA_ERR_INVALID_ARG
    assert "workspace" in B.ba_last_error()


def test_text_arrays_reject_before_any_launch():
    # the text K/V as [heads][text_cap][head_dim] arrays: the copy into a
    # text ring and the attention call that makes that ring in its workspace
    f = B.raw.ba_text_ring_set
    t = _ring(1, 100)
    tr = ctypes.byref(t)
    assert f(tr, 0, None, FAKE, 120, 50, None) == B.BA_ERR_INVALID_ARG
    assert f(tr, 0, FAKE, FAKE + 8, 120, 50, None) == B.BA_ERR_INVALID_ARG
    assert f(tr, 1, FAKE, FAKE, 120, 50, None) == B.BA_ERR_OUT_OF_RANGE      # slot
    assert f(tr, 0, FAKE, FAKE, 120, 0, None) == B.BA_ERR_OUT_OF_RANGE       # text_len
    assert f(tr, 0, FAKE, FAKE, 40, 50, None) == B.BA_ERR_OUT_OF_RANGE       # text_len > text_cap
    assert f(tr, 0, FAKE, FAKE, 120, 101, None) == B.BA_ERR_OUT_OF_RANGE     # text_len > slot_tokens
    assert f(tr, 0, FAKE, FAKE, 0, 1, None) == B.BA_ERR_OUT_OF_RANGE         # text_cap
    bad = _ring(1, 100); bad.slot_stride_tokens = 100
    assert f(ctypes.byref(bad), 0, FAKE, FAKE, 120, 50, None) == B.BA_ERR_INVALID_ARG

    c = _ring()
    cap = 30
    ring_bytes = -(-B.ba_ring_bytes(1, cap, 2, 64, B.BA_BF16) // 256) * 256
    assert B.ba_attention_text_arrays_workspace_bytes(64, B.BA_BF16, 1, 16, 2, cap) == \
        ring_bytes + B.ba_attention_workspace_bytes(64, B.BA_BF16, 1, 16, 2)
    assert B.ba_attention_text_arrays_workspace_bytes(96, B.BA_BF16, 1, 16, 2, cap) == 0
    assert B.ba_attention_text_arrays_workspace_bytes(64, B.BA_BF16, 1, 16, 2, 0) == 0

    def attn(metas, tk=FAKE, tv=FAKE, text_cap=cap, ws=FAKE, ws_bytes=ring_bytes, q=FAKE):
        arr = (B.ba_block_meta * len(metas))(*metas)
        return B.raw.ba_block_attention_text_arrays(q, 16, ctypes.byref(c), tk, tv, text_cap, arr, len(metas), 0.0,
                                                    FAKE, None, ws, ws_bytes, None)
    assert attn([_meta(text_len=3)], tk=None) == B.BA_ERR_INVALID_ARG
    assert attn([_meta(text_len=3)], tv=FAKE + 8) == B.BA_ERR_INVALID_ARG
    assert attn([_meta(text_len=3)], ws=None, ws_bytes=0) == B.BA_ERR_INVALID_ARG
    assert "text ring" in B.ba_last_error()
    assert attn([_meta(text_len=3)], ws_bytes=ring_bytes - 1) == B.BA_ERR_INVALID_ARG
    assert attn([_meta(text_len=3)], ws=FAKE + 64) == B.BA_ERR_INVALID_ARG               # alignment
    assert attn([_meta(text_len=cap + 1)]) == B.BA_ERR_OUT_OF_RANGE                       # text_len > text_cap
    assert attn([_meta(text_len=3, text_slot=1)]) == B.BA_ERR_OUT_OF_RANGE
    assert attn([_meta(text_len=3)], text_cap=0) == B.BA_ERR_OUT_OF_RANGE
    assert attn([_meta(text_len=3), _meta(segs=((2, 5),))]) == B.BA_ERR_OUT_OF_RANGE     # a cache slot
    assert attn([_meta(text_len=3)], q=FAKE + 2) == B.BA_ERR_INVALID_ARG
    # no block reads text: the arrays may be absent, the plain call's checks apply
    assert attn([_meta(segs=((2, 5),))], tk=None, tv=None, ws=None, ws_bytes=0) == B.BA_ERR_OUT_OF_RANGE


def test_static_attention_rejects_before_any_device_work():
    c = _ring()
    f = B.raw.ba_block_attention_static

    def call(q=FAKE, out=FAKE, lse=None):
        arr = (B.ba_block_meta * 1)(_meta())
        return f(q, 16, ctypes.byref(c), None, arr, 1, 0.0, out, lse, None)
    assert call(q=None) == B.BA_ERR_INVALID_ARG
    assert call(out=None) == B.BA_ERR_INVALID_ARG
    assert call(q=FAKE + 8) == B.BA_ERR_INVALID_ARG
    assert call(lse=FAKE + 2) == B.BA_ERR_INVALID_ARG
    arr = (B.ba_block_meta * 1)(_meta())
    assert f(FAKE, 16, None, None, arr, 1, 0.0, FAKE, None, None) == B.BA_ERR_INVALID_ARG


def test_attention_plan_on_the_host():
    # no workspace: whole query tiles, decided without a device; the same
    # argument checks as the attention call
    c, t = _ring(), _ring(1, 30)
    tail = ctypes.c_int32(-1)

    def plan(cache, text, metas, q_stride=16, ws_bytes=0, out=ctypes.byref(tail)):
        arr = (B.ba_block_meta * len(metas))(*metas)
        return B.raw.ba_attention_plan(q_stride, ctypes.byref(cache) if cache is not None else None,
                                       ctypes.byref(text) if text is not None else None,
                                       arr, len(metas), ws_bytes, out)
    assert plan(c, t, [_meta(text_len=3)]) == B.BA_OK and tail.value == 0
    assert plan(c, None, [_meta(segs=((2, 5),))]) == B.BA_ERR_OUT_OF_RANGE
    assert plan(c, None, [_meta(text_len=3)]) == B.BA_ERR_INVALID_ARG
    assert plan(None, None, [_meta()]) == B.BA_ERR_INVALID_ARG
    assert plan(c, None, [_meta()], q_stride=0) == B.BA_ERR_INVALID_ARG
    assert plan(c, None, [_meta()], out=None) == B.BA_ERR_INVALID_ARG


def test_attention_rejects_ring_strides_past_32bit_copy_offsets():
    # the bf16 kernel addresses a lane's V^T chunk by a 32-bit byte offset
    # below 2 * 32 * slot stride: strides from 2^26 tokens on are refused
    # before anything is planned or launched; the fp32 kernel has no such limit
    tail = ctypes.c_int32(-1)

    def plan(cache, text, metas):
        arr = (B.ba_block_meta * len(metas))(*metas)
        return B.raw.ba_attention_plan(16, ctypes.byref(cache), ctypes.byref(text) if text is not None else None,
                                       arr, len(metas), 0, ctypes.byref(tail))
    lim = 1 << 26
    assert plan(_ring(slot_tokens=lim - 64), None, [_meta()]) == B.BA_OK
    assert plan(_ring(slot_tokens=lim - 63), None, [_meta()]) == B.BA_ERR_OUT_OF_RANGE
    assert "stride" in B.ba_last_error()
    assert plan(_ring(slot_tokens=lim), None, [_meta()]) == B.BA_ERR_OUT_OF_RANGE
    assert plan(_ring(), _ring(1, lim - 63), [_meta(text_len=3)]) == B.BA_ERR_OUT_OF_RANGE
    assert plan(_ring(), _ring(1, lim - 64), [_meta(text_len=3)]) == B.BA_OK
    assert plan(_ring(slot_tokens=lim, dtype=B.BA_F32), None, [_meta()]) == B.BA_OK
    assert _attn(_ring(slot_tokens=lim), None, [_meta()]) == B.BA_ERR_OUT_OF_RANGE


def test_workspace_bytes_without_device():
    # fp32 never uses one; with no device to size the grid, none is asked for
    # query tiles: whole waves of 32 queries (bf16), 64 (fp32); 0 when unsupported
    for d in (64, 128):
        for keys in (0, 1, 512, 513, 3072, 3073, 11026, 1 << 20):
            t = B.ba_attention_query_tile(d, B.BA_BF16, keys)
            # head dim 64 with at most 8 tiles of keys: the resident shape's 32-query units
            assert t == 32 if (d == 64 and keys <= 512) else (t % 32 == 0 and t >= 128)
            assert B.ba_attention_query_tile(d, B.BA_F32, keys) == 64
    # head dim 64: the narrow shape for short key sets, the wide one above 3072 keys
    assert B.ba_attention_query_tile(64, B.BA_BF16, 513) == B.ba_attention_query_tile(64, B.BA_BF16, 3072)
    assert B.ba_attention_query_tile(64, B.BA_BF16, 3072) < B.ba_attention_query_tile(64, B.BA_BF16, 3073)
    assert B.ba_attention_query_tile(128, B.BA_BF16, 3072) == B.ba_attention_query_tile(128, B.BA_BF16, 3073)
    assert B.ba_attention_query_tile(96, B.BA_BF16, 64) == 0 and B.ba_attention_query_tile(64, 7, 64) == 0
    assert B.ba_attention_query_tile(64, B.BA_BF16, -1) == 0
    assert B.ba_attention_workspace_bytes(64, B.BA_F32, 1, 128, 2) == 0
    assert B.ba_attention_workspace_bytes(96, B.BA_BF16, 1, 128, 2) == 0
    assert B.ba_attention_workspace_bytes(64, B.BA_BF16, 0, 128, 2) == 0


def test_update_rejects():
    t = (ctypes.c_int32 * 2)(10, 2000)
    f = B.raw.ba_block_update
    assert f(FAKE, FAKE, 100, t, 2, None, None) == B.BA_ERR_OUT_OF_RANGE
    t = (ctypes.c_int32 * 2)(10, -1)
    assert f(FAKE, FAKE, 100, t, 2, None, None) == B.BA_ERR_OUT_OF_RANGE
    t = (ctypes.c_int32 * 2)(10, 20)
    assert f(None, FAKE, 100, t, 2, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE + 2, FAKE, 100, t, 2, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, -1, t, 2, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 100, None, 2, None, None) == B.BA_ERR_INVALID_ARG
    # one thread per 8 elements must stay within the launch limits
    assert f(FAKE, FAKE, (1 << 40) + 8, t, 2, None, None) == B.BA_ERR_OUT_OF_RANGE


def test_status_strings():
    for s in range(5):
        assert B.ba_status_string(s).startswith("BA_")
    assert B.ba_status_string(99) == "BA_ERR_UNKNOWN"


@pytest.mark.parametrize("n,T,L,text", [(1, 10, 5, 0), (3, 30, 100, 16), (8, 1000, 5400, 226), (5, 1000, 64, 1)])
def test_queue_plan_matches_oracle(n, T, L, text):
    q = B.ba_queue_init(n, T, L, text)
    assert B.ba_queue_ring_slots(n) == 2 * n
    for g in range(3 * n + 4):
        slots, metas, t, stride = B.ba_queue_plan(q)
        ref, rstride = oqueue.plan(n, T, L, text, g, g)
        assert stride == rstride
        for m in range(n):
            assert slots[m] == ref[m]["write_slot"] and t[m] == ref[m]["t"]
            mt = metas[m]
            segs = [(mt.seg[j].slot, mt.seg[j].len) for j in range(mt.n_segs)]
            r = ref[m]["meta"]
            assert (mt.q_len, segs, mt.text_slot, mt.text_len) == (r["q_len"], r["segs"], r["text_slot"],
                                                                   r["text_len"])
        B.ba_queue_advance(q)
        assert q.step == g + 1 and q.head_id == g + 1


def test_queue_rejects():
    q = B.ba_queue()
    f = B.raw.ba_queue_init
    assert f(None, 3, 30, 10, 0) == B.BA_ERR_INVALID_ARG
    assert f(ctypes.byref(q), 0, 30, 10, 0) == B.BA_ERR_OUT_OF_RANGE
    assert f(ctypes.byref(q), 4, 30, 10, 0) == B.BA_ERR_OUT_OF_RANGE      # T not a multiple
    assert f(ctypes.byref(q), 3, 30, 0, 0) == B.BA_ERR_OUT_OF_RANGE
    assert f(ctypes.byref(q), 3, 30, 10, -1) == B.BA_ERR_OUT_OF_RANGE
    assert B.ba_queue_ring_slots(0) == 0 and B.ba_queue_ring_slots(B.BA_QUEUE_MAX + 1) == 0
    bad = B.ba_queue()                                                 # never initialised
    s = (ctypes.c_int32 * 1)()
    m = (B.ba_block_meta * 1)()
    st = ctypes.c_int32()
    assert B.raw.ba_queue_plan(ctypes.byref(bad), s, m, s, ctypes.byref(st)) == B.BA_ERR_INVALID_ARG
    q = B.ba_queue_init(1, 10, 5)
    assert B.raw.ba_queue_plan(ctypes.byref(q), None, m, s, ctypes.byref(st)) == B.BA_ERR_INVALID_ARG
    assert B.raw.ba_queue_advance(None) == B.BA_ERR_INVALID_ARG


def test_project_rejects():
    f = B.raw.ba_qkv_project
    r = _ring(n_slots=2, slot_tokens=100, heads=2, head_dim=64)
    rr = ctypes.byref(r)
    assert f(None, 100, 128, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE, 100, 128, None, FAKE, rr, 1, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE + 2, 100, 128, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_INVALID_ARG
    assert f(FAKE, 100, 128, FAKE, FAKE, rr, 1, FAKE + 4, None) == B.BA_ERR_INVALID_ARG     # rope alignment
    assert f(FAKE, 100, 128, FAKE, FAKE, rr, 2, None, None) == B.BA_ERR_OUT_OF_RANGE        # slot
    assert f(FAKE, 101, 128, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_OUT_OF_RANGE        # n_tokens
    assert f(FAKE, 0, 128, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_OUT_OF_RANGE
    assert f(FAKE, 100, 96, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_OUT_OF_RANGE         # dim % 64
    assert f(FAKE, 100, 0, FAKE, FAKE, rr, 1, None, None) == B.BA_ERR_OUT_OF_RANGE
    r32 = _ring(n_slots=2, slot_tokens=100, heads=2, head_dim=64, dtype=B.BA_F32)
    assert f(FAKE, 100, 128, FAKE, FAKE, ctypes.byref(r32), 1, None, None) == B.BA_ERR_UNSUPPORTED
    g = B.raw.ba_qkv_project_batched
    r4 = ctypes.byref(_ring(n_slots=4, slot_tokens=100, heads=2, head_dim=64))
    sl = (ctypes.c_int32 * 3)(0, 2, 3)
    assert g(FAKE, 0, 100, 128, FAKE, FAKE, r4, sl, None, 0, None) == B.BA_ERR_OUT_OF_RANGE      # n_blocks
    assert g(FAKE, 65, 100, 128, FAKE, FAKE, r4, sl, None, 0, None) == B.BA_ERR_OUT_OF_RANGE
    assert g(FAKE, 3, 100, 128, FAKE, FAKE, r4, None, None, 0, None) == B.BA_ERR_INVALID_ARG     # slots NULL
    dup = (ctypes.c_int32 * 3)(0, 2, 0)
    assert g(FAKE, 3, 100, 128, FAKE, FAKE, r4, dup, None, 0, None) == B.BA_ERR_INVALID_ARG      # shared slot
    bad = (ctypes.c_int32 * 3)(0, 2, 4)
    assert g(FAKE, 3, 100, 128, FAKE, FAKE, r4, bad, None, 0, None) == B.BA_ERR_OUT_OF_RANGE
    assert g(FAKE, 3, 100, 128, FAKE, FAKE, r4, sl, FAKE, 100, None) == B.BA_ERR_INVALID_ARG     # table stride
    assert "rope_block_stride" in B.ba_last_error()


@pytest.mark.parametrize("pool,excl,bf", [(21, 3, 4), (21, 0, 21), (9, 8, 1), (64, 0, 64), (200, 17, 64), (5, 1, 3)])
def test_noise_assign_matches_oracle(pool, excl, bf):
    # the library's host bookkeeping and the oracle, from one published
    # generator definition each: identical frame lists
    from oracle import noise as NZ
    for seed in (0, 1, 20251, 2 ** 64 - 1, 0x0123456789ABCDEF):
        for b in (0, 1, 2, 7, 40, 999):
            assert B.ba_noise_assign(seed, b, pool, excl, bf) == NZ.assign(seed, b, pool, excl, bf)


def test_noise_rejects():
    f = B.raw.ba_noise_assign
    out = (ctypes.c_int32 * 64)()
    assert f(0, 0, 10, 3, 8, out) == B.BA_ERR_OUT_OF_RANGE         # more frames than candidates
    assert f(0, 0, 10, 10, 1, out) == B.BA_ERR_OUT_OF_RANGE        # no candidates
    assert f(0, -1, 10, 0, 1, out) == B.BA_ERR_OUT_OF_RANGE
    assert f(0, 0, 100, 0, 65, out) == B.BA_ERR_OUT_OF_RANGE       # kernarg table
    assert f(0, 0, 10, 0, 0, out) == B.BA_ERR_OUT_OF_RANGE
    assert f(0, 0, 10, 0, 1, None) == B.BA_ERR_INVALID_ARG
    g = B.raw.ba_noise_block
    fr = (ctypes.c_int32 * 2)(0, 3)
    big = FAKE + (1 << 30)
    assert g(FAKE, 2, 3, 64, fr, 2, big, None) == B.BA_ERR_OUT_OF_RANGE        # frame 3 >= pool_frames
    assert g(FAKE, 2, 4, 40, fr, 2, big, None) == B.BA_ERR_INVALID_ARG         # frame bytes
    assert g(FAKE + 8, 2, 4, 64, fr, 2, big, None) == B.BA_ERR_INVALID_ARG     # alignment
    assert g(FAKE, 2, 4, 64, fr, 2, FAKE + 64, None) == B.BA_ERR_INVALID_ARG   # overlaps the pool
    assert g(FAKE, 0, 4, 64, fr, 2, big, None) == B.BA_ERR_OUT_OF_RANGE
    assert g(FAKE, 2000, 4, 64, fr, 64, big, None) == B.BA_ERR_OUT_OF_RANGE    # grid rows
    assert g(None, 2, 4, 64, fr, 2, big, None) == B.BA_ERR_INVALID_ARG
