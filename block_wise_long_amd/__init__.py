"""Python binding of libblockattn (argument marshalling only).

Each function has the name of the C entry point it calls (see
include/blockattn.h) and takes torch tensors for device buffers; every step
of the computation runs in the library's HIP kernels.  The stream is torch's
current stream.  There is no fallback: importing this package fails when
libblockattn.so has not been built (python -m block_wise_long_amd.build).
"""
import ctypes
import os
import re

# torch ships its own HIP runtime (libamdhip64.so.7).  Load it first so that
# the library's dependency on that soname resolves to the same copy: two HIP
# runtimes in one process do not share devices, memory or streams.
import torch  # noqa: F401  (load order matters, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblockattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "blockattn.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m block_wise_long_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

BA_OK, BA_ERR_INVALID_ARG, BA_ERR_UNSUPPORTED, BA_ERR_OUT_OF_RANGE, BA_ERR_HIP = range(5)
BA_BF16, BA_F32 = 0, 1
BA_TOKEN_ALIGN = 64
BA_MAX_SEGS = 8


class ba_ring(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("slot_tokens", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("slot_stride_tokens", ctypes.c_int32), ("appended", ctypes.c_int64)]


class ba_seg(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("len", ctypes.c_int32)]


class ba_block_meta(ctypes.Structure):
    _fields_ = [("q_len", ctypes.c_int32), ("n_segs", ctypes.c_int32),
                ("seg", ba_seg * BA_MAX_SEGS), ("text_slot", ctypes.c_int32),
                ("text_len", ctypes.c_int32)]


BA_SCHED_DDIM, BA_SCHED_FLOW = 0, 1
BA_QUEUE_MAX = 4096


class ba_queue(ctypes.Structure):
    _fields_ = [("n_queue", ctypes.c_int32), ("T", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("text_len", ctypes.c_int32), ("step", ctypes.c_int64), ("head_id", ctypes.c_int64)]


class ba_schedule(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("beta_start", ctypes.c_double), ("beta_end", ctypes.c_double),
                ("kind", ctypes.c_int32), ("shift", ctypes.c_double)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "ba_ring_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32]),
    "ba_ring_init": (_I32, [ctypes.POINTER(ba_ring), _P, ctypes.c_size_t, _I32, _I32, _I32, _I32, _I32, _P]),
    "ba_cache_append": (_I32, [ctypes.POINTER(ba_ring), _P, _P, _I32, ctypes.POINTER(_I32), _P]),
    "ba_cache_append_batched": (_I32, [ctypes.POINTER(ba_ring), _P, _P, _I32, ctypes.POINTER(_I32), _I32, _P]),
    "ba_block_attention": (_I32, [_P, _I32, ctypes.POINTER(ba_ring), ctypes.POINTER(ba_ring),
                                  ctypes.POINTER(ba_block_meta), _I32, ctypes.c_float, _P, _P,
                                  _P, ctypes.c_size_t, _P]),
    "ba_block_attention_static": (_I32, [_P, _I32, ctypes.POINTER(ba_ring), ctypes.POINTER(ba_ring),
                                         ctypes.POINTER(ba_block_meta), _I32, ctypes.c_float, _P, _P, _P]),
    "ba_attention_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32]),
    "ba_text_ring_set": (_I32, [ctypes.POINTER(ba_ring), _I32, _P, _P, _I32, _I32, _P]),
    "ba_block_attention_text_arrays": (_I32, [_P, _I32, ctypes.POINTER(ba_ring), _P, _P, _I32,
                                              ctypes.POINTER(ba_block_meta), _I32, ctypes.c_float, _P, _P,
                                              _P, ctypes.c_size_t, _P]),
    "ba_attention_text_arrays_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "ba_attention_query_tile": (_I32, [_I32, _I32, _I32]),
    "ba_attention_plan": (_I32, [_I32, ctypes.POINTER(ba_ring), ctypes.POINTER(ba_ring),
                                 ctypes.POINTER(ba_block_meta), _I32, ctypes.c_size_t, ctypes.POINTER(_I32)]),
    "ba_block_update": (_I32, [_P, _P, _I64, ctypes.POINTER(_I32), _I32, ctypes.POINTER(ba_schedule), _P]),
    "ba_schedule_coefficients": (_I32, [ctypes.POINTER(ba_schedule), ctypes.POINTER(_I32), _I32,
                                        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    "ba_qkv_project": (_I32, [_P, _I32, _I32, _P, _P, ctypes.POINTER(ba_ring), _I32, _P, _P]),
    "ba_qkv_project_batched": (_I32, [_P, _I32, _I32, _I32, _P, _P, ctypes.POINTER(ba_ring), ctypes.POINTER(_I32),
                                      _P, _I64, _P]),
    "ba_queue_init": (_I32, [ctypes.POINTER(ba_queue), _I32, _I32, _I32, _I32]),
    "ba_queue_ring_slots": (_I32, [_I32]),
    "ba_queue_plan": (_I32, [ctypes.POINTER(ba_queue), ctypes.POINTER(_I32), ctypes.POINTER(ba_block_meta),
                             ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "ba_queue_advance": (_I32, [ctypes.POINTER(ba_queue)]),
    "ba_noise_assign": (_I32, [ctypes.c_uint64, _I64, _I32, _I32, _I32, ctypes.POINTER(_I32)]),
    "ba_noise_block": (_I32, [_P, _I32, _I32, _I64, ctypes.POINTER(_I32), _I32, _P, _P]),
    "ba_status_string": (ctypes.c_char_p, [_I32]),
    "ba_last_error": (ctypes.c_char_p, []),
    "ba_version": (_I32, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args
raw = _lib   # the C entry points themselves, for callers that marshal by hand


def header_symbols():
    """Names of the functions include/blockattn.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(ba_\w+)\s*\(", text, re.M)))


class BlockAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.ba_last_error().decode()
        super().__init__(f"{where}: {_lib.ba_status_string(status).decode()}: {msg}")


def _check(status, where):
    if status != BA_OK:
        raise BlockAttnError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):

    if t.dtype == torch.bfloat16:
        return BA_BF16
    if t.dtype == torch.float32:
        return BA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def ba_status_string(status):
    return _lib.ba_status_string(status).decode()


def ba_last_error():
    return _lib.ba_last_error().decode()


def ba_version():
    return _lib.ba_version()


def ba_ring_bytes(n_slots, slot_tokens, heads, head_dim, dtype=BA_BF16):
    return _lib.ba_ring_bytes(n_slots, slot_tokens, heads, head_dim, dtype)


class Ring:
    """A ba_ring descriptor plus the torch buffer that backs it."""

    def __init__(self, desc, buffer):
        self.desc = desc
        self.buffer = buffer

    @property
    def appended(self):
        return self.desc.appended

    @property
    def slot_stride_tokens(self):
        return self.desc.slot_stride_tokens


def ba_ring_init(n_slots, slot_tokens, heads, head_dim, dtype=BA_BF16, device="cuda"):
    """Allocate (via torch) and initialise a zero-filled ring; returns a Ring."""

    nbytes = ba_ring_bytes(n_slots, slot_tokens, heads, head_dim, dtype)
    if nbytes == 0:
        # let the library produce the precise error
        desc = ba_ring()
        _check(_lib.ba_ring_init(ctypes.byref(desc), None, 0, n_slots, slot_tokens, heads,
                                 head_dim, dtype, None), "ba_ring_init")
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    view = buf[off:off + nbytes]
    desc = ba_ring()
    _check(_lib.ba_ring_init(ctypes.byref(desc), ctypes.c_void_p(view.data_ptr()), nbytes, n_slots,
                             slot_tokens, heads, head_dim, dtype, _stream()), "ba_ring_init")
    return Ring(desc, view)


def ba_cache_append(ring, k, v, n_tokens=None):
    """FIFO append of k, v ([n_tokens][heads][head_dim]); returns the slot written."""
    n = k.shape[0] if n_tokens is None else n_tokens
    _shape_check(ring, k, v, n, 1)
    slot = _I32(-1)
    _check(_lib.ba_cache_append(ctypes.byref(ring.desc), _dev(k, "k"), _dev(v, "v"), n,
                                ctypes.byref(slot), _stream()), "ba_cache_append")
    return slot.value


def ba_cache_append_batched(ring, k, v, slots):
    """k, v: [n_blocks][n_tokens][heads][head_dim]; block i -> slots[i]."""
    nb = len(slots)
    n = k.shape[1]
    _shape_check(ring, k, v, n, nb)
    arr = (_I32 * max(nb, 1))(*slots)
    _check(_lib.ba_cache_append_batched(ctypes.byref(ring.desc), _dev(k, "k"), _dev(v, "v"), n,
                                        arr, nb, _stream()), "ba_cache_append_batched")


def _shape_check(ring, k, v, n, nb):
    d = ring.desc
    want = n * d.heads * d.head_dim * nb
    if k.numel() < want or v.numel() < want:
        raise ValueError("k/v smaller than n_blocks * n_tokens * heads * head_dim")
    if _dtype_code(k) != d.dtype or _dtype_code(v) != d.dtype:
        raise TypeError("k/v dtype differs from the ring's")


def make_meta(q_len, segs, text_slot=0, text_len=0):
    """One ba_block_meta from (slot, len) segments."""
    if len(segs) > BA_MAX_SEGS:
        raise ValueError("too many segments")
    m = ba_block_meta()
    m.q_len, m.n_segs, m.text_slot, m.text_len = q_len, len(segs), text_slot, text_len
    for i, (s, n) in enumerate(segs):
        m.seg[i].slot, m.seg[i].len = s, n
    return m


def ba_attention_plan(q_stride, cache, text, metas, workspace_bytes):
    """Tail workgroups per XCD the attention call would use with a workspace
    of workspace_bytes (0: whole query tiles per workgroup); launches nothing."""
    nb = len(metas)
    arr = (ba_block_meta * max(nb, 1))()
    for i, m in enumerate(metas):
        arr[i] = m if isinstance(m, ba_block_meta) else make_meta(
            m["q_len"], m["segs"], m.get("text_slot", 0), m.get("text_len", 0))
    tail = ctypes.c_int32(-1)
    _check(_lib.ba_attention_plan(q_stride, ctypes.byref(cache.desc),
                                  ctypes.byref(text.desc) if text is not None else None,
                                  arr, nb, workspace_bytes, ctypes.byref(tail)), "ba_attention_plan")
    return tail.value


def ba_attention_query_tile(head_dim, dtype, max_keys):
    """Queries of one head per workgroup of ba_block_attention in a launch
    whose longest key set has max_keys keys (0: unsupported)."""
    return _lib.ba_attention_query_tile(head_dim, dtype, max_keys)


def ba_attention_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads):
    return _lib.ba_attention_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads)


_WORKSPACES = {}


def attention_workspace(head_dim, dtype, n_blocks, q_stride, heads, device=None):
    """A workspace for ba_block_attention, cached per (device, stream, size):
    calls on one stream are ordered and may share it, calls on different
    streams get different buffers.  None when none is used."""
    nbytes = ba_attention_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads)
    if nbytes == 0:
        return None
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    key = (dev, torch.cuda.current_stream(dev).cuda_stream, nbytes)
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def ba_block_attention(q, cache, text, metas, scale=0.0, out=None, lse=None, workspace="auto"):
    """q: [n_blocks][q_stride][heads][head_dim]; metas: list of ba_block_meta
    or dicts (q_len, segs, text_slot, text_len).  Returns out (allocated if
    not given); lse, when given, is filled in.  workspace: "auto" (a cached
    one), None (one workgroup per query tile), or a uint8 device tensor."""
    nb, q_stride = q.shape[0], q.shape[1]
    if q.shape[2] != cache.desc.heads or q.shape[3] != cache.desc.head_dim:
        raise ValueError("q shape does not match the cache ring")
    if len(metas) != nb:
        raise ValueError("one meta per block")
    arr = (ba_block_meta * max(nb, 1))()
    for i, m in enumerate(metas):
        arr[i] = m if isinstance(m, ba_block_meta) else make_meta(
            m["q_len"], m["segs"], m.get("text_slot", 0), m.get("text_len", 0))
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() < nb * cache.desc.heads * q_stride):
        raise ValueError("lse must be fp32 [n_blocks][heads][q_stride]")
    if isinstance(workspace, str) and workspace == "auto":
        workspace = attention_workspace(cache.desc.head_dim, cache.desc.dtype, nb, q_stride,
                                        cache.desc.heads, q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(_lib.ba_block_attention(_dev(q, "q"), q_stride, ctypes.byref(cache.desc),
                                   ctypes.byref(text.desc) if text is not None else None,
                                   arr, nb, float(scale), _dev(out, "out"),
                                   _dev(lse, "lse") if lse is not None else None,
                                   ws_ptr, ws_bytes, _stream()),
           "ba_block_attention")
    return out


def ba_text_ring_set(text, text_k, text_v, text_len=None, slot=0):
    """text_k, text_v: [heads][text_cap][head_dim] (head-major) in the ring's
    dtype; tokens [0, text_len) (default: all text_cap) into slot `slot` of
    the ring `text`, zeros after them."""
    if text_k.dim() != 3 or text_k.shape != text_v.shape or text_k.dtype != text_v.dtype:
        raise ValueError("text_k, text_v must be [heads][text_cap][head_dim] of one dtype")
    cap = text_k.shape[1]
    n = cap if text_len is None else int(text_len)
    _check(_lib.ba_text_ring_set(ctypes.byref(text.desc), slot, _dev(text_k, "text_k"), _dev(text_v, "text_v"),
                                 cap, n, _stream()), "ba_text_ring_set")


def ba_attention_text_arrays_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads, text_cap):
    return _lib.ba_attention_text_arrays_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads, text_cap)


def ba_block_attention_text_arrays(q, cache, text_k, text_v, metas, workspace, scale=0.0, out=None, lse=None):
    """ba_block_attention with the text K/V as [heads][text_cap][head_dim]
    arrays (or None when no block reads text); workspace: a uint8 device
    tensor of at least the text ring's bytes
    (ba_attention_text_arrays_workspace_bytes gives the full size)."""
    nb, q_stride = q.shape[0], q.shape[1]
    if q.shape[2] != cache.desc.heads or q.shape[3] != cache.desc.head_dim:
        raise ValueError("q shape does not match the cache ring")
    if len(metas) != nb:
        raise ValueError("one meta per block")
    arr = (ba_block_meta * max(nb, 1))()
    for i, m in enumerate(metas):
        arr[i] = m if isinstance(m, ba_block_meta) else make_meta(
            m["q_len"], m["segs"], m.get("text_slot", 0), m.get("text_len", 0))
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() < nb * cache.desc.heads * q_stride):
        raise ValueError("lse must be fp32 [n_blocks][heads][q_stride]")
    cap = 0
    if text_k is not None:
        if text_k.dim() != 3 or text_v is None or text_k.shape != text_v.shape:
            raise ValueError("text_k, text_v must be [heads][text_cap][head_dim]")
        cap = text_k.shape[1]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(_lib.ba_block_attention_text_arrays(
        _dev(q, "q"), q_stride, ctypes.byref(cache.desc),
        _dev(text_k, "text_k") if text_k is not None else None,
        _dev(text_v, "text_v") if text_v is not None else None, cap,
        arr, nb, float(scale), _dev(out, "out"), _dev(lse, "lse") if lse is not None else None,
        ws_ptr, ws_bytes, _stream()), "ba_block_attention_text_arrays")
    return out


def ba_block_attention_static(q, cache, text, metas, scale=0.0, out=None, lse=None):
    """ba_block_attention without a workspace argument: the library's own
    per-GPU device array holds the split schedule's partial results (calls
    on one GPU must not overlap).  Same arguments and results otherwise."""
    nb, q_stride = q.shape[0], q.shape[1]
    if q.shape[2] != cache.desc.heads or q.shape[3] != cache.desc.head_dim:
        raise ValueError("q shape does not match the cache ring")
    if len(metas) != nb:
        raise ValueError("one meta per block")
    arr = (ba_block_meta * max(nb, 1))()
    for i, m in enumerate(metas):
        arr[i] = m if isinstance(m, ba_block_meta) else make_meta(
            m["q_len"], m["segs"], m.get("text_slot", 0), m.get("text_len", 0))
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() < nb * cache.desc.heads * q_stride):
        raise ValueError("lse must be fp32 [n_blocks][heads][q_stride]")
    _check(_lib.ba_block_attention_static(_dev(q, "q"), q_stride, ctypes.byref(cache.desc),
                                          ctypes.byref(text.desc) if text is not None else None,
                                          arr, nb, float(scale), _dev(out, "out"),
                                          _dev(lse, "lse") if lse is not None else None, _stream()),
           "ba_block_attention_static")
    return out


def _schedule(s):
    if s is None:
        return None
    if isinstance(s, ba_schedule):
        return ctypes.byref(s)
    kind = s.get("kind", BA_SCHED_DDIM)
    if kind in ("ddim", "flow"):
        kind = BA_SCHED_FLOW if kind == "flow" else BA_SCHED_DDIM
    return ctypes.byref(ba_schedule(s.get("T", 1000), s.get("stride", 20),
                                    s.get("beta_start", 1e-4), s.get("beta_end", 0.02),
                                    kind, s.get("shift", 1.0)))


def ba_block_update(x, eps, t_per_block, schedule=None):
    """In place on x ([n_blocks][elems] bf16) with eps of the same shape (the
    predicted velocity for a flow-matching schedule).  schedule: None, a
    ba_schedule, or a dict of its fields (kind "ddim" or "flow")."""
    nb = len(t_per_block)
    if x.shape != eps.shape or x.shape[0] != nb:
        raise ValueError("x, eps must be [n_blocks][elems] with one timestep per block")
    elems = x.numel() // max(nb, 1)
    arr = (_I32 * max(nb, 1))(*[int(t) for t in t_per_block])
    _check(_lib.ba_block_update(_dev(x, "x"), _dev(eps, "eps"), elems, arr, nb, _schedule(schedule),
                                _stream()), "ba_block_update")
    return x


def ba_schedule_coefficients(t, schedule=None):
    """Host-only: the fp32 (c1, c2) lists ba_block_update applies."""
    n = len(t)
    arr = (_I32 * max(n, 1))(*[int(v) for v in t])
    c1 = (ctypes.c_float * max(n, 1))()
    c2 = (ctypes.c_float * max(n, 1))()
    _check(_lib.ba_schedule_coefficients(_schedule(schedule), arr, n, c1, c2), "ba_schedule_coefficients")
    return list(c1)[:n], list(c2)[:n]


# ---- single-GPU FIFO block queue (host bookkeeping in the library) ----------

def ba_queue_init(n_queue, T, block_tokens, text_len=0):
    q = ba_queue()
    _check(_lib.ba_queue_init(ctypes.byref(q), n_queue, T, block_tokens, text_len), "ba_queue_init")
    return q


def ba_queue_ring_slots(n_queue):
    return int(_lib.ba_queue_ring_slots(n_queue))


def ba_queue_plan(q):
    """The next step's plan by latent slot: (write_slots, metas, t, stride)."""
    n = q.n_queue
    slots = (_I32 * n)()
    metas = (ba_block_meta * n)()
    t = (_I32 * n)()
    stride = _I32()
    _check(_lib.ba_queue_plan(ctypes.byref(q), slots, metas, t, ctypes.byref(stride)), "ba_queue_plan")
    return list(slots), list(metas), list(t), int(stride.value)


def ba_queue_advance(q):
    _check(_lib.ba_queue_advance(ctypes.byref(q)), "ba_queue_advance")
    return q


# ---- fused K/V producer -------------------------------------------------------

def ba_qkv_project(x, w, cache, slot, q=None, rope=None):
    """x: [n_tokens][dim] bf16, w: [3 * heads * head_dim][dim] bf16 (a linear
    layer's weight, rows q | k | v); K and V go to ring slot `slot`, Q to q
    ([n_tokens][heads][head_dim] bf16) when given.  rope: optional
    [head_dim / 2][n_tokens][2] fp32 (cos, sin) table for q and k, pair-major."""
    if x.dim() != 2 or w.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError("x must be [n_tokens][dim] and w [3 * heads * head_dim][dim]")
    d = cache.desc
    if w.shape[0] != 3 * d.heads * d.head_dim:
        raise ValueError("w must have 3 * heads * head_dim rows")
    if q is not None and q.numel() < x.shape[0] * d.heads * d.head_dim:
        raise ValueError("q too small")
    if rope is not None and (rope.dtype != torch.float32 or rope.numel() < x.shape[0] * d.head_dim):
        raise ValueError("rope must be fp32 [head_dim / 2][n_tokens][2]")
    _check(_lib.ba_qkv_project(_dev(x, "x"), x.shape[0], x.shape[1], _dev(w, "w"),
                               _dev(q, "q") if q is not None else None, ctypes.byref(d), slot,
                               _dev(rope, "rope") if rope is not None else None, _stream()),
           "ba_qkv_project")


def ba_qkv_project_batched(x, w, cache, slots, q=None, rope=None):
    """x: [n_blocks][n_tokens][dim] bf16; block b's K/V go to ring slot
    slots[b], its Q to q[b] ([n_blocks][n_tokens][heads][head_dim]) when q is
    given.  rope: None, one [head_dim / 2][n_tokens][2] fp32 table for every
    block, or [n_blocks][head_dim / 2][n_tokens][2]."""
    if x.dim() != 3 or w.dim() != 2 or w.shape[1] != x.shape[2] or len(slots) != x.shape[0]:
        raise ValueError("x must be [n_blocks][n_tokens][dim], w [3 * heads * head_dim][dim], one slot per block")
    d = cache.desc
    nb, L = x.shape[0], x.shape[1]
    if w.shape[0] != 3 * d.heads * d.head_dim:
        raise ValueError("w must have 3 * heads * head_dim rows")
    if q is not None and q.numel() < nb * L * d.heads * d.head_dim:
        raise ValueError("q too small")
    stride = 0
    if rope is not None:
        table = L * d.head_dim
        if rope.dtype != torch.float32 or rope.numel() not in (table, nb * table):
            raise ValueError("rope must be fp32 [head_dim / 2][n_tokens][2] or [n_blocks][...]")
        stride = table if rope.numel() == nb * table and nb > 1 else 0
    arr = (_I32 * nb)(*slots)
    _check(_lib.ba_qkv_project_batched(_dev(x, "x"), nb, L, x.shape[2], _dev(w, "w"),
                                       _dev(q, "q") if q is not None else None, ctypes.byref(d), arr,
                                       _dev(rope, "rope") if rope is not None else None, stride, _stream()),
           "ba_qkv_project_batched")


BA_NOISE_MAX_FRAMES = 64


def ba_noise_assign(seed, block_id, pool_frames, n_exclude, block_frames):
    """Pool frames (a list of ints) block block_id takes; host only."""
    arr = (_I32 * max(block_frames, 1))()
    _check(_lib.ba_noise_assign(seed & (2 ** 64 - 1), block_id, pool_frames, n_exclude, block_frames, arr),
           "ba_noise_assign")
    return list(arr[:block_frames])


def ba_noise_block(pool, frames, out):
    """pool: [channels][pool_frames][...] device tensor; out: [channels]
    [len(frames)][...] of the same element type and frame size."""
    if pool.dim() < 3 or out.dim() < 3 or pool.shape[0] != out.shape[0] or out.shape[1] != len(frames) \
            or pool.shape[2:] != out.shape[2:] or pool.dtype != out.dtype:
        raise ValueError("pool [C][F_pool][...] and out [C][len(frames)][...] must match")
    if not (pool.is_contiguous() and out.is_contiguous()):
        raise ValueError("pool and out must be contiguous")
    frame_bytes = pool[0, 0].numel() * pool.element_size()
    arr = (_I32 * max(len(frames), 1))(*frames)
    _check(_lib.ba_noise_block(_dev(pool, "pool"), pool.shape[0], pool.shape[1], frame_bytes, arr, len(frames),
                               _dev(out, "out"), _stream()), "ba_noise_block")
    return out
