"""Block attention over the [cached segments | text] key set, fp64 (oracle).

What is computed (restated from the sources named in the package header):
  * Key set.  The queries of one temporal block attend over the cached
    self-attention K/V of the neighbouring, already processed block and the
    block's own K/V ("Minute-Long Videos with Dual Parallelisms", Abstract:
    features of the prior block are stored and reused as context; pith.science
    verdict, pith_extraction.core_discovery: the per-GPU cache holds the
    neighbouring block's self-attention K/V), followed by the text-conditioning
    K/V.  Each block names its cache segments (ring slot, token count) in key
    order; the text segment comes last.  Only valid keys take part: tokens past
    a segment's length and text past text_len are not keys (the only mask).
  * Scores s_ij = scale * <q_i, k_j>, scale = 1/sqrt(head_dim) unless given.
  * Weights p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij).
  * Output o_i = sum_j p_ij v_j; log-sum-exp lse_i = max_j s_ij + ln sum_j exp(s_ij - max_j s_ij).
  ("Attention Is All You Need", scaled dot-product attention, applied per head.)
"""
import math

import numpy as np


def softmax_attention(q, k, v, scale, chunk=256):
    """q [n, D], k [L, D], v [L, Dv] (fp64) -> (o [n, Dv], lse [n]).

    BLAS dgemm is used for the two products; rows are processed in chunks
    only to bound memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for a in range(0, n, chunk):
        s = scale * (q[a:a + chunk] @ k.T)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        z = e.sum(axis=1)
        o[a:a + chunk] = (e @ v) / z[:, None]
        lse[a:a + chunk] = m + np.log(z)
    return o, lse


def key_set(ring, text_ring, meta, head):
    """Concatenate the block's key/value segments in key order for one head.

    meta: dict with ``segs`` [(slot, len), ...] (cache segments in key order),
    ``text_slot`` and ``text_len``.
    """
    ks, vs = [], []
    for slot, n in meta["segs"]:
        if n:
            ks.append(ring.keys(slot, head, n))
            vs.append(ring.values(slot, head, n))
    if meta.get("text_len", 0):
        ks.append(text_ring.keys(meta.get("text_slot", 0), head, meta["text_len"]))
        vs.append(text_ring.values(meta.get("text_slot", 0), head, meta["text_len"]))
    return np.concatenate(ks), np.concatenate(vs)


def block_attention_ref(q, ring, text_ring, metas, scale=None, heads=None, rows=None):
    """Oracle for one batched call.

    q: [n_blocks][q_stride][heads][head_dim] fp64 (decoded device values).
    metas: one dict per block (``q_len``, ``segs``, ``text_slot``, ``text_len``).
    heads / rows: optional subsets (rows is a list of query indices applied to
    every block) so that large workloads can be checked on sampled outputs.
    Returns (out, lse): out has q's shape, lse is [n_blocks][heads][q_stride];
    entries that were not computed are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    nb, qs, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.full(q.shape, np.nan)
    lse = np.full((nb, H, qs), np.nan)
    heads = range(H) if heads is None else heads
    for b, meta in enumerate(metas):
        r = np.arange(meta["q_len"]) if rows is None else np.asarray(
            [i for i in rows if i < meta["q_len"]], dtype=np.int64)
        for h in heads:
            K, V = key_set(ring, text_ring, meta, h)
            o, l = softmax_attention(q[b, r, h, :], K, V, scale)
            out[b, r, h, :] = o
            lse[b, h, r] = l
    return out, lse


def merge_partials(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint key sets, from each part's
    normalised output o [..., Dv] and log-sum-exp lse [...]: a key's weight in
    the union is its weight in its part times exp(lse_part - lse_union), with
    lse_union = log(exp(lse1) + exp(lse2)).  fp64."""
    o1, o2 = np.asarray(o1, np.float64), np.asarray(o2, np.float64)
    l1, l2 = np.asarray(lse1, np.float64), np.asarray(lse2, np.float64)
    with np.errstate(invalid="ignore"):             # rows not computed stay NaN
        lse = np.logaddexp(l1, l2)
        w1 = np.exp(l1 - lse)[..., None]
        w2 = np.exp(l2 - lse)[..., None]
    return w1 * o1 + w2 * o2, lse


def split_text_attention_ref(q, ring, text_ring, metas, scale=None, heads=None, rows=None):
    """Separate text cross-attention (Wan-style, the alternative to the joint
    key set): the cache segments form one softmax (self-attention), the text
    keys another (cross-attention), each normalised on its own.  Returns
    ((o_self, lse_self), (o_text, lse_text)) in block_attention_ref's layout;
    a block with no cache segments (or no text) gives NaN for that part."""
    self_m = [dict(m, text_len=0) for m in metas]
    text_m = [dict(m, segs=[]) for m in metas]
    res = []
    for ms in (self_m, text_m):
        ok = [bool(sum(n for _, n in m["segs"]) + m.get("text_len", 0)) for m in ms]
        safe = [m if g else dict(m, q_len=0) for m, g in zip(ms, ok)]
        res.append(block_attention_ref(q, ring, text_ring, safe, scale=scale, heads=heads, rows=rows))
    return tuple(res)
