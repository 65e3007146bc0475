"""Fused K/V producer (oracle side; test infrastructure only).

The feature cache of "Minute-Long Videos with Dual Parallelisms" (Abstract)
holds the self-attention keys and values a block produced; in a DiT layer
those come out of the block's QKV projection.  The producer computes that
projection and writes K and V straight into the cache slot (and Q to its own
buffer), so no separate append pass copies them there.

Definition (a linear layer and the rotary position rotation, written out):
  Y = X W^T                      X: [tokens][dim], W: [3 H D][dim] (the
                                  layout of a linear layer's weight: output
                                  rows q | k | v, each head-major)
  q, k, v = Y[:, 0:HD], Y[:, HD:2HD], Y[:, 2HD:3HD], viewed [tokens][H][D]
  rotation (optional, on q and k): for every token t and pair p < D/2 the
  pair (y[2p], y[2p+1]) is multiplied, as the complex number
  y[2p] + i y[2p+1], by c + i s, with (c, s) = table[t][p] (the caller's
  cos/sin table, shared by all heads): (y0 c - y1 s, y0 s + y1 c).
The pages say nothing about positions; the table keeps the frequency scheme
with the caller and fixes only the pairing.  Everything in fp64, each output
rounded once to bf16.
"""
import numpy as np

from .numerics import bf16_bits_to_f64, f64_to_bf16_bits


def rotate_pairs(y, table):
    """y: [tokens][H][D] fp64; table: [tokens][D/2][2] (cos, sin)."""
    c = np.asarray(table[..., 0], dtype=np.float64)[:, None, :]
    s = np.asarray(table[..., 1], dtype=np.float64)[:, None, :]
    a, b = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qkv_project_ref(x_bits, w_bits, heads, head_dim, table=None):
    """x_bits: [tokens][dim], w_bits: [3 H D][dim] bf16 patterns.  Returns fp64
    q, k, v ([tokens][H][D]) before rounding."""
    X = bf16_bits_to_f64(x_bits)
    W = bf16_bits_to_f64(w_bits)
    Y = X @ W.T
    L, HD = X.shape[0], heads * head_dim
    q, k, v = (Y[:, j * HD:(j + 1) * HD].reshape(L, heads, head_dim) for j in range(3))
    if table is not None:
        q, k = rotate_pairs(q, table), rotate_pairs(k, table)
    return q, k, v


def qkv_project_bits(x_bits, w_bits, heads, head_dim, table=None):
    """The same, each output rounded once to bf16 (bit patterns)."""
    return tuple(f64_to_bf16_bits(y) for y in qkv_project_ref(x_bits, w_bits, heads, head_dim, table))
