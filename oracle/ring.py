"""Byte-level model of the K/V ring buffer (oracle side).

The feature cache of "Minute-Long Videos with Dual Parallelisms" (Abstract)
stores the keys/values a block produced so that the neighbouring block can
reuse them as context; the FIFO queue of the pith.science verdict
(pith_extraction.key_machinery) appends a block at the tail each step.  The
ring is that cache: ``n_slots`` slots, the next FIFO slot is
``appended mod n_slots``.

Layout (the library's documented contract, modelled here element by element):
  T_pad = slot_tokens rounded up to a multiple of 64
  K[s][h][t][d] at element ((s*2 + 0)*H + h)*T_pad*D + t*D + d
  V[s][h][t][d] at element ((s*2 + 1)*H + h)*T_pad*D + d*T_pad + t
i.e. per (slot, head) K is a token-major [T_pad][D] matrix and V a
dim-major [D][T_pad] matrix.  An append of n tokens writes tokens [0, n) and
zeroes tokens [n, T_pad) of both K and V of that slot.
"""
import numpy as np

from .numerics import decode

TOKEN_ALIGN = 64


def padded_tokens(slot_tokens: int) -> int:
    return -(-slot_tokens // TOKEN_ALIGN) * TOKEN_ALIGN


class RingModel:
    def __init__(self, n_slots, slot_tokens, heads, head_dim, dtype="bf16"):
        self.n_slots, self.slot_tokens = n_slots, slot_tokens
        self.heads, self.head_dim, self.dtype = heads, head_dim, dtype
        self.t_pad = padded_tokens(slot_tokens)
        self.elem = {"bf16": np.uint16, "f32": np.uint32}[dtype]
        n = n_slots * 2 * heads * self.t_pad * head_dim
        self.mem = np.zeros(n, dtype=self.elem)   # a fresh ring reads as zeros
        self.appended = 0

    # --- element offsets of the documented layout ------------------------
    def k_offset(self, s, h, t, d):
        H, D, T = self.heads, self.head_dim, self.t_pad
        return ((s * 2 + 0) * H + h) * T * D + t * D + d

    def v_offset(self, s, h, t, d):
        H, D, T = self.heads, self.head_dim, self.t_pad
        return ((s * 2 + 1) * H + h) * T * D + d * T + t

    def nbytes(self):
        return self.mem.nbytes

    # --- append ------------------------------------------------------------
    def _raw(self, a):
        a = np.asarray(a)
        if self.dtype == "f32":
            return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return np.ascontiguousarray(a, dtype=np.uint16)

    def append(self, k, v, n_tokens, slot=None):
        """Copy k, v ([n_tokens][heads][head_dim]) into a slot; return the slot.

        With ``slot=None`` the FIFO slot ``appended mod n_slots`` is written and
        ``appended`` advances; an explicit slot leaves ``appended`` alone.
        """
        if not (0 < n_tokens <= self.slot_tokens):
            raise ValueError("n_tokens out of range")
        fifo = slot is None
        if fifo:
            slot = self.appended % self.n_slots
        if not (0 <= slot < self.n_slots):
            raise ValueError("slot out of range")
        k, v = self._raw(k), self._raw(v)
        H, D = self.heads, self.head_dim
        t = np.arange(self.t_pad)[:, None, None]
        h = np.arange(H)[None, :, None]
        d = np.arange(D)[None, None, :]
        kk = np.zeros((self.t_pad, H, D), dtype=self.elem)
        vv = np.zeros((self.t_pad, H, D), dtype=self.elem)
        kk[:n_tokens] = k[:n_tokens]
        vv[:n_tokens] = v[:n_tokens]
        self.mem[self.k_offset(slot, h, t, d)] = kk
        self.mem[self.v_offset(slot, h, t, d)] = vv
        if fifo:
            self.appended += 1
        return slot

    # --- logical read-back -------------------------------------------------
    def keys(self, slot, head, n):
        t = np.arange(n)[:, None]
        d = np.arange(self.head_dim)[None, :]
        return self._decode(self.mem[self.k_offset(slot, head, t, d)])

    def values(self, slot, head, n):
        t = np.arange(n)[:, None]
        d = np.arange(self.head_dim)[None, :]
        return self._decode(self.mem[self.v_offset(slot, head, t, d)])

    def _decode(self, raw):
        if self.dtype == "f32":
            return raw.view(np.float32).astype(np.float64)
        return decode(raw, "bf16")

    def as_bytes(self) -> bytes:
        return self.mem.tobytes()
