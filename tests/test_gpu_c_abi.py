"""The library from plain C: tests/c/abi_demo (built by __graft_entry__.build()
with gcc against the in-tree libblockattn.so and the HIP runtime, no Python,
no torch in that process) appends a context block, the current block and the
text, runs block attention (with a text ring, and again with the text as
plain arrays) and one DDIM update, and writes its inputs and outputs; they
are checked here against the oracle."""
import math
import os
import subprocess

import numpy as np
import pytest

from _util import check_contract
from oracle import attention as A
from oracle import numerics as N
from oracle import ring as oring
from oracle import schedule as S

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(__file__), "c", "abi_demo")


def test_plain_c_caller(tmp_path):
    assert os.path.exists(DEMO), "tests/c/abi_demo is built by __graft_entry__.build()"
    out_file = str(tmp_path / "abi_demo.bin")
    r = subprocess.run([DEMO, out_file], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "abi_demo ok: slots ctx 0 cur 1 text 0" in r.stdout
    raw = open(out_file, "rb").read()
    hdr = np.frombuffer(raw[:28], dtype=np.int32)
    magic, L, H, D, TXT, E, t = (int(v) for v in hdr)
    assert magic == 0x62616331
    sizes = [L * H * D] * 5 + [TXT * H * D] * 2 + [L * H * D] + [E] * 3
    data = np.frombuffer(raw[28:28 + 2 * sum(sizes)], dtype=np.uint16)
    parts, off = [], 0
    for n in sizes:
        parts.append(data[off:off + n])
        off += n
    rest = raw[28 + 2 * sum(sizes):]
    tail = np.frombuffer(rest[:48], dtype=np.int32)
    out2 = np.frombuffer(rest[48:], dtype=np.uint16)
    assert tail.size == 12 and out2.size == L * H * D
    # host bookkeeping from C: the noise frames and the queue plan at step 2
    from oracle import noise as NZ
    from oracle import queue as OQ
    assert tail[:4].tolist() == NZ.assign(7, 3, 21, 3, 4)
    plan, _ = OQ.plan(4, 1000, L, TXT, 2, 2)
    assert tail[4:8].tolist() == [e["write_slot"] for e in plan]
    assert tail[8:12].tolist() == [e["t"] for e in plan]
    q, kc, vc, ku, vu, kt, vt, out, x, eps, xa = parts
    blk = lambda a, n: a.reshape(n, H, D)
    ring = oring.RingModel(2, L, H, D, "bf16")
    ring.append(blk(kc, L), blk(vc, L), L)
    ring.append(blk(ku, L), blk(vu, L), L)
    text = oring.RingModel(1, TXT, H, D, "bf16")
    text.append(blk(kt, TXT), blk(vt, TXT), TXT)
    meta = [{"q_len": L, "segs": [(0, L), (1, L)], "text_slot": 0, "text_len": TXT}]
    ref, _ = A.block_attention_ref(N.bf16_bits_to_f64(blk(q, L))[None], ring, text, meta)
    got = N.bf16_bits_to_f64(blk(out, L))[None]
    check_contract(got, ref, "bf16", gate2=False)
    # the text as [H][TXT][D] arrays (ba_block_attention_text_arrays): the ring form's bits
    assert np.array_equal(out2, out)
    rms = math.sqrt(np.nanmean(ref ** 2))
    assert np.nanmax(np.abs(got - ref)) <= 2 ** -7 * np.nanmax(np.abs(ref)) + 0.05 * rms
    # the update: within one bf16 ulp of the oracle's (plus the fp32 evaluation error)
    exact = S.ddim_step(N.bf16_bits_to_f64(x), N.bf16_bits_to_f64(eps), t, S.prev_timestep(t, 20),
                        S.alpha_bar(1000, 1e-4, 0.02))
    c1, c2 = S.ddim_coefficients(t, S.prev_timestep(t, 20), S.alpha_bar(1000, 1e-4, 0.02))
    e32 = 4 * 2.0 ** -24 * (np.abs(c1 * N.bf16_bits_to_f64(x)) + np.abs(c2 * N.bf16_bits_to_f64(eps)))
    mag = np.abs(exact) + e32
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(mag, 2.0 ** -126))).astype(int) - 7)
    assert not (np.abs(N.bf16_bits_to_f64(xa) - exact) > ulp + e32).any()
