"""Per-block DDIM update through the C ABI against the fp64 oracle.

The kernel applies fp32 coefficients with one FMA and rounds once to bf16;
the oracle rounds the exact fp64 step once.  The kernel's value before its
final rounding differs from the exact step by the fp32 evaluation error
e32 <= 4 * 2^-24 * (|c1 x| + |c2 eps|) (coefficient roundings, the product
and the FMA), which only shows where the two terms cancel.  Bar: every
element within one bf16 ulp of the result plus e32 of the oracle's value,
at least 99.9 % bit-exact, and t' = t bit-exact identity."""
import numpy as np
import pytest

from oracle import numerics as N
from oracle import schedule as S
from workloads import CONFIGS, draw, make_attention_inputs, make_update_inputs

pytestmark = pytest.mark.gpu


def _run(x_bits, e_bits, ts, sched=None):
    import torch
    import block_wise_long_amd as B
    from _util import to_dev, to_host_bits
    x = to_dev(x_bits, "bf16")
    e = to_dev(e_bits, "bf16")
    B.ba_block_update(x, e, ts, sched)
    torch.cuda.synchronize()
    return to_host_bits(x)


def _check(got, x, e, ts, **sched):
    T = sched.get("T", 1000)
    flow = sched.get("kind", "ddim") == "flow"
    ab = S.alpha_bar(T, sched.get("beta_start", 1e-4), sched.get("beta_end", 0.02))
    ref = S.block_update_ref(x, e, ts, **sched)
    xf, ef = N.bf16_bits_to_f64(x), N.bf16_bits_to_f64(e)
    g = N.bf16_bits_to_f64(got)
    r = N.bf16_bits_to_f64(ref)
    for b, t in enumerate(ts):
        tp = S.prev_timestep(t, sched.get("stride", 20))
        if flow:
            shift = sched.get("shift", 1.0)
            c1, c2 = S.flow_coefficients(int(t), tp, T, shift)
            exact = S.flow_step(xf[b], ef[b], int(t), tp, T, shift)
        else:
            c1, c2 = S.ddim_coefficients(int(t), tp, ab)
            exact = S.ddim_step(xf[b], ef[b], int(t), tp, ab)
        e32 = 4 * 2.0 ** -24 * (np.abs(c1 * xf[b]) + np.abs(c2 * ef[b]))
        mag = np.abs(exact) + e32
        ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(mag, 2.0 ** -126))).astype(int) - 7)
        bad = np.abs(g[b] - r[b]) > ulp + e32
        assert not bad.any(), (t, g[b][bad][:4], r[b][bad][:4])
    assert (got == ref).mean() >= 0.999, f"exact fraction {(got == ref).mean():.5f}"


@pytest.mark.parametrize("E", [345600, 1, 7, 8, 9, 1001])
def test_update_matches_oracle(E):
    rng = np.random.Generator(np.random.PCG64(E))
    ts = [1 + (999 * b) // 7 for b in range(8)]
    x = draw(rng, (8, E), 1.0, "bf16")
    e = draw(rng, (8, E), 1.0, "bf16")
    _check(_run(x, e, ts), x, e, ts)


def test_large_block_spans_many_workgroups():
    # 40M elements in one block: 20k workgroups of one 16-byte vector per
    # thread, plus the scalar head and tail
    rng = np.random.Generator(np.random.PCG64(41))
    E = 40_000_003
    x = draw(rng, (1, E), 1.0, "bf16")
    e = draw(rng, (1, E), 1.0, "bf16")
    _check(_run(x, e, [571]), x, e, [571])


def test_identity_is_bit_exact():
    rng = np.random.Generator(np.random.PCG64(3))
    x = draw(rng, (3, 4099), 1.0, "bf16")
    e = draw(rng, (3, 4099), 1.0, "bf16")
    got = _run(x, e, [0, 0, 0])
    assert np.array_equal(got, x)
    got = _run(x, e, [5, 300, 1000], {"stride": 0})
    assert np.array_equal(got, x)


def test_queued_block_config_and_custom_schedule():
    cfg = CONFIGS[3]
    rng = make_attention_inputs(cfg)["_rng"]
    u = make_update_inputs(cfg, rng)
    ts = [int(t) for t in u["t"]]
    _check(_run(u["x"], u["eps"], ts), u["x"], u["eps"], ts)
    sched = {"T": 50, "stride": 3, "beta_start": 1e-3, "beta_end": 0.05}
    ts = [50, 49, 3, 2, 1, 0, 25, 10]
    _check(_run(u["x"], u["eps"], ts, sched), u["x"], u["eps"], ts, **sched)


def test_many_blocks_split_launches():
    rng = np.random.Generator(np.random.PCG64(11))
    nb = 70                                   # more than one launch's worth of coefficients
    ts = [int(t) for t in rng.integers(0, 1001, nb)]
    x = draw(rng, (nb, 333), 1.0, "bf16")
    e = draw(rng, (nb, 333), 1.0, "bf16")
    _check(_run(x, e, ts), x, e, ts)


@pytest.mark.parametrize("shift", [1.0, 5.0])
def test_flow_update_matches_oracle(shift):
    # velocity-prediction flow matching: x' = x + (sigma(t') - sigma(t)) v
    rng = np.random.Generator(np.random.PCG64(int(shift * 7)))
    ts = [1 + (999 * b) // 7 for b in range(8)]
    x = draw(rng, (8, 345600), 1.0, "bf16")
    v = draw(rng, (8, 345600), 1.0, "bf16")
    sched = {"kind": "flow", "T": 1000, "stride": 20, "shift": shift}
    _check(_run(x, v, ts, sched), x, v, ts, **sched)


def test_flow_identity_is_bit_exact():
    rng = np.random.Generator(np.random.PCG64(9))
    x = draw(rng, (2, 1001), 1.0, "bf16")
    v = draw(rng, (2, 1001), 1.0, "bf16")
    got = _run(x, v, [0, 700], {"kind": "flow", "stride": 0, "shift": 3.0})
    assert np.array_equal(got, x)
