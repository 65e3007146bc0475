"""The fused K/V producer on seeded random shapes against the fp64 oracle:
token counts from 1 to 600 (ragged token tiles), input dims from 64 to 512,
1-5 heads of 64 or 128 (channel tiles spanning q, k and v), with and without
q and the rotation, any slot of a 1-3 slot ring.  Same bar as the fixed
shapes: within one bf16 ulp plus the fp32 bound, >= 99 % bit-exact, the
slot's tail zero and every other slot untouched."""
import numpy as np
import pytest

from test_gpu_project import _case

pytestmark = pytest.mark.gpu


def _params(seed):
    r = np.random.Generator(np.random.PCG64(seed))
    D = int(r.choice([64, 128]))
    H = int(r.integers(1, 6))
    L = int(r.integers(1, 601))
    dim = 64 * int(r.integers(1, 9))
    n_slots = int(r.integers(1, 4))
    slot = int(r.integers(0, n_slots))
    return L, dim, H, D, slot, n_slots, bool(r.random() < 0.7), bool(r.random() < 0.6)


@pytest.mark.parametrize("seed", range(16))
def test_random_producer_shape(seed):
    L, dim, H, D, slot, n_slots, with_q, with_rope = _params(7000 + seed)
    _case(L, dim, H, D, slot=slot, n_slots=n_slots, with_q=with_q, with_rope=with_rope, seed=7000 + seed)
