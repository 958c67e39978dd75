"""The per-element rounding bar of the 16-bit pool tests (CPU only): the
16-bit ulp helper against independent definitions of the formats' spacing."""

import numpy as np
import torch

from tests.gpu_util import rounding_excess, ulp16


def _values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(size=4000), rng.normal(size=2000) * 1e-3, rng.normal(size=2000) * 300,
                        [0.0, 1.0, -2.0, 0.5, 6.1e-5, 3e-7]])
    return x


def test_fp16_ulp_is_the_spacing_of_the_interval_holding_x():
    x = _values()
    u = ulp16(x, "f16")
    # numpy's spacing at x rounded to fp16 agrees except where x rounds up to
    # the next power of two; there the interval holding x is half as wide
    ref = np.spacing(np.abs(x).astype(np.float16)).astype(np.float64)
    rounds_up = np.abs(x).astype(np.float16).astype(np.float64) > np.abs(x)
    pow2 = np.log2(np.abs(x).astype(np.float16).astype(np.float64), where=np.abs(x) > 0,
                   out=np.zeros_like(x)) % 1 == 0
    special = rounds_up & pow2
    assert np.array_equal(u[~special], ref[~special])
    assert np.array_equal(u[special], ref[special] / 2)


def test_bf16_ulp_is_the_gap_between_neighbouring_bf16_values():
    x = _values()
    bits = torch.tensor(np.abs(x), dtype=torch.float32).view(torch.int32)
    lo = (bits & ~0xFFFF).view(torch.float32)                 # the bf16 value at or below |x|
    hi = ((bits & ~0xFFFF) + 0x10000).view(torch.float32)     # the next bf16 value up
    gap = (hi - lo).double().numpy()
    nz = np.abs(x) > 0
    assert np.array_equal(ulp16(x, "bf16")[nz], gap[nz])


def test_rounding_excess_of_a_once_rounded_state_is_at_most_one():
    rng = np.random.default_rng(3)
    ref = rng.normal(size=(2, 64, 64))
    for name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        got = torch.tensor(ref).to(dt).double().numpy()
        ex = rounding_excess(got, ref, name)
        assert ex.max() <= 1.0
        # an element moved one ulp further from ref than its rounding left it
        # is caught (about twice the bar)
        bad = got.copy()
        e = bad[0, 5, 7] - ref[0, 5, 7]
        bad[0, 5, 7] += np.copysign(ulp16(ref[0, 5, 7], name), e if e != 0 else 1.0)
        assert rounding_excess(bad, ref, name).max() > 1.9
