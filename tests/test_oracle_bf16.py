"""Pins for the oracle's float64 -> bfloat16 rounding (oracle/bf16.py).

* On float32-representable inputs the direct rounding must agree with
  torch's float32 -> bfloat16 conversion (a library routine; no double
  rounding is possible there).
* On arbitrary float64 inputs the result must be a nearest bfloat16 with ties
  to the even significand, checked with exact rational arithmetic against both
  neighbouring bfloat16 values.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16


def _finite_f32_sample(rng, n):
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_agrees_with_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    f = _finite_f32_sample(rng, 200_000)
    # keep values whose rounding does not overflow to inf
    f = f[np.abs(f) < 3.38e38]
    ours = bf16.round_rne(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _exact(bits):
    return Fraction(float(bf16.widen(np.array([bits], np.uint16))[0]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nearest_and_ties_even_exact(seed):
    rng = np.random.default_rng(seed)
    # values at many scales plus exact midpoints between bfloat16 neighbours
    mant = rng.uniform(1.0, 2.0, size=400)
    expo = rng.integers(-130, 120, size=400)
    xs = list(np.ldexp(mant, expo) * rng.choice([-1.0, 1.0], size=400))
    base = rng.integers(0x0081, 0x7F00, size=200).astype(np.uint16)
    mids = (bf16.widen(base) + bf16.widen(base + 1)) / 2.0  # exact in float64
    xs += list(mids) + list(-mids)
    for x in xs:
        r = int(bf16.round_rne(np.array([x]))[0])
        X = Fraction(float(x))
        R = _exact(r)
        mag = r & 0x7FFF
        for nb in (mag - 1, mag + 1):
            if 0 <= nb < 0x7F80:
                N = _exact(nb | (r & 0x8000))
                assert abs(X - R) <= abs(X - N), (x, hex(r), hex(nb))
                if abs(X - R) == abs(X - N):
                    assert mag % 2 == 0, (x, hex(r))


def test_special_values():
    x = np.array([0.0, -0.0, 1.0, -2.0, 3.4e38, 1e39, -1e39, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135])
    b = bf16.round_rne(x)
    assert b[0] == 0x0000 and b[1] == 0x8000
    assert b[2] == 0x3F80 and b[3] == 0xC000
    assert b[4] == 0x7F80 or b[4] == 0x7F7F  # rounds to max or inf per magnitude
    assert b[5] == 0x7F80 and b[6] == 0xFF80
    assert b[7] == 0x0001          # smallest subnormal is exact
    assert b[8] == 0x0000          # half of it ties to even (zero)
    assert b[9] == 0x0001          # 0.75 of it rounds up


def test_widen_is_exact_roundtrip():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(bf16.round_rne(bf16.widen(bits)), bits)
