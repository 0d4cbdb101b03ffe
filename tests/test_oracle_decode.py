"""Pins for the oracle's FP8 decode tables and its BF16 rounding (CPU only).

FP8 formats: "DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores",
section 3.1 (E4M3 = 4 exponent + 3 mantissa bits, E5M2 = 5 + 2).  The pages do
not print code values, so the tables are pinned against torch's own
float8 -> float32 conversions (an external library) and against the closed
properties of the OCP formats.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests._exact import bf16_nearest_even, fp8_values


@pytest.mark.parametrize("fmt,dt", [(oracle.E4M3, torch.float8_e4m3fn), (oracle.E5M2, torch.float8_e5m2)])
def test_decode_matches_torch(fmt, dt):
    ours = oracle.decode_table(fmt)
    ref = torch.arange(256, dtype=torch.uint8).view(dt).float().double().numpy()
    assert np.array_equal(ours, ref, equal_nan=True)


def test_e4m3_anchors_and_counts():
    t = oracle.decode_table(oracle.E4M3)
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    nan = [c for c in range(256) if math.isnan(t[c])]
    assert nan == [0x7F, 0xFF]
    assert not np.isinf(t).any()
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0


def test_e5m2_anchors_and_counts():
    t = oracle.decode_table(oracle.E5M2)
    assert t[0x3C] == 1.0
    assert t[0x7B] == 57344.0
    assert t[0x04] == 2.0 ** -14         # smallest normal
    assert t[0x01] == 2.0 ** -16         # smallest subnormal
    assert t[0x7C] == math.inf and t[0xFC] == -math.inf
    assert sum(math.isnan(v) for v in t) == 6
    assert sum(math.isinf(v) for v in t) == 2


@pytest.mark.parametrize("fmt,top", [(oracle.E4M3, 0x7E), (oracle.E5M2, 0x7B)])
def test_decode_monotone_and_odd(fmt, top):
    t = oracle.decode_table(fmt)
    pos = t[: top + 1]
    assert np.all(np.diff(pos) > 0)
    for c in range(0x80):
        if math.isnan(t[c]):
            continue
        assert t[c | 0x80] == -t[c]


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_roundtrips_through_torch_encoder(fmt):
    """encode(dec(c)) == c for every non-NaN code (torch's float -> fp8 encoder)."""
    t = oracle.decode_table(fmt)
    dt = torch.float8_e4m3fn if fmt == oracle.E4M3 else torch.float8_e5m2
    for c in range(256):
        if math.isnan(t[c]):
            continue
        back = torch.tensor([t[c]], dtype=torch.float32).to(dt).view(torch.uint8).item()
        if t[c] == 0.0:
            assert back in (0x00, 0x80)
        else:
            assert back == c


# ---------------------------------------------------------------------------
# BF16 round-to-nearest-even from double
# ---------------------------------------------------------------------------

def test_bf16_special_values():
    assert oracle.bf16_rne(float("nan")) == 0x7FC0
    assert oracle.bf16_rne(math.inf) == 0x7F80
    assert oracle.bf16_rne(-math.inf) == 0xFF80
    assert oracle.bf16_rne(0.0) == 0x0000
    assert oracle.bf16_rne(-0.0) == 0x8000
    assert oracle.bf16_rne(1.0) == 0x3F80
    top = (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.bf16_rne(top) == 0x7F7F
    assert oracle.bf16_rne(top + 2.0 ** 119) == 0x7F80          # tie rounds to even = inf
    assert oracle.bf16_rne(top + 2.0 ** 119 * 0.999) == 0x7F7F
    assert oracle.bf16_rne(2.0 ** -133) == 0x0001               # smallest subnormal
    assert oracle.bf16_rne(2.0 ** -134) == 0x0000               # tie to even (zero)
    assert oracle.bf16_rne(3 * 2.0 ** -134) == 0x0002           # tie 1.5 ulp -> 2 (even)


def test_bf16_ties():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even pattern is 1.0
    assert oracle.bf16_rne(1 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert oracle.bf16_rne(1 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_rne(-(1 + 3 * 2.0 ** -8)) == 0xBF82


def test_bf16_matches_torch_on_float32_values():
    """For values exactly representable in float32, torch's float32 -> bfloat16
    conversion (round to nearest even) is an independent reference."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_rne(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_matches_bruteforce_search_on_doubles():
    """Doubles that are not float32 values: compare with a search over every
    finite BF16 value in exact rational arithmetic."""
    rng = np.random.default_rng(8)
    xs = list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 128, 300)))
    # values at and next to ties
    for e in (-130, -20, 0, 9, 100):
        for m in (128, 129, 200, 255):
            mid = (m + 0.5) * 2.0 ** (e - 7)
            xs += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid]
    for x in xs:
        assert oracle.bf16_rne(float(x)) == bf16_nearest_even(Fraction(float(x))), x


def test_exact_helper_uses_torch_values():
    assert fp8_values(0)[0x38] == 1.0 and fp8_values(1)[0x3C] == 1.0
