"""Pins for oracle/formats.py (RNE to binary16 / bfloat16, decoding).

The oracle's rounding is checked against
  * hand-derived conversions in tests/golden/rne_cases.txt (halfway cases,
    overflow, subnormals, signed zero),
  * numpy's float64 -> float16 conversion (an independent implementation of
    the IEEE conversion) over a wide random sample,
  * torch's float32 -> bfloat16 conversion (round to nearest even) over a wide
    random sample of binary32 values,
  * exhaustive decode of every 16-bit pattern against numpy / torch.
"""
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rne_cases.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, val, bits = line.split()[:3]
            rows.append((fmt, float.fromhex(val), int(bits, 16)))
    return rows


@pytest.mark.parametrize("fmt,val,bits", _golden_rows())
def test_golden_rne(fmt, val, bits):
    got = int(formats.encode(np.array([val]), fmt)[0])
    assert got == bits, f"{fmt} {val.hex()} -> {got:#06x}, expected {bits:#06x}"
    # the rounded value decodes to the same number the bits denote
    r = formats.round_to(np.array([val]), fmt)[0]
    d = formats.decode(np.array([bits], dtype=np.uint16), fmt)[0]
    assert (r == d) or (np.isnan(r) and np.isnan(d))
    if r == 0:
        assert np.signbit(r) == np.signbit(d)


def _wide_sample(rng, n):
    # magnitudes spanning subnormal .. overflow of binary16, plus exact halfway
    # points between neighbouring binary16 values
    mag = np.exp2(rng.uniform(-27, 17, n))
    x = mag * rng.choice([-1.0, 1.0], n)
    h = rng.integers(0, 0x7BFF, n // 4).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    return np.concatenate([x, 0.5 * (lo + hi), -0.5 * (lo + hi)])


def test_f16_matches_numpy_conversion():
    rng = np.random.default_rng(1234)
    x = _wide_sample(rng, 400_000)
    ours = formats.encode(x, "f16")
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def test_bf16_matches_torch_conversion_on_binary32_inputs():
    rng = np.random.default_rng(99)
    # random binary32 bit patterns: every exponent, every fraction
    b = rng.integers(0, 1 << 32, 400_000, dtype=np.uint64).astype(np.uint32)
    x32 = b.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    # exact ties of bfloat16: low 16 bits == 0x8000
    t = (rng.integers(0, 1 << 16, 50_000).astype(np.uint32) << 16) | 0x8000
    t32 = t.view(np.float32)
    x32 = np.concatenate([x32, t32[np.isfinite(t32)]])
    ours = formats.encode(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={float(x32[bad[0]]).hex()}"


def test_decode_all_patterns():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    d16 = formats.decode(allb, "f16")
    r16 = allb.view(np.float16).astype(np.float64)
    same = (d16 == r16) | (np.isnan(d16) & np.isnan(r16))
    assert same.all()
    dbf = formats.decode(allb, "bf16")
    rbf = torch.from_numpy(allb.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (dbf == rbf) | (np.isnan(dbf) & np.isnan(rbf))
    assert same.all()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_round_trip_is_identity_on_representable(fmt):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = formats.decode(allb, fmt)
    keep = np.isfinite(v)
    back = formats.encode(v[keep], fmt)
    assert np.array_equal(back, allb[keep])


def test_round_f32_is_binary32():
    # 1 + 2^-24 is a binary32 tie -> 1; 1 + 3*2^-24 -> 1 + 2^-22
    x = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** 24 + 1])
    r = formats.round_f32(x)
    assert r[0] == 1.0 and r[1] == 1 + 2.0 ** -22 and r[2] == 2.0 ** 24
