"""Pins of the oracle's number codecs (BF16, E4M3, E2M1, E8M0) against independent
library routines (torch's BF16 / float8 conversions), the OCP MX v1.0 value tables,
and closed forms.  CPU only."""
import math

import numpy as np
import torch

# OCP MX v1.0, E2M1 element values for codes 0..7 (sign in bit 3)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_bf16_decode_exhaustive(orc):
    pats = np.arange(65536, dtype=np.uint32)
    ref = (pats << 16).view(np.float32)
    for b in range(0, 65536, 7):
        v = orc.bf16_to_f32(b)
        r = float(ref[b])
        assert (math.isnan(v) and math.isnan(r)) or v == r, b


def test_bf16_encode_matches_torch(orc):
    g = np.random.default_rng(1)
    bits = g.integers(0, 2**32, size=60000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([0.0, -0.0, 1.0, 3.3895314e38, 3.3961776e38, 3.40282347e38, -3.3961776e38,
                      1e-45, -1e-45, 1.1754942e-38, 9.18355e-41, 1.00390625, 1.01171875,
                      1.0078125 + 2**-9], np.float32)
    f = np.concatenate([f, extra])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(x)) for x in f], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(f[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_round_trip_exhaustive(orc):
    for b in range(65536):
        e = (b >> 7) & 0xFF
        if e == 0xFF and (b & 0x7F):
            continue  # NaN
        assert orc.f32_to_bf16(orc.bf16_to_f32(b)) == b


def test_e4m3_decode_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = orc.e4m3_value(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(v)
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c


def test_e4m3_closed_forms(orc):
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6  # smallest normal
    assert orc.e4m3_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_encode(448.0) == 0x7E
    assert orc.e4m3_encode(1e9) == 0x7E and orc.e4m3_encode(-1e9) == 0xFE  # saturation
    assert orc.e4m3_encode(432.0) == 0x7E  # tie between 416 (odd code) and 448 (even code)
    assert orc.e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9 -> even
    assert orc.e4m3_encode(3 * 2.0 ** -11) == 0x01
    assert orc.e4m3_encode(-0.0) == 0x80 and orc.e4m3_encode(0.0) == 0x00
    assert orc.e4m3_encode(-1e-30) == 0x80  # rounds to a zero that keeps its sign


def test_e4m3_encode_matches_torch_in_range(orc):
    g = np.random.default_rng(2)
    v = np.concatenate([g.standard_normal(20000) * 50, g.standard_normal(5000) * 0.01,
                        np.linspace(-448, 448, 4001)]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in v], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_every_midpoint_ties_to_even(orc):
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = 0.5 * (vals[c] + vals[c + 1])
        want = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == want, (c, mid)
        assert orc.e4m3_encode(-mid) == 0x80 | want


def test_e2m1_table(orc):
    for n in range(16):
        want = E2M1_TABLE[n & 7] * (-1 if n & 8 else 1)
        got = orc.e2m1_value(n)
        assert got == want and math.copysign(1, got) == (-1 if n & 8 else 1), n


def test_e8m0_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for b in range(255):
        assert orc.e8m0_value(b) == ref[b] == 2.0 ** (b - 127)
    assert math.isnan(orc.e8m0_value(255))
