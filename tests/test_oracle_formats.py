"""Pins of the oracle's element formats and scale rule against the pages'
definitions, library casts and hand-worked values (CPU only)."""
import math
import struct

import numpy as np
import pytest
import torch

from conftest import read_golden


def test_e2m1_value_set(orc):
    """Codes 0..7 decode to the E2M1 magnitudes; bit 3 is the sign."""
    for code, val in read_golden("e2m1_values.txt"):
        code, val = int(code), float(val)
        assert orc.e2m1_value(code) == val
        assert orc.e2m1_value(code | 8) == -val
        assert math.copysign(1.0, orc.e2m1_value(code | 8)) == -1.0
    mags = [orc.e2m1_value(c) for c in range(8)]
    assert mags == sorted(mags) and len(set(mags)) == 8


def test_e4m3_decode_matches_torch(orc):
    """Every E4M3FN byte decodes as torch.float8_e4m3fn does (NaN for 0x7f/0xff)."""
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(256):
        v = orc.e4m3_value(i)
        if math.isnan(ref[i]):
            assert math.isnan(v)
        else:
            assert v == ref[i], i


def test_e8m0_matches_torch(orc):
    """E8M0 bytes decode to 2^(b-127) as torch.float8_e8m0fnu does, and the
    byte of 2^k is k+127."""
    b = torch.arange(255, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for i in range(255):
        assert orc.e8m0_value(i) == ref[i]
    for k in range(-127, 128):
        enc = torch.tensor([2.0 ** k], dtype=torch.float64).to(torch.float8_e8m0fnu)
        assert enc.view(torch.uint8).item() == k + 127
        # the oracle's scale for a block whose amax is exactly 6*2^k
        assert orc.truncfree_exponent(6.0 * 2.0 ** k) + 127 == k + 127


def test_scale_bytes_golden(orc):
    for M, qmax, byte in read_golden("scale_bytes.txt"):
        assert orc.truncfree_exponent(float(M), float(qmax)) + 127 == int(byte), M


def _f32(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def _scan_values():
    """fp32 amax values over every exponent with boundary and random mantissas."""
    rng = np.random.default_rng(5)
    vals = []
    for e in range(0, 255):
        for m in (0, 1, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFF, int(rng.integers(0, 1 << 23)),
                  int(rng.integers(0, 1 << 23))):
            if e == 0 and m == 0:
                continue
            vals.append(_f32((e << 23) | m))
    return vals


def test_truncation_free_invariant(orc):
    """Sec. 3.1 property: after scaling, the block amax lies in (3, 6] --
    never clipped, and one smaller power of two would clip it."""
    for M in _scan_values():
        k = orc.truncfree_exponent(M, 6.0)
        v = math.ldexp(M, -k)
        if k > -127:
            assert 3.0 < v <= 6.0, (M, k)
        else:
            assert v <= 6.0 and M <= 6.0 * 2.0 ** -127


def test_scale_matches_floor_rule_plus_overflow_bump(orc):
    """A second derivation: floor(log2 M) - 2 (the OCP MX rule for E2M1,
    emax 2), plus one exactly when the mantissa exceeds 1.5, where the floor
    rule would clip.  Computed from frexp, not from the oracle's comparison."""
    for M in _scan_values():
        mant, ex = math.frexp(M)          # M = mant * 2^ex, mant in [0.5, 1)
        k = (ex - 1) - 2 + (1 if 2 * mant > 1.5 else 0)
        k = max(-127, min(127, k))
        assert orc.truncfree_exponent(M, 6.0) == k, M


def test_scale_matches_library_log2(orc):
    """Away from power-of-two boundaries, ceil(math.log2(M/6)) agrees."""
    rng = np.random.default_rng(11)
    for M in np.exp(rng.uniform(-80, 80, 4000)):
        q = math.log2(M / 6.0)
        if abs(q - round(q)) < 1e-9:
            continue
        assert orc.truncfree_exponent(M, 6.0) == max(-127, min(127, math.ceil(q)))
    for M in np.exp(rng.uniform(-80, 80, 2000)):
        q = math.log2(M / 448.0)
        if abs(q - round(q)) < 1e-9:
            continue
        assert orc.truncfree_exponent(M, 448.0) == max(-127, min(127, math.ceil(q)))


def test_e4m3_round_matches_torch(orc):
    """RNE onto E4M3FN equals torch's float32 -> float8_e4m3fn cast, including
    exact midpoints between neighbours."""
    rng = np.random.default_rng(3)
    pos = np.arange(127)
    grid = np.array([orc.e4m3_value(int(c)) for c in pos])
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids, rng.uniform(0, 448, 20000),
                           np.exp(rng.uniform(-20, 6, 5000))]).astype(np.float32)
    vals = vals[vals <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r in zip(vals.tolist(), ref.tolist()):
        assert orc.e4m3_round(v) == r, v


def test_rne_ties_golden(orc):
    for v, code in read_golden("rne_ties.txt"):
        assert orc.e2m1_round(float(v), orc.ROUND_RNE, 0) == int(code), v


def test_round_rejects_out_of_range(orc):
    assert orc.e2m1_round(6.0000001, orc.ROUND_SR, 0) == -1
    assert orc.e2m1_round(-0.1, orc.ROUND_SR, 0) == -1
    assert orc.e4m3_round(448.5) == -1
