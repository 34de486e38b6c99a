"""CPU check of the kernels' building blocks (fp4q_device.hpp built for the
host): the element rounding, the block exponents, Philox and the in-register
transposes agree with the oracle and with numpy, exhaustively over bf16
patterns.  No GPU needed."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_microscaling_quantization_quant2d_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("h") / "harness")
    subprocess.run([hipcc, "-O2", "-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include",
                    "-I", CSRC, os.path.join(ROOT, "tests", "device_logic_harness.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                             check=True).stdout
        return out.strip().splitlines()
    return run


def _bf16_patterns():
    p = np.arange(0x10000, dtype=np.uint32)
    return p[((p >> 7) & 0xFF) != 0xFF]


@pytest.mark.parametrize("rne", [0, 1])
def test_element_rounding_exhaustive_bf16(orc, harness, rne):
    rng = np.random.default_rng(1 + rne)
    pats = _bf16_patterns()
    x32 = (pats << 16).astype(np.uint32)
    xf = x32.view(np.float32).astype(np.float64)
    lines, expect = [], []
    for k in (-127, -126, -120, -110, -109, -108, -100, -30, -3, 0, 1, 7, 126):
        ok = np.abs(xf) * 2.0 ** -k <= 6.0
        for xb, v in zip(x32[ok].tolist(), xf[ok].tolist()):
            r = int(rng.integers(0, 65536)) if not rne else 0
            lines.append("nib %x %d %d %d" % (xb, k, r, rne))
            code = orc.e2m1_round(abs(v) * 2.0 ** -k, orc.ROUND_RNE if rne else orc.ROUND_SR, r)
            expect.append(code | (8 if xb >> 31 else 0))
    got = [int(t) for t in harness(lines)]
    bad = [i for i, (g, e) in enumerate(zip(got, expect)) if g != e]
    assert not bad, [lines[i] for i in bad[:5]]


def test_element_rounding_fp32_and_boundaries(orc, harness):
    rng = np.random.default_rng(7)
    lines, expect = [], []
    for k in (-127, -115, -109, -60, 0, 3, 100):
        lim = 6.0 * 2.0 ** k
        xs = np.concatenate([rng.uniform(-1, 1, 3000) * lim,
                             rng.uniform(-1, 1, 500) * lim * 2.0 ** -rng.integers(1, 40, 500),
                             rng.integers(1, 1 << 23, 300).astype(np.uint32).view(np.float32)]
                            ).astype(np.float32)
        xs = xs[np.abs(xs.astype(np.float64)) * 2.0 ** -k <= 6.0]
        for x in xs.tolist():
            xb = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
            for r in (0, 65535, int(rng.integers(0, 65536))):
                lines.append("nib %x %d %d 0" % (xb, k, r))
                expect.append(orc.e2m1_round(abs(x) * 2.0 ** -k, orc.ROUND_SR, r) | (8 if xb >> 31 else 0))
    got = [int(t) for t in harness(lines)]
    bad = [i for i, (g, e) in enumerate(zip(got, expect)) if g != e]
    assert not bad, [lines[i] for i in bad[:5]]


def test_block_exponents(orc, harness):
    rng = np.random.default_rng(3)
    vals = []
    for e in range(0, 255):
        for m in (0, 1, 0x3FFFFF, 0x400000, 0x400001, 0x5FFFFF, 0x600000, 0x600001, 0x7FFFFF,
                  int(rng.integers(0, 1 << 23))):
            vals.append((e << 23) | m)
    lines = ["exp2 %x" % v for v in vals] + ["exp8 %x" % v for v in vals]
    got = [int(t) for t in harness(lines)]
    f = np.array(vals, dtype=np.uint32).view(np.float32).astype(np.float64)
    exp = [orc.truncfree_exponent(v, 6.0) for v in f] + [orc.truncfree_exponent(v, 448.0) for v in f]
    assert got == exp


def test_philox(orc, harness):
    rng = np.random.default_rng(5)
    cases = rng.integers(0, 1 << 32, size=(500, 6), dtype=np.uint64)
    got = harness(["phx " + " ".join("%x" % v for v in c) for c in cases])
    for c, line in zip(cases, got):
        ref = orc.philox4x32_10(c[:4], c[4:])
        assert [int(t, 16) for t in line.split()] == ref.tolist()


def test_register_transposes(harness):
    rng = np.random.default_rng(11)
    for _ in range(50):
        nib = rng.integers(0, 16, size=(8, 8), dtype=np.uint32)
        words = [int(sum(int(nib[i, j]) << (4 * j) for j in range(8))) for i in range(8)]
        out = [int(t, 16) for t in harness(["ntr " + " ".join("%x" % w for w in words)])[0].split()]
        assert np.array_equal(np.array([[(out[j] >> (4 * i)) & 15 for i in range(8)]
                                        for j in range(8)]), nib.T)
        h = rng.integers(0, 1 << 16, size=(8, 8), dtype=np.uint32)
        dw = [(int(h[i, 2 * d]) | (int(h[i, 2 * d + 1]) << 16)) for i in range(8) for d in range(4)]
        out = [int(t, 16) for t in harness(["htr " + " ".join("%x" % w for w in dw)])[0].split()]
        ht = np.array([[(out[i * 4 + (j >> 1)] >> (16 * (j & 1))) & 0xFFFF for j in range(8)]
                       for i in range(8)])
        assert np.array_equal(ht, h.T)
