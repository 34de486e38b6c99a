"""CPU check of the kernels' building blocks (fp4q_device.hpp built for the
host): the block exponents, Philox and the in-register transposes agree with
the oracle and with numpy.  No GPU needed.  (Element rounding runs on the
hardware converters; the GPU tests pin it against the oracle over every bf16
pattern and every block exponent.)"""
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
