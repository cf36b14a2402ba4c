"""Accuracy of the router kernel's binary64 sqrtsoftplus (csrc/ssp64.h).

The kernel certifies the binary32 rounding of each score with a relative
error allowance of 2^-40; this test measures the function (compiled for the
host from the same source) against 120-digit decimal arithmetic and requires
a 16x margin (<= 2^-44)."""
import ctypes
import os
import subprocess
import tempfile
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_expert_ds4moe_amd", "csrc")


@pytest.fixture(scope="module")
def ssp():
    d = tempfile.mkdtemp(prefix="ssp64_")
    src = os.path.join(d, "shim.cpp")
    with open(src, "w") as f:
        f.write('#include "ssp64.h"\nextern "C" double ds4_ssp64(float z) { return ds4::ssp64(z); }\n')
    so = os.path.join(d, "libshim.so")
    subprocess.run(["g++", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-I", CSRC, "-o", so, src],
                   check=True)
    L = ctypes.CDLL(so)
    L.ds4_ssp64.argtypes = [ctypes.c_float]
    L.ds4_ssp64.restype = ctypes.c_double
    return L.ds4_ssp64


def exact(z):
    getcontext().prec = 120
    zd = Decimal(float(z))
    if zd > 0:
        sp = zd + (1 + (-zd).exp()).ln()
    else:
        y = zd.exp()
        sp = (1 + y).ln() if y > Decimal("1e-40") else y - y * y / 2 + y * y * y / 3
    return sp.sqrt()


def test_ssp64_relative_error(ssp):
    zs = np.concatenate([np.linspace(-80, 80, 4001), np.random.default_rng(0).normal(0, 2, 3000),
                         [0.0, 1e-30, -1e-30, 1e-7, -1e-7, 0.34657, -0.34657, 200.0, -200.0]])
    worst = 0.0
    for z in zs.astype(np.float32):
        want = exact(z)
        got = Decimal(ssp(float(z)))
        if want == 0:
            assert got == 0
            continue
        rel = abs((got - want) / want)
        worst = max(worst, float(rel))
    assert worst <= 2.0 ** -44, worst


def test_ssp64_tail_and_zero(ssp):
    assert ssp(-800.0) == 0.0          # below binary64 range of e^z; binary32 score is 0 anyway
    assert abs(ssp(0.0) - float(Decimal(2).ln().sqrt())) < 1e-15
    assert abs(ssp(1e6) - 1000.0) < 1e-9
