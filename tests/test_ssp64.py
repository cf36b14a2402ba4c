"""Accuracy of the router's sqrtsoftplus evaluations (csrc/ssp64.h).

The scoring kernel certifies the binary32 rounding of each score with a
relative error allowance of 2^-40 on its binary64 evaluation; this test
measures that function (compiled for the host from the same source) against
120-digit decimal arithmetic and requires a 16x margin (<= 2^-44).  Scores it
leaves undecided are re-evaluated in double-double, whose rounding decision
allows 2^-90: the test requires <= 2^-96 and checks the decision on logits
whose score lies within 2^-40 of a binary32 rounding midpoint."""
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
def lib():
    d = tempfile.mkdtemp(prefix="ssp64_")
    src = os.path.join(d, "shim.cpp")
    with open(src, "w") as f:
        f.write('#include "ssp64.h"\n'
                'extern "C" double ds4_ssp64(float z) { return ds4::ssp64(z); }\n'
                'extern "C" void ds4_ssp_dd(float z, double* h, double* l) {\n'
                '  ds4::DD v = ds4::ssp_dd(z); *h = v.hi; *l = v.lo; }\n'
                'extern "C" float ds4_dd_round(double h, double l, double eps, int* ok) {\n'
                '  bool b; float r = ds4::dd_round_f32(ds4::DD{h, l}, eps, b); *ok = b; return r; }\n')
    so = os.path.join(d, "libshim.so")
    subprocess.run(["g++", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-I", CSRC, "-o", so, src],
                   check=True)
    L = ctypes.CDLL(so)
    L.ds4_ssp64.argtypes = [ctypes.c_float]
    L.ds4_ssp64.restype = ctypes.c_double
    L.ds4_ssp_dd.argtypes = [ctypes.c_float, ctypes.POINTER(ctypes.c_double),
                             ctypes.POINTER(ctypes.c_double)]
    L.ds4_dd_round.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                               ctypes.POINTER(ctypes.c_int)]
    L.ds4_dd_round.restype = ctypes.c_float
    return L


@pytest.fixture(scope="module")
def ssp(lib):
    return lib.ds4_ssp64


def ssp_dd(lib, z):
    h, l = ctypes.c_double(), ctypes.c_double()
    lib.ds4_ssp_dd(float(z), ctypes.byref(h), ctypes.byref(l))
    return h.value, l.value


def dd_round(lib, h, l, eps=2.0 ** -90):
    ok = ctypes.c_int()
    r = lib.ds4_dd_round(h, l, eps, ctypes.byref(ok))
    return np.float32(r), bool(ok.value)


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


def rn_f32_decimal(v):
    """Nearest binary32 to a positive Decimal, ties to even (exact comparisons
    of the neighbours against v)."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Decimal(float(c)) - v),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))


def hard_logits(lo, hi, n, limit=2.0 ** -40):
    """binary32 logits in [lo, hi] whose score lies within `limit` (relative)
    of a binary32 rounding midpoint, screened in x87 extended precision (64
    significant bits) and confirmed in 120-digit decimal arithmetic."""
    z = np.linspace(lo, hi, n).astype(np.float32)
    zl = z.astype(np.longdouble)
    s = np.sqrt(np.where(zl > 0, zl + np.log1p(np.exp(-zl)), np.log1p(np.exp(zl))))
    c = s.astype(np.float32)
    mh = (c.astype(np.longdouble) + np.nextafter(c, np.float32(np.inf))) / 2
    ml = (c.astype(np.longdouble) + np.nextafter(c, np.float32(-np.inf))) / 2
    d = np.minimum(np.abs(s - mh), np.abs(s - ml)) / s
    out = []
    for i in np.where(d < 2 * limit)[0]:
        v = exact(z[i])
        f = rn_f32_decimal(v)
        up = Decimal(float(np.nextafter(f, np.float32(np.inf))))
        dn = Decimal(float(np.nextafter(f, np.float32(-np.inf))))
        fd = Decimal(float(f))
        dist = min(abs(v - (fd + up) / 2), abs(v - (fd + dn) / 2)) / v
        if dist < Decimal(limit):
            out.append((z[i], f, float(dist)))
    return out


def test_ssp_dd_relative_error(lib):
    # down to z = -600 (below, e^z is subnormal in binary64 and the score is
    # far under the least binary32 subnormal: see the next test)
    zs = np.concatenate([np.linspace(-120, 120, 1201), np.random.default_rng(1).normal(0, 2, 600),
                         [0.0, 1e-30, -1e-30, 1e-7, -1e-7, 0.34657, -0.34657, 300.0, -300.0,
                          -600.0, 700.0, 1e6, 3.0e38]])
    worst = 0.0
    for z in zs.astype(np.float32):
        want = exact(z)
        h, l = ssp_dd(lib, z)
        rel = abs((Decimal(h) + Decimal(l) - want) / want)
        worst = max(worst, float(rel))
    assert worst <= 2.0 ** -96, worst


def test_ssp_dd_deep_negative_tail_rounds_to_zero(lib):
    # z <= -210: the score sqrt(ln(1 + e^z)) < 2^-151 rounds to binary32 0,
    # decided by the rounding test however imprecise the tiny value is;
    # z = -200 still gives a subnormal score, decided and correct
    for z in (-210.0, -300.0, -700.0, -744.0, -800.0, -3.0e38):
        h, l = ssp_dd(lib, np.float32(z))
        assert dd_round(lib, h, l) == (np.float32(0.0), True), z
    h, l = ssp_dd(lib, np.float32(-200.0))
    got, ok = dd_round(lib, h, l)
    assert ok and got == rn_f32_decimal(exact(np.float32(-200.0))) and 0 < got < 2.0 ** -126


def test_dd_rounding_decides_where_binary64_cannot(lib):
    # logits whose score sits within 2^-40 of a rounding midpoint: the binary64
    # allowance cannot decide them, the double-double evaluation must, and
    # must agree with decimal arithmetic and with the oracle's binary128
    import oracle
    hard = hard_logits(-12.0, 12.0, 1_000_001)
    assert len(hard) >= 5, len(hard)
    for z, want, dist in hard:
        h, l = ssp_dd(lib, z)
        got, ok = dd_round(lib, h, l)
        assert ok, (z, dist)
        assert got == want, (z, got, want)
        assert np.float32(oracle.sqrtsoftplus(z)) == want


def test_dd_round_f32_cases(lib):
    # exact binary32 values, values just off a midpoint either way, a value on
    # a midpoint (undecidable), zero and the subnormal range
    one = 1.0
    assert dd_round(lib, one, 0.0) == (np.float32(1.0), True)
    m = 1.0 + 2.0 ** -24                        # midpoint of 1 and 1 + 2^-23
    assert dd_round(lib, m, 2.0 ** -80) == (np.float32(1.0 + 2.0 ** -23), True)
    assert dd_round(lib, m, -2.0 ** -80) == (np.float32(1.0), True)
    assert dd_round(lib, m, 0.0)[1] is False
    assert dd_round(lib, m, 2.0 ** -95)[1] is False   # within eps * v of the midpoint
    assert dd_round(lib, 0.0, 0.0) == (np.float32(0.0), True)
    assert dd_round(lib, 2.0 ** -151, 0.0) == (np.float32(0.0), True)
    assert dd_round(lib, 3 * 2.0 ** -151, 0.0) == (np.float32(2.0 ** -149), True)
    assert dd_round(lib, 2.0 ** -150, 0.0)[1] is False
