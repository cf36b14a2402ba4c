"""Router inputs built on the host so that the binary64 certification of the
scoring kernel cannot decide the top-6 and the exact recomputation must.

FLOW (qiita.com/sukimaengineer/items/cd76fec76d49a098abed) § "MoE FFN 部の中身":
the router logit is x . W_r (4096 x 256, F16), the score sqrtsoftplus(logit),
the key score + bias, top-6 by key.  The logit is read as the exact dot
product rounded once to binary32; equal keys go to the lower expert index.

Every case has five experts far above the rest (bias +10), experts A and B
competing for the sixth slot (bias chosen as stated), and every other expert
far below (bias -10).  Router rows are zero except A's and B's.

"logit" cases: A's exact logit is a binary32 midpoint m plus or minus 2^-60;
the products sit in the columns one thread of the scoring kernel sums first,
in the order 2^20, the parts of m, +-2^-60, -2^20, so its binary64 sum loses
the 2^-60 and lands exactly on m, whose ties-to-even rounding is the wrong
neighbour.  B's logit is that wrong neighbour's other side: B's key equals
A's exact key, and the tie goes to the lower index.

"score" cases: A's logit is a binary32 value whose score lies within 2^-40
(relative) of a binary32 midpoint, beyond the binary64 evaluation's error
allowance; B's key is set equal to the correctly rounded score.

For each case the helpers also give the selection a summation in the
kernel's binary64 order followed by correct rounding would produce, so a
test can check that the case discriminates.
"""
from decimal import Decimal, getcontext

import numpy as np

H, E, K = 4096, 256, 6
TOP5 = (3, 17, 99, 130, 250)


def bf16_bits(v):
    """bf16 bits of a value with at most 8 significant bits (exact)."""
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, v
    return b >> 16


def f16_bits(v):
    h = np.array([v], np.float16)
    assert float(h[0]) == v, v
    return int(h.view(np.uint16)[0])


def chunks8(v):
    """A binary32 value as at most three parts of at most 8 significant bits
    each (exactly representable in bf16), summing to it exactly."""
    f = np.float32(v)
    if f == 0:
        return []
    u = int(np.array([f], np.float32).view(np.uint32)[0])
    sign = -1.0 if u >> 31 else 1.0
    ex, fr = (u >> 23) & 0xFF, u & 0x7FFFFF
    m, e = (fr | 0x800000, ex - 150) if ex else (fr, -149)
    parts = [(m >> 16) << 16, ((m >> 8) & 255) << 8, m & 255]
    return [sign * float(p) * 2.0 ** e for p in parts if p]


def exact_ssp(z):
    getcontext().prec = 80
    zd = Decimal(float(z))
    sp = zd + (1 + (-zd).exp()).ln() if zd > 0 else (1 + zd.exp()).ln()
    return sp.sqrt()


def rn_f32(v):
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Decimal(float(c)) - v),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))


def score(z):
    return rn_f32(exact_ssp(z))


def flip_pair(even_lower):
    """Adjacent binary32 logits zl < zh near 1 whose scores round apart; the
    lower one's last significand bit is even (even_lower) or odd."""
    z = np.float32(1.0)
    while True:
        zl, z = z, np.nextafter(z, np.float32(np.inf))
        if score(zl) != score(z):
            even = (int(np.array([zl], np.float32).view(np.uint32)[0]) & 1) == 0
            if even == even_lower:
                return zl, z


class Case:
    def __init__(self, name, a, b):
        self.name, self.A, self.B = name, a, b
        self.x = np.zeros(H, np.float64)    # values, bf16-exact
        self.W = np.zeros((E, H), np.float64)
        self.bias = np.full(E, -10.0, np.float32)
        self.bias[list(TOP5)] = 10.0
        self.naive_sA = None

    def x_bits(self):
        return np.array([bf16_bits(v) for v in self.x], np.uint16)

    def w_bits(self):
        out = np.zeros((E, H), np.uint16)
        for e in (self.A, self.B):
            for c in np.nonzero(self.W[e])[0]:
                out[e, c] = f16_bits(self.W[e, c])
        return out

    def naive_ids(self):
        """Top-6 with A's score rounded the wrong way (from the binary64 sum's
    rounding of its logit, or across the score's near midpoint)."""
        keys = np.full(E, np.float32(-1e30), np.float32)
        s0 = score(np.float32(0.0))
        for e in range(E):
            keys[e] = np.float32(s0 + self.bias[e])
        zb = np.float32(sum(float(v) for v in self.x * self.W[self.B]))
        keys[self.B] = np.float32(score(zb) + self.bias[self.B])
        keys[self.A] = np.float32(self.naive_sA + self.bias[self.A])
        order = sorted(range(E), key=lambda e: (-float(keys[e]), e))
        return np.array(order[:K], np.int32)


def logit_case(a, b, up):
    """A's exact logit just above (up) or below a midpoint of two binary32
    logits whose scores round apart; B's key equals A's exact key."""
    zl, zh = flip_pair(even_lower=up)
    m = (float(zl) + float(zh)) / 2          # exact: 25 significant bits
    c = Case("logit-%s-A%d-B%d" % ("up" if up else "down", a, b), a, b)
    # thread 0 of the scoring kernel sums columns 0..7 in order
    parts = [(2.0 ** 10, 2.0 ** 10), (1.0, 1.0)]
    parts += [(p, 1.0) for p in chunks8(m - 1.0)]
    parts += [((2.0 ** -60) if up else -(2.0 ** -60), 1.0), (2.0 ** 10, -(2.0 ** 10))]
    assert len(parts) <= 8
    for col, (xv, wv) in enumerate(parts):
        c.x[col], c.W[a, col] = xv, wv
    acc = 0.0
    for xv, wv in parts:                     # the kernel's binary64 order
        acc += xv * wv
    assert acc == m
    naive_z = np.float32(acc)                # ties to even: the wrong side
    want = zh if up else zl
    assert naive_z != want
    c.naive_sA = score(naive_z)
    # B: the exact logit `want`, in thread 1's columns, certified
    for j, p in enumerate(chunks8(want)):
        c.x[8 + j], c.W[b, 8 + j] = p, 1.0
    c.bias[[a, b]] = 0.0
    c.zA = want
    return c


def score_case(a, b, hard_z):
    """A's logit hard_z (its score within 2^-40 of a rounding midpoint);
    B's key set to A's correctly rounded score."""
    c = Case("score-A%d-B%d" % (a, b), a, b)
    for j, p in enumerate(chunks8(hard_z)):
        c.x[16 + j], c.W[a, 16 + j] = p, 1.0
    s_true = score(hard_z)
    s_b = score(np.float32(0.0))             # B's row is zero: logit 0
    c.bias[a] = 0.0
    c.bias[b] = np.float32(s_true) - np.float32(s_b)   # exact (Sterbenz)
    assert np.float32(s_b + c.bias[b]) == s_true
    # the wrong rounding of A's score: the neighbour across the near midpoint
    side = np.float32(np.inf) if exact_ssp(hard_z) > Decimal(float(s_true)) else np.float32(-np.inf)
    c.naive_sA = np.nextafter(s_true, side)
    c.zA = hard_z
    c.s_true = s_true
    return c


def hard_score_logit(lo=-0.5, hi=1.5, n=2_000_001, limit=2.0 ** -40):
    """A binary32 logit in [lo, hi] whose score lies within `limit` of a
    rounding midpoint, screened in x87 extended precision and confirmed in
    80-digit decimal arithmetic."""
    z = np.linspace(lo, hi, n).astype(np.float32)
    zl = z.astype(np.longdouble)
    s = np.sqrt(np.where(zl > 0, zl + np.log1p(np.exp(-zl)), np.log1p(np.exp(zl))))
    cc = s.astype(np.float32)
    mh = (cc.astype(np.longdouble) + np.nextafter(cc, np.float32(np.inf))) / 2
    ml = (cc.astype(np.longdouble) + np.nextafter(cc, np.float32(-np.inf))) / 2
    d = np.minimum(np.abs(s - mh), np.abs(s - ml)) / s
    for i in np.argsort(d)[:20]:
        v = exact_ssp(z[i])
        f = rn_f32(v)
        fd = Decimal(float(f))
        up = Decimal(float(np.nextafter(f, np.float32(np.inf))))
        dn = Decimal(float(np.nextafter(f, np.float32(-np.inf))))
        dist = min(abs(v - (fd + up) / 2), abs(v - (fd + dn) / 2)) / v
        if dist < Decimal(limit):
            return z[i]
    raise AssertionError("no hard logit found")


def all_cases():
    hz = hard_score_logit()
    return [logit_case(60, 190, up=True), logit_case(190, 60, up=False),
            score_case(60, 190, hz), score_case(190, 60, hz)]
