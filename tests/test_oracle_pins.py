"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test pins one function of oracle/ to something other than itself:
hand-built blocks with hand-derived values (tests/golden), the pages'
packing statement, exact rational arithmetic (fractions), high-precision
decimal evaluation, brute-force dense matmul on decoded weights, and
invariants of the method.  Pages: FLOW = qiita.com/sukimaengineer/items/
cd76fec76d49a098abed, DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec.
"""
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import ds4gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------
def rn_f32(fr):
    """Nearest binary32 to a Fraction, ties to even (exact comparisons)."""
    if fr == 0:
        return np.float32(0.0)
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    def key(c):
        return (abs(Fraction(float(c)) - fr), int(np.array(c, np.float32).view(np.uint32)) & 1)
    return min(cands, key=key)


def f16_frac(bits):
    v = np.array([bits], np.uint16).view(np.float16)[0]
    return Fraction(float(v))


def bf16_frac(bits):
    v = np.array([int(bits) << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(v))


def read_cases(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------
# Q2_K (DS4C2 sec. 3)
# --------------------------------------------------------------------------
def q2k_block(scales, qs, d, dmin):
    b = np.zeros(84, np.uint8)
    b[0:16] = scales
    b[16:80] = qs
    b[80:82] = np.array([d], np.uint16).view(np.uint8)
    b[82:84] = np.array([dmin], np.uint16).view(np.uint8)
    return b


def test_q2k_block_size_matches_page():
    # 16 scale bytes + 64 code bytes + fp16 d + fp16 dmin = 84 bytes per 256 values
    assert 16 + 64 + 2 + 2 == 84 == ds4gen.BLOCK_BYTES[ds4gen.Q2_K]


@pytest.mark.parametrize("case", read_cases("q2k_blocks.txt"), ids=lambda c: c[0])
def test_q2k_hand_built(case):
    name, sb, qb, d, dmin, expect = case
    b = q2k_block(np.full(16, int(sb, 16)), np.full(64, int(qb, 16)), int(d, 16), int(dmin, 16))
    y = oracle.dequant(oracle.Q2_K, b)
    if expect == "pair":
        want = np.array([(i % 128) // 32 for i in range(256)], np.float64)
    else:
        want = np.full(256, float(expect))
    np.testing.assert_array_equal(y, want)


def pack_q2k_codes(L):
    """The page's packing statement: for each half (j = 0, 128) and l < 32,
    qs[j/4 + l] = L[j+l] | L[j+l+32]<<2 | L[j+l+64]<<4 | L[j+l+96]<<6."""
    qs = np.zeros(64, np.uint8)
    for j in (0, 128):
        for l in range(32):
            qs[j // 4 + l] = (L[j + l] | (L[j + l + 32] << 2) | (L[j + l + 64] << 4)
                              | (L[j + l + 96] << 6))
    return qs


def test_q2k_code_positions_follow_page_packing():
    # one non-zero code at each of the 256 positions, sc=1, d=1, no min
    for pos in range(256):
        L = np.zeros(256, np.int64)
        L[pos] = 3
        y = oracle.dequant(oracle.Q2_K, q2k_block(np.full(16, 1), pack_q2k_codes(L), 0x3C00, 0))
        want = np.zeros(256)
        want[pos] = 3.0
        np.testing.assert_array_equal(y, want)


def test_q2k_subblock_scales_and_mins():
    # scale j = j, min j = 15-j; all codes 2; d = 1, dmin = 0.5:
    # value i lies in 16-value sub-block i//16 -> 2*(i//16) - 0.5*(15 - i//16)
    scales = np.array([(15 - j) << 4 | j for j in range(16)], np.uint8)
    y = oracle.dequant(oracle.Q2_K, q2k_block(scales, np.full(64, 0xAA), 0x3C00, 0x3800))
    for i in range(256):
        j = i // 16
        assert y[i] == 2 * j - 0.5 * (15 - j)


# --------------------------------------------------------------------------
# IQ2_XXS-style (DS4C2 sec. 4)
# --------------------------------------------------------------------------
TEST_GRID = np.array([[1 + j + 8 * (i % 4) for j in range(8)] for i in range(256)], np.uint8)


def test_iq2_block_size_matches_page():
    assert 2 + 8 * (4 + 4) == 66 == ds4gen.BLOCK_BYTES[ds4gen.IQ2_XXS]


@pytest.mark.parametrize("case", read_cases("iq2xxs_blocks.txt"), ids=lambda c: c[0])
def test_iq2_hand_built(case):
    name, W = case[0], int(case[1], 16)
    num = np.array([int(v) for v in case[2:]], np.float64)
    assert num.size == 32
    b = np.zeros(66, np.uint8)
    b[0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    for g in range(8):
        b[2 + 8 * g: 6 + 8 * g] = [0, 1, 2, 3]
        b[6 + 8 * g: 10 + 8 * g] = np.array([W], np.uint32).view(np.uint8)
    y = oracle.dequant(oracle.IQ2_XXS, b, TEST_GRID.ravel())
    grid_vals = np.array([TEST_GRID[k][j] for k in range(4) for j in range(8)], np.float64)
    want = num / 8.0 * grid_vals
    for g in range(8):
        np.testing.assert_array_equal(y[32 * g: 32 * g + 32], want)


def test_iq2_grid_index_selects_entry():
    # group g, sub-vector k uses index byte k of the group: put index 4g+k
    grid = np.arange(2048, dtype=np.int64).reshape(256, 8) % 251 + 1
    b = np.zeros(66, np.uint8)
    b[0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    for g in range(8):
        b[2 + 8 * g: 6 + 8 * g] = [4 * g + k + 17 for k in range(4)]
    y = oracle.dequant(oracle.IQ2_XXS, b, grid.astype(np.uint8).ravel())
    for g in range(8):
        for k in range(4):
            np.testing.assert_array_equal(y[32 * g + 8 * k: 32 * g + 8 * k + 8],
                                          grid[4 * g + k + 17] / 8.0)


def test_q80_closed_form():
    b = np.zeros(34, np.uint8)
    b[0:2] = np.array([0x3800], np.uint16).view(np.uint8)  # d = 0.5
    b[2:] = np.array([i - 16 for i in range(32)], np.int8).view(np.uint8)
    np.testing.assert_array_equal(oracle.dequant(oracle.Q8_0, b), [(i - 16) / 2 for i in range(32)])


# --------------------------------------------------------------------------
# exact dot product -> binary32 (router logit definition)
# --------------------------------------------------------------------------
def exact_dot_frac(x, xfmt, w, wfmt):
    fx = {"bf16": bf16_frac, "f16": f16_frac, "f32": lambda v: Fraction(float(v))}
    return sum((fx[xfmt](a) * fx[wfmt](b) for a, b in zip(x, w)), Fraction(0))


def test_exact_dot_random_bf16_f16():
    rng = np.random.default_rng(1)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        x = ds4gen.normal(trial, 10, n, 0, 1, "bf16")
        w = ds4gen.normal(trial, 1, n, 0, 0.02, "f16")
        got = oracle.exact_dot(x, "bf16", w, "f16")
        assert np.float32(got) == rn_f32(exact_dot_frac(x, "bf16", w, "f16"))


def test_exact_dot_cancellation_beats_fp64():
    # huge terms cancel exactly; fp64 left-to-right summation loses the tail
    x = np.array([1e30, 1.0, -1e30, 3e-8], np.float32)
    w = np.array([1.0, 1.0, 1.0, 1.0], np.float32)
    want = rn_f32(exact_dot_frac(x, "f32", w, "f32"))
    assert np.float32(oracle.exact_dot(x, "f32", w, "f32")) == want
    assert want == np.float32(1.0 + 3e-8)


def test_exact_dot_ties_to_even():
    one = np.float32(1.0)
    u = np.float32(2.0 ** -24)
    # 1 + 2^-24 is half-way between 1 and 1+2^-23 -> even (1.0)
    assert oracle.exact_dot(np.array([one, u], np.float32), "f32", np.ones(2, np.float32), "f32") == 1.0
    # 1 + 3*2^-24 is half-way between 1+2^-23 (odd) and 1+2^-22 (even)
    v = oracle.exact_dot(np.array([one, u, u, u], np.float32), "f32", np.ones(4, np.float32), "f32")
    assert v == np.float32(1.0 + 2.0 ** -22)
    # a tail far below the half-ulp still breaks the tie upwards
    v = oracle.exact_dot(np.array([one, u, np.float32(2.0 ** -100)], np.float32), "f32",
                         np.ones(3, np.float32), "f32")
    assert v == np.float32(1.0 + 2.0 ** -23)


def test_exact_dot_subnormal_and_zero():
    x = np.array([2.0 ** -75, -(2.0 ** -75)], np.float32)
    w = np.abs(x)
    assert oracle.exact_dot(x, "f32", w, "f32") == 0.0
    # two products of 2^-150 each sum to the least binary32 subnormal 2^-149
    assert oracle.exact_dot(x, "f32", x, "f32") == np.float32(2.0 ** -149)
    x = np.array([2.0 ** -75, 2.0 ** -76], np.float32)
    w = np.array([2.0 ** -75, 2.0 ** -76], np.float32)
    want = rn_f32(Fraction(2) ** -150 + Fraction(2) ** -152)
    assert np.float32(oracle.exact_dot(x, "f32", w, "f32")) == want


# --------------------------------------------------------------------------
# sqrtsoftplus (FLOW config table: scoring function name only)
# --------------------------------------------------------------------------
def ssp_decimal(z):
    getcontext().prec = 120
    zd = Decimal(float(z))
    if zd > 0:
        sp = zd + (1 + (-zd).exp()).ln()
    else:
        y = zd.exp()
        sp = (1 + y).ln() if y > Decimal("1e-40") else y - y * y / 2 + y * y * y / 3
    return Fraction(sp.sqrt())


def test_sqrtsoftplus_zero_is_sqrt_ln2():
    getcontext().prec = 60
    assert np.float32(oracle.sqrtsoftplus(0.0)) == rn_f32(Fraction(Decimal(2).ln().sqrt()))


@pytest.mark.parametrize("z", [-200.0, -60.0, -17.5, -3.0, -1.0, -0.125, 1e-6, 0.5, 1.0,
                               2.75, 7.0, 19.0, 40.0, 100.0])
def test_sqrtsoftplus_correctly_rounded(z):
    assert np.float32(oracle.sqrtsoftplus(z)) == rn_f32(ssp_decimal(np.float32(z)))


def test_sqrtsoftplus_random_and_monotone():
    zs = np.sort(ds4gen.normal(5, 1, 300, 0.0, 1.5, "f32"))
    got = [np.float32(oracle.sqrtsoftplus(z)) for z in zs]
    for z, g in zip(zs[:60], got[:60]):
        assert g == rn_f32(ssp_decimal(z))
    assert all(a <= b for a, b in zip(got, got[1:]))


# --------------------------------------------------------------------------
# router selection and gates (FLOW "MoE FFN" section)
# --------------------------------------------------------------------------
def small_router(seed, T=6, H=64, E=16):
    x = ds4gen.normal(seed, 10, T * H, 0, 1, "bf16").reshape(T, H)
    W = ds4gen.normal(seed, 1, E * H, 0, 0.05, "f16").reshape(E, H)
    b = ds4gen.uniform_f32(seed, 2, E, -0.1, 0.1)
    return x, W, b


def test_route_invariants():
    x, W, b = small_router(3)
    ids, w, z, s = oracle.route(x, "bf16", W, "f16", b, K=4)
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == 4
        assert ids[t].min() >= 0 and ids[t].max() < 16
        assert np.all(w[t] > 0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.5) <= 1.5 * 4e-7
        # logits are the exact dot products rounded once
        for e in range(16):
            assert z[t, e] == rn_f32(exact_dot_frac(x[t], "bf16", W[e], "f16"))


def test_route_zero_bias_is_topk_of_logits():
    x, W, b = small_router(4)
    ids, _, z, _ = oracle.route(x, "bf16", W, "f16", np.zeros(16, np.float32), K=5)
    for t in range(ids.shape[0]):
        order = sorted(range(16), key=lambda e: (-float(z[t, e]), e))
        assert ids[t].tolist() == order[:5]


def test_route_bias_forces_expert_but_not_its_gate():
    x, W, b = small_router(5)
    ids0, w0, _, s = oracle.route(x, "bf16", W, "f16", np.zeros(16, np.float32), K=3)
    bias = np.zeros(16, np.float32)
    bias[11] = 1000.0
    ids1, w1, _, s1 = oracle.route(x, "bf16", W, "f16", bias, K=3)
    for t in range(ids1.shape[0]):
        assert ids1[t, 0] == 11
        sel = ids1[t]
        # gate = 1.5 * s_k / sum s over the selected, without the bias
        ssum = sum(Fraction(float(s1[t, e])) for e in sel)
        assert np.float32(w1[t, 0]) == rn_f32(Fraction(3, 2) * Fraction(float(s1[t, 11])) / ssum) or \
            abs(float(w1[t, 0]) - float(Fraction(3, 2) * Fraction(float(s1[t, 11])) / ssum)) < 1e-7


def test_route_k_equals_e_selects_all_in_key_order():
    x, W, b = small_router(6, E=8)
    ids, w, _, s = oracle.route(x, "bf16", W, "f16", b, K=8)
    for t in range(ids.shape[0]):
        assert sorted(ids[t].tolist()) == list(range(8))
        keys = [np.float32(s[t, e] + b[e]) for e in ids[t]]
        assert all(keys[i] >= keys[i + 1] for i in range(7))


def test_route_ties_go_to_lower_index():
    x, W, b = small_router(7)
    W[9] = W[3]  # identical rows -> identical logits, scores and (zero-bias) keys
    ids, _, z, _ = oracle.route(x, "bf16", W, "f16", np.zeros(16, np.float32), K=16)
    for t in range(ids.shape[0]):
        row = ids[t].tolist()
        assert row.index(3) + 1 == row.index(9) or z[t, 3] != z[t, 9]
        assert row.index(3) < row.index(9)


def test_route_hash_is_table_lookup():
    table = ds4gen.tid2eid(4, 11, 0, 1000, 256, 6)
    tok = ds4gen.uniform_int(4, 16, 50, 1000)
    ids, w = oracle.route_hash(tok, table, 256, 6)
    np.testing.assert_array_equal(ids, table[tok])
    assert np.all(w == np.float32(0.25))
    with pytest.raises(ValueError):
        oracle.route_hash(np.array([1000], np.int32), table, 256, 6)
    bad = table.copy()
    bad[5, 3] = bad[5, 1]
    with pytest.raises(ValueError):
        oracle.route_hash(np.array([5], np.int32), bad, 256, 6)


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
def test_permute_invariants():
    ids, _ = ds4gen.zipf_routing(3, 200, 64, 6)
    counts, offsets, perm, inv = oracle.permute(ids, 64)
    n = ids.size
    assert counts.sum() == n and offsets[0] == 0 and offsets[-1] == n
    assert np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(n))
    np.testing.assert_array_equal(inv[perm], np.arange(n))
    flat = ids.ravel()
    keys = [(int(flat[p]), int(p)) for p in perm]
    assert all(a < b for a, b in zip(keys, keys[1:]))
    for e in range(64):
        assert np.all(flat[perm[offsets[e]:offsets[e + 1]]] == e)


def test_permute_rejects_bad_id():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 64]], np.int32), 64)


# --------------------------------------------------------------------------
# expert FFN: brute force on tiny shapes
# --------------------------------------------------------------------------
def tiny_experts(w, n_e, grid=None):
    mats = {}
    for e in range(n_e):
        mats[e] = tuple(ds4gen.expert_tensor_blocks(w, 0, which, e, 1)
                        for which in ("gate", "up", "down"))
    return mats


def dense(qt, blocks, R, C, grid=None):
    return oracle.dequant(qt, blocks, grid).reshape(R, C)


def brute_ffn(x64, mats, ids, wts, qts, H, I, grid=None):
    out = np.zeros((x64.shape[0], H))
    for t in range(x64.shape[0]):
        for k in range(ids.shape[1]):
            g_, u_, d_ = mats[int(ids[t, k])]
            Wg, Wu, Wd = dense(qts[0], g_, I, H, grid), dense(qts[1], u_, I, H, grid), dense(qts[2], d_, H, I, grid)
            g = Wg @ x64[t]
            u = Wu @ x64[t]
            h = g / (1.0 + np.exp(-g)) * u
            out[t] += float(wts[t, k]) * (Wd @ h)
    return out


def test_ffn_matches_dense_bruteforce_tiny_q2k():
    w = ds4gen.WORKLOADS[0]  # H=256, I=128, E=16, K=2, all Q2_K (down blocks span 2 rows)
    mats = tiny_experts(w, w.E)
    x = ds4gen.activations(w)
    ids = np.array([[0, 5], [15, 3], [7, 8], [5, 0]], np.int32)
    wts = np.array([[1.0, 0.5], [0.75, 0.75], [1.25, 0.25], [0.5, 1.0]], np.float32)
    qts = (w.gate_qt, w.up_qt, w.down_qt)
    got = oracle.moe_ffn(x, "f32", ids, wts, mats, qts, w.H, w.I, w.E)
    want = brute_ffn(x.astype(np.float64), mats, ids, wts, qts, w.H, w.I)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


def test_ffn_iq2_gate_up_bruteforce_and_identical_experts():
    # small IQ2_XXS/Q2_K shape; identical experts -> out = 1.5 * E(x)
    w = ds4gen.Workload("t", 9, 2, 256, 256, 4, 3, ds4gen.IQ2_XXS, ds4gen.IQ2_XXS, ds4gen.Q2_K,
                        "bf16", "f16")
    grid = ds4gen.grid(9)
    one = tuple(ds4gen.expert_tensor_blocks(w, 0, which, 0, 1) for which in ("gate", "up", "down"))
    mats = {e: one for e in range(4)}
    x = ds4gen.activations(w)
    x64 = np.array([[bf16_frac(v) for v in row] for row in x], dtype=np.float64)
    ids = np.array([[0, 1, 2], [3, 2, 1]], np.int32)
    wts = np.array([[0.5, 0.5, 0.5], [0.2, 0.3, 1.0]], np.float32)
    qts = (w.gate_qt, w.up_qt, w.down_qt)
    got = oracle.moe_ffn(x, "bf16", ids, wts, mats, qts, w.H, w.I, w.E, grid=grid)
    single = brute_ffn(x64, {0: one}, np.zeros((2, 1), np.int32), np.ones((2, 1), np.float32),
                       qts, w.H, w.I, grid)
    np.testing.assert_allclose(got, 1.5 * single, rtol=1e-6, atol=1e-6 * np.abs(single).max())


def test_ffn_shared_expert_added_unscaled():
    w = ds4gen.WORKLOADS[0]
    mats = tiny_experts(w, 2)
    x = ds4gen.activations(w)[:1]
    sh = tuple(ds4gen.blocks(ds4gen.Q8_0, 0, ds4gen.stream(0, k), 0, w.I * w.H // 32)
               for k in (ds4gen.SH_GATE, ds4gen.SH_UP, ds4gen.SH_DOWN))
    ids = np.array([[0, 1]], np.int32)
    wts = np.array([[0.0, 0.0]], np.float32)
    qts = (w.gate_qt, w.up_qt, w.down_qt)
    got = oracle.moe_ffn(x, "f32", ids, wts, mats, qts, w.H, w.I, w.E, shared=sh, sh_I=w.I)
    Wg, Wu, Wd = (dense(ds4gen.Q8_0, sh[0], w.I, w.H), dense(ds4gen.Q8_0, sh[1], w.I, w.H),
                  dense(ds4gen.Q8_0, sh[2], w.H, w.I))
    xx = x[0].astype(np.float64)
    g, u = Wg @ xx, Wu @ xx
    want = Wd @ (g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(got[0], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


# --------------------------------------------------------------------------
# RMSNorm and rounding
# --------------------------------------------------------------------------
def test_round_bf16_ties_to_even():
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.round_bf16(-2.5) == 0xC020
    assert oracle.round_bf16(2.0 ** -133) == 0x0001  # least bf16 subnormal
    assert oracle.round_bf16(3.0e38 * 1.2) == 0x7F80


def test_rmsnorm_constant_and_scale_invariance():
    h = np.full((1, 4096), 2.0, np.float32)
    xn = oracle.rmsnorm_bf16(h, np.ones(4096, np.float32), 1e-6)
    # 2 / sqrt(4 + 1e-6) = 0.999999875 -> nearest bf16 is 1.0
    assert np.all(xn == 0x3F80)
    h = ds4gen.normal(3, 10, 2 * 4096, 0, 1, "f32").reshape(2, 4096)
    w = ds4gen.normal(3, 12, 4096, 1.0, 0.1, "f32")
    a = oracle.rmsnorm_bf16(h, w, 0.0)
    b = oracle.rmsnorm_bf16(h * np.float32(8.0), w, 0.0)
    np.testing.assert_array_equal(a, b)


def rn_bf16_bits(fr):
    """Bits of the bfloat16 nearest to a Fraction in the normal range, ties to
    even (Python rounds Fractions half to even)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(Fraction(fr))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    n = round(a / Fraction(2) ** (e - 7))   # 128 <= n <= 256
    if n == 256:
        n, e = 128, e + 1
    assert 128 <= n < 256 and -126 <= e <= 127
    return sign | ((e + 127) << 7) | (n - 128)


def frac_sqrt_inv(fr, digits=60):
    """1/sqrt(fr) to `digits` significant digits, as a Fraction."""
    getcontext().prec = digits
    d = Decimal(fr.numerator) / Decimal(fr.denominator)
    return Fraction(1 / d.sqrt())


def test_rmsnorm_hand_values_weight_mean_and_eps():
    # FLOW § "1 トークンの旅: 全体フロー": each layer normalises the residual
    # stream before the MoE block.  xn = h * (mean h^2 + eps)^(-1/2) * w, per
    # element, rounded once to bfloat16.  Hand cases, chosen so that dropping
    # w, summing h^2 instead of averaging it, moving eps outside the root or
    # ignoring it each give different bits.
    # h = (3, 4, 0, 0), w = (2, 1/2, 1, 1), eps = 0: mean h^2 = 25/4, factor
    # 2/5, xn = (12/5, 4/5, 0, 0) -> bf16 2.40625 and 0.80078125
    h = np.array([[3.0, 4.0, 0.0, 0.0]], np.float32)
    w = np.array([2.0, 0.5, 1.0, 1.0], np.float32)
    xn = oracle.rmsnorm_bf16(h, w, 0.0)
    assert rn_bf16_bits(Fraction(12, 5)) == 0x401A and rn_bf16_bits(Fraction(4, 5)) == 0x3F4D
    assert xn.tolist() == [[0x401A, 0x3F4D, 0, 0]]
    # without w: (6/5, 8/5); with sum instead of mean: (6/5, 2/5)
    assert rn_bf16_bits(Fraction(6, 5)) != 0x401A and rn_bf16_bits(Fraction(2, 5)) != 0x3F4D
    # eps inside the root: h = (1, 1), eps = 3 -> (1 + 3)^(-1/2) = 1/2 exactly
    # (eps outside the root would give 1/4, no eps 1)
    xn = oracle.rmsnorm_bf16(np.ones((1, 2), np.float32), np.ones(2, np.float32), 3.0)
    assert xn.tolist() == [[0x3F00, 0x3F00]]
    # h = (1, 2, 2), eps = 1: mean h^2 = 3, (3 + 1)^(-1/2) = 1/2 -> (1/2, 1, 1)
    xn = oracle.rmsnorm_bf16(np.array([[1.0, 2.0, 2.0]], np.float32), np.ones(3, np.float32), 1.0)
    assert xn.tolist() == [[0x3F00, 0x3F80, 0x3F80]]
    # the layer's eps = 1e-6 moves a small constant row: h = 2^-10 everywhere,
    # xn = 2^-10 / sqrt(2^-20 + 1e-6) ~= 0.6987 (not 1)
    c = Fraction(1, 1024)
    want = rn_bf16_bits(c * frac_sqrt_inv(c * c + Fraction(1e-6)))
    assert want == 0x3F33
    xn = oracle.rmsnorm_bf16(np.full((2, 8), 2.0 ** -10, np.float32), np.ones(8, np.float32), 1e-6)
    assert np.all(xn == want)


def test_rmsnorm_rows_and_columns_independent():
    # each token is normalised by its own mean; each column takes its own
    # weight: token 1 = 4 x token 0 gives the same xn (eps = 0), and swapping
    # two columns of h and w swaps the outputs
    h0 = np.array([1.0, -2.0, 0.5, 3.0, 0.25, -1.5, 2.0, 1.0], np.float32)
    w = np.array([1.5, 0.75, 2.0, 0.5, 1.0, 3.0, 0.25, 1.25], np.float32)
    xn = oracle.rmsnorm_bf16(np.stack([h0, 4 * h0]), w, 0.0)
    np.testing.assert_array_equal(xn[0], xn[1])
    ms = sum(Fraction(float(v)) ** 2 for v in h0) / 8
    inv = frac_sqrt_inv(ms)
    assert xn[0].tolist() == [rn_bf16_bits(Fraction(float(a)) * inv * Fraction(float(b)))
                              for a, b in zip(h0, w)]
    p = [1, 0, 2, 3, 4, 5, 7, 6]
    xp = oracle.rmsnorm_bf16(h0[p][None, :], w[p], 0.0)
    np.testing.assert_array_equal(xp[0], xn[0][p])


def test_residual_add_binary32():
    # FLOW token flow: the block's output is added to the residual stream,
    # held in binary32 here, so the sum is rounded once to binary32.
    r = oracle.residual_add(np.array([1.0, 2.0, -3.0], np.float32),
                            np.array([10.0, -5.0, 1.0], np.float32))
    assert r.tolist() == [11.0, -3.0, -2.0]
    one = np.float32(1.0)
    r = oracle.residual_add(np.array([1.0, 1.0, 2.0 ** 24, 0.5], np.float32),
                            np.array([2.0 ** -24, 3 * 2.0 ** -24, 1.0, 0.25], np.float32))
    # 1 + 2^-24: a tie, to even (1); 1 + 3 * 2^-24: a tie, to even (1 + 2^-22);
    # 2^24 + 1: a tie, to even (2^24); 0.5 + 0.25 exact
    assert r[0] == one and r[1] == np.float32(1.0 + 2.0 ** -22)
    assert r[2] == np.float32(2.0 ** 24) and r[3] == np.float32(0.75)
    # the second operand is not modified and the first is returned updated
    out = np.array([2.0, 3.0], np.float32)
    res = np.array([1.0, 1.0], np.float32)
    assert oracle.residual_add(res, out).tolist() == [3.0, 4.0]
    assert out.tolist() == [2.0, 3.0]


# --------------------------------------------------------------------------
# size arithmetic printed on the pages (FLOW config table and decode reads)
# --------------------------------------------------------------------------
def test_sizes_match_pages():
    w = ds4gen.WORKLOADS[1]
    assert 3 * w.H * w.I == 25_165_824            # params per routed expert
    assert w.expert_bytes() == 7_077_888
    per_tok_layer = 6 * w.expert_bytes()
    assert per_tok_layer == 42_467_328              # "about 42 MB"
    assert abs(per_tok_layer / 1e6 - 42) < 1
    assert 43 * per_tok_layer == 1_826_095_104      # "about 1.8 GB per token"
    assert 256 * w.expert_bytes() == 1_811_939_328  # "about 1.8 GB per layer"


def test_mixed_stack_sizes_match_pages():
    # FLOW § "パラメータはどこにあるか: 層別の内訳": one layer of routed experts
    # is about 3.6 GB in Q4_K (about 4.5 bpw) and raising one layer from the
    # q2 mix to Q4_K costs about 1.8 GB.  DS4C2 §10: the best mixed file takes
    # the routed experts of layers 37-42 from the Q4 file, about 91 GB against
    # about 153 GB for all-Q4; BENCH16: the q2 file is 80.76 GiB.  With gate,
    # up and down all in Q4_K those three sizes agree to within rounding.
    w = ds4gen.WORKLOADS[5]
    q2, q4 = w.at_layer(0), w.at_layer(37)
    assert (q2.gate_qt, q2.up_qt, q2.down_qt) == (ds4gen.IQ2_XXS, ds4gen.IQ2_XXS, ds4gen.Q2_K)
    assert (q4.gate_qt, q4.up_qt, q4.down_qt) == (ds4gen.Q4_K,) * 3
    assert [l for l in range(43) if w.at_layer(l).gate_qt == ds4gen.Q4_K] == list(range(37, 43))
    assert q4.expert_bytes() == 3 * 2048 * 4096 // 256 * 144 == 14_155_776
    assert abs(q4.expert_bytes() * 8 / (3 * 2048 * 4096) - 4.5) < 1e-12
    assert 256 * q4.expert_bytes() == 3_623_878_656                 # "about 3.6 GB"
    step = 256 * (q4.expert_bytes() - q2.expert_bytes())
    assert step == 1_811_939_328                                     # "about 1.8 GB"
    q2_file = 80.76 * 2 ** 30
    assert abs((q2_file + 6 * step) / 2 ** 30 - 91) < 0.5
    assert abs((q2_file + 43 * step) / 2 ** 30 - 153) < 0.5
    assert w.stack_expert_bytes() == 37 * 256 * 7_077_888 + 6 * 256 * 14_155_776
    assert ds4gen.WORKLOADS[4].stack_expert_bytes() == 43 * 256 * 7_077_888
    assert w.token_expert_bytes() == 37 * 6 * 7_077_888 + 6 * 6 * 14_155_776 == 2_080_899_072


# --------------------------------------------------------------------------
# importance statistics (imatrix): DS4C2 sec. 5 and 7
# --------------------------------------------------------------------------
def q80_identity(n):
    """Q8_0 matrix [n][n] = identity (one 32-value block per row, d = 1.0)."""
    assert n == 32
    rows = np.zeros((n, 34), np.uint8)
    for i in range(n):
        rows[i, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
        rows[i, 2 + i] = 1
    return rows.ravel()


def test_imatrix_gate_up_hand_values():
    # x[t][c] = t + 1; pairs (t, e): (0,0) (0,1) (1,1) (1,2) (2,0) (2,2)
    H = I = 32
    x = np.array([[t + 1.0] * H for t in range(3)], np.float32)
    ids = np.array([[0, 1], [1, 2], [0, 2]], np.int32)
    wts = np.full((3, 2), 0.75, np.float32)
    blk = ds4gen.blocks(ds4gen.Q8_0, 5, 1, 0, I * H // 32)
    mats = {e: (blk, blk) for e in range(3)}
    gu, _ = oracle.imatrix(x, "f32", ids, wts, mats, (ds4gen.Q8_0, ds4gen.Q8_0), H, I, 4)
    np.testing.assert_array_equal(gu[0], 10.0)   # 1 + 9
    np.testing.assert_array_equal(gu[1], 5.0)    # 1 + 4
    np.testing.assert_array_equal(gu[2], 13.0)   # 4 + 9
    np.testing.assert_array_equal(gu[3], 0.0)    # never selected


def test_imatrix_down_is_square_of_weighted_swiglu_row():
    # with W_down = identity, E(x) = h, so a single pair's FFN output is w*h:
    # the down statistic of an expert is the sum of its pairs' squared outputs
    H = I = 32
    ident = q80_identity(32)
    mats = {e: (ds4gen.blocks(ds4gen.Q8_0, 7, 2 * e, 0, 32),
                ds4gen.blocks(ds4gen.Q8_0, 7, 2 * e + 1, 0, 32), ident) for e in range(2)}
    qts = (ds4gen.Q8_0, ds4gen.Q8_0, ds4gen.Q8_0)
    x = np.random.default_rng(3).normal(size=(3, H)).astype(np.float32)
    ids = np.array([[0, 1], [1, 0], [1, 0]], np.int32)
    wts = np.array([[1.25, 0.25], [0.5, 1.0], [0.75, 0.75]], np.float32)
    _, dn = oracle.imatrix(x, "f32", ids, wts, mats, qts, H, I, 2)
    want = np.zeros((2, I))
    for t in range(3):
        for k in range(2):
            e = int(ids[t, k])
            y = oracle.moe_ffn(x[t:t + 1], "f32", ids[t:t + 1, k:k + 1], wts[t:t + 1, k:k + 1],
                               {e: mats[e]}, qts, H, I, 2)
            want[e] += y[0].astype(np.float64) ** 2
    np.testing.assert_allclose(dn, want, rtol=2e-7)


def test_imatrix_invariants():
    # every token feeds K experts: sum over experts of the gate/up statistic is
    # K * sum_t x^2; doubling the routing weights multiplies the down statistic
    # by exactly 4; the expert bytes do not enter the gate/up statistic
    w = ds4gen.WORKLOADS[0]
    mats = tiny_experts(w, w.E)
    x = ds4gen.activations(w)
    ids = np.array([[0, 5], [15, 3], [7, 8], [5, 0]], np.int32)
    wts = np.array([[1.0, 0.5], [0.75, 0.75], [1.25, 0.25], [0.5, 1.0]], np.float32)
    qts = (w.gate_qt, w.up_qt, w.down_qt)
    gu, dn = oracle.imatrix(x, "f32", ids, wts, mats, qts, w.H, w.I, w.E)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose(gu.sum(0), ids.shape[1] * (x64 ** 2).sum(0), rtol=1e-15)
    gu2, dn2 = oracle.imatrix(x, "f32", ids, 2 * wts, mats, qts, w.H, w.I, w.E)
    np.testing.assert_array_equal(gu2, gu)
    np.testing.assert_array_equal(dn2, 4 * dn)
    other = {e: tiny_experts(w, w.E)[(e + 1) % w.E] for e in range(w.E)}
    gu3, dn3 = oracle.imatrix(x, "f32", ids, wts, other, qts, w.H, w.I, w.E)
    np.testing.assert_array_equal(gu3, gu)
    assert not np.array_equal(dn3, dn)


# --------------------------------------------------------------------------
# Q4_K decode (DS4C2 sec. 3 type table: 256 values in 144 bytes; layout by
# reading, see oracle/ds4_oracle.c)
# --------------------------------------------------------------------------
def q4k_block(d_bits, dmin_bits, sc, mn, codes):
    """Pack a Q4_K block from its fields (the inverse of the reading)."""
    b = np.zeros(144, np.uint8)
    b[0:2] = np.array([d_bits], np.uint16).view(np.uint8)
    b[2:4] = np.array([dmin_bits], np.uint16).view(np.uint8)
    S = np.zeros(12, np.int64)
    for j in range(4):
        S[j] = sc[j] & 63
        S[j + 4] = mn[j] & 63
    for j in range(4, 8):
        S[j + 4] = (sc[j] & 15) | ((mn[j] & 15) << 4)
        S[j - 4] |= (sc[j] >> 4) << 6
        S[j] |= (mn[j] >> 4) << 6
    b[4:16] = S.astype(np.uint8)
    for c in range(4):
        for l in range(32):
            b[16 + 32 * c + l] = (codes[64 * c + l] & 15) | ((codes[64 * c + 32 + l] & 15) << 4)
    return b


def test_q4k_block_size_matches_page():
    assert ds4gen.BLOCK_BYTES[ds4gen.Q4_K] == 144 == 2 + 2 + 12 + 128
    assert ds4gen.BLOCK_VALUES[ds4gen.Q4_K] == 256


def test_q4k_literal_block():
    # every code 15, every scale and min 63, d = 2^-10, dmin = 2^-11:
    # y = 945 * 2^-10 - 63 * 2^-11 = 0.89208984375 everywhere
    b = q4k_block(0x1400, 0x1000, [63] * 8, [63] * 8, [15] * 256)
    assert (b[4:16] == 255).all()
    np.testing.assert_array_equal(oracle.dequant(oracle.Q4_K, b), 0.89208984375)


def test_q4k_six_bit_scales_and_mins():
    # distinct 6-bit scale/min per sub-block, all codes 1: sub-block j is
    # d*sc_j - dmin*m_j (the upper four use the split high bits)
    sc = [1, 2, 45, 63, 20, 33, 48, 17]
    mn = [0, 5, 62, 31, 37, 16, 63, 50]
    b = q4k_block(0x3C00, 0x3800, sc, mn, [1] * 256)  # d = 1, dmin = 0.5
    y = oracle.dequant(oracle.Q4_K, b)
    for j in range(8):
        np.testing.assert_array_equal(y[32 * j: 32 * j + 32], sc[j] - 0.5 * mn[j])


def test_q4k_code_positions():
    # a single nonzero code at each position lands on its value index
    sc, mn = [3] * 8, [0] * 8
    for i in (0, 31, 32, 63, 64, 100, 191, 200, 255):
        codes = [0] * 256
        codes[i] = 9
        b = q4k_block(0x3C00, 0x0000, sc, mn, codes)
        want = np.zeros(256)
        want[i] = 27.0
        np.testing.assert_array_equal(oracle.dequant(oracle.Q4_K, b), want)
        # the byte holding value i: low nibble for the first 32 of each 64
        c, r = divmod(i, 64)
        assert b[16 + 32 * c + (r % 32)] == (9 if r < 32 else 9 << 4)


def test_ffn_q4k_experts_bruteforce():
    # all three expert matrices in Q4_K (down blocks span a row exactly)
    w = ds4gen.Workload("t4", 21, 3, 256, 256, 4, 2, ds4gen.Q4_K, ds4gen.Q4_K, ds4gen.Q4_K,
                        "f32", "f32")
    mats = tiny_experts(w, w.E)
    x = ds4gen.activations(w)
    ids = np.array([[0, 3], [2, 1], [3, 2]], np.int32)
    wts = np.array([[1.0, 0.5], [0.75, 0.75], [1.25, 0.25]], np.float32)
    qts = (w.gate_qt, w.up_qt, w.down_qt)
    got = oracle.moe_ffn(x, "f32", ids, wts, mats, qts, w.H, w.I, w.E)
    want = brute_ffn(x.astype(np.float64), mats, ids, wts, qts, w.H, w.I)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
