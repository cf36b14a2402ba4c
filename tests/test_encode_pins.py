"""Pins of the oracle's block encoders (oracle/ds4_encode.c) against things
other than the encoders themselves: numpy's binary16 rounding, exact round
trips of blocks the format can represent (decoded by the separately pinned
decoder), brute force over codes and grid entries through that decoder,
exact scaling invariances, a hand-built neighbour map, and statistical
properties of the importance weighting (DS4C2 sec. 3-5, 8)."""
import numpy as np
import pytest

import ds4gen
import oracle

Q2_K, IQ2_XXS = oracle.Q2_K, oracle.IQ2_XXS
LEVELS = np.array([8, 25, 43], np.uint8)


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# binary16 rounding
# --------------------------------------------------------------------------
def test_f16_rounding_matches_numpy():
    r = rng(1)
    v = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-9, 5, 4000),
                        [0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
                         3 * 2.0 ** -26, 6.1e-5, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]])
    v = v.astype(np.float32)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f16_bits(x) for x in v], np.uint16)
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------
# Q2_K
# --------------------------------------------------------------------------
def q2k_representable(seed, n_blocks):
    """Blocks whose decoded values the encoder must reproduce exactly: every
    sub-block holds codes 0 and 3 (so its range is exact), scale nibbles 1..15
    and min nibbles 0..15 with a 15 of each in the block, d and dmin within a
    factor 4 of each other (decoded values exact in binary32)."""
    r = rng(seed)
    out = np.zeros((n_blocks, 84), np.uint8)
    for b in range(n_blocks):
        sc = r.integers(1, 16, 16)
        mn = r.integers(0, 16, 16)
        sc[r.integers(16)] = 15
        mn[r.integers(16)] = 15
        out[b, :16] = sc | (mn << 4)
        codes = r.integers(0, 4, 256)
        for j in range(16):
            p = r.permutation(16)[:2]
            codes[16 * j + p[0]] = 0
            codes[16 * j + p[1]] = 3
        for i in range(256):
            h, s, l = i // 128, (i % 128) // 32, i % 32
            out[b, 16 + 32 * h + l] |= codes[i] << (2 * s)
        d = np.float16(r.uniform(1e-3, 1e-2))
        dmin = np.float16(float(d) * r.uniform(0.3, 3.0))
        out[b, 80:82] = np.array([d]).view(np.uint8)
        out[b, 82:84] = np.array([dmin]).view(np.uint8)
    return out


@pytest.mark.parametrize("weighted", [False, True])
def test_q2k_round_trip_of_representable_blocks(weighted):
    blocks = q2k_representable(3, 24)
    x = oracle.dequant(Q2_K, blocks).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), oracle.dequant(Q2_K, blocks))  # exact in f32
    x = x.reshape(4, 6 * 256)
    imp = rng(4).uniform(0.1, 10.0, 6 * 256).astype(np.float32) if weighted else None
    got = oracle.quantize(Q2_K, x, imp)
    np.testing.assert_array_equal(got.reshape(24, 84), blocks)


def set_q2k_code(block, i, q):
    b = block.copy()
    h, s, l = i // 128, (i % 128) // 32, i % 32
    byte = 16 + 32 * h + l
    b[byte] = (int(b[byte]) & (0xFF ^ (3 << (2 * s)))) | (q << (2 * s))
    return b


def test_q2k_codes_are_nearest_for_the_stored_scales():
    # brute force through the decoder: no other code of a value decodes closer
    r = rng(5)
    x = (r.standard_normal((1, 512)) * 0.05).astype(np.float32)
    x[0, 40:56] = -0.01                       # a constant negative sub-block
    x[0, 300:316] = np.linspace(0.0, 0.2, 16)  # a non-negative ramp
    blocks = oracle.quantize(Q2_K, x).reshape(2, 84)
    for b in range(2):
        base = oracle.dequant(Q2_K, blocks[b])
        for i in range(0, 256, 3):
            xi = float(x[0, 256 * b + i])
            errs = [abs(xi - oracle.dequant(Q2_K, set_q2k_code(blocks[b], i, q))[i])
                    for q in range(4)]
            assert abs(xi - base[i]) <= min(errs) + 1e-12


def test_q2k_error_is_within_half_a_step_inside_the_range():
    # each sub-block's values inside [-dmin m, 3 d sc - dmin m] are within half
    # a step d*sc of their decoded value; a constant negative sub-block is
    # carried by its min alone, within half of dmin
    r = rng(6)
    x = (r.standard_normal((8, 256)) * 0.05).astype(np.float32)
    x[3, :16] = -0.02
    blocks = oracle.quantize(Q2_K, x).reshape(8, 84)
    y = oracle.dequant(Q2_K, blocks).reshape(8, 256)
    assert blocks[3, 0] & 15 == 0
    assert np.all(y[3, :16] == y[3, 0])
    assert abs(y[3, 0] + 0.02) <= float(blocks[3, 82:84].view(np.float16)[0]) / 2
    for b in range(8):
        d = float(blocks[b, 80:82].view(np.float16)[0])
        dm = float(blocks[b, 82:84].view(np.float16)[0])
        for j in range(16):
            sc, mn = blocks[b, j] & 15, blocks[b, j] >> 4
            lo, hi = -dm * mn, 3 * d * sc - dm * mn
            xs = x[b, 16 * j:16 * j + 16].astype(np.float64)
            inside = (xs >= lo) & (xs <= hi)
            if sc > 0:
                assert np.all(np.abs(xs - y[b, 16 * j:16 * j + 16])[inside] <= d * sc / 2 + 1e-9)


def test_q2k_power_of_two_scaling():
    # binary32 steps commute with scaling by 2^k: the same codes and nibbles,
    # d and dmin scaled; scaling the importance changes nothing
    r = rng(7)
    x = (r.standard_normal((2, 512)) * 0.05).astype(np.float32)
    imp = r.uniform(0.5, 2.0, 512).astype(np.float32)
    a = oracle.quantize(Q2_K, x, imp).reshape(4, 84)
    b = oracle.quantize(Q2_K, x * np.float32(4.0), imp).reshape(4, 84)
    c = oracle.quantize(Q2_K, x, imp * np.float32(8.0)).reshape(4, 84)
    np.testing.assert_array_equal(a[:, :80], b[:, :80])
    np.testing.assert_array_equal(a.copy()[:, 80:].view(np.float16) * 4, b.copy()[:, 80:].view(np.float16))
    np.testing.assert_array_equal(a, c)


def weighted_err(x, y, w):
    return float(np.sum(w * (x - y) ** 2))


def test_q2k_importance_lowers_the_weighted_error():
    # 4 of each 16 columns carry 50x the importance: the weighted encoder has
    # a clearly lower weighted error than the plain one, and the plain encoder
    # the lower unweighted error (each optimises its own measure)
    r = rng(8)
    x = (r.standard_normal((64, 1024)) * 0.05).astype(np.float32)
    imp = np.ones(1024, np.float32)
    imp[r.permutation(1024)[:256]] = 50.0
    yw = oracle.dequant(Q2_K, oracle.quantize(Q2_K, x, imp)).reshape(x.shape)
    yp = oracle.dequant(Q2_K, oracle.quantize(Q2_K, x)).reshape(x.shape)
    assert weighted_err(x, yw, imp) < 0.8 * weighted_err(x, yp, imp)
    assert weighted_err(x, yp, 1.0) < weighted_err(x, yw, 1.0)


def test_q2k_all_zero_and_constant_blocks():
    x = np.zeros((2, 256), np.float32)
    x[1] = 0.25
    b = oracle.quantize(Q2_K, x).reshape(2, 84)
    y = oracle.dequant(Q2_K, b).reshape(2, 256)
    assert np.all(y[0] == 0.0) and not b[0].any()
    np.testing.assert_allclose(y[1], 0.25, rtol=2e-3)   # 3 d sc with fp16 d


# --------------------------------------------------------------------------
# IQ2_XXS neighbour map
# --------------------------------------------------------------------------
def key_of(levels):
    return int(sum(int(l) * 3 ** k for k, l in enumerate(levels)))


def test_iq2_map_by_hand():
    # a three-entry grid: all-8, all-43, and 25 in the first position only
    grid = np.array([[8] * 8, [43] * 8, [25] + [8] * 7], np.uint8)
    count, idx, _ = oracle.iq2_map(grid)
    assert count[key_of([0] * 8)] == 1 and idx[key_of([0] * 8), 0] == 0          # on the grid
    assert count[key_of([2] * 8)] == 1 and idx[key_of([2] * 8), 0] == 1
    assert count[key_of([1] + [0] * 7)] == 1 and idx[key_of([1] + [0] * 7), 0] == 2
    # levels (0,1,0,...): distances 1 (entry 0), 32 (entry 1), 2 (entry 2) ->
    # two shells {1, 2}: entries 0 and 2
    k = key_of([0, 1] + [0] * 6)
    assert count[k] == 2 and list(idx[k, :2]) == [0, 2]
    # levels (2,2,2,2,2,2,2,1): distances 29, 1, 28 -> shells {1, 28}: 1 and 2
    k = key_of([2] * 7 + [1])
    assert count[k] == 2 and list(idx[k, :2]) == [1, 2]
    # levels (1,1,1,1,1,1,1,1): distances 8, 8, 7 -> shells {7, 8}: all three
    k = key_of([1] * 8)
    assert count[k] == 3 and list(idx[k, :3]) == [0, 1, 2]


def test_iq2_map_of_the_seeded_grid_by_brute_force():
    grid = ds4gen.grid(1).reshape(256, 8)
    count, idx, _ = oracle.iq2_map(grid)
    glev = np.searchsorted(LEVELS, grid)              # levels 0..2 per entry
    keys = np.arange(6561)
    lev = (keys[:, None] // 3 ** np.arange(8)) % 3    # [6561][8]
    dist = ((lev[:, None, :] - glev[None, :, :]) ** 2).sum(-1)  # [6561][256]
    for k in range(0, 6561, 7):
        dk = dist[k]
        if dk.min() == 0:
            want = [int(np.flatnonzero(dk == 0)[0])]
        else:
            u = np.unique(dk)
            want = list(np.flatnonzero(dk <= (u[1] if u.size > 1 else u[0])))
        assert count[k] == len(want) and list(idx[k, :count[k]]) == want, k
    assert count.sum() > 6561


# --------------------------------------------------------------------------
# IQ2_XXS
# --------------------------------------------------------------------------
def iq2_representable(seed, n_blocks, grid):
    """Blocks the encoder must reproduce exactly: grid entries that are the
    lowest index of their tuple, each group holding a 43, an even number of
    negatives per tuple (the format's own constraint), nibbles 0..15 with a
    15 in every block."""
    r = rng(seed)
    g = grid.reshape(256, 8)
    first = {}
    for i in range(256):
        first.setdefault(g[i].tobytes(), i)
    reps = np.array(sorted(first.values()))
    with43 = np.array([i for i in reps if (g[i] == 43).any()])
    out = np.zeros((n_blocks, 66), np.uint8)
    for b in range(n_blocks):
        d = np.float16(r.uniform(1e-4, 2e-3))
        out[b, 0:2] = np.array([d]).view(np.uint8)
        nib = r.integers(0, 16, 8)
        nib[r.integers(8)] = 15
        for grp in range(8):
            ids = r.choice(reps, 4)
            ids[r.integers(4)] = r.choice(with43)
            word = int(nib[grp]) << 28
            for u in range(4):
                s7 = int(r.integers(0, 128))
                word |= s7 << (7 * u)
            out[b, 2 + 8 * grp:6 + 8 * grp] = ids
            out[b, 6 + 8 * grp:10 + 8 * grp] = np.array([word], np.uint32).view(np.uint8)
    return out


@pytest.mark.parametrize("uniform", [True, False])
def test_iq2_round_trip_of_representable_blocks(uniform):
    grid = ds4gen.grid(1)
    blocks = iq2_representable(9, 16, grid)
    x64 = oracle.dequant(IQ2_XXS, blocks, grid=grid)
    x = x64.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), x64)
    x = x.reshape(4, 1024)
    imp = np.ones(1024, np.float32) if uniform else rng(10).uniform(0.1, 5.0, 1024).astype(np.float32)
    got = oracle.quantize(IQ2_XXS, x, imp, grid)
    np.testing.assert_array_equal(got.reshape(16, 66), blocks)


def iq2_fields(block):
    w = block[2:].reshape(8, 8)
    idx = w[:, :4]
    word = w[:, 4:].copy().view(np.uint32)[:, 0]
    return idx, word


def test_iq2_sign_parity_flips_the_least_important_value():
    # a tuple with an odd number of negatives: the decoded signs differ from
    # x's exactly at the value of smallest w x^2
    grid = ds4gen.grid(1)
    r = rng(11)
    x = (r.standard_normal((1, 256)) * 0.05).astype(np.float32)
    w = r.uniform(0.5, 2.0, 256).astype(np.float32)
    for o in range(0, 256, 8):
        neg = np.flatnonzero(x[0, o:o + 8] < 0)
        if neg.size % 2 == 0:          # make the count odd
            x[0, o] = -x[0, o] if x[0, o] != 0 else -0.01
    y = oracle.dequant(IQ2_XXS, oracle.quantize(IQ2_XXS, x, w, grid), grid=grid)
    for o in range(0, 256, 8):
        xs, ys, ws = x[0, o:o + 8], y[o:o + 8], w[o:o + 8]
        differ = np.flatnonzero(np.sign(xs) != np.sign(ys))
        score = ws * (xs * xs)
        assert differ.tolist() == [int(np.argmin(score))]


def test_iq2_chosen_entry_is_optimal_within_its_list():
    # recompute the key of each tuple at the stored scale (levels of t/S) and
    # check, through the decoder, that no entry of that list beats the choice
    grid = ds4gen.grid(1)
    count, idx, _ = oracle.iq2_map(grid)
    r = rng(13)
    x = (r.standard_normal((2, 256)) * 0.05).astype(np.float32)
    w = r.uniform(0.2, 3.0, 256).astype(np.float32)
    blocks = oracle.quantize(IQ2_XXS, x, w, grid).reshape(2, 66)
    n_multi = 0
    for b in range(2):
        blk = blocks[b]
        base = oracle.dequant(IQ2_XXS, blk, grid=grid)
        ids, word = iq2_fields(blk)
        d = np.float32(blk[0:2].view(np.float16)[0])
        for g in range(8):
            s = int(word[g] >> 28)
            S = np.float32(np.float32(d * np.float32(2 * s + 1)) / np.float32(8))
            for u in range(4):
                o = 32 * g + 8 * u
                xs = x[b, o:o + 8]
                tt = np.where(np.sign(base[o:o + 8]) < 0, -xs, xs).astype(np.float32)
                v = tt / S
                lev = np.where(v < 16.5, 0, np.where(v < 34.0, 1, 2))
                k = key_of(lev)
                lst = list(idx[k, :count[k]])
                assert int(ids[g, u]) in lst
                if len(lst) > 1:
                    n_multi += 1
                    e0 = float(np.sum(w[o:o + 8] * (xs - base[o:o + 8]) ** 2))
                    for alt in lst:
                        b2 = blk.copy()
                        b2[2 + 8 * g + u] = alt
                        y2 = oracle.dequant(IQ2_XXS, b2, grid=grid)[o:o + 8]
                        assert float(np.sum(w[o:o + 8] * (xs - y2) ** 2)) >= e0 * (1 - 1e-6)
    assert n_multi > 0


def test_iq2_power_of_two_scaling():
    grid = ds4gen.grid(1)
    r = rng(14)
    x = (r.standard_normal((2, 512)) * 0.05).astype(np.float32)
    imp = r.uniform(0.5, 2.0, 512).astype(np.float32)
    a = oracle.quantize(IQ2_XXS, x, imp, grid).reshape(4, 66)
    b = oracle.quantize(IQ2_XXS, x * np.float32(0.5), imp, grid).reshape(4, 66)
    c = oracle.quantize(IQ2_XXS, x, imp * np.float32(4.0), grid).reshape(4, 66)
    np.testing.assert_array_equal(a[:, 2:], b[:, 2:])
    np.testing.assert_array_equal(a.copy()[:, :2].view(np.float16) / 2, b.copy()[:, :2].view(np.float16))
    np.testing.assert_array_equal(a, c)


def test_iq2_importance_lowers_the_weighted_error():
    grid = ds4gen.grid(1)
    r = rng(15)
    x = (r.standard_normal((32, 1024)) * 0.05).astype(np.float32)
    imp = np.ones(1024, np.float32)
    imp[r.permutation(1024)[:256]] = 50.0
    yw = oracle.dequant(IQ2_XXS, oracle.quantize(IQ2_XXS, x, imp, grid), grid=grid).reshape(x.shape)
    yu = oracle.dequant(IQ2_XXS, oracle.quantize(IQ2_XXS, x, np.ones(1024, np.float32), grid),
                        grid=grid).reshape(x.shape)
    assert weighted_err(x, yw, imp) < 0.8 * weighted_err(x, yu, imp)
    assert weighted_err(x, yu, 1.0) < weighted_err(x, yw, 1.0)


def test_iq2_zero_groups_and_zero_importance():
    grid = ds4gen.grid(1)
    count, idx, _ = oracle.iq2_map(grid)
    x = np.zeros((1, 256), np.float32)
    x[0, 32:64] = (rng(16).standard_normal(32) * 0.05).astype(np.float32)
    blk = oracle.quantize(IQ2_XXS, x, np.ones(256, np.float32), grid)
    y = oracle.dequant(IQ2_XXS, blk, grid=grid)
    ids, word = iq2_fields(blk)
    # an all-zero group: nibble 0, no signs, every tuple the first entry of
    # the all-zero-level key; it decodes to d/8 times that entry
    assert word[0] == 0 and all(int(i) == idx[0, 0] for i in ids[0])
    assert np.abs(y[32:64] - x[0, 32:64]).max() < 0.6 * np.abs(x[0, 32:64]).max()
    # zero importance everywhere is valid and deterministic
    z = oracle.quantize(IQ2_XXS, x, np.zeros(256, np.float32), grid)
    np.testing.assert_array_equal(z, oracle.quantize(IQ2_XXS, x, np.zeros(256, np.float32), grid))


# --------------------------------------------------------------------------
# column energy, per-expert importance, errors
# --------------------------------------------------------------------------
def test_column_energy_by_hand():
    w = np.array([[[1, 2], [3, -4]], [[0.5, 0], [0, 2]]], np.float32)
    np.testing.assert_array_equal(oracle.column_energy(w), [[10, 20], [0.25, 4]])


def test_per_matrix_importance_slices():
    # importance [n_mats][cols]: matrix m uses its own vector, like separate calls
    r = rng(17)
    x = (r.standard_normal((3, 2, 512)) * 0.05).astype(np.float32)
    imp = r.uniform(0.1, 5.0, (3, 512)).astype(np.float32)
    whole = oracle.quantize(Q2_K, x, imp)
    parts = np.concatenate([oracle.quantize(Q2_K, x[m], imp[m]) for m in range(3)])
    np.testing.assert_array_equal(whole, parts)
    shared = oracle.quantize(Q2_K, x, imp[1])
    np.testing.assert_array_equal(shared[4 * 84:8 * 84], parts[4 * 84:8 * 84])  # matrix 1


def test_encoder_argument_errors():
    grid = ds4gen.grid(1)
    x = np.zeros((1, 256), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(IQ2_XXS, x, None, grid)                 # importance required
    with pytest.raises(ValueError):
        oracle.quantize(Q2_K, np.zeros((1, 200), np.float32))   # not whole blocks
    bad = x.copy()
    bad[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize(Q2_K, bad)
    with pytest.raises(ValueError):
        oracle.quantize(Q2_K, x, -np.ones(256, np.float32))
    g2 = grid.copy()
    g2[5] = 9
    with pytest.raises(ValueError):
        oracle.iq2_map(g2)


# --------------------------------------------------------------------------
# Q4_K and Q8_0 (the mixed stacks' Q4 layers and the shared expert)
# --------------------------------------------------------------------------
Q4_K, Q8_0 = oracle.Q4_K, oracle.Q8_0


def q4k_pack_scales(sc, mn):
    """The 12 scale bytes of the Q4_K layout (the decoder's reading)."""
    S = np.zeros(12, np.uint8)
    for j in range(8):
        if j < 4:
            S[j] |= sc[j]
            S[j + 4] |= mn[j]
        else:
            S[j + 4] = (sc[j] & 15) | ((mn[j] & 15) << 4)
            S[j - 4] |= (sc[j] >> 4) << 6
            S[j] |= (mn[j] >> 4) << 6
    return S


def q4k_representable(seed, n_blocks):
    """Q4_K blocks the encoder must reproduce exactly: codes 0 and 15 in every
    32-value sub-block, 6-bit scales 1..63 and mins 0..63 with a 63 of each,
    d and dmin within a factor 3 (decoded values exact in binary32)."""
    r = rng(seed)
    out = np.zeros((n_blocks, 144), np.uint8)
    for b in range(n_blocks):
        sc = r.integers(1, 64, 8)
        mn = r.integers(0, 64, 8)
        sc[r.integers(8)] = 63
        mn[r.integers(8)] = 63
        out[b, 4:16] = q4k_pack_scales(sc, mn)
        codes = r.integers(0, 16, 256)
        for j in range(8):
            p = r.permutation(32)[:2]
            codes[32 * j + p[0]] = 0
            codes[32 * j + p[1]] = 15
        for i in range(256):
            c, hi, l = i // 64, (i % 64) // 32, i % 32
            out[b, 16 + 32 * c + l] |= codes[i] << (4 * hi)
        d = np.float16(r.uniform(1e-4, 1e-3))
        dmin = np.float16(float(d) * r.uniform(0.3, 3.0))
        out[b, 0:2] = np.array([d]).view(np.uint8)
        out[b, 2:4] = np.array([dmin]).view(np.uint8)
    return out


@pytest.mark.parametrize("weighted", [False, True])
def test_q4k_round_trip_of_representable_blocks(weighted):
    blocks = q4k_representable(41, 16)
    x64 = oracle.dequant(Q4_K, blocks)
    x = x64.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), x64)
    x = x.reshape(4, 1024)
    imp = rng(42).uniform(0.1, 10.0, 1024).astype(np.float32) if weighted else None
    np.testing.assert_array_equal(oracle.quantize(Q4_K, x, imp).reshape(16, 144), blocks)


def set_q4k_code(block, i, q):
    b = block.copy()
    c, hi, l = i // 64, (i % 64) // 32, i % 32
    byte = 16 + 32 * c + l
    keep = 0x0F if hi else 0xF0
    b[byte] = (int(b[byte]) & keep) | (q << (4 * hi))
    return b


def test_q4k_codes_are_nearest_for_the_stored_scales():
    r = rng(43)
    x = (r.standard_normal((1, 256)) * 0.05).astype(np.float32)
    blk = oracle.quantize(Q4_K, x)
    base = oracle.dequant(Q4_K, blk)
    for i in range(0, 256, 5):
        errs = [abs(float(x[0, i]) - oracle.dequant(Q4_K, set_q4k_code(blk, i, q))[i])
                for q in range(16)]
        assert abs(float(x[0, i]) - base[i]) <= min(errs) + 1e-12


def test_q4k_importance_lowers_the_weighted_error():
    r = rng(44)
    x = (r.standard_normal((32, 1024)) * 0.05).astype(np.float32)
    imp = np.ones(1024, np.float32)
    imp[r.permutation(1024)[:256]] = 50.0
    yw = oracle.dequant(Q4_K, oracle.quantize(Q4_K, x, imp)).reshape(x.shape)
    yp = oracle.dequant(Q4_K, oracle.quantize(Q4_K, x)).reshape(x.shape)
    assert weighted_err(x, yw, imp) < 0.9 * weighted_err(x, yp, imp)
    assert weighted_err(x, yp, 1.0) < weighted_err(x, yw, 1.0)
    # 4-bit codes: well below the 2-bit error
    y2 = oracle.dequant(Q2_K, oracle.quantize(Q2_K, x)).reshape(x.shape)
    assert weighted_err(x, yp, 1.0) < 0.2 * weighted_err(x, y2, 1.0)


def test_q80_closed_form():
    # x = d c with |c| = 127 present: exact round trip; otherwise every value
    # within half a step d/2 of its code, d = fp16(max|x| / 127)
    r = rng(45)
    d = np.float16(3e-4)
    c = r.integers(-127, 128, (2, 256))
    c[:, ::32] = 127
    x = (np.float32(d) * c.astype(np.float32)).astype(np.float32)
    blk = oracle.quantize(Q8_0, x).reshape(16, 34)
    assert (blk[:, 0:2].copy().view(np.float16).ravel() == d).all()
    np.testing.assert_array_equal(blk[:, 2:].view(np.int8).reshape(2, 256), c)
    y = (r.standard_normal((2, 256)) * 0.05).astype(np.float32)
    b2 = oracle.quantize(Q8_0, y).reshape(16, 34)
    dd = b2[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    amax = np.abs(y.reshape(16, 32)).max(1)
    np.testing.assert_array_equal(dd, (amax / np.float32(127)).astype(np.float32).astype(np.float16))
    dec = oracle.dequant(Q8_0, b2).reshape(16, 32)
    assert np.all(np.abs(dec - y.reshape(16, 32)) <= dd[:, None] / 2 * (1 + 1e-6) + 1e-12)
