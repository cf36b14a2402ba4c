"""GPU block encoders against the oracle, through the C ABI: the IQ2_XXS
neighbour map and every encoded byte must match bit for bit (both sides take
each integer decision in binary32 in the same order); the column energy
within its rounding bound.  Inputs are seeded: weights N(0, 0.02) with a
sprinkle of 10x outliers (the shape of a V4-Flash expert matrix and smaller
ragged stacks), importance as squared normals (sums of squared activations),
plus edge rows (zeros, constants, tiny and wide-range values) and blocks the
format represents exactly."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g
import oracle
from gpu_util import ptr, say, stream
from test_encode_pins import iq2_representable, q2k_representable

pytestmark = pytest.mark.gpu

WS_BYTES = 256


def ws():
    return torch.zeros(WS_BYTES, dtype=torch.uint8, device="cuda")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(seed, n_mats, rows, cols):
    n = n_mats * rows * cols
    x = g.normal(seed, 40, n, 0.0, 0.02, "f32")
    pick = g.uniform_f32(seed, 41, n, 0.0, 1.0) < 0.01
    x = np.where(pick, x * np.float32(10.0), x).astype(np.float32)
    return x.reshape(n_mats, rows, cols)


def importance(seed, n_vec, cols):
    return (g.normal(seed, 42, n_vec * cols, 0.0, 1.0, "f32") ** 2).astype(np.float32).reshape(
        n_vec, cols)


def edge_rows(x):
    """Overwrite a few rows of x [n_mats][rows][cols] with edge cases."""
    x = x.copy()
    cols = x.shape[2]
    x[0, 0] = 0.0
    x[0, 1] = 0.25
    x[0, 2] = -0.01
    x[0, 3] = x[0, 3] * np.float32(1e-6)
    x[0, 4, ::7] = 50.0
    x[0, 5, : cols // 2] = np.abs(x[0, 5, : cols // 2])
    x[0, 6, 16:32] = -0.03           # one constant negative sub-block
    return x


def gpu_quantize(qt, x, imp=None, imp_stride=0, grid_d=None, map_d=None):
    n_mats, rows, cols = x.shape
    bb = {ds4.Q2_K: 84, ds4.IQ2_XXS: 66, ds4.Q4_K: 144, ds4.Q8_0: 34}[qt]
    per = 32 if qt == ds4.Q8_0 else 256
    xd = dev(x)
    impd = None if imp is None else dev(imp)
    out = torch.zeros(n_mats * rows * cols // per * bb, dtype=torch.uint8, device="cuda")
    w = ws()
    ds4.quantize(qt, ptr(xd), n_mats, rows, cols, ptr(impd), imp_stride, ptr(grid_d), ptr(map_d),
                 ptr(out), ptr(w), WS_BYTES, stream())
    faults = ds4.check(ptr(w), stream())
    return out.cpu().numpy(), faults


@pytest.fixture(scope="module")
def grid_map():
    grid = g.grid(1)
    grid_d = dev(grid)
    map_d = torch.zeros(ds4.iq2_map_bytes(), dtype=torch.uint8, device="cuda")
    w = ws()
    ds4.iq2_map_build(ptr(grid_d), ptr(map_d), ptr(w), WS_BYTES, stream())
    assert ds4.check(ptr(w), stream()) == 0
    return grid, grid_d, map_d


def test_iq2_map_matches_oracle(grid_map):
    grid, _, map_d = grid_map
    say("iq2 map")
    want = oracle.iq2_map(grid)[2]
    np.testing.assert_array_equal(map_d.cpu().numpy(), want)


def test_iq2_map_of_a_small_grid_and_a_bad_grid():
    # the hand grid of the oracle pins padded with copies of its first entry
    say("iq2 map small / bad grid")
    hand = np.array([[8] * 8, [43] * 8, [25] + [8] * 7], np.uint8)
    grid = np.concatenate([hand, np.repeat(hand[:1], 253, 0)])
    map_d = torch.zeros(ds4.iq2_map_bytes(), dtype=torch.uint8, device="cuda")
    w = ws()
    ds4.iq2_map_build(ptr(dev(grid)), ptr(map_d), ptr(w), WS_BYTES, stream())
    assert ds4.check(ptr(w), stream()) == 0
    np.testing.assert_array_equal(map_d.cpu().numpy(), oracle.iq2_map(grid)[2])
    bad = grid.copy()
    bad[100, 3] = 9
    ds4.iq2_map_build(ptr(dev(bad)), ptr(map_d), ptr(w), WS_BYTES, stream())
    assert ds4.check(ptr(w), stream()) == ds4.FAULT_BAD_INPUT


@pytest.mark.parametrize("mode", ["plain", "shared-importance", "per-matrix-importance"])
def test_q2k_ragged_stack(mode):
    x = edge_rows(weights(21, 3, 37, 512))
    imp, stride = None, 0
    if mode == "shared-importance":
        imp = importance(22, 1, 512)[0]
        imp[5:9] = 0.0
    elif mode == "per-matrix-importance":
        imp, stride = importance(23, 3, 512), 512
    say("q2k", mode, x.shape)
    got, faults = gpu_quantize(ds4.Q2_K, x, imp, stride)
    assert faults == 0
    want = oracle.quantize(oracle.Q2_K, x, imp, imp_stride=stride if imp is not None else None)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("mode", ["shared-importance", "per-matrix-importance", "zero-importance"])
def test_iq2_ragged_stack(mode, grid_map):
    grid, grid_d, map_d = grid_map
    x = edge_rows(weights(24, 3, 37, 512))
    if mode == "per-matrix-importance":
        imp, stride = importance(25, 3, 512), 512
    else:
        imp, stride = importance(26, 1, 512)[0], 0
        if mode == "zero-importance":
            imp[:] = 0.0
    say("iq2", mode, x.shape)
    got, faults = gpu_quantize(ds4.IQ2_XXS, x, imp, stride, grid_d, map_d)
    assert faults == 0
    want = oracle.quantize(oracle.IQ2_XXS, x, imp, grid, imp_stride=stride)
    np.testing.assert_array_equal(got, want)


def test_representable_blocks_round_trip(grid_map):
    grid, grid_d, map_d = grid_map
    say("representable blocks")
    qb = q2k_representable(31, 32)
    x = oracle.dequant(oracle.Q2_K, qb).astype(np.float32).reshape(1, 4, 2048)
    got, faults = gpu_quantize(ds4.Q2_K, x)
    assert faults == 0
    np.testing.assert_array_equal(got.reshape(32, 84), qb)
    ib = iq2_representable(32, 32, grid)
    x = oracle.dequant(oracle.IQ2_XXS, ib, grid=grid).astype(np.float32).reshape(1, 4, 2048)
    got, faults = gpu_quantize(ds4.IQ2_XXS, x, np.ones(2048, np.float32), 0, grid_d, map_d)
    assert faults == 0
    np.testing.assert_array_equal(got.reshape(32, 66), ib)


@pytest.mark.parametrize("qt", [ds4.Q2_K, ds4.IQ2_XXS])
def test_full_expert_matrix(qt, grid_map):
    # one V4-Flash expert matrix at full size: gate/up shape [2048][4096]
    # (IQ2_XXS) or down [4096][2048] (Q2_K), every byte compared
    grid, grid_d, map_d = grid_map
    rows, cols = (2048, 4096) if qt == ds4.IQ2_XXS else (4096, 2048)
    x = weights(27, 1, rows, cols)
    imp = importance(28, 1, cols)[0]
    say("full expert matrix", qt, (rows, cols))
    got, faults = gpu_quantize(qt, x, imp, 0, grid_d, map_d)
    assert faults == 0
    want = oracle.quantize(qt, x, imp, grid if qt == ds4.IQ2_XXS else None)
    np.testing.assert_array_equal(got, want)
    again, _ = gpu_quantize(qt, x, imp, 0, grid_d, map_d)
    np.testing.assert_array_equal(again, got)                    # deterministic


def test_bad_values_raise_the_input_fault(grid_map):
    _, grid_d, map_d = grid_map
    say("bad input faults")
    x = weights(29, 1, 2, 256)
    x[0, 1, 7] = np.inf
    _, faults = gpu_quantize(ds4.Q2_K, x)
    assert faults == ds4.FAULT_BAD_INPUT
    x = weights(29, 1, 2, 256)
    imp = np.ones(256, np.float32)
    imp[3] = -1.0
    _, faults = gpu_quantize(ds4.IQ2_XXS, x, imp, 0, grid_d, map_d)
    assert faults == ds4.FAULT_BAD_INPUT
    x[0, 0, 0] = np.nan
    _, faults = gpu_quantize(ds4.IQ2_XXS, x, np.ones(256, np.float32), 0, grid_d, map_d)
    assert faults == ds4.FAULT_BAD_INPUT


def test_column_energy():
    x = weights(30, 2, 2048, 768)
    say("column energy", x.shape)
    out = torch.zeros(2 * 768, dtype=torch.float32, device="cuda")
    ds4.column_energy(ptr(dev(x)), 2, 2048, 768, ptr(out), stream())
    got = out.cpu().numpy().reshape(2, 768)
    want = oracle.column_energy(x)
    # fp32 sum of 2048 non-negative terms with fused multiply-adds: relative
    # error below 2048 * 2^-24
    np.testing.assert_array_less(np.abs(got - want), want * 2048 * 2.0 ** -24 + 1e-30)


# --------------------------------------------------------------------------
# Q4_K and Q8_0
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["plain", "per-matrix-importance"])
def test_q4k_and_q80_ragged_stack(mode):
    x = edge_rows(weights(51, 3, 37, 512))
    imp, stride = (None, 0) if mode == "plain" else (importance(52, 3, 512), 512)
    say("q4k", mode, x.shape)
    got, faults = gpu_quantize(ds4.Q4_K, x, imp, stride)
    assert faults == 0
    want = oracle.quantize(oracle.Q4_K, x, imp, imp_stride=stride if imp is not None else None)
    np.testing.assert_array_equal(got, want)
    if mode == "plain":
        say("q80", x.shape)
        got, faults = gpu_quantize(ds4.Q8_0, x)
        assert faults == 0
        np.testing.assert_array_equal(got, oracle.quantize(oracle.Q8_0, x))


def test_q4k_representable_and_full_matrix():
    from test_encode_pins import q4k_representable
    say("q4k representable + full expert matrix")
    qb = q4k_representable(53, 32)
    x = oracle.dequant(oracle.Q4_K, qb).astype(np.float32).reshape(1, 4, 2048)
    got, faults = gpu_quantize(ds4.Q4_K, x)
    assert faults == 0
    np.testing.assert_array_equal(got.reshape(32, 144), qb)
    x = weights(54, 1, 2048, 4096)
    imp = importance(55, 1, 4096)[0]
    got, faults = gpu_quantize(ds4.Q4_K, x, imp, 0)
    assert faults == 0
    np.testing.assert_array_equal(got, oracle.quantize(oracle.Q4_K, x, imp))
    got, faults = gpu_quantize(ds4.Q8_0, x)
    assert faults == 0
    np.testing.assert_array_equal(got, oracle.quantize(oracle.Q8_0, x))
