"""Host-side checks of the C ABI: the library loads, exports every entry
point the header declares, sizes its workspace and rejects bad arguments
before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

import bit_quantized_expert_ds4moe_amd as ds4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "ds4moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(ds4moe_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ds4.LIB_PATH):
        import bit_quantized_expert_ds4moe_amd.build as b
        b.build()
    return ds4.lib()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(ds4.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_size(lib):
    s = ds4.shape(4096, 2048, 256, 6)
    one = ds4.workspace_size(s, 1)
    assert one > 0
    assert ds4.workspace_size(s, 512) > ds4.workspace_size(s, 8) > one
    assert ds4.workspace_size(ds4.shape(4000, 2048, 256, 6), 1) == 0   # hidden not /256
    assert ds4.workspace_size(ds4.shape(4096, 2048, 300, 6), 1) == 0   # > 256 experts
    assert ds4.workspace_size(ds4.shape(4096, 2048, 4, 6), 1) == 0     # top_k > n_expert


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_route_rejects_bad_arguments(lib):
    s = ds4.shape(4096, 2048, 256, 6)
    r = ds4.router(w=FAKE, w_dtype=ds4.F16, bias=FAKE)
    ws_need = ds4.workspace_size(s, 1)
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.route(s, r, FAKE, ds4.BF16, 1, None, None, FAKE, FAKE, ws_need)
    assert e.value.status == ds4.EINVAL
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.route(s, r, FAKE, ds4.BF16, 1, None, FAKE, FAKE, FAKE, ws_need - 1)
    assert e.value.status == ds4.EWORKSPACE
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.route(s, r, FAKE, 7, 1, None, FAKE, FAKE, FAKE, ws_need)
    assert e.value.status == ds4.EINVAL
    hr = ds4.router(tid2eid=FAKE, vocab=10)
    with pytest.raises(ds4.Ds4moeError) as e:  # hash layer needs token ids
        ds4.route(s, hr, None, ds4.BF16, 1, None, FAKE, FAKE, FAKE, ws_need)
    assert e.value.status == ds4.EINVAL


def test_ffn_rejects_bad_arguments(lib):
    s = ds4.shape(4096, 2048, 256, 6)
    ex = ds4.experts(FAKE, FAKE, FAKE, 2048, (ds4.IQ2_XXS, ds4.IQ2_XXS, ds4.Q2_K), grid=None)
    need = ds4.workspace_size(s, 1)
    with pytest.raises(ds4.Ds4moeError) as e:  # IQ2_XXS without grid
        ds4.expert_ffn(s, ex, None, FAKE, ds4.BF16, 1, FAKE, FAKE, FAKE, None, FAKE, need)
    assert e.value.status == ds4.EINVAL
    ex.grid = FAKE
    ex.gate = FAKE + 2  # misaligned
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.expert_ffn(s, ex, None, FAKE, ds4.BF16, 1, FAKE, FAKE, FAKE, None, FAKE, need)
    assert e.value.status == ds4.EINVAL
    ex.gate = FAKE
    ex.inter = 1024  # disagrees with the shape
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.expert_ffn(s, ex, None, FAKE, ds4.BF16, 1, FAKE, FAKE, FAKE, None, FAKE, need)
    assert e.value.status == ds4.EINVAL
    ex.inter = 2048
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.expert_ffn(s, ex, None, FAKE, ds4.BF16, 1, FAKE, FAKE, FAKE, None, FAKE, 16)
    assert e.value.status == ds4.EWORKSPACE
    big = ds4.shape(4096, 2048, 256, 64)
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.expert_ffn(big, ex, None, FAKE, ds4.BF16, 1000, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
    assert e.value.status == ds4.EUNSUPPORTED


def test_layer_and_permute_reject_bad_arguments(lib):
    s = ds4.shape(4096, 2048, 256, 6)
    ex = ds4.experts(FAKE, FAKE, FAKE, 2048, (ds4.IQ2_XXS, ds4.IQ2_XXS, ds4.Q2_K), grid=FAKE)
    d = ds4.layer_desc(ds4.router(w=FAKE, bias=FAKE), ex, norm_w=FAKE)
    need = ds4.workspace_size(s, 1)
    with pytest.raises(ds4.Ds4moeError) as e:  # norm requires a residual
        ds4.layer(s, d, None, ds4.BF16, None, None, None, 1, None, None, None, FAKE, need)
    assert e.value.status == ds4.EINVAL
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.permute(s, FAKE, 6000, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40)
    assert e.value.status == ds4.EUNSUPPORTED
    assert ds4.status_string(ds4.EDATA) == "device-detected data fault"


def test_encoder_entry_points_reject_bad_arguments(lib):
    assert ds4.iq2_map_bytes() == 6561 * 2 + 6561 * 256
    bad = [
        (7, FAKE, 1, 1, 256, None, 0, None, None, FAKE),            # type
        (ds4.Q4_K, FAKE, 1, 1, 256, None, 0, None, None, FAKE + 8), # Q4_K dst alignment
        (ds4.Q2_K, FAKE, 1, 1, 200, None, 0, None, None, FAKE),     # not whole blocks
        (ds4.Q2_K, FAKE + 4, 1, 1, 256, None, 0, None, None, FAKE), # src alignment
        (ds4.Q2_K, FAKE, 1, 1, 256, None, 0, None, None, FAKE + 2), # Q2_K dst alignment
        (ds4.Q2_K, FAKE, 1, 1, 256, FAKE, 6, None, None, FAKE),     # importance stride
        (ds4.IQ2_XXS, FAKE, 1, 1, 256, None, 0, FAKE, FAKE, FAKE),  # importance required
        (ds4.IQ2_XXS, FAKE, 1, 1, 256, FAKE, 0, None, FAKE, FAKE),  # grid required
        (ds4.IQ2_XXS, FAKE, 1, 1, 256, FAKE, 0, FAKE, None, FAKE),  # map required
        (ds4.IQ2_XXS, FAKE, 1, 1, 256, FAKE, 0, FAKE + 4, FAKE, FAKE),  # grid alignment
        (ds4.Q2_K, FAKE, -1, 1, 256, None, 0, None, None, FAKE),    # negative size
    ]
    for args in bad:
        with pytest.raises(ds4.Ds4moeError) as e:
            ds4.quantize(*args, FAKE, 256)
        assert e.value.status == ds4.EINVAL, args
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.quantize(ds4.Q2_K, FAKE, 1, 1, 256, None, 0, None, None, FAKE, FAKE, 255)
    assert e.value.status == ds4.EINVAL                              # workspace too small
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.iq2_map_build(FAKE + 1, FAKE, FAKE, 256)
    assert e.value.status == ds4.EINVAL
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.column_energy(None, 1, 1, 256, FAKE)
    assert e.value.status == ds4.EINVAL
    # empty inputs are valid and launch nothing
    ds4.quantize(ds4.Q2_K, FAKE, 0, 4, 256, None, 0, None, None, FAKE, FAKE, 256)
    ds4.column_energy(FAKE, 0, 4, 256, FAKE)
