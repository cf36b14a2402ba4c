"""Exact routing where the binary64 certification cannot decide (GPU).

The router inputs of tests/route_cases.py put the sixth slot between two
experts whose keys are equal once computed exactly, while the scoring
kernel's binary64 interval of one of them spans two binary32 values: its
exact logit lies 2^-60 past a rounding midpoint inside a cancelling sum, or
its score lies within 2^-40 of one.  The selecting wave must recompute such
keys exactly (integer-limb logit, double-double score) and agree with the
oracle bit for bit, with no fault bit.  FLOW (qiita.com/sukimaengineer/items/
cd76fec76d49a098abed) § "MoE FFN 部の中身".

Paths: ds4moe_route (selection kernel), ds4moe_layer with the selection
fused into the batch-1 gate/up kernel (1 and 2 tokens), the same after an RMSNorm of the
residual stream (the router input then comes from the workspace), and a
5-token layer call (selection kernel, then the few-token matvecs).  The
constructed token sits at a non-zero row so that the per-token offsets of
the exact recomputation are exercised."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g
import oracle
import route_cases as rc
from gpu_util import TOL_FP32, check_clean, experts_of, max_rel_err, ptr, say, shape_of, stream, workspace

pytestmark = pytest.mark.gpu

W1 = g.WORKLOADS[1]


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ds4gen.device import make_layer
    return make_layer(W1, 0)


@pytest.fixture(scope="module")
def cases():
    return rc.all_cases()


def dev(a):
    from ds4gen.device import to_dev
    return to_dev(a)


def tokens_with(case, T, row):
    """T tokens of bf16 activations: seeded ones, the case's row at `row`."""
    x = g.activations(W1, n_tok=T).copy()
    x[row] = case.x_bits()
    return x


def oracle_route(case, x):
    return oracle.route(x, "bf16", case.w_bits(), "f16", case.bias, rc.K)


def check_ffn(lt, x, ids, wts, got, toks):
    from ds4gen.device import host_experts
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(W1, 0, np.unique(ids[toks])),
                          (W1.gate_qt, W1.up_qt, W1.down_qt), W1.H, W1.I, W1.E,
                          grid=g.grid(W1.seed), tokens=toks)
    err = max_rel_err(got[toks], want)
    say("  ffn max|err|/rms = %g" % err)
    assert err <= TOL_FP32


@pytest.mark.parametrize("ci", range(4), ids=["logit-up", "logit-down", "score-a", "score-b"])
def test_route_call_exact(cases, ci):
    case = cases[ci]
    say("exact route", case.name)
    T, row = 2, 1
    x = tokens_with(case, T, row)
    shp = shape_of(W1)
    ws, nb = workspace(shp, T)
    Wd, bd, xd = dev(case.w_bits()), dev(case.bias), dev(x)
    ids = torch.empty((T, rc.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, rc.K), dtype=torch.float32, device="cuda")
    r = ds4.router(w=ptr(Wd), w_dtype=ds4.F16, bias=ptr(bd))
    ds4.route(shp, r, ptr(xd), ds4.BF16, T, None, ptr(ids), ptr(wts), ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle_route(case, x)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(wts.cpu().numpy(), owts, rtol=2e-6, atol=0)
    assert oids[row, 5] == min(case.A, case.B)


@pytest.mark.parametrize("T,row", [(1, 0), (2, 1), (5, 4)], ids=["fused-1", "fused-2", "selkernel-5"])
@pytest.mark.parametrize("ci", range(4), ids=["logit-up", "logit-down", "score-a", "score-b"])
def test_layer_call_exact(layer, cases, ci, T, row):
    case = cases[ci]
    say("exact layer", case.name, "T", T)
    x = tokens_with(case, T, row)
    shp = shape_of(W1)
    ws, nb = workspace(shp, T)
    Wd, bd, xd = dev(case.w_bits()), dev(case.bias), dev(x)
    d = ds4.layer_desc(ds4.router(w=ptr(Wd), w_dtype=ds4.F16, bias=ptr(bd)), experts_of(layer, W1))
    out = torch.empty((T, W1.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, rc.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, rc.K), dtype=torch.float32, device="cuda")
    ds4.layer(shp, d, ptr(xd), ds4.BF16, None, ptr(out), None, T, ptr(ids), ptr(wts), None,
              ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle_route(case, x)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(wts.cpu().numpy(), owts, rtol=2e-6, atol=0)
    check_ffn(layer, x, oids, owts, out.cpu().numpy(), np.array([row]))


@pytest.mark.parametrize("ci", range(4), ids=["logit-up", "logit-down", "score-a", "score-b"])
def test_norm_layer_call_exact(layer, cases, ci):
    # the residual stream holds the case's values and the norm weight undoes
    # the RMS scale, so the normalised router input is the case's row exactly
    case = cases[ci]
    say("exact layer with RMSNorm", case.name)
    T, row = 2, 1
    x = tokens_with(case, T, row)
    h = (x.astype(np.uint32) << 16).view(np.float32)
    ms = np.mean(h[row].astype(np.float64) ** 2)
    nw = np.full(W1.H, np.float32(np.sqrt(ms + 1e-6)), np.float32)
    xo = oracle.rmsnorm_bf16(h, nw, 1e-6)
    np.testing.assert_array_equal(xo[row], x[row])
    shp = shape_of(W1)
    ws, nb = workspace(shp, T)
    Wd, bd, nwd = dev(case.w_bits()), dev(case.bias), dev(nw)
    d = ds4.layer_desc(ds4.router(w=ptr(Wd), w_dtype=ds4.F16, bias=ptr(bd)), experts_of(layer, W1),
                       norm_w=ptr(nwd), norm_eps=1e-6)
    resid = dev(h)
    ids = torch.empty((T, rc.K), dtype=torch.int32, device="cuda")
    xn = torch.empty((T, W1.H), dtype=torch.int16, device="cuda")
    ds4.layer(shp, d, None, ds4.BF16, ptr(resid), None, None, T, ptr(ids), None, ptr(xn), ptr(ws),
              nb, stream())
    check_clean(ws)
    np.testing.assert_array_equal(xn.cpu().numpy().view(np.uint16), xo)
    oids, owts, _, _ = oracle_route(case, xo)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    got = resid.cpu().numpy() - h
    check_ffn(layer, xo, oids, owts, got, np.array([row]))
