"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Expert ids, permutations and hash lookups must match bit
for bit; outputs within max|err| <= 2e-3 * RMS(out) (fp32 accumulation)."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g
import oracle
from gpu_util import (TOL_FP32, check_clean, covering_tokens, experts_of, max_rel_err, ptr, say,
                      shape_of, shared_of, stream, workspace, x_dtype, x_fmt)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ds4.lib()
    yield
    torch.cuda.synchronize()


def dev(a):
    from ds4gen.device import to_dev
    return to_dev(a)


# --------------------------------------------------------------------------
# generator: device fill == host bytes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qt", [g.Q2_K, g.IQ2_XXS, g.Q8_0, g.Q4_K, g.Q2_K_ZM])
def test_device_fill_matches_host(qt):
    say("device fill qt", qt)
    n, first = 1000 + 37, 12345
    t = torch.empty(n * g.BLOCK_BYTES[qt], dtype=torch.uint8, device="cuda")
    g.fill_device(qt, 3, 77, first, n, t.data_ptr(), stream())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t.cpu().numpy(), g.blocks(qt, 3, 77, first, n))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def run_route(w, x, W, bias, T):
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    wdt = ds4.F32 if w.router_fmt == "f32" else ds4.F16
    r = ds4.router(w=ptr(W), w_dtype=wdt, bias=ptr(bias))
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    ds4.route(shp, r, ptr(x), x_dtype(w), T, None, ptr(ids), ptr(wts), ptr(ws), nb, stream())
    check_clean(ws)
    return ids.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("widx,T", [(0, 4), (1, 16)])
def test_route_bit_exact(widx, T):
    w = g.WORKLOADS[widx]
    say("route", w.name, "T", T)
    x = g.activations(w, n_tok=T)
    W = g.router_weight(w, 0)
    b = g.router_bias(w, 0)
    ids, wts = run_route(w, dev(x), dev(W), dev(b), T)
    oids, owts, _, _ = oracle.route(x, x_fmt(w), W, w.router_fmt, b, w.K)
    np.testing.assert_array_equal(ids, oids)
    np.testing.assert_allclose(wts, owts, rtol=2e-6, atol=0)
    assert np.allclose(wts.astype(np.float64).sum(1), 1.5, rtol=2e-6)


def test_route_ties_and_bias():
    # identical router rows give identical keys: the lower index must win,
    # and a large bias forces an expert in without changing its gate
    w = g.WORKLOADS[1]
    T = 4
    x = g.activations(w, n_tok=T)
    W = g.router_weight(w, 0).copy()
    W[200] = W[10]
    b = g.router_bias(w, 0).copy()
    b[200] = b[10]
    b[77] = 50.0
    ids, wts = run_route(w, dev(x), dev(W), dev(b), T)
    oids, owts, _, _ = oracle.route(x, "bf16", W, "f16", b, w.K)
    np.testing.assert_array_equal(ids, oids)
    assert np.all(ids[:, 0] == 77)
    np.testing.assert_allclose(wts, owts, rtol=2e-6)


def tied_router(w, near=False):
    """Router with experts 10, 74 (same lane slot set), 138 and 200 given
    identical keys that beat all others but expert 77: the order must be
    77, 10, 74, 138, 200 (equal keys go to the lower index).  With near, the
    four biases step up by two units in the last place of 30 (2^-18) with the
    expert index, so the keys differ only in their lowest bits and the order
    must be 77, 200, 138, 74, 10."""
    W = g.router_weight(w, 0).copy()
    b = g.router_bias(w, 0).copy()
    for e in (74, 138, 200):
        W[e] = W[10]
    b[[10, 74, 138, 200]] = 30.0
    if near:
        b[[10, 74, 138, 200]] += np.float32(2.0 ** -18) * np.arange(4, dtype=np.float32)
    b[77] = 50.0
    return W, b


NEAR_TIE_ORDER = [77, 200, 138, 74, 10]


@pytest.mark.parametrize("near", [False, True], ids=["equal", "near"])
def test_route_many_ties(near):
    w = g.WORKLOADS[1]
    T = 4
    x = g.activations(w, n_tok=T)
    W, b = tied_router(w, near)
    ids, wts = run_route(w, dev(x), dev(W), dev(b), T)
    oids, owts, _, _ = oracle.route(x, "bf16", W, "f16", b, w.K)
    np.testing.assert_array_equal(ids, oids)
    assert np.all(ids[:, :5] == (NEAR_TIE_ORDER if near else [77, 10, 74, 138, 200]))
    np.testing.assert_allclose(wts, owts, rtol=2e-6)


@pytest.mark.parametrize("near", [False, True], ids=["equal", "near"])
def test_layer_fused_selection_ties(near):
    """Batch-1 layer call (selection fused into the gate/up kernel) on tied
    keys, and on keys that differ only in their lowest bits."""
    from ds4gen.device import make_layer, host_experts
    w = g.WORKLOADS[1]
    say("layer fused selection ties", "near" if near else "equal")
    lt = make_layer(w, 0)
    W, b = tied_router(w, near)
    x = g.activations(w, n_tok=1)
    shp = shape_of(w)
    ws, nb = workspace(shp, 1)
    Wd, bd = dev(W), dev(b)
    d = ds4.layer_desc(ds4.router(w=ptr(Wd), w_dtype=ds4.F16, bias=ptr(bd)), experts_of(lt, w))
    out = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((1, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, w.K), dtype=torch.float32, device="cuda")
    xd = dev(x)
    ds4.layer(shp, d, ptr(xd), x_dtype(w), None, ptr(out), None, 1, ptr(ids), ptr(wts), None,
              ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle.route(x, "bf16", W, "f16", b, w.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    assert list(oids[0, :5]) == (NEAR_TIE_ORDER if near else [77, 10, 74, 138, 200])
    np.testing.assert_allclose(wts.cpu().numpy(), owts, rtol=2e-6)
    want = oracle.moe_ffn(x, "bf16", oids, owts, host_experts(w, 0, np.unique(oids)),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed))
    err = max_rel_err(out.cpu().numpy(), want)
    say("  max|err|/rms =", err)
    assert err <= TOL_FP32


def test_hash_route_is_table_lookup():
    w = g.WORKLOADS[4]
    say("hash route")
    table = g.hash_table(w, 1)
    tok = g.token_ids(w, 64)
    shp = shape_of(w)
    ws, nb = workspace(shp, 64)
    tabd = dev(table)
    r = ds4.router(tid2eid=ptr(tabd), vocab=w.vocab)
    tokd = dev(tok)
    ids = torch.empty((64, 6), dtype=torch.int32, device="cuda")
    wts = torch.empty((64, 6), dtype=torch.float32, device="cuda")
    ds4.route(shp, r, None, ds4.BF16, 64, ptr(tokd), ptr(ids), ptr(wts), ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts = oracle.route_hash(tok, table, 256, 6)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_array_equal(wts.cpu().numpy(), owts)
    # a token id out of range is reported and routed to experts 0..5
    bad = dev(np.array([w.vocab + 5, -1], np.int32))
    ds4.route(shp, r, None, ds4.BF16, 2, ptr(bad), ptr(ids), ptr(wts), ptr(ws), nb, stream())
    f = ds4.check(ptr(ws), stream())
    assert f & ds4.FAULT_BAD_TOKEN
    np.testing.assert_array_equal(ids.cpu().numpy()[:2], [list(range(6))] * 2)


@pytest.mark.parametrize("T", [1, 3])
def test_layer_norm_hash_one_launch(T):
    """Hash-routed layer with an RMSNorm: one launch normalises the residual and
    routes by the table.  ids and the normalised row are bit-exact against
    the oracle, the output within tolerance; a bad token id in the same
    launch raises BAD_TOKEN and routes to experts 0..5."""
    from ds4gen.device import make_layer, host_experts, step_inputs, to_dev
    w = g.WORKLOADS[4]
    say("layer norm + hash", "T", T)
    lt = make_layer(w, 0, hashed=True, norm=True)
    h0, tok = step_inputs(w, T, first_step=11)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    d = ds4.layer_desc(ds4.router(tid2eid=ptr(lt.tid2eid), vocab=w.vocab), experts_of(lt, w),
                       norm_w=ptr(lt.norm_w), norm_eps=1e-6)
    resid = to_dev(h0)
    tokd = to_dev(tok)
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    xn = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    ds4.layer(shp, d, None, ds4.BF16, ptr(resid), None, ptr(tokd), T, ptr(ids), ptr(wts), ptr(xn),
              ptr(ws), nb, stream())
    check_clean(ws)
    table = lt.tid2eid.cpu().numpy()
    oids, owts = oracle.route_hash(tok, table, w.E, w.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_array_equal(wts.cpu().numpy(), owts)
    nw = lt.norm_w.cpu().numpy()
    oxn = oracle.rmsnorm_bf16(h0, nw, 1e-6)
    np.testing.assert_array_equal(xn.cpu().numpy().view(np.uint16), oxn)
    y = oracle.moe_ffn(oxn, "bf16", oids, owts, host_experts(w, 0, np.unique(oids)),
                       (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed))
    want = oracle.residual_add(h0, y)
    err = max_rel_err(resid.cpu().numpy() - h0, want - h0)
    say("  max|err|/rms =", err)
    assert err <= TOL_FP32
    # a token id out of range: reported, routed to experts 0..5, nothing else breaks
    bad = tok.copy()
    bad[0] = w.vocab + 5
    tokd = to_dev(bad)
    resid = to_dev(h0)
    ds4.layer(shp, d, None, ds4.BF16, ptr(resid), None, ptr(tokd), T, ptr(ids), ptr(wts), None,
              ptr(ws), nb, stream())
    f = ds4.check(ptr(ws), stream())
    assert f & ds4.FAULT_BAD_TOKEN
    np.testing.assert_array_equal(ids.cpu().numpy()[0], list(range(6)))
    if T > 1:
        np.testing.assert_array_equal(ids.cpu().numpy()[1:], oids[1:])


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 8, 512, 2000])
def test_permute_bit_exact(T):
    say("permute T", T)
    ids, _ = g.zipf_routing(3, T, 256, 6)
    shp = ds4.shape(4096, 2048, 256, 6)
    ws, nb = workspace(shp, T)
    idd = dev(ids)
    counts = torch.empty(256, dtype=torch.int32, device="cuda")
    offs = torch.empty(257, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * 6, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * 6, dtype=torch.int32, device="cuda")
    ds4.permute(shp, ptr(idd), T, ptr(counts), ptr(offs), ptr(perm), ptr(inv), ptr(ws), nb, stream())
    check_clean(ws)
    oc, oo, op, oi = oracle.permute(ids, 256)
    np.testing.assert_array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_array_equal(offs.cpu().numpy(), oo)
    np.testing.assert_array_equal(perm.cpu().numpy(), op)
    np.testing.assert_array_equal(inv.cpu().numpy(), oi)


def test_permute_flags_bad_id():
    shp = ds4.shape(4096, 2048, 256, 6)
    ws, nb = workspace(shp, 1)
    idd = dev(np.array([[1, 2, 300, 4, 5, 6]], np.int32))
    bufs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (256, 257, 6, 6)]
    ds4.permute(shp, ptr(idd), 1, *[ptr(b) for b in bufs], ptr(ws), nb, stream())
    assert ds4.check(ptr(ws), stream()) & ds4.FAULT_BAD_ID


# --------------------------------------------------------------------------
# expert FFN
# --------------------------------------------------------------------------
def ffn_case(widx, T, tokens_for_oracle=None, given=None):
    from ds4gen.device import make_layer, host_experts, host_shared
    w = g.WORKLOADS[widx]
    say("ffn", w.name, "T", T)
    lt = make_layer(w, 0)
    x = g.activations(w, n_tok=T)
    if given is None:
        ids, wts, _, _ = oracle.route(x, x_fmt(w), g.router_weight(w, 0), w.router_fmt,
                                      g.router_bias(w, 0), w.K)
    else:
        ids, wts = given
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), shared_of(lt, w), ptr(xd), x_dtype(w), T, ptr(idd),
                   ptr(wd), ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    got = out.cpu().numpy()
    toks = np.arange(T) if tokens_for_oracle is None else np.asarray(tokens_for_oracle)
    used = np.unique(ids[toks])
    sh = host_shared(w, 0) if w.shared else None
    want = oracle.moe_ffn(x, x_fmt(w), ids, wts, host_experts(w, 0, used),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E,
                          grid=g.grid(w.seed), tokens=toks, shared=sh, sh_I=w.I)
    err = max_rel_err(got[toks], want)
    say("  max|err|/rms =", err)
    return err


def test_ffn_tiny_q2k():
    assert ffn_case(0, 4) <= TOL_FP32


def test_ffn_v4_decode_b1():
    assert ffn_case(1, 1) <= TOL_FP32


@pytest.mark.parametrize("T", [2, 3, 4, 5])
def test_ffn_v4_decode_few_tokens(T):
    # the matvec kernels with one grid row per token: the down kernel's
    # per-wave SwiGLU reads up to 4 tokens, LDS staging from 5; every output
    assert ffn_case(1, T) <= TOL_FP32


@pytest.mark.parametrize("tok", [1, 2, 3])
def test_ffn_v4_decode_b1_more_tokens(tok):
    from ds4gen.device import make_layer, host_experts
    w = g.WORKLOADS[1]
    lt = make_layer(w, 0)
    x = g.activations(w, n_tok=1, first_tok=tok)
    ids, wts, _, _ = oracle.route(x, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0), 6)
    shp = shape_of(w)
    ws, nb = workspace(shp, 1)
    out = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, 1, ptr(idd), ptr(wd), ptr(out),
                   None, ptr(ws), nb, stream())
    check_clean(ws)
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, ids[0]),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed))
    err = max_rel_err(out.cpu().numpy(), want)
    say("  token", tok, "max|err|/rms =", err)
    assert err <= TOL_FP32


def test_ffn_v4_decode_b8_shared_q8():
    assert ffn_case(2, 8) <= TOL_FP32


@pytest.mark.parametrize("T", [1, 4, 5, 17, 64])
def test_ffn_v4_decode_batch_shared_split(T):
    # the Q8_0 shared expert as per-token matvecs after the routed matvec
    # kernels (1 and 4 tokens), alone through the grouped kernels after them
    # (5 tokens: its single item split along K, 16 and 4 shares), and just
    # past the few-token path (routed experts through the grouped kernels too)
    assert ffn_case(2, T, tokens_for_oracle=sorted({0, T // 2, T - 1})) <= TOL_FP32


@pytest.mark.parametrize("T", [1, 3])
def test_layer_norm_residual_with_shared_expert(T):
    # a stack-style layer call (RMSNorm of the fp32 residual stream, learned
    # routing, residual += output) with the Q8_0 shared expert: the shared
    # matvec kernels add into the residual
    from ds4gen.device import make_layer, host_experts, host_shared, step_inputs
    from dataclasses import replace
    w = replace(g.WORKLOADS[2], T=T)
    say("layer norm + residual + shared T", T)
    lt = make_layer(w, 0, norm=True)
    h0, _ = step_inputs(w, T)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    d = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                       experts_of(lt, w), shared=shared_of(lt, w), norm_w=ptr(lt.norm_w),
                       norm_eps=1e-6)
    resid = dev(h0)
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    xn = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    ds4.layer(shp, d, None, ds4.BF16, ptr(resid), None, None, T, ptr(ids), None, ptr(xn), ptr(ws),
              nb, stream())
    check_clean(ws)
    xo = oracle.rmsnorm_bf16(h0, g.norm_weight(w, 0), 1e-6)
    np.testing.assert_array_equal(xn.cpu().numpy().view(np.uint16), xo)
    oids, owts, _, _ = oracle.route(xo, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0),
                                    w.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    y = oracle.moe_ffn(xo, "bf16", oids, owts, host_experts(w, 0, np.unique(oids)),
                       (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                       shared=host_shared(w, 0), sh_I=w.I)
    err = max_rel_err(resid.cpu().numpy() - h0, y)
    say("  max|err|/rms = %g" % err)
    assert err <= TOL_FP32


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
Q4_LAYER = g.Workload("v4flash-layer-q4k", 33, 1, 4096, 2048, 256, 6, g.Q4_K, g.Q4_K, g.Q4_K,
                      "bf16", "f16")
MIXED_LAYER = g.Workload("v4flash-layer-iq2-q4k-down", 34, 1, 4096, 2048, 256, 6, g.IQ2_XXS,
                         g.IQ2_XXS, g.Q4_K, "bf16", "f16")


def _layer_workload(widx):
    from dataclasses import replace
    if widx == "q4k":
        return Q4_LAYER
    if widx == "mixed":
        return MIXED_LAYER
    if widx == "q4k-t3":
        return replace(Q4_LAYER, T=3)
    if widx == "q4k-shared-t2":
        return replace(Q4_LAYER, T=2, shared=True)
    if widx == "q4k-shared-t6":
        return replace(Q4_LAYER, T=6, shared=True)
    if isinstance(widx, str) and widx.startswith("b8-t"):
        return replace(g.WORKLOADS[2], T=int(widx[4:]))
    return g.WORKLOADS[widx]


@pytest.mark.parametrize("widx", [0, 1, "q4k", "mixed", "q4k-t3", "q4k-shared-t2", "q4k-shared-t6", 2,
                                  "b8-t1", "b8-t2", "b8-t3", "b8-t5", "b8-t7", "b8-t10", "b8-t13",
                                  "b8-t14"])
def test_layer_route_and_ffn(widx):
    # configs 0, 1 and 2; the config-1 layer with Q4_K experts (1 and 3
    # tokens, and 2 and 6 with a Q8_0 shared expert) and with IQ2_XXS gate/up
    # and Q4_K down; with a shared expert up to 10 tokens its gate/up runs in
    # the scoring launch; config 2 (Q8_0 shared expert) at 1 and 2 tokens (few-token
    # kernels, the top-6 selection of each token fused into gate/up, shared
    # expert per token), 3 (the same, shared expert read once for all
    # tokens), 5, 7, 8 and 10 (selection kernel listing the distinct experts,
    # gate/up reading each once; 10 tokens: three rows of the shared
    # kernels), 13 and 14 (grouped kernels: at most 16 rows per item, so the
    # small-item kernels alone)
    from ds4gen.device import make_layer, host_experts, host_shared
    w = _layer_workload(widx)
    say("layer", w.name, "T", w.T)
    T = w.T
    lt = make_layer(w, 0)
    x = g.activations(w, n_tok=T)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    wdt = ds4.F32 if w.router_fmt == "f32" else ds4.F16
    d = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=wdt, bias=ptr(lt.bias)),
                       experts_of(lt, w), shared=shared_of(lt, w))
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    xd = dev(x)
    ds4.layer(shp, d, ptr(xd), x_dtype(w), None, ptr(out), None, T, ptr(ids), ptr(wts), None,
              ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle.route(x, x_fmt(w), g.router_weight(w, 0), w.router_fmt,
                                    g.router_bias(w, 0), w.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(wts.cpu().numpy(), owts, rtol=2e-6)
    want = oracle.moe_ffn(x, x_fmt(w), oids, owts, host_experts(w, 0, np.unique(oids)),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          shared=host_shared(w, 0) if w.shared else None, sh_I=w.I)
    err = max_rel_err(out.cpu().numpy(), want)
    say("  max|err|/rms =", err)
    assert err <= TOL_FP32


@pytest.mark.parametrize("T", [9, 10])
def test_layer_identical_tokens(T):
    # config 2's layer with every token equal: all T tokens pick the same six
    # experts, so each distinct-expert item holds T pairs (the gate/up passes
    # of 4, 4 and 1 or 2 tokens) and the shared expert runs three grid rows
    from ds4gen.device import make_layer, host_experts, host_shared
    from dataclasses import replace
    w = replace(g.WORKLOADS[2], T=T)
    say("layer, identical tokens, T", T)
    lt = make_layer(w, 0)
    x = np.repeat(g.activations(w, n_tok=1), T, axis=0)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    d = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                       experts_of(lt, w), shared=shared_of(lt, w))
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    xd = dev(x)
    ds4.layer(shp, d, ptr(xd), ds4.BF16, None, ptr(out), None, T, ptr(ids), ptr(wts), None,
              ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle.route(x, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0), w.K)
    assert np.unique(oids).size == w.K
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    want = oracle.moe_ffn(x[:1], "bf16", oids[:1], owts[:1], host_experts(w, 0, np.unique(oids)),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          shared=host_shared(w, 0), sh_I=w.I)
    got = out.cpu().numpy()
    for t in range(T):
        err = max_rel_err(got[t:t + 1], want)
        assert err <= TOL_FP32, (t, err)
    # every token's row is computed from the same values in the same order
    assert (got == got[:1]).all()


@pytest.mark.parametrize("widx", [1, "q4k-t3", "b8-t2"])
def test_ffn_nonfinite_activation_propagates(widx):
    # a NaN (token 1) or an infinity (token 2) in x makes that token's whole
    # output NaN, as the exact products would (every down row sums over every
    # SwiGLU value); the other tokens are unaffected and no fault bit is set.
    # Paths: IQ2_XXS/Q2_K matvecs (3 tokens), Q4_K matvecs (3 tokens), and the
    # Q8_0 shared expert's matvecs (2 tokens)
    from dataclasses import replace
    from ds4gen.device import make_layer, host_experts, host_shared
    w = _layer_workload(widx)
    if widx == 1:
        w = replace(w, T=3)
    T = w.T
    say("non-finite x", w.name, "T", T)
    lt = make_layer(w, 0)
    x = g.activations(w, n_tok=T)
    ids, wts, _, _ = oracle.route(x, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0), w.K)
    bad = x.copy()
    bad[1, 100] = 0x7FC0            # bf16 quiet NaN
    if T > 2:
        bad[2, 3000] = 0xFF80       # bf16 -Inf
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(bad), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), shared_of(lt, w), ptr(xd), ds4.BF16, T, ptr(idd),
                   ptr(wd), ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    got = out.cpu().numpy()
    assert np.isnan(got[1:]).all()
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids[0])),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=[0], shared=host_shared(w, 0) if w.shared else None, sh_I=w.I)
    err = max_rel_err(got[:1], want)
    say("  clean token max|err|/rms =", err)
    assert err <= TOL_FP32


def test_layer_one_token_calls_in_sequence():
    """Consecutive one-token layer calls on one workspace (scoring kernel,
    selection fused into gate/up, down), each with its own token, must each
    select exactly the oracle's experts and gates: nothing a call leaves in
    the workspace may leak into the next."""
    from ds4gen.device import make_layer, host_experts
    w = g.WORKLOADS[1]
    say("one-token calls in sequence")
    lt = make_layer(w, 0)
    T = 8
    xh = g.activations(w, n_tok=T)
    x = dev(xh)
    shp = shape_of(w)
    ws, nb = workspace(shp, 1)
    d = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                       experts_of(lt, w))
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    for i in range(T):
        ds4.layer(shp, d, x.data_ptr() + i * w.H * 2, ds4.BF16, None, out.data_ptr() + i * w.H * 4,
                  None, 1, ids.data_ptr() + i * w.K * 4, wts.data_ptr() + i * w.K * 4, None,
                  ptr(ws), nb, stream())
    check_clean(ws)
    oids, owts, _, _ = oracle.route(xh, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0), w.K)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(wts.cpu().numpy(), owts, rtol=2e-6, atol=0)
    toks = np.array([0, T - 1])
    want = oracle.moe_ffn(xh, "bf16", oids, owts, host_experts(w, 0, np.unique(oids[toks])),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=toks)
    err = max_rel_err(out.cpu().numpy()[toks], want)
    say("  max|err|/rms = %g" % err)
    assert err <= TOL_FP32


def test_layer_graph_replays_match_eager():
    """Captured layer calls replayed several times, with eager work and
    synchronisations in between, must reproduce the eager results bit for bit."""
    from ds4gen.device import make_layer
    w = g.WORKLOADS[1]
    say("graph replay")
    lt = make_layer(w, 0)
    T = 6
    x = dev(g.activations(w, n_tok=T))
    shp = shape_of(w)
    ws, nb = workspace(shp, 1)
    d = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                       experts_of(lt, w))
    ref = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, w.H), dtype=torch.float32, device="cuda")
    row = w.H * 2

    def run(dst, st):
        for i in range(T):
            ds4.layer(shp, d, x.data_ptr() + i * row, ds4.BF16, None, dst.data_ptr() + i * w.H * 4,
                      None, 1, None, None, None, ptr(ws), nb, st)

    run(ref, stream())
    check_clean(ws)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        run(out, torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs" % rep
        run(ref, stream())  # eager work between replays
        torch.cuda.synchronize()
    check_clean(ws)


# --------------------------------------------------------------------------
# grouped (several tokens per expert) path
# --------------------------------------------------------------------------
def grouped_case(w, ids, wts, tokens_for_oracle=None, tol=TOL_FP32):
    from ds4gen.device import make_layer, host_experts, host_shared
    lt = make_layer(w, 0)
    T = ids.shape[0]
    x = g.activations(w, n_tok=T)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    pdbg = torch.empty(w.E + 1 + 2 * T * w.K, dtype=torch.int32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), shared_of(lt, w), ptr(xd), x_dtype(w), T, ptr(idd),
                   ptr(wd), ptr(out), ptr(pdbg), ptr(ws), nb, stream())
    check_clean(ws)
    _, oo, op, oi = oracle.permute(ids, w.E)
    pd = pdbg.cpu().numpy()
    np.testing.assert_array_equal(pd[:w.E + 1], oo)
    np.testing.assert_array_equal(pd[w.E + 1:w.E + 1 + T * w.K], op)
    np.testing.assert_array_equal(pd[w.E + 1 + T * w.K:], oi)
    toks = np.arange(T) if tokens_for_oracle is None else np.asarray(tokens_for_oracle)
    sh = host_shared(w, 0) if w.shared else None
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids[toks])),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=toks, shared=sh, sh_I=w.I)
    err = max_rel_err(out.cpu().numpy()[toks], want)
    say("  grouped T=%d max|err|/rms = %g" % (T, err))
    assert err <= tol


def test_grouped_ragged_items_all_outputs():
    # 12 experts, 150 tokens x top-4: several experts get > 64 pairs (multiple
    # work items, ragged last tile); shared Q8_0 expert; every output checked
    w = g.Workload("grouped-small", 11, 150, 512, 256, 12, 4, g.IQ2_XXS, g.IQ2_XXS, g.Q2_K,
                   "bf16", "f16", shared=True)
    say("grouped ragged")
    ids, wts = g.zipf_routing(11, w.T, w.E, w.K)
    grouped_case(w, ids, wts)


def test_grouped_prefill_512_zipf_every_expert():
    # the prefill workload: 512 tokens, 256 experts, Zipf(1.1) routing; every
    # output of a set of tokens whose routes cover all touched experts (about
    # 108 tokens for the 246 experts) and of the first and last token
    w = g.WORKLOADS[3]
    ids, wts = g.zipf_routing(w.seed, w.T, w.E, w.K)
    toks = covering_tokens(ids, extra=(0, w.T - 1))
    say("prefill 512: %d tokens cover %d experts" % (toks.size, np.unique(ids).size))
    grouped_case(w, ids, wts, tokens_for_oracle=toks, tol=TOL_FP32)


def _grouped_fast_case(zero_d):
    # hidden 512, inter 512: both pipelined kernels (IQ2_XXS gate/up with four
    # 128-column stages, Q2_K down with four), 160 tokens x top-4 over 16
    # experts with Zipf(1.1) routing: items of 64 rows, ragged last pieces and
    # small items (at most 16 rows); every output checked.  zero_d: every
    # third gate/up block and every third down block has d = 0 (a block of
    # zeros in the main term; the down mins still count), every fifth down
    # block dmin = 0.
    from ds4gen.device import make_layer, host_experts
    w = g.Workload("grouped-fast", 13, 160, 512, 512, 16, 4, g.IQ2_XXS, g.IQ2_XXS, g.Q2_K,
                   "bf16", "f16")
    lt = make_layer(w, 0)
    ids, wts = g.zipf_routing(13, w.T, w.E, w.K)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert (counts > 64).any() and ((counts > 0) & (counts <= 16)).any()
    assert ((counts > 64) & (counts % 64 > 0) & (counts % 64 <= 16)).any()
    bpe = w.blocks_per_expert

    def patch(a, nbytes, views):
        v = a.reshape(-1, nbytes)
        for rows, lo, hi in views:
            v[rows, lo:hi] = 0

    iq2_z = [(slice(1, None, 3), 0, 2)]
    q2k_z = [(slice(1, None, 3), 80, 82), (slice(2, None, 5), 82, 84)]
    if zero_d:
        for t, nbytes, views in ((lt.gate, 66, iq2_z), (lt.up, 66, iq2_z), (lt.down, 84, q2k_z)):
            tv = t.view(w.E, -1)
            for e in range(w.E):
                row = tv[e].view(-1, nbytes)
                for rows, lo, hi in views:
                    row[rows, lo:hi] = 0
    hx = host_experts(w, 0, np.unique(ids))
    if zero_d:
        for e in hx:
            gb, ub, db = (np.array(a, copy=True) for a in hx[e])
            patch(gb, 66, iq2_z)
            patch(ub, 66, iq2_z)
            patch(db, 84, q2k_z)
            assert gb.size == bpe["gate"] * 66 and db.size == bpe["down"] * 84
            hx[e] = (gb, ub, db)
    x = g.activations(w, n_tok=w.T)
    shp = shape_of(w)
    ws, nb = workspace(shp, w.T)
    out = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), x_dtype(w), w.T, ptr(idd), ptr(wd),
                   ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    want = oracle.moe_ffn(x, "bf16", ids, wts, hx, (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I,
                          w.E, grid=g.grid(w.seed), tokens=np.arange(w.T))
    err = max_rel_err(out.cpu().numpy(), want)
    say("  grouped-fast zero_d=%d max|err|/rms = %g" % (zero_d, err))
    assert err <= TOL_FP32


def test_grouped_pipelined_kernels_all_outputs():
    say("grouped pipelined kernels")
    _grouped_fast_case(False)


def test_grouped_pipelined_kernels_zero_scales():
    say("grouped pipelined kernels, d = 0 blocks")
    _grouped_fast_case(True)


@pytest.mark.parametrize("mag", [0.0, 200.0])
@pytest.mark.parametrize("gu", ["q4k", "iq2"])
def test_grouped_q4k_down_all_outputs(gu, mag):
    # the pipelined Q4_K down (hidden 512, inter 512: four 128-column stages,
    # two Q4_K blocks per row) behind the Q4_K gate/up (one binary16 exponent
    # per 64 features) and behind the pipelined IQ2_XXS gate/up (one per 128):
    # 160 tokens x top-4 over 16 experts, Zipf(1.1) routing, so 64-row items,
    # ragged pieces and small items; every output checked.  mag > 0: eight
    # channels of every token at +-mag, which puts |h| of every 64-feature
    # range above 2^11, at maxima between 2^12 and 2^16: the items' ranges
    # take different power-of-two exponents and the accumulators follow them
    # from chunk to chunk.
    from ds4gen.device import make_layer, host_experts
    qts = (g.Q4_K, g.Q4_K, g.Q4_K) if gu == "q4k" else (g.IQ2_XXS, g.IQ2_XXS, g.Q4_K)
    w = g.Workload("grouped-q4k", 17, 160, 512, 512, 16, 4, *qts, "bf16", "f16")
    say("grouped q4k down, gate/up %s, outliers %g" % (gu, mag))
    lt = make_layer(w, 0)
    ids, wts = g.zipf_routing(17, w.T, w.E, w.K)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert (counts > 64).any() and ((counts > 0) & (counts <= 16)).any()
    x = outlier_x(w, w.T, mag) if mag else g.activations(w, n_tok=w.T)
    shp = shape_of(w)
    ws, nb = workspace(shp, w.T)
    out = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, w.T, ptr(idd), ptr(wd),
                   ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids)), qts, w.H, w.I,
                          w.E, grid=g.grid(w.seed), tokens=np.arange(w.T))
    err = max_rel_err(out.cpu().numpy(), want)
    say("  max|err|/rms = %g" % err)
    assert err <= TOL_FP32


# --------------------------------------------------------------------------
# importance statistics (ds4moe_expert_ffn_imatrix)
# --------------------------------------------------------------------------
def _imatrix_case(w, T, ids=None, wts=None, lt=None):
    from ds4gen.device import make_layer, host_experts
    lt = make_layer(w, 0) if lt is None else lt
    x = g.activations(w, n_tok=T)
    if ids is None:
        ids, wts, _, _ = oracle.route(x, x_fmt(w), g.router_weight(w, 0), w.router_fmt,
                                      g.router_bias(w, 0), w.K)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    gu = torch.zeros((w.E, w.H), dtype=torch.float32, device="cuda")
    dn = torch.zeros((w.E, w.I), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    for rep in range(2):  # the second call adds the same sums again
        ds4.expert_ffn_imatrix(shp, experts_of(lt, w), shared_of(lt, w), ptr(xd), x_dtype(w), T,
                               ptr(idd), ptr(wd), ptr(out), ptr(gu), ptr(dn), ptr(ws), nb, stream())
        check_clean(ws)
        if rep == 0:
            gu1, dn1 = gu.cpu().numpy().copy(), dn.cpu().numpy().copy()
    gu2, dn2 = gu.cpu().numpy(), dn.cpu().numpy()
    np.testing.assert_array_equal(gu2, 2 * gu1)
    np.testing.assert_array_equal(dn2, 2 * dn1)
    hx = host_experts(w, 0, np.unique(ids))
    want_gu, want_dn = oracle.imatrix(x, x_fmt(w), ids, wts, hx, (w.gate_qt, w.up_qt), w.H, w.I,
                                      w.E, grid=g.grid(w.seed))
    np.testing.assert_allclose(gu1, want_gu, rtol=2e-7, atol=0)
    err = np.abs(dn1 - want_dn).max() / np.sqrt((want_dn ** 2).mean())
    say("  imatrix %s T=%d: down max|err|/rms = %g" % (w.name, T, err))
    assert err <= TOL_FP32
    assert (want_dn[np.unique(ids)] > 0).all() and not want_dn[np.setdiff1d(np.arange(w.E), ids)].any()
    return lt


def test_imatrix_decode_paths():
    # matvec kernels (4 tokens of config 1), the same with a Q8_0 shared expert
    # (config 2, 8 tokens: the shared expert's rows reuse the routed rows'
    # memory after the statistics), the generic kernels (config 0, f32 x)
    say("imatrix decode")
    _imatrix_case(g.WORKLOADS[1], 4)
    _imatrix_case(g.WORKLOADS[2], 8)
    _imatrix_case(g.WORKLOADS[0], 4)


def test_imatrix_grouped_path():
    say("imatrix grouped")
    w = g.Workload("grouped-fast", 13, 160, 512, 512, 16, 4, g.IQ2_XXS, g.IQ2_XXS, g.Q2_K,
                   "bf16", "f16")
    ids, wts = g.zipf_routing(13, w.T, w.E, w.K)
    _imatrix_case(w, w.T, ids, wts)


# --------------------------------------------------------------------------
# Q4_K experts (generic kernels)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 5, 40, 512])
def test_ffn_q4k_experts(T):
    # V4-Flash expert shape with gate/up/down all in Q4_K, and the mixed form
    # (IQ2_XXS gate/up, Q4_K down): the matvec kernels at 1 and 5 tokens
    # (learned routing), the grouped MFMA kernels at 40 (learned routing) and
    # 512 (Zipf-routed prefill); above 5 tokens every output of tokens that
    # together cover every touched expert
    for qts in ((g.Q4_K, g.Q4_K, g.Q4_K), (g.IQ2_XXS, g.IQ2_XXS, g.Q4_K)):
        w = g.Workload("q4k", 31, T, 4096, 2048, 256, 6, *qts, "bf16", "f16")
        say("ffn q4k", qts, "T", T)
        from ds4gen.device import make_layer, host_experts
        lt = make_layer(w, 0)
        x = g.activations(w, n_tok=T)
        if T == 512:
            ids, wts = g.zipf_routing(31, T, w.E, w.K)
        else:
            ids, wts, _, _ = oracle.route(x, x_fmt(w), g.router_weight(w, 0), w.router_fmt,
                                          g.router_bias(w, 0), w.K)
        shp = shape_of(w)
        ws, nb = workspace(shp, T)
        out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
        xd, idd, wd = dev(x), dev(ids), dev(wts)
        ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), x_dtype(w), T, ptr(idd), ptr(wd),
                       ptr(out), None, ptr(ws), nb, stream())
        check_clean(ws)
        if T <= 5:
            toks = np.arange(min(T, 2))
        else:  # every touched expert through at least one checked token
            toks = covering_tokens(ids, extra=(0, T - 1))
        want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids[toks])), qts,
                              w.H, w.I, w.E, grid=g.grid(w.seed), tokens=toks)
        err = max_rel_err(out.cpu().numpy()[toks], want)
        say("  max|err|/rms = %g" % err)
        assert err <= TOL_FP32


# --------------------------------------------------------------------------
# activation outliers
# --------------------------------------------------------------------------
def outlier_x(w, T, mag, seed=7):
    """bf16 activations N(0,1) with eight channels of every token set to
    +-mag (as hidden states with a few large channels have)."""
    x = g.activations(w, n_tok=T).copy()
    rng = np.random.default_rng(seed)
    ch = rng.choice(w.H, 8, replace=False)
    sign = rng.choice([-1.0, 1.0], (T, 8))
    vals = (sign * mag).astype(np.float32)
    x[:, ch] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    return x


@pytest.mark.parametrize("mag", [200.0, 3000.0])
@pytest.mark.parametrize("T", [1, 8, 40, 512])
def test_ffn_activation_outliers(T, mag):
    # matvec kernels (1, 8 tokens) and grouped MFMA kernels (40, 512 tokens):
    # every output of tokens covering all touched experts within 2e-3 * RMS,
    # no fault bit
    from ds4gen.device import make_layer, host_experts
    w = g.WORKLOADS[1]
    say("outliers +-%g T %d" % (mag, T))
    lt = make_layer(w, 0)
    x = outlier_x(w, T, mag)
    if T == 512:
        ids, wts = g.zipf_routing(w.seed, T, w.E, w.K)
    else:
        ids, wts, _, _ = oracle.route(x, "bf16", g.router_weight(w, 0), "f16", g.router_bias(w, 0),
                                      w.K)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, T, ptr(idd), ptr(wd),
                   ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    toks = covering_tokens(ids, extra=(0, T - 1))
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids[toks])),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=toks)
    err = max_rel_err(out.cpu().numpy()[toks], want)
    say("  max|err|/rms = %g (rms %g)" % (err, np.sqrt(np.mean(want.astype(np.float64) ** 2))))
    assert err <= TOL_FP32
