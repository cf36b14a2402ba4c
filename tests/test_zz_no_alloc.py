"""ds4moe_layer_noalloc (the layer call on the library's static device
workspace, for callers that cannot allocate) against ds4moe_layer on the
same inputs: expert ids, gates, normalised inputs and outputs must be
identical, on consecutive calls whose second is smaller than the first, on a
layer with a shared expert at the largest accepted token count, for a
hash-routed layer whose fault bits the call reports and clears, under HIP
graph capture, and with a token count past the static workspace refused
before anything runs."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g
from gpu_util import experts_of, ptr, say, shape_of, shared_of, stream, workspace

pytestmark = pytest.mark.gpu

MAX_T = 17   # the static workspace holds 17 tokens of the V4-Flash shape


@pytest.fixture(scope="module")
def layers():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ds4gen.device import make_layer
    w1, w2 = g.WORKLOADS[1], g.WORKLOADS[2]
    return {1: (w1, make_layer(w1, 0, norm=True)), 2: (w2, make_layer(w2, 0))}


def dev(a):
    from ds4gen.device import to_dev
    return to_dev(a)


def run_both(w, desc, T, x=None, h0=None, tok=None):
    """The same layer call through ds4moe_layer and ds4moe_layer_noalloc;
    returns the two sets of results and the fault word of the latter."""
    shp = shape_of(w)
    res = []
    faults = torch.full((1,), 0xDEAD, dtype=torch.int32, device="cuda")
    for noalloc in (False, True):
        out = torch.full((T, w.H), 7.0, dtype=torch.float32, device="cuda")
        resid = dev(h0) if h0 is not None else None
        ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
        xn = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
        xp = ptr(x) if x is not None else None
        args = (shp, desc, xp, ds4.BF16, ptr(resid), None if resid is not None else ptr(out),
                ptr(tok), T, ptr(ids), ptr(wts), ptr(xn))
        if noalloc:
            ds4.layer_noalloc(*args, ptr(faults), stream())
        else:
            ws, nb = workspace(shp, T)
            ds4.layer(*args, ptr(ws), nb, stream())
            assert ds4.check(ptr(ws), stream()) == 0
        torch.cuda.synchronize()
        res.append({"out": (resid if resid is not None else out).cpu().numpy(),
                    "ids": ids.cpu().numpy(), "wts": wts.cpu().numpy(),
                    "xn": xn.cpu().numpy()})
    return res[0], res[1], int(faults.cpu().numpy()[0])


def assert_same(a, b):
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_noalloc_matches_layer_two_calls_second_smaller(layers):
    # a stack-style layer (RMSNorm of the residual stream, learned router,
    # residual += output): 8 tokens (selection kernel, few-token matvecs),
    # then 1 token (selection fused into gate/up) on the same static array
    from ds4gen.device import step_inputs
    w, lt = layers[1]
    desc = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                          experts_of(lt, w), norm_w=ptr(lt.norm_w), norm_eps=1e-6)
    for T in (8, 1):
        say("noalloc stack-style layer T", T)
        h0, _ = step_inputs(w, T, first_step=3 * T)
        a, b, f = run_both(w, desc, T, h0=h0)
        assert_same(a, b)
        assert f == 0


def test_noalloc_shared_expert_at_the_limit(layers):
    # the config-2 layer (Q8_0 shared expert) on x -> out: 17 tokens (the
    # largest the static array holds), then 2
    w, lt = layers[2]
    desc = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                          experts_of(lt, w), shared=shared_of(lt, w))
    for T in (MAX_T, 2):
        say("noalloc shared-expert layer T", T)
        x = dev(g.activations(w, n_tok=T))
        a, b, f = run_both(w, desc, T, x=x)
        assert_same(a, b)
        assert f == 0


def test_noalloc_reports_and_clears_faults(layers):
    # hash routing with a token id out of range: the fault word carries
    # BAD_TOKEN; the next, clean call reports 0 (the status is cleared per call)
    w, lt = layers[1]
    table = dev(g.hash_table(w, 0))
    desc = ds4.layer_desc(ds4.router(tid2eid=ptr(table), vocab=w.vocab), experts_of(lt, w))
    x = dev(g.activations(w, n_tok=2))
    shp = shape_of(w)
    out = torch.empty((2, w.H), dtype=torch.float32, device="cuda")
    faults = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = dev(np.array([5, w.vocab + 3], np.int32))
    ds4.layer_noalloc(shp, desc, ptr(x), ds4.BF16, None, ptr(out), ptr(bad), 2, None, None, None,
                      ptr(faults), stream())
    assert int(faults.cpu().numpy()[0]) & ds4.FAULT_BAD_TOKEN
    good = dev(np.array([5, 6], np.int32))
    a, b, f = run_both(w, desc, 2, x=x, tok=good)
    assert_same(a, b)
    assert f == 0


def test_noalloc_graph_replays(layers):
    # captured once, replayed three times with eager calls in between: every
    # replay reproduces the eager result bit for bit
    w, lt = layers[2]
    desc = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                          experts_of(lt, w), shared=shared_of(lt, w))
    shp = shape_of(w)
    T = 4
    x = dev(g.activations(w, n_tok=T))
    ref = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, w.H), dtype=torch.float32, device="cuda")
    faults = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call(dst, st):
        ds4.layer_noalloc(shp, desc, ptr(x), ds4.BF16, None, ptr(dst), None, T, None, None, None,
                          ptr(faults), st)

    call(ref, stream())
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call(out, torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs" % rep
        assert int(faults.cpu().numpy()[0]) == 0
        call(ref, stream())
        torch.cuda.synchronize()


def test_noalloc_refuses_past_the_static_workspace(layers):
    w, lt = layers[2]
    shp = shape_of(w)
    assert ds4.workspace_size(shp, MAX_T) <= 8 << 20 < ds4.workspace_size(shp, MAX_T + 1)
    desc = ds4.layer_desc(ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias)),
                          experts_of(lt, w))
    T = MAX_T + 1
    x = dev(g.activations(w, n_tok=T))
    out = torch.full((T, w.H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.layer_noalloc(shp, desc, ptr(x), ds4.BF16, None, ptr(out), None, T, None, None, None,
                          None, stream())
    assert e.value.status == ds4.EWORKSPACE
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 7.0).all()
