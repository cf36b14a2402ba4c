"""Edge cases of the layer entry points on the GPU: empty inputs, the largest
token count the path accepts (32,768 token-expert pairs) and one past it,
and degenerate routing (every token on the same six experts, zero gates)."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g
import oracle
from gpu_util import (TOL_FP32, check_clean, covering_tokens, experts_of, max_rel_err, ptr, say,
                      shape_of, stream, workspace)

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def test_empty_inputs_touch_nothing():
    from ds4gen.device import make_layer
    w = g.WORKLOADS[1]
    say("empty inputs")
    lt = make_layer(w, 0)
    shp = shape_of(w)
    ws, nb = workspace(shp, 1)
    sentinel = torch.full((64,), 7, dtype=torch.int32, device="cuda")
    fsent = torch.full((4096,), 3.0, dtype=torch.float32, device="cuda")
    x = torch.zeros(4096, dtype=torch.int16, device="cuda")
    rt = ds4.router(w=ptr(lt.router_w), w_dtype=ds4.F16, bias=ptr(lt.bias))
    ds4.route(shp, rt, ptr(x), ds4.BF16, 0, None, ptr(sentinel), ptr(fsent), ptr(ws), nb, stream())
    ds4.permute(shp, ptr(sentinel), 0, ptr(sentinel), ptr(sentinel), ptr(sentinel), ptr(sentinel),
                ptr(ws), nb, stream())
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(x), ds4.BF16, 0, ptr(sentinel), ptr(fsent),
                   ptr(fsent), None, ptr(ws), nb, stream())
    desc = ds4.layer_desc(rt, experts_of(lt, w))
    ds4.layer(shp, desc, ptr(x), ds4.BF16, None, ptr(fsent), None, 0, None, None, None, ptr(ws),
              nb, stream())
    check_clean(ws)
    assert (sentinel.cpu().numpy() == 7).all() and (fsent.cpu().numpy() == 3.0).all()


def big_case(T):
    # the V4-Flash layer at T tokens with Zipf(1.1)-routed experts given
    from ds4gen.device import make_layer, host_experts
    w = g.Workload("v4flash-layer-max-tokens", 41, T, 4096, 2048, 256, 6, g.IQ2_XXS, g.IQ2_XXS,
                   g.Q2_K, "bf16", "f16", routing="given-zipf")
    ids, wts = g.zipf_routing(w.seed, T, w.E, w.K)
    return w, ids, wts, make_layer(w, 0), host_experts


def test_max_tokens():
    T = 32768 // 6   # 5461 tokens x top-6 = 32,766 pairs
    say("max tokens", T)
    w, ids, wts, lt, host_experts = big_case(T)
    x = g.activations(w, n_tok=T)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    pdbg = torch.empty(w.E + 1 + 2 * T * w.K, dtype=torch.int32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, T, ptr(idd), ptr(wd),
                   ptr(out), ptr(pdbg), ptr(ws), nb, stream())
    check_clean(ws)
    _, oo, op, oi = oracle.permute(ids, w.E)
    pd = pdbg.cpu().numpy()
    np.testing.assert_array_equal(pd[:w.E + 1], oo)
    np.testing.assert_array_equal(pd[w.E + 1:w.E + 1 + T * w.K], op)
    np.testing.assert_array_equal(pd[w.E + 1 + T * w.K:], oi)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    heavy = int(np.argmax(counts))
    t_heavy = int(np.where((ids == heavy).any(1))[0][-1])
    # every touched expert through at least one checked token, and the last
    # pair of the heaviest expert
    toks = covering_tokens(ids, extra=(0, T // 2, t_heavy, T - 1))
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.unique(ids[toks])),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=toks)
    err = max_rel_err(out.cpu().numpy()[toks], want)
    say("  max tokens: heaviest expert %d pairs, max|err|/rms = %g" % (counts.max(), err))
    assert err <= TOL_FP32
    # one token more is refused before anything runs
    with pytest.raises(ds4.Ds4moeError) as e:
        ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, T + 1, ptr(idd), ptr(wd),
                       ptr(out), None, ptr(ws), nb, stream())
    assert e.value.status in (ds4.EUNSUPPORTED, ds4.EWORKSPACE)


@pytest.mark.parametrize("T", [1, 9, 300])
def test_degenerate_routing(T):
    # every token on experts 0..5 with equal gates, one slot with gate 0:
    # matvec kernels at 1 and 9 tokens, the grouped path at 300 (items of 64
    # rows per expert and a ragged last piece)
    from ds4gen.device import make_layer, host_experts
    w = g.Workload("v4flash-layer-degenerate", 42, T, 4096, 2048, 256, 6, g.IQ2_XXS, g.IQ2_XXS,
                   g.Q2_K, "bf16", "f16")
    say("degenerate routing T", T)
    lt = make_layer(w, 0)
    ids = np.tile(np.arange(6, dtype=np.int32), (T, 1))
    wts = np.full((T, 6), 0.3, np.float32)
    wts[:, 3] = 0.0
    x = g.activations(w, n_tok=T)
    shp = shape_of(w)
    ws, nb = workspace(shp, T)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(wts)
    ds4.expert_ffn(shp, experts_of(lt, w), None, ptr(xd), ds4.BF16, T, ptr(idd), ptr(wd),
                   ptr(out), None, ptr(ws), nb, stream())
    check_clean(ws)
    toks = np.unique(np.array([0, T // 3, T - 1]))
    want = oracle.moe_ffn(x, "bf16", ids, wts, host_experts(w, 0, np.arange(6)),
                          (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I, w.E, grid=g.grid(w.seed),
                          tokens=toks)
    err = max_rel_err(out.cpu().numpy()[toks], want)
    say("  max|err|/rms = %g" % err)
    assert err <= TOL_FP32
