#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on 2-bit weights (one MI355X).

Default workload: one DeepSeek-V4-Flash-shaped routed-expert layer at batch-1
decode (hidden 4096, expert intermediate 2048, 256 experts, top-6, IQ2_XXS
gate/up, Q2_K down, fp16 router, bf16 activations), one step = routing +
expert FFN + weighted combine for one token.  Every step uses a different
seeded token, all resident in HBM before timing starts.  Steps are captured
once into a HIP graph and replayed, so host launch cost is outside the timed
region.  Prints one JSON line.

Other workloads (--workload): decode-b8 (8 correlated tokens + Q8_0 shared
expert), prefill-512 (Zipf-routed 512-token chunk), stack-43 (43-layer
decode stack, hash routing in layers 0-2), stack-43-q4k (the same stack with
Q4_K routed experts in layers 37-42), stack-43-shared (with the Q8_0 shared
expert of every layer), decode-sweep (the decode-b8 layer at 1
to 64 tokens per call), prefill-512-q4k (the prefill chunk through a layer
with Q4_K experts), encode (fp32 experts to IQ2_XXS / Q2_K blocks).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
METRIC = "MoE layer tokens/s + expert-weight HBM GB/s (% of peak), batch-1 decode"

# HBM bytes per dispatch of the gate/up kernel from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes, FETCH_SIZE scaled by what it reads for the 2 GiB read
# probe (a 256 MiB device copy agrees; the summary sits in
# profiles/decode_b1_hbm_traffic.txt).  Reported only while
# the kernel source still hashes to what was measured.
GATEUP_TRAFFIC = {
    "sources": ("bit_quantized_expert_ds4moe_amd/csrc/ffn_b1.hip",
                "bit_quantized_expert_ds4moe_amd/csrc/dev_common.h",
                "bit_quantized_expert_ds4moe_amd/csrc/route.hip"),
    "sha256": "beb81eface1de7703d8cbbdac1963520f9b80627b9773c42318bf392d5e76e50",
    "bytes": 26303165,
}


# The same for the Q4_K gate/up kernel of the mixed stack (summary, with the
# raw counters and the copy calibration, in profiles/stack43_q4k_hbm_traffic.txt).
Q4K_GATEUP_TRAFFIC = {
    "sources": ("bit_quantized_expert_ds4moe_amd/csrc/ffn_q4k.hip",
                "bit_quantized_expert_ds4moe_amd/csrc/ffn_b1.hip",
                "bit_quantized_expert_ds4moe_amd/csrc/dev_common.h",
                "bit_quantized_expert_ds4moe_amd/csrc/route.hip"),
    "sha256": "10e6891d6d42c10bcd30e9c298e3dd506169537d13253b637dc5db040c099603",
    "bytes": 56954311,
}


def batched_gateup_kernel(w, T):
    """The routed gate/up kernel that a layer call of T decode tokens runs
    (the library's token thresholds, learned router)."""
    import ds4gen as g
    if w.gate_qt == g.Q4_K:
        return "k_gateup_q4k_b1<true>" if T <= 4 else "k_gateup_q4k_b1<false>" if T <= 13 else "grouped gate/up"
    return "k_gateup_b1<true>" if T <= 4 else "k_gateup_few" if T <= 10 else "grouped gate/up"


def measured_traffic(rec):
    import hashlib
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if rec["sha256"] and h.hexdigest() == rec["sha256"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def event_handle(ev):
    import torch
    ev.record()
    torch.cuda.synchronize()
    return ev.cuda_event


def mean_event_us(pairs):
    """Mean span in microseconds of the recorded (start, stop) event pairs;
    None when no launch of the class recorded them (a one-token layer call
    scores inside its gate/up kernel, so no scoring kernel runs)."""
    import numpy as np
    t = []
    for a, b in pairs:
        try:
            t.append(a.elapsed_time(b))
        except RuntimeError:
            continue
    return float(np.mean(t)) * 1e3 if t else None


def time_replays(replay, n):
    """Times n passes of replay() (each a whole timed region: a graph replay
    or a sequence of them), each bracketed by device synchronisations, with
    events on the current stream.  Returns the milliseconds of each pass."""
    import torch
    out = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def replay_summary(ms_list):
    import numpy as np
    return {"passes": len(ms_list), "median_ms": round(float(np.median(ms_list)), 5),
            "min_ms": round(float(np.min(ms_list)), 5), "max_ms": round(float(np.max(ms_list)), 5)}


def read_bandwidth(nbytes=2 << 30, reps=11):
    """The box's streaming-read bandwidth: the library's read probe (a plain
    16-byte-load streaming kernel) over nbytes, median of reps launches timed
    with events on the launch stream."""
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    ds4.read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), st)
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        ds4.read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), st)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = float(np.median(ms))
    del buf
    torch.cuda.empty_cache()
    gbs = nbytes / (med * 1e-3) / 1e9
    log("read probe: %d bytes in %.1f us (median of %d) = %.0f GB/s" % (nbytes, med * 1e3, reps, gbs))
    return {"kernel": "k_read_probe (ds4moe_read_probe)", "bytes": nbytes, "median_us": round(med * 1e3, 2),
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def add_stream_fracs(res, stream):
    """Every bandwidth of a result line also as a fraction of the measured
    streaming-read bandwidth."""
    res["hbm_stream"] = stream
    if "expert_gbs" in res:
        res["expert_stream_frac"] = round(res["expert_gbs"] / stream["gbs"], 4)
    for key in ("roofline", "roofline_q4k"):
        r = res.get(key)
        if r and r.get("unit") == "GB/s":
            r["frac_of_stream"] = round(r["achieved"] / stream["gbs"], 4)
    return res


def bench_decode_b1(args):
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    import ds4gen as g
    from ds4gen.device import make_layer, to_dev

    w = g.WORKLOADS[1]
    n_tok = args.warmup + args.steps
    log("building layer tensors (%s)" % w.name)
    layers = [make_layer(w, l) for l in range(args.layer_copies)]
    x = to_dev(g.activations(w, n_tok=n_tok))
    shp = ds4.shape(w.H, w.I, w.E, w.K, 1.5)
    nb = ds4.workspace_size(shp, 1)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((n_tok, w.H), dtype=torch.float32, device="cuda")
    descs = []
    for lt in layers:
        ex = ds4.experts(lt.gate.data_ptr(), lt.up.data_ptr(), lt.down.data_ptr(), w.I,
                         (w.gate_qt, w.up_qt, w.down_qt), grid=lt.grid.data_ptr())
        descs.append(ds4.layer_desc(ds4.router(w=lt.router_w.data_ptr(), w_dtype=ds4.F16,
                                               bias=lt.bias.data_ptr()), ex))
    row = w.H * 2

    def step(i, st):
        ds4.layer(shp, descs[i % len(descs)], x.data_ptr() + i * row, ds4.BF16, None,
                  out.data_ptr() + i * w.H * 4, None, 1, None, None, None, ws.data_ptr(), nb, st)

    # eager warm-up (also checks the fault word once)
    st = torch.cuda.current_stream().cuda_stream
    for i in range(min(args.warmup, 4)):
        step(i, st)
    assert ds4.check(ws.data_ptr(), st) == 0

    def capture(first, count, per_step=None):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream().cuda_stream
            for j in range(count):
                if per_step:
                    per_step(j)
                step(first + j, cs)
        return gr

    log("capturing graphs")
    g_warm = capture(0, args.warmup)
    g_main = capture(args.warmup, args.steps)
    g_warm.replay()
    torch.cuda.synchronize()
    # the timed region: the K steps, replayed `replays` times; the median pass
    passes = time_replays(g_main.replay, args.replays)
    ms = float(np.median(passes))
    assert ds4.check(ws.data_ptr(), st) == 0
    log("timed %d steps x %d passes: median %.3f ms (min %.3f, max %.3f)"
        % (args.steps, len(passes), ms, min(passes), max(passes)))

    # second pass: per-kernel HIP events around each launch, recorded by the
    # library on the launch stream.  The GPU first spins in a sleep kernel so
    # that the host has enqueued every launch before the first one runs.
    classes = {"route": ds4.K_ROUTE, "gateup": ds4.K_GATEUP, "down": ds4.K_DOWN}
    n_prof = min(args.steps, 400)
    evs = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_prof)] for c in classes}
    handles = {c: [(event_handle(a), event_handle(b)) for a, b in evs[c]] for c in classes}
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    torch.cuda._sleep(args.sleep_cycles)
    s1.record()
    h0 = time.perf_counter()
    for j in range(n_prof):
        for c, k in classes.items():
            ds4.profile_events(k, handles[c][j][0], handles[c][j][1])
        step(args.warmup + j, st)
    host_ms = (time.perf_counter() - h0) * 1e3
    for k in classes.values():
        ds4.profile_events(k, None, None)
    torch.cuda.synchronize()
    sleep_ms = s0.elapsed_time(s1)
    if sleep_ms < host_ms:
        log("warning: GPU sleep %.2f ms shorter than host enqueue %.2f ms" % (sleep_ms, host_ms))
    kern_us = {c: mean_event_us(evs[c]) for c in classes}
    kern_us = {c: v for c, v in kern_us.items() if v is not None}
    log("kernel averages (us):", kern_us, "sleep %.2f ms, enqueue %.2f ms" % (sleep_ms, host_ms))
    assert ds4.check(ws.data_ptr(), st) == 0

    expert_bytes = w.K * w.expert_bytes()                 # 42,467,328 per token-layer
    gateup_bytes = w.K * 2 * w.blocks_per_expert["gate"] * g.BLOCK_BYTES[w.gate_qt]
    tok_s = args.steps / (ms * 1e-3)
    gbs = expert_bytes * tok_s / 1e9
    ach = gateup_bytes / (kern_us["gateup"] * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "hidden": w.H, "inter": w.I, "experts": w.E,
                   "top_k": w.K, "tokens_per_step": 1, "gate_up": "IQ2_XXS", "down": "Q2_K",
                   "router": "f16", "activations": "bf16", "layer_copies": args.layer_copies,
                   "timing": "hip-graph replay, distinct token per step, step i on layer copy "
                             "i mod copies (cold: %.0f GB of experts cycled); median of %d passes"
                             % (args.layer_copies * 256 * w.expert_bytes() / 1e9, args.replays)},
        "timed_passes": replay_summary(passes),
        "expert_gbs": round(gbs, 1), "expert_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "kernel_timing": "HIP events recorded by the library around each launch, %d eager steps" % n_prof,
        "roofline": {"bound": "hbm", "kernel": "k_gateup_b1<true>", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(GATEUP_TRAFFIC),
                     "bytes_per_launch": gateup_bytes},
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = with_single_thread(cpu_baseline_decode, (w, args.cpu_sample), (w, 1))
    return res


def stack_descs(ds4, w, layers):
    descs = []
    for l, lt in enumerate(layers):
        wl = w.at_layer(l)
        ex = ds4.experts(lt.gate.data_ptr(), lt.up.data_ptr(), lt.down.data_ptr(), w.I,
                         (wl.gate_qt, wl.up_qt, wl.down_qt), grid=lt.grid.data_ptr())
        if l < w.n_hash:
            rt = ds4.router(tid2eid=lt.tid2eid.data_ptr(), vocab=w.vocab)
        else:
            rt = ds4.router(w=lt.router_w.data_ptr(), w_dtype=ds4.F16, bias=lt.bias.data_ptr())
        sh = None
        if lt.shared is not None:
            sh = ds4.experts(lt.shared[0].data_ptr(), lt.shared[1].data_ptr(),
                             lt.shared[2].data_ptr(), w.I, (ds4.Q8_0, ds4.Q8_0, ds4.Q8_0))
        descs.append(ds4.layer_desc(rt, ex, shared=sh, norm_w=lt.norm_w.data_ptr(), norm_eps=1e-6))
    return descs


def bench_stack(args, mixed=False, shared=False):
    """43-layer routed-expert stack at batch-1 decode: one step = one token
    through every layer (RMSNorm -> routing -> experts -> residual add).
    mixed: the routed experts of layers 37-42 are Q4_K (gate, up and down);
    shared: every layer also has its Q8_0 shared expert."""
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    import ds4gen as g
    from ds4gen.device import make_stack, step_inputs, to_dev

    w = g.WORKLOADS[5 if mixed else 4]
    if shared:
        from dataclasses import replace
        w = replace(w, name=w.name + "-shared-q8", shared=True)
    log("generating %d layers x %d experts on the device" % (w.n_layers, w.E))
    t0 = time.perf_counter()
    layers = make_stack(w, log)
    torch.cuda.synchronize()
    log("  done in %.1f s" % (time.perf_counter() - t0))
    descs = stack_descs(ds4, w, layers)
    n_steps = args.warmup + args.steps
    h0, tok = step_inputs(w, n_steps)
    h0_all, tok_all = to_dev(h0), to_dev(tok)
    resid = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
    tokbuf = torch.empty(1, dtype=torch.int32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int64, device="cuda")
    shp = ds4.shape(w.H, w.I, w.E, w.K, 1.5)
    nb = ds4.workspace_size(shp, 1)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")

    # each step runs the 43 layers on its own residual row (reset from the
    # step inputs before every pass, outside the timed region) and reads its
    # own token id, so the graph holds the library's launches only
    resid_all = torch.empty((n_steps, w.H), dtype=torch.float32, device="cuda")

    def step(j, st):
        rp = resid_all.data_ptr() + j * w.H * 4
        tp = tok_all.data_ptr() + j * 4
        for d in descs:
            ds4.layer(shp, d, None, ds4.BF16, rp, None, tp, 1, None, None, None, ws.data_ptr(), nb, st)

    def capture(first, count):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream().cuda_stream
            for j in range(count):
                step(first + j, cs)
        return gr

    st = torch.cuda.current_stream().cuda_stream
    resid_all.copy_(h0_all)
    step(0, st)
    assert ds4.check(ws.data_ptr(), st) == 0
    log("capturing graphs")
    g_warm = capture(0, args.warmup)
    g_main = capture(args.warmup, args.steps)
    resid_all.copy_(h0_all)
    g_warm.replay()
    torch.cuda.synchronize()

    passes = []
    for _ in range(args.replays):
        resid_all.copy_(h0_all)  # untimed: every pass starts from the step inputs
        passes += time_replays(g_main.replay, 1)
    ms = float(np.median(passes))
    assert ds4.check(ws.data_ptr(), st) == 0
    log("timed %d steps x %d passes: median %.3f ms (min %.3f, max %.3f)"
        % (args.steps, len(passes), ms, min(passes), max(passes)))

    # per-kernel events over a few eager steps behind a GPU sleep
    classes = {"route": ds4.K_ROUTE, "gateup": ds4.K_GATEUP, "down": ds4.K_DOWN, "other": ds4.K_OTHER}
    n_prof = 2
    n_ev = n_prof * w.n_layers
    evs = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_ev)] for c in classes}
    handles = {c: [(event_handle(a), event_handle(b)) for a, b in evs[c]] for c in classes}
    used = {c: 0 for c in classes}
    ev_q4 = {c: [] for c in classes}     # whether each recorded launch is in a Q4_K layer
    # the eager steps read rows 0 .. n_prof-1 of the step inputs
    assert n_prof <= n_steps
    torch.cuda.synchronize()
    torch.cuda._sleep(args.sleep_cycles)
    for j in range(n_prof):
        torch.index_select(h0_all, 0, idx, out=resid)
        torch.index_select(tok_all, 0, idx, out=tokbuf)
        for l, d in enumerate(descs):
            for c, k in classes.items():
                if c == "other" and l >= w.n_hash and not w.shared:
                    ds4.profile_events(k, None, None)
                    continue
                ds4.profile_events(k, handles[c][used[c]][0], handles[c][used[c]][1])
                ev_q4[c].append(l in w.q4_layers)
                used[c] += 1
            ds4.layer(shp, d, None, ds4.BF16, resid.data_ptr(), None, tokbuf.data_ptr(), 1, None,
                      None, None, ws.data_ptr(), nb, st)
        idx.add_(1)
    for k in classes.values():
        ds4.profile_events(k, None, None)
    torch.cuda.synchronize()
    def mean_us(c, q4):
        return mean_event_us([ab for ab, f in zip(evs[c][:used[c]], ev_q4[c]) if f == q4])

    kern_us = {c: mean_us(c, False) for c in classes if used[c]}
    kern_us = {c: v for c, v in kern_us.items() if v is not None}
    log("kernel averages (us):", kern_us)
    kern_us_q4 = {c: mean_us(c, True) for c in ("gateup", "down")} if w.q4_layers else None
    if kern_us_q4:
        log("kernel averages in the Q4_K layers (us):", kern_us_q4)

    # 1,826,095,104 per token (all q2); 2,080,899,072 with layers 37-42 in Q4_K
    expert_bytes = w.token_expert_bytes()
    if w.shared:  # the Q8_0 shared expert of every layer
        expert_bytes += w.n_layers * 3 * w.I * w.H // 32 * g.BLOCK_BYTES[g.Q8_0]
    gateup_bytes = w.K * 2 * w.blocks_per_expert["gate"] * g.BLOCK_BYTES[w.gate_qt]
    tok_s = args.steps / (ms * 1e-3)
    gbs = expert_bytes * tok_s / 1e9
    ach = gateup_bytes / (kern_us["gateup"] * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "hash_layers": w.n_hash,
                   "hidden": w.H, "inter": w.I, "experts": w.E, "top_k": w.K,
                   "q4k_layers": list(w.q4_layers), "shared_q8_0": bool(w.shared),
                   "resident_expert_bytes": w.stack_expert_bytes(),
                   "timing": "hip-graph replay of the timed steps (43 layers per token, each step "
                             "on its own residual row); median of %d passes" % args.replays},
        "timed_passes": replay_summary(passes),
        "expert_gbs": round(gbs, 1), "expert_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "roofline": {"bound": "hbm", "kernel": "k_gateup_b1<true>", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(GATEUP_TRAFFIC),
                     "bytes_per_launch": gateup_bytes},
    }
    if kern_us_q4:
        # the Q4_K layers' gate/up kernel, beside the dominant one: 40 IQ2_XXS
        # layers against 6 Q4_K layers
        w4 = w.at_layer(w.q4_layers[0])
        b4 = w4.K * 2 * w4.blocks_per_expert["gate"] * g.BLOCK_BYTES[w4.gate_qt]
        a4 = b4 / (kern_us_q4["gateup"] * 1e-6) / 1e9
        n4 = len(w.q4_layers)
        assert kern_us["gateup"] * (w.n_layers - n4) > kern_us_q4["gateup"] * n4
        res["kernels_us_q4k_layers"] = {k: round(v, 3) for k, v in kern_us_q4.items()}
        res["roofline_q4k"] = {"bound": "hbm", "kernel": "k_gateup_q4k_b1<true>", "achieved": round(a4, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(a4 / PEAK_HBM_GBS, 4),
                               "traffic": measured_traffic(Q4K_GATEUP_TRAFFIC),
                               "bytes_per_launch": b4}
    if args.cpu_baseline:
        res["cpu_baseline"] = with_single_thread(cpu_baseline_stack, (w, args.cpu_sample),
                                                 (w, 2))
    return res


def bench_batched(args, which):
    """Batched decode (8 correlated tokens, learned router, Q8_0 shared expert:
    one ds4moe_layer call per step) or prefill (512 tokens with Zipf-routed
    experts given: one ds4moe_expert_ffn call per step).  Timed like
    decode-b1: hip-graph replay of the steps, then eager steps with per-launch
    events."""
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    import ds4gen as g
    from ds4gen.device import make_layer, to_dev

    prefill = which.startswith("prefill-512")
    w = g.WORKLOADS[3 if prefill else 2]
    if which == "prefill-512-q4k":  # a Q4 layer of the mixed stacks
        from dataclasses import replace
        w = replace(w, name=w.name + "-q4k", gate_qt=g.Q4_K, up_qt=g.Q4_K, down_qt=g.Q4_K)
    T = w.T
    log("building layer tensors (%s)" % w.name)
    lt = make_layer(w, 0)
    ex = ds4.experts(lt.gate.data_ptr(), lt.up.data_ptr(), lt.down.data_ptr(), w.I,
                     (w.gate_qt, w.up_qt, w.down_qt), grid=lt.grid.data_ptr())
    sh = None
    if w.shared:
        sh = ds4.experts(lt.shared[0].data_ptr(), lt.shared[1].data_ptr(), lt.shared[2].data_ptr(),
                         w.I, (g.Q8_0, g.Q8_0, g.Q8_0))
    shp = ds4.shape(w.H, w.I, w.E, w.K, 1.5)
    nb = ds4.workspace_size(shp, T)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    n_batches = 1 if prefill else args.warmup + args.steps
    x = to_dev(g.activations(w, n_tok=T * n_batches))
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    row = w.H * 2
    if prefill:
        ids_h, wts_h = g.zipf_routing(w.seed, T, w.E, w.K)
        ids, wts = to_dev(ids_h), to_dev(wts_h)
        touched = int(np.unique(ids_h).size)

        if args.imatrix:  # importance statistics collected in the same call
            imx_gu = torch.zeros((w.E, w.H), dtype=torch.float32, device="cuda")
            imx_dn = torch.zeros((w.E, w.I), dtype=torch.float32, device="cuda")

            def step(i, st):
                ds4.expert_ffn_imatrix(shp, ex, None, x.data_ptr(), ds4.BF16, T, ids.data_ptr(),
                                       wts.data_ptr(), out.data_ptr(), imx_gu.data_ptr(),
                                       imx_dn.data_ptr(), ws.data_ptr(), nb, st)
        else:
            def step(i, st):
                ds4.expert_ffn(shp, ex, None, x.data_ptr(), ds4.BF16, T, ids.data_ptr(),
                               wts.data_ptr(), out.data_ptr(), None, ws.data_ptr(), nb, st)
    else:
        desc = ds4.layer_desc(ds4.router(w=lt.router_w.data_ptr(), w_dtype=ds4.F16,
                                         bias=lt.bias.data_ptr()), ex, shared=sh)
        ids_d = torch.empty((n_batches, T, w.K), dtype=torch.int32, device="cuda")

        def step(i, st, ids_out=None):
            ds4.layer(shp, desc, x.data_ptr() + i * T * row, ds4.BF16, None, out.data_ptr(), None, T,
                      ids_out, None, None, ws.data_ptr(), nb, st)

    st = torch.cuda.current_stream().cuda_stream
    step(0, st)
    assert ds4.check(ws.data_ptr(), st) == 0

    def capture(first, count):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream().cuda_stream
            for j in range(count):
                step(0 if prefill else first + j, cs)
        return gr

    g_warm = capture(0, args.warmup)
    g_main = capture(args.warmup, args.steps)
    g_warm.replay()
    torch.cuda.synchronize()
    passes = time_replays(g_main.replay, args.replays)
    ms = float(np.median(passes))
    assert ds4.check(ws.data_ptr(), st) == 0
    log("timed %d steps x %d passes: median %.3f ms" % (args.steps, len(passes), ms))
    if not prefill:  # experts touched per step, from untimed calls
        for i in range(args.warmup, n_batches):
            step(i, st, ids_d[i].data_ptr())
        touched_per = [int(np.unique(a).size) for a in ids_d[args.warmup:].cpu().numpy()]
        touched = float(np.mean(touched_per))

    if prefill:
        classes = {"permute": ds4.K_PERMUTE, "gateup": ds4.K_GATEUP, "down": ds4.K_DOWN,
                   "combine": ds4.K_OTHER}
    else:  # few-token path: routed experts per token, then the shared expert as one class
        classes = {"route": ds4.K_ROUTE, "gateup": ds4.K_GATEUP, "down": ds4.K_DOWN,
                   "shared_expert": ds4.K_OTHER}
    n_prof = min(args.steps, 50)
    evs = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_prof)] for c in classes}
    handles = {c: [(event_handle(a), event_handle(b)) for a, b in evs[c]] for c in classes}
    torch.cuda.synchronize()
    torch.cuda._sleep(args.sleep_cycles)
    for j in range(n_prof):
        for c, k in classes.items():
            ds4.profile_events(k, handles[c][j][0], handles[c][j][1])
        step(0 if prefill else args.warmup + j, st)
    for k in classes.values():
        ds4.profile_events(k, None, None)
    torch.cuda.synchronize()
    kern_us = {c: mean_event_us(evs[c]) for c in classes}
    kern_us = {c: v for c, v in kern_us.items() if v is not None}
    log("kernel averages (us):", kern_us)

    per_expert = w.expert_bytes()
    gateup_expert = 2 * w.blocks_per_expert["gate"] * g.BLOCK_BYTES[w.gate_qt]
    sh_bytes = 3 * w.I * w.H // 32 * g.BLOCK_BYTES[g.Q8_0] if w.shared else 0
    step_bytes = touched * per_expert + sh_bytes
    sec = ms * 1e-3 / args.steps
    flops = 2.0 * T * (3 * w.H * w.I) * (w.K + (1 if w.shared else 0))
    # dominant kernel: gate/up of the routed experts; algorithmic bytes = the
    # distinct experts' gate and up tensors (repeats within a step are cache hits)
    gu_bytes = touched * gateup_expert
    gu_flops = 2.0 * T * (2 * w.H * w.I) * w.K
    gu_s = kern_us["gateup"] * 1e-6
    res = {
        "metric": ("prefill tokens/s through one routed-expert layer" if prefill
                   else "batched-decode tokens/s through one routed-expert layer"),
        "value": round(T / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "tokens_per_step": T, "hidden": w.H, "inter": w.I,
                   "experts": w.E, "top_k": w.K, "shared_q8_0": bool(w.shared),
                   "experts_touched_per_step": touched,
                   "routing": "given Zipf(1.1)" if prefill else "learned router",
                   "imatrix": bool(prefill and args.imatrix),
                   "timing": "hip-graph replay; median of %d passes" % args.replays},
        "timed_passes": replay_summary(passes),
        "expert_gbs": round(step_bytes / sec / 1e9, 1),
        "expert_hbm_frac": round(step_bytes / sec / 1e9 / PEAK_HBM_GBS, 4),
        "mfma_tflops": round(flops / sec / 1e12, 2),
        "mfma_frac": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "roofline": {"bound": "hbm", "kernel": (("grouped Q4_K gate/up: k_x_to_f16 + k_grouped_gateup_q4k"
                                                 if w.gate_qt == g.Q4_K else
                                                 "grouped IQ2_XXS gate/up: k_x_to_f16 + k_grouped_gateup_iq2_all")
                                                if prefill else batched_gateup_kernel(w, T)),
                     "achieved": round(gu_bytes / gu_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gu_bytes / gu_s / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_launch": int(gu_bytes),
                     "mfma_tflops": round(gu_flops / gu_s / 1e12, 2)},
    }
    return res


def bench_sweep(args):
    """Decode batch sweep: the config-2 layer (learned router, Q8_0 shared
    expert, correlated tokens) at T = 1 .. 64 tokens per call, one
    ds4moe_layer call per step.  Up to 8 tokens the routed experts run
    through the streaming matvec kernels (one grid row per token), above that
    through the grouped MFMA kernels; the sweep shows where the union of
    experts makes the grouped form pay.  Each T: hip-graph replay of `steps` calls on distinct
    tokens after `warmup` calls."""
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    import ds4gen as g
    from ds4gen.device import make_layer, to_dev

    w = g.WORKLOADS[2]
    sizes = [1, 2, 4, 8, 9, 12, 13, 14, 16, 24, 32, 48, 64]
    tmax = max(sizes)
    log("building layer tensors (%s)" % w.name)
    lt = make_layer(w, 0)
    ex = ds4.experts(lt.gate.data_ptr(), lt.up.data_ptr(), lt.down.data_ptr(), w.I,
                     (w.gate_qt, w.up_qt, w.down_qt), grid=lt.grid.data_ptr())
    sh = ds4.experts(lt.shared[0].data_ptr(), lt.shared[1].data_ptr(), lt.shared[2].data_ptr(),
                     w.I, (g.Q8_0, g.Q8_0, g.Q8_0))
    shp = ds4.shape(w.H, w.I, w.E, w.K, 1.5)
    nb = ds4.workspace_size(shp, tmax)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    n_calls = args.warmup + args.steps
    x = to_dev(g.activations(w, n_tok=tmax * n_calls))
    out = torch.empty((tmax, w.H), dtype=torch.float32, device="cuda")
    ids_d = torch.empty((n_calls, tmax, w.K), dtype=torch.int32, device="cuda")
    row = w.H * 2
    desc = ds4.layer_desc(ds4.router(w=lt.router_w.data_ptr(), w_dtype=ds4.F16,
                                     bias=lt.bias.data_ptr()), ex, shared=sh)
    st = torch.cuda.current_stream().cuda_stream
    per_expert = w.expert_bytes()
    sh_bytes = 3 * w.I * w.H // 32 * g.BLOCK_BYTES[g.Q8_0]
    # untimed: bring the clocks up before the first (smallest) size
    for i in range(200):
        ds4.layer(shp, desc, x.data_ptr() + (i % n_calls) * 8 * row, ds4.BF16, None, out.data_ptr(),
                  None, 8, None, None, None, ws.data_ptr(), nb, st)
    torch.cuda.synchronize()
    rows = []
    for T in sizes:
        def step(i, s, ids_out=None):
            ds4.layer(shp, desc, x.data_ptr() + i * T * row, ds4.BF16, None, out.data_ptr(), None, T,
                      ids_out, None, None, ws.data_ptr(), nb, s)

        step(0, st)
        assert ds4.check(ws.data_ptr(), st) == 0

        def capture(first, count):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                cs = torch.cuda.current_stream().cuda_stream
                for j in range(count):
                    step(first + j, cs)
            return gr

        g_warm = capture(0, args.warmup)
        g_main = capture(args.warmup, args.steps)
        g_warm.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g_main.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        assert ds4.check(ws.data_ptr(), st) == 0
        for i in range(args.warmup, n_calls):
            step(i, st, ids_d[i].data_ptr())
        torch.cuda.synchronize()
        idh = ids_d[args.warmup:, :T].cpu().numpy()
        touched = float(np.mean([np.unique(a).size for a in idh]))
        sec = ms * 1e-3 / args.steps
        rows.append({"T": T, "tokens_per_s": round(T / sec, 1), "us_per_step": round(sec * 1e6, 2),
                     "experts_touched": round(touched, 2),
                     "expert_gbs": round((touched * per_expert + sh_bytes) / sec / 1e9, 1)})
        log("T=%d: %s" % (T, rows[-1]))
        del g_warm, g_main
    last = rows[-1]
    return {
        "metric": "batched-decode tokens/s through one routed-expert layer (sweep; value at T=%d)" % tmax,
        "value": last["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": last["us_per_step"] * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "v4flash-layer-decode-sweep-1-64", "hidden": w.H, "inter": w.I,
                   "experts": w.E, "top_k": w.K, "shared_q8_0": True, "routing": "learned router",
                   "tokens_per_call": sizes},
        "sweep": rows,
        "expert_gbs": last["expert_gbs"],
        "expert_hbm_frac": round(last["expert_gbs"] / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "whole layer call at T=%d" % tmax,
                     "achieved": last["expert_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(last["expert_gbs"] / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": None},
    }


# fp32 operations the encoder definitions perform per unit, list searches of
# the IQ2_XXS neighbour map excluded (their length depends on the data), a
# division counted as one operation.  IQ2_XXS group of 32 values: 16
# candidates x (32 level divisions + 96 refit-numerator + 96 refit-denominator
# + 160 error operations) + the final 32 level divisions.  Q2_K sub-block of
# 16 values: start error 128, four refits of 16 codes x 2 + 16 sums x 9 + 10
# + error 128, final codes 32.
ENC_OPS_IQ2_GROUP = 16 * (32 + 96 + 96 + 160) + 32
ENC_OPS_Q2K_SUB = 128 + 4 * (32 + 144 + 10 + 128) + 32
# unpacked fp32 VALU operations per second: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz (the published 157.3 TFLOP/s counts a fused multiply-add as two and
# packed-fp32 pairs twice)
PEAK_FP32_OPS = 256 * 4 * 16 * 2.4e9


def bench_encode(args):
    """Block encoders: one step quantises n experts of the V4-Flash shape from
    fp32 resident in HBM, gate and up [2048][4096] to IQ2_XXS and down
    [4096][2048] to Q2_K, each weighted by a per-expert importance vector
    (n_expert x n_columns)."""
    import numpy as np
    import torch

    import bit_quantized_expert_ds4moe_amd as ds4
    import ds4gen as g

    n, I, H = args.encode_experts, 2048, 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    log("generating %d experts of fp32 weights on the device" % n)
    gate = torch.randn((n, I, H), generator=gen, device="cuda") * 0.02
    up = torch.randn((n, I, H), generator=gen, device="cuda") * 0.02
    down = torch.randn((n, H, I), generator=gen, device="cuda") * 0.02
    imp_gu = torch.randn((n, H), generator=gen, device="cuda") ** 2
    imp_dn = torch.randn((n, I), generator=gen, device="cuda") ** 2
    grid = torch.from_numpy(g.grid(1)).cuda()
    qmap = torch.zeros(ds4.iq2_map_bytes(), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    ds4.iq2_map_build(grid.data_ptr(), qmap.data_ptr(), ws.data_ptr(), 256, st)
    out_g = torch.empty(n * I * H // 256 * 66, dtype=torch.uint8, device="cuda")
    out_u = torch.empty_like(out_g)
    out_d = torch.empty(n * H * I // 256 * 84, dtype=torch.uint8, device="cuda")

    def enc(kind):
        if kind == "gate" or kind == "up":
            src, out = (gate, out_g) if kind == "gate" else (up, out_u)
            ds4.quantize(ds4.IQ2_XXS, src.data_ptr(), n, I, H, imp_gu.data_ptr(), H,
                         grid.data_ptr(), qmap.data_ptr(), out.data_ptr(), ws.data_ptr(), 256, st)
        else:
            ds4.quantize(ds4.Q2_K, down.data_ptr(), n, H, I, imp_dn.data_ptr(), I, None, None,
                         out_d.data_ptr(), ws.data_ptr(), 256, st)

    def step():
        for k in ("gate", "up", "down"):
            enc(k)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert ds4.check(ws.data_ptr(), st) == 0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert ds4.check(ws.data_ptr(), st) == 0
    # per-kernel durations: events around each launch on the launch stream
    kev = {k: [] for k in ("gate", "up", "down")}
    for _ in range(max(2, args.steps // 2)):
        for k in kev:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            enc(k)
            b.record()
            kev[k].append((a, b))
    torch.cuda.synchronize()
    k_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in kev.items()}
    log("kernel averages (ms):", k_ms)
    vals = 3 * n * I * H
    groups = n * I * H // 32                       # per IQ2_XXS matrix
    iq2_ops = groups * ENC_OPS_IQ2_GROUP
    q2_ops = (n * H * I // 16) * ENC_OPS_Q2K_SUB
    iq2_ms = (k_ms["gate"] + k_ms["up"]) / 2
    ach = iq2_ops / (iq2_ms * 1e-3)
    res = {
        "metric": "block encoder throughput (fp32 expert weights to IQ2_XXS / Q2_K blocks, "
                  "importance-weighted)",
        "value": round(vals / (ms * 1e-3 / args.steps) / 1e9, 4), "unit": "Gvalues/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "v4flash-expert-encode", "experts_per_step": n, "hidden": H,
                   "inter": I, "gate_up": "IQ2_XXS", "down": "Q2_K",
                   "importance": "per expert and column"},
        "experts_per_s": round(n / (ms * 1e-3 / args.steps), 2),
        "kernels_ms": {k: round(v, 4) for k, v in k_ms.items()},
        "q2k_tops": round(q2_ops / (k_ms["down"] * 1e-3) / 1e12, 3),
        "roofline": {"bound": "alu", "kernel": "k_encode_iq2", "achieved": round(ach / 1e12, 3),
                     "peak": round(PEAK_FP32_OPS / 1e12, 2), "unit": "Tops/s (fp32)",
                     "frac": round(ach / PEAK_FP32_OPS, 4), "traffic": None,
                     "ops_per_launch": iq2_ops},
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = with_single_thread(cpu_baseline_encode, (args.cpu_sample,),
                                                 (max(64, args.cpu_sample // 16),))
    return res


def with_single_thread(fn, args_all, args_one):
    """The oracle baseline at all host threads (the reported value) and, on a
    smaller sample of the same workload, at one thread."""
    import oracle
    res = fn(*args_all)
    n = oracle.max_threads()
    oracle.set_threads(1)
    try:
        one = fn(*args_one)
    finally:
        oracle.set_threads(n)
    res["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                            "sample": one["sample"]}
    res["host"] = host_cpu()
    return res


def host_cpu():
    """The host's CPU model and logical CPU count (the oracle's machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline_encode(n_rows):
    """The oracle encoders on a bounded sample: n_rows rows of each matrix of
    one expert (gate and up rows of 4096 values to IQ2_XXS, down rows of 2048
    to Q2_K), scaled to values per second."""
    import numpy as np

    import ds4gen as g
    import oracle

    grid = g.grid(1)
    m = oracle.iq2_map(grid)[2]
    gu = g.normal(5, 50, 2 * n_rows * 4096, 0.0, 0.02, "f32").reshape(2, n_rows, 4096)
    dn = g.normal(5, 51, n_rows * 2 * 2048, 0.0, 0.02, "f32").reshape(1, 2 * n_rows, 2048)
    igu = (g.normal(5, 52, 4096, 0.0, 1.0, "f32") ** 2).astype(np.float32)
    idn = (g.normal(5, 53, 2048, 0.0, 1.0, "f32") ** 2).astype(np.float32)
    t0 = time.perf_counter()
    oracle.quantize(oracle.IQ2_XXS, gu, igu, grid, map_raw=m)
    oracle.quantize(oracle.Q2_K, dn, idn)
    dt = time.perf_counter() - t0
    vals = gu.size + dn.size
    return {"value": round(vals / dt / 1e9, 6), "unit": "Gvalues/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "%d rows each of one expert's gate and up (IQ2_XXS) and %d rows of its down "
                      "(Q2_K), with the workload's proportions of values" % (n_rows, 2 * n_rows)}


def cpu_baseline_stack(w, n_layers):
    """The oracle on one decode step through a sample of n_layers layers
    (normalisation, routing, experts, residual), scaled to 43 layers: the
    first n_layers layers, or, with Q4_K layers, the first n_layers/2 layers
    and then the first Q4_K layers, each kind scaled by its own layer count."""
    import ds4gen as g
    import oracle
    from ds4gen.device import host_experts, host_shared, step_inputs

    h0, tok = step_inputs(w, 1)
    resid = h0.copy()
    grid = g.grid(w.seed)
    if w.q4_layers:
        n2 = max(1, n_layers // 2)
        sample = list(range(n2)) + list(w.q4_layers[:max(1, n_layers - n2)])
    else:
        sample = list(range(n_layers))
    t_kind = {}
    for l in sample:
        t_total = 0.0
        wl = w.at_layer(l)
        nw = g.norm_weight(w, l)
        if l < w.n_hash:
            table = g.hash_table(w, l)
        else:
            W, b = g.router_weight(w, l), g.router_bias(w, l)
        t0 = time.perf_counter()
        xn = oracle.rmsnorm_bf16(resid, nw, 1e-6)
        if l < w.n_hash:
            ids, wts = oracle.route_hash(tok, table, w.E, w.K)
        else:
            ids, wts, _, _ = oracle.route(xn, "bf16", W, "f16", b, w.K)
        t_total += time.perf_counter() - t0
        mats = host_experts(w, l, ids[0])
        t0 = time.perf_counter()
        shm = host_shared(w, l) if w.shared else None
        y = oracle.moe_ffn(xn, "bf16", ids, wts, mats, (wl.gate_qt, wl.up_qt, wl.down_qt), w.H,
                           w.I, w.E, grid=grid, shared=shm, sh_I=w.I)
        resid = oracle.residual_add(resid, y)
        t_total += time.perf_counter() - t0
        t_kind.setdefault(l in w.q4_layers, []).append(t_total)
    n4 = len(w.q4_layers)
    per_token = sum(sum(t) / len(t) * (n4 if q4 else w.n_layers - n4) for q4, t in t_kind.items())
    return {"value": round(1.0 / per_token, 5), "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "one decode step through layers %s (hash and learned routing%s), "
                      "scaled to %d layers; weights regenerated outside the timed region"
                      % (",".join(map(str, sample)), ", Q4_K layers timed separately" if n4 else "",
                         w.n_layers)}


def cpu_baseline_decode(w, n_tokens):
    """The oracle (routing + expert FFN) on a bounded sample of the workload."""
    import numpy as np

    import ds4gen as g
    import oracle
    from ds4gen.device import host_experts

    threads = oracle.max_threads()
    W = g.router_weight(w, 0)
    b = g.router_bias(w, 0)
    grid = g.grid(w.seed)
    t_total = 0.0
    for i in range(n_tokens):
        x = g.activations(w, n_tok=1, first_tok=i)
        t0 = time.perf_counter()
        ids, wts, _, _ = oracle.route(x, "bf16", W, "f16", b, w.K)
        # expert blocks regenerated outside the timed region
        t_total += time.perf_counter() - t0
        mats = host_experts(w, 0, ids[0])
        t0 = time.perf_counter()
        oracle.moe_ffn(x, "bf16", ids, wts, mats, (w.gate_qt, w.up_qt, w.down_qt), w.H, w.I,
                       w.E, grid=grid)
        t_total += time.perf_counter() - t0
    return {"value": round(n_tokens / t_total, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d distinct tokens of the one-layer decode workload (routing + 6-expert "
                      "FFN in fp64), weights regenerated outside the timed region" % n_tokens}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 2000 tokens for decode-b1, 256 for stack-43)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode-b1",
                    choices=["decode-b1", "stack-43", "stack-43-q4k", "stack-43-shared", "decode-b8",
                             "prefill-512",
                             "prefill-512-q4k", "decode-sweep", "encode"])
    ap.add_argument("--encode-experts", type=int, default=8,
                    help="encode: experts quantised per step")
    ap.add_argument("--layer-copies", type=int, default=48,
                    help="decode-b1: step i runs on layer copy i mod this many independently "
                         "seeded layers (48 copies cycle 87 GB of experts and 96 MB of router "
                         "weights, so no step finds its weights in the 256 MB last-level cache)")
    ap.add_argument("--replays", type=int, default=21,
                    help="timed passes over the K steps; the median pass gives the value")
    ap.add_argument("--no-stream-probe", dest="stream_probe", action="store_false",
                    help="skip the 2 GiB streaming-read measurement")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="oracle sample: tokens (decode-b1, default 3) or layers (stack-43, default 6)")
    ap.add_argument("--sleep-cycles", type=int, default=200_000_000,
                    help="GPU spin before the per-kernel event pass")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--imatrix", action="store_true",
                    help="prefill-512: collect the importance statistics in the same call")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB, so that hardware "
                         "byte counters can be scaled against a transfer of known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; the path shards by expert or by "
              "intermediate rows across GPUs but no multi-GPU run is implemented (--gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    stack = args.workload in ("stack-43", "stack-43-q4k", "stack-43-shared")
    batched = args.workload in ("decode-b8", "prefill-512", "prefill-512-q4k")
    if args.workload == "encode":
        args.steps = 10 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
    if args.steps is None:
        args.steps = 256 if stack else 200 if batched else 50 if args.workload == "decode-sweep" else 2000
    if args.warmup is None:
        args.warmup = 8 if stack else 20 if batched else 5 if args.workload == "decode-sweep" else 200
    if args.cpu_sample is None:
        args.cpu_sample = 6 if stack else 8192 if args.workload == "encode" else 3
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d written" % (n, n))
        del src, dst
    if stack:
        res = bench_stack(args, mixed=args.workload == "stack-43-q4k",
                          shared=args.workload == "stack-43-shared")
    elif batched:
        res = bench_batched(args, args.workload)
    elif args.workload == "decode-sweep":
        res = bench_sweep(args)
    elif args.workload == "encode":
        res = bench_encode(args)
    else:
        res = bench_decode_b1(args)
    if args.stream_probe:
        res = add_stream_fracs(res, read_bandwidth())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
