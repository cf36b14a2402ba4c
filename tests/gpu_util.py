"""Helpers shared by the GPU parity tests: device workspace, pointers, the
tolerance check, and calls into the oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import bit_quantized_expert_ds4moe_amd as ds4
import ds4gen as g

# Tolerances of the path (max |err| relative to the RMS of the oracle output)
TOL_FP32 = 2e-3
TOL_BF16_MFMA = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ptr(t):
    return None if t is None else t.data_ptr()


def stream():
    return torch.cuda.current_stream().cuda_stream


def workspace(shp, n_tok):
    nb = ds4.workspace_size(shp, n_tok)
    assert nb > 0
    return torch.zeros(nb, dtype=torch.uint8, device="cuda"), nb


def check_clean(ws):
    f = ds4.check(ptr(ws), stream())
    assert f == 0, "device fault bits 0x%x" % f


def covering_tokens(ids, extra=()):
    """Tokens whose routes together touch every expert that any token uses
    (greedy set cover), plus `extra`: checking their whole outputs checks
    every touched expert's gate, up and down at least once."""
    ids = np.asarray(ids)
    left = set(np.unique(ids).tolist())
    rows = [set(r.tolist()) for r in ids]
    toks = set(int(t) for t in extra)
    for t in toks:
        left -= rows[t]
    while left:
        best = max(range(len(rows)), key=lambda t: len(left & rows[t]))
        toks.add(best)
        left -= rows[best]
    return np.array(sorted(toks))


def max_rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want * want))
    return float(np.max(np.abs(got - want)) / rms)


def shape_of(w):
    return ds4.shape(w.H, w.I, w.E, w.K, 1.5)


def experts_of(lt, w):
    return ds4.experts(ptr(lt.gate), ptr(lt.up), ptr(lt.down), w.I,
                       (w.gate_qt, w.up_qt, w.down_qt), grid=ptr(lt.grid))


def shared_of(lt, w):
    if lt.shared is None:
        return None
    return ds4.experts(ptr(lt.shared[0]), ptr(lt.shared[1]), ptr(lt.shared[2]), w.I,
                       (g.Q8_0, g.Q8_0, g.Q8_0), grid=ptr(lt.grid))


def x_fmt(w):
    return "f32" if w.x_fmt == "f32" else "bf16"


def x_dtype(w):
    return ds4.F32 if w.x_fmt == "f32" else ds4.BF16
