"""Seeded synthetic inputs for the routed-expert MoE FFN workloads.

Thin ctypes layer over libds4gen.so (host) and libds4gen_dev.so (device
block fill).  Every tensor is a pure function of (seed, stream, index); see
ds4gen.h for the stream definition.  This package draws inputs only: it does
not decode, route or multiply anything.
"""
import ctypes
import math
import os
from dataclasses import dataclass, replace

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# stream kinds (ds4gen.h)
ROUTER_W, ROUTER_B, GATE, UP, DOWN, SH_GATE, SH_UP, SH_DOWN, GRID, X, TID2EID, NORM, \
    ROUTE, GATES, COMMON, TOKID, RANKPERM = range(1, 18)

Q2_K, IQ2_XXS, Q8_0, Q4_K = 0, 1, 2, 3
# generator-only: Q2_K bytes drawn so that the decoded weights are zero-mean
# (dmin ~ U[3e-3, 1.35e-2] instead of the configs' U[0, 5e-3])
Q2_K_ZM = 4
BLOCK_BYTES = {Q2_K: 84, IQ2_XXS: 66, Q8_0: 34, Q4_K: 144, Q2_K_ZM: 84}
BLOCK_VALUES = {Q2_K: 256, IQ2_XXS: 256, Q8_0: 32, Q4_K: 256, Q2_K_ZM: 256}

_host = None
_dev = None


def _lib():
    global _host
    if _host is None:
        path = os.path.join(HERE, "libds4gen.so")
        if not os.path.exists(path):
            raise RuntimeError("libds4gen.so not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.ds4gen_blocks.argtypes = [ctypes.c_int, u64, u64, u64, u64, vp]
        L.ds4gen_grid.argtypes = [u64, vp]
        for f in ("ds4gen_normal_f64", "ds4gen_normal_f16", "ds4gen_normal_bf16", "ds4gen_normal_f32"):
            getattr(L, f).argtypes = [u64, u64, u64, u64, dbl, dbl, vp]
        L.ds4gen_uniform_f32.argtypes = [u64, u64, u64, u64, dbl, dbl, vp]
        L.ds4gen_uniform_int.argtypes = [u64, u64, u64, u64, ctypes.c_uint32, vp]
        L.ds4gen_mixed_bf16.argtypes = [u64, u64, u64, i64, i64, dbl, dbl, vp]
        L.ds4gen_tid2eid.argtypes = [u64, u64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
        L.ds4gen_tid2eid.restype = ctypes.c_int
        L.ds4gen_zipf_routing.argtypes = [u64, ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl, dbl, vp, vp]
        _host = L
    return _host


def _devlib():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libds4gen_dev.so")
        if not os.path.exists(path):
            raise RuntimeError("libds4gen_dev.so not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        L.ds4gen_dev_blocks.argtypes = [ctypes.c_int, u64, u64, u64, u64, vp, vp]
        L.ds4gen_dev_blocks.restype = ctypes.c_int
        _dev = L
    return _dev


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def stream(layer, kind):
    return layer * 64 + kind


def blocks(qtype, seed, strm, first, n):
    out = np.empty(int(n) * BLOCK_BYTES[qtype], dtype=np.uint8)
    _lib().ds4gen_blocks(qtype, seed, strm, first, n, _ptr(out))
    return out


def fill_device(qtype, seed, strm, first, n, dev_ptr, hip_stream=0):
    """Write blocks [first, first+n) of a stream to device memory at dev_ptr."""
    rc = _devlib().ds4gen_dev_blocks(qtype, seed, strm, first, n, ctypes.c_void_p(dev_ptr),
                                     ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError("ds4gen_dev_blocks failed (%d)" % rc)


def grid(seed):
    out = np.empty(2048, dtype=np.uint8)
    _lib().ds4gen_grid(seed, _ptr(out))
    return out


def normal(seed, strm, n, mean=0.0, std=1.0, fmt="f64", first=0):
    fn = {"f64": ("ds4gen_normal_f64", np.float64), "f32": ("ds4gen_normal_f32", np.float32),
          "f16": ("ds4gen_normal_f16", np.uint16), "bf16": ("ds4gen_normal_bf16", np.uint16)}[fmt]
    out = np.empty(int(n), dtype=fn[1])
    getattr(_lib(), fn[0])(seed, strm, first, n, mean, std, _ptr(out))
    return out


def uniform_f32(seed, strm, n, a, b, first=0):
    out = np.empty(int(n), dtype=np.float32)
    _lib().ds4gen_uniform_f32(seed, strm, first, n, a, b, _ptr(out))
    return out


def uniform_int(seed, strm, n, bound, first=0):
    out = np.empty(int(n), dtype=np.int32)
    _lib().ds4gen_uniform_int(seed, strm, first, n, bound, _ptr(out))
    return out


def mixed_bf16(seed, strm_c, strm_n, T, H, alpha, beta):
    out = np.empty((T, H), dtype=np.uint16)
    _lib().ds4gen_mixed_bf16(seed, strm_c, strm_n, T, H, alpha, beta, _ptr(out))
    return out


def tid2eid(seed, strm, first_tok, n_tok, E, K):
    out = np.empty((int(n_tok), K), dtype=np.int32)
    fails = _lib().ds4gen_tid2eid(seed, strm, first_tok, n_tok, E, K, _ptr(out))
    if fails:
        raise RuntimeError("tid2eid generation failed for %d rows" % fails)
    return out


def zipf_routing(seed, T, E, K, s=1.1, total=1.5):
    ids = np.empty((T, K), dtype=np.int32)
    gates = np.empty((T, K), dtype=np.float32)
    _lib().ds4gen_zipf_routing(seed, T, E, K, s, total, _ptr(ids), _ptr(gates))
    return ids, gates


# ---------------------------------------------------------------------------
# Workload descriptions (shapes, formats, distributions) of the five cases.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int            # tokens per call
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    K: int            # experts per token
    gate_qt: int
    up_qt: int
    down_qt: int
    x_fmt: str        # "f32" or "bf16"
    router_fmt: str   # "f32" or "f16"
    shared: bool = False
    n_layers: int = 1
    n_hash: int = 0
    vocab: int = 129280
    steps: int = 1
    routing: str = "router"   # "router" | "given-zipf"
    corr: float = 0.0         # token correlation (alpha) for batched decode
    q4_layers: tuple = ()     # layers whose routed experts are all Q4_K
    q2k_zero_mean: bool = False  # Q2_K blocks drawn zero-mean (a named variant)

    def at_layer(self, layer):
        """The description of one layer of a stack: the same workload, with
        Q4_K gate/up/down where the layer is one of q4_layers."""
        if layer in self.q4_layers:
            return replace(self, gate_qt=Q4_K, up_qt=Q4_K, down_qt=Q4_K, q4_layers=())
        return self

    def stack_expert_bytes(self):
        """Bytes of every routed expert of every layer."""
        return self.E * sum(self.at_layer(l).expert_bytes() for l in range(self.n_layers))

    def token_expert_bytes(self):
        """Routed-expert bytes one decode token reads through all layers."""
        return self.K * sum(self.at_layer(l).expert_bytes() for l in range(self.n_layers))

    @property
    def blocks_per_expert(self):
        return {"gate": self.I * self.H // BLOCK_VALUES[self.gate_qt],
                "up": self.I * self.H // BLOCK_VALUES[self.up_qt],
                "down": self.H * self.I // BLOCK_VALUES[self.down_qt]}

    def qtype(self, which):
        return {"gate": self.gate_qt, "up": self.up_qt, "down": self.down_qt,
                "sh_gate": Q8_0, "sh_up": Q8_0, "sh_down": Q8_0}[which]

    def gen_qtype(self, which):
        """The generator's block kind for a tensor: its format, with Q2_K drawn
        zero-mean in the zero-mean variant."""
        qt = self.qtype(which)
        return Q2_K_ZM if (qt == Q2_K and self.q2k_zero_mean) else qt

    def expert_bytes(self):
        b = self.blocks_per_expert
        return (b["gate"] * BLOCK_BYTES[self.gate_qt] + b["up"] * BLOCK_BYTES[self.up_qt]
                + b["down"] * BLOCK_BYTES[self.down_qt])


WORKLOADS = [
    Workload("tiny-moe-ffn-q2k", 0, 4, 256, 128, 16, 2, Q2_K, Q2_K, Q2_K, "f32", "f32"),
    Workload("v4flash-layer-decode-b1", 1, 1, 4096, 2048, 256, 6, IQ2_XXS, IQ2_XXS, Q2_K,
             "bf16", "f16"),
    Workload("v4flash-layer-decode-b8-shared-q8", 2, 8, 4096, 2048, 256, 6, IQ2_XXS, IQ2_XXS,
             Q2_K, "bf16", "f16", shared=True, corr=0.9),
    Workload("v4flash-layer-prefill-512-zipf", 3, 512, 4096, 2048, 256, 6, IQ2_XXS, IQ2_XXS,
             Q2_K, "bf16", "f16", routing="given-zipf"),
    Workload("v4flash-43-layer-stack-decode-b1", 4, 1, 4096, 2048, 256, 6, IQ2_XXS, IQ2_XXS,
             Q2_K, "bf16", "f16", n_layers=43, n_hash=3, steps=256),
    # the same stack with the routed experts of the last six layers in Q4_K
    Workload("v4flash-43-layer-stack-decode-b1-q4k-37-42", 5, 1, 4096, 2048, 256, 6, IQ2_XXS,
             IQ2_XXS, Q2_K, "bf16", "f16", n_layers=43, n_hash=3, steps=256,
             q4_layers=(37, 38, 39, 40, 41, 42)),
    # the 2-bit stack with zero-mean Q2_K down blocks (a departure from the
    # stated dmin range, kept as a named variant)
    Workload("v4flash-43-layer-stack-decode-b1-zero-mean-q2k", 6, 1, 4096, 2048, 256, 6, IQ2_XXS,
             IQ2_XXS, Q2_K, "bf16", "f16", n_layers=43, n_hash=3, steps=256, q2k_zero_mean=True),
]

KIND = {"gate": GATE, "up": UP, "down": DOWN, "sh_gate": SH_GATE, "sh_up": SH_UP,
        "sh_down": SH_DOWN}


def expert_tensor_blocks(w, layer, which, first_expert, n_experts):
    """Host bytes of experts [first, first+n) of one stacked tensor."""
    w = w.at_layer(layer)
    qt = w.gen_qtype(which)
    bpe = w.blocks_per_expert[which] if not which.startswith("sh_") else w.I * w.H // 32
    return blocks(qt, w.seed, stream(layer, KIND[which]), first_expert * bpe, n_experts * bpe)


def router_weight(w, layer):
    """Router weight [E][H]: fp32 (tiny case) or fp16 bits, N(0, 0.02^2)."""
    n = w.E * w.H
    fmt = "f32" if w.router_fmt == "f32" else "f16"
    return normal(w.seed, stream(layer, ROUTER_W), n, 0.0, 0.02, fmt).reshape(w.E, w.H)


def router_bias(w, layer):
    return uniform_f32(w.seed, stream(layer, ROUTER_B), w.E, -0.1, 0.1)


def activations(w, n_tok=None, first_tok=0, layer=0):
    """Token activations [T][H]: fp32 or bf16 bits."""
    T = w.T if n_tok is None else n_tok
    if w.corr > 0.0:
        beta = math.sqrt(1.0 - w.corr * w.corr)
        return mixed_bf16(w.seed, stream(layer, COMMON), stream(layer, X), T, w.H, w.corr, beta)
    fmt = "f32" if w.x_fmt == "f32" else "bf16"
    return normal(w.seed, stream(layer, X), T * w.H, 0.0, 1.0, fmt, first=first_tok * w.H).reshape(T, w.H)


def norm_weight(w, layer):
    return normal(w.seed, stream(layer, NORM), w.H, 1.0, 0.1, "f32")


def token_ids(w, n, first=0):
    return uniform_int(w.seed, stream(0, TOKID), n, w.vocab, first=first)


def hash_table(w, layer, first_tok=0, n_tok=None):
    n_tok = w.vocab if n_tok is None else n_tok
    return tid2eid(w.seed, stream(layer, TID2EID), first_tok, n_tok, w.E, w.K)
