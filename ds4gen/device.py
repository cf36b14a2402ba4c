"""Device-resident synthetic inputs (PyTorch tensors on the GPU).

Input construction only: expert blocks are written on the device by the
generator's fill kernel (identical bytes to the host generator), small
tensors are drawn on the host and copied.  PyTorch serves as the allocator.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import ds4gen as g


def _stream():
    return torch.cuda.current_stream().cuda_stream


def expert_tensor(w, layer, which, n_experts=None):
    """All experts of one stacked tensor, filled on the device."""
    w = w.at_layer(layer)
    qt = w.gen_qtype(which)
    if which.startswith("sh_"):
        n_experts = 1
        bpe = w.I * w.H // g.BLOCK_VALUES[qt]
    else:
        n_experts = w.E if n_experts is None else n_experts
        bpe = w.blocks_per_expert[which]
    nb = n_experts * bpe
    t = torch.empty(nb * g.BLOCK_BYTES[qt], dtype=torch.uint8, device="cuda")
    g.fill_device(qt, w.seed, g.stream(layer, g.KIND[which]), 0, nb, t.data_ptr(), _stream())
    return t


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


@dataclass
class LayerTensors:
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    grid: torch.Tensor
    router_w: Optional[torch.Tensor]
    bias: Optional[torch.Tensor]
    tid2eid: Optional[torch.Tensor]
    norm_w: Optional[torch.Tensor]
    shared: Optional[tuple]


def make_layer(w, layer, hashed=False, norm=False, grid=None):
    gate = expert_tensor(w, layer, "gate")
    up = expert_tensor(w, layer, "up")
    down = expert_tensor(w, layer, "down")
    gd = grid if grid is not None else to_dev(g.grid(w.seed))
    rw = bias = tab = nw = None
    if hashed:
        tab = to_dev(g.hash_table(w, layer))
    else:
        rw = to_dev(g.router_weight(w, layer))
        bias = to_dev(g.router_bias(w, layer))
    if norm:
        nw = to_dev(g.norm_weight(w, layer))
    sh = None
    if w.shared:
        sh = tuple(expert_tensor(w, layer, k) for k in ("sh_gate", "sh_up", "sh_down"))
    return LayerTensors(gate, up, down, gd, rw, bias, tab, nw, sh)


def host_experts(w, layer, experts):
    """Host bytes of the listed experts, for the oracle: {e: (gate, up, down)}."""
    return {int(e): tuple(g.expert_tensor_blocks(w, layer, which, int(e), 1)
                          for which in ("gate", "up", "down")) for e in experts}


def host_shared(w, layer):
    return tuple(g.expert_tensor_blocks(w, layer, k, 0, 1) for k in ("sh_gate", "sh_up", "sh_down"))


def make_stack(w, log=None):
    """All layers of a decode stack: layers < w.n_hash use hash routing, the
    rest a learned router; every layer has an RMSNorm weight; the formats of
    each layer's experts are w.at_layer(layer)'s.  Expert
    tensors of every layer are distinct (the layer index is part of the
    stream) and generated on the device."""
    grid = to_dev(g.grid(w.seed))
    layers = []
    done = 0
    for l in range(w.n_layers):
        layers.append(make_layer(w, l, hashed=l < w.n_hash, norm=True, grid=grid))
        done += w.E * w.at_layer(l).expert_bytes()
        if log and (l % 8 == 7 or l == w.n_layers - 1):
            log("  generated layer %d / %d (%.1f GB of experts)" % (l + 1, w.n_layers, done / 1e9))
    return layers


def step_inputs(w, n_steps, first_step=0):
    """Per decode step: a fresh hidden state bf16 N(0,1) widened to fp32 (the
    residual stream entering layer 0) and a token id uniform over the vocab."""
    h0 = g.normal(w.seed, g.stream(0, g.X), n_steps * w.H, 0.0, 1.0, "bf16",
                  first=first_step * w.H).reshape(n_steps, w.H)
    h0f = (h0.astype(np.uint32) << 16).view(np.float32)
    tok = g.token_ids(w, n_steps, first=first_step)
    return h0f, tok
