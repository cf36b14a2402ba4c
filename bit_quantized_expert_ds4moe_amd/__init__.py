"""Python binding of libds4moe (C ABI in include/ds4moe.h).

Argument marshalling only: every step of the MoE path runs in the HIP
kernels of libds4moe.so.  Pointers are passed as integers (for example
torch.Tensor.data_ptr()), streams as HIP stream handles
(torch.cuda.current_stream().cuda_stream).  There is no fallback: if the
library is missing, loading fails loudly.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libds4moe.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EDEVICE, EDATA = 0, -1, -2, -3, -4, -5
F32, F16, BF16 = 0, 1, 2
Q2_K, IQ2_XXS, Q8_0, Q4_K = 0, 1, 2, 3
FAULT_BAD_ID, FAULT_BAD_TOKEN, FAULT_BAD_TABLE, FAULT_UNCERTIFIED, FAULT_F16_RANGE = 1, 2, 4, 8, 16
FAULT_BAD_INPUT = 32

EXPORTED = ("ds4moe_workspace_size", "ds4moe_route", "ds4moe_permute", "ds4moe_expert_ffn",
            "ds4moe_expert_ffn_imatrix", "ds4moe_layer", "ds4moe_layer_noalloc",
            "ds4moe_profile_events", "ds4moe_read_probe", "ds4moe_check",
            "ds4moe_status_string", "ds4moe_iq2_map_bytes", "ds4moe_iq2_map_build",
            "ds4moe_quantize", "ds4moe_column_energy")
K_ROUTE, K_GATEUP, K_DOWN, K_PERMUTE, K_OTHER = range(5)


class Ds4moeError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_expert", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("routed_scale", ctypes.c_float)]


class Experts(ctypes.Structure):
    _fields_ = [("gate_qtype", ctypes.c_int32), ("up_qtype", ctypes.c_int32),
                ("down_qtype", ctypes.c_int32), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("inter", ctypes.c_int32), ("grid", ctypes.c_void_p)]


class Router(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("w_dtype", ctypes.c_int32), ("bias", ctypes.c_void_p),
                ("tid2eid", ctypes.c_void_p), ("vocab", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("router", Router), ("routed", Experts), ("shared", ctypes.POINTER(Experts)),
                ("norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libds4moe.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.ds4moe_workspace_size.argtypes = [ctypes.POINTER(Shape), i32]
        L.ds4moe_workspace_size.restype = sz
        L.ds4moe_route.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Router), vp, i32, i32, vp,
                                   vp, vp, vp, sz, vp]
        L.ds4moe_route.restype = i32
        L.ds4moe_permute.argtypes = [ctypes.POINTER(Shape), vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.ds4moe_permute.restype = i32
        L.ds4moe_expert_ffn.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Experts),
                                        ctypes.POINTER(Experts), vp, i32, i32, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.ds4moe_expert_ffn.restype = i32
        L.ds4moe_expert_ffn_imatrix.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Experts),
                                                ctypes.POINTER(Experts), vp, i32, i32, vp, vp, vp,
                                                vp, vp, vp, sz, vp]
        L.ds4moe_expert_ffn_imatrix.restype = i32
        L.ds4moe_layer.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(LayerDesc), vp, i32, vp,
                                   vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.ds4moe_layer.restype = i32
        L.ds4moe_layer_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(LayerDesc), vp,
                                           i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]
        L.ds4moe_layer_noalloc.restype = i32
        L.ds4moe_profile_events.argtypes = [i32, vp, vp]
        L.ds4moe_profile_events.restype = i32
        L.ds4moe_read_probe.argtypes = [vp, sz, vp, vp]
        L.ds4moe_read_probe.restype = i32
        L.ds4moe_check.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.ds4moe_check.restype = i32
        L.ds4moe_status_string.argtypes = [i32]
        L.ds4moe_status_string.restype = ctypes.c_char_p
        i64 = ctypes.c_int64
        L.ds4moe_iq2_map_bytes.argtypes = []
        L.ds4moe_iq2_map_bytes.restype = sz
        L.ds4moe_iq2_map_build.argtypes = [vp, vp, vp, sz, vp]
        L.ds4moe_iq2_map_build.restype = i32
        L.ds4moe_quantize.argtypes = [i32, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, sz, vp]
        L.ds4moe_quantize.restype = i32
        L.ds4moe_column_energy.argtypes = [vp, i64, i64, i64, vp, vp]
        L.ds4moe_column_energy.restype = i32
        _lib = L
    return _lib


def status_string(s):
    return lib().ds4moe_status_string(int(s)).decode()


def _ok(rc, what):
    if rc != OK:
        raise Ds4moeError(rc, what)


def shape(hidden, inter, n_expert, top_k, routed_scale=1.5):
    return Shape(hidden, inter, n_expert, top_k, routed_scale)


def experts(gate, up, down, inter, qtypes, grid=None):
    """gate/up/down/grid: device pointers (int); qtypes: (gate, up, down)."""
    return Experts(qtypes[0], qtypes[1], qtypes[2], gate, up, down, inter, grid)


def router(w=None, w_dtype=F16, bias=None, tid2eid=None, vocab=0):
    return Router(w, w_dtype, bias, tid2eid, vocab)


def layer_desc(rt, routed, shared=None, norm_w=None, norm_eps=1e-6):
    d = LayerDesc(rt, routed, None, norm_w, norm_eps)
    if shared is not None:
        d.shared = ctypes.pointer(shared)
    return d


def workspace_size(shp, n_tok):
    return lib().ds4moe_workspace_size(ctypes.byref(shp), n_tok)


def route(shp, rt, x, x_dtype, n_tok, token_ids, ids, weights, ws, ws_bytes, stream=0):
    _ok(lib().ds4moe_route(ctypes.byref(shp), ctypes.byref(rt), x, x_dtype, n_tok, token_ids, ids,
                           weights, ws, ws_bytes, stream), "ds4moe_route")


def permute(shp, ids, n_tok, counts, offsets, perm, inv, ws, ws_bytes, stream=0):
    _ok(lib().ds4moe_permute(ctypes.byref(shp), ids, n_tok, counts, offsets, perm, inv, ws,
                             ws_bytes, stream), "ds4moe_permute")


def expert_ffn(shp, routed, shared, x, x_dtype, n_tok, ids, weights, out, perm_dbg, ws, ws_bytes,
               stream=0):
    sh = ctypes.byref(shared) if shared is not None else None
    _ok(lib().ds4moe_expert_ffn(ctypes.byref(shp), ctypes.byref(routed), sh, x, x_dtype, n_tok,
                                ids, weights, out, perm_dbg, ws, ws_bytes, stream),
        "ds4moe_expert_ffn")


def expert_ffn_imatrix(shp, routed, shared, x, x_dtype, n_tok, ids, weights, out, imx_gateup,
                       imx_down, ws, ws_bytes, stream=0):
    """expert_ffn plus the importance statistics, accumulated into imx_gateup
    (fp32 [E][hidden]) and imx_down (fp32 [E][inter]), device pointers."""
    sh = ctypes.byref(shared) if shared is not None else None
    _ok(lib().ds4moe_expert_ffn_imatrix(ctypes.byref(shp), ctypes.byref(routed), sh, x, x_dtype,
                                        n_tok, ids, weights, out, imx_gateup, imx_down, ws,
                                        ws_bytes, stream),
        "ds4moe_expert_ffn_imatrix")


def layer(shp, desc, x, x_dtype, residual, out, token_ids, n_tok, ids_dbg, w_dbg, xn_dbg, ws,
          ws_bytes, stream=0):
    _ok(lib().ds4moe_layer(ctypes.byref(shp), ctypes.byref(desc), x, x_dtype, residual, out,
                           token_ids, n_tok, ids_dbg, w_dbg, xn_dbg, ws, ws_bytes, stream),
        "ds4moe_layer")


def layer_noalloc(shp, desc, x, x_dtype, residual, out, token_ids, n_tok, ids_dbg, w_dbg, xn_dbg,
                  faults, stream=0):
    """ds4moe_layer on the library's static workspace (no allocation); faults:
    device pointer to one uint32 receiving the call's fault bits, or None."""
    _ok(lib().ds4moe_layer_noalloc(ctypes.byref(shp), ctypes.byref(desc), x, x_dtype, residual,
                                   out, token_ids, n_tok, ids_dbg, w_dbg, xn_dbg, faults, stream),
        "ds4moe_layer_noalloc")


def profile_events(cls, begin, end):
    """begin/end: HIP event handles (int) or None to stop."""
    _ok(lib().ds4moe_profile_events(cls, begin, end), "ds4moe_profile_events")


def read_probe(src, nbytes, sink, stream=0):
    """Streaming read of nbytes at src (measurement only); checksum to sink."""
    _ok(lib().ds4moe_read_probe(src, nbytes, sink, stream), "ds4moe_read_probe")


def iq2_map_bytes():
    return int(lib().ds4moe_iq2_map_bytes())


def iq2_map_build(grid, map_out, ws, ws_bytes, stream=0):
    """Neighbour map of an IQ2_XXS grid (device pointers)."""
    _ok(lib().ds4moe_iq2_map_build(grid, map_out, ws, ws_bytes, stream), "ds4moe_iq2_map_build")


def quantize(qtype, src, n_mats, rows, cols, importance, imp_stride, grid, iq2_map, dst, ws,
             ws_bytes, stream=0):
    """fp32 matrices [n_mats][rows][cols] -> Q2_K / IQ2_XXS blocks (device pointers)."""
    _ok(lib().ds4moe_quantize(qtype, src, n_mats, rows, cols, importance, imp_stride, grid,
                              iq2_map, dst, ws, ws_bytes, stream), "ds4moe_quantize")


def column_energy(src, n_mats, rows, cols, out, stream=0):
    _ok(lib().ds4moe_column_energy(src, n_mats, rows, cols, out, stream), "ds4moe_column_energy")


def check(ws, stream=0):
    """Waits for the stream; returns the fault bits (0 when clean)."""
    f = ctypes.c_uint32(0)
    rc = lib().ds4moe_check(ws, stream, ctypes.byref(f))
    if rc not in (OK, EDATA):
        raise Ds4moeError(rc, "ds4moe_check")
    return f.value
