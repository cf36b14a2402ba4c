"""ctypes binding of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; never by the GPU library or its binding.  The
oracle and the GPU path share no code.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
F32, F16, BF16 = 0, 1, 2
Q2_K, IQ2_XXS, Q8_0, Q4_K = 0, 1, 2, 3

_L = None


def lib():
    global _L
    if _L is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError("liboracle.so not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.or_f16_value.argtypes = [ctypes.c_uint16]
        L.or_f16_value.restype = dbl
        L.or_bf16_value.argtypes = [ctypes.c_uint16]
        L.or_bf16_value.restype = dbl
        L.or_round_bf16.argtypes = [dbl]
        L.or_round_bf16.restype = ctypes.c_uint16
        L.or_dequant.argtypes = [i32, vp, i64, vp, vp]
        L.or_dequant.restype = i32
        L.or_exact_dot.argtypes = [vp, i32, vp, i32, i64]
        L.or_exact_dot.restype = ctypes.c_float
        L.or_sqrtsoftplus.argtypes = [ctypes.c_float]
        L.or_sqrtsoftplus.restype = ctypes.c_float
        L.or_route.argtypes = [i32, i32, i32, i32, vp, i32, vp, i32, vp, dbl, vp, vp, vp, vp]
        L.or_route.restype = i32
        L.or_route_hash.argtypes = [i32, i32, i32, vp, vp, i32, dbl, vp, vp]
        L.or_route_hash.restype = i32
        L.or_permute.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.or_permute.restype = i32
        L.or_moe_ffn.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, vp, i32,
                                 i32, vp, i32, vp, i32, vp, vp, i32, i32, vp, vp, vp, vp]
        L.or_moe_ffn.restype = i32
        L.or_imatrix.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, vp, i32, vp, vp,
                                 vp, vp]
        L.or_imatrix.restype = i32
        L.or_rmsnorm_bf16.argtypes = [i32, i32, vp, vp, dbl, vp]
        L.or_rmsnorm_bf16.restype = i32
        L.or_residual_add.argtypes = [i64, vp, vp]
        L.or_max_threads.restype = i32
        L.or_set_threads.argtypes = [i32]
        L.en_f16_bits.argtypes = [ctypes.c_float]
        L.en_f16_bits.restype = ctypes.c_uint16
        L.en_iq2_map_bytes.restype = i64
        L.en_iq2_map_build.argtypes = [vp, i32, vp]
        L.en_iq2_map_build.restype = i32
        L.en_quantize.argtypes = [i32, vp, i64, i64, i64, vp, i64, vp, vp, vp]
        L.en_quantize.restype = i32
        L.en_column_energy.argtypes = [vp, i64, i64, i64, vp]
        _L = L
    return _L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def dtype_code(a, fmt):
    return {"f32": F32, "f16": F16, "bf16": BF16}[fmt]


def f16_value(bits):
    return lib().or_f16_value(int(bits))


def bf16_value(bits):
    return lib().or_bf16_value(int(bits))


def round_bf16(v):
    return lib().or_round_bf16(float(v))


def dequant(qt, blocks, grid=None):
    blocks = _c(blocks, np.uint8)
    bb = {Q2_K: 84, IQ2_XXS: 66, Q8_0: 34, Q4_K: 144}[qt]
    bv = {Q2_K: 256, IQ2_XXS: 256, Q8_0: 32, Q4_K: 256}[qt]
    n = blocks.size // bb
    out = np.empty(n * bv, dtype=np.float64)
    g = None if grid is None else _c(grid, np.uint8)
    rc = lib().or_dequant(qt, _p(blocks), n, _p(g), _p(out))
    if rc != 0:
        raise ValueError("or_dequant rc=%d" % rc)
    return out


def exact_dot(x, xfmt, w, wfmt):
    x = _c(x, np.float32 if xfmt == "f32" else np.uint16)
    w = _c(w, np.float32 if wfmt == "f32" else np.uint16)
    return lib().or_exact_dot(_p(x), dtype_code(x, xfmt), _p(w), dtype_code(w, wfmt), x.size)


def sqrtsoftplus(z):
    return lib().or_sqrtsoftplus(float(np.float32(z)))


def route(x, xfmt, W, wfmt, bias, K, scale=1.5):
    """Returns ids [T,K] int32, weights [T,K] f32, logits [T,E], scores [T,E]."""
    x = _c(x, np.float32 if xfmt == "f32" else np.uint16)
    W = _c(W, np.float32 if wfmt == "f32" else np.uint16)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = W.shape[0]
    ids = np.empty((T, K), np.int32)
    wts = np.empty((T, K), np.float32)
    z = np.empty((T, E), np.float32)
    s = np.empty((T, E), np.float32)
    rc = lib().or_route(T, H, E, K, _p(x), dtype_code(x, xfmt), _p(W), dtype_code(W, wfmt),
                        _p(bias), scale, _p(ids), _p(wts), _p(z), _p(s))
    if rc != 0:
        raise ValueError("or_route rc=%d" % rc)
    return ids, wts, z, s


def route_hash(tok, table, E, K, scale=1.5):
    tok = _c(tok, np.int32)
    table = _c(table, np.int32)
    T = tok.size
    ids = np.empty((T, K), np.int32)
    wts = np.empty((T, K), np.float32)
    rc = lib().or_route_hash(T, K, E, _p(tok), _p(table), table.shape[0], scale, _p(ids), _p(wts))
    if rc != 0:
        raise ValueError("or_route_hash rc=%d" % rc)
    return ids, wts


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, K = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    rc = lib().or_permute(T, K, E, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv))
    if rc != 0:
        raise ValueError("or_permute rc=%d" % rc)
    return counts, offsets, perm, inv


def moe_ffn(x, xfmt, ids, wts, experts, qts, H, I, E, grid=None, tokens=None, shared=None,
            sh_I=0, sh_qt=Q8_0):
    """experts: dict e -> (gate_bytes, up_bytes, down_bytes) for every expert used.
    qts: (gate_qt, up_qt, down_qt).  shared: (gate, up, down) bytes or None.
    Returns out [len(tokens), H] float32."""
    x = _c(x, np.float32 if xfmt == "f32" else np.uint16)
    ids = _c(ids, np.int32)
    wts = _c(wts, np.float32)
    T, K = ids.shape
    tokens = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    keep = []
    arrs = [(ctypes.c_void_p * E)() for _ in range(3)]
    for e, mats in experts.items():
        for j in range(3):
            a = _c(mats[j], np.uint8)
            keep.append(a)
            arrs[j][e] = a.ctypes.data
    sh = [None, None, None]
    if shared is not None:
        sh = [_c(m, np.uint8) for m in shared]
    g = None if grid is None else _c(grid, np.uint8)
    out = np.empty((tokens.size, H), np.float32)
    rc = lib().or_moe_ffn(H, I, E, K, _p(x), dtype_code(x, xfmt), _p(ids), _p(wts), _p(tokens),
                          tokens.size, qts[0], arrs[0], qts[1], arrs[1], qts[2], arrs[2], _p(g),
                          sh_I, sh_qt, _p(sh[0]), _p(sh[1]), _p(sh[2]), _p(out))
    if rc != 0:
        raise ValueError("or_moe_ffn rc=%d" % rc)
    return out


def imatrix(x, xfmt, ids, wts, experts, qts, H, I, E, grid=None):
    """Importance statistics of one call (DS4C2 sec. 5): per expert and
    column, the sum over its (token, slot) pairs of x^2 (gate/up input, [E][H])
    and of (w * h)^2 (down input, [E][I]), fp64.  experts: dict e -> (gate,
    up[, down]) bytes for every expert used; qts: (gate_qt, up_qt, ...)."""
    x = _c(x, np.float32 if xfmt == "f32" else np.uint16)
    ids = _c(ids, np.int32)
    wts = _c(wts, np.float32)
    T, K = ids.shape
    keep = []
    arrs = [(ctypes.c_void_p * E)() for _ in range(2)]
    for e, mats in experts.items():
        for j in range(2):
            a = _c(mats[j], np.uint8)
            keep.append(a)
            arrs[j][e] = a.ctypes.data
    g = None if grid is None else _c(grid, np.uint8)
    gu = np.zeros((E, H), np.float64)
    dn = np.zeros((E, I), np.float64)
    rc = lib().or_imatrix(H, I, E, K, T, _p(x), dtype_code(x, xfmt), _p(ids), _p(wts), qts[0],
                          arrs[0], qts[1], arrs[1], _p(g), _p(gu), _p(dn))
    if rc != 0:
        raise ValueError("or_imatrix rc=%d" % rc)
    return gu, dn


def rmsnorm_bf16(h, w, eps=1e-6):
    h = _c(h, np.float32)
    w = _c(w, np.float32)
    T, H = h.shape
    out = np.empty((T, H), np.uint16)
    lib().or_rmsnorm_bf16(T, H, _p(h), _p(w), eps, _p(out))
    return out


def residual_add(residual, out):
    r = _c(residual, np.float32).copy()
    o = _c(out, np.float32)
    lib().or_residual_add(r.size, _p(r), _p(o))
    return r


def set_threads(n):
    lib().or_set_threads(int(n))


def max_threads():
    return lib().or_max_threads()


# ---------------------------------------------------------------------------
# block encoders (ds4_encode.c)
# ---------------------------------------------------------------------------
IQ2_KEYS = 6561


def f16_bits(v):
    """binary32 value -> binary16 bits, round to nearest even."""
    return int(lib().en_f16_bits(float(np.float32(v))))


def iq2_map(grid, n_grid=None):
    """Neighbour map of an IQ2_XXS grid ([n][8] bytes of 8, 25, 43):
    (count [6561] uint16, idx [6561][256] uint8, raw bytes)."""
    g = _c(grid, np.uint8)
    n = g.size // 8 if n_grid is None else n_grid
    raw = np.zeros(lib().en_iq2_map_bytes(), np.uint8)
    rc = lib().en_iq2_map_build(_p(g), n, _p(raw))
    if rc != 0:
        raise ValueError("en_iq2_map_build rc=%d" % rc)
    count = raw[:2 * IQ2_KEYS].view(np.uint16)
    idx = raw[2 * IQ2_KEYS:].reshape(IQ2_KEYS, 256)
    return count, idx, raw


def quantize(qt, src, importance=None, grid=None, imp_stride=None, map_raw=None):
    """Encode src [n_mats][rows][cols] (or [rows][cols]) float32 into blocks
    (uint8, n_mats*rows*cols/256 blocks).  importance: None, [cols] (shared)
    or [n_mats][cols]."""
    x = _c(src, np.float32)
    if x.ndim == 2:
        x = x[None]
    n_mats, rows, cols = x.shape
    imp = None if importance is None else _c(importance, np.float32)
    if imp_stride is None:
        imp_stride = 0 if imp is None or imp.ndim == 1 else cols
    g = None if grid is None else _c(grid, np.uint8)
    if qt == IQ2_XXS and map_raw is None and g is not None:
        map_raw = iq2_map(g)[2]
    bb = {Q2_K: 84, IQ2_XXS: 66, Q4_K: 144, Q8_0: 34}[qt]
    out = np.zeros(n_mats * rows * cols // (32 if qt == Q8_0 else 256) * bb, np.uint8)
    rc = lib().en_quantize(qt, _p(x), n_mats, rows, cols, None if imp is None else _p(imp),
                           imp_stride, None if g is None else _p(g),
                           None if map_raw is None else _p(map_raw), _p(out))
    if rc != 0:
        raise ValueError("en_quantize rc=%d" % rc)
    return out


def column_energy(src):
    """sum_r W[r][c]^2 per matrix of src [n_mats][rows][cols], fp64."""
    x = _c(src, np.float32)
    if x.ndim == 2:
        x = x[None]
    n_mats, rows, cols = x.shape
    out = np.empty((n_mats, cols), np.float64)
    lib().en_column_energy(_p(x), n_mats, rows, cols, _p(out))
    return out
