"""Python access to the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU product
path never imports it.

The C library is single-threaded plain loops; ctypes releases the GIL during
each call, so callers may run independent tokens in threads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_HDR = os.path.join(_HERE, "moe_oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_c_int, _c_uint, _c_double = ctypes.c_int, ctypes.c_uint, ctypes.c_double


class Dims(ctypes.Structure):
    _fields_ = [("hidden", _c_int), ("latent", _c_int), ("inter", _c_int),
                ("n_experts", _c_int), ("top_k", _c_int), ("norm_eps", _c_double),
                ("gain_per_expert", _c_int), ("expert_format", _c_int),
                ("w13_global", ctypes.POINTER(ctypes.c_float)),
                ("w2_global", ctypes.POINTER(ctypes.c_float)),
                ("post_norm_identity", _c_int)]


MXFP4, NVFP4 = 0, 1  # expert weight formats


def _dims(dims: dict, eps: float, gain_per_expert: int, fmt: int = MXFP4, w13_global=None,
          w2_global=None, post_norm_identity: int = 0):
    """Dims for the C calls; returns (Dims, keep-alive list)."""
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    keep = []
    ptrs = []
    for g in (w13_global, w2_global):
        if g is None:
            ptrs.append(None)
        else:
            a = np.ascontiguousarray(g, np.float32)
            keep.append(a)
            ptrs.append(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return Dims(H, L, I, E, K, eps, int(gain_per_expert), int(fmt), ptrs[0], ptrs[1],
                int(post_norm_identity)), keep


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain -O2, IEEE semantics)."""
    stale = (not os.path.exists(_LIB) or
             os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra",
                               "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                               "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.moe_ref_e2m1_value.restype = _c_double
        L.moe_ref_e2m1_value.argtypes = [_c_uint]
        L.moe_ref_e8m0_value.restype = _c_double
        L.moe_ref_e8m0_value.argtypes = [_c_uint]
        L.moe_ref_e4m3_value.restype = _c_double
        L.moe_ref_e4m3_value.argtypes = [_c_uint]
        L.moe_ref_nvfp4_value.restype = _c_double
        L.moe_ref_nvfp4_value.argtypes = [_u8p, _u8p, ctypes.c_float, _c_int, _c_int, _c_int]
        L.moe_ref_expert_row_fmt.restype = None
        L.moe_ref_expert_row_fmt.argtypes = [_c_int, _c_int, _c_int, _u16p, _u8p, _u8p,
                                             ctypes.c_float, _u8p, _u8p, ctypes.c_float, _u16p,
                                             _f32p]
        L.moe_ref_bf16_value.restype = _c_double
        L.moe_ref_bf16_value.argtypes = [ctypes.c_uint16]
        L.moe_ref_round_bf16.restype = ctypes.c_uint16
        L.moe_ref_round_bf16.argtypes = [_c_double]
        L.moe_ref_router_logits.restype = None
        L.moe_ref_router_logits.argtypes = [_c_int, _c_int, _c_int, _u16p, _f32p, _f32p]
        L.moe_ref_topk.restype = None
        L.moe_ref_topk.argtypes = [_c_int, _c_int, _c_int, _f32p, _i32p, _f32p]
        L.moe_ref_permute.restype = None
        L.moe_ref_permute.argtypes = [_c_int, _c_int, _c_int, _i32p, _i32p, _i32p]
        L.moe_ref_linear_bf16.restype = None
        L.moe_ref_linear_bf16.argtypes = [_c_int, _c_int, _c_int, _u16p, _u16p, _u16p]
        L.moe_ref_mxfp4_value.restype = _c_double
        L.moe_ref_mxfp4_value.argtypes = [_u8p, _u8p, _c_int, _c_int, _c_int]
        L.moe_ref_expert_row.restype = None
        L.moe_ref_expert_row.argtypes = [_c_int, _c_int, _u16p, _u8p, _u8p, _u8p, _u8p,
                                         _u16p, _f32p]
        L.moe_ref_rmsnorm_row.restype = None
        L.moe_ref_rmsnorm_row.argtypes = [_c_int, _f32p, _u16p, _c_double, _f64p]
        L.moe_ref_combine.restype = None
        L.moe_ref_combine.argtypes = [_c_int, _c_int, _f32p, _f32p, _i32p, _u16p, _c_int,
                                      _c_double, _u16p]
        L.moe_ref_combine_norm.restype = None
        L.moe_ref_combine_norm.argtypes = [_c_int, _c_int, _f32p, _f32p, _i32p, _u16p, _c_int,
                                           _c_double, _c_int, _u16p]
        L.moe_ref_latent_forward.restype = _c_int
        L.moe_ref_latent_forward.argtypes = [ctypes.POINTER(Dims), _c_int, _u16p, _f32p,
                                             _u16p, _u8p, _u8p, _u8p, _u8p, _u16p, _u16p,
                                             _u16p, _f32p, _i32p, _f32p, _u16p, _u16p,
                                             _f32p, _u16p]
        L.moe_ref_latent_forward_routed.restype = _c_int
        L.moe_ref_latent_forward_routed.argtypes = [ctypes.POINTER(Dims), _c_int, _u16p, _i32p,
                                                    _f32p, _u16p, _u8p, _u8p, _u8p, _u8p, _u16p,
                                                    _u16p, _u16p, _u16p, _u16p, _f32p, _u16p]
        L.moe_ref_router_logits_f32.restype = None
        L.moe_ref_router_logits_f32.argtypes = [_c_int, _c_int, _c_int, _f32p, _f32p, _f32p]
        L.moe_ref_pre_norm.restype = None
        L.moe_ref_pre_norm.argtypes = [_c_int, _c_int, _u16p, _u16p, _c_double, _f32p, _u16p]
        L.moe_ref_post_norm_residual.restype = None
        L.moe_ref_post_norm_residual.argtypes = [_c_int, _c_int, _u16p, _u16p, _u16p, _c_double,
                                                 _u16p]
        L.moe_ref_block_forward.restype = _c_int
        L.moe_ref_block_forward.argtypes = [ctypes.POINTER(Dims), _c_int, _u16p, _u16p, _u16p,
                                            _c_double, _f32p, _u16p, _u8p, _u8p, _u8p, _u8p,
                                            _u16p, _u16p, _u16p, _f32p, _u16p, _f32p, _i32p,
                                            _f32p, _u16p]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- number formats ----------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().moe_ref_e2m1_value(code)


def e8m0_value(byte: int) -> float:
    return lib().moe_ref_e8m0_value(byte)


def bf16_value(bits: int) -> float:
    return lib().moe_ref_bf16_value(bits)


def round_bf16(v: float) -> int:
    return int(lib().moe_ref_round_bf16(float(v)))


def e4m3_value(byte: int) -> float:
    return lib().moe_ref_e4m3_value(byte)


def nvfp4_value(codes, scales, global_scale: float, cols: int, n: int, k: int) -> float:
    return lib().moe_ref_nvfp4_value(_c(codes, np.uint8), _c(scales, np.uint8), global_scale,
                                     cols, n, k)


def expert_row_fmt(fmt: int, lat_row, w13_codes, w13_scales, w13_global, w2_codes, w2_scales,
                   w2_global):
    """expert_row in either format (NVFP4: E4M3 scales per 16 and the two
    tensors' global scales)."""
    lat_row = _c(lat_row, np.uint16)
    L = lat_row.shape[0]
    I = w2_codes.shape[1] * 2
    h = np.empty(I, np.uint16)
    row = np.empty(L, np.float32)
    lib().moe_ref_expert_row_fmt(int(fmt), L, I, lat_row, _c(w13_codes, np.uint8),
                                 _c(w13_scales, np.uint8), float(w13_global),
                                 _c(w2_codes, np.uint8), _c(w2_scales, np.uint8),
                                 float(w2_global), h, row)
    return h, row


def mxfp4_value(codes, scales, cols: int, n: int, k: int) -> float:
    return lib().moe_ref_mxfp4_value(_c(codes, np.uint8), _c(scales, np.uint8), cols, n, k)


# ---- the layer's steps ---------------------------------------------------------
def router_logits(x, router):
    """A1. x [T][H] bf16 bits, router [E][H] fp32 -> logits [T][E] fp32."""
    x = _c(x, np.uint16)
    router = _c(router, np.float32)
    T, H = x.shape
    E = router.shape[0]
    out = np.empty((T, E), np.float32)
    lib().moe_ref_router_logits(T, H, E, x, router, out)
    return out


def topk(logits, K: int):
    """A2. logits [T][E] -> ids [T][K] int32, w [T][K] fp32."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    lib().moe_ref_topk(T, E, K, logits, ids, w)
    return ids, w


def permute(ids, E: int):
    """A3. ids [T][K] -> offsets [E+1], sorted_routes [T*K] (int32)."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sr = np.empty(T * K, np.int32)
    lib().moe_ref_permute(T, K, E, ids, offsets, sr)
    return offsets, sr


def linear_bf16(x, w):
    """A4/A8. x [T][Kd] bf16, w [N][Kd] bf16 -> [T][N] bf16 bits."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    T, Kd = x.shape
    N = w.shape[0]
    y = np.empty((T, N), np.uint16)
    lib().moe_ref_linear_bf16(T, N, Kd, x, w, y)
    return y


def expert_row(lat_row, w13_codes, w13_scales, w2_codes, w2_scales):
    """A5+A6 for one route row through one expert -> (h [I] bf16, row [L] fp32)."""
    lat_row = _c(lat_row, np.uint16)
    L = lat_row.shape[0]
    I = w13_codes.shape[0] // 2
    h = np.empty(I, np.uint16)
    row = np.empty(L, np.float32)
    lib().moe_ref_expert_row(L, I, lat_row, _c(w13_codes, np.uint8), _c(w13_scales, np.uint8),
                             _c(w2_codes, np.uint8), _c(w2_scales, np.uint8), h, row)
    return h, row


def rmsnorm_row(row, gain, eps: float):
    row = _c(row, np.float32)
    out = np.empty(row.shape[0], np.float64)
    lib().moe_ref_rmsnorm_row(row.shape[0], row, _c(gain, np.uint16), eps, out)
    return out


def combine(rows, w, ids, gain, gain_per_expert: int, eps: float, post_norm_identity: int = 0):
    """A7 for one token: rows [K][L] fp32, w [K], ids [K] -> ybf [L] bf16 bits.
    post_norm_identity=1 replaces the post-expert norm by the identity."""
    rows = _c(rows, np.float32)
    K, L = rows.shape
    y = np.empty(L, np.uint16)
    lib().moe_ref_combine_norm(K, L, rows, _c(w, np.float32), _c(ids, np.int32),
                               _c(gain, np.uint16), int(gain_per_expert), eps,
                               int(post_norm_identity), y)
    return y


def latent_forward(dims: dict, x, router, pooler, w13_codes, w13_scales, w2_codes,
                   w2_scales, gain, unpooler, eps: float, gain_per_expert: int = 0,
                   fmt: int = MXFP4, w13_global=None, w2_global=None,
                   post_norm_identity: int = 0):
    """The whole layer for all tokens, with every intermediate.

    Expert tensors are the full [E][...] arrays. Returns a dict with out,
    logits, ids, w, lat, h and rows (route-major, r = t*K + k) and ybf.
    post_norm_identity=1 replaces the post-expert norm by the identity."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    d, _keep = _dims(dims, eps, gain_per_expert, fmt, w13_global, w2_global, post_norm_identity)
    r = dict(out=np.empty((T, H), np.uint16), logits=np.empty((T, E), np.float32),
             ids=np.empty((T, K), np.int32), w=np.empty((T, K), np.float32),
             lat=np.empty((T, L), np.uint16), h=np.empty((T * K, I), np.uint16),
             rows=np.empty((T * K, L), np.float32), ybf=np.empty((T, L), np.uint16))
    rc = lib().moe_ref_latent_forward(
        ctypes.byref(d), T, x, _c(router, np.float32), _c(pooler, np.uint16),
        _c(w13_codes, np.uint8), _c(w13_scales, np.uint8), _c(w2_codes, np.uint8),
        _c(w2_scales, np.uint8), _c(gain, np.uint16), _c(unpooler, np.uint16),
        r["out"], r["logits"], r["ids"], r["w"], r["lat"], r["h"], r["rows"], r["ybf"])
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return r


def latent_forward_routed(dims: dict, x, ids, w, pooler, w13_codes, w13_scales, w2_codes,
                          w2_scales, gain, unpooler, eps: float, gain_per_expert: int = 0,
                          fmt: int = MXFP4, w13_global=None, w2_global=None,
                          post_norm_identity: int = 0):
    """Steps A4 to A8 with the routing given: the replay of a recorded MoE
    routing ("Soporte de día 0 para Muse Spark Open en vLLM", section
    "Aprendizaje por refuerzo en vLLM": the trainer reuses the rollout's
    routing, R3). ids [T][K] in [0, E), a token may list an expert more than
    once, and w [T][K] is used as given. Returns out, lat, h, rows
    (route-major) and ybf."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    ids = _c(ids, np.int32).reshape(T, K)
    w = _c(w, np.float32).reshape(T, K)
    d, _keep = _dims(dims, eps, gain_per_expert, fmt, w13_global, w2_global, post_norm_identity)
    r = dict(out=np.empty((T, H), np.uint16), lat=np.empty((T, L), np.uint16),
             h=np.empty((T * K, I), np.uint16), rows=np.empty((T * K, L), np.float32),
             ybf=np.empty((T, L), np.uint16))
    rc = lib().moe_ref_latent_forward_routed(
        ctypes.byref(d), T, x, ids, w, _c(pooler, np.uint16), _c(w13_codes, np.uint8),
        _c(w13_scales, np.uint8), _c(w2_codes, np.uint8), _c(w2_scales, np.uint8),
        _c(gain, np.uint16), _c(unpooler, np.uint16), r["out"], r["lat"], r["h"], r["rows"],
        r["ybf"])
    if rc == -2:
        raise ValueError("expert id outside [0, E)")
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return r


# ---- the block around the layer ("Soporte de día 0 para Muse Spark Open en
# vLLM", "Arquitectura del modelo": out = x + post_norm(F(norm(x))); section
# "Nvidia": the router is fed by the norm's fp32 output) ----------------------
def router_logits_f32(x, router):
    x = _c(x, np.float32)
    T, H = x.shape
    E = router.shape[0]
    out = np.empty((T, E), np.float32)
    lib().moe_ref_router_logits_f32(T, H, E, x, _c(router, np.float32), out)
    return out


def pre_norm(resid, gain, eps: float):
    """RMS norm of each H-wide row: (fp32, bf16) roundings of the double result."""
    resid = _c(resid, np.uint16)
    T, H = resid.shape
    nf = np.empty((T, H), np.float32)
    nb = np.empty((T, H), np.uint16)
    lib().moe_ref_pre_norm(T, H, resid, _c(gain, np.uint16), eps, nf, nb)
    return nf, nb


def post_norm_residual(resid, f, gain, eps: float):
    resid = _c(resid, np.uint16)
    T, H = resid.shape
    out = np.empty((T, H), np.uint16)
    lib().moe_ref_post_norm_residual(T, H, resid, _c(f, np.uint16), _c(gain, np.uint16), eps, out)
    return out


def block_forward(dims: dict, resid, pre_gain, post_gain, block_eps: float, router, pooler,
                  w13_codes, w13_scales, w2_codes, w2_scales, gain, unpooler, eps: float,
                  gain_per_expert: int = 0, fmt: int = MXFP4, w13_global=None, w2_global=None):
    """out = resid + post_norm(layer(pre_norm(resid))) with every intermediate
    (n_f32, n_bf16, logits, ids, w, f = the layer's output)."""
    resid = _c(resid, np.uint16)
    T = resid.shape[0]
    H, L, I, E, K = (dims[k] for k in ("hidden", "latent", "inter", "n_experts", "top_k"))
    d, _keep = _dims(dims, eps, gain_per_expert, fmt, w13_global, w2_global)
    r = dict(out=np.empty((T, H), np.uint16), n_f32=np.empty((T, H), np.float32),
             n_bf16=np.empty((T, H), np.uint16), logits=np.empty((T, E), np.float32),
             ids=np.empty((T, K), np.int32), w=np.empty((T, K), np.float32),
             f=np.empty((T, H), np.uint16))
    rc = lib().moe_ref_block_forward(
        ctypes.byref(d), T, resid, _c(pre_gain, np.uint16), _c(post_gain, np.uint16), block_eps,
        _c(router, np.float32), _c(pooler, np.uint16), _c(w13_codes, np.uint8),
        _c(w13_scales, np.uint8), _c(w2_codes, np.uint8), _c(w2_scales, np.uint8),
        _c(gain, np.uint16), _c(unpooler, np.uint16), r["out"], r["n_f32"], r["n_bf16"],
        r["logits"], r["ids"], r["w"], r["f"])
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return r


def token_forward(dims: dict, x_row, router, pooler, gain, unpooler, eps: float,
                  gain_per_expert: int, get_expert, fmt: int = MXFP4):
    """The whole layer for one token, composed from the step functions.

    ``get_expert(e)`` returns that expert's (w13_codes, w13_scales, w2_codes,
    w2_scales) arrays (NVFP4: followed by the two tensors' global scales), so
    only touched experts need to exist on the host."""
    K = dims["top_k"]
    xr = _c(x_row, np.uint16).reshape(1, -1)
    logits = router_logits(xr, router)                       # A1
    ids, w = topk(logits, K)                                 # A2
    lat = linear_bf16(xr, pooler)[0]                         # A4
    hs, rows = [], []
    for k in range(K):                                       # A5, A6
        if fmt == NVFP4:
            c13, s13, c2, s2, g13, g2 = get_expert(int(ids[0, k]))
            h, row = expert_row_fmt(NVFP4, lat, c13, s13, g13, c2, s2, g2)
        else:
            h, row = expert_row(lat, *get_expert(int(ids[0, k])))
        hs.append(h)
        rows.append(row)
    rows = np.stack(rows)
    ybf = combine(rows, w[0], ids[0], gain, gain_per_expert, eps)   # A7
    out = linear_bf16(ybf.reshape(1, -1), unpooler)[0]       # A8
    return dict(out=out, logits=logits[0], ids=ids[0], w=w[0], lat=lat,
                h=np.stack(hs), rows=rows, ybf=ybf)
