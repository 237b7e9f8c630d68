"""The plain CPU oracle of one wide-batch latent-MoE decode step (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The GPU library never uses it.
Arrays are numpy, row-major and contiguous; BF16 tensors are ``uint16`` bit patterns.
Each function mirrors one step of the layer; the C source cites the passage of the
pages each step follows.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


class Dims(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("T", "H", "L", "E", "K", "I", "S", "unit_tokens",
                                        "expert_format", "renormalize")] + \
               [("routed_scale", C.c_float), ("rms_eps", C.c_float)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_gate", "bias", "w_down", "w_shared_gu",
                                           "w_shared_dn", "norm_w", "w_up", "w13", "s13",
                                           "w2", "s2")]


class Trace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("logits", "ids", "weights", "latent", "codes",
                                           "scales", "rows", "routed", "normed", "shared")]


def _declare(L):
    v, i, f, u8, u16 = C.c_void_p, C.c_int, C.c_float, C.c_uint8, C.c_uint16
    sig = {
        "orc_bf16_to_f32": (f, [u16]),
        "orc_f32_to_bf16": (u16, [f]),
        "orc_e4m3_value": (C.c_double, [u8]),
        "orc_e4m3_encode": (u8, [C.c_double]),
        "orc_e2m1_value": (C.c_double, [u8]),
        "orc_e8m0_value": (C.c_double, [u8]),
        "orc_exp_defined": (f, [f]),
        "orc_sigmoid": (f, [f]),
        "orc_sigmoid_constants": (None, [v]),
        "orc_linear_f32": (None, [i, i, i, v, v, v]),
        "orc_topk": (None, [i, i, i, v, v, i, f, v, v]),
        "orc_build_lists": (i, [i, i, i, i, v, v, v, v, v, v]),
        "orc_quant_mxfp8_bf16": (None, [i, i, v, v, v]),
        "orc_quant_mxfp8_f32": (None, [i, i, v, v, v]),
        "orc_ffn_up_mx": (None, [i, v, v, i, i, i, v, v, v, v, v, v, v]),
        "orc_ffn_down_mx": (None, [i, v, i, i, v, v, v, v, v]),
        "orc_ffn_bf16": (None, [i, v, v, i, i, i, v, v, v, v]),
        "orc_finalize": (None, [i, i, i, v, v, v, v]),
        "orc_rmsnorm": (None, [i, i, v, v, f, v]),
        "orc_linear_bf16": (None, [i, i, i, v, v, v]),
        "orc_linear_add_bf16": (None, [i, i, i, v, v, v, v]),
        "orc_silu_mul_bf16": (None, [i, i, v, v]),
        "orc_layer": (None, [C.POINTER(Dims), C.POINTER(Weights), v, v, C.POINTER(Trace)]),
        "orc_threads": (i, []),
        "orc_set_threads": (None, [i]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array expected"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- codecs (scalar) -------------------------------------------------------------------
def bf16_to_f32(b):
    return lib().orc_bf16_to_f32(int(b))


def f32_to_bf16(x):
    return lib().orc_f32_to_bf16(float(x))


def e4m3_value(c):
    return lib().orc_e4m3_value(int(c))


def e4m3_encode(x):
    return lib().orc_e4m3_encode(float(x))


def e2m1_value(n):
    return lib().orc_e2m1_value(int(n))


def e8m0_value(b):
    return lib().orc_e8m0_value(int(b))


def exp_defined(z):
    return lib().orc_exp_defined(float(z))


def sigmoid(x):
    return lib().orc_sigmoid(float(x))


def sigmoid_constants():
    out = np.zeros(11, np.float32)
    lib().orc_sigmoid_constants(_p(out))
    return out


def threads():
    return lib().orc_threads()


def set_threads(n):
    """Thread count of the oracle's parallel loops (for timing; results do not depend on it)."""
    lib().orc_set_threads(int(n))


# ---- steps ------------------------------------------------------------------------------
def linear_f32(x, w):
    x, w = _c(x, np.uint16), _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N), np.float32)
    lib().orc_linear_f32(M, N, K, _p(x), _p(w), _p(out))
    return out


def linear_bf16(x, w):
    x, w = _c(x, np.uint16), _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N), np.uint16)
    lib().orc_linear_bf16(M, N, K, _p(x), _p(w), _p(out))
    return out


def linear_add_bf16(x, w, add):
    x, w, add = _c(x, np.uint16), _c(w, np.uint16), _c(add, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N), np.uint16)
    lib().orc_linear_add_bf16(M, N, K, _p(x), _p(w), _p(add), _p(out))
    return out


def silu_mul_bf16(gu):
    gu = _c(gu, np.uint16)
    M, S2 = gu.shape
    out = np.empty((M, S2 // 2), np.uint16)
    lib().orc_silu_mul_bf16(M, S2 // 2, _p(gu), _p(out))
    return out


def topk(logits, bias, K, renormalize=1, scale=2.5):
    logits, bias = _c(logits, np.float32), _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    lib().orc_topk(T, E, K, _p(logits), _p(bias), int(renormalize), float(scale), _p(ids), _p(w))
    return ids, w


def build_lists(ids, E, unit_tokens=8):
    ids = _c(ids, np.int32)
    T, K = ids.shape
    P = T * K
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pairs = np.full(max(P, 1), -1, np.int32)
    units = np.zeros((P + E + 1, 4), np.int32)
    nu = np.zeros(4, np.int32)
    lib().orc_build_lists(T, K, E, unit_tokens, _p(ids), _p(counts), _p(offsets), _p(pairs),
                          _p(units), _p(nu))
    n = int(offsets[E])
    return dict(counts=counts, offsets=offsets, pairs=pairs[:n].copy(),
                units=units[: int(nu[0])].copy(), num_units=int(nu[0]), dropped=int(nu[1]),
                touched=int(nu[2]))


def quant_mxfp8_bf16(x):
    x = _c(x, np.uint16)
    R, Cc = x.shape
    codes = np.empty((R, Cc), np.uint8)
    scales = np.empty((R, Cc // 32), np.uint8)
    lib().orc_quant_mxfp8_bf16(R, Cc, _p(x), _p(codes), _p(scales))
    return codes, scales


def quant_mxfp8_f32(x):
    x = _c(x, np.float32)
    R, Cc = x.shape
    codes = np.empty((R, Cc), np.uint8)
    scales = np.empty((R, Cc // 32), np.uint8)
    lib().orc_quant_mxfp8_f32(R, Cc, _p(x), _p(codes), _p(scales))
    return codes, scales


def ffn_up_mx(pair_ids, pair_experts, K, codes, scales, w13, s13):
    """hidden MXFP8 codes [n, I], scales [n, I/32], and the FP32 act before quantisation"""
    pair_ids, pair_experts = _c(pair_ids, np.int32), _c(pair_experts, np.int32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    w13, s13 = _c(w13, np.uint8), _c(s13, np.uint8)
    n = len(pair_ids)
    L = codes.shape[1]
    I = w13.shape[1] // 2
    hc = np.empty((n, I), np.uint8)
    hs = np.empty((n, I // 32), np.uint8)
    hf = np.empty((n, I), np.float32)
    lib().orc_ffn_up_mx(n, _p(pair_ids), _p(pair_experts), K, L, I, _p(codes), _p(scales),
                        _p(w13), _p(s13), _p(hc), _p(hs), _p(hf))
    return hc, hs, hf


def ffn_down_mx(pair_experts, hid_codes, hid_scales, w2, s2):
    pair_experts = _c(pair_experts, np.int32)
    hid_codes, hid_scales = _c(hid_codes, np.uint8), _c(hid_scales, np.uint8)
    w2, s2 = _c(w2, np.uint8), _c(s2, np.uint8)
    n, I = hid_codes.shape
    L = w2.shape[1]
    rows = np.empty((n, L), np.uint16)
    lib().orc_ffn_down_mx(n, _p(pair_experts), L, I, _p(hid_codes), _p(hid_scales), _p(w2),
                          _p(s2), _p(rows))
    return rows


def ffn_bf16(pair_ids, pair_experts, K, latent, w13, w2):
    pair_ids, pair_experts = _c(pair_ids, np.int32), _c(pair_experts, np.int32)
    latent, w13, w2 = _c(latent, np.uint16), _c(w13, np.uint16), _c(w2, np.uint16)
    n = len(pair_ids)
    L = latent.shape[1]
    I = w13.shape[1] // 2
    rows = np.empty((n, L), np.uint16)
    lib().orc_ffn_bf16(n, _p(pair_ids), _p(pair_experts), K, L, I, _p(latent), _p(w13), _p(w2),
                       _p(rows))
    return rows


def finalize(rows, weights, ids=None):
    weights = _c(weights, np.float32)
    T, K = weights.shape
    rows = _c(rows, np.uint16)
    cols = rows.shape[-1]
    out = np.empty((T, cols), np.uint16)
    ids = None if ids is None else _c(ids, np.int32)
    lib().orc_finalize(T, K, cols, _p(rows), _p(weights), _p(ids), _p(out))
    return out


def rmsnorm(r, g, eps=1e-5):
    r, g = _c(r, np.uint16), _c(g, np.uint16)
    T, cols = r.shape
    out = np.empty((T, cols), np.uint16)
    lib().orc_rmsnorm(T, cols, _p(r), _p(g), float(eps), _p(out))
    return out


def layer(dims: dict, weights: dict, x, trace: bool = False):
    """The whole layer on the rows of x.  dims: T,H,L,E,K,I,S,unit_tokens,expert_format,
    renormalize,routed_scale,rms_eps.  weights: numpy arrays named as in Weights."""
    x = _c(x, np.uint16)
    d = Dims(**{k: dims[k] for k, _ in Dims._fields_})
    keep = {}
    wargs = {}
    for name, _ in Weights._fields_:
        a = weights.get(name)
        if a is not None:
            a = np.ascontiguousarray(a)
            keep[name] = a
            wargs[name] = a.ctypes.data
    w = Weights(**wargs)
    T, H, L, E, K = d.T, d.H, d.L, d.E, d.K
    out = np.empty((T, H), np.uint16)
    tr = None
    bufs = {}
    if trace:
        bufs = dict(logits=np.empty((T, E), np.float32), ids=np.empty((T, K), np.int32),
                    weights=np.empty((T, K), np.float32), latent=np.empty((T, L), np.uint16),
                    codes=np.zeros((T, L), np.uint8), scales=np.zeros((T, L // 32), np.uint8),
                    rows=np.empty((T * K, L), np.uint16), routed=np.empty((T, L), np.uint16),
                    normed=np.empty((T, L), np.uint16), shared=np.empty((T, H), np.uint16))
        tr = Trace(**{k: v.ctypes.data for k, v in bufs.items()})
    lib().orc_layer(C.byref(d), C.byref(w), _p(x), _p(out), C.byref(tr) if tr else None)
    del keep
    if trace:
        return out, bufs
    return out
