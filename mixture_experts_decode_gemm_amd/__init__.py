"""Python binding of libmoedecode (one wide-batch latent-MoE decode step on gfx950).

Argument marshalling only: every function has the name of the C entry point it calls
(include/moedecode.h), takes torch tensors on the GPU (or None), checks dtype, device
and contiguity, passes raw pointers and the current HIP stream, and raises MoeError on
a non-zero status.  All arithmetic runs in the library's HIP kernels; there is no CPU
fallback: without the built library every call raises.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoedecode.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_FORMAT, \
    MOE_ERR_LAUNCH = range(7)
STATUS_NAMES = ["MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_ALIGN", "MOE_ERR_WORKSPACE",
                "MOE_ERR_FORMAT", "MOE_ERR_LAUNCH"]
MOE_FMT_MXFP4_MXFP8, MOE_FMT_BF16, MOE_FMT_MXFP4_MXFP8_PACKED = 0, 1, 2
MOE_LOGITS_GIVEN = 1
MOE_GATE_PACKED = 2
MOE_LINEAR_F32, MOE_LINEAR_BF16, MOE_LINEAR_ADD_BF16 = 0, 1, 2
MOE_DENSE_ROWMAJOR, MOE_DENSE_PACKED = 0, 1
WORKSPACE_FIELDS = ["logits", "ids", "weights", "counts", "offsets", "pairs", "units", "num_units",
                    "latent", "codes", "scales", "rows", "routed", "shared", "normed", "hidden",
                    "hidden_scales", "scratch"]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{fn} failed: {name}")
        self.status = status


class moe_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("tokens", "max_tokens", "hidden", "latent", "experts",
                                          "top_k", "expert_inter", "shared_inter", "unit_tokens",
                                          "expert_format", "renormalize")] + \
               [("routed_scale", C.c_float), ("rms_eps", C.c_float)]


class moe_expert_weights(C.Structure):
    _fields_ = [("w13", C.c_void_p), ("s13", C.c_void_p), ("w2", C.c_void_p), ("s2", C.c_void_p)]


class moe_layer_weights(C.Structure):
    _fields_ = [("w_gate", C.c_void_p), ("bias", C.c_void_p), ("w_down", C.c_void_p),
                ("w_shared_gu", C.c_void_p), ("w_shared_down", C.c_void_p),
                ("norm_w", C.c_void_p), ("w_up", C.c_void_p), ("experts", moe_expert_weights),
                ("dense_format", C.c_int32)]


EXPORTS = ["moe_router_topk", "moe_router_workspace_size", "moe_build_lists",
           "moe_lists_workspace_size", "moe_quant_mxfp8", "moe_grouped_ffn", "moe_grouped_ffn_stages",
           "moe_grouped_ffn_noalloc", "moe_grouped_ffn_noalloc_max_bytes", "moe_pack_expert_weights",
           "moe_ffn_workspace_size", "moe_finalize", "moe_rmsnorm", "moe_linear",
           "moe_linear_workspace_size", "moe_pack_dense_weight", "moe_silu_mul", "moe_layer",
           "moe_workspace_size",
           "moe_workspace_layout", "moe_version"]

_lib = None


def lib():
    """Load libmoedecode.so (raises if it was not built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoedecode.so is not built ({LIB_PATH}); run "
                              "`python mixture_experts_decode_gemm_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        v, i32, sz, f = C.c_void_p, C.c_int32, C.c_size_t, C.c_float
        D = C.POINTER(moe_dims)
        sig = {
            "moe_router_topk": (i32, [D, v, v, v, v, v, v, i32, v, sz, v]),
            "moe_router_workspace_size": (sz, [D]),
            "moe_build_lists": (i32, [D, v, v, v, v, v, v, v, sz, v]),
            "moe_lists_workspace_size": (sz, [D]),
            "moe_quant_mxfp8": (i32, [i32, i32, v, v, v, v]),
            "moe_grouped_ffn": (i32, [D, C.POINTER(moe_expert_weights), v, v, v, v, v, v, v, sz, v]),
            "moe_grouped_ffn_stages": (i32, [D, C.POINTER(moe_expert_weights), v, v, v, v, v, v, v,
                                             sz, i32, v]),
            "moe_grouped_ffn_noalloc": (i32, [D, C.POINTER(moe_expert_weights), v, v, v, v, v, v,
                                              v]),
            "moe_grouped_ffn_noalloc_max_bytes": (sz, []),
            "moe_ffn_workspace_size": (sz, [D]),
            "moe_pack_expert_weights": (i32, [D, C.POINTER(moe_expert_weights),
                                              C.POINTER(moe_expert_weights), v]),
            "moe_finalize": (i32, [i32, i32, i32, v, v, v, v, v]),
            "moe_rmsnorm": (i32, [i32, i32, v, v, f, v, v]),
            "moe_linear": (i32, [i32, i32, i32, v, v, v, v, i32, v, sz, v]),
            "moe_linear_workspace_size": (sz, [i32, i32, i32]),
            "moe_pack_dense_weight": (i32, [i32, i32, v, v, v]),
            "moe_silu_mul": (i32, [i32, i32, v, v, v]),
            "moe_layer": (i32, [D, C.POINTER(moe_layer_weights), v, v, v, sz, v]),
            "moe_workspace_size": (sz, [D]),
            "moe_workspace_layout": (i32, [D, C.POINTER(C.c_size_t * len(WORKSPACE_FIELDS))]),
            "moe_version": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def dims(tokens, max_tokens=None, hidden=7168, latent=3584, experts=896, top_k=16,
         expert_inter=512, shared_inter=6144, unit_tokens=8, expert_format=MOE_FMT_MXFP4_MXFP8,
         renormalize=1, routed_scale=2.5, rms_eps=1e-5):
    return moe_dims(tokens, max_tokens or tokens, hidden, latent, experts, top_k, expert_inter,
                    shared_inter, unit_tokens, expert_format, renormalize, routed_scale, rms_eps)


def dims_from(d: dict, max_tokens=None):
    """moe_dims from the oracle-style dict (T, H, L, E, K, I, S, ...)."""
    return dims(d["T"], max_tokens or d["T"], d["H"], d["L"], d["E"], d["K"], d["I"], d["S"],
                d["unit_tokens"], d["expert_format"], d["renormalize"], d["routed_scale"],
                d["rms_eps"])


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: torch.Tensor expected")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


U8, I32, F32, BF16 = torch.uint8, torch.int32, torch.float32, torch.bfloat16


def moe_version():
    return lib().moe_version().decode()


def moe_router_workspace_size(d):
    return lib().moe_router_workspace_size(C.byref(d))


def moe_lists_workspace_size(d):
    return lib().moe_lists_workspace_size(C.byref(d))


def moe_ffn_workspace_size(d):
    return lib().moe_ffn_workspace_size(C.byref(d))


def moe_workspace_size(d):
    return lib().moe_workspace_size(C.byref(d))


def moe_linear_workspace_size(M, N, K):
    return lib().moe_linear_workspace_size(M, N, K)


def moe_workspace_layout(d):
    arr = (C.c_size_t * len(WORKSPACE_FIELDS))()
    _check("moe_workspace_layout", lib().moe_workspace_layout(C.byref(d), C.byref(arr)))
    return dict(zip(WORKSPACE_FIELDS, list(arr)))


def moe_router_topk(d, x, w_gate, bias, logits, ids, weights, flags=0, workspace=None, stream=None):
    ws = _ptr(workspace, U8, "workspace")
    st = lib().moe_router_topk(C.byref(d), _ptr(x, BF16, "x"), _ptr(w_gate, BF16, "w_gate"),
                               _ptr(bias, F32, "bias"), _ptr(logits, F32, "logits"),
                               _ptr(ids, I32, "ids"), _ptr(weights, F32, "weights"), flags, ws,
                               workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("moe_router_topk", st)


def moe_build_lists(d, ids, counts, offsets, pairs, units, num_units, workspace, stream=None):
    st = lib().moe_build_lists(C.byref(d), _ptr(ids, I32, "ids"), _ptr(counts, I32, "counts"),
                               _ptr(offsets, I32, "offsets"), _ptr(pairs, I32, "pairs"),
                               _ptr(units, I32, "units"), _ptr(num_units, I32, "num_units"),
                               _ptr(workspace, U8, "workspace"), workspace.numel(),
                               _stream(stream))
    _check("moe_build_lists", st)


def moe_quant_mxfp8(x, codes, scales, stream=None):
    rows, cols = x.shape
    st = lib().moe_quant_mxfp8(rows, cols, _ptr(x, BF16, "x"), _ptr(codes, U8, "codes"),
                               _ptr(scales, U8, "scales"), _stream(stream))
    _check("moe_quant_mxfp8", st)


def expert_weights(w13, s13, w2, s2):
    """The C struct of expert weight pointers; it holds the tensors, so that their memory
    lives as long as the struct does."""
    w = moe_expert_weights(_ptr(w13, (U8, BF16), "w13"), _ptr(s13, U8, "s13"),
                           _ptr(w2, (U8, BF16), "w2"), _ptr(s2, U8, "s2"))
    w._tensors = (w13, s13, w2, s2)
    return w


def moe_grouped_ffn(d, w13, s13, w2, s2, act, act_scales, pairs, units, num_units, rows,
                    workspace, stream=None):
    w = expert_weights(w13, s13, w2, s2)
    st = lib().moe_grouped_ffn(C.byref(d), C.byref(w), _ptr(act, (U8, BF16), "act"),
                               _ptr(act_scales, U8, "act_scales"), _ptr(pairs, I32, "pairs"),
                               _ptr(units, I32, "units"), _ptr(num_units, I32, "num_units"),
                               _ptr(rows, BF16, "rows"), _ptr(workspace, U8, "workspace"),
                               workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("moe_grouped_ffn", st)


def moe_grouped_ffn_noalloc(d, w13, s13, w2, s2, act, act_scales, pairs, units, num_units, rows,
                            stream=None):
    """moe_grouped_ffn with its scratch in the library's own device array (no workspace)."""
    w = expert_weights(w13, s13, w2, s2)
    st = lib().moe_grouped_ffn_noalloc(C.byref(d), C.byref(w), _ptr(act, (U8, BF16), "act"),
                                       _ptr(act_scales, U8, "act_scales"),
                                       _ptr(pairs, I32, "pairs"), _ptr(units, I32, "units"),
                                       _ptr(num_units, I32, "num_units"), _ptr(rows, BF16, "rows"),
                                       _stream(stream))
    _check("moe_grouped_ffn_noalloc", st)


def moe_grouped_ffn_noalloc_max_bytes():
    return lib().moe_grouped_ffn_noalloc_max_bytes()


MOE_FFN_UP, MOE_FFN_DOWN = 1, 2


def moe_pack_expert_weights(d, w13, s13, w2, s2, stream=None):
    """The packed copies (w13, s13, w2, s2) of MXFP4 expert weights, for
    expert_format = MOE_FMT_MXFP4_MXFP8_PACKED (new tensors of the same shapes)."""
    out = [torch.empty_like(t) for t in (w13, s13, w2, s2)]
    src = expert_weights(w13, s13, w2, s2)
    dst = expert_weights(*out)
    st = lib().moe_pack_expert_weights(C.byref(d), C.byref(src), C.byref(dst), _stream(stream))
    _check("moe_pack_expert_weights", st)
    return tuple(out)


def moe_grouped_ffn_stages(d, w13, s13, w2, s2, act, act_scales, pairs, units, num_units, rows,
                           workspace, stages, stream=None):
    """One or both passes of the grouped FFN (MOE_FFN_UP, MOE_FFN_DOWN or their OR)."""
    w = expert_weights(w13, s13, w2, s2)
    st = lib().moe_grouped_ffn_stages(C.byref(d), C.byref(w), _ptr(act, (U8, BF16), "act"),
                                      _ptr(act_scales, U8, "act_scales"),
                                      _ptr(pairs, I32, "pairs"), _ptr(units, I32, "units"),
                                      _ptr(num_units, I32, "num_units"), _ptr(rows, BF16, "rows"),
                                      _ptr(workspace, U8, "workspace"),
                                      workspace.numel() if workspace is not None else 0,
                                      int(stages), _stream(stream))
    _check("moe_grouped_ffn_stages", st)


def moe_finalize(rows, weights, out, ids=None, stream=None):
    T, K = weights.shape
    cols = out.shape[1]
    st = lib().moe_finalize(T, K, cols, _ptr(rows, BF16, "rows"), _ptr(weights, F32, "weights"),
                            _ptr(ids, I32, "ids"), _ptr(out, BF16, "out"), _stream(stream))
    _check("moe_finalize", st)


def moe_rmsnorm(r, g, out, eps=1e-5, stream=None):
    rows, cols = r.shape
    st = lib().moe_rmsnorm(rows, cols, _ptr(r, BF16, "r"), _ptr(g, BF16, "g"), float(eps),
                           _ptr(out, BF16, "out"), _stream(stream))
    _check("moe_rmsnorm", st)


def moe_linear(x, w, out, add=None, mode=MOE_LINEAR_BF16, workspace=None, stream=None):
    M, K = x.shape
    N = w.shape[0]
    st = lib().moe_linear(M, N, K, _ptr(x, BF16, "x"), _ptr(w, BF16, "w"),
                          _ptr(out, (F32, BF16), "out"), _ptr(add, BF16, "add"), mode,
                          _ptr(workspace, U8, "workspace"),
                          workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("moe_linear", st)


def moe_pack_dense_weight(w, stream=None):
    """The packed copy of a dense BF16 weight W [N, K] (MOE_DENSE_PACKED; same shape)."""
    N, K = w.shape
    out = torch.empty_like(w)
    st = lib().moe_pack_dense_weight(N, K, _ptr(w, BF16, "w"), _ptr(out, BF16, "out"),
                                     _stream(stream))
    _check("moe_pack_dense_weight", st)
    return out


def moe_silu_mul(gu, out, stream=None):
    M, S2 = gu.shape
    st = lib().moe_silu_mul(M, S2 // 2, _ptr(gu, BF16, "gu"), _ptr(out, BF16, "out"),
                            _stream(stream))
    _check("moe_silu_mul", st)


def layer_weights(w_gate, bias, w_down, w_shared_gu, w_shared_down, norm_w, w_up, w13, s13, w2,
                  s2, dense_format=MOE_DENSE_ROWMAJOR):
    """The C struct of layer weight pointers; it holds the tensors, so that their memory
    lives as long as the struct does."""
    ew = expert_weights(w13, s13, w2, s2)
    lw = moe_layer_weights(_ptr(w_gate, BF16, "w_gate"), _ptr(bias, F32, "bias"),
                           _ptr(w_down, BF16, "w_down"), _ptr(w_shared_gu, BF16, "w_shared_gu"),
                           _ptr(w_shared_down, BF16, "w_shared_down"),
                           _ptr(norm_w, BF16, "norm_w"), _ptr(w_up, BF16, "w_up"), ew,
                           int(dense_format))
    lw._tensors = (w_gate, bias, w_down, w_shared_gu, w_shared_down, norm_w, w_up, ew._tensors)
    return lw


def moe_layer(d, weights: moe_layer_weights, x, out, workspace, stream=None):
    st = lib().moe_layer(C.byref(d), C.byref(weights), _ptr(x, BF16, "x"), _ptr(out, BF16, "out"),
                         _ptr(workspace, U8, "workspace"), workspace.numel(), _stream(stream))
    _check("moe_layer", st)


def workspace_views(d, workspace):
    """Typed views of the moe_layer workspace intermediates (first d.tokens rows)."""
    lo = moe_workspace_layout(d)
    T, E, K, L, H = d.tokens, d.experts, d.top_k, d.latent, d.hidden
    P = T * K

    def view(name, n, dtype, shape):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return workspace[lo[name]:lo[name] + nbytes].view(dtype).view(*shape)

    return dict(logits=view("logits", T * E, F32, (T, E)), ids=view("ids", P, I32, (T, K)),
                weights=view("weights", P, F32, (T, K)), counts=view("counts", E, I32, (E,)),
                offsets=view("offsets", E + 1, I32, (E + 1,)), pairs=view("pairs", P, I32, (P,)),
                num_units=view("num_units", 4, I32, (4,)),
                latent=view("latent", T * L, BF16, (T, L)), codes=view("codes", T * L, U8, (T, L)),
                scales=view("scales", T * L // 32, U8, (T, L // 32)),
                rows=view("rows", P * L, BF16, (P, L)), routed=view("routed", T * L, BF16, (T, L)),
                shared=view("shared", T * H, BF16, (T, H)),
                normed=view("normed", T * L, BF16, (T, L)),
                hidden=view("hidden", P * d.expert_inter, U8, (P, d.expert_inter)),
                hidden_scales=view("hidden_scales", P * d.expert_inter // 32, U8,
                                   (P, d.expert_inter // 32)),
                units_raw=workspace[lo["units"]:lo["num_units"]].view(I32).view(-1, 4))
