"""Helpers of the GPU parity tests: numpy <-> device tensors, BF16 views, the
tolerance rules (max |gpu - oracle| <= 2e-2 x RMS(oracle) for floating outputs; ulp
distance for BF16), and cached full-size synthetic weights."""
import functools
import sys

import numpy as np
import torch

import moe_synth as syn

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """numpy -> cuda tensor; uint16 arrays become bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    """cuda tensor -> numpy; bfloat16 becomes uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32(bits_u16):
    return (np.asarray(bits_u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_close(got, ref, what, tol=TOL):
    """max |got - ref| <= tol x RMS(ref) over FP32/FP64 outputs."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    say(f"  {what}: max|err| = {err:.3e}, rms = {rms:.3e}, ratio = {err / max(rms, 1e-30):.2e}")
    assert np.all(np.isfinite(got)), what
    assert err <= tol * rms, f"{what}: max err {err} > {tol} x rms {rms}"


def assert_close_bf16(got_bits, ref_bits, what, tol=TOL):
    """BF16 outputs: every element within tol x RMS(ref), or one BF16 ulp of the oracle's
    element (two correct roundings of nearly equal FP32 values can land one ulp apart, and
    one ulp of an element above ~4 x RMS already exceeds 2e-2 x RMS)."""
    g, r = f32(got_bits).astype(np.float64), f32(ref_bits).astype(np.float64)
    rms = np.sqrt(np.mean(r * r))
    err = np.abs(g - r)
    ulp = bf16_ulp_dist(got_bits, ref_bits)
    bad = (err > tol * rms) & (ulp > 1)
    big = err[ulp > 1].max() if np.any(ulp > 1) else 0.0
    say(f"  {what}: rms = {rms:.3e}, elements 1 ulp apart: {int(np.sum(ulp == 1))}/{ulp.size}, "
        f"max|err| beyond 1 ulp = {big:.3e} (ratio {big / max(rms, 1e-30):.2e})")
    assert np.all(np.isfinite(g)), what
    assert not np.any(bad), f"{what}: {int(bad.sum())} elements beyond {tol} x rms and 1 ulp"


def bf16_ulp_dist(a, b):
    """|a - b| in BF16 ulps (sign-magnitude bit patterns mapped to a monotone integer)."""
    def key(x):
        x = np.asarray(x, np.uint16).astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


@functools.lru_cache(maxsize=1)
def _base_weights(seed=0):
    d = syn.full_dims(256)
    w = syn.layer_weights(d, seed=seed)
    dw = {k: (dev(v) if v is not None else None) for k, v in w.items()}
    return w, dw


def full_weights(seed=0, zipf=False):
    """The full-size layer's weights (hidden 7168, latent 3584, 896 MXFP4 experts),
    generated once per process (numpy host copies and device tensors); the Zipf variant
    differs only in the routing bias (seed 1, Zipf(1.1)-skewed)."""
    w, dw = _base_weights(seed)
    if not zipf:
        return w, dw
    w = dict(w)
    dw = dict(dw)
    w["bias"] = syn.routing_bias(896, 1, True)
    dw["bias"] = dev(w["bias"])
    return w, dw


_E4M3 = None


def e4m3_table():
    global _E4M3
    if _E4M3 is None:
        import torch as _t
        _E4M3 = _t.arange(256, dtype=_t.uint8).view(_t.float8_e4m3fn).double().numpy()
    return _E4M3


def deq_mxfp8(codes, scales):
    v = e4m3_table()[codes].reshape(*codes.shape[:-1], -1, 32)
    return (v * np.exp2(scales.astype(np.float64) - 127)[..., None]).reshape(codes.shape)


def check_hidden(got_codes, got_scales, ref_codes, ref_scales, what="hidden", min_exact=0.99):
    """MXFP8 hidden codes decided from FP32 values that differ only in accumulation order:
    most codes equal, and every differing element within one E4M3 step (1/8 of its binade,
    or one subnormal step) of the oracle's value at the larger of the two block scales."""
    exact = np.mean(got_codes == ref_codes)
    sc_exact = np.mean(got_scales == ref_scales)
    g = deq_mxfp8(got_codes, got_scales)
    r = deq_mxfp8(ref_codes, ref_scales)
    xs = np.maximum(got_scales, ref_scales).astype(np.float64) - 127
    xs = np.repeat(xs, 32, axis=-1)
    bound = np.maximum(np.abs(g), np.abs(r)) / 8 + np.exp2(xs - 9) + 1e-30
    worst = np.max(np.abs(g - r) / bound)
    say(f"  {what}: codes exact {exact:.5f}, scales exact {sc_exact:.5f}, "
        f"worst diff / one-step bound {worst:.3f}")
    assert exact >= min_exact and sc_exact >= min_exact
    assert worst <= 1.0 + 1e-9
