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


_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def deq_mxfp4(packed, scales):
    """MXFP4 bytes [..., n/2] (element 2j in the low nibble) and E8M0 [..., n/32] -> FP64."""
    v = np.stack([_E2M1[packed & 15], _E2M1[packed >> 4]], axis=-1)
    v = v.reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    sh = v.reshape(*v.shape[:-1], -1, 32) * np.exp2(scales.astype(np.float64) - 127)[..., None]
    return sh.reshape(v.shape)


_E2M1_LUT = None


def _mxfp4_rows(packed, scales):
    """MXFP4 bytes [R, n/2] and E8M0 [R, n/32] of one expert -> FP64 [R, n] (byte lookup)."""
    global _E2M1_LUT
    if _E2M1_LUT is None:
        b = np.arange(256)
        _E2M1_LUT = np.stack([_E2M1[b & 15], _E2M1[b >> 4]], axis=-1)  # [256, 2]
    v = _E2M1_LUT[packed].reshape(packed.shape[0], -1)
    return (v.reshape(v.shape[0], -1, 32) * np.exp2(scales.astype(np.float64) - 127)[..., None]
            ).reshape(v.shape)


def hidden_error_bound(codes, scales, w13, s13, pairs, experts, K, I):
    """Per hidden element, a bound on |act_fp32 - act_exact| for any FP32 summation order
    of h = A W13^T: |dh| <= 64 * 2^-24 * sum_k |a_k w_k| for the gate and the up value,
    propagated through silu(g) * u (plus one FP32 rounding of act).  Computed one expert
    at a time (its weights dequantised once for all of its pairs)."""
    pairs = np.asarray(pairs)
    experts = np.asarray(experts)
    out = np.zeros((len(pairs), I))
    eps = 64 * 2.0 ** -24
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        toks = pairs[sel] // K
        A = torch.from_numpy(deq_mxfp8(codes[toks], scales[toks]))
        W = torch.from_numpy(_mxfp4_rows(w13[e], s13[e]))
        h = (A @ W.T).numpy()
        S = (A.abs() @ W.abs().T).numpy()
        g, u = h[:, :I], h[:, I:]
        sg = 1 / (1 + np.exp(-g))
        silu = g * sg
        dsilu = sg * (1 + g * (1 - sg))
        out[sel] = (np.abs(dsilu * u) * eps * S[:, :I] + np.abs(silu) * eps * S[:, I:] +
                    2.0 ** -23 * np.abs(silu * u))
    return out


def mx_latent(orc, g, T, L):
    """An MXFP8 latent quantised by the oracle from a BF16 latent N(0, 1) in which some
    elements are scaled down by 2^-13 .. 2^-16 (their codes fall on the E4M3 subnormal
    grid) and some blocks carry a largest element whose scaled value lies in [448, 512)
    (it saturates to 448), so that every code class reaches the expert kernels."""
    v = g.standard_normal((T, L)).astype(np.float32)
    small = g.random((T, L)) < 1 / 16
    v[small] *= np.exp2(-g.integers(13, 17, size=int(small.sum()))).astype(np.float32)
    blocks = v.reshape(T, L // 32, 32)
    sat = g.random((T, L // 32)) < 0.25
    tt, bb = np.nonzero(sat)
    j = g.integers(0, 32, size=len(tt))
    mag = np.abs(blocks[tt, bb]).max(axis=1)
    e = np.floor(np.log2(mag))
    blocks[tt, bb, j] = np.float32(1.9375) * np.exp2(e + 1).astype(np.float32) * np.sign(
        g.standard_normal(len(tt))).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    codes, scales = orc.quant_mxfp8_bf16(bits)
    return codes, scales


def check_hidden(got_codes, got_scales, ref_codes, ref_scales, act_exact, delta,
                 what="hidden", min_exact=0.99):
    """The MXFP8 hidden is a quantisation decided from FP32 values whose summation order
    differs between the two sides.  Most codes must equal the oracle's; every GPU code
    must be valid: within one E4M3 step (at its own block scale) of a value that lies
    within the FP32 summation-error bound `delta` of the oracle's exact act."""
    exact = np.mean(got_codes == ref_codes)
    sc_exact = np.mean(got_scales == ref_scales)
    g = deq_mxfp8(got_codes, got_scales)
    X = np.repeat(got_scales.astype(np.float64) - 127, 32, axis=-1)
    q = np.abs(g) / np.exp2(X)
    binade = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    step = np.exp2(binade - 3 + X)
    excess = np.abs(g - act_exact) - (step + delta)
    excess[q >= 448] = np.minimum(excess[q >= 448], 0)  # saturated codes: any larger value
    ratio = np.max(np.abs(g - act_exact) / (step + delta))
    say(f"  {what}: codes exact {exact:.5f}, scales exact {sc_exact:.5f}, "
        f"worst |gpu - exact| / (step + order bound) {ratio:.3f}")
    assert exact >= min_exact and sc_exact >= min_exact
    assert np.all(excess <= 1e-12)
