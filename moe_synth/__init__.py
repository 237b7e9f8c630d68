"""Seeded synthetic inputs for the latent-MoE decode layer.

The one module that both the GPU path (tests, bench) and the CPU oracle draw their
inputs from.  It holds none of the method's arithmetic: it draws random numbers,
truncates FP32 draws to BF16 bit patterns, and draws MXFP4 weight bytes directly
(codes from a fixed bell-shaped table, scale bytes from the fan-in), so no codec of
the method runs here.  BF16 tensors are numpy ``uint16`` bit patterns.

Every tensor has its own Philox stream keyed by (seed, tensor id[, expert]), so any
tensor or any single expert can be regenerated on its own.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids of the independent streams
_X, _W_GATE, _BIAS, _W_DOWN, _W_SGU, _W_SDN, _NORM, _W_UP, _W13, _W2, _ROWS, _WTS = range(12)

TOY = dict(T=8, H=256, L=128, E=32, K=4, I=64, S=128, unit_tokens=8, expert_format=1,
           renormalize=1, routed_scale=2.5, rms_eps=1e-5)


def full_dims(T=256, expert_format=0):
    """The wide latent MoE layer: hidden 7168, latent 3584, 896 experts, top-16,
    expert intermediate 512, shared intermediate 6144, 8-token units."""
    return dict(T=T, H=7168, L=3584, E=896, K=16, I=512, S=6144, unit_tokens=8,
                expert_format=expert_format, renormalize=1, routed_scale=2.5, rms_eps=1e-5)


def rng(seed, *key):
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(seed), *map(int, key)])))


def bf16_normal(g, shape, std=1.0):
    """N(0, std) drawn in FP32 and truncated (round toward zero) to BF16 bits."""
    v = (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_const(value, shape):
    v = np.full(shape, value, np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


# MXFP4 magnitude-code table: 7 random bits pick a magnitude code 0..7 (values
# 0, .5, 1, 1.5, 2, 3, 4, 6) with these counts out of 128, one more bit the sign.
_MAG_COUNTS = (10, 20, 20, 18, 15, 22, 15, 8)
_CODE_RMS = 2.58  # root mean square of the magnitude table above
_NIBBLE_LUT = np.concatenate([np.repeat(np.arange(8, dtype=np.uint8), _MAG_COUNTS),
                              np.repeat(np.arange(8, dtype=np.uint8) | 8, _MAG_COUNTS)])
assert _NIBBLE_LUT.shape == (256,)


def mxfp4_random(g, rows, cols, std):
    """MXFP4 weight bytes [rows, cols/2] (element 2j in the low nibble of byte j) and
    E8M0 scale bytes [rows, cols/32], drawn directly: the scale exponent of each
    32-element block is floor(log2(std / code_rms)) plus a fair coin, so element
    values have about the requested standard deviation."""
    r = np.frombuffer(g.bytes(rows * cols), dtype=np.uint8)
    nib = _NIBBLE_LUT[r]
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8).reshape(rows, cols // 2)
    base = int(np.floor(np.log2(std / _CODE_RMS)))
    coin = g.integers(0, 2, size=(rows, cols // 32), dtype=np.uint8)
    scales = (np.uint8(127 + base) + coin).astype(np.uint8)
    return packed, scales


def mxfp8_random(g, rows, cols):
    """MXFP8 activation bytes drawn directly: E4M3 codes with a uniform sign and mantissa
    and an exponent field 2 + (sum of four 2-bit draws) in [2, 14] (never the NaN code),
    and E8M0 scale bytes 120 or 121 (about the scale of an N(0,1) block)."""
    r = np.frombuffer(g.bytes(rows * cols * 2), dtype=np.uint8).reshape(2, rows * cols)
    b = r[1]
    ex = 2 + (b & 3) + ((b >> 2) & 3) + ((b >> 4) & 3) + ((b >> 6) & 3)
    codes = ((r[0] & 0x80) | (ex.astype(np.uint8) << 3) | (r[0] & 7)).astype(np.uint8)
    scales = (np.uint8(120) + g.integers(0, 2, size=(rows, cols // 32), dtype=np.uint8))
    return codes.reshape(rows, cols), scales.astype(np.uint8)


def layer_weights(d, seed=0, zipf=False, bias_seed=None, experts=True):
    """All weights of one layer.  Dense weights BF16 N(0, 1/sqrt(fan_in)); router
    bias FP32 N(0, 0.05) (toy: 0.01) or, with zipf, 0.5*(r+1)^-1.1 over a seeded
    permutation of the experts; RMSNorm weight 1 + N(0, 0.1); experts MXFP4
    (mxfp4_random, fan-in std) or, for the BF16 format, BF16 N(0, 1/sqrt(fan_in))."""
    H, L, E, I, S = d["H"], d["L"], d["E"], d["I"], d["S"]
    bseed = seed if bias_seed is None else bias_seed
    w = {}
    w["w_gate"] = bf16_normal(rng(seed, _W_GATE), (E, H), 1 / np.sqrt(H))
    w["bias"] = routing_bias(E, bseed, zipf, std=0.01 if d is TOY or E <= 64 else 0.05)
    w["w_down"] = bf16_normal(rng(seed, _W_DOWN), (L, H), 1 / np.sqrt(H))
    w["w_shared_gu"] = bf16_normal(rng(seed, _W_SGU), (2 * S, H), 1 / np.sqrt(H))
    w["w_shared_dn"] = bf16_normal(rng(seed, _W_SDN), (H, S), 1 / np.sqrt(S))
    nv = (1.0 + 0.1 * rng(seed, _NORM).standard_normal(L)).astype(np.float32)
    w["norm_w"] = (nv.view(np.uint32) >> 16).astype(np.uint16)
    w["w_up"] = bf16_normal(rng(seed, _W_UP), (H, L), 1 / np.sqrt(L))
    if experts:
        w.update(expert_weights(d, seed))
    return w


def expert_weights(d, seed=0, only=None):
    """Expert weights for every expert (or the experts in `only`, others left zero)."""
    L, E, I = d["L"], d["E"], d["I"]
    if d["expert_format"] == 1:
        w13 = np.zeros((E, 2 * I, L), np.uint16)
        w2 = np.zeros((E, L, I), np.uint16)
        for e in (range(E) if only is None else only):
            w13[e] = bf16_normal(rng(seed, _W13, e), (2 * I, L), 1 / np.sqrt(L))
            w2[e] = bf16_normal(rng(seed, _W2, e), (L, I), 1 / np.sqrt(I))
        return dict(w13=w13, w2=w2, s13=None, s2=None)
    w13 = np.zeros((E, 2 * I, L // 2), np.uint8)
    s13 = np.zeros((E, 2 * I, L // 32), np.uint8)
    w2 = np.zeros((E, L, I // 2), np.uint8)
    s2 = np.zeros((E, L, I // 32), np.uint8)

    def one(e):  # each expert has its own streams: the result is thread-order free
        w13[e], s13[e] = mxfp4_random(rng(seed, _W13, e), 2 * I, L, 1 / np.sqrt(L))
        w2[e], s2[e] = mxfp4_random(rng(seed, _W2, e), L, I, 1 / np.sqrt(I))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(one, range(E) if only is None else only))
    return dict(w13=w13, s13=s13, w2=w2, s2=s2)


def routing_bias(E, seed, zipf=False, std=0.05):
    g = rng(seed, _BIAS)
    if not zipf:
        return (g.standard_normal(E) * std).astype(np.float32)
    perm = g.permutation(E)
    b = np.zeros(E, np.float32)
    b[perm] = (0.5 * (np.arange(E, dtype=np.float64) + 1.0) ** -1.1).astype(np.float32)
    return b


def layer_input(d, seed=0, T=None):
    T = d["T"] if T is None else T
    return bf16_normal(rng(seed, _X), (T, d["H"]), 1.0)


def router_input(T=1020, H=7168, seed=0):
    return bf16_normal(rng(seed, _X), (T, H), 1.0)


def finalize_inputs(T=256, K=16, cols=3584, seed=0, invalid=False):
    """Expanded rows BF16 N(0,1) [T*K, cols]; weights FP32 = softmax over k of N(0,1);
    with invalid, slot k = t mod K of token t is marked invalid (id -1, weight 0)."""
    rows = bf16_normal(rng(seed, _ROWS), (T * K, cols), 1.0)
    z = rng(seed, _WTS).standard_normal((T, K))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    if invalid:
        t = np.arange(T)
        ids[t, t % K] = -1
        w[t, t % K] = 0.0
    return rows, w, ids


def small_int_bf16(g, shape, lo=-4, hi=4):
    """Small integers as BF16 bits (exact in BF16; products and sums stay exact in FP32
    while fewer than 2^24 / (hi^2) terms are summed)."""
    v = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)
