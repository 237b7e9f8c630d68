"""Pins of the oracle's grouped expert FFN against torch FP64 on tensors dequantised
here independently (torch's float8 E4M3 / E8M0 decoders, the OCP E2M1 table, the
low-nibble-first packing), the exact small-value case, and the BF16-weight variant.
CPU only."""
import numpy as np
import torch

import moe_synth as syn

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def deq_e4m3(codes, scales):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).double()
    return (v.reshape(*codes.shape[:-1], -1, 32) * s[..., None]).reshape(codes.shape)


def deq_fp4(packed, scales):
    lo = E2M1[packed & 15]
    hi = E2M1[packed >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).double().numpy()
    return torch.from_numpy((v.reshape(*v.shape[:-1], -1, 32) * s[..., None]).reshape(v.shape))


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)


def small_case(seed=0, T=5, K=3, L=128, I=64, E=4):
    d = dict(L=L, I=I, E=E, expert_format=0)
    w = syn.expert_weights(d, seed)
    g = syn.rng(seed, 500)
    latent = syn.bf16_normal(g, (T, L))
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    return d, w, latent, ids


def test_ffn_mx_vs_torch_fp64(orc):
    d, w, latent, ids = small_case()
    T, K = ids.shape
    codes, scales = orc.quant_mxfp8_bf16(latent)
    pairs = np.arange(T * K, dtype=np.int32)
    pexp = ids.reshape(-1)
    hc, hs, hf = orc.ffn_up_mx(pairs, pexp, K, codes, scales, w["w13"], w["s13"])
    rows = orc.ffn_down_mx(pexp, hc, hs, w["w2"], w["s2"])
    a = deq_e4m3(codes, scales)
    I = d["I"]
    for i, p in enumerate(pairs):
        e, t = pexp[i], p // K
        W13 = deq_fp4(w["w13"][e], w["s13"][e])
        h = (W13 @ a[t]).float().double()
        g, u = h[:I], h[I:]
        act = (torch.nn.functional.silu(g) * u).float()
        got = torch.from_numpy(hf[i])
        assert torch.allclose(got, act, rtol=2e-7, atol=1e-30), (i, (got - act).abs().max())
        # the hidden codes are the quantisation of the FP32 act
        c2, s2 = orc.quant_mxfp8_f32(hf[i][None])
        assert np.array_equal(c2[0], hc[i]) and np.array_equal(s2[0], hs[i])
        W2 = deq_fp4(w["w2"][e], w["s2"][e])
        y = (W2 @ deq_e4m3(hc[i][None], hs[i][None])[0]).float().to(torch.bfloat16)
        assert torch.equal(bf(rows[i]), y), i


def test_ffn_mx_exact_small_values(orc):
    # E4M3 activations and E2M1 weights with all scales 2^0: every product and every
    # partial sum is a small dyadic rational, exact in FP32 -> h is exact
    L, I, E = 64, 32, 2
    g = np.random.default_rng(9)
    codes = g.choice(np.array([0x38, 0x30, 0x40, 0xB8, 0x00, 0x3C], np.uint8), size=(2, L))
    scales = np.full((2, L // 32), 127, np.uint8)
    w13 = g.integers(0, 256, size=(E, 2 * I, L // 2), dtype=np.uint8)
    s13 = np.full((E, 2 * I, L // 32), 127, np.uint8)
    pairs = np.array([0, 1, 2, 3], np.int32)
    pexp = np.array([0, 1, 1, 0], np.int32)
    _, _, hf = orc.ffn_up_mx(pairs, pexp, 2, codes, scales, w13, s13)
    a = deq_e4m3(codes, scales).numpy()
    for i, p in enumerate(pairs):
        W = deq_fp4(w13[pexp[i]], s13[pexp[i]]).numpy()
        h = W @ a[p // 2]
        assert np.all(h == h.astype(np.float32))
        ref = (h[:I] / (1 + np.exp(-h[:I]))) * h[I:]
        assert np.allclose(hf[i], ref.astype(np.float32), rtol=2e-7, atol=0)


def test_nibble_order_matters(orc):
    # a weight row whose even elements are 1 and odd elements 0: only even latent
    # positions contribute, which pins the low-nibble-first packing
    L, I = 64, 32
    w13 = np.zeros((1, 2 * I, L // 2), np.uint8)
    w13[0, :, :] = 0x02  # low nibble = code 2 (1.0), high nibble = 0
    s13 = np.full((1, 2 * I, L // 32), 127, np.uint8)
    codes = np.zeros((1, L), np.uint8)
    codes[0, 0::2] = 0x38  # 1.0 at even positions
    codes[0, 1::2] = 0x40  # 2.0 at odd positions
    scales = np.full((1, L // 32), 127, np.uint8)
    _, _, hf = orc.ffn_up_mx(np.array([0], np.int32), np.array([0], np.int32), 1, codes, scales,
                             w13, s13)
    g = 32.0  # 32 even positions x 1.0
    assert np.allclose(hf[0], np.float32(g / (1 + np.exp(-g)) * g))


def test_ffn_bf16_vs_torch_fp64(orc):
    L, I, E, K, T = 128, 64, 5, 2, 4
    d = dict(L=L, I=I, E=E, expert_format=1)
    w = syn.expert_weights(d, 3)
    latent = syn.bf16_normal(syn.rng(3, 501), (T, L))
    ids = np.array([[0, 4], [1, 2], [3, 0], [2, 4]], np.int32)
    pairs = np.arange(T * K, dtype=np.int32)
    rows = orc.ffn_bf16(pairs, ids.reshape(-1), K, latent, w["w13"], w["w2"])
    for p in pairs:
        e, t = ids.reshape(-1)[p], p // K
        a = bf(latent[t]).double()
        h = (bf(w["w13"][e]).double() @ a).float().to(torch.bfloat16).double()
        act = (torch.nn.functional.silu(h[:I]) * h[I:]).float().to(torch.bfloat16).double()
        y = (bf(w["w2"][e]).double() @ act).float().to(torch.bfloat16)
        got = bf(rows[p])
        # one BF16 ulp: the act rounding (FP64->FP32->BF16) may differ in a last place
        diff = (got.float() - y.float()).abs()
        assert torch.all(diff <= y.float().abs() * 2 ** -7 + 1e-6), p
