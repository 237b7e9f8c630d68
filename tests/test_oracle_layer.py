"""Pin of the oracle's whole layer on the toy latent MoE (T=8, hidden 256, latent 128,
32 experts, top-4, BF16 experts) against a composition written here with torch FP64
ops (torch's own sigmoid, sort and matmul), and a check that the layer is per-token
independent (the full-size sampled parity relies on it).  CPU only."""
import numpy as np
import torch

import moe_synth as syn


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double()


def rb(t):
    """round an FP64 tensor through FP32 to BF16 and back to FP64"""
    return t.float().to(torch.bfloat16).double()


def torch_layer(d, w, x):
    T, E, K, I = d["T"], d["E"], d["K"], d["I"]
    xt = bf(x)
    logits = (xt @ bf(w["w_gate"]).T).float().double()
    s = torch.sigmoid(logits)
    key = s.float() + torch.from_numpy(w["bias"])
    order = torch.sort(key, dim=1, descending=True, stable=True).indices[:, :K]
    ws = torch.gather(s.float(), 1, order)
    ws = ws / ws.sum(dim=1, keepdim=True)
    ws = (ws * d["routed_scale"]).double()
    latent = rb(xt @ bf(w["w_down"]).T)
    routed = torch.zeros(T, d["L"], dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(order[t, k])
            h = rb(bf(w["w13"][e]) @ latent[t])
            act = rb(torch.nn.functional.silu(h[:I]) * h[I:])
            y = rb(bf(w["w2"][e]) @ act)
            routed[t] += ws[t, k] * y
    routed = rb(routed)
    ms = (routed * routed).mean(dim=1, keepdim=True)
    normed = rb(routed / torch.sqrt(ms + d["rms_eps"]) * bf(w["norm_w"]))
    gu = rb(xt @ bf(w["w_shared_gu"]).T)
    S = d["S"]
    a = rb(torch.nn.functional.silu(gu[:, :S]) * gu[:, S:])
    shared = rb(a @ bf(w["w_shared_dn"]).T)
    out = rb(shared + normed @ bf(w["w_up"]).T)
    return out, order.numpy().astype(np.int32)


def test_toy_layer_vs_torch_fp64(orc):
    d = dict(syn.TOY)
    w = syn.layer_weights(d, seed=0)
    x = syn.layer_input(d, seed=0)
    out, tr = orc.layer(d, w, x, trace=True)
    ref, ids = torch_layer(d, w, x)
    assert np.array_equal(tr["ids"], ids)
    o = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double()
    rms = ref.pow(2).mean().sqrt()
    assert (o - ref).abs().max() <= 2e-2 * rms


def test_layer_is_per_token(orc):
    d = dict(syn.TOY)
    w = syn.layer_weights(d, seed=0)
    x = syn.layer_input(d, seed=0)
    full = orc.layer(d, w, x)
    sub = [1, 6]
    d2 = dict(d, T=len(sub))
    part = orc.layer(d2, w, x[sub])
    assert np.array_equal(full[sub], part)


# ---- the MXFP4 x MXFP8 layer ---------------------------------------------------------------
# Written here from the definitions, independently of the oracle: OCP MX v1.0 block scales
# (X = floor(log2 amax) - 8, via torch.frexp), E4M3 codes by torch's float8_e4m3fn cast after a
# clamp to +-448 (RNE, saturating), E8M0 and E4M3 decoding by torch's float8 views, E2M1 by the
# OCP value table with the even element in the low nibble.  The dense weights and x are small
# integers times powers of two, so every dense dot product is exact in FP32 and FP64 alike, and
# every expert dot product (E4M3 x E2M1 times power-of-two scales) is exact in FP64: the
# discrete results (ids, latent, codes, expert rows) can be compared bit for bit.
E2M1 = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6],
                    dtype=torch.float64)


def pow2_ints(g, shape, lo, hi, shift):
    """BF16 bits of integers in [lo, hi] times 2^-shift (exact in BF16)."""
    v = (g.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(2.0 ** -shift))
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def mx_quant(v):
    """FP64 [R, C] (values exact in FP32) -> E4M3 codes [R, C] and E8M0 bytes [R, C/32]."""
    R, C = v.shape
    b = v.reshape(R, C // 32, 32)
    amax = b.abs().amax(-1)
    _, ex = torch.frexp(amax)              # amax = m 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    X = (ex.long() - 1 - 8).clamp(-127, 127)
    X = torch.where(amax == 0, torch.full_like(X, -127), X)
    q = (b * torch.exp2(-X.double())[..., None]).float().clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return codes, (X + 127).to(torch.uint8)


def mx_dequant8(codes, scales):
    v = codes.view(torch.float8_e4m3fn).double()
    s = scales.view(torch.float8_e8m0fnu).double()
    return (v.reshape(*codes.shape[:-1], -1, 32) * s[..., None]).reshape(codes.shape)


def mx_dequant4(packed, scales):
    p = torch.from_numpy(np.ascontiguousarray(packed)).long()
    v = torch.stack([E2M1[p & 15], E2M1[p >> 4]], dim=-1).reshape(*p.shape[:-1], -1)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).double()
    return (v.reshape(*v.shape[:-1], -1, 32) * s[..., None]).reshape(v.shape)


def torch_mx_layer(d, w, x):
    """The layer with MXFP4 experts and MXFP8 activations, composed from torch FP64 ops in
    the stock order: routing, the BF16 latent and its MXFP8 codes, per (token, slot) pair the
    expert's gate/up product, SiLU-and-mul, the MXFP8 hidden and the down product rounded to
    BF16 (stored at row t K + k), Finalize, RMSNorm, the shared expert and the up-projection
    added into it.  Returns the output and the intermediates."""
    T, E, K, I, S, L = d["T"], d["E"], d["K"], d["I"], d["S"], d["L"]
    xt = bf(x)
    logits = (xt @ bf(w["w_gate"]).T).float()
    s = torch.sigmoid(logits.double()).float()
    key = s + torch.from_numpy(w["bias"])
    ids = torch.sort(key, dim=1, descending=True, stable=True).indices[:, :K]
    ws = torch.gather(s, 1, ids)
    tot = torch.zeros(T, dtype=torch.float32)
    for k in range(K):                      # the slot-order FP32 sum
        tot = tot + ws[:, k]
    ws = (ws / tot[:, None]) * torch.tensor(d["routed_scale"], dtype=torch.float32)
    latent = rb(xt @ bf(w["w_down"]).T)
    codes, scales = mx_quant(latent)
    a = mx_dequant8(codes, scales)
    rows = torch.zeros(T * K, L, dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            h = (mx_dequant4(w["w13"][e], w["s13"][e]) @ a[t]).float().double()
            act = (torch.nn.functional.silu(h[:I]) * h[I:]).float().double()
            hc, hs = mx_quant(act[None])
            y = (mx_dequant4(w["w2"][e], w["s2"][e]) @ mx_dequant8(hc, hs)[0]).float()
            rows[t * K + k] = y.to(torch.bfloat16).double()
    routed = torch.zeros(T, L, dtype=torch.float64)
    for t in range(T):
        acc = torch.zeros(L, dtype=torch.float32)
        for k in range(K):                  # FP32 multiply-add chain in slot order
            acc = (acc.double() + ws[t, k].double() * rows[t * K + k]).float()
        routed[t] = acc.to(torch.bfloat16).double()
    ms = (routed * routed).mean(dim=1, keepdim=True)
    normed = rb(routed / torch.sqrt(ms + d["rms_eps"]) * bf(w["norm_w"]))
    gu = rb(xt @ bf(w["w_shared_gu"]).T)
    act_s = rb(torch.nn.functional.silu(gu[:, :S]) * gu[:, S:])
    shared = rb(act_s @ bf(w["w_shared_dn"]).T)
    out = rb(shared.float().double() + (normed @ bf(w["w_up"]).T).float().double())
    return out, dict(ids=ids.numpy().astype(np.int32), latent=latent, codes=codes.numpy(),
                     scales=scales.numpy(), rows=rows, routed=routed, shared=shared)


def bf16_bits(t):
    return t.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def mx_case(T=24, seed=2):
    d = dict(T=T, H=256, L=128, E=16, K=4, I=64, S=128, unit_tokens=8, expert_format=0,
             renormalize=1, routed_scale=2.5, rms_eps=1e-5)
    w = syn.layer_weights(d, seed=seed)
    g = syn.rng(seed, 900)
    H, L, E, S = d["H"], d["L"], d["E"], d["S"]
    w["w_gate"] = pow2_ints(g, (E, H), -3, 3, 6)
    w["w_down"] = pow2_ints(g, (L, H), -3, 3, 5)
    w["w_shared_gu"] = pow2_ints(g, (2 * S, H), -3, 3, 6)
    w["w_shared_dn"] = pow2_ints(g, (H, S), -3, 3, 5)
    w["w_up"] = pow2_ints(g, (H, L), -3, 3, 4)
    w["norm_w"] = pow2_ints(g, (L,), 12, 20, 4)
    x = pow2_ints(g, (T, H), -4, 4, 0)
    return d, w, x


def test_mx_layer_vs_torch_fp64(orc):
    """The oracle's MXFP4 x MXFP8 layer against the independent torch composition above:
    ids, latent, latent codes and scales, and every expert row (by pair id) bit for bit;
    routed within one BF16 ulp (the composition's multiply-add rounds twice); the output
    within 2e-2 x RMS."""
    d, w, x = mx_case()
    out, tr = orc.layer(d, w, x, trace=True)
    ref, rt = torch_mx_layer(d, w, x)
    assert np.array_equal(tr["ids"], rt["ids"])
    # some expert takes more than one 8-token window, so the unit windows are exercised
    assert np.bincount(rt["ids"].reshape(-1), minlength=d["E"]).max() > d["unit_tokens"]
    assert np.array_equal(tr["latent"], bf16_bits(rt["latent"]))
    assert np.array_equal(tr["codes"], rt["codes"]) and np.array_equal(tr["scales"], rt["scales"])
    assert np.array_equal(tr["rows"], bf16_bits(rt["rows"]))
    r = tr["routed"].astype(np.int32) - bf16_bits(rt["routed"]).astype(np.int32)
    assert np.abs(r).max() <= 1
    assert np.array_equal(tr["shared"], bf16_bits(rt["shared"]))
    o = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double()
    rms = ref.pow(2).mean().sqrt()
    assert (o - ref).abs().max() <= 2e-2 * rms


def test_mx_layer_pin_catches_wiring_mistakes(orc):
    """The composition above tells apart plausible wiring mistakes of the MX layer: expert
    rows stored by list position instead of pair id, or the pair ids used as expert ids."""
    d, w, x = mx_case()
    _, tr = orc.layer(d, w, x, trace=True)
    _, rt = torch_mx_layer(d, w, x)
    ref_rows = bf16_bits(rt["rows"])
    lists = orc.build_lists(tr["ids"], d["E"], d["unit_tokens"])
    by_list = np.zeros_like(ref_rows)
    by_list[: len(lists["pairs"])] = ref_rows[lists["pairs"]]
    assert not np.array_equal(by_list, ref_rows)
    K = d["K"]
    pexp = tr["ids"].reshape(-1)[lists["pairs"]]
    codes, scales = tr["codes"], tr["scales"]
    swapped = np.clip(lists["pairs"], 0, d["E"] - 1).astype(np.int32)
    hc, hs, _ = orc.ffn_up_mx(lists["pairs"], swapped, K, codes, scales, w["w13"], w["s13"])
    wrong = orc.ffn_down_mx(swapped, hc, hs, w["w2"], w["s2"])
    assert not np.array_equal(wrong, ref_rows[lists["pairs"]])
    hc, hs, _ = orc.ffn_up_mx(lists["pairs"], pexp, K, codes, scales, w["w13"], w["s13"])
    right = orc.ffn_down_mx(pexp, hc, hs, w["w2"], w["s2"])
    assert np.array_equal(right, ref_rows[lists["pairs"]])
