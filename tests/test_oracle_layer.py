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


def test_mx_layer_small_runs(orc):
    # the MXFP4 expert format through the whole layer at a reduced shape
    d = dict(T=6, H=256, L=128, E=16, K=4, I=64, S=128, unit_tokens=8, expert_format=0,
             renormalize=1, routed_scale=2.5, rms_eps=1e-5)
    w = syn.layer_weights(d, seed=2)
    x = syn.layer_input(d, seed=2)
    out, tr = orc.layer(d, w, x, trace=True)
    o = (out.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(o)) and np.abs(o).max() > 0
    c, s = orc.quant_mxfp8_bf16(tr["latent"])
    assert np.array_equal(c, tr["codes"]) and np.array_equal(s, tr["scales"])
