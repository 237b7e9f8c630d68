"""GPU parity of the whole layer (moe_layer) against the oracle.

Toy latent MoE (T=8, BF16 experts): every output against the free-running oracle layer.
Full layer (hidden 7168, latent 3584, 896 MXFP4 experts) at every batch of the sweep
(T = 65, 130, 255, 510, 1020 with uniform and Zipf routing; T = 256 and 192 besides):
every intermediate read from the documented workspace layout and checked teacher-forced
-- each oracle step is fed the GPU's upstream outputs where a discrete decision follows
(routing on the GPU's logits, quantisation on its latent, the experts on its codes and
lists, Finalize on its rows): discrete results bit-exact on every token, floating results
within 2e-2 x RMS, Finalize exact; the projections and experts on sampled tokens, and at
T=256 (uniform) on every token and every pair; plus a free-running oracle layer on a few
sampled tokens."""
import functools

import numpy as np
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import (assert_close, assert_close_bf16, bf16_ulp_dist, check_hidden, dev, f32,
                      full_weights, hidden_error_bound, host, say)

pytestmark = pytest.mark.gpu


def run_layer(d, dw, x, dense_format=moe.MOE_DENSE_ROWMAJOR):
    lw = moe.layer_weights(dw["w_gate"], dw["bias"], dw["w_down"], dw["w_shared_gu"],
                           dw["w_shared_dn"], dw["norm_w"], dw["w_up"], dw["w13"], dw["s13"],
                           dw["w2"], dw["s2"], dense_format=dense_format)
    ws = torch.zeros(moe.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    out = torch.empty(d.tokens, d.hidden, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer(d, lw, dev(x), out, ws)
    torch.cuda.synchronize()
    return host(out), ws


def test_toy_layer(orc):
    d0 = dict(syn.TOY)
    w = syn.layer_weights(d0, seed=0)
    x = syn.layer_input(d0, seed=0)
    dw = {k: (dev(v) if v is not None else None) for k, v in w.items()}
    out, ws = run_layer(moe.dims_from(d0), dw, x)
    ref, tr = orc.layer(d0, w, x, trace=True)
    v = moe.workspace_views(moe.dims_from(d0), ws)
    assert np.array_equal(host(v["ids"]), tr["ids"])
    assert_close_bf16(out, ref, "toy layer out")


@functools.lru_cache(maxsize=2)
def layer_run(T, zipf):
    """One GPU layer call at T tokens of the full layer: (weights, x, out, intermediates)."""
    w, dw = full_weights(0, zipf)
    x = syn.layer_input(syn.full_dims(T), seed=1)
    d = moe.dims(T, 1020)
    out, ws = run_layer(d, dw, x)
    v = {k: host(t) for k, t in moe.workspace_views(d, ws).items()}
    del ws
    return w, x, out, v


# T=510 and 1020: past 256 tokens the shared expert is forked after the routing lists;
# T=1020: the lists no longer fit one workgroup's LDS, so the top-K writes the slot map and
# the three-launch list build reads it; T=130, 192 and 255: the up-projection's split plan
# runs 128-token chunks, the second one ragged
# T=1..64: the narrow batches below the pages' wide range (one token; one unit window per
# expert; ragged 32-token tiles)
@pytest.mark.parametrize("T,zipf", [(256, False), (256, True), (65, False), (65, True),
                                    (130, False), (192, True), (255, False), (510, False),
                                    (510, True), (1020, False), (1020, True), (1, False),
                                    (8, False), (32, True), (64, False)])
def test_full_layer_teacher_forced(orc, T, zipf):
    say(f"full layer T={T} zipf={zipf}")
    w, x, out, v = layer_run(T, zipf)
    d0 = syn.full_dims(T)
    K, E = 16, 896
    rng = np.random.default_rng(T)
    toks = np.unique(np.r_[0, T - 1, rng.choice(T, min(4, T), replace=False)])
    # router logits (sampled tokens) and routing on the GPU's logits (all tokens)
    assert_close(v["logits"][toks], orc.linear_f32(x[toks], w["w_gate"]), "logits")
    rid, rw = orc.topk(v["logits"], w["bias"], K, 1, 2.5)
    assert np.array_equal(v["ids"], rid)
    assert np.array_equal(v["weights"].view(np.uint32), rw.view(np.uint32))
    rl = orc.build_lists(v["ids"], E, 8)
    assert np.array_equal(v["counts"], rl["counts"]) and np.array_equal(v["pairs"], rl["pairs"])
    assert v["num_units"][0] == rl["num_units"]
    assert np.array_equal(v["units_raw"][:rl["num_units"]], rl["units"])
    assert np.array_equal(v["offsets"], rl["offsets"])
    assert list(v["num_units"][:3]) == [rl["num_units"], rl["dropped"], rl["touched"]]
    D = int(np.count_nonzero(rl["counts"]))
    say(f"  D={D} touched experts, {rl['num_units']} units")
    # latent (sampled) and its MXFP8 codes (all tokens, on the GPU's latent)
    assert_close_bf16(v["latent"][toks], orc.linear_bf16(x[toks], w["w_down"]), "latent")
    rc, rs = orc.quant_mxfp8_bf16(v["latent"])
    assert np.array_equal(v["codes"], rc) and np.array_equal(v["scales"], rs)
    # experts on the GPU's codes, sampled pairs of the sampled tokens
    pairs = np.array([t * K + k for t in toks for k in range(K)], np.int32)
    pexp = v["ids"].reshape(-1)[pairs]
    hc, hs, hf = orc.ffn_up_mx(pairs, pexp, K, v["codes"], v["scales"], w["w13"], w["s13"])
    delta = hidden_error_bound(v["codes"], v["scales"], w["w13"], w["s13"], pairs, pexp, K, 512)
    check_hidden(v["hidden"][pairs], v["hidden_scales"][pairs], hc, hs, hf, delta)
    rows_tf = orc.ffn_down_mx(pexp, v["hidden"][pairs], v["hidden_scales"][pairs], w["w2"],
                              w["s2"])
    assert_close_bf16(v["rows"][pairs], rows_tf, "expert rows (oracle fed GPU hidden)")
    rows_ref = orc.ffn_down_mx(pexp, hc, hs, w["w2"], w["s2"])
    assert_close(f32(v["rows"][pairs]), f32(rows_ref), "expert rows (free-running, sanity)",
                 tol=0.1)
    # Finalize on the GPU's rows (all tokens): bit-exact
    fin = orc.finalize(v["rows"], v["weights"])
    assert np.array_equal(v["routed"], fin)
    # RMSNorm on the GPU's routed latent, shared expert and output (sampled tokens)
    nrm = orc.rmsnorm(v["routed"], w["norm_w"], 1e-5)
    assert_close_bf16(v["normed"], nrm, "normed")
    assert bf16_ulp_dist(v["normed"], nrm).max() <= 2
    gu = orc.linear_bf16(x[toks], w["w_shared_gu"])
    sh = orc.linear_bf16(orc.silu_mul_bf16(gu), w["w_shared_dn"])
    assert_close_bf16(v["shared"][toks], sh, "shared expert")
    o = orc.linear_add_bf16(v["normed"][toks], w["w_up"], v["shared"][toks])
    assert_close_bf16(out[toks], o, "out (teacher-forced)")
    # free-running oracle layer on two tokens (hidden code flips propagate: sanity bound)
    sub = toks[:2]
    d1 = dict(d0, T=len(sub))
    ref = orc.layer(d1, w, x[sub])
    assert_close(f32(out[sub]), f32(ref), "out (free-running oracle, sanity)", tol=0.1)


def test_full_layer_every_pair_experts_T256(orc):
    """T=256, uniform routing: the MXFP8 hidden and the expert row of EVERY (token, slot)
    pair against the oracle fed the GPU's codes and lists (the expert passes hand their
    last items out by work tickets at this size, so no item goes unchecked)."""
    T, K = 256, 16
    w, x, out, v = layer_run(T, False)
    pairs = v["pairs"][:int(v["offsets"][-1])].astype(np.int32)
    assert len(pairs) == T * K  # nothing dropped: every pair is listed
    pexp = v["ids"].reshape(-1)[pairs]
    say(f"  oracle gate/up pass on all {len(pairs)} pairs")
    hc, hs, hf = orc.ffn_up_mx(pairs, pexp, K, v["codes"], v["scales"], w["w13"], w["s13"])
    gh, gs = v["hidden"][pairs], v["hidden_scales"][pairs]
    # the FP32 summation-error bound, only where a code or scale differs (an equal code is
    # the rounding of the oracle's value and within half a step of it)
    odd = np.nonzero(np.any(gh != hc, axis=1) | np.any(gs != hs, axis=1))[0]
    delta = np.zeros(hf.shape)
    if len(odd):
        delta[odd] = hidden_error_bound(v["codes"], v["scales"], w["w13"], w["s13"], pairs[odd],
                                        pexp[odd], K, 512)
    say(f"  {len(odd)} pairs with a code that differs from the oracle's")
    check_hidden(gh, gs, hc, hs, hf, delta)
    say("  oracle down pass on all pairs (fed the GPU's hidden)")
    rows_tf = orc.ffn_down_mx(pexp, gh, gs, w["w2"], w["s2"])
    assert_close_bf16(v["rows"][pairs], rows_tf, "every expert row (oracle fed GPU hidden)")


def test_full_layer_every_token_dense_T256(orc):
    """T=256, uniform routing: logits, latent, shared expert and output of EVERY token
    against the oracle (the output teacher-forced on the GPU's normed latent and shared)."""
    T = 256
    w, x, out, v = layer_run(T, False)
    assert_close(v["logits"], orc.linear_f32(x, w["w_gate"]), "logits, every token")
    assert_close_bf16(v["latent"], orc.linear_bf16(x, w["w_down"]), "latent, every token")
    say("  oracle shared expert on every token")
    gu = orc.linear_bf16(x, w["w_shared_gu"])
    sh = orc.linear_bf16(orc.silu_mul_bf16(gu), w["w_shared_dn"])
    assert_close_bf16(v["shared"], sh, "shared expert, every token")
    o = orc.linear_add_bf16(v["normed"], w["w_up"], v["shared"])
    assert_close_bf16(out, o, "out (teacher-forced), every token")


def test_full_layer_packed_equals_row_major():
    """moe_layer on packed expert weights gives the row-major layer's output bit for bit."""
    w, dw = full_weights(0, False)
    T = 256
    x = syn.layer_input(syn.full_dims(T), seed=1)
    d = moe.dims(T, T)
    out_ref, _ = run_layer(d, dw, x)
    pk = moe.moe_pack_expert_weights(d, dw["w13"], dw["s13"], dw["w2"], dw["s2"])
    dwp = dict(dw, w13=pk[0], s13=pk[1], w2=pk[2], s2=pk[3])
    dp = moe.dims(T, T, expert_format=moe.MOE_FMT_MXFP4_MXFP8_PACKED)
    out, _ = run_layer(dp, dwp, x)
    assert np.array_equal(out, out_ref)


# 8 and 1 tokens: the narrow batches' one-token-tile GEMM plans
@pytest.mark.parametrize("T", [256, 65, 8, 1])
def test_full_layer_dense_packed_equals_row_major(T):
    """moe_layer on packed dense weights (moe_pack_dense_weight) gives the row-major
    layer's output bit for bit; with the workspace intermediates equal too."""
    w, dw = full_weights(0, False)
    x = syn.layer_input(syn.full_dims(T), seed=2)
    d = moe.dims(T, 1020)
    say(f"dense packed vs row-major T={T}")
    out_ref, ws_ref = run_layer(d, dw, x)
    dwp = dict(dw)
    for k in ("w_gate", "w_down", "w_shared_gu", "w_shared_dn", "w_up"):
        dwp[k] = moe.moe_pack_dense_weight(dw[k])
    out, ws = run_layer(d, dwp, x, dense_format=moe.MOE_DENSE_PACKED)
    assert np.array_equal(out, out_ref)
    v, vr = moe.workspace_views(d, ws), moe.workspace_views(d, ws_ref)
    for k in ("logits", "latent", "shared"):
        assert torch.equal(v[k], vr[k]), k


@pytest.mark.parametrize("zipf", [False, True])
def test_full_layer_repeat_covers_every_pair(zipf):
    """Two layer calls on one workspace give the same bytes, the second after the expert
    rows and the MXFP8 hidden were overwritten with a NaN pattern: every listed pair's
    row and hidden are rewritten by each call (the expert passes hand their last items
    out by work tickets, so coverage depends on the counters being reset per call), and
    a T=65 call in between leaves nothing behind that the next call depends on."""
    _, dw = full_weights(0, zipf)
    T = 256
    x = syn.layer_input(syn.full_dims(T), seed=4)
    d = moe.dims(T, 1020)
    lw = moe.layer_weights(dw["w_gate"], dw["bias"], dw["w_down"], dw["w_shared_gu"],
                           dw["w_shared_dn"], dw["norm_w"], dw["w_up"], dw["w13"], dw["s13"],
                           dw["w2"], dw["s2"])
    ws = torch.zeros(moe.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    xd = dev(x)
    out1 = torch.empty(T, d.hidden, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer(d, lw, xd, out1, ws)
    torch.cuda.synchronize()
    v = moe.workspace_views(d, ws)
    rows1, hid1, hsc1 = v["rows"].clone(), v["hidden"].clone(), v["hidden_scales"].clone()
    d65 = moe.dims(65, 1020)
    out65 = torch.empty(65, d.hidden, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer(d65, lw, xd[:65].contiguous(), out65, ws)
    for k in ("rows", "hidden", "hidden_scales"):
        v[k].view(torch.uint8).fill_(0xFF)
    out2 = torch.empty_like(out1)
    moe.moe_layer(d, lw, xd, out2, ws)
    torch.cuda.synchronize()
    v = moe.workspace_views(d, ws)
    assert torch.equal(v["rows"].view(torch.uint8), rows1.view(torch.uint8))
    assert torch.equal(v["hidden"], hid1) and torch.equal(v["hidden_scales"], hsc1)
    assert torch.equal(out2.view(torch.int16), out1.view(torch.int16))
