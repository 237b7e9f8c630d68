"""GPU parity of the grouped expert FFN (MXFP4 weights x MXFP8 activations with the
MXFP8 hidden; and the BF16-weight variant) against the oracle: hidden codes
(teacher-forced on identical MXFP8 inputs; bit-exact except where FP32 accumulation
order moves a value across a rounding boundary), expanded rows (tolerance; with the
oracle's second half fed the GPU's hidden codes, and free-running), at small ragged
shapes and at the full latent/intermediate sizes with multi-unit experts."""
import numpy as np
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import (assert_close, assert_close_bf16, check_hidden, dev, f32,
                      hidden_error_bound, host, mx_latent, say)

pytestmark = pytest.mark.gpu

def build_lists(d, ids_dev):
    T, K, E = d.tokens, d.top_k, d.experts
    P = T * K
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pairs = torch.empty(P, dtype=torch.int32, device="cuda")
    units = torch.empty(-(-P // d.unit_tokens) + E, 4, dtype=torch.int32, device="cuda")
    nu = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_lists_workspace_size(d), dtype=torch.uint8, device="cuda")
    moe.moe_build_lists(d, ids_dev, counts, offsets, pairs, units, nu, ws)
    return pairs, units, nu


def run_ffn_mx(d, w, codes, scales, ids):
    T, K, L, I = d.tokens, d.top_k, d.latent, d.expert_inter
    ids_d = dev(ids)
    pairs, units, nu = build_lists(d, ids_d)
    rows = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
    moe.moe_grouped_ffn(d, dev(w["w13"]), dev(w["s13"]), dev(w["w2"]), dev(w["s2"]), dev(codes),
                        dev(scales), pairs, units, nu, rows, ws)
    torch.cuda.synchronize()
    P = T * K
    hid = host(ws[:P * I]).reshape(P, I)
    off = (P * I + 255) // 256 * 256
    hsc = host(ws[off:off + P * (I // 32)]).reshape(P, I // 32)
    return host(rows), hid, hsc


def random_ids(g, T, K, E, hot=None):
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    if hot is not None:  # make expert `hot` appear in every token
        for t in range(T):
            if hot not in ids[t]:
                ids[t, t % K] = hot
    return ids


def check_mx(orc, d, w, codes, scales, ids, sample):
    T, K, I = d.tokens, d.top_k, d.expert_inter
    rows, hid, hsc = run_ffn_mx(d, w, codes, scales, ids)
    pexp = ids.reshape(-1)[sample]
    hc, hs, hf = orc.ffn_up_mx(sample, pexp, K, codes, scales, w["w13"], w["s13"])
    delta = hidden_error_bound(codes, scales, w["w13"], w["s13"], sample, pexp, K, I)
    check_hidden(hid[sample], hsc[sample], hc, hs, hf, delta)
    # second half teacher-forced on the GPU's hidden codes
    ref_tf = orc.ffn_down_mx(pexp, hid[sample], hsc[sample], w["w2"], w["s2"])
    assert_close_bf16(rows[sample], ref_tf, "rows (oracle fed GPU hidden)")
    # free-running: a one-step hidden code flip is a correct outcome, so informational
    ref = orc.ffn_down_mx(pexp, hc, hs, w["w2"], w["s2"])
    assert_close(f32(rows[sample]), f32(ref), "rows (free-running oracle, sanity)", tol=0.1)


# the last two shapes take the generic kernels: I = 384 (I / 128 = 3) the generic down pass,
# L = 768 (not a multiple of 512) the generic gate/up pass and, with I = 640, the generic
# down pass
@pytest.mark.parametrize("T,K,E,L,I,unit", [(16, 4, 8, 512, 128, 8), (13, 3, 5, 256, 256, 16),
                                            (1, 1, 3, 256, 128, 8), (24, 4, 6, 512, 384, 8),
                                            (9, 2, 4, 768, 640, 8)])
def test_ffn_mx_small(orc, T, K, E, L, I, unit):
    say(f"ffn mx T={T} K={K} E={E} L={L} I={I} unit={unit}")
    dd = dict(L=L, I=I, E=E, expert_format=0)
    w = syn.expert_weights(dd, seed=T)
    g = syn.rng(T, 700)
    codes, scales = mx_latent(orc, g, T, L)
    ids = random_ids(np.random.default_rng(T), T, K, E)
    d = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I,
                 unit_tokens=unit)
    check_mx(orc, d, w, codes, scales, ids, np.arange(T * K, dtype=np.int32))


def test_ffn_mx_full_size_multi_unit(orc):
    T, K, E, L, I = 256, 16, 64, 3584, 512
    say(f"ffn mx full T={T} K={K} E={E} L={L} I={I}")
    dd = dict(L=L, I=I, E=E, expert_format=0)
    w = syn.expert_weights(dd, seed=1)
    codes, scales = mx_latent(orc, syn.rng(1, 701), T, L)
    ids = random_ids(np.random.default_rng(5), T, K, E, hot=3)
    d = moe.dims(T, T)
    d.experts = E
    sample = np.sort(np.random.default_rng(6).choice(T * K, 40, replace=False)).astype(np.int32)
    check_mx(orc, d, w, codes, scales, ids, sample)


def grouped_ids(counts, K):
    """ids [T, K] in which expert e is chosen by exactly counts[e] tokens (T = sum / K):
    the sorted expert labels dealt round-robin, so that a token's K slots lie T apart in
    the sorted order and name K distinct experts (every count is below T)."""
    labels = np.repeat(np.arange(len(counts)), counts)
    T = len(labels) // K
    assert T * K == len(labels) and max(counts) < T
    return np.stack([labels[T * k:T * (k + 1)] for k in range(K)], axis=1).astype(np.int32)


# 32 experts, 186 tokens: the two-area gate/up build (from 128 tokens) at 512 items; 16
# experts, 93 tokens: the one-area build, whose later groups reload the one area
@pytest.mark.parametrize("copies", [2, 1])
def test_ffn_mx_token_groups_every_pair(orc, copies):
    """Experts whose lists end on each side of the token-group boundaries of the expert
    passes (16 tokens per MFMA column tile, the second group's loads issued ahead with the
    first's, a third and later group loaded on their own; 8 of a group's tokens per direct
    load): every pair's hidden and rows against the oracle, at 512 gate/up items (two full
    passes of 256 workgroups, whose two stages take neighbouring column tiles of one
    expert, the second reusing the first's activations) or 256; and the packed weights'
    run bit for bit equal to the row-major one."""
    counts = [1, 7, 8, 9, 15, 16, 17, 20, 24, 25, 28, 32, 33, 40, 48, 49] * copies
    K, L, I = 4, 512, 512
    ids = grouped_ids(counts, K)
    T, E = ids.shape[0], len(counts)
    say(f"ffn mx token groups T={T} K={K} E={E} L={L} I={I}")
    assert (np.bincount(ids.ravel(), minlength=E) == counts).all()
    w = syn.expert_weights(dict(L=L, I=I, E=E, expert_format=0), seed=8)
    codes, scales = mx_latent(orc, syn.rng(8, 704), T, L)
    d = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I)
    check_mx(orc, d, w, codes, scales, ids, np.arange(T * K, dtype=np.int32))
    ref_rows, ref_hid, _ = run_ffn_mx(d, w, codes, scales, ids)
    pk = moe.moe_pack_expert_weights(d, dev(w["w13"]), dev(w["s13"]), dev(w["w2"]), dev(w["s2"]))
    dp = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I,
                  expert_format=moe.MOE_FMT_MXFP4_MXFP8_PACKED)
    pairs, units, nu = build_lists(dp, dev(ids))
    rows = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(moe.moe_ffn_workspace_size(dp), dtype=torch.uint8, device="cuda")
    moe.moe_grouped_ffn(dp, *pk, dev(codes), dev(scales), pairs, units, nu, rows, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(ws[:T * K * I]).reshape(T * K, I), ref_hid)
    assert np.array_equal(host(rows), ref_rows)


def test_ffn_stages_match_grouped():
    """The up pass then the down pass, as two calls, give the one-call result bit for bit."""
    T, K, E, L, I = 40, 4, 12, 512, 256
    dd = dict(L=L, I=I, E=E, expert_format=0)
    w = syn.expert_weights(dd, seed=2)
    codes, scales = syn.mxfp8_random(syn.rng(2, 702), T, L)
    ids = random_ids(np.random.default_rng(7), T, K, E)
    d = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I)
    ref_rows, ref_hid, ref_hsc = run_ffn_mx(d, w, codes, scales, ids)
    pairs, units, nu = build_lists(d, dev(ids))
    rows = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
    args = (d, dev(w["w13"]), dev(w["s13"]), dev(w["w2"]), dev(w["s2"]))
    moe.moe_grouped_ffn_stages(*args, dev(codes), dev(scales), pairs, units, nu, None, ws,
                               moe.MOE_FFN_UP)
    moe.moe_grouped_ffn_stages(*args, None, None, pairs, units, nu, rows, ws, moe.MOE_FFN_DOWN)
    torch.cuda.synchronize()
    P = T * K
    assert np.array_equal(host(ws[:P * I]).reshape(P, I), ref_hid)
    assert np.array_equal(host(rows), ref_rows)


def pack_host(w13, s13, w2, s2, L, I):
    """The packed layout of moe_pack_expert_weights, written out from its definition."""
    E, SPW, IS = w13.shape[0], L // 512, I // 128
    pw13 = np.empty_like(w13).reshape(E, -1)
    ps13 = np.empty_like(s13).reshape(E, -1)
    pw2 = np.empty_like(w2).reshape(E, -1)
    for e in range(E):
        o = 0
        for j in range(I // 32):
            for w in range(4):
                for m in range(4):
                    for i in range(SPW):
                        for lane in range(64):
                            r, g = lane % 16, lane // 16
                            row = (m // 2) * I + 32 * j + 16 * (m % 2) + r
                            k0 = (4 * (SPW * w + i) + g) * 16  # byte offset of K block
                            pw13[e, o:o + 16] = w13[e, row, k0:k0 + 16]
                            o += 16
        o = 0
        for j in range(I // 32):
            for w in range(4):
                for m in range(4):
                    for r in range(16):
                        row = (m // 2) * I + 32 * j + 16 * (m % 2) + r
                        ps13[e, o:o + 4 * SPW] = s13[e, row, 4 * SPW * w:4 * SPW * (w + 1)]
                        o += 4 * SPW
        o = 0
        for jd in range(L // 512):
            for w in range(4):
                for m in range(8):
                    for st in range(IS):
                        for lane in range(64):
                            r, g = lane % 16, lane // 16
                            row = 512 * jd + 128 * w + 16 * m + r
                            k0 = (4 * st + g) * 16
                            pw2[e, o:o + 16] = w2[e, row, k0:k0 + 16]
                            o += 16
    return pw13.reshape(w13.shape), ps13.reshape(s13.shape), pw2.reshape(w2.shape), s2.copy()


def test_pack_layout_matches_definition():
    """moe_pack_expert_weights against the layout its header states, built on the host."""
    E, L, I = 2, 1024, 256
    w = syn.expert_weights(dict(L=L, I=I, E=E, expert_format=0), seed=4)
    d = moe.dims(8, 8, hidden=256, latent=L, experts=E, top_k=2, expert_inter=I)
    got = moe.moe_pack_expert_weights(d, dev(w["w13"]), dev(w["s13"]), dev(w["w2"]), dev(w["s2"]))
    torch.cuda.synchronize()
    ref = pack_host(w["w13"], w["s13"], w["w2"], w["s2"], L, I)
    for name, g_, r_ in zip(("w13", "s13", "w2", "s2"), got, ref):
        assert np.array_equal(host(g_), r_), name


@pytest.mark.parametrize("T,K,E,L,I,hot", [(16, 4, 8, 512, 128, None), (40, 4, 12, 1024, 256, 3),
                                           (256, 16, 64, 3584, 512, 3)])
def test_ffn_packed_equals_row_major(T, K, E, L, I, hot):
    """The packed-weight FFN computes the same MFMAs on the same operands: rows and
    hidden bit for bit equal to the row-major run (hot: an expert in every token)."""
    say(f"ffn packed T={T} K={K} E={E} L={L} I={I}")
    w = syn.expert_weights(dict(L=L, I=I, E=E, expert_format=0), seed=5)
    codes, scales = syn.mxfp8_random(syn.rng(5, 703), T, L)
    ids = random_ids(np.random.default_rng(T + 1), T, K, E, hot=hot)
    d = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I)
    ref_rows, ref_hid, ref_hsc = run_ffn_mx(d, w, codes, scales, ids)
    pk = moe.moe_pack_expert_weights(d, dev(w["w13"]), dev(w["s13"]), dev(w["w2"]), dev(w["s2"]))
    dp = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I,
                  expert_format=moe.MOE_FMT_MXFP4_MXFP8_PACKED)
    pairs, units, nu = build_lists(dp, dev(ids))
    rows = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(moe.moe_ffn_workspace_size(dp), dtype=torch.uint8, device="cuda")
    moe.moe_grouped_ffn(dp, *pk, dev(codes), dev(scales), pairs, units, nu, rows, ws)
    torch.cuda.synchronize()
    P = T * K
    assert np.array_equal(host(ws[:P * I]).reshape(P, I), ref_hid)
    assert np.array_equal(host(rows), ref_rows)


def test_ffn_bf16_toy(orc):
    d0 = dict(syn.TOY)
    T, K, E, L, I = d0["T"], d0["K"], d0["E"], d0["L"], d0["I"]
    w = syn.expert_weights(d0, seed=0)
    latent = syn.bf16_normal(syn.rng(0, 702), (T, L))
    ids = random_ids(np.random.default_rng(7), T, K, E)
    d = moe.dims_from(d0)
    pairs, units, nu = build_lists(d, dev(ids))
    rows = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_ffn(d, dev(w["w13"]), None, dev(w["w2"]), None, dev(latent), None, pairs,
                        units, nu, rows, None)
    torch.cuda.synchronize()
    allp = np.arange(T * K, dtype=np.int32)
    ref = orc.ffn_bf16(allp, ids.reshape(-1), K, latent, w["w13"], w["w2"])
    assert_close_bf16(host(rows), ref, "toy BF16 expert rows")
