"""GPU parity of the routing front: router GEMM logits (tolerance, sampled rows of the
1020-token workload), sigmoid top-16 fed identical FP32 logits (ids and weights
bit-exact), routing lists and unit windows (bit-exact, every field), with uniform and
Zipf-skewed bias, small ragged shapes (the router GEMM with row-major and packed W_gate
too), and dropped ids."""
import numpy as np
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu


def run_topk(d, logits, bias):
    T, K = d.tokens, d.top_k
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    moe.moe_router_topk(d, None, None, dev(bias), dev(logits), ids, w, flags=moe.MOE_LOGITS_GIVEN)
    torch.cuda.synchronize()
    return host(ids), host(w)


def run_lists(d, ids):
    T, K, E = d.tokens, d.top_k, d.experts
    P = T * K
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pairs = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    nu_max = -(-P // d.unit_tokens) + E
    units = torch.full((nu_max, 4), -7, dtype=torch.int32, device="cuda")
    num_units = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_lists_workspace_size(d), dtype=torch.uint8, device="cuda")
    moe.moe_build_lists(d, dev(ids), counts, offsets, pairs, units, num_units, ws)
    torch.cuda.synchronize()
    n = int(host(offsets)[E])
    nu = host(num_units)
    return dict(counts=host(counts), offsets=host(offsets), pairs=host(pairs)[:n],
                units=host(units)[:nu[0]], num_units=int(nu[0]), dropped=int(nu[1]))


def check_lists(orc, d, ids):
    got = run_lists(d, ids)
    ref = orc.build_lists(ids, d.experts, d.unit_tokens)
    for k in ("counts", "offsets", "pairs", "units", "num_units", "dropped"):
        assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), k
    return got


@pytest.mark.parametrize("zipf,packed", [(False, False), (True, False), (False, True)])
def test_router_front_1020(orc, zipf, packed):
    T, E, H, K = 1020, 896, 7168, 16
    say(f"router front T={T} zipf={zipf} packed={packed}")
    x = syn.router_input(T, H, seed=0)
    wg = syn.bf16_normal(syn.rng(0, 1), (E, H), 1 / np.sqrt(H))
    bias = syn.routing_bias(E, 1 if zipf else 0, zipf)
    d = moe.dims(T, T)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_router_workspace_size(d), dtype=torch.uint8, device="cuda")
    if packed:  # the packed W_gate gives the row-major run's logits bit for bit
        moe.moe_router_topk(d, dev(x), dev(wg), dev(bias), logits, ids, w, workspace=ws)
        torch.cuda.synchronize()
        lg_rm = host(logits).copy()
        logits.fill_(0)
        moe.moe_router_topk(d, dev(x), moe.moe_pack_dense_weight(dev(wg)), dev(bias), logits,
                            ids, w, flags=moe.MOE_GATE_PACKED, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(logits).view(np.uint32), lg_rm.view(np.uint32))
    else:
        moe.moe_router_topk(d, dev(x), dev(wg), dev(bias), logits, ids, w, workspace=ws)
    torch.cuda.synchronize()
    lg = host(logits)
    sample = np.r_[0:4, 500:504, T - 4:T]
    ref_l = orc.linear_f32(x[sample], wg)
    assert_close(lg[sample], ref_l, "router logits (12 sampled rows)")
    # top-k on identical FP32 logits: bit-exact ids and weights
    rid, rw = orc.topk(lg, bias, K, 1, 2.5)
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(w).view(np.uint32), rw.view(np.uint32))
    got = check_lists(orc, d, host(ids))
    D = int(np.count_nonzero(got["counts"]))
    say(f"  touched experts D={D}, units={got['num_units']}, max count={got['counts'].max()}")


# the router GEMM and the top-K in one call at small ragged shapes: E = 96 (a multiple of
# 32, not of 64: row-major W_gate only), E = 128 (also packed), T across chunk boundaries
@pytest.mark.parametrize("T,E,K,packed", [(37, 96, 6, False), (129, 128, 8, False),
                                          (129, 128, 8, True), (1, 128, 16, True)])
def test_router_small_shapes(orc, T, E, K, packed):
    H = 512
    say(f"router T={T} E={E} K={K} packed={packed}")
    x = syn.router_input(T, H, seed=T)
    wg = syn.bf16_normal(syn.rng(T, 2), (E, H), 1 / np.sqrt(H))
    bias = syn.routing_bias(E, 0, False)
    d = moe.dims(T, T, hidden=H, experts=E, top_k=K)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_router_workspace_size(d), dtype=torch.uint8, device="cuda")
    wd = moe.moe_pack_dense_weight(dev(wg)) if packed else dev(wg)
    moe.moe_router_topk(d, dev(x), wd, dev(bias), logits, ids, w,
                        flags=moe.MOE_GATE_PACKED if packed else 0, workspace=ws)
    torch.cuda.synchronize()
    lg = host(logits)
    assert_close(lg, orc.linear_f32(x, wg), "router logits (every row)")
    rid, rw = orc.topk(lg, bias, K, 1, 2.5)  # on identical FP32 logits: bit-exact
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(w).view(np.uint32), rw.view(np.uint32))


@pytest.mark.parametrize("T,E,K,unit", [(8, 32, 4, 8), (37, 23, 6, 8), (130, 896, 16, 16),
                                        (1, 5, 5, 8), (255, 1024, 16, 8)])
def test_topk_and_lists_shapes(orc, T, E, K, unit):
    g = np.random.default_rng(T * 1000 + E)
    logits = (g.standard_normal((T, E)) * 2).astype(np.float32)
    logits[0, : min(E, 6)] = 0.0  # exact ties -> lower id first
    bias = (g.standard_normal(E) * 0.05).astype(np.float32)
    d = moe.dims(T, T, experts=E, top_k=K, unit_tokens=unit)
    ids, w = run_topk(d, logits, bias)
    rid, rw = orc.topk(logits, bias, K, 1, 2.5)
    assert np.array_equal(ids, rid)
    assert np.array_equal(w.view(np.uint32), rw.view(np.uint32))
    check_lists(orc, d, ids)


@pytest.mark.parametrize("K", [16, 6])
def test_topk_exact_ties_across_wavefronts(orc, K):
    # five logit values and two bias values: many keys s + bias are bit-identical, within a
    # wavefront, across the four wavefronts and among their winners; equal keys must go
    # to the lower expert id in every slot
    T, E = 9, 896
    g = np.random.default_rng(21 + K)
    logits = g.integers(-2, 3, size=(T, E)).astype(np.float32)
    bias = g.choice(np.array([0.0, 0.25], np.float32), size=E)
    d = moe.dims(T, T, experts=E, top_k=K)
    ids, w = run_topk(d, logits, bias)
    rid, rw = orc.topk(logits, bias, K, 1, 2.5)
    assert np.array_equal(ids, rid)
    assert np.array_equal(w.view(np.uint32), rw.view(np.uint32))


def test_topk_saturated_logits(orc):
    # logits far in both tails exercise the sigmoid's boundary rules
    T, E, K = 4, 64, 16
    g = np.random.default_rng(11)
    logits = (g.standard_normal((T, E)) * 60).astype(np.float32)
    bias = np.zeros(E, np.float32)
    d = moe.dims(T, T, experts=E, top_k=K)
    for renorm in (0, 1):
        d.renormalize = renorm
        ids, w = run_topk(d, logits, bias)
        rid, rw = orc.topk(logits, bias, K, renorm, 2.5)
        assert np.array_equal(ids, rid) and np.array_equal(w.view(np.uint32), rw.view(np.uint32))


# (70, 4, 9): the one-workgroup build (bitmaps in LDS); (1100, 4, 1024): bitmaps past the
# LDS bound, the three-launch build
@pytest.mark.parametrize("T,K,E", [(70, 4, 9), (1100, 4, 1024)])
def test_lists_drop_invalid_and_repeated_ids(orc, T, K, E):
    g = np.random.default_rng(12)
    ids = g.integers(-2, E + 2, size=(T, K)).astype(np.int32)
    d = moe.dims(T, T, experts=E, top_k=K)
    got = check_lists(orc, d, ids)
    assert got["dropped"] > 0


@pytest.mark.parametrize("T", [256, 1020])  # one-workgroup build, three-launch build
def test_lists_hot_expert_many_units(orc, T):
    K, E = 16, 896
    ids = np.zeros((T, K), np.int32)
    for t in range(T):
        ids[t] = np.r_[0, 1 + (np.arange(15) + t) % (E - 1)]
    d = moe.dims(T, T)
    got = check_lists(orc, d, ids)
    assert got["counts"][0] == T


def test_lists_deterministic(orc):
    T, K, E = 512, 16, 896
    g = np.random.default_rng(13)
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    d = moe.dims(T, T)
    a = run_lists(d, ids)
    b = run_lists(d, ids)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k]))
