"""Pins of the oracle's routing: the defined exponential / sigmoid (accuracy against
libm in double and the boundary rules), the router logits (exact small-integer case
and torch FP64), sigmoid top-k (brute-force sort, exhaustive permutations, torch.topk,
tie-break, weight sum), and the routing lists / unit windows (invariants and a brute
force written here).  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

import moe_synth as syn


def ulp32(x):
    x = abs(float(np.float32(x)))
    return float(np.spacing(np.float32(x)))


def test_constants_definitions(orc):
    c = orc.sigmoid_constants()
    log2e, hi, lo = float(c[0]), float(c[1]), float(c[2])
    assert abs(log2e - 1 / math.log(2)) <= 0.5 * ulp32(log2e)
    # head: at most 16 significant bits, within half a unit of its last place of ln 2
    assert hi * 65536 == int(hi * 65536) and abs(hi - math.log(2)) <= 2.0 ** -17
    assert abs(hi + lo - math.log(2)) < 1e-12
    for k in range(8):
        assert float(c[3 + k]) == float(np.float32(1.0 / math.factorial(k)))


def test_exp_defined_accuracy(orc):
    g = np.random.default_rng(3)
    zs = np.concatenate([g.uniform(-87, 88, 20000), g.uniform(-1, 1, 5000),
                         [0.0, 1.0, -1.0, 88.0, -87.0, 0.5, 1e-8]]).astype(np.float32)
    worst = 0.0
    for z in zs:
        got = orc.exp_defined(float(z))
        ref = math.exp(float(z))
        worst = max(worst, abs(got - ref) / ulp32(ref))
    # the defined steps land within one FP32 ulp of e^z (0.85 ulp measured); a dropped
    # polynomial term or a wrong reduction constant lands beyond it (no r^7 term: 2.5 ulp)
    assert worst <= 1.0, worst
    assert orc.exp_defined(0.0) == 1.0


def test_sigmoid_accuracy_and_boundaries(orc):
    g = np.random.default_rng(4)
    xs = np.concatenate([g.uniform(-90, 90, 10000), g.standard_normal(10000) * 3]).astype(np.float32)
    prev = None
    for x in np.sort(xs):
        s = orc.sigmoid(float(x))
        ref = 1.0 / (1.0 + math.exp(-float(x)))
        if -x > 88:
            assert s == 0.0
        elif -x < -87:
            assert s == 1.0
        else:
            assert abs(s - ref) <= 3 * ulp32(ref) + 1e-45, (x, s, ref)
        if prev is not None:
            assert s >= prev  # monotone
        prev = s
    assert orc.sigmoid(0.0) == 0.5
    assert orc.sigmoid(-88.5) == 0.0 and orc.sigmoid(100.0) == 1.0


def test_router_logits_small_int_exact(orc):
    g = np.random.default_rng(5)
    x = syn.small_int_bf16(g, (5, 300))
    w = syn.small_int_bf16(g, (7, 300))
    got = orc.linear_f32(x, w)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.int64)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.int64)
    assert np.array_equal(got, (xf @ wf.T).astype(np.float32))


def test_router_logits_vs_torch_fp64(orc):
    g = syn.rng(0, 99)
    x = syn.bf16_normal(g, (4, 512))
    w = syn.bf16_normal(g, (9, 512), 1 / math.sqrt(512))
    got = orc.linear_f32(x, w)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double()
    ref = (xt @ wt.T).float().numpy()
    assert np.array_equal(got, ref)


def brute_topk(orc, logits, bias, K, renorm, scale):
    T, E = logits.shape
    ids = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float32)
    for t in range(T):
        s = [np.float32(orc.sigmoid(float(logits[t, e]))) for e in range(E)]
        keys = [np.float32(s[e] + np.float32(bias[e])) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-float(keys[e]), e))[:K]
        ws = [s[e] for e in order]
        tot = np.float32(0)
        for v in ws:
            tot = np.float32(tot + v)
        for k, e in enumerate(order):
            ids[t, k] = e
            v = np.float32(ws[k] / tot) if renorm else ws[k]
            w[t, k] = np.float32(v * np.float32(scale))
    return ids, w


@pytest.mark.parametrize("renorm", [0, 1])
def test_topk_vs_brute_force(orc, renorm):
    g = np.random.default_rng(6)
    logits = g.standard_normal((6, 40)).astype(np.float32)
    bias = (g.standard_normal(40) * 0.05).astype(np.float32)
    ids, w = orc.topk(logits, bias, 5, renorm, 2.5)
    bi, bw = brute_topk(orc, logits, bias, 5, renorm, 2.5)
    assert np.array_equal(ids, bi)
    assert np.array_equal(w.view(np.uint32), bw.view(np.uint32))


def test_topk_weights_are_unbiased_scores(orc):
    # a large bias changes the selection but never the weight of a chosen expert
    logits = np.array([[0.0, 1.0, 2.0, 3.0]], np.float32)
    bias = np.array([10.0, 0.0, 0.0, 0.0], np.float32)
    ids, w = orc.topk(logits, bias, 2, 0, 1.0)
    assert list(ids[0]) == [0, 3]
    assert w[0, 0] == np.float32(orc.sigmoid(0.0)) == 0.5
    assert w[0, 1] == np.float32(orc.sigmoid(3.0))


def test_topk_exhaustive_permutations(orc):
    base = np.array([-2.0, -1.0, -0.5, 0.0, 0.25, 0.5, 1.0, 2.0], np.float32)
    bias = np.zeros(8, np.float32)
    for perm in itertools.permutations(range(8)):
        logits = base[list(perm)][None, :]
        ids, _ = orc.topk(logits, bias, 2, 1, 2.5)
        ref = torch.topk(torch.from_numpy(logits), 2, dim=1).indices.numpy()
        assert np.array_equal(ids, ref)


def test_topk_matches_torch_topk_without_bias(orc):
    g = np.random.default_rng(7)
    logits = g.standard_normal((32, 896)).astype(np.float32)
    ids, w = orc.topk(logits, np.zeros(896, np.float32), 16, 1, 2.5)
    ref = torch.topk(torch.from_numpy(logits), 16, dim=1).indices.numpy()
    assert np.array_equal(ids, ref)
    sums = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(sums - 2.5) <= 16 * ulp32(2.5))


def test_topk_ties_go_to_lower_id(orc):
    logits = np.zeros((1, 10), np.float32)
    ids, w = orc.topk(logits, np.zeros(10, np.float32), 4, 1, 1.0)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.all(w == np.float32(0.25))


def brute_lists(ids, E, unit):
    T, K = ids.shape
    listed = []
    dropped = 0
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(ids[t, k])
            if 0 <= e < E and e not in seen:
                listed.append((e, t * K + k))
                seen.add(e)
            else:
                dropped += 1
    listed.sort()
    counts = np.array([sum(1 for e, _ in listed if e == x) for x in range(E)], np.int32)
    offs = np.concatenate([[0], np.cumsum(counts)])
    first = [(e, offs[e], min(unit, counts[e]), counts[e]) for e in range(E) if counts[e] > 0]
    later = [(e, offs[e] + j, min(unit, counts[e] - j), 0)
             for e in range(E) for j in range(unit, counts[e], unit)]
    units = np.array(first + later, np.int32).reshape(-1, 4)
    return counts, np.array([p for _, p in listed], np.int32), units, dropped


def test_lists_vs_brute_force_and_invariants(orc):
    g = np.random.default_rng(8)
    T, K, E = 37, 6, 23
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = orc.topk(logits, (g.standard_normal(E) * 0.05).astype(np.float32), K, 1, 2.5)
    r = orc.build_lists(ids, E, 8)
    c, p, u, d = brute_lists(ids, E, 8)
    assert np.array_equal(r["counts"], c) and np.array_equal(r["pairs"], p)
    assert np.array_equal(r["units"], u) and r["dropped"] == d == 0
    # every (t, k) pair in exactly one list, lists ascending, units tile each list
    assert sorted(r["pairs"].tolist()) == list(range(T * K))
    assert r["counts"].sum() == T * K and r["counts"].max() <= T
    for e in range(E):
        seg = r["pairs"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(ids.reshape(-1)[seg] == e)
    assert r["num_units"] == sum(-(-int(x) // 8) for x in r["counts"])
    assert r["touched"] == int(np.count_nonzero(r["counts"]))
    assert np.all(r["units"][:, 2] <= 8) and np.all(r["units"][:, 2] >= 1)
    # the windows of each expert tile its list exactly
    for e in range(E):
        win = sorted((b, c) for x, b, c, _ in r["units"] if x == e)
        pos = r["offsets"][e]
        for b, c in win:
            assert b == pos
            pos += c
        assert pos == r["offsets"][e + 1]


def test_lists_drop_invalid_and_repeated(orc):
    ids = np.array([[0, 1, 1, 9], [-1, 2, 0, 2]], np.int32)
    r = orc.build_lists(ids, 3, 2)
    assert r["dropped"] == 4
    assert r["counts"].tolist() == [2, 1, 1]
    assert r["pairs"].tolist() == [0, 6, 1, 5]
    assert r["units"].tolist() == [[0, 0, 2, 2], [1, 2, 1, 1], [2, 3, 1, 1]]


def test_lists_unit_windows_hot_expert(orc):
    T, K, E = 50, 2, 4
    ids = np.stack([np.zeros(T, np.int32), 1 + (np.arange(T, dtype=np.int32) % 3)], axis=1)
    r = orc.build_lists(ids, E, 8)
    assert r["counts"].tolist() == [50, 17, 17, 16]
    assert r["num_units"] == 7 + 3 + 3 + 2 and r["touched"] == 4
    assert r["units"][:4].tolist() == [[0, 0, 8, 50], [1, 50, 8, 17], [2, 67, 8, 17],
                                       [3, 84, 8, 16]]
    assert r["units"][4].tolist() == [0, 8, 8, 0] and r["units"][9].tolist() == [0, 48, 2, 0]
    assert r["units"][10].tolist() == [1, 58, 8, 0] and r["units"][14].tolist() == [3, 92, 8, 0]
