"""Pins of the oracle's Finalize, RMSNorm, dense BF16 linears and shared-expert
activation: a hand-computed Finalize example, exact special cases (one-hot and
power-of-two weights), the fused-multiply-add order, the invalid-slot rule, the
RMSNorm closed form, small-integer exact linears and torch FP64.  CPU only."""
import json
import os

import numpy as np
import torch

import moe_synth as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_finalize_hand_example(orc):
    with open(os.path.join(GOLDEN, "finalize_hand.json")) as f:
        g = json.load(f)
    rows = bits(np.array(g["rows"], np.float32))
    w = np.array(g["weights"], np.float32)
    out = orc.finalize(rows, w)
    assert np.array_equal(val(out), np.array(g["out"], np.float32))
    ids = np.array(g["ids_invalid"], np.int32)
    out2 = orc.finalize(rows, w, ids)
    assert np.array_equal(val(out2), np.array(g["out_invalid"], np.float32))


def test_finalize_one_hot_copies_row(orc):
    g = syn.rng(1, 600)
    rows = syn.bf16_normal(g, (3 * 16, 64))
    w = np.zeros((3, 16), np.float32)
    w[0, 5] = w[1, 0] = w[2, 15] = 1.0
    out = orc.finalize(rows, w)
    assert np.array_equal(out[0], rows[5]) and np.array_equal(out[1], rows[16])
    assert np.array_equal(out[2], rows[47])


def test_finalize_power_of_two_exact(orc):
    g = np.random.default_rng(10)
    rows = syn.small_int_bf16(g, (4 * 16, 40), -100, 100)
    w = (2.0 ** g.integers(-3, 3, size=(4, 16))).astype(np.float32)
    out = orc.finalize(rows, w)
    ref = (val(rows).reshape(4, 16, 40).astype(np.float64) * w[:, :, None]).sum(axis=1)
    ref_b = torch.from_numpy(ref).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref_b)


def test_finalize_uses_fused_multiply_add(orc):
    # slot 0: w = -(1 + 2^-7 + 2^-20), row 1 -> acc = -(1 + 2^-7 + 2^-20) exactly.
    # slot 1: w = 1 + 2^-20, row = 1 + 2^-7 -> product 1 + 2^-7 + 2^-20 + 2^-27.
    # One fused rounding leaves 2^-27; rounding the product to FP32 first leaves 0.
    rows = np.zeros((16, 8), np.uint16)
    rows[0, :] = bits([1.0])[0]
    rows[1, :] = bits([1 + 2 ** -7])[0]
    w = np.zeros((1, 16), np.float32)
    w[0, 0] = -(1 + 2 ** -7 + 2 ** -20)
    w[0, 1] = 1 + 2 ** -20
    out = orc.finalize(rows, w)
    assert np.all(val(out[0]) == np.float32(2.0 ** -27))


def test_finalize_invalid_equals_zero_weight(orc):
    rows, w, ids = syn.finalize_inputs(T=8, K=16, cols=64, seed=1, invalid=True)
    a = orc.finalize(rows, w, ids)
    b = orc.finalize(rows, w)  # weights of invalid slots are 0 already
    assert np.array_equal(a, b)
    # an invalid slot's row is never read: poisoning it changes nothing
    rows2 = rows.copy()
    t = np.arange(8)
    for tt in t:
        rows2[tt * 16 + tt % 16] = 0x7FC0
    assert np.array_equal(orc.finalize(rows2, w, ids), a)


def test_rmsnorm_closed_form_and_scale_invariance(orc):
    c = np.float32(0.75)
    r = bits(np.full((1, 256), c))
    g = bits(np.full(256, 2.0))
    out = orc.rmsnorm(r, g, 1e-5)
    ref = np.float32(float(c) / np.sqrt(float(c) ** 2 + float(np.float32(1e-5))) * 2.0)
    refb = torch.tensor([float(ref)]).to(torch.bfloat16).float().item()
    assert np.all(val(out) == refb)
    x = syn.bf16_normal(syn.rng(0, 601), (4, 512), 1.0)
    gg = syn.bf16_normal(syn.rng(0, 602), (512,), 1.0)
    a = orc.rmsnorm(x, gg, 0.0)
    b = orc.rmsnorm(bits(val(x) * 4.0), gg, 0.0)  # x4 is exact in BF16
    assert np.array_equal(a, b)
    xt = torch.from_numpy(val(x)).double()
    ref = xt / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + float(np.float32(1e-5)))
    ref = (ref * torch.from_numpy(val(gg)).double()).float().to(torch.bfloat16).float().numpy()
    got = val(orc.rmsnorm(x, gg, 1e-5))
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2 ** -8


def test_linear_bf16_small_int_exact(orc):
    g = np.random.default_rng(11)
    x = syn.small_int_bf16(g, (6, 200))
    w = syn.small_int_bf16(g, (5, 200))
    out = orc.linear_bf16(x, w)
    ref = val(x).astype(np.int64) @ val(w).astype(np.int64).T
    refb = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(val(out), refb)


def test_linear_add_zero_input_returns_addend(orc):
    g = syn.rng(0, 603)
    add = syn.bf16_normal(g, (3, 40))
    x = np.zeros((3, 16), np.uint16)
    w = syn.bf16_normal(g, (40, 16))
    assert np.array_equal(orc.linear_add_bf16(x, w, add), add)


def test_linear_add_vs_torch(orc):
    g = syn.rng(0, 604)
    x = syn.bf16_normal(g, (3, 64))
    w = syn.bf16_normal(g, (24, 64), 0.125)
    add = syn.bf16_normal(g, (3, 24))
    out = orc.linear_add_bf16(x, w, add)
    tx = torch.from_numpy(val(x)).double()
    tw = torch.from_numpy(val(w)).double()
    acc = (tx @ tw.T).float()
    ref = (torch.from_numpy(val(add)) + acc).to(torch.bfloat16).float().numpy()
    assert np.array_equal(val(out), ref)


def test_silu_mul_vs_torch(orc):
    gu = syn.bf16_normal(syn.rng(0, 605), (5, 2 * 96), 2.0)
    out = orc.silu_mul_bf16(gu)
    t = torch.from_numpy(val(gu)).double()
    ref = (torch.nn.functional.silu(t[:, :96]) * t[:, 96:]).float().to(torch.bfloat16).float()
    assert np.array_equal(val(out), ref.numpy())
