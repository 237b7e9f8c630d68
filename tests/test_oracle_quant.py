"""Pins of the oracle's MXFP8 quantiser (OCP MX v1.0 reading): every BF16 pattern in
a block of known amax against torch's E4M3 conversion, the scale byte's closed form,
the all-zero block, signed zeros, saturation, idempotence and the error bound.  CPU."""
import numpy as np
import torch

import moe_synth as syn


def bf16_bits(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_every_bf16_pattern_in_unit_block(orc):
    # block = [1.0, v, 0 ...]: amax 1 -> floor(log2) = 0 -> X = 2^-8 -> scale byte 119
    pats = np.arange(65536, dtype=np.uint16)
    v = bf16_val(pats)
    keep = np.isfinite(v) & (np.abs(v) <= 1.0)
    pats = pats[keep]
    x = np.zeros((pats.size, 32), np.uint16)
    x[:, 0] = bf16_bits([1.0])[0]
    x[:, 7] = pats
    codes, scales = orc.quant_mxfp8_bf16(x)
    assert np.all(scales == 119)
    ref = torch.from_numpy(bf16_val(pats) * np.float32(256.0)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    assert np.array_equal(codes[:, 7], ref)
    assert np.all(codes[:, 0] == 0x78)  # 1.0 * 2^8 = 256: E4M3 exponent field 8 + 7 = 15, mantissa 0
    assert np.all(codes[:, 1:7] == 0) and np.all(codes[:, 8:] == 0)


def test_scale_byte_closed_form(orc):
    for e in range(-60, 60, 7):
        for frac in (1.0, 1.5, 1.9921875):
            a = frac * 2.0 ** e
            x = np.zeros((1, 32), np.float32)
            x[0, 3] = -a
            codes, scales = orc.quant_mxfp8_f32(x)
            want = min(max(e - 8, -127), 127) + 127
            assert scales[0, 0] == want
            # the amax element lands in [256, 512) -> at least 256, saturating at 448
            v = orc.e4m3_value(int(codes[0, 3]))
            assert -448 <= v <= -256


def test_zero_block_and_signed_zeros(orc):
    x = np.zeros((1, 64), np.float32)
    x[0, 5] = -0.0
    x[0, 40] = 3.0
    x[0, 41] = -0.0
    codes, scales = orc.quant_mxfp8_f32(x)
    assert scales[0, 0] == 0 and codes[0, 5] == 0x80 and np.all(np.delete(codes[0, :32], 5) == 0)
    assert codes[0, 41] == 0x80 and scales[0, 1] == 1 - 8 + 127


def test_saturation(orc):
    # amax = 1.999 * 2^k -> amax / 2^(k-8) = 511.7 > 448 -> saturates to 0x7E
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.999 * 4.0
    x[0, 1] = -1.999 * 4.0
    codes, _ = orc.quant_mxfp8_f32(x)
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0xFE


def test_idempotence_and_error_bound(orc):
    g = syn.rng(0, 77)
    x = syn.bf16_normal(g, (64, 256), 3.0)
    codes, scales = orc.quant_mxfp8_bf16(x)
    xs = bf16_val(x).astype(np.float64).reshape(64, 8, 32)
    X = np.array([[orc.e8m0_value(int(s)) for s in row] for row in scales])[:, :, None]
    table = np.array([orc.e4m3_value(c) for c in range(256)])
    deq = table[codes].reshape(64, 8, 32) * X
    # error bound: half an E4M3 step at the element's binade (x 2^X), except saturation
    q = xs / X
    binade = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
    half_step = 0.5 * 2.0 ** (binade - 3)
    sat = np.abs(q) > 448
    err = np.abs(deq - xs) / X
    assert np.all(err[~sat] <= half_step[~sat] + 1e-12)
    assert np.all(err[sat] <= 64 + 1e-9)
    # idempotence: the dequantised block quantises back to the same codes and scales
    back = deq.reshape(64, 256).astype(np.float32)
    c2, s2 = orc.quant_mxfp8_f32(back)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_bf16_and_f32_paths_agree(orc):
    g = syn.rng(0, 78)
    x = syn.bf16_normal(g, (16, 128), 0.01)
    c1, s1 = orc.quant_mxfp8_bf16(x)
    c2, s2 = orc.quant_mxfp8_f32(bf16_val(x))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_subnormal_amax(orc):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(2.0 ** -140)  # FP32 subnormal
    codes, scales = orc.quant_mxfp8_f32(x)
    assert scales[0, 0] == 0  # floor(log2) = -140 -> -148 clamps to -127
    # 2^-140 * 2^127 = 2^-13 lies below half the smallest E4M3 subnormal (2^-10)
    assert codes[0, 0] == 0x00
