"""GPU parity of the dense BF16 linears (router FP32 out, BF16 out, BF16 out + addend) at
the layer's projection shapes (sampled rows), with small-integer inputs (exact in any
summation order: bit-exact), and at ragged shapes that exercise every tile edge and
both the split-K and the single-pass paths."""
import numpy as np
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import assert_close, assert_close_bf16, dev, f32, host, say

pytestmark = pytest.mark.gpu


def run_linear(x, w, mode, add=None):
    M, K = x.shape
    N = w.shape[0]
    out = torch.empty(M, N, dtype=torch.float32 if mode == 0 else torch.bfloat16, device="cuda")
    ws_bytes = moe.moe_linear_workspace_size(M, N, K)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    moe.moe_linear(dev(x), dev(w), out, add=None if add is None else dev(add), mode=mode,
                   workspace=ws)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("M,N,K", [(256, 896, 7168), (3, 40, 64), (130, 136, 192),
                                   (1020, 256, 512), (65, 1000, 1024)])
def test_linear_small_int_exact(orc, M, N, K):
    g = np.random.default_rng(M + N + K)
    x = syn.small_int_bf16(g, (M, K), -2, 2)
    w = syn.small_int_bf16(g, (N, K), -2, 2)
    ref = (f32(x).astype(np.int64) @ f32(w).astype(np.int64).T).astype(np.float32)
    assert np.array_equal(run_linear(x, w, 0), ref)


# the weight-streaming path (K % 128 == 0, N % 32 == 0): one token, ragged 32-token tiles,
# a second 256-token chunk that is partly empty, every token-tile count 1..8, split-K; the
# narrow batches of 1..8 tokens at the front GEMM's and the up-projection's shapes
@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (2, 96, 256), (3, 4480, 7168), (4, 64, 384),
                                   (5, 7168, 3584), (8, 224, 640),
                                   (300, 224, 384), (510, 512, 1024),
                                   (33, 4480, 7168), (97, 96, 256), (161, 64, 640),
                                   (200, 320, 896), (230, 128, 2048)])
def test_linear_streaming_small_int_exact(orc, M, N, K):
    say(f"streaming linear M={M} N={N} K={K}")
    g = np.random.default_rng(7 * M + N + K)
    x = syn.small_int_bf16(g, (M, K), -2, 2)
    w = syn.small_int_bf16(g, (N, K), -2, 2)
    ref = (f32(x).astype(np.int64) @ f32(w).astype(np.int64).T).astype(np.float32)
    assert np.array_equal(run_linear(x, w, 0), ref)


def test_pack_dense_layout():
    """moe_pack_dense_weight against the layout stated in the header, built here by
    indexing: block (g, s, i, q), lane l, element e = W[64g + 32i + l%32, 64s + 16q + 8(l//32) + e]."""
    N, K = 192, 384
    g = np.random.default_rng(5)
    w = g.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    got = host(moe.moe_pack_dense_weight(dev(w))).view(np.uint16).reshape(-1)
    ref = np.empty(N * K, np.uint16)
    at = 0
    lane = np.arange(64)
    for gi in range(N // 64):
        for si in range(K // 64):
            for i in range(2):
                for q in range(4):
                    rows = 64 * gi + 32 * i + lane % 32
                    cols = 64 * si + 16 * q + 8 * (lane // 32)
                    blk = w[rows[:, None], cols[:, None] + np.arange(8)[None, :]]
                    ref[at:at + 512] = blk.reshape(-1)
                    at += 512
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K,mode", [(256, 3584, 7168, 1), (256, 7168, 6144, 1),
                                        (256, 7168, 3584, 2), (256, 12288, 7168, 1),
                                        (1020, 896, 7168, 0), (7, 72, 128, 2), (129, 200, 256, 0)])
def test_linear_vs_oracle(orc, M, N, K, mode):
    say(f"linear M={M} N={N} K={K} mode={mode}")
    g = syn.rng(M, N, K)
    x = syn.bf16_normal(g, (M, K))
    w = syn.bf16_normal(g, (N, K), 1 / np.sqrt(K))
    add = syn.bf16_normal(g, (M, N)) if mode == 2 else None
    got = run_linear(x, w, mode, add)
    rows = np.unique(np.r_[0, 1, M // 2, M - 1])
    if mode == 0:
        ref = orc.linear_f32(x[rows], w)
        assert_close(got[rows], ref, "FP32 out")
    elif mode == 1:
        ref = orc.linear_bf16(x[rows], w)
        assert_close_bf16(got[rows], ref, "BF16 out")
    else:
        ref = orc.linear_add_bf16(x[rows], w, add[rows])
        assert_close_bf16(got[rows], ref, "BF16 out + add")


def test_linear_add_aliases_output(orc):
    g = syn.rng(3, 3)
    M, N, K = 64, 256, 512
    x = syn.bf16_normal(g, (M, K))
    w = syn.bf16_normal(g, (N, K), 1 / np.sqrt(K))
    add = syn.bf16_normal(g, (M, N))
    buf = dev(add)
    ws = torch.empty(max(moe.moe_linear_workspace_size(M, N, K), 16), dtype=torch.uint8,
                     device="cuda")
    moe.moe_linear(dev(x), dev(w), buf, add=buf, mode=moe.MOE_LINEAR_ADD_BF16, workspace=ws)
    torch.cuda.synchronize()
    assert_close_bf16(host(buf), orc.linear_add_bf16(x, w, add), "in-place add")
