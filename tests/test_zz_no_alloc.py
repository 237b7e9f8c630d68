"""moe_grouped_ffn_noalloc (the grouped FFN with its scratch in the library's own device
array, for callers that cannot allocate) against moe_grouped_ffn with a caller workspace:
rows bit for bit equal, on two calls in a row -- the second with a smaller input, so that
whatever the first left in the shared array must not leak into it -- for row-major and
packed expert weights."""
import numpy as np
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def lists(d, ids):
    T, K, E = d.tokens, d.top_k, d.experts
    P = T * K
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pairs = torch.empty(P, dtype=torch.int32, device="cuda")
    units = torch.empty(-(-P // d.unit_tokens) + E, 4, dtype=torch.int32, device="cuda")
    nu = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_lists_workspace_size(d), dtype=torch.uint8, device="cuda")
    moe.moe_build_lists(d, dev(ids), counts, offsets, pairs, units, nu, ws)
    return pairs, units, nu


def case(T, K, E, L, I, seed, packed):
    """Expert weights, an MXFP8 latent and top-K ids (one expert in every token)."""
    w = syn.expert_weights(dict(L=L, I=I, E=E, expert_format=0), seed=seed)
    codes, scales = syn.mxfp8_random(syn.rng(seed, 710), T, L)
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[:, 0] = np.where((ids == 1).any(axis=1), ids[:, 0], 1)
    fmt = moe.MOE_FMT_MXFP4_MXFP8_PACKED if packed else moe.MOE_FMT_MXFP4_MXFP8
    d = moe.dims(T, T, hidden=256, latent=L, experts=E, top_k=K, expert_inter=I,
                 expert_format=fmt)
    wd = [dev(w[k]) for k in ("w13", "s13", "w2", "s2")]
    if packed:
        wd = list(moe.moe_pack_expert_weights(d, *wd))
    return d, wd, dev(codes), dev(scales), ids


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_workspace_call(packed):
    assert moe.moe_grouped_ffn_noalloc_max_bytes() == 9 << 20
    for T, K, E, L, I, seed in ((256, 16, 64, 3584, 512, 1), (13, 4, 9, 1024, 256, 2)):
        say(f"noalloc packed={packed} T={T} K={K} E={E} L={L} I={I}")
        d, wd, codes, scales, ids = case(T, K, E, L, I, seed, packed)
        pairs, units, nu = lists(d, ids)
        ref = torch.zeros(T * K, L, dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
        moe.moe_grouped_ffn(d, *wd, codes, scales, pairs, units, nu, ref, ws)
        got = torch.full((T * K, L), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_grouped_ffn_noalloc(d, *wd, codes, scales, pairs, units, nu, got)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint16), host(ref).view(np.uint16))


def test_noalloc_rejects_oversize():
    d = moe.dims(2048, 2048, expert_format=moe.MOE_FMT_MXFP4_MXFP8)  # 2048 x 16 x 528 B > 9 MiB
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_grouped_ffn_noalloc(d, t, t, t, t, t, t, t.view(torch.int32), t.view(torch.int32),
                                    t.view(torch.int32), t.view(torch.bfloat16))
    assert "MOE_ERR_WORKSPACE" in str(e.value)
