"""The C-ABI library loads, exports every entry point include/moedecode.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every call here
fails validation, so nothing is enqueued).  CPU only."""
import ctypes as C
import os
import re

import pytest

import mixture_experts_decode_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # a 256-aligned address that is never dereferenced here


def header_entry_points():
    with open(os.path.join(ROOT, "include", "moedecode.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*)\s+(moe_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_exports_every_declared_entry_point(L):
    names = header_entry_points()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert sorted(moe.EXPORTS) == names
    assert "gfx950" in moe.moe_version()


def test_exports_nothing_undeclared(L):
    """The library's dynamic symbol table holds exactly the header's entry points: every
    kernel, launcher and helper stays internal."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    from mixture_experts_decode_gemm_amd import build
    r = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True,
                       text=True, check=True)
    syms = sorted(line.split()[-1] for line in r.stdout.splitlines() if line.strip())
    assert syms == header_entry_points()


def test_noalloc_ffn_rejects_oversize_on_host(L):
    """The allocation-free grouped FFN refuses, before any launch, a call whose scratch
    exceeds its fixed device array (2048 tokens x top-16 x (512 + 16) bytes > 9 MiB)."""
    d = moe.dims(2048, 2048)
    w = moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE)
    st = L.moe_grouped_ffn_noalloc(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None)
    assert st == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn_noalloc_max_bytes() == 9 << 20


def good_dims(**kw):
    d = moe.dims(256, 1020)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_sizes_are_positive_and_monotone(L):
    small = moe.moe_workspace_size(moe.dims(8, 8))
    big = moe.moe_workspace_size(moe.dims(8, 1020))
    assert 0 < small < big
    assert moe.moe_router_workspace_size(moe.dims(256, 256)) > 0
    assert moe.moe_ffn_workspace_size(moe.dims(256, 256)) >= 256 * 16 * 512
    lo = moe.moe_workspace_layout(moe.dims(256, 256))
    offs = [lo[k] for k in moe.WORKSPACE_FIELDS]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert moe.moe_workspace_size(good_dims(tokens=0)) == 0


@pytest.mark.parametrize("field,value,status", [
    ("tokens", 0, moe.MOE_ERR_SHAPE),
    ("tokens", 1021, moe.MOE_ERR_SHAPE),
    ("max_tokens", 5000, moe.MOE_ERR_SHAPE),
    ("latent", 3584 + 32, moe.MOE_ERR_SHAPE),
    ("hidden", 7000, moe.MOE_ERR_SHAPE),
    ("experts", 2000, moe.MOE_ERR_SHAPE),
    ("top_k", 17, moe.MOE_ERR_SHAPE),
    ("top_k", 0, moe.MOE_ERR_SHAPE),
    ("expert_inter", 500, moe.MOE_ERR_SHAPE),
    ("unit_tokens", 4, moe.MOE_ERR_SHAPE),
    ("expert_format", 7, moe.MOE_ERR_FORMAT),
])
def test_layer_rejects_bad_dims(L, field, value, status):
    d = good_dims(**{field: value})
    w = moe.moe_layer_weights(*([FAKE] * 7), moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE))
    st = L.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == status


def test_layer_rejects_null_align_workspace(L):
    d = good_dims()
    w = moe.moe_layer_weights(*([FAKE] * 7), moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE))
    assert L.moe_layer(C.byref(d), C.byref(w), None, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_NULL
    w2 = moe.moe_layer_weights(*([FAKE] * 7), moe.moe_expert_weights(FAKE, None, FAKE, FAKE))
    assert L.moe_layer(C.byref(d), C.byref(w2), FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_NULL
    assert L.moe_layer(C.byref(d), C.byref(w), FAKE + 8, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_ALIGN
    need = moe.moe_workspace_size(d)
    assert L.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, need - 1, None) == moe.MOE_ERR_WORKSPACE


def test_finalize_rejects(L):
    assert L.moe_finalize(0, 16, 3584, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_finalize(4, 17, 3584, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_finalize(4, 16, 3580, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_finalize(4, 16, 3584, None, FAKE, None, FAKE, None) == moe.MOE_ERR_NULL
    assert L.moe_finalize(4, 16, 3584, FAKE, FAKE, FAKE + 4, FAKE, None) == moe.MOE_ERR_ALIGN


def test_quant_rejects(L):
    assert L.moe_quant_mxfp8(4, 48, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quant_mxfp8(0, 64, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quant_mxfp8(4, 64, FAKE, None, FAKE, None) == moe.MOE_ERR_NULL
    assert L.moe_quant_mxfp8(4, 64, FAKE + 2, FAKE, FAKE, None) == moe.MOE_ERR_ALIGN


def test_router_rejects(L):
    d = good_dims()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.moe_router_topk(C.byref(d), *args, 4, FAKE, 1 << 40, None) == moe.MOE_ERR_FORMAT
    # a packed W_gate needs experts % 64 == 0
    d32 = good_dims()
    d32.experts, d32.top_k = 32, 4
    assert L.moe_router_topk(C.byref(d32), *args, moe.MOE_GATE_PACKED, FAKE, 1 << 40,
                             None) == moe.MOE_ERR_FORMAT
    need = moe.moe_router_workspace_size(d)
    assert need > 0
    assert L.moe_router_topk(C.byref(d), *args, 0, FAKE, 16, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_router_topk(C.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, need,
                             None) == moe.MOE_ERR_NULL
    d.top_k = 1000
    assert L.moe_router_topk(C.byref(d), *args, 1, None, 0, None) == moe.MOE_ERR_SHAPE


def test_lists_and_ffn_reject(L):
    d = good_dims()
    assert L.moe_build_lists(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                             None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_build_lists(C.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                             None) == moe.MOE_ERR_NULL
    w = moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE)
    assert L.moe_grouped_ffn(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                             None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn(C.byref(d), C.byref(w), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             1 << 30, None) == moe.MOE_ERR_NULL
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30)
    for bad in (0, 4, -1):
        assert L.moe_grouped_ffn_stages(C.byref(d), C.byref(w), *args, bad,
                                        None) == moe.MOE_ERR_FORMAT
    # the down pass alone needs no activations; the up pass alone no rows
    assert L.moe_grouped_ffn_stages(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, 16, moe.MOE_FFN_UP, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn_stages(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, 16, moe.MOE_FFN_DOWN, None) == moe.MOE_ERR_NULL
    assert L.moe_grouped_ffn_stages(C.byref(d), C.byref(w), None, None, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, 16, moe.MOE_FFN_DOWN, None) == moe.MOE_ERR_WORKSPACE
    d.expert_format = moe.MOE_FMT_BF16
    assert L.moe_grouped_ffn_stages(C.byref(d), C.byref(w), *args, moe.MOE_FFN_UP,
                                    None) == moe.MOE_ERR_FORMAT


def test_packed_format_and_pack_reject(L):
    d = good_dims()
    d.expert_format = moe.MOE_FMT_MXFP4_MXFP8_PACKED
    assert moe.moe_workspace_size(d) > 0  # latent 3584, inter 512: accepted
    w = moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE)
    for latent, inter in ((3584 - 256, 512), (3584, 384), (4096, 512)):
        d.latent, d.expert_inter = latent, inter
        assert moe.moe_workspace_size(d) == 0
        assert L.moe_pack_expert_weights(C.byref(d), C.byref(w), C.byref(w),
                                         None) == moe.MOE_ERR_SHAPE
    d = good_dims()
    bad = moe.moe_expert_weights(FAKE, None, FAKE, FAKE)
    assert L.moe_pack_expert_weights(C.byref(d), C.byref(w), C.byref(bad), None) == moe.MOE_ERR_NULL
    assert L.moe_pack_expert_weights(None, C.byref(w), C.byref(w), None) == moe.MOE_ERR_NULL


def test_dense_format_and_pack_dense_reject(L):
    d = good_dims()
    ew = moe.moe_expert_weights(FAKE, FAKE, FAKE, FAKE)
    w = moe.moe_layer_weights(*([FAKE] * 7), ew, 5)
    assert L.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_FORMAT
    # packed dense weights need every matrix's rows in whole 64-row groups
    d = good_dims(experts=96)
    w = moe.moe_layer_weights(*([FAKE] * 7), ew, moe.MOE_DENSE_PACKED)
    assert L.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_dense_weight(32, 128, FAKE, FAKE + 4096, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_dense_weight(64, 64, FAKE, FAKE + 4096, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_dense_weight(64, 128, None, FAKE, None) == moe.MOE_ERR_NULL
    assert L.moe_pack_dense_weight(64, 128, FAKE + 8, FAKE + (1 << 20), None) == moe.MOE_ERR_ALIGN
    assert L.moe_pack_dense_weight(64, 128, FAKE, FAKE + 16, None) == moe.MOE_ERR_SHAPE  # overlap


def test_linear_rmsnorm_silu_reject(L):
    assert L.moe_linear(8, 64, 100, FAKE, FAKE, FAKE, None, 1, None, 0, None) == moe.MOE_ERR_SHAPE
    assert L.moe_linear(8, 64, 128, FAKE, FAKE, FAKE, None, 5, None, 0, None) == moe.MOE_ERR_FORMAT
    assert L.moe_linear(8, 64, 128, FAKE, FAKE, FAKE, None, 2, None, 0, None) == moe.MOE_ERR_NULL
    assert L.moe_linear(256, 896, 7168, FAKE, FAKE, FAKE, None, 0, None, 0,
                        None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_rmsnorm(4, 12, FAKE, FAKE, C.c_float(1e-5), FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_rmsnorm(4, 16, FAKE, FAKE, C.c_float(-1.0), FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_silu_mul(4, 12, FAKE, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_silu_mul(4, 16, FAKE, None, None) == moe.MOE_ERR_NULL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_quant_mxfp8(x, torch.zeros(4, 64, dtype=torch.uint8),
                            torch.zeros(4, 2, dtype=torch.uint8))
