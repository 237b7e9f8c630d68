"""moe_layer captured in a HIP graph (stream capture through torch.cuda.CUDAGraph): the
library allocates nothing, issues no memset and joins its side stream back into the
caller's stream with events, so one layer step can be captured whole -- the shared
expert's side-stream kernels included -- and replayed.  Every replay, with eager layer
steps and synchronisations between them, gives the eager step's output bit for bit."""
import pytest
import torch

import moe_synth as syn
import mixture_experts_decode_gemm_amd as moe
from gpu_util import dev, full_weights, say

pytestmark = pytest.mark.gpu


# 256 tokens: the shared expert forked at the start of the step; 510: forked after the
# lists, its GEMMs unsplit; 8: planned for the whole GPU
@pytest.mark.parametrize("T", [256, 510, 8])
def test_layer_graph_replays_equal_eager(T):
    say(f"layer in a HIP graph T={T}")
    _, dw0 = full_weights(0, False)
    dw = dict(dw0)  # (the cached weights stay row-major for the other tests)
    for k in ("w_gate", "w_down", "w_shared_gu", "w_shared_dn", "w_up"):
        dw[k] = moe.moe_pack_dense_weight(dw[k])
    pk = moe.moe_pack_expert_weights(moe.dims(1, 1), dw["w13"], dw["s13"], dw["w2"], dw["s2"])
    dw.update(w13=pk[0], s13=pk[1], w2=pk[2], s2=pk[3])
    lw = moe.layer_weights(dw["w_gate"], dw["bias"], dw["w_down"], dw["w_shared_gu"],
                           dw["w_shared_dn"], dw["norm_w"], dw["w_up"], dw["w13"], dw["s13"],
                           dw["w2"], dw["s2"], dense_format=moe.MOE_DENSE_PACKED)
    d = moe.dims(T, 1020, expert_format=moe.MOE_FMT_MXFP4_MXFP8_PACKED)
    x = dev(syn.layer_input(syn.full_dims(T), seed=3))
    ws = torch.zeros(moe.moe_workspace_size(d), dtype=torch.uint8, device="cuda")
    out_e = torch.empty(T, d.hidden, dtype=torch.bfloat16, device="cuda")
    out_g = torch.empty_like(out_e)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        moe.moe_layer(d, lw, x, out_e, ws, s)
    torch.cuda.synchronize()
    ref = out_e.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_layer(d, lw, x, out_g, ws, s)
    torch.cuda.synchronize()
    for rep in range(4):
        out_g.fill_(0)  # (eager work outside the graph)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), rep
        with torch.cuda.stream(s):  # an eager step between replays, same workspace
            moe.moe_layer(d, lw, x, out_e, ws, s)
        torch.cuda.synchronize()
        assert torch.equal(out_e.view(torch.int16), ref.view(torch.int16)), rep
