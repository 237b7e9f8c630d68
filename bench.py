"""Benchmark of one wide-batch latent-MoE decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--tokens 256] [--zipf]
                    [--no-cpu-baseline] [--sweep]

A step is one moe_layer call (router GEMM, sigmoid top-16, lists and unit windows,
latent down, MXFP8 latent, grouped MXFP4 x MXFP8 experts, Finalize, RMSNorm, shared
expert, up-projection add) over T tokens of synthetic input resident in HBM: hidden
7168, latent 3584, 896 experts, top-16, expert intermediate 512, shared intermediate
6144.  Prints one JSON line: tokens/s, the layer's HBM-roofline fraction over the weight
bytes it must stream (dense + each touched expert once), the grouped-FFN kernel's
roofline (HIP events on the launch stream), and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
DENSE_BYTES = 379_857_408          # router + shared gate_up + shared down + latent down + up + norm + bias
EXPERT_BYTES = 2_924_544           # one MXFP4 expert: W13 + scales + W2 + scales
UP_EXPERT_BYTES = 1_949_696        # W13 [1024, 3584] MXFP4 + E8M0 scales
DOWN_EXPERT_BYTES = 974_848        # W2 [3584, 512] MXFP4 + E8M0 scales
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_ffn_up_fast_T256_uniform_traffic.md")
KERNEL_SOURCES = ["mixture_experts_decode_gemm_amd/csrc/ffn.hip",
                  "mixture_experts_decode_gemm_amd/csrc/device.h"]


def source_digest():
    """Hash of the gate/up kernel's sources with comments and blank space removed, so that
    only a change of code (not of its comments) retires the recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(T, zipf, row_major):
    """HBM bytes per launch of the gate/up kernel from the committed PMC summary (FETCH_SIZE
    and WRITE_SIZE, each scaled by the same counter's reading for a copy of known size), or
    None when there is none for this workload or the kernel's source changed since."""
    if T != 256 or zipf or row_major or not os.path.exists(TRAFFIC_FILE):
        return None
    import re
    m = re.search(r"```json\n(.*?)\n```", open(TRAFFIC_FILE).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_digest") != source_digest():
        return None
    return rec["traffic_bytes_per_launch"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # the GPU lowers its clocks when idle and takes some 0.1 s of load to reach them
    # again: the default warmup (~0.2 s of layers) measures the steady state
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--tokens", type=int, default=256)
    p.add_argument("--zipf", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=192)
    p.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                   help="finish with one plain copy kernel of this many MiB (read and written), "
                        "the reference for scaling the HBM byte counters")
    p.add_argument("--sweep", action="store_true", help="also time T in {65,130,255,510,1020}")
    p.add_argument("--row-major", action="store_true",
                   help="run on the row-major expert and dense weights instead of the packed layouts")
    return p.parse_args()


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs at TP1 on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_synth as syn
    import mixture_experts_decode_gemm_amd as moe

    moe.lib()  # raises when the HIP library is not built: there is no fallback
    T = a.tokens
    d0 = syn.full_dims(T)
    t0 = time.time()
    w = syn.layer_weights(d0, seed=0)
    if a.zipf:
        w["bias"] = syn.routing_bias(896, 1, True)
    x = syn.layer_input(syn.full_dims(1020), seed=1)  # the widest batch; the first T rows are used

    def dev(arr):
        arr = np.ascontiguousarray(arr)
        if arr.dtype == np.uint16:
            return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(arr).cuda()

    dw = {k: dev(v) for k, v in w.items() if v is not None}
    xd = dev(x)
    fmt = moe.MOE_FMT_MXFP4_MXFP8
    if not a.row_major:  # load-time preparation of the expert weights, outside any timing
        pk = moe.moe_pack_expert_weights(moe.dims(1, 1), dw["w13"], dw["s13"], dw["w2"], dw["s2"])
        dw.update(w13=pk[0], s13=pk[1], w2=pk[2], s2=pk[3])
        fmt = moe.MOE_FMT_MXFP4_MXFP8_PACKED
        for k in ("w_gate", "w_down", "w_shared_gu", "w_shared_dn", "w_up"):  # dense weights too
            dw[k] = moe.moe_pack_dense_weight(dw[k])
        torch.cuda.synchronize()
    print(f"# inputs generated and resident in HBM in {time.time() - t0:.1f} s", file=sys.stderr,
          flush=True)
    lw = moe.layer_weights(dw["w_gate"], dw["bias"], dw["w_down"], dw["w_shared_gu"],
                           dw["w_shared_dn"], dw["norm_w"], dw["w_up"], dw["w13"], dw["s13"],
                           dw["w2"], dw["s2"],
                           dense_format=moe.MOE_DENSE_ROWMAJOR if a.row_major else moe.MOE_DENSE_PACKED)
    dmax = moe.dims(1020, 1020, expert_format=fmt)
    ws = torch.zeros(moe.moe_workspace_size(dmax), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run_T(t, steps, warmup):
        d = moe.dims(t, 1020, expert_format=fmt)
        xin = xd[:t].contiguous()
        out = torch.empty(t, 7168, dtype=torch.bfloat16, device="cuda")
        for _ in range(warmup):
            moe.moe_layer(d, lw, xin, out, ws, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            moe.moe_layer(d, lw, xin, out, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        v = moe.workspace_views(d, ws)
        D = int(torch.count_nonzero(v["counts"]).item())
        nu = int(v["num_units"][0].item())
        return ms, D, nu, d, v

    ms, D, nu, d, v = run_T(T, a.steps, a.warmup)
    layer_bytes = DENSE_BYTES + D * EXPERT_BYTES
    layer_gbs = layer_bytes / (ms * 1e-3) / 1e9
    print(f"# T={T}: {ms * 1e3:.1f} us/layer, D={D} touched experts, {nu} units, "
          f"{layer_gbs:.0f} GB/s = {100 * layer_gbs / HBM_PEAK_GBS:.1f}% of HBM", file=sys.stderr,
          flush=True)

    # the dominant kernel: the grouped FFN's gate/up pass (one launch of k_ffn_up_fast),
    # timed with HIP events on its launch stream and fed the layer's own codes, lists and
    # units; then the down pass and the whole grouped FFN the same way
    rows = torch.empty(T * 16, 3584, dtype=torch.bfloat16, device="cuda")
    fws = torch.zeros(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
    ffn_w = (d, dw["w13"], dw["s13"], dw["w2"], dw["s2"])
    lists = (v["pairs"], v["units_raw"], v["num_units"])

    def time_stage(stages):
        def call():
            moe.moe_grouped_ffn_stages(*ffn_w, v["codes"], v["scales"], *lists, rows, fws,
                                       stages, stream=stream)
        for _ in range(max(a.warmup // 2, 3)):  # back to steady-state clocks after the host work
            call()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(a.steps):
            call()
        f1.record(stream)
        torch.cuda.synchronize()
        return f0.elapsed_time(f1) / a.steps * 1e3

    moe.moe_grouped_ffn_stages(*ffn_w, v["codes"], v["scales"], *lists, rows, fws, moe.MOE_FFN_UP,
                               stream=stream)
    up_us = time_stage(moe.MOE_FFN_UP)
    down_us = time_stage(moe.MOE_FFN_DOWN)
    ffn_us = time_stage(moe.MOE_FFN_UP | moe.MOE_FFN_DOWN)
    # algorithmic bytes per launch: each touched expert's W13 (+ scales) once, the MXFP8
    # latent once, the MXFP8 hidden of every pair written once (up); each touched expert's
    # W2 (+ scales) once, the hidden read once, the BF16 rows written once (down)
    hid_bytes = T * 16 * 512 * 33 // 32
    up_bytes = D * UP_EXPERT_BYTES + T * 3584 * 33 // 32 + hid_bytes
    down_bytes = D * DOWN_EXPERT_BYTES + hid_bytes + T * 16 * 3584 * 2
    up_gbs = up_bytes / up_us / 1e3
    traffic = recorded_traffic(T, a.zipf, a.row_major)

    res = {
        "metric": "MoE-layer decode tokens/s at 256 tokens; % of HBM roofline (GB/s achieved)",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+mxfp4xmxfp8",
        "data": "synthetic (seeded; random-init weights of the layer's shapes)",
        "config": {"workload": f"wide latent-MoE decode layer, T={T} tokens, hidden 7168, latent "
                               f"3584, 896 MXFP4 experts top-16, expert inter 512, shared inter "
                               f"6144, {'Zipf' if a.zipf else 'uniform'} routing bias, "
                               f"{'row-major' if a.row_major else 'packed'} expert and dense weights",
                   "tokens": T, "touched_experts": D, "units": nu},
        "layer_roofline": {"bound": "hbm", "weight_bytes": layer_bytes,
                           "achieved": layer_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": layer_gbs / HBM_PEAK_GBS},
        "roofline": {"kernel": "k_ffn_up_fast (gate/up pass of the grouped expert FFN, "
                               + ("row-major" if a.row_major else "packed") + " expert weights)",
                     "bound": "hbm", "achieved": up_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": up_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": up_bytes, "us_per_launch": up_us},
        "ffn_down": {"kernel": "k_ffn_down_fast", "us_per_launch": down_us,
                     "bytes_per_launch": down_bytes, "achieved_gbs": down_bytes / down_us / 1e3},
        "grouped_ffn": {"us_per_call": ffn_us, "bytes_per_call": up_bytes + down_bytes,
                        "achieved_gbs": (up_bytes + down_bytes) / ffn_us / 1e3},
    }
    if a.sweep:
        sweep = {}
        for t in (65, 130, 255, 510, 1020):
            m, Dt, nut, _, _ = run_T(t, max(5, a.steps // 2), 50)
            bt = DENSE_BYTES + Dt * EXPERT_BYTES
            sweep[str(t)] = {"us": m * 1e3, "tokens_per_s": t / (m * 1e-3), "D": Dt, "units": nut,
                             "gbs": bt / (m * 1e-3) / 1e9,
                             "hbm_frac": bt / (m * 1e-3) / 1e9 / HBM_PEAK_GBS}
            print(f"# sweep T={t}: {m * 1e3:.1f} us", file=sys.stderr, flush=True)
        res["sweep"] = sweep
    if not a.no_cpu_baseline:
        import oracle as orc
        n = a.cpu_tokens
        sub = np.arange(n)
        dsub = dict(d0, T=n)
        orc.lib()
        c0 = time.time()
        orc.layer(dsub, w, x[sub])
        sec = time.time() - c0
        res["cpu_baseline"] = {"value": n / sec, "unit": "tokens/s", "cores": orc.threads(),
                               "kind": "oracle",
                               "sample": f"the oracle layer on the first {n} of the {T} tokens "
                                         f"(same weights and inputs), {sec:.1f} s"}
    if a.copy_probe:
        n = a.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_probe MiB
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n * 4
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
