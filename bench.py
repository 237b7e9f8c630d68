"""Benchmark of one wide-batch latent-MoE decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--tokens 256] [--zipf]
                    [--no-cpu-baseline] [--no-sweep] [--no-extras] [--row-major]

A step is one moe_layer call (router GEMM, sigmoid top-16, lists and unit windows,
latent down, MXFP8 latent, grouped MXFP4 x MXFP8 experts, Finalize, RMSNorm, shared
expert, up-projection add) over T tokens of synthetic input resident in HBM: hidden
7168, latent 3584, 896 experts, top-16, expert intermediate 512, shared intermediate
6144.  Prints one JSON line: tokens/s, the layer's HBM-roofline fraction over the weight
bytes it must stream (dense + each touched expert once), the grouped-FFN kernel's
roofline (HIP events on the launch stream), the GPU clocks sampled while the steps ran,
and the CPU oracle timed on a bounded sample of the same workload.  By default it also
times the batch sweep (65 .. 1020 tokens, uniform and Zipf routing), Finalize alone and
the routing front alone (each over rotated input sets larger than the 256 MB last-level
cache), and a plain 1 GiB device copy as the achievable-bandwidth reference.

Warm-up: after the W requested warm-up steps, steps continue untimed until the warm-up
has run for at least WARM_FLOOR_S seconds of GPU work (the GPU lowers its clocks when
idle and takes ~0.1 s of load to raise them); the line states how many ran.
"""
import argparse
import json
import os
import statistics
import sys
import threading
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_FLOPS = 2.5e15
FP8_PEAK_FLOPS = 5.0e15
DENSE_BYTES = 379_857_408          # router + shared gate_up + shared down + latent down + up + norm + bias
DENSE_FLOPS_PER_TOKEN = 379_846_656
EXPERT_FLOPS_PER_PAIR = 11_010_048
EXPERT_BYTES = 2_924_544           # one MXFP4 expert: W13 + scales + W2 + scales
UP_EXPERT_BYTES = 1_949_696        # W13 [1024, 3584] MXFP4 + E8M0 scales
DOWN_EXPERT_BYTES = 974_848        # W2 [3584, 512] MXFP4 + E8M0 scales
WARM_FLOOR_S = 0.3                 # seconds of GPU work before the first timed layer step
STAGE_FLOOR_S = 0.1                # the same before each other timed measurement
ROTATE_SETS = 10                   # input sets rotated by the single-call timings (> 256 MB)
SWEEP_MIN_STEPS = 200              # timed steps of each batch-sweep point, at least
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


class Clocks:
    """GFX and memory clocks sampled from a thread (amdsmi) while the GPU works; None
    where the tool or the device's counters are not available to this process."""

    def __init__(self, torch):
        self.samples, self.err, self.h, self.mod = [], None, None, None
        self._stop = threading.Event()
        self._t = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            h = hs[0] if len(hs) == 1 else None
            if h is None:  # pick the handle of cuda:0 by its PCI bus
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for cand in hs:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(cand)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        h = cand
            if h is None:
                raise RuntimeError(f"{len(hs)} GPUs visible to amdsmi, none matched cuda:0")
            self.mod, self.h = amdsmi, h
            self.read()
        except Exception as e:  # noqa: BLE001 -- a missing tool is reported, not fatal
            self.err = f"{type(e).__name__}: {e}"[:200]
            self.mod = None

    def read(self):
        """(lowest and highest current GFX clock over the XCDs, the firmware's average GFX
        clock, the memory clock) in MHz, from the SMU's metrics table"""
        m = self.mod.amdsmi_get_gpu_metrics_info(self.h)

        def num(v):
            return v if isinstance(v, (int, float)) and not isinstance(v, bool) else None
        xcd = [c for c in (num(v) for v in (m.get("current_gfxclks") or [])) if c]
        return (min(xcd) if xcd else num(m.get("current_gfxclk")),
                max(xcd) if xcd else num(m.get("current_gfxclk")),
                num(m.get("average_gfxclk_frequency")), num(m.get("current_uclk")))

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append((time.perf_counter(), *self.read()))
            except Exception as e:  # noqa: BLE001
                self.err = f"{type(e).__name__}: {e}"[:200]
                return
            time.sleep(0.002)

    def start(self):
        if self.mod is not None and self._t is None:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()

    def stop(self):
        if self._t is not None:
            self._stop.set()
            self._t.join()
            self._t = None

    def count(self, t0, t1):
        return sum(1 for smp in self.samples if t0 <= smp[0] <= t1)

    def summary(self, t0, t1):
        if self.mod is None:
            return {"source": "amdsmi", "error": self.err}
        win = [s for s in self.samples if t0 <= s[0] <= t1]
        if not win:  # the window was shorter than one sample: the nearest earlier ones
            win = [s for s in self.samples if s[0] <= t1][-3:]

        def st(i):
            v = [s[i] for s in win if s[i] is not None]
            return {"min": min(v), "median": statistics.median(v), "max": max(v)} if v else None
        return {"source": "amdsmi gpu metrics", "samples": len(win), "sclk_xcd_min_mhz": st(1),
                "sclk_xcd_max_mhz": st(2), "sclk_average_mhz": st(3), "mclk_mhz": st(4)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--tokens", type=int, default=256)
    p.add_argument("--zipf", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=192)
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the batch sweep (1..64 narrow batches and the 65..1020 wide ones)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the Finalize, routing-front and copy-probe timings")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                   help="finish with one plain copy kernel of this many MiB (read and written), "
                        "the reference for scaling the HBM byte counters")
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
    uniform_bias = w["bias"]                     # N(0, 0.05), seed 0
    zipf_bias = syn.routing_bias(896, 1, True)   # Zipf(1.1)-skewed over a seeded permutation
    if a.zipf:
        w["bias"] = zipf_bias
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
    dense_format = moe.MOE_DENSE_ROWMAJOR if a.row_major else moe.MOE_DENSE_PACKED

    def lw_with(bias):
        return moe.layer_weights(dw["w_gate"], bias, dw["w_down"], dw["w_shared_gu"],
                                 dw["w_shared_dn"], dw["norm_w"], dw["w_up"], dw["w13"], dw["s13"],
                                 dw["w2"], dw["s2"], dense_format=dense_format)

    lw = lw_with(dw["bias"])
    dmax = moe.dims(1020, 1020, expert_format=fmt)
    ws = torch.zeros(moe.moe_workspace_size(dmax), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    clocks = Clocks(torch)

    def warm(call, n_min, floor_s):
        """n_min calls, then more until floor_s seconds of GPU work ran; returns the count."""
        n = 0
        t_start = time.perf_counter()
        while n < n_min or time.perf_counter() - t_start < floor_s:
            for _ in range(10):
                call()
            n += 10
            torch.cuda.synchronize()
        return n

    def run_T(t, steps, warmup, floor_s, weights=None):
        d = moe.dims(t, 1020, expert_format=fmt)
        xin = xd[:t].contiguous()
        out = torch.empty(t, 7168, dtype=torch.bfloat16, device="cuda")
        lwt = lw if weights is None else weights

        def step():
            moe.moe_layer(d, lwt, xin, out, ws, stream)
        hw = time.perf_counter()
        n_warm = warm(step, warmup, floor_s)
        # the K timed steps back to back, one event before and one after them
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            step()
        e1.record(stream)
        h1 = time.perf_counter()  # host enqueue time of the steps (the GPU runs behind)
        torch.cuda.synchronize()
        h2 = time.perf_counter()
        ms = e0.elapsed_time(e1) / steps
        # the per-step spread from a second run of K steps with an event after each step
        # (each event is one more marker packet in the stream, a few us of the step)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        ms_ev = ev[0].elapsed_time(ev[steps]) / steps
        v = moe.workspace_views(d, ws)
        D = int(torch.count_nonzero(v["counts"]).item())
        nu = int(v["num_units"][0].item())
        return dict(ms=ms, ms_median=statistics.median(per), ms_min=min(per), ms_ev=ms_ev,
                    D=D, units=nu,
                    d=d, v=v, warm_steps=n_warm, host_us=(h1 - h0) / steps * 1e6,
                    window=(h0, h2), warm_window=(hw, h2))

    def phase_bound_us(t, D):
        """The phase-wise speed of light: the dense projections at max(weight bytes / HBM,
        FLOPs / BF16 MFMA) plus the experts at max(expert bytes / HBM, FLOPs / FP8 MFMA)."""
        dense = max(DENSE_BYTES / (HBM_PEAK_GBS * 1e3), DENSE_FLOPS_PER_TOKEN * t / BF16_PEAK_FLOPS * 1e6)
        expert = max(D * EXPERT_BYTES / (HBM_PEAK_GBS * 1e3),
                     EXPERT_FLOPS_PER_PAIR * t * 16 / FP8_PEAK_FLOPS * 1e6)
        return dense + expert

    clocks.start()
    r = run_T(T, a.steps, a.warmup, WARM_FLOOR_S)
    # the clocks over the last 0.1 s of the same work up to the end of the timed steps (the
    # end of the warm-up included: a short timed run alone holds too few of the firmware's
    # samples to go by; the start of the warm-up, where the clocks still ramp, left out)
    h0, h2 = r["window"]
    t0 = max(r["warm_window"][0], min(h0, h2 - 0.1))
    clk = clocks.summary(t0, h2)
    clk["window_s"] = round(h2 - t0, 3)
    clk["samples_in_timed_steps"] = clocks.count(h0, h2)
    # the firmware's table at times returns idle values while the GPU runs at full load
    # (seen: every sample of a loaded window at ~150-250 MHz): flagged, not corrected
    med = (clk.get("sclk_xcd_max_mhz") or {}).get("median")
    if med is not None:
        clk["plausible"] = med >= 1000
    ms, D, nu, d, v = r["ms"], r["D"], r["units"], r["d"], r["v"]
    layer_bytes = DENSE_BYTES + D * EXPERT_BYTES
    layer_gbs = layer_bytes / (ms * 1e-3) / 1e9
    print(f"# T={T}: {ms * 1e3:.1f} us/layer (with an event per step: mean "
          f"{r['ms_ev'] * 1e3:.1f}, median {r['ms_median'] * 1e3:.1f}, min "
          f"{r['ms_min'] * 1e3:.1f}), D={D} touched experts, {nu} units, {layer_gbs:.0f} GB/s = "
          f"{100 * layer_gbs / HBM_PEAK_GBS:.1f}% of HBM; {r['warm_steps']} warm-up steps; "
          f"clocks {clk}", file=sys.stderr, flush=True)

    # the dominant kernel: the grouped FFN's gate/up pass (one launch of k_ffn_up_fast),
    # timed with HIP events on its launch stream and fed the layer's own codes, lists and
    # units; then the down pass and the whole grouped FFN the same way
    rows = torch.empty(T * 16, 3584, dtype=torch.bfloat16, device="cuda")
    fws = torch.zeros(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
    ffn_w = (d, dw["w13"], dw["s13"], dw["w2"], dw["s2"])
    lists = (v["pairs"], v["units_raw"], v["num_units"])

    def time_calls(call, n, floor_s=STAGE_FLOOR_S):
        warm(call, 3, floor_s)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        for i in range(n):
            call(i)
        f1.record(stream)
        torch.cuda.synchronize()
        return f0.elapsed_time(f1) / n * 1e3

    def stage(stages):
        return lambda *_: moe.moe_grouped_ffn_stages(*ffn_w, v["codes"], v["scales"], *lists, rows,
                                                     fws, stages, stream=stream)

    stage(moe.MOE_FFN_UP)()
    up_us = time_calls(stage(moe.MOE_FFN_UP), a.steps)
    down_us = time_calls(stage(moe.MOE_FFN_DOWN), a.steps)
    ffn_us = time_calls(stage(moe.MOE_FFN_UP | moe.MOE_FFN_DOWN), a.steps)
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
        "warmup_floor": {"seconds": WARM_FLOOR_S, "steps_run": r["warm_steps"],
                         "why": "untimed steps past --warmup until the GPU clocks are up"},
        "ms_per_step": ms,
        "ms_per_step_median": r["ms_median"],
        "ms_per_step_min": r["ms_min"],
        "per_step_spread": {"mean_ms": r["ms_ev"],
                            "why": "median and min come from a second run of the K steps with "
                                   "a timing event after every step; its mean, with those "
                                   "events in the stream, is this"},
        "host_enqueue_us_per_step": r["host_us"],
        "clocks": clk,
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
                           "frac": layer_gbs / HBM_PEAK_GBS,
                           "phase_bound_us": phase_bound_us(T, D),
                           "phase_frac": phase_bound_us(T, D) / (ms * 1e3),
                           # the pages' unit-window streaming (each touched expert once per
                           # window of up to 8 of its tokens): reported, not the denominator
                           "nominal_unit_window_bytes": DENSE_BYTES + nu * EXPERT_BYTES,
                           "nominal_unit_window_gbs": (DENSE_BYTES + nu * EXPERT_BYTES) / (ms * 1e-3) / 1e9,
                           # activations the step must move, kept out of the denominator
                           "activation_bytes": activation_bytes(T),
                           "activation_gbs": activation_bytes(T) / (ms * 1e-3) / 1e9},
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
    del rows, fws

    if not a.no_sweep:  # the batch sweep: every T, uniform and Zipf routing
        sweep = {}
        biases = {"uniform": dev(uniform_bias), "zipf": dev(zipf_bias)}  # (held while in use)
        for name in ("uniform", "zipf"):
            weights = lw_with(biases[name])
            for t in (1, 8, 32, 64, 65, 130, 255, 256, 510, 1020):
                # at least SWEEP_MIN_STEPS timed steps a point (a narrow batch's step time
                # varies from step to step: its shared expert and routed path take about as
                # long), a few ms of GPU time each
                st = run_T(t, max(a.steps, SWEEP_MIN_STEPS), 3, STAGE_FLOOR_S, weights)
                m, Dt = st["ms"], st["D"]
                bt = DENSE_BYTES + Dt * EXPERT_BYTES
                pb = phase_bound_us(t, Dt)
                sweep[f"{name}_T{t}"] = {
                    "tokens": t, "routing": name, "us": m * 1e3, "us_median": st["ms_median"] * 1e3,
                    "us_min": st["ms_min"] * 1e3, "tokens_per_s": t / (m * 1e-3), "D": Dt,
                    "units": st["units"], "weight_bytes": bt, "gbs": bt / (m * 1e-3) / 1e9,
                    "hbm_frac": bt / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "phase_bound_us": pb, "phase_frac": pb / (m * 1e3),
                    "host_enqueue_us": st["host_us"]}
                print(f"# sweep {name} T={t}: {m * 1e3:.1f} us, D={Dt}", file=sys.stderr, flush=True)
        res["sweep"] = sweep

    if not a.no_extras:
        res["finalize"] = bench_finalize(torch, moe, stream, time_calls, a.steps)
        print(f"# finalize {res['finalize']}", file=sys.stderr, flush=True)
        res["router_front"] = bench_router_front(torch, moe, syn, stream, time_calls, a.steps, dev)
        print(f"# router front {res['router_front']}", file=sys.stderr, flush=True)
        res["copy_probe"] = bench_copy(torch, stream, time_calls)
        ach = res["copy_probe"]["gbs_read_plus_write"]
        res["layer_roofline"]["achievable_gbs"] = ach
        res["layer_roofline"]["frac_of_achievable"] = layer_gbs / ach
    clocks.stop()

    if not a.no_cpu_baseline:
        import oracle as orc
        orc.lib()
        n = a.cpu_tokens
        sub = np.arange(n)
        dsub = dict(d0, T=n)
        c0 = time.time()
        orc.layer(dsub, w, x[sub])
        sec = time.time() - c0
        res["cpu_baseline"] = {"value": n / sec, "unit": "tokens/s", "cores": orc.threads(),
                               "kind": "oracle",
                               "sample": f"the oracle layer on the first {n} of the {T} tokens "
                                         f"(same weights and inputs), {sec:.1f} s"}
        res["cpu_baseline_single_thread"] = bench_oracle_single(orc, syn)
    if a.copy_probe:
        n = a.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_probe MiB
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n * 4
    print(json.dumps(res), flush=True)


def bench_finalize(torch, moe, stream, time_calls, steps):
    """Finalize alone at 256 tokens x top-16 x 3584 columns: run A (every slot valid) and
    run B (slot t mod 16 of token t invalid: id -1, weight 0, its row not read), each over
    ROTATE_SETS input sets so that no call finds its rows in the last-level cache."""
    T, K, C = 256, 16, 3584
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = [torch.randn(T * K, C, generator=g, device="cuda").to(torch.bfloat16)
            for _ in range(ROTATE_SETS)]
    wts = [torch.softmax(torch.randn(T, K, generator=g, device="cuda"), dim=1).contiguous()
           for _ in range(ROTATE_SETS)]
    outs = [torch.empty(T, C, dtype=torch.bfloat16, device="cuda") for _ in range(ROTATE_SETS)]
    ids = torch.arange(K, dtype=torch.int32, device="cuda").repeat(T, 1)
    t = torch.arange(T, device="cuda")
    ids[t, t % K] = -1
    wb = [w.clone() for w in wts]
    for w in wb:
        w[t, t % K] = 0.0
    res = {"tokens": T, "top_k": K, "cols": C, "input_sets": ROTATE_SETS}
    for run, wl, idl, nbytes in (("A", wts, None, T * K * C * 2 + T * K * 4 + T * C * 2),
                                 ("B", wb, ids, T * (K - 1) * C * 2 + T * K * 4 + T * C * 2)):
        def call(i=0, wl=wl, idl=idl):
            j = i % ROTATE_SETS
            moe.moe_finalize(rows[j], wl[j], outs[j], ids=idl, stream=stream)
        us = time_calls(call, max(steps, 20) * ROTATE_SETS)
        res[run] = {"us_per_call": us, "bytes_per_call": nbytes, "gbs": nbytes / us / 1e3,
                    "roofline_us": nbytes / (HBM_PEAK_GBS * 1e3),
                    "frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    return res


def bench_router_front(torch, moe, syn, stream, time_calls, steps, dev):
    """The routing front at 1020 tokens: router GEMM (x [1020, 7168] x W_gate [896, 7168],
    FP32 logits), sigmoid top-16 with the correction bias, lists and unit windows;
    uniform and Zipf routing bias; ROTATE_SETS sets of x and W_gate (275 MB).  W_gate is in
    the packed layout, as the layer's dense weights are (prepared once, ahead of the
    steps); the row-major W_gate's router time is reported beside it."""
    T, H, E = 1020, 7168, 896
    g = torch.Generator(device="cuda").manual_seed(3)
    xs = [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
          for _ in range(ROTATE_SETS)]
    wrm = [(torch.randn(E, H, generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
           for _ in range(ROTATE_SETS)]
    wgs = [moe.moe_pack_dense_weight(w) for w in wrm]
    d = moe.dims(T, T)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, 16, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, 16, dtype=torch.float32, device="cuda")
    rws = torch.empty(moe.moe_router_workspace_size(d), dtype=torch.uint8, device="cuda")
    lws = torch.empty(moe.moe_lists_workspace_size(d), dtype=torch.uint8, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pairs = torch.empty(T * 16, dtype=torch.int32, device="cuda")
    units = torch.empty((T * 16 + 7) // 8 + E, 4, dtype=torch.int32, device="cuda")
    nu = torch.empty(4, dtype=torch.int32, device="cuda")
    gemm_bytes = T * H * 2 + E * H * 2 + T * E * 4
    gemm_flops = 2 * T * E * H
    res = {"tokens": T, "experts": E, "input_sets": ROTATE_SETS,
           "router_gemm_roofline_us": {"hbm": gemm_bytes / (HBM_PEAK_GBS * 1e3),
                                       "bf16_mfma": gemm_flops / BF16_PEAK_FLOPS * 1e6}}
    for name, bias in (("uniform", syn.routing_bias(E, 0, False)), ("zipf", syn.routing_bias(E, 1, True))):
        b = dev(bias)

        def topk(i=0, b=b):
            j = i % ROTATE_SETS
            moe.moe_router_topk(d, xs[j], wgs[j], b, logits, ids, wts,
                                flags=moe.MOE_GATE_PACKED, workspace=rws, stream=stream)

        def topk_rm(i=0, b=b):
            j = i % ROTATE_SETS
            moe.moe_router_topk(d, xs[j], wrm[j], b, logits, ids, wts, workspace=rws,
                                stream=stream)

        def lists(i=0):
            moe.moe_build_lists(d, ids, counts, offsets, pairs, units, nu, lws, stream=stream)

        def both(i=0, b=b):
            topk(i, b)
            lists(i)
        t_topk_rm = time_calls(topk_rm, max(steps, 20) * ROTATE_SETS)
        t_topk = time_calls(topk, max(steps, 20) * ROTATE_SETS)
        t_lists = time_calls(lists, max(steps, 20) * ROTATE_SETS)
        t_both = time_calls(both, max(steps, 20) * ROTATE_SETS)
        torch.cuda.synchronize()
        res[name] = {"router_gemm_topk_us": t_topk, "router_gemm_topk_row_major_us": t_topk_rm,
                     "lists_us": t_lists, "front_us": t_both,
                     "touched_experts": int(torch.count_nonzero(counts).item()),
                     "units": int(nu[0].item())}
    return res


def activation_bytes(t, h=7168, l=3584, k=16, i=512, s=6144, e=896):
    """Activation bytes one step must move (split partials excluded: an artefact of the
    kernels): x read by the front and the shared gate/up GEMMs; FP32 logits written; the
    latent written in BF16 and MXFP8 and its codes read; the MXFP8 hidden written and read;
    the BF16 expert rows written and read; the routed and normed latent written and the
    normed one read; the shared activation written and read; the shared output written and
    read; the output written."""
    mx = lambda n: n * 33 // 32  # E4M3 codes + one E8M0 scale per 32
    return (2 * t * h * 2 + t * e * 4 + t * l * 2 + 2 * mx(t * l) + 2 * mx(t * k * i)
            + 2 * t * k * l * 2 + 3 * t * l * 2 + 2 * t * s * 2 + 2 * t * h * 2 + t * h * 2)


def bench_copy(torch, stream, time_calls):
    """A plain 1 GiB device-to-device copy (read + write): the achievable-bandwidth reference."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    us = time_calls(lambda *_: dst.copy_(src), 10)
    return {"bytes_read": n * 4, "bytes_written": n * 4, "us": us,
            "gbs_read_plus_write": 2 * n * 4 / us / 1e3}


def bench_oracle_single(orc, syn):
    """The oracle on one host thread: the toy layer (8 tokens, BF16 experts) and Finalize
    alone at 256 tokens x top-16 x 3584 columns."""
    d = dict(syn.TOY)
    w = syn.layer_weights(d, seed=0)
    x = syn.layer_input(d, seed=0)
    rows, wt, _ = syn.finalize_inputs()
    n0 = orc.threads()
    orc.set_threads(1)
    try:
        c0 = time.time()
        reps = 5
        for _ in range(reps):
            orc.layer(d, w, x)
        toy = (time.time() - c0) / reps
        c0 = time.time()
        orc.finalize(rows, wt)
        fin = time.time() - c0
    finally:
        orc.set_threads(n0)
    return {"cores": 1, "kind": "oracle",
            "toy_layer": {"value": d["T"] / toy, "unit": "tokens/s", "seconds_per_call": toy},
            "finalize": {"value": 256 / fin, "unit": "tokens/s", "seconds_per_call": fin}}


if __name__ == "__main__":
    main()
