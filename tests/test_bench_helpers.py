"""CPU checks of bench.py's bookkeeping (no GPU): the activation bytes it reports beside the
roofline, the committed HBM-traffic record it reads for the dominant kernel (present and
matching the kernel's current source), and its refusal of more than one GPU."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_activation_bytes_by_hand():
    b = load_bench()
    t, h, l, k, i, s, e = 256, 7168, 3584, 16, 512, 6144, 896
    x_reads = 2 * t * h * 2                  # front GEMM and shared gate/up GEMM
    logits = t * e * 4
    latent = t * l * 2 + 2 * (t * l + t * l // 32)         # BF16, then codes written + read
    hidden = 2 * (t * k * i + t * k * i // 32)             # written by gate/up, read by down
    rows = 2 * t * k * l * 2                               # written by down, read by Finalize
    norm = 3 * t * l * 2                                   # routed, normed written; normed read
    shared = 2 * t * s * 2 + 2 * t * h * 2                 # activation and output, each twice
    out = t * h * 2
    want = x_reads + logits + latent + hidden + rows + norm + shared + out
    assert b.activation_bytes(t) == want
    assert 90e6 < want < 110e6  # the ~0.1 GB the step moves besides weights at 256 tokens


def test_traffic_record_matches_kernel_source():
    b = load_bench()
    rec = b.recorded_traffic(256, False, False)
    assert rec is not None, "profiles/ traffic record missing or stale for the current ffn.hip"
    # HBM traffic of the gate/up pass within a few percent of its algorithmic bytes
    alg = 639 * b.UP_EXPERT_BYTES + 256 * 3584 * 33 // 32 + 256 * 16 * 512 * 33 // 32
    assert 1.0 <= rec / alg < 1.10
    assert b.recorded_traffic(255, False, False) is None
    assert b.recorded_traffic(256, True, False) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
