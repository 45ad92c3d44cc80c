"""CPU checks of bench.py's contract and bookkeeping: the multi-GPU refusal,
the FLOP and algorithmic-byte formulas, the attribution of reduce kernels
to the pass that launched them in profiler output, and the scaling of
profiler byte counters into per-pass HBM traffic (which is reported only
while the kernel sources match the digest it was recorded for)."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_graph_replay_refuses_cold_caches():
    """--graph replays whole passes, so there is no point between them to
    flush the caches: the combination is refused before anything runs."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--graph", "--cold"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--graph" in r.stderr and "--cold" in r.stderr
    assert r.stdout.strip() == ""


def test_stem_layer_flops_and_algorithmic_bytes():
    N, C, K, H, W = 32, 64, 64, 64, 64
    assert bench.flops_per_pass(N, C, K, H, W) == 2 * 32 * 4096 * 64 * 64 * 9
    M = N * H * W
    # fwd: x and w in, bias in, y out (fp32 everywhere on this layer)
    assert bench.alg_bytes("fwd", N, C, K, H, W, "f32") == 4 * (M * C + 9 * K * C) + 4 * K + 4 * M * K
    assert bench.alg_bytes("bwd_data", N, C, K, H, W, "f32") == 4 * (M * K + 9 * K * C) + 4 * M * C
    assert bench.alg_bytes("bwd_weight", N, C, K, H, W, "f32") == 4 * (M * C + M * K) + 4 * (9 * K * C + K)
    # bf16 inputs halve the input bytes, outputs stay fp32
    assert bench.alg_bytes("fwd", N, C, K, H, W, "bf16") == 2 * (M * C + 9 * K * C) + 4 * K + 4 * M * K


def test_fused_activation_bytes():
    N, C, K, H, W = 32, 64, 64, 64, 64
    M = N * H * W
    z = 4 * M * K
    for p in ("fwd", "bwd_data", "bwd_weight"):
        plain = bench.alg_bytes(p, N, C, K, H, W, "f32")
        assert bench.alg_bytes(p, N, C, K, H, W, "f32", "silu") == plain + z
    # bf16: the forward writes z; the backward passes run unfused
    assert bench.alg_bytes("fwd", N, C, K, H, W, "bf16", "silu") == \
        bench.alg_bytes("fwd", N, C, K, H, W, "bf16") + z
    assert bench.alg_bytes("bwd_data", N, C, K, H, W, "bf16", "silu") == \
        bench.alg_bytes("bwd_data", N, C, K, H, W, "bf16")


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid,
                        "Counter_Name": counter, "Counter_Value": value})


COPY = ("__amd_rocclr_copyBuffer", 1 << 20)
WG = ("void conv3x3::wgrad_f32_kernel<64, 1, 1, true>(...)", 196608)
RED = ("conv3x3::wgrad_reduce4_kernel(...)", 74240)
FW = ("void conv3x3::fwd_f32_kernel<0, 64, 4, 1, 64, 1, 8, true, 4>(...)", 131072)
SPL = ("void conv3x3::split_reduce_kernel(...)", 4096)
BD = ("void conv3x3::fwd_f32_kernel<1, 64, 4, 1, 64, 1, 8, true, 4>(...)", 131072)


def test_counter_bytes_are_scaled_by_the_copy_and_summed_per_pass(tmp_path, monkeypatch):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # dispatch order: copy, fwd, bwd_data + its split reduce, two backward-weight
    # launches each with its reduce
    order = [COPY, FW, BD, SPL, WG, RED, WG, RED]
    # the copy moves 512 MiB: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    fv = [262144, 10, 30, 4, 100, 40, 100, 40]
    wv = [524288, 20, 25, 3, 50, 1, 50, 1]
    _write_counters(fetch, "FETCH_SIZE", [(*k, v) for k, v in zip(order, fv)])
    _write_counters(write, "WRITE_SIZE", [(*k, v) for k, v in zip(order, wv)])
    out = tmp_path / "traffic.json"
    rec = bench.record_traffic(str(fetch), str(write), out_path=str(out))
    assert abs(rec["calibration"]["fetch_factor"] - 2.0) < 1e-12
    assert rec["calibration"]["write_factor"] == 1.0
    p = rec["passes"]
    # each backward-weight launch counts its reduce; bytes are per launch
    assert p["f32/bwd_weight"]["launches"] == 2
    assert len(p["f32/bwd_weight"]["kernels"]) == 2
    assert p["f32/bwd_weight"]["hbm_bytes"] == ((100 + 40) * 2 + (50 + 1)) * 1024
    assert p["f32/fwd"]["hbm_bytes"] == (10 * 2 + 20) * 1024
    # the split reduce after the backward-data kernel belongs to backward-data
    assert p["f32/bwd_data"]["hbm_bytes"] == ((30 + 4) * 2 + (25 + 3)) * 1024

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.recorded_traffic("f32/bwd_weight") == ((100 + 40) * 2 + (50 + 1)) * 1024
    # a record made for other kernel sources is not reported
    stale = json.loads(out.read_text())
    stale["source_digest"] = "0" * 64
    out.write_text(json.dumps(stale))
    assert bench.recorded_traffic("f32/bwd_weight") is None


def test_trace_summary_attributes_reduces_to_their_pass(tmp_path):
    path = tmp_path / "trace.csv"
    rows = [(COPY, 0, 5000), (FW, 10000, 110000), (BD, 120000, 200000), (SPL, 200500, 210500),
            (WG, 220000, 320000), (RED, 320500, 328500), (FW, 330000, 420000)]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        for i, ((name, _), t0, t1) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": t0,
                        "End_Timestamp": t1})
    s = bench.summarize_trace(str(path))
    assert s["f32/fwd"]["launches"] == 2
    assert s["f32/fwd"]["avg_us_per_launch"] == (100.0 + 90.0) / 2
    assert s["f32/bwd_data"]["avg_us_per_launch"] == 80.0 + 10.0
    assert s["f32/bwd_weight"]["avg_us_per_launch"] == 100.0 + 8.0
    assert "__amd_rocclr_copyBuffer" not in json.dumps(s)


def test_stats_percentiles():
    st = bench._stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert st["median"] == 3.0 and st["mean"] == 3.0
    assert abs(st["p10"] - 1.4) < 1e-12 and abs(st["p90"] - 4.6) < 1e-12


def test_unet_sweep_flops():
    import workloads as wl
    layers = [l for l in wl.CONFIGS[5] if l.dtype == "f32"]
    assert len(layers) == 32
    total = sum(3 * bench.flops_per_pass(*l.shape) for l in layers)
    assert abs(total / 1e9 - 3370.2) < 0.1
