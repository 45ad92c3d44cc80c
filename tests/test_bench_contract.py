"""CPU checks of bench.py's contract and bookkeeping: the multi-GPU refusal,
the FLOP and algorithmic-byte formulas of the stem layer, and the scaling
of profiler byte counters into per-pass HBM traffic (which is reported only
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
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_bytes_are_scaled_by_the_copy_and_summed_per_pass(tmp_path, monkeypatch):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    copy = ("__amd_rocclr_copyBuffer", 1 << 20)
    wg = ("void conv3x3::wgrad_f32_kernel<64, 1, 1, true>(...)", 196608)
    red = ("conv3x3::wgrad_reduce4_kernel(...)", 74240)
    fw = ("void conv3x3::fwd_f32_kernel<0, 64, 4, 1, 64, 1, 8, true, 4>(...)", 131072)
    # the copy moves 512 MiB: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    _write_counters(fetch, "FETCH_SIZE", [(*copy, 262144), (*wg, 100), (*wg, 100), (*red, 40),
                                          (*fw, 10)])
    _write_counters(write, "WRITE_SIZE", [(*copy, 524288), (*wg, 50), (*wg, 50), (*red, 1),
                                          (*fw, 20)])
    out = tmp_path / "traffic.json"
    rec = bench.record_traffic(str(fetch), str(write), out_path=str(out))
    assert abs(rec["calibration"]["fetch_factor"] - 2.0) < 1e-12
    assert rec["calibration"]["write_factor"] == 1.0
    # both backward-weight kernels count toward the pass
    assert len(rec["passes"]["bwd_weight"]["kernels"]) == 2
    assert rec["passes"]["bwd_weight"]["hbm_bytes"] == ((100 + 40) * 2 + (50 + 1)) * 1024
    assert rec["passes"]["fwd"]["hbm_bytes"] == (10 * 2 + 20) * 1024
    assert rec["passes"]["bwd_data"]["hbm_bytes"] == 0

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.recorded_traffic("bwd_weight") == ((100 + 40) * 2 + (50 + 1)) * 1024
    # a record made for other kernel sources is not reported
    stale = json.loads(out.read_text())
    stale["source_digest"] = "0" * 64
    out.write_text(json.dumps(stale))
    assert bench.recorded_traffic("bwd_weight") is None
