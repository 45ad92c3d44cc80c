"""Benchmark of the gfx950 conv3x3 path: forward + bias, backward-data and
backward-weight (+ bias gradient) of one UNet stem layer on one GPU.

One step = the whole path over one batch of seeded synthetic input already
resident in device memory: conv3x3_fwd, conv3x3_bwd_data, conv3x3_bwd_weight.
The workload is the UNet stem convolution at 64x64 image resolution
(N=32, C=64 -> K=64, H=W=64, float32); the diffusion UNet these layers come
from is trained on ImageNet 64x64 in the sources, and seeded N(0,1)
activations / gradients with Kaiming-uniform weights stand in for that data.

Prints ONE JSON line: throughput in TFLOP/s (2*N*H*W*C*K*9 per pass, three
passes per step), the roofline figure of the slowest kernel (timed with HIP
events on the stream the kernels run on) and the fp64 CPU oracle's
throughput on a bounded sample of the same layer (test infrastructure, timed
only as a reported baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--sweep OUT.json]
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv3x3 fwd+bwd TFLOP/s and % of MFMA/HBM roofline on 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv3x3_f32_unet_stem_32x64to64_64x64_traffic.json")
# Kernels launched by each pass of the stem layer (name prefixes in profiler output).
PASS_KERNELS = {"fwd": ["conv3x3::fwd_f32_kernel<0,"],
                "bwd_data": ["conv3x3::fwd_f32_kernel<1,"],
                "bwd_weight": ["conv3x3::wgrad_f32_kernel<", "conv3x3::wgrad_reduce"]}
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}   # dense MFMA peaks, MI355X
PEAK_HBM_GBS = 8000.0


def library_source_digest():
    """sha256 over the HIP library's sources: profiler byte counts recorded
    for one digest are reported only while the sources still match it."""
    import hashlib
    csrc = os.path.join(ROOT, "diffusion_unet_x3_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def record_traffic(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of `bench.py --copy-calibration-mb 512` into per-pass HBM bytes.  Each
    counter is scaled so that the 512 MiB device copy reads what it moved."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                name = r["Kernel_Name"].replace("void ", "")
                vals.setdefault((name, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    big = max((k for k in write if k[0].startswith("__amd_rocclr_copyBuffer")), key=lambda k: k[1])
    copy_kib = 512 * 1024
    f_factor = copy_kib / statistics.median(fetch[big])
    w_factor = copy_kib / statistics.median(write[big])
    kernels = {}
    for (name, grid), v in fetch.items():
        if name.startswith("conv3x3::"):
            kernels[name] = {"grid": grid, "fetch_kib": statistics.median(v),
                             "write_kib": statistics.median(write[(name, grid)])}
    passes = {}
    for p, prefixes in PASS_KERNELS.items():
        ks = [k for k in kernels if any(k.startswith(q) for q in prefixes)]
        passes[p] = {"kernels": ks, "hbm_bytes": sum(
            (kernels[k]["fetch_kib"] * f_factor + kernels[k]["write_kib"] * w_factor) * 1024
            for k in ks)}
    rec = {"source_digest": library_source_digest(),
           "calibration": {"copy_mib": 512, "fetch_kib_read": statistics.median(fetch[big]),
                           "write_kib_read": statistics.median(write[big]),
                           "fetch_factor": f_factor, "write_factor": w_factor},
           "kernels": kernels, "passes": passes}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def recorded_traffic(pass_name):
    """HBM bytes per launch of a pass, or None if not recorded for these sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != library_source_digest():
        return None
    b = rec.get("passes", {}).get(pass_name, {}).get("hbm_bytes")
    return int(b) if b else None


def flops_per_pass(N, C, K, H, W):
    return 2.0 * N * H * W * C * K * 9


ACT_CODES = {"none": 0, "silu": 1, "lrelu": 2}


def fused_backward(act, dtype):
    """The backward passes fuse the activation on float32 only."""
    return act != "none" and dtype == "f32"


def alg_bytes(pass_, N, C, K, H, W, dtype, act="none", prologue=False, out_bf16=False):
    """Each tensor crosses HBM once: inputs at their dtype, outputs float32.
    With a fused activation the forward also writes z and the fused backward
    passes also read it (float32, the output's shape).  With the input
    prologue every pass reads scale and shift ([N, C] float32) and
    backward-data also reads x.  out_bf16: y and dx are written as bf16."""
    s = 4 if dtype == "f32" else 2
    o = 2 if out_bf16 else 4
    M = N * H * W
    z = 4 * M * K
    pro = 8 * N * C if prologue else 0
    if pass_ == "fwd":
        return s * (M * C + 9 * K * C) + 4 * K + o * M * K + (z if act != "none" else 0) + pro
    extra = z if fused_backward(act, dtype) else 0
    if pass_ == "bwd_data":
        return s * (M * K + 9 * K * C) + o * M * C + extra + pro + (s * M * C if prologue else 0)
    return s * (M * C + M * K) + 4 * (9 * K * C + K) + extra + pro


class LayerRun:
    """Device buffers and the three pass launches of one layer.  act: the
    forward fuses the activation (and writes z), the float32 backward passes
    read z and fuse its derivative; the bfloat16 backward passes run on gy
    as is.  cat: a layer whose input is a skip concatenation (layer.cat > 0)
    runs the *_cat entry points on its two halves.  prologue: the *_gnsilu
    entry points (GroupNorm-apply + SiLU in the loader; float32)."""

    def __init__(self, layer, act="none", cat=False, prologue=False, out_bf16=False,
                 split=True):
        import torch
        import diffusion_unet_x3_amd as lib3
        import workloads as wl
        self.lib3, self.layer = lib3, layer
        dev = torch.device("cuda", 0)
        inp = wl.make_inputs(layer)
        self.x, self.w, self.g = (inp[k].to(dev) for k in ("x", "w", "g"))
        self.b = inp["b"].to(dev)
        N, C, K, H, W = layer.shape
        if out_bf16 and layer.dtype != "bf16":
            raise ValueError("bfloat16 outputs need a bfloat16 layer")
        od = torch.bfloat16 if out_bf16 else torch.float32
        self.y = torch.empty((N, K, H, W), device=dev, dtype=od)
        self.dx = torch.empty((N, C, H, W), device=dev, dtype=od)
        self.dw = torch.empty((K, C, 3, 3), device=dev)
        self.db = torch.empty((K,), device=dev)
        self.act = ACT_CODES[act]
        self.fused_bwd = fused_backward(act, layer.dtype)
        self.z = torch.empty((N, K, H, W), device=dev) if self.act else None
        code = lib3.CONV3X3_F32 if layer.dtype == "f32" else lib3.CONV3X3_BF16
        self.split = split
        self.C0 = layer.cat if cat else 0
        self.pro = prologue
        if prologue:
            if self.act or cat or layer.dtype != "f32":
                raise ValueError("the *_gnsilu entry points: float32, no other fusion")
            self.scale, self.shift = (v.to(dev) for v in wl.make_prologue(layer))
        if self.C0:
            if self.act:
                raise ValueError("the *_cat entry points take no activation")
            C0 = self.C0
            self.x0 = self.x[:, :C0].contiguous()
            self.x1 = self.x[:, C0:].contiguous()
            self.dx0 = torch.empty((N, C0, H, W), device=dev, dtype=od)
            self.dx1 = torch.empty((N, C - C0, H, W), device=dev, dtype=od)
            ws = lib3.conv3x3_bwd_weight_cat_workspace_size(N, C0, C - C0, K, H, W, code)
        else:
            ws = lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

    def concat_copy_ms(self, steps=10):
        """Average time of the copy that forms [x0 ; x1] as one tensor (what
        the *_cat entry points avoid), for comparison only."""
        import torch
        for _ in range(2):
            torch.cat([self.x0, self.x1], 1, out=self.x)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            torch.cat([self.x0, self.x1], 1, out=self.x)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def fwd(self):
        if self.pro:
            self.lib3.conv3x3_fwd_gnsilu(self.x, self.scale, self.shift, self.w, self.b,
                                         out=self.y)
        elif self.C0:
            self.lib3.conv3x3_fwd_cat(self.x0, self.x1, self.w, self.b, out=self.y)
        elif self.act:
            self.lib3.conv3x3_fwd_act(self.x, self.w, self.b, act=self.act, out=self.y, z=self.z)
        else:
            self.lib3.conv3x3_fwd(self.x, self.w, self.b, out=self.y, split=self.split)

    def bwd_data(self):
        if self.pro:
            self.lib3.conv3x3_bwd_data_gnsilu(self.g, self.w, self.x, self.scale, self.shift,
                                              out=self.dx)
        elif self.C0:
            self.lib3.conv3x3_bwd_data_cat(self.g, self.w, self.C0, out0=self.dx0,
                                           out1=self.dx1)
        elif self.fused_bwd:
            self.lib3.conv3x3_bwd_data_act(self.g, self.z, self.w, act=self.act, out=self.dx)
        else:
            self.lib3.conv3x3_bwd_data(self.g, self.w, out=self.dx, split=self.split)

    def bwd_weight(self):
        if self.pro:
            self.lib3.conv3x3_bwd_weight_gnsilu(self.x, self.scale, self.shift, self.g,
                                                dw=self.dw, db=self.db, workspace=self.ws)
        elif self.C0:
            self.lib3.conv3x3_bwd_weight_cat(self.x0, self.x1, self.g, dw=self.dw, db=self.db,
                                             workspace=self.ws)
        elif self.fused_bwd:
            self.lib3.conv3x3_bwd_weight_act(self.x, self.g, self.z, act=self.act, dw=self.dw,
                                             db=self.db, workspace=self.ws)
        else:
            self.lib3.conv3x3_bwd_weight(self.x, self.g, dw=self.dw, db=self.db,
                                         workspace=self.ws)

    def passes(self):
        return (("fwd", self.fwd), ("bwd_data", self.bwd_data), ("bwd_weight", self.bwd_weight))


class Up2Run:
    """The three passes of an upsample-then-convolve layer (conv3x3_*_up2):
    x at H x W, y and g at 2H x 2W."""

    def __init__(self, layer):
        import torch
        import diffusion_unet_x3_amd as lib3
        import workloads as wl
        from dataclasses import replace
        self.lib3 = lib3
        dev = torch.device("cuda", 0)
        N, C, K, H, W = layer.shape
        big = wl.make_inputs(replace(layer, H=2 * H, W=2 * W))
        self.x = big["x"][:, :, :H, :W].contiguous().to(dev)
        self.w, self.b, self.g = (big[k].to(dev) for k in ("w", "b", "g"))
        self.y = torch.empty((N, K, 2 * H, 2 * W), device=dev)
        self.dx = torch.empty((N, C, H, W), device=dev)
        self.dw = torch.empty((K, C, 3, 3), device=dev)
        self.db = torch.empty((K,), device=dev)
        self.ws_d = torch.empty(max(lib3.conv3x3_up2_workspace_size(1, N, C, K, H, W), 1),
                                dtype=torch.uint8, device=dev)
        self.ws_w = torch.empty(max(lib3.conv3x3_up2_workspace_size(2, N, C, K, H, W), 1),
                                dtype=torch.uint8, device=dev)

    def passes(self):
        return [("fwd", lambda: self.lib3.conv3x3_fwd_up2(self.x, self.w, self.b, out=self.y)),
                ("bwd_data", lambda: self.lib3.conv3x3_bwd_data_up2(self.g, self.w, out=self.dx,
                                                                    workspace=self.ws_d)),
                ("bwd_weight", lambda: self.lib3.conv3x3_bwd_weight_up2(
                    self.x, self.g, dw=self.dw, db=self.db, workspace=self.ws_w))]


class S2Run:
    """The three passes of a stride-2 layer (conv3x3_*_s2): x at H x W, y and
    g at H/2 x W/2."""

    def __init__(self, layer):
        import torch
        import diffusion_unet_x3_amd as lib3
        import workloads as wl
        self.lib3 = lib3
        dev = torch.device("cuda", 0)
        N, C, K, H, W = layer.shape
        inp = wl.make_inputs(layer)
        self.x, self.w, self.b = (inp[k].to(dev) for k in ("x", "w", "b"))
        self.g = inp["g"][:, :, :H // 2, :W // 2].contiguous().to(dev)
        self.y = torch.empty((N, K, H // 2, W // 2), device=dev)
        self.dx = torch.empty((N, C, H, W), device=dev)
        self.dw = torch.empty((K, C, 3, 3), device=dev)
        self.db = torch.empty((K,), device=dev)
        self.ws = torch.empty(max(lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W), 1),
                              dtype=torch.uint8, device=dev)

    def passes(self):
        return [("fwd", lambda: self.lib3.conv3x3_fwd_s2(self.x, self.w, self.b, out=self.y)),
                ("bwd_data", lambda: self.lib3.conv3x3_bwd_data_s2(self.g, self.w, out=self.dx)),
                ("bwd_weight", lambda: self.lib3.conv3x3_bwd_weight_s2(
                    self.x, self.g, dw=self.dw, db=self.db, workspace=self.ws))]


def time_layer(run, steps, warmup):
    """Per-pass average ms (events between the passes) and per-step ms."""
    import torch
    for _ in range(warmup):
        for _, f in run.passes():
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        ev[i][0].record()
        for j, (_, f) in enumerate(run.passes()):
            f()
            ev[i][j + 1].record()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    per = {}
    for j, (name, _) in enumerate(run.passes()):
        per[name] = sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
    return total_ms / steps, per


def cpu_baseline(layer, budget_s=15.0, min_s=10.0):
    """fp64 oracle on the layer's shape with the batch cut to fit the budget."""
    import oracle
    import workloads as wl
    from dataclasses import replace
    N, C, K, H, W = layer.shape
    probe = replace(layer, N=1)
    inp = wl.make_inputs(probe)
    t = time.perf_counter()
    oracle.conv3x3_fwd(inp["x"], inp["w"], inp["b"])
    t1 = time.perf_counter() - t
    n = int(max(1, min(N, budget_s / max(3 * t1, 1e-6))))
    sample = replace(layer, N=n)
    inp = wl.make_inputs(sample)
    x, w, b, g = (oracle._f64(inp[k]) for k in ("x", "w", "b", "g"))
    # When the whole batch takes less than the minimum, the three passes are
    # repeated until it is reached, so the figure rests on seconds of work.
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min_s and reps < 64):
        t = time.perf_counter()
        oracle.conv3x3_fwd(x, w, b)
        oracle.conv3x3_bwd_data(g, w)
        oracle.conv3x3_bwd_weight(x, g)
        dt += time.perf_counter() - t
        reps += 1
    fl = 3 * flops_per_pass(n, C, K, H, W) * reps
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"all three passes of the same layer at N={n} of {N} images, "
                      f"{reps} run(s) ({fl / 1e9:.1f} GFLOP fp64, {dt:.1f} s); "
                      f"cpu: {platform.processor() or platform.machine()}"}


def sweep(out_path, steps, warmup, match=None, act="none", cat=False, prologue=False,
          out_bf16=False, split=True, up2=False, s2=False):
    import re
    import torch
    import workloads as wl
    rows = []
    if up2 or s2:
        for layer in (wl.UPSAMPLE if up2 else wl.DOWNSAMPLE):
            run = Up2Run(layer) if up2 else S2Run(layer)
            ms, per = time_layer(run, steps, warmup)
            N, C, K, H, W = layer.shape
            # useful FLOPs: at the output's resolution
            f = flops_per_pass(N, C, K, 2 * H, 2 * W) if up2 else \
                flops_per_pass(N, C, K, H // 2, W // 2)
            row = {"layer": layer.name, "dtype": "f32", "up2": up2, "s2": s2,
                   "shape": [N, C, K, H, W], "ms_step": ms}
            for p, t in per.items():
                row[p] = {"ms": t, "tflops": f / (t * 1e-3) / 1e12}
            rows.append(row)
            print(f"{layer.name:44s} " + " ".join(f"{p}={row[p]['ms'] * 1e3:8.1f}us" for p in per),
                  file=sys.stderr, flush=True)
        with open(out_path, "w") as fh:
            json.dump(rows, fh, indent=1)
        return
    for cfg, layers in sorted(wl.CONFIGS.items()):
        for layer in layers:
            if match and not re.search(match, layer.name):
                continue
            if (cat and not layer.cat) or (prologue and layer.dtype != "f32") or \
                    (out_bf16 and layer.dtype != "bf16"):
                continue
            run = LayerRun(layer, act, cat, prologue, out_bf16, split)
            ms, per = time_layer(run, steps, warmup)
            N, C, K, H, W = layer.shape
            f = flops_per_pass(N, C, K, H, W)
            row = {"config": cfg, "layer": layer.name, "dtype": layer.dtype, "act": act,
                   "prologue": prologue, "out_bf16": out_bf16, "shape": [N, C, K, H, W],
                   "ms_step": ms}
            if cat:
                row["cat"] = layer.cat
                row["concat_copy_ms"] = run.concat_copy_ms()
            for p, t in per.items():
                tf = f / (t * 1e-3) / 1e12
                row[p] = {"ms": t, "tflops": tf, "mfma_frac": tf / PEAK_TFLOPS[layer.dtype],
                          "alg_gbs": alg_bytes(p, N, C, K, H, W, layer.dtype, act, prologue,
                                               out_bf16) / (t * 1e-3) / 1e9}
            rows.append(row)
            print(f"{layer.name:44s} " + " ".join(
                f"{p}={row[p]['ms'] * 1e3:8.1f}us {row[p]['tflops']:7.1f}TF" for p in per),
                file=sys.stderr, flush=True)
            del run
            torch.cuda.empty_cache()
    with open(out_path, "w") as fh:
        json.dump(rows, fh, indent=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", metavar="OUT_JSON", help="also time every configured layer")
    ap.add_argument("--sweep-match", metavar="REGEX", help="only sweep layers whose name matches")
    ap.add_argument("--act", choices=sorted(ACT_CODES), default="none",
                    help="time the fused-activation entry points (forward epilogue; "
                         "float32 backward prologue) instead of the plain ones")
    ap.add_argument("--cat", action="store_true",
                    help="with --sweep: time only the layers whose input is a skip "
                         "concatenation, through the *_cat entry points")
    ap.add_argument("--gnsilu", action="store_true",
                    help="with --sweep: time the float32 layers through the *_gnsilu entry "
                         "points (GroupNorm-apply + SiLU input prologue)")
    ap.add_argument("--out-bf16", action="store_true",
                    help="with --sweep: time the bfloat16 layers with y and dx written as "
                         "bfloat16 (CONV3X3_BF16_IO)")
    ap.add_argument("--no-split", action="store_true",
                    help="with --sweep: call the entry points without a workspace (no split "
                         "reduction on small bf16 images)")
    ap.add_argument("--up2", action="store_true",
                    help="with --sweep: time the UNet's upsample convolutions through the "
                         "*_up2 entry points (nearest 2x upsampling in the loader)")
    ap.add_argument("--s2", action="store_true",
                    help="with --sweep: time the UNet's stride-2 downsample convolutions "
                         "(*_s2 entry points)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc counter CSVs "
                         "(FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--copy-calibration-mb", type=int, default=0, metavar="MB",
                    help="also run a plain device-to-device copy of MB megabytes (a known "
                         "amount of HBM traffic for scaling profiler byte counters)")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic)["passes"]))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    layer = wl.CONFIGS[2][0]
    N, C, K, H, W = layer.shape
    run = LayerRun(layer, args.act)
    ms, per = time_layer(run, args.steps, args.warmup)
    f = flops_per_pass(N, C, K, H, W)
    value = 3 * f / (ms * 1e-3) / 1e12
    dom = max(per, key=per.get)
    achieved = f / (per[dom] * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": layer.dtype, "data": "synthetic",
        "config": {"workload": "unet_stem_conv3x3_fwd_bias+bwd_data+bwd_weight" if args.act == "none"
                   else f"unet_stem_conv3x3_fwd_bias_{args.act}+bwd_data+bwd_weight (fused {args.act})",
                   "N": N, "C_in": C, "C_out": K, "H": H, "W": W, "stride": 1, "pad": 1,
                   "layout": "NCHW", "seed": layer.seed, "global_batch": N,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "kernel": dom, "kernels": PASS_KERNELS[dom],
                     "achieved": round(achieved, 3),
                     "peak": PEAK_TFLOPS[layer.dtype], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS[layer.dtype], 4),
                     "traffic": recorded_traffic(dom) if args.act == "none" else None,
                     "alg_bytes": alg_bytes(dom, N, C, K, H, W, layer.dtype, args.act)},
        "passes": {p: {"us": round(t * 1e3, 2),
                       "tflops": round(f / (t * 1e-3) / 1e12, 2),
                       "alg_gbs": round(alg_bytes(p, N, C, K, H, W, layer.dtype, args.act) /
                                        (t * 1e-3) / 1e9, 1)} for p, t in per.items()},
    }
    del run
    torch.cuda.empty_cache()
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    if args.sweep:
        sweep(args.sweep, max(5, args.steps // 5), 3, args.sweep_match, args.act, args.cat,
              args.gnsilu, args.out_bf16, not args.no_split, args.up2, args.s2)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layer)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
