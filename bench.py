"""Benchmark of the gfx950 conv3x3 path: forward + bias, backward-data and
backward-weight (+ bias gradient) over the 32 convolutions of one 64x64
diffusion-UNet training step, on one GPU.

One step = the whole path over one batch of seeded synthetic input already
resident in device memory: conv3x3_fwd, conv3x3_bwd_data and
conv3x3_bwd_weight of every stride-1 3x3 convolution of the UNet (N=32,
channel multipliers [1,2,3,4] on base 128 at 64/32/16/8 pixels, two convs
per residual block, two blocks per level, down and up paths, the up-path
inputs carrying the skip concatenation), float32; the same sweep in
bfloat16 (bf16 x, w, g; float32 accumulation and outputs) is reported in an
extra key.  The diffusion UNet these layers come from is trained on
ImageNet 64x64 in the sources; seeded N(0,1) activations / gradients with
Kaiming-uniform weights stand in for that data.

Prints ONE JSON line: throughput in TFLOP/s (2*N*H*W*C*K*9 per pass, three
passes per layer) over the step time -- each timed step one replay of a HIP
graph holding the step's kernels (`--eager`: launched from Python instead)
-- per-pass median / p10 / p90 times from HIP events around eager launches
on the stream the kernels run on, the roofline figure of the pass family
that takes the most time, and the fp64 CPU oracle's throughput on a sampled
subset of the same outputs (test infrastructure, timed only as a reported
baseline; its full-sweep time is extrapolated from the sample).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--workload unet_sweep|stem|small|mid|bottleneck|image_stem]
                    [--sweep OUT.json] [--cold] [--eager] [--detail OUT.json]
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv3x3_f32_unet_sweep_32layers_traffic.json")
PASSES = ("fwd", "bwd_data", "bwd_weight")
# The main kernel of each pass, by dtype (name prefixes in profiler output).
# A pass may add a second, fixed-order reduce kernel right after its main
# kernel on the same stream: split_reduce_kernel (split forward /
# backward-data) or wgrad_reduce*_kernel (backward-weight split-K); profile
# summaries count it toward the pass whose main kernel precedes it.
MAIN_KERNELS = {("f32", "fwd"): ("conv3x3::fwd_f32_kernel<0,",),
                ("f32", "bwd_data"): ("conv3x3::fwd_f32_kernel<1,",
                                      "conv3x3::bwd_data_stem_kernel<float,"),
                ("f32", "bwd_weight"): ("conv3x3::wgrad_f32_kernel<",
                                        "conv3x3::wgrad_stem_kernel<float,"),
                ("bf16", "fwd"): ("conv3x3::fwd_bf16_kernel<0,", "conv3x3::fwd_stem_bf16_kernel<"),
                ("bf16", "bwd_data"): ("conv3x3::fwd_bf16_kernel<1,",
                                       "conv3x3::bwd_data_stem_kernel<unsigned short,"),
                ("bf16", "bwd_weight"): ("conv3x3::wgrad_bf16_kernel<",
                                         "conv3x3::wgrad_stem_kernel<unsigned short,")}
REDUCE_KERNELS = ("conv3x3::split_reduce_kernel", "conv3x3::wgrad_reduce",
                  "conv3x3::stem_reduce_kernel")


def pass_kernels(dtype, pass_):
    """Name prefixes of the kernels one pass launches."""
    return list(MAIN_KERNELS[(dtype, pass_)]) + list(REDUCE_KERNELS)


PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}   # dense MFMA peaks, MI355X
PEAK_HBM_GBS = 8000.0


def _kernel_name(row):
    return row["Kernel_Name"].replace("void ", "")


def attribute_passes(rows):
    """Group profiler rows (dicts with Kernel_Name and Dispatch_Id) into
    pass launches: each main kernel starts a launch of its (dtype, pass), and
    a reduce kernel joins the launch of the main kernel dispatched before it.
    Returns a list of ((dtype, pass), [rows]) in dispatch order."""
    launches = []
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        name = _kernel_name(r)
        fam = next((k for k, pre in MAIN_KERNELS.items() if name.startswith(pre)), None)
        # (str.startswith takes the tuple of a family's prefixes)
        if fam is not None:
            launches.append((fam, [r]))
        elif name.startswith(REDUCE_KERNELS) and launches:
            launches[-1][1].append(r)
    return launches


def summarize_trace(trace_csv):
    """Per (dtype, pass): number of pass launches, total and average
    duration (ns, main kernel + its reduce), and per-kernel averages, from a
    rocprofv3 kernel-trace CSV."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(trace_csv)))
    out = {}
    for fam, rs in attribute_passes(rows):
        d = out.setdefault(f"{fam[0]}/{fam[1]}", {"launches": 0, "total_ns": 0, "kernels": {}})
        d["launches"] += 1
        for r in rs:
            dt = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            d["total_ns"] += dt
            d["kernels"].setdefault(_kernel_name(r).split("(")[0], []).append(dt)
    for d in out.values():
        d["avg_us_per_launch"] = d["total_ns"] / d["launches"] / 1e3
        d["kernels"] = {k: {"dispatches": len(v), "avg_us": statistics.mean(v) / 1e3}
                        for k, v in d["kernels"].items()}
    return out


def summarize_counters(csv_paths):
    """Per (dtype, pass): sums of every counter over all launches and the
    launch count, from rocprofv3 --pmc counter-collection CSVs (one row per
    dispatch and counter).  Derived: MFMA busy fraction =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * 4 SIMDs * 256 CUs), MFMA
    FLOPs = 512 * SQ_INSTS_VALU_MFMA_MOPS_*, LDS bank-conflict fraction =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    import csv
    rows = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            rows.setdefault(key, {"Dispatch_Id": r["Dispatch_Id"],
                                  "Kernel_Name": r["Kernel_Name"]})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
    out = {}
    for fam, rs in attribute_passes(list(rows.values())):
        d = out.setdefault(f"{fam[0]}/{fam[1]}", {"launches": 0})
        d["launches"] += 1
        for r in rs[:1]:  # main kernel only: the reduce has no MFMA work
            for k, v in r.items():
                if k not in ("Dispatch_Id", "Kernel_Name"):
                    d[k] = d.get(k, 0.0) + v
    for d in out.values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("GRBM_GUI_ACTIVE"):
            d["mfma_busy_frac"] = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] * 4 * 256)
        for dt in ("F32", "BF16"):
            if f"SQ_INSTS_VALU_MFMA_MOPS_{dt}" in d:
                d[f"mfma_flops_{dt.lower()}"] = 512.0 * d[f"SQ_INSTS_VALU_MFMA_MOPS_{dt}"]
        if d.get("SQ_LDS_IDX_ACTIVE"):
            d["lds_bank_conflict_frac"] = d.get("SQ_LDS_BANK_CONFLICT", 0.0) / d["SQ_LDS_IDX_ACTIVE"]
    return out


def _per_launch(rows_by_family, nlayers):
    """Split each family's launches (dispatch order) by layer: launch i of a
    family belongs to layer i mod nlayers (every step runs the layers in
    order)."""
    out = {}
    for fam, launches in rows_by_family.items():
        for i, rs in enumerate(launches):
            out.setdefault((fam, i % nlayers), []).append(rs)
    return out


def profile_report(trace_csv, counter_csvs, layers_by_dtype, title, commands, focus=()):
    """Markdown summary of one profiled bench run: per pass family, the
    trace's average time per launch (main kernel + its reduce) and, from
    the counter runs, MFMA busy fraction, MFMA FLOPs against the algorithmic
    count and the LDS bank-conflict fraction; then the same per layer for
    the layers whose names contain one of the `focus` strings.
    layers_by_dtype: dtype -> the layers of that dtype in timing order."""
    import csv
    trace = list(csv.DictReader(open(trace_csv)))
    fams = {}
    for fam, rs in attribute_passes(trace):
        fams.setdefault(fam, []).append(rs)
    ctr = {}
    if counter_csvs:
        rows = {}
        for path in counter_csvs:
            for r in csv.DictReader(open(path)):
                d = rows.setdefault(r["Dispatch_Id"], {"Dispatch_Id": r["Dispatch_Id"],
                                                       "Kernel_Name": r["Kernel_Name"],
                                                       "Start_Timestamp": r["Start_Timestamp"],
                                                       "End_Timestamp": r["End_Timestamp"]})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
        for fam, rs in attribute_passes(list(rows.values())):
            ctr.setdefault(fam, []).append(rs)
    order = sorted(fams, key=lambda f: (f[0] != "f32", PASSES.index(f[1])))

    def dur(rs):
        return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs) / 1e3

    def counters(launches):
        tot = {}
        for rs in launches:
            m = rs[0]  # the main kernel (the reduce has no MFMA work)
            for k in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                      "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
                tot[k] = tot.get(k, 0.0) + m.get(k, 0.0)
            tot["ns"] = tot.get("ns", 0.0) + int(m["End_Timestamp"]) - int(m["Start_Timestamp"])
        if not tot.get("GRBM_GUI_ACTIVE"):
            return None
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (8 x the clock per ns)
        busy = tot["SQ_VALU_MFMA_BUSY_CYCLES"] / (tot["GRBM_GUI_ACTIVE"] / 8 * 1024)
        flops = 512.0 * (tot["SQ_INSTS_VALU_MFMA_MOPS_F32"] + tot["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        lds = (tot["SQ_LDS_BANK_CONFLICT"] / tot["SQ_LDS_IDX_ACTIVE"]
               if tot["SQ_LDS_IDX_ACTIVE"] else 0.0)
        return busy, flops, lds, tot["GRBM_GUI_ACTIVE"] / tot["ns"]

    lines = [f"# {title}", "", "Commands (from /tmp with TMPDIR=/tmp; ROOT = the repository):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Per pass family over all its layers.  Time: kernel-trace duration per pass "
              "launch (main kernel + its reduce).  MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / "
              "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); GRBM_GUI_ACTIVE is reported summed over "
              "the 8 XCDs (the last column is that sum per ns).  MFMA FLOPs: 512 x "
              "SQ_INSTS_VALU_MFMA_MOPS_*, against 2*N*H*W*C*K*9 per layer.  LDS conflict: "
              "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
              "| pass family | launches | avg us / launch | TFLOP/s | of peak | MFMA busy | "
              "MFMA FLOPs / algorithmic | LDS conflict | GRBM cycles / ns |",
              "|---|---|---|---|---|---|---|---|---|"]
    for fam in order:
        layers = layers_by_dtype.get(fam[0], [])
        if not layers:
            continue
        n = len(layers)
        launches = fams[fam]
        t = sum(dur(rs) for rs in launches) / len(launches)
        gf = sum(flops_per_pass(*l.shape) for l in layers) / 1e9
        tf = gf / (t * n) * 1e3 if t else 0.0
        c = counters(ctr.get(fam, []))
        extra = ["-"] * 4 if c is None else [
            f"{c[0]:.3f}", f"{c[1] / (gf * 1e9 * len(ctr[fam]) / n):.4f}", f"{c[2]:.3f}",
            f"{c[3]:.2f}"]
        lines.append(f"| {fam[0]}/{fam[1]} | {len(launches)} ({len(launches) / n:g} per layer) "
                     f"| {t:.1f} | {tf:.1f} | {tf / PEAK_TFLOPS[fam[0]]:.3f} | "
                     + " | ".join(extra) + " |")
    lines += ["", "Kernels per family (dispatches, average us):", ""]
    for fam in order:
        ks = {}
        for rs in fams[fam]:
            for r in rs:
                ks.setdefault(_kernel_name(r).split("(")[0], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append(f"- {fam[0]}/{fam[1]}: " + "; ".join(
            f"`{k}` {len(v)}, {sum(v) / len(v):.1f}" for k, v in sorted(ks.items())))
    if focus:
        lines += ["", "Selected layers (trace average per launch; counters as above):", "",
                  "| layer | pass | avg us | TFLOP/s | of peak | MFMA busy | LDS conflict |",
                  "|---|---|---|---|---|---|---|"]
        for dt, layers in layers_by_dtype.items():
            n = len(layers)
            tl = _per_launch({f: v for f, v in fams.items() if f[0] == dt}, n)
            cl = _per_launch({f: v for f, v in ctr.items() if f[0] == dt}, n)
            for i, layer in enumerate(layers):
                if not any(k in layer.name for k in focus):
                    continue
                for fam in order:
                    if (fam, i) not in tl:
                        continue
                    ls = tl[(fam, i)]
                    t = sum(dur(rs) for rs in ls) / len(ls)
                    tf = flops_per_pass(*layer.shape) / (t * 1e-6) / 1e12
                    c = counters(cl.get((fam, i), []))
                    cc = "- | -" if c is None else f"{c[0]:.3f} | {c[2]:.3f}"
                    lines.append(f"| {layer.name} | {fam[1]} | {t:.1f} | {tf:.1f} | "
                                 f"{tf / PEAK_TFLOPS[fam[0]]:.3f} | {cc} |")
    return "\n".join(lines) + "\n"


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
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-calibration-mb 512` into HBM bytes per pass
    launch.  Each counter is scaled so that the 512 MiB device copy reads
    what it moved; a pass launch counts its main kernel and its reduce."""
    import csv
    import statistics

    def by_dispatch(path, counter):
        return {r["Dispatch_Id"]: r for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter}

    fetch, write = by_dispatch(fetch_csv, "FETCH_SIZE"), by_dispatch(write_csv, "WRITE_SIZE")

    def copy_kib(rows):
        big = [r for r in rows.values() if _kernel_name(r).startswith("__amd_rocclr_copyBuffer")]
        grid = max(int(r["Grid_Size"]) for r in big)
        return statistics.median(float(r["Counter_Value"]) for r in big
                                 if int(r["Grid_Size"]) == grid)

    copy_kib_moved = 512 * 1024
    f_factor = copy_kib_moved / copy_kib(fetch)
    w_factor = copy_kib_moved / copy_kib(write)
    passes = {}
    for fam, rs in attribute_passes(list(fetch.values())):
        d = passes.setdefault(f"{fam[0]}/{fam[1]}", {"launches": 0, "hbm_bytes_total": 0.0,
                                                      "kernels": set()})
        d["launches"] += 1
        for r in rs:
            w = write.get(r["Dispatch_Id"])
            wk = float(w["Counter_Value"]) if w is not None else 0.0
            d["hbm_bytes_total"] += (float(r["Counter_Value"]) * f_factor + wk * w_factor) * 1024
            d["kernels"].add(_kernel_name(r).split("(")[0])
    for d in passes.values():
        d["hbm_bytes"] = d["hbm_bytes_total"] / d["launches"]
        d["kernels"] = sorted(d["kernels"])
    rec = {"source_digest": library_source_digest(),
           "calibration": {"copy_mib": 512, "fetch_kib_read": copy_kib(fetch),
                           "write_kib_read": copy_kib(write),
                           "fetch_factor": f_factor, "write_factor": w_factor},
           "passes": passes}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def recorded_traffic(family, path=None):
    """HBM bytes per launch of a pass family ("f32/bwd_weight"), or None if
    not recorded for these kernel sources."""
    try:
        with open(path or TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != library_source_digest():
        return None
    b = rec.get("passes", {}).get(family, {}).get("hbm_bytes")
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
                 split=True, inputs=None):
        import torch
        import diffusion_unet_x3_amd as lib3
        import workloads as wl
        self.lib3, self.layer = lib3, layer
        dev = torch.device("cuda", 0)
        inp = inputs if inputs is not None else wl.make_inputs(layer)
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
            if self.act or cat:
                raise ValueError("the *_gnsilu entry points take no other fusion")
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
        # split forward / backward-data workspaces, allocated here and not in
        # the timed calls
        self.ws_f = self.ws_d = None
        if split:
            n_f = lib3.conv3x3_workspace_size(lib3.PASS_FWD, N, C, K, H, W, code)
            n_d = lib3.conv3x3_workspace_size(lib3.PASS_BWD_DATA, N, C, K, H, W, code)
            self.ws_f = torch.empty(max(n_f, 1), dtype=torch.uint8, device=dev)
            self.ws_d = torch.empty(max(n_d, 1), dtype=torch.uint8, device=dev)

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
            self.lib3.conv3x3_fwd(self.x, self.w, self.b, out=self.y, split=self.split,
                                  workspace=self.ws_f)

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
            self.lib3.conv3x3_bwd_data(self.g, self.w, out=self.dx, split=self.split,
                                       workspace=self.ws_d)

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
        code = lib3.CONV3X3_BF16 if layer.dtype == "bf16" else lib3.CONV3X3_F32
        self.ws_d = torch.empty(max(lib3.conv3x3_up2_workspace_size(1, N, C, K, H, W, code), 1),
                                dtype=torch.uint8, device=dev)
        self.ws_w = torch.empty(max(lib3.conv3x3_up2_workspace_size(2, N, C, K, H, W, code), 1),
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
        code = lib3.CONV3X3_BF16 if layer.dtype == "bf16" else lib3.CONV3X3_F32
        self.ws = torch.empty(max(lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code), 1),
                              dtype=torch.uint8, device=dev)

    def passes(self):
        return [("fwd", lambda: self.lib3.conv3x3_fwd_s2(self.x, self.w, self.b, out=self.y)),
                ("bwd_data", lambda: self.lib3.conv3x3_bwd_data_s2(self.g, self.w, out=self.dx)),
                ("bwd_weight", lambda: self.lib3.conv3x3_bwd_weight_s2(
                    self.x, self.g, dw=self.dw, db=self.db, workspace=self.ws))]


def _stats(v):
    """mean, median, p10, p90 of a list of times (ms)."""
    import statistics
    q = sorted(v)

    def pct(p):
        k = (len(q) - 1) * p
        lo = int(k)
        hi = min(lo + 1, len(q) - 1)
        return q[lo] + (q[hi] - q[lo]) * (k - lo)
    return {"mean": statistics.mean(q), "median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9)}


def time_runs(runs, steps, warmup, flush=None):
    """Time `steps` steps of every pass of every run, in order, with HIP
    events recorded between the passes on the current stream.  Returns the
    per-step ms (events around the whole step loop) and, per run, a dict
    pass -> list of per-step ms.  flush: a tensor overwritten before every
    pass, outside its event pair (cold caches); the step time then includes
    the flushes and only the pass times are meaningful."""
    import torch
    for _ in range(warmup):
        for run in runs:
            for _, f in run.passes():
                f()
    torch.cuda.synchronize()
    npass = sum(len(run.passes()) for run in runs)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(npass)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        j = 0
        for run in runs:
            for _, f in run.passes():
                if flush is not None:
                    flush.fill_(i + j)
                ev[i][j][0].record()
                f()
                ev[i][j][1].record()
                j += 1
    t1.record()
    torch.cuda.synchronize()
    per = []
    j = 0
    for run in runs:
        d = {}
        for name, _ in run.passes():
            d[name] = [ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)]
            j += 1
        per.append(d)
    return t0.elapsed_time(t1) / steps, per


def time_runs_graph(runs, steps, warmup):
    """Per-pass times as in time_runs (eager launches, an event pair around
    each pass), then the step time from one HIP graph holding the whole
    step (every pass of every run, captured once after the eager timing),
    replayed `steps` times between one event pair -- the same kernels on
    the same buffers, without the host's launch overhead between them.
    Every input, output and workspace is allocated before the capture.
    Returns (graph step ms, per-pass lists, eager step ms)."""
    import torch
    ms_eager, per = time_runs(runs, steps, warmup)
    step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step):
        for run in runs:
            for _, f in run.passes():
                f()
    for _ in range(max(warmup, 1)):
        step.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        step.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, per, ms_eager


def time_layer(run, steps, warmup):
    """Per-pass average ms and per-step ms of one run."""
    ms, per = time_runs([run], steps, warmup)
    return ms, {p: _stats(v)["mean"] for p, v in per[0].items()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _sample_idx(rng, shape, n):
    """n seeded flat indices into a tensor of `shape`, always including the
    first and last element."""
    import numpy as np
    total = int(np.prod(shape))
    n = max(2, min(n, total))
    idx = rng.choice(total, size=n - 2, replace=False) if total > n else np.arange(total)
    return np.unique(np.concatenate([idx, [0, total - 1]]))


def cpu_baseline_sampled(layers, inputs, budget_s=15.0):
    """fp64 oracle on a seeded sample of the outputs of every layer's three
    passes: y and dx elements (one output each, 18*C or 18*K FLOPs) and dw
    elements (2*N*H*W FLOPs), with the same padded-tap FLOP count as the
    GPU figure (only the oracle calls are timed).  Returns the
    rate in TFLOP/s and the full sweep's time extrapolated from it.  The
    sample grows until one run takes at least 60% of budget_s; only the
    last run is reported."""
    import numpy as np
    import oracle

    def run(scale):
        rng = np.random.default_rng(12345)
        dt, fl = 0.0, 0.0
        for layer in layers:
            inp = inputs[layer.name]
            x, w, b, g = (oracle._f64(inp[k]) for k in ("x", "w", "b", "g"))
            N, C, K, H, W = layer.shape
            n_out = max(2, int(scale * 4096))
            n_dw = max(2, int(scale * 64))
            iy = _sample_idx(rng, (N, K, H, W), n_out)
            ix = _sample_idx(rng, (N, C, H, W), n_out)
            iw = _sample_idx(rng, (K, C, 3, 3), n_dw)
            t = time.perf_counter()
            oracle.conv3x3_fwd_at(x, w, b, iy)
            oracle.conv3x3_bwd_data_at(g, w, ix)
            oracle.conv3x3_bwd_weight_at(x, g, iw)
            dt += time.perf_counter() - t
            fl += iy.size * 18.0 * C + ix.size * 18.0 * K + iw.size * 2.0 * N * H * W
        return dt, fl

    scale = 0.05
    for _ in range(4):
        dt, fl = run(scale)
        if dt >= 0.6 * budget_s or scale >= 1000.0:
            break
        scale = min(1000.0, scale * budget_s / max(dt, 1e-3))
    rate = fl / dt
    total = sum(3 * flops_per_pass(*layer.shape) for layer in layers)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"seeded sample of every layer's outputs, all {len(layers)} layers: "
                      f"{max(2, int(scale * 4096))} y and dx elements and "
                      f"{max(2, int(scale * 64))} dw elements per layer ({fl / 1e9:.1f} GFLOP "
                      f"fp64 in {dt:.1f} s); full sweep extrapolated to "
                      f"{total / rate / 3600:.2f} h at this rate; cpu: {cpu_model()}",
            "extrapolated_full_step_s": total / rate}


def cpu_baseline(layer, budget_s=15.0, min_s=10.0):
    """fp64 oracle on one layer's shape with the batch cut to fit the budget."""
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
                      f"cpu: {cpu_model()}"}


def measure_layers(layers, dtype, inputs, steps, warmup, flush=None, act="none", graph=False):
    """Time the three passes of every layer (one step = all of them, in
    order).  Returns (step ms, per-layer rows with per-pass statistics,
    per-pass totals, note).  act: the *_act entry points (fused
    activation).  graph: the step time from a HIP graph of the whole step
    (per-pass statistics stay eager); if the capture fails the eager step
    time is used and `note` says why."""
    import torch
    runs = [LayerRun(layer, act, inputs=inputs[layer.name]) for layer in layers]
    note = None
    if graph:
        try:
            ms, per, ms_eager = time_runs_graph(runs, steps, warmup)
            note = {"step": "hip_graph", "eager_ms_per_step": round(ms_eager, 4)}
        except Exception as e:  # noqa: BLE001 -- fall back to eager timing
            torch.cuda.synchronize()
            ms, per = time_runs(runs, steps, warmup, flush)
            note = {"step": "eager", "graph_capture_failed": f"{type(e).__name__}: {e}"[:200]}
    else:
        ms, per = time_runs(runs, steps, warmup, flush)
    del runs
    torch.cuda.empty_cache()
    rows, fam = [], {p: {"ms": 0.0, "gflop": 0.0, "alg_gb": 0.0} for p in PASSES}
    for layer, d in zip(layers, per):
        N, C, K, H, W = layer.shape
        f = flops_per_pass(N, C, K, H, W)
        row = {"layer": layer.name, "shape": [N, C, K, H, W]}
        for p, v in d.items():
            st = _stats(v)
            ab = alg_bytes(p, N, C, K, H, W, dtype, act)
            row[p] = {k: round(t * 1e3, 2) for k, t in st.items()}  # us
            row[p]["tflops"] = round(f / (st["median"] * 1e-3) / 1e12, 2)
            fam[p]["ms"] += st["mean"]
            fam[p]["gflop"] += f / 1e9
            fam[p]["alg_gb"] += ab / 1e9
        rows.append(row)
    return ms, rows, fam, note


def sweep_summary(dtype, layers, ms, fam, act="none"):
    """The throughput and roofline entries of one timed sweep."""
    total = sum(3 * flops_per_pass(*layer.shape) for layer in layers)
    dom = max(PASSES, key=lambda p: fam[p]["ms"])
    n = len(layers)
    # the binding roof of the family: MFMA unless its arithmetic intensity
    # (algorithmic FLOPs / bytes) is below the ridge peak / 8 TB/s
    hbm = fam[dom]["gflop"] / fam[dom]["alg_gb"] < PEAK_TFLOPS[dtype] * 1e3 / PEAK_HBM_GBS
    if hbm:
        achieved, peak, unit = fam[dom]["alg_gb"] / fam[dom]["ms"] * 1e3, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = fam[dom]["gflop"] / fam[dom]["ms"], PEAK_TFLOPS[dtype], "TFLOP/s"
    roof = {"bound": "hbm" if hbm else "mfma", "kernel": f"{dtype}/{dom}",
            "kernels": pass_kernels(dtype, dom),
            "launches_per_step": n,
            "flops_per_launch": fam[dom]["gflop"] * 1e9 / n,
            "avg_launch_us": fam[dom]["ms"] * 1e3 / n,
            "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": (recorded_traffic(f"{dtype}/{dom}")
                        if dtype == "f32" and act == "none" and len(layers) == 32 else None),
            "alg_bytes_per_launch": int(fam[dom]["alg_gb"] * 1e9 / n)}
    passes = {p: {"ms_per_step": round(fam[p]["ms"], 4),
                  "tflops": round(fam[p]["gflop"] / fam[p]["ms"], 2),
                  "mfma_frac": round(fam[p]["gflop"] / fam[p]["ms"] / PEAK_TFLOPS[dtype], 4),
                  "alg_gbs": round(fam[p]["alg_gb"] / fam[p]["ms"] * 1e3, 1)} for p in PASSES}
    return {"value": round(total / (ms * 1e-3) / 1e12, 3), "ms_per_step": round(ms, 4),
            "gflop_per_step": round(total / 1e9, 2), "roofline": roof, "passes": passes}


def sweep(out_path, steps, warmup, match=None, act="none", cat=False, prologue=False,
          out_bf16=False, split=True, up2=False, s2=False, geo_bf16=False):
    import re
    import torch
    import workloads as wl
    from dataclasses import replace
    rows = []
    if up2 or s2:
        for layer in (wl.UPSAMPLE if up2 else wl.DOWNSAMPLE):
            if geo_bf16:
                layer = replace(layer, dtype="bf16", name=layer.name.replace("_f32", "_bf16"))
            run = Up2Run(layer) if up2 else S2Run(layer)
            ms, per = time_layer(run, steps, warmup)
            N, C, K, H, W = layer.shape
            # useful FLOPs: at the output's resolution
            f = flops_per_pass(N, C, K, 2 * H, 2 * W) if up2 else \
                flops_per_pass(N, C, K, H // 2, W // 2)
            row = {"layer": layer.name, "dtype": layer.dtype, "up2": up2, "s2": s2,
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
            if (cat and not layer.cat) or (out_bf16 and layer.dtype != "bf16"):
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


WORKLOADS = {"unet_sweep": 5, "small": 1, "stem": 2, "mid": 3, "bottleneck": 4,
             "image_stem": 6}


def workload_layers(cfg):
    """(main layers, bfloat16 layers timed beside them or None) of a workload:
    the configured layer groups, or (6) the UNet's first convolution on the
    3-channel image in both dtypes."""
    import workloads as wl
    if cfg == 6:
        return [wl.IMAGE_STEM["f32"]], [wl.IMAGE_STEM["bf16"]]
    layers = [l for l in wl.CONFIGS[cfg] if l.dtype == "f32"] or list(wl.CONFIGS[cfg])
    extra = [l for l in wl.CONFIGS[5] if l.dtype == "bf16"] if cfg == 5 else None
    return layers, extra


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="unet_sweep",
                    help="unet_sweep: the 32 convolutions of a 64x64 UNet training step, "
                         "float32 (bfloat16 in an extra key); the others time one "
                         "configured layer group")
    ap.add_argument("--graph", action="store_true",
                    help="time each step as one HIP graph replay (the default; per-pass "
                         "times stay eager)")
    ap.add_argument("--eager", action="store_true",
                    help="time each step as eager launches from Python instead of a "
                         "HIP graph replay")
    ap.add_argument("--no-bf16", action="store_true",
                    help="unet_sweep: skip the bfloat16 sweep")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 512 MiB buffer before every pass (outside its event "
                         "pair), so each pass starts with cold caches; reported as "
                         "per-pass times")
    ap.add_argument("--detail", metavar="OUT_JSON",
                    help="write per-layer, per-pass time statistics to OUT_JSON")
    ap.add_argument("--sweep", metavar="OUT_JSON", help="also time every configured layer")
    ap.add_argument("--sweep-match", metavar="REGEX", help="only sweep layers whose name matches")
    ap.add_argument("--act", choices=sorted(ACT_CODES), default="none",
                    help="time the fused-activation entry points (forward epilogue; "
                         "backward prologue) instead of the plain ones")
    ap.add_argument("--cat", action="store_true",
                    help="with --sweep: time only the layers whose input is a skip "
                         "concatenation, through the *_cat entry points")
    ap.add_argument("--gnsilu", action="store_true",
                    help="with --sweep: time the layers through the *_gnsilu entry points "
                         "(GroupNorm-apply + SiLU input prologue)")
    ap.add_argument("--out-bf16", action="store_true",
                    help="with --sweep: time the bfloat16 layers with y and dx written as "
                         "bfloat16 (CONV3X3_BF16_IO)")
    ap.add_argument("--no-split", action="store_true",
                    help="with --sweep: call the entry points without a workspace (no split "
                         "reduction on small images)")
    ap.add_argument("--up2", action="store_true",
                    help="with --sweep: time the UNet's upsample convolutions through the "
                         "*_up2 entry points (nearest 2x upsampling in the loader)")
    ap.add_argument("--s2", action="store_true",
                    help="with --sweep: time the UNet's stride-2 downsample convolutions "
                         "(*_s2 entry points)")
    ap.add_argument("--geo-bf16", action="store_true",
                    help="with --up2 or --s2: bfloat16 inputs (the stride-1 bfloat16 kernels "
                         "over the full-resolution grid)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc counter CSVs "
                         "(FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-pass kernel times from a rocprofv3 kernel trace and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV",
                    help="print per-pass sums of rocprofv3 --pmc counters and exit")
    ap.add_argument("--profile-report", nargs="+", metavar="CSV",
                    help="KERNEL_TRACE_CSV [COUNTER_CSV ...]: print a markdown summary of a "
                         "profiled run of this workload (with --workload, --focus, "
                         "--commands) and exit")
    ap.add_argument("--focus", default="", help="with --profile-report: comma-separated layer "
                                                "names (substrings) to list one by one")
    ap.add_argument("--commands", nargs="*", default=[],
                    help="with --profile-report: the commands that made the CSVs")
    ap.add_argument("--copy-calibration-mb", type=int, default=0, metavar="MB",
                    help="also run a plain device-to-device copy of MB megabytes (a known "
                         "amount of HBM traffic for scaling profiler byte counters)")
    ap.add_argument("--traffic-out", metavar="JSON",
                    help="with --record-traffic: write the summary here instead of the "
                         "headline workload's record")
    args = ap.parse_args()
    if args.graph and (args.cold or args.eager):
        ap.error("--graph replays whole passes: no cache flush between them, and not "
                 "with --eager (drop --cold / --eager)")
    # a step is one HIP graph replay unless caches are flushed between passes
    # or eager launches are asked for
    args.graph = not (args.eager or args.cold)
    if args.record_traffic:
        out = args.traffic_out or TRAFFIC_FILE
        print(json.dumps(record_traffic(*args.record_traffic, out_path=out)["passes"]))
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return
    if args.profile_report:
        import workloads as wl
        cfg = WORKLOADS[args.workload]
        by_dt = {}
        main_l, extra_l = workload_layers(cfg)
        for l in main_l + ([] if args.no_bf16 else (extra_l or [])):
            by_dt.setdefault(l.dtype, []).append(l)
        print(profile_report(args.profile_report[0], args.profile_report[1:], by_dt,
                             f"conv3x3 {args.workload}: kernel times and counters",
                             args.commands, [k for k in args.focus.split(",") if k]), end="")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    cfg = WORKLOADS[args.workload]
    layers, extra_layers = workload_layers(cfg)
    dtype = layers[0].dtype
    t_gen = time.perf_counter()
    inputs = {l.name: wl.make_inputs(l) for l in layers}
    print(f"inputs drawn for {len(layers)} {dtype} layers in "
          f"{time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    flush = torch.empty(512 << 18, device="cuda") if args.cold else None
    ms, rows, fam, note = measure_layers(layers, dtype, inputs, args.steps, args.warmup,
                                         flush, args.act, args.graph)
    summ = sweep_summary(dtype, layers, ms, fam, args.act)
    if args.cold:
        # the step bracket holds the flushes too: the step is the passes' sum
        ms = sum(fam[p]["ms"] for p in PASSES)
        summ["value"] = round(sum(3 * flops_per_pass(*l.shape) for l in layers) /
                              (ms * 1e-3) / 1e12, 3)
        summ["ms_per_step"] = round(ms, 4)
    print(f"{dtype}: {summ['ms_per_step']} ms/step, {summ['value']} TFLOP/s",
          file=sys.stderr, flush=True)
    names = {5: "unet64_conv3x3_sweep_32layers_fwd_bias+bwd_data+bwd_weight",
             1: "single_conv3x3_2x64to64_32x32_fwd_bias+bwd_data+bwd_weight",
             2: "unet_stem_conv3x3_32x64to64_64x64_fwd_bias+bwd_data+bwd_weight",
             3: "unet_mid_resblock_convs_32x(128to256,256to256)_32x32_fwd_bias+bwd_data+bwd_weight",
             4: "unet_bottleneck_convs_64x512to512_(16x16,8x8)_fwd_bias+bwd_data+bwd_weight",
             6: "unet_image_stem_conv3x3_32x3to128_64x64_fwd_bias+bwd_data+bwd_weight"}
    wname = names[cfg] if args.act == "none" else names[cfg].replace(
        "fwd_bias", f"fwd_bias_{args.act}") + f" (fused {args.act})"
    config = {"workload": wname, "layers": len(layers), "N": layers[0].N,
              "layout": "NCHW", "stride": 1, "pad": 1, "seed": layers[0].seed,
              "global_batch": layers[0].N, "parallelism": "single_gpu",
              "timing": "HIP events on the kernels' stream; inputs resident in HBM; "
                        + ("512 MiB overwritten before every pass (cold caches)"
                           if args.cold else "passes back to back in sweep order")
                        + ("; each timed step is one replay of a HIP graph holding the "
                           "step's kernels (per-pass times: eager launches, an event "
                           "pair each)" if args.graph else "; eager launches")}
    if cfg == 6:
        config["shapes"] = [list(l.shape) for l in layers]
    elif cfg == 5:
        config.update({"channels": "128x[1,2,3,4]", "resolutions": [64, 32, 16, 8],
                       "convs": "2 per resblock, 2 resblocks per level, down and up paths; "
                                "up-path C_in includes the skip concatenation"})
    else:
        config["shapes"] = [list(l.shape) for l in layers]
    result = {
        "metric": METRIC, "value": summ["value"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": summ["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32" if dtype == "f32" else "bf16", "data": "synthetic",
        "config": config, "roofline": summ["roofline"], "passes": summ["passes"],
    }
    if note:
        result["step_timing"] = note
    detail = {dtype: rows}
    if extra_layers and not args.no_bf16:
        blayers = extra_layers
        by_idx = {l.index: l for l in layers}
        binputs = {}
        for l in blayers:
            src = inputs[by_idx[l.index].name]  # the same draws, rounded to bfloat16
            binputs[l.name] = {"x": src["x"].bfloat16(), "w": src["w"].bfloat16(),
                               "b": src["b"], "g": src["g"].bfloat16()}
        bms, brows, bfam, bnote = measure_layers(blayers, "bf16", binputs, args.steps,
                                                 args.warmup, flush, args.act, args.graph)
        bsum = sweep_summary("bf16", blayers, bms, bfam, args.act)
        if bnote:
            bsum["step_timing"] = bnote
        if args.cold:
            bms = sum(bfam[p]["ms"] for p in PASSES)
            bsum["value"] = round(sum(3 * flops_per_pass(*l.shape) for l in blayers) /
                                  (bms * 1e-3) / 1e12, 3)
            bsum["ms_per_step"] = round(bms, 4)
        print(f"bf16: {bsum['ms_per_step']} ms/step, {bsum['value']} TFLOP/s",
              file=sys.stderr, flush=True)
        bsum["dtype"] = "bf16 inputs, fp32 accumulation and outputs"
        result["bf16_sweep" if cfg == 5 else "bf16"] = bsum
        detail["bf16"] = brows
        del binputs
    if args.detail:
        with open(args.detail, "w") as fh:
            json.dump(detail, fh, indent=1)
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
        sweep(args.sweep, max(5, args.steps // 4), 3, args.sweep_match, args.act, args.cat,
              args.gnsilu, args.out_bf16, not args.no_split, args.up2, args.s2, args.geo_bf16)
    if not args.no_cpu_baseline:
        if cfg == 5:
            result["cpu_baseline"] = cpu_baseline_sampled(layers, inputs)
        else:
            result["cpu_baseline"] = cpu_baseline(layers[0])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
