"""Build libconv3x3.so (the HIP library) in-tree for gfx950.

Usage: python diffusion_unet_x3_amd/build.py   (or __graft_entry__.build()).
Every source is compiled with hipcc to an object next to the sources, in
parallel, then linked into diffusion_unet_x3_amd/libconv3x3.so.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libconv3x3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "planner.cpp", "noalloc.hip", "conv_fwd_f32.hip", "conv_fwd_bf16.hip",
           "conv_wgrad_f32.hip", "conv_wgrad_bf16.hip", "conv_stem.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-I", os.path.join(HERE, "..", "include")]
# Packed-FP32 VALU forms stay disabled for all device code.
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + \
          ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return out, "\n".join(noise)


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msg in results:
        if msg and verbose:
            print(msg, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


# Host-code sanitizer build, for the CPU tests only: the host parts of these
# sources (argument checks, planning, the entry points) are compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer, device code as usual
# (-Xarch_host keeps the sanitizers off the GPU code), every other object is
# the regular build's.  The library then needs the sanitizer runtime
# preloaded into the process.
SANITIZED = ["api.cpp", "planner.cpp", "noalloc.hip"]
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(out_lib):
    """Link a host-sanitized copy of the library at out_lib (the regular
    objects must exist: run build() first)."""
    objs = []
    for src in SOURCES:
        stem = os.path.splitext(src)[0]
        if src in SANITIZED:
            o = os.path.join(OBJ, "sanitized_" + stem + ".o")
            cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + SANITIZE + \
                  ["-c", os.path.join(CSRC, src), "-o", o]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        else:
            o = os.path.join(OBJ, stem + ".o")
            if not os.path.exists(o):
                raise RuntimeError(f"{o} is missing: run build() first")
        objs.append(o)
    subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", out_lib] + objs)
    return out_lib


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--sanitize":
        print(build_sanitized(sys.argv[2]))
    else:
        print(build())
