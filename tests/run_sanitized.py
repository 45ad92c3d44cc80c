"""The CPU test suite against host-sanitized builds of the fp64 oracle and
of the library's host code (AddressSanitizer + UndefinedBehaviorSanitizer,
any finding fatal).  Not collected by pytest; run it here, on the CPU:

    python tests/run_sanitized.py [extra pytest arguments]

It builds oracle/build.sh --sanitize and diffusion_unet_x3_amd/build.py
--sanitize into a scratch folder (the regular library objects must exist),
then runs `pytest -m "not gpu"` with clang's sanitizer runtime preloaded and
CONV3X3_ORACLE_LIB / CONV3X3_LIB pointing at those builds."""
import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main(args):
    out = os.environ.get("CONV3X3_SANITIZE_DIR") or tempfile.mkdtemp(prefix="conv3x3_sanitize_")
    os.makedirs(out, exist_ok=True)
    oracle_lib = os.path.join(out, "liboracle_conv3x3_sanitized.so")
    lib = os.path.join(out, "libconv3x3_sanitized.so")
    subprocess.check_call(["sh", os.path.join(ROOT, "oracle", "build.sh"), "--sanitize",
                           oracle_lib])
    subprocess.check_call([sys.executable, os.path.join(ROOT, "diffusion_unet_x3_amd", "build.py"),
                           "--sanitize", lib])
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang's AddressSanitizer runtime was not found")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt[-1], CONV3X3_LIB=lib, CONV3X3_ORACLE_LIB=oracle_lib,
               # the Python interpreter and torch are not instrumented: their
               # allocations at exit are not leaks of this code
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x",
           "-q", "-p", "no:cacheprovider"] + args
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
