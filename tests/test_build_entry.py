"""The build entry point must work on a checkout where the library is not
built yet: the package refuses to import without libconv3x3.so, so the build
script is loaded by path and must not pull the package in."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_module_loads_without_the_package():
    code = ("import sys, __graft_entry__ as g; m = g._build_module(); "
            "assert callable(m.build) and m.SOURCES; "
            "assert 'diffusion_unet_x3_amd' not in sys.modules, sorted(sys.modules)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr


def test_build_script_imports_only_the_standard_library():
    src = open(os.path.join(ROOT, "diffusion_unet_x3_amd", "build.py")).read()
    for line in src.splitlines():
        if line.startswith(("import ", "from ")):
            mod = line.split()[1].split(".")[0]
            assert mod in {"concurrent", "os", "subprocess", "sys", "shutil", "hashlib",
                           "tempfile"}, line
