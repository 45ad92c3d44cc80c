"""The pins must be sharp: plant one plausible mistake at a time in a copy of
the oracle's C source (a flipped tap offset, a dropped bias, an unflipped or
transposed weight, a dropped channel, a wrong padding bound, a short bias
gradient, a wrong activation value or slope), build it with
gcc into a temporary directory, and check that the
oracle pin suite fails against every mutant while it passes on the real
build.  Everything here runs on the CPU."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "conv3x3_oracle.c")
PIN_FILES = ["test_oracle_hand.py", "test_oracle_invariants.py", "test_oracle_adjoint.py",
             "test_oracle_fd.py", "test_oracle_torch.py", "test_oracle_act.py"]


def _func(src, name):
    """(start, end) of a static function's text in the source."""
    m = re.search(r"static double " + name + r"\(", src)
    assert m, name
    end = src.index("\n}\n", m.start()) + 3
    return m.start(), end


def _mutate(src, func, old, new):
    a, b = _func(src, func)
    body = src[a:b]
    assert old in body, (func, old)
    return src[:a] + body.replace(old, new, 1) + src[b:]


MUTANTS = {
    "fwd_flipped_taps": ("fwd_one", "int ih = h + r - 1;", "int ih = h - r + 1;"),
    "fwd_dropped_bias": ("fwd_one", "double acc = b ? b[k] : 0.0;", "double acc = 0.0;"),
    "fwd_dropped_channel": ("fwd_one", "c < C;", "c + 1 < C;"),
    "fwd_padding_bound": ("fwd_one", "iw >= W", "iw > W"),
    "fwd_weight_rs_swapped": ("fwd_one", "wt[IDX4(k, c, r, s, C, 3, 3)]", "wt[IDX4(k, c, s, r, C, 3, 3)]"),
    "bwd_data_unflipped": ("bwd_data_one", "int oh = h - r + 1;", "int oh = h + r - 1;"),
    "bwd_data_col_sign": ("bwd_data_one", "int ow = w - s + 1;", "int ow = w + s - 1;"),
    "bwd_weight_row_sign": ("bwd_weight_one", "int ih = h + r - 1;", "int ih = h - r + 1;"),
    "bwd_weight_roles_swapped": ("bwd_weight_one",
                                 "g[IDX4(n, k, h, w, K, H, W)] * x[IDX4(n, c, ih, iw, C, H, W)]",
                                 "g[IDX4(n, k, ih, iw, K, H, W)] * x[IDX4(n, c, h, w, C, H, W)]"),
    "bias_grad_short_row": ("bias_grad_one", "w < W;", "w + 1 < W;"),
    "silu_sigmoid_sign": ("act_value", "exp(-z)", "exp(z)"),
    "lrelu_value_slope": ("act_value", "0.2 * z", "0.02 * z"),
    "silu_slope_dropped_term": ("act_slope", "sg * (1.0 + z * (1.0 - sg))", "sg"),
    "lrelu_slope_sides_swapped": ("act_slope", "z > 0.0 ? 1.0 : 0.2", "z > 0.0 ? 0.2 : 1.0"),
}


def _run_pins(lib):
    env = dict(os.environ)
    if lib:
        env["CONV3X3_ORACLE_LIB"] = lib
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + \
          [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    func, old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    mutated = _mutate(src, func, old, new)
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(so), str(c), "-lm"])
    r = _run_pins(str(so))
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
