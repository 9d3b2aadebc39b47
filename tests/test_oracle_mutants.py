"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/gspn_oracle.c``, plants one mistake by a textual
edit, builds the copy with gcc into a temporary directory and runs the pin
checks against it.  Every mutant must fail at least one check; the unmodified
source must pass all of them.  Nothing here touches the GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from bruteforce import bruteforce_fwd

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "gspn_oracle.c")

MUTANTS = {
    "drop_input_term": [("double v = xl;", "double v = 0.0;")],
    "group_start_off_by_one": [("if (i % L == 0) {", "if (i % L == 1) {")],
    "mirrored_taps": [("const int64_t pp = p + t - 1;", "const int64_t pp = p - t + 1;")],
    "border_not_renormalised": [("        if (pp < 0 || pp >= m)\n                        continue;\n"
                                 "                    s[t] = sigmoid",
                                 "        s[t] = sigmoid")],
    "softmax_instead_of_sigmoid": [("s[t] = sigmoid(", "s[t] = exp(")],
    "bt_not_reversed": [("case DIR_BT: *r = H - 1 - i;", "case DIR_BT: *r = i;        ")],
    "rl_not_reversed": [("default:     *r = p;         *q = W - 1 - i;",
                         "default:     *r = p;         *q = i;")],
    "lr_axes_swapped": [("case DIR_LR: *r = p;         *q = i;",
                         "case DIR_LR: *r = i;         *q = p;")],
    "gate_not_applied": [("y[j] = u[j] * acc[j];", "y[j] = acc[j];")],
    "lambda_dropped": [("const double xl = lam[r * W + q] * x[r * W + q];",
                        "const double xl = x[r * W + q];")],
    "weight_set_modulo": [("k = c / cpw;", "k = c % Cw;")],
    "state_not_carried": [("h[p] = hn[p];", "(void)0;")],
    "no_normalisation": [("v += (s[t] / ssum) * h[pp];", "v += s[t] * h[pp];")],
    "weights_from_previous_line": [
        ("s[t] = sigmoid(wd[(int64_t)t * HW + r * W + q]);",
         "{ int64_t r0, q0; pixel_of(d, H, W, i - 1, p, &r0, &q0);"
         " s[t] = sigmoid(wd[(int64_t)t * HW + r0 * W + q0]); }")],
    "tap_index_swapped": [("s[t] = sigmoid(wd[(int64_t)t * HW", "s[t] = sigmoid(wd[(int64_t)(2 - t) * HW")],
}


def _build(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor for {name} not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(c), "-o", str(so),
                    "-lm"], check=True)
    return oracle.open_library(str(so))


def _pin_failures(lib):
    """Run the pins against one oracle build; return the names that fail."""
    failed = []
    rng = np.random.default_rng(1234)

    def run(x, w, lam, u, **kw):
        return oracle.scan_fwd(x, w, lam, u, lib=lib, **kw)

    def close(a, b, tol=1e-11):
        return a.shape == b.shape and np.all(np.isfinite(a)) and np.abs(a - b).max() <= tol * max(1, np.abs(b).max())

    # dense closed form: rectangular grid, all directions, groups, compact mode
    for (H, W, g, cpw) in [(5, 4, 1, 1), (6, 4, 2, 2)]:
        B, C = 2, 4
        x = rng.standard_normal((B, C, H, W))
        lam = rng.random((B, C, H, W))
        u = rng.random((B, C, H, W))
        w = rng.standard_normal((4, B, C // cpw, 3, H, W))
        if not close(run(x, w, lam, u, groups=g, cpw=cpw),
                     bruteforce_fwd(x, w, lam, u, groups=g, cpw=cpw, check=False)):
            failed.append(f"bruteforce{H}x{W}g{g}c{cpw}")
    # ones invariant
    H, W = 6, 5
    one = np.ones((1, 2, H, W))
    w = 2 * rng.standard_normal((4, 1, 2, 3, H, W))
    if not close(run(one, w, one, one), np.full(one.shape, (H + 1) + (W + 1.0))):
        failed.append("ones")
    # hand example
    x = np.array([1, 2, 3, 0, 0, 0.0]).reshape(1, 1, 2, 3)
    l3 = np.log(3.0)
    taps = np.array([[7, -7, 3, 1e3, 0, l3], [-40, 40, 9, 0, 0, -l3], [5, 5, -5, l3, 0, -1e3]])
    o = np.ones_like(x)
    if not close(run(x, taps.reshape(1, 1, 1, 3, 2, 3), o, o, dirs=1),
                 np.array([1, 2, 3, 1.6, 2, 2.25]).reshape(x.shape)):
        failed.append("hand")
    return failed


def test_unmodified_oracle_passes_every_pin(tmp_path):
    assert _pin_failures(_build(tmp_path, "original", [])) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failed = _pin_failures(_build(tmp_path, name, MUTANTS[name]))
    assert failed, f"mutant {name} passed every pin"
