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

# Mistakes planted in the backward pass; the forward pins above cannot see them.
BWD_MUTANTS = {
    "bwd_no_carry": [("g[pp] += wt[t] * gn[pq];", "(void)gn;")],
    "bwd_carry_not_transposed": [("g[pp] += wt[t] * gn[pq];", "g[pq] += wt[t] * gn[pp];")],
    "bwd_carry_across_groups": [("if (i + 1 < n && (i + 1) % L != 0) {", "if (i + 1 < n) {")],
    "bwd_carry_uses_own_line_weights": [("line_taps(wd, d, H, W, i + 1, pq, m, wt, st);",
                                         "line_taps(wd, d, H, W, i, pq, m, wt, st);")],
    "bwd_no_normalise_coupling": [("(*gp[t] - dot)", "(*gp[t])")],
    "bwd_no_sigmoid_slope": [("st[t] * (1.0 - st[t]) / ssum", "st[t] / ssum")],
    "bwd_gx_uses_x": [("gx[c * HW + j] = lc[j] * G[j];", "gx[c * HW + j] = xc[j] * G[j];")],
    "bwd_gu_last_direction_only": [("S[r * W + q] += v;", "S[r * W + q] = v;")],
    "bwd_tap_grad_uses_current_line": [("g[p] * hist[(i - 1) * m + pp]", "g[p] * hist[i * m + pp]")],
    "bwd_gate_not_applied": [("g[p] = gyc[r * W + q] * uc[r * W + q];", "g[p] = gyc[r * W + q];")],
    "bwd_tap_grad_not_summed_over_channels": [
        ("gwd[(int64_t)t * HW + r * W + q] += g[p]", "gwd[(int64_t)t * HW + r * W + q] = g[p]")],
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


def _bwd_pin_failures(lib):
    """Backward pins: directional derivatives of the dense closed form, the
    exact linear identities for x / lambda / u, zero tap gradient on ones."""
    failed = []
    rng = np.random.default_rng(4321)

    def loss(x, w, lam, u, gy, **kw):
        return float((bruteforce_fwd(x, w, lam, u, check=False, **kw) * gy).sum())

    for (H, W, g, cpw) in [(5, 4, 1, 1), (6, 4, 2, 2)]:
        B, C = 1, 4
        kw = dict(groups=g, cpw=cpw)
        x = rng.standard_normal((B, C, H, W))
        lam = rng.random((B, C, H, W))
        u = rng.random((B, C, H, W))
        gy = rng.standard_normal((B, C, H, W))
        w = rng.standard_normal((4, B, C // cpw, 3, H, W))
        gx, gw, glam, gu = oracle.scan_bwd(x, w, lam, u, gy, lib=lib, **kw)
        if not all(np.all(np.isfinite(a)) for a in (gx, gw, glam, gu)):
            failed.append(f"finite{H}x{W}")
            continue
        v = rng.standard_normal(w.shape)
        eps = 1e-5
        fd = (loss(x, w + eps * v, lam, u, gy, **kw) - loss(x, w - eps * v, lam, u, gy, **kw)) / (2 * eps)
        if abs(float((gw * v).sum()) - fd) > 1e-7 * max(1.0, abs(fd)):
            failed.append(f"tap_fd{H}x{W}g{g}c{cpw}")
        v = rng.standard_normal(x.shape)
        for name, got, args in (("x", gx, (v, w, lam, u)), ("lam", glam, (x, w, v, u)),
                                ("u", gu, (x, w, lam, v))):
            want = loss(*args, gy, **kw)
            if abs(float((got * v).sum()) - want) > 1e-10 * max(1.0, abs(want)):
                failed.append(f"linear_{name}{H}x{W}g{g}c{cpw}")
    one = np.ones((1, 2, 6, 5))
    gw = oracle.scan_bwd(one, 2 * rng.standard_normal((4, 1, 2, 3, 6, 5)), one, one,
                         rng.standard_normal(one.shape), lib=lib)[1]
    if np.abs(gw).max() > 1e-11:
        failed.append("ones_zero_tap_grad")
    return failed


def test_unmodified_oracle_passes_every_pin(tmp_path):
    lib = _build(tmp_path, "original", [])
    assert _pin_failures(lib) == []
    assert _bwd_pin_failures(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failed = _pin_failures(_build(tmp_path, name, MUTANTS[name]))
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(tmp_path, name):
    failed = _bwd_pin_failures(_build(tmp_path, name, BWD_MUTANTS[name]))
    assert failed, f"mutant {name} passed every backward pin"
