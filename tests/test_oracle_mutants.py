"""Shows that the oracle's pins catch plausible mistakes.

Each case copies the oracle sources to a temporary directory, plants one
mistake by text substitution (a dropped term, a wrong sign, a wrong index or
range, a transposed operand), builds it with gcc, and runs a small battery of
the pins in a child process: the dense Golub-Kahan comparison, exact zeros
off the bidiagonal, and Frobenius invariance.  Every planted mistake must make
the battery fail (an abort from the bounds-checked accessor counts as caught).
The real oracle must pass the same battery.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BODY = "bb_oracle_body.h"

MUTANTS = {
    "dropped_head_term_right": ("REAL w = FMA(s, inv, p[0]);", "REAL w = s * inv;", 1),
    "tau_sign": ("*tau = (bt - alpha) / bt;", "*tau = (alpha - bt) / bt;", 1),
    "norm_drops_first_tail": ("for (int64_t j = 1; j < m; ++j) s = FMA(x[j], x[j], s);",
                              "for (int64_t j = 2; j < m; ++j) s = FMA(x[j], x[j], s);", 1),
    "left_range_drops_bulge": ("min64(c + t + b, n - 1)", "min64(c + b, n - 1)", 1),
    "right_rows_start": ("for (int64_t i = r + 1; i <= ch; ++i)", "for (int64_t i = r + 2; i <= ch; ++i)", 1),
    "row_index_of_chase": ("(k == 0) ? R : c - b;", "(k == 0) ? R : c - b + 1;", 1),
    "transposed_left_operand": ("s = FMA(x[i], p[i * st], s);", "s = FMA(x[i], p[i], s);", 1),
    "unscaled_update_vector": ("p[j] = FMA(-tw, v[j], p[j]);", "p[j] = FMA(-tw, x[j], p[j]);", 1),
    "last_sweep_skipped": ("for (int64_t R = 0; R + bp <= n - 2 && !stop; ++R)",
                           "for (int64_t R = 0; R + bp <= n - 3 && !stop; ++R)", 1),
    "threshold_instead_of_zero": ("if (s == 0) {", "if (s < (REAL)1e-3) {", 1),
    "left_update_wrong_vector": ("p[i * st] = FMA(-tw, v[i], p[i * st]);", "p[i * st] = FMA(tw, v[i], p[i * st]);", 1),
}

BATTERY = textwrap.dedent(r'''
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, sys.argv[2])
    sys.path.insert(0, sys.argv[2] + "/tests")
    import bb_inputs
    from refs import dense_from_band, dense_golub_kahan
    L = ctypes.CDLL(sys.argv[1])
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.bb_oracle_reduce_f64.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i64, ctypes.POINTER(i64)]
    L.bb_oracle_ld.restype = i64
    L.bb_oracle_ld.argtypes = [i64, i32, i32]
    L.bb_oracle_T.restype = i64
    L.bb_oracle_T.argtypes = [i64, i32, i32]
    def red(band, bw, tw):
        n = band.shape[0]
        ld = L.bb_oracle_ld(n, bw, tw)
        d = np.zeros(n); e = np.zeros(n - 1); w = np.zeros((n, ld))
        rc = L.bb_oracle_reduce_f64(band.ctypes.data, band.shape[1], n, bw, tw, d.ctypes.data,
                                    e.ctypes.data, w.ctypes.data, -1, None)
        assert rc == 0
        return d, e, w, L.bb_oracle_T(n, bw, tw)
    for (n, bw, tw) in [(40, 6, 2), (64, 16, 8), (33, 32, 16), (120, 16, 8)]:
        band = bb_inputs.make_band(n, bw, "f64", "normal", seed=3)
        A = dense_from_band(band, bw)
        d, e, w, T = red(band, bw, tw)
        fro = np.linalg.norm(A)
        dg, eg = dense_golub_kahan(A)
        assert np.all(np.isfinite(d)) and np.all(np.isfinite(e)), "non-finite"
        assert np.max(np.abs(np.abs(d) - np.abs(dg))) <= 1e-12 * fro, "d vs dense GK"
        assert np.max(np.abs(np.abs(e) - np.abs(eg))) <= 1e-12 * fro, "e vs dense GK"
        assert abs(np.sum(d * d) + np.sum(e * e) - fro * fro) <= 1e-13 * fro * fro, "Frobenius"
        off = [o for o in range(w.shape[1]) if o - T not in (0, 1)]
        assert np.all(w[:, off] == 0), "nonzero off the bidiagonal"
    print("BATTERY-PASSED")
''')


def _build_and_run(tmp_path, subst=None):
    src = tmp_path / "src"
    src.mkdir()
    for f in ("bb_oracle.c", BODY):
        shutil.copy(os.path.join(ROOT, "oracle", f), src / f)
    if subst:
        old, new, count = subst
        text = (src / BODY).read_text()
        assert text.count(old) >= count, "mutation site not found: " + old
        (src / BODY).write_text(text.replace(old, new, count))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-mfma",
                    "-fno-math-errno", "-o", str(lib), str(src / "bb_oracle.c"), "-lm"], check=True)
    script = tmp_path / "battery.py"
    script.write_text(BATTERY)
    r = subprocess.run([sys.executable, str(script), str(lib), ROOT], capture_output=True, text=True,
                       timeout=300)
    return r.returncode == 0 and "BATTERY-PASSED" in r.stdout


def test_real_oracle_passes_battery(tmp_path):
    assert _build_and_run(tmp_path)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert not _build_and_run(tmp_path, MUTANTS[name]), name
