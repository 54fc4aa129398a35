"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a dropped decay, a wrong
sign, a dropped beta, the wrong key-head map, a transposed state read, a norm without
epsilon or with a sum instead of a mean, a SiLU-style gate, a truncating FP16 encoder; in
the step before the recurrence, reversed conv taps or history rows, a missing q scale, k
normalised by q's norm, a wrong-signed SiLU, a positive gate, a stale history out),
builds it with the oracle's own compiler line, and runs the pins against it in a fresh
process through ``ORACLE_LIB_OVERRIDE``: at least one pin must fail.  The oracle under
test is never modified; the copies live in a temporary directory.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

# (the stored regression record of tests/golden is left out of every group: it would catch
# any change, and the point here is that the independent pins do)
RECURRENCE_PINS = "not dense_form_full and not norm and not f16 and not pre and not stored"
NORM_PINS = "(norm or f16) and not pre"
PRE_PINS = "pre"

# name: (exact text in the oracle, planted replacement, pins expected to catch it)
MUTANTS = {
    "kv_sum_without_decay": ("kv[j] = bt * (vt[j] - a * kv[j]);",
                             "kv[j] = bt * (vt[j] - kv[j]);", RECURRENCE_PINS),
    "update_wrong_sign": ("Si[j] = a * Si[j] + ki * kv[j];",
                          "Si[j] = a * Si[j] - ki * kv[j];", RECURRENCE_PINS),
    "update_without_decay": ("Si[j] = a * Si[j] + ki * kv[j];",
                             "Si[j] = Si[j] + ki * kv[j];", RECURRENCE_PINS),
    "key_head_by_division": ("const int kh = h % n_k_heads;",
                             "const int kh = h / (n_v_heads / n_k_heads);", RECURRENCE_PINS),
    "beta_dropped": ("kv[j] = bt * (vt[j] - a * kv[j]);",
                     "kv[j] = (vt[j] - a * kv[j]);", RECURRENCE_PINS),
    "state_read_transposed": ("for (int j = 0; j < dv; ++j) kv[j] += Si[j] * ki;",
                              "for (int j = 0; j < dv; ++j) kv[j] += S[(size_t)j * dv + i] * ki;",
                              RECURRENCE_PINS),
    "norm_without_eps": ("sqrt(ss / dv + eps)", "sqrt(ss / dv)", NORM_PINS),
    "norm_sum_not_mean": ("sqrt(ss / dv + eps)", "sqrt(ss + eps)", NORM_PINS),
    "norm_silu_gate": ("const double val = orow[j] * rs * wrow[j] * gate;",
                       "const double val = orow[j] * rs * wrow[j] * gate * zrow[j];", NORM_PINS),
    "f16_truncating": ("if (rem > halfway || (rem == halfway && (qv & 1))) ++qv;",
                       "if (0) ++qv;", NORM_PINS),
    "pre_taps_reversed": ("s += (double)w[c * 4 + j] * xv;",
                          "s += (double)w[c * 4 + 3 - j] * xv;", PRE_PINS),
    "pre_history_rows_reversed": ("const double xv = r < 3 ? (double)hist_in[r * C + c]",
                                  "const double xv = r < 3 ? (double)hist_in[(2 - r) * C + c]",
                                  PRE_PINS),
    "pre_q_without_scale": ("const double rq = 1.0 / sqrt(sq + eps) / sqrt((double)dk);",
                            "const double rq = 1.0 / sqrt(sq + eps);", PRE_PINS),
    "pre_k_normalised_by_q": ("const double rk = 1.0 / sqrt(sk + eps);",
                              "const double rk = 1.0 / sqrt(sq + eps);", PRE_PINS),
    "pre_silu_wrong_sign": ("u[c] = activation ? s / (1.0 + exp(-s)) : s;",
                            "u[c] = activation ? s / (1.0 + exp(s)) : s;", PRE_PINS),
    "pre_gate_positive": ("g[e] = -exp((double)A_log[h])", "g[e] = exp((double)A_log[h])",
                          PRE_PINS),
    "pre_history_out_stale": ("hist_out[j * C + c] = r < 3 ? (double)hist_in[r * C + c]",
                              "hist_out[j * C + c] = r < 3 ? (double)hist_in[j * C + c]",
                              PRE_PINS),
}


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, source, tmp_path):
    old, new, pins = MUTANTS[name]
    assert source.count(old) >= 1, "the oracle changed: update the planted mistake " + name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(source.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant_src),
                    "-o", str(lib), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    summary = [ln for ln in r.stdout.splitlines() if ln.strip()][-1:]
    assert r.returncode == 1 and "failed" in r.stdout, (name, summary)


@pytest.mark.parametrize("pins", [RECURRENCE_PINS, NORM_PINS, PRE_PINS])
def test_pins_pass_on_unmodified_copy(pins, source, tmp_path):
    """Control: the same build and run of the unmodified source passes, so a failure above
    comes from the planted mistake."""
    src = tmp_path / "copy.c"
    src.write_text(source)
    lib = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(src),
                    "-o", str(lib), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
