"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of ssm_oracle.c (on the CPU, in a
temporary directory), builds it, and runs the pin suite against that build in
a subprocess.  The suite must fail for every mutant.  The whole-model oracle
(mamba_model.py) gets the same treatment for the order of its projection
splits.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTANTS = {
    "softplus_sign": ("log1p(exp(-fabs(r)))", "log1p(exp(fabs(r)))"),
    "zoh_coef_sign": ("return expm1(delta * A) / A;", "return expm1(delta * A) / (-A);"),
    "decay_sign": ("    return exp(delta * A);\n}", "    return exp(-delta * A);\n}"),
    # constant decay source
    "const_decay_base2": ("        return exp(A);\n", "        return exp2(A);\n"),
    "const_write_scaled_by_dt": ("    if (disc == ORC_DECAY_CONST)\n        return 1.0;",
                                 "    if (disc == ORC_DECAY_CONST)\n        return delta;"),
    "const_write_uses_zoh": ("    if (disc == ORC_DECAY_CONST)\n        return 1.0;",
                             "    if (disc == ORC_DECAY_CONST)\n        return expm1(A) / A;"),
    "const_bwd_dA_missing_decay": ("dA[n] += da * a;\n", "dA[n] += da;\n"),
    "const_bwd_du_uses_output_weight": ("dut += g[n] * Bv;\n", "dut += g[n] * Cm[(b * L + t) * N + n];\n"),
    "A_not_exponentiated": ("A[n] = -exp(A_log[d * N + n]);\n                    h[n] = h0",
                            "A[n] = -(A_log[d * N + n]);\n                    h[n] = h0"),
    "readout_before_update": ("yv += Cm[(b * L + t) * N + n] * h[n];",
                              "yv += Cm[(b * L + t) * N + n] * (h[n] - wr) / a;"),
    "dropped_skip_term": ("                    if (Dskip)\n                        yv += Dskip[d] * ut;\n                    y[i]",
                          "                    y[i]"),
    "gate_sigmoid_not_silu": ("y[i] = z ? yv * orc_silu(z[i]) : yv;", "y[i] = z ? yv * orc_sigmoid(z[i]) : yv;"),
    "h0_ignored": ("h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "dt_bias_ignored": ("(dt_bias ? dt_bias[i % D] : 0.0)", "0.0"),
    # the forward conv's window read backwards (= taps reversed)
    "conv_taps_reversed": ("t - (W - 1) + k);\n            y[(b * L + t) * D + d] = silu",
                           "t - k);\n            y[(b * L + t) * D + d] = silu"),
    "conv_state_out_off_by_one": ("int64_t i = L - (W - 1) + j;", "int64_t i = L - W + j;"),
    "step_history_not_shifted": ("conv_state[(s * (int64_t)(W - 1) + k + 1) * D + d];",
                                 "conv_state[(s * (int64_t)(W - 1) + k) * D + d];"),
    "bwd_dA_missing_decay": ("dA[n] += da * a * dt;\n", "dA[n] += da * dt;\n"),
    "bwd_dz_wrong": ("(1.0 + z[i] * (1.0 - s))", "(1.0 + z[i] * s)"),
    "bwd_ddt_raw_missing_sigmoid": ("if (d_dt_raw) d_dt_raw[i] = ddt * sg;", "if (d_dt_raw) d_dt_raw[i] = ddt;"),
    "bwd_dC_uses_previous_state": ("gC[t * N + n] += hh[t * N + n] * dyv;", "gC[t * N + n] += hprev * dyv;"),
    "bwd_zoh_dA_sign": ("(dt * a * An - em1)", "(dt * a * An + em1)"),
    "bwd_adjoint_not_decayed": ("                            g[n] *= a;\n", ""),
    "conv_bwd_silu_derivative": ("g *= sg * (1.0 + acc * (1.0 - sg));", "g *= sg;"),
    "conv_bwd_taps_reversed": ("int64_t t = i + (W - 1) - k;", "int64_t t = i + k;"),
    "step_bf16_state_read_rounded": ("yv += Cm[s * N + n] * hnew;",
                                     "yv += Cm[s * N + n] * (state_bf16 ? orc_round_bf16(hnew) : hnew);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique / missing: %s" % name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mut), "-lm"], check=True)
    env = dict(os.environ, SSM_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])


MODEL_SRC = os.path.join(ROOT, "oracle", "mamba_model.py")

# Each entry: a list of (old, new) replacements applied together, so that a
# mix-up made the same way in both the token step and the sequence form
# (which the streaming == sequence pin cannot see) is planted.
MODEL_MUTANTS = {
    "swap_xin_z": [("xin, z = xz[:, :Di], xz[:, Di:]", "z, xin = xz[:, :Di], xz[:, Di:]"),
                   ("xin, z = xz[..., :Di], xz[..., Di:]", "z, xin = xz[..., :Di], xz[..., Di:]")],
    "swap_dt_C": [("dt_low, Bm, Cm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]",
                   "Cm, Bm, dt_low = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]"),
                  ("dt_raw = xp[..., :R] @", "dt_raw = xp[..., R + N:] @"),
                  ("xp[..., R:R + N], xp[..., R + N:],", "xp[..., R:R + N], xp[..., :R],")],
    "swap_dt_B": [("dt_low, Bm, Cm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]",
                   "Bm, dt_low, Cm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]"),
                  ("dt_raw = xp[..., :R] @", "dt_raw = xp[..., R:R + N] @"),
                  ("xp[..., R:R + N], xp[..., R + N:],", "xp[..., :R], xp[..., R + N:],")],
    "swap_B_C": [("dt_low, Bm, Cm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]",
                  "dt_low, Cm, Bm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]"),
                 ("xp[..., R:R + N], xp[..., R + N:],", "xp[..., R + N:], xp[..., R:R + N],")],
}


def _run_model_pins(src, tmp_path, oracle_lib):
    """Run the whole-model pins against a copy of the model oracle whose
    source is `src`; returns the pytest subprocess result."""
    import shutil
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    (pkg / "mamba_model.py").write_text(src)
    # the copy loads the built C oracle; the copied package is found first
    # (python -m puts the working directory at the head of sys.path)
    env = dict(os.environ, SSM_ORACLE_LIB=oracle_lib.build(force=False), OMP_NUM_THREADS="2",
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_model_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider", "--rootdir", ROOT], cwd=str(tmp_path),
                          env=env, capture_output=True, text=True, timeout=600)


def test_model_pins_pass_on_an_unmutated_copy(tmp_path, oracle_lib):
    """Control: the copy mechanism itself passes the pins, so a failure
    below is the planted mix-up."""
    r = _run_model_pins(open(MODEL_SRC).read(), tmp_path, oracle_lib)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MODEL_MUTANTS))
def test_model_pins_catch_mutant(name, tmp_path, oracle_lib):
    """Plant one mix-up of the projections' split order in a copy of the
    whole-model oracle and run its pins against that copy."""
    src = open(MODEL_SRC).read()
    for old, new in MODEL_MUTANTS[name]:
        assert src.count(old) == 1, "mutation site not unique / missing: %s: %s" % (name, old)
        src = src.replace(old, new)
    r = _run_model_pins(src, tmp_path, oracle_lib)
    assert r.returncode == 1 and " failed" in r.stdout, \
        "model pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
