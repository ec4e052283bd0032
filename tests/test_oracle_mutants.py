"""The oracle's pins must reject plausible mistakes.

Each case copies ``oracle/psi_oracle.c``, plants one mistake in the copy (a
dropped term, a wrong sign or index, a skipped step), builds it into a
temporary library and runs the pin suite against it in a subprocess; the
suite must fail.  The committed oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "psi_oracle.c")

MUTANTS = {
    "linear_drops_bias": ("out = acc + orc_f(b[n]);", "out = acc;"),
    "linear_wrong_k_index": ("orc_f(x[k]) * orc_f(w[k])", "orc_f(x[k]) * orc_f(w[K - 1 - k])"),
    "linear_ignores_carry": ("float init = acc_in ? acc_in[(size_t)m * N + n] : 0.0f;",
                             "float init = 0.0f;"),
    "linear_variants_swapped": ("else if (variant == 1)", "else if (variant == 0)"),
    "rounding_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "rounding_truncates": ("kept += 1u;", "kept += 0u;"),
    "gelu_wrong_sign": ("v / (1.0 + exp(-2.0 * z))", "v / (1.0 + exp(2.0 * z))"),
    "gelu_negative_branch_dropped": ("return v * e / (1.0 + e);", "return v * e;"),
    "gelu_literal_tanh_cancels": ("  if (z >= 0.0) return v / (1.0 + exp(-2.0 * z));",
                                  "  return 0.5 * v * (1.0 + tanh(z));"),
    "gelu_cubic_dropped": ("(v + 0.044715 * v * v * v)", "(v)"),
    "ffn_skips_gelu": ("orc_gelu_bf16(pre, (size_t)M * h, H);",
                       "memcpy(H, pre, (size_t)M * h * sizeof(uint16_t));"),
    "ffn_drops_residual": ("y[i] = residual ? orc_bf16_from_float(orc_f(x[i]) + orc_f(ysub[i])) : ysub[i];",
                           "y[i] = ysub[i];"),
    "attn_no_max_shift": ("float diff = s[j] - m;", "float diff = s[j];"),
    "attn_wrong_scale": ("(float)(1.0 / sqrt((double)dh))", "(float)(1.0 / (double)dh)"),
    "attn_values_from_keys": ("const uint16_t* vj = v + (size_t)j * ldv", "const uint16_t* vj = k + (size_t)j * ldk"),
    "attn_unnormalised": ("orc_bf16_from_float(z[c] / l)", "orc_bf16_from_float(z[c])"),
    "sublayer_kv_from_x": ("const uint16_t* src = ctx ? ctx : x;", "const uint16_t* src = x;"),
}
MUTANTS["double_rounding_via_float"] = (
    "uint16_t orc_bf16_from_double(double v) {\n  if (isnan(v))",
    "uint16_t orc_bf16_from_double(double v) {\n  return orc_bf16_from_float((float)v);\n  if (isnan(v))")


# Mistakes in the q/k normalisation, rotary and BF16-numerator parts; their
# pins are selected by keyword so the case stays short.
EXT_PINS = "rmsnorm or rope or bf16_numerator or sublayer_ext"
EXT_MUTANTS = {
    "rms_drops_eps": ("const double den = sqrt(s / d + eps);", "const double den = sqrt(s / d);"),
    "rms_mean_over_tile": ("const double den = sqrt(s / d + eps);", "const double den = sqrt(s / tile + eps);"),
    "rms_no_square": ("sj += (double)orc_f(xr[i]) * (double)orc_f(xr[i]);", "sj += fabs((double)orc_f(xr[i]));"),
    "rms_drops_gain": ("orc_bf16_from_double((double)orc_f(g[i]) * (double)orc_f(xr[i]) / den)",
                       "orc_bf16_from_double((double)orc_f(xr[i]) / den)"),
    "rms_last_tile_only": ("      s += sj;", "      s = sj;"),
    "rope_sign": ("orc_bf16_from_double(c * a - sv * b)", "orc_bf16_from_double(c * a + sv * b)"),
    "rope_ignores_head": ("const uint16_t* xr = x + (size_t)t * ldx + (size_t)h * dh;",
                          "const uint16_t* xr = x + (size_t)t * ldx;"),
    "rope_table_row": ("const double c = cs[(size_t)t * hh + j], sv = sn[(size_t)t * hh + j];",
                       "const double c = cs[j], sv = sn[j];"),
    "bf16p_not_rounded": ("float pb = orc_f(orc_bf16_from_float(p));", "float pb = p;"),
    "bf16p_rounds_normaliser": ("float p = (float)exp((double)(s[j] - m));\n            l = l + p;",
                                "float p = (float)exp((double)(s[j] - m));\n            l = l + orc_f(orc_bf16_from_float(p));"),
    "ext_k_uses_q_gain": ("if (gk) orc_rmsnorm(Kb, Ms, d, d, gk,", "if (gk) orc_rmsnorm(Kb, Ms, d, d, gq,"),
}


# Mistakes in the residual write y = B(f(x) + f(Y)).
RESIDUAL_PINS = "residual"
_RES = "x[i] = orc_bf16_from_float(orc_f(x[i]) + orc_f(y[i]));"
RESIDUAL_MUTANTS = {
    "residual_wrong_operand": (_RES, "x[i] = orc_bf16_from_float(orc_f(y[i]) + orc_f(y[i]));"),
    "residual_subtracts": (_RES, "x[i] = orc_bf16_from_float(orc_f(x[i]) - orc_f(y[i]));"),
    "residual_truncates": (_RES, "{ float s_ = orc_f(x[i]) + orc_f(y[i]); uint32_t w_; "
                                 "memcpy(&w_, &s_, sizeof w_); x[i] = (uint16_t)(w_ >> 16); }"),
    "residual_drops_sublayer": (_RES, "x[i] = x[i];"),
    "residual_ties_away": (_RES, "{ float s_ = orc_f(x[i]) + orc_f(y[i]); uint32_t w_; "
                                 "memcpy(&w_, &s_, sizeof w_); x[i] = (uint16_t)((w_ + 0x8000u) >> 16); }"),
}


def _run_mutant(old, new, tmp_path, select=None):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation pattern not found"
    mut = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mut)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-w", "-o", str(lib), str(csrc), "-lm"], check=True)
    env = dict(os.environ, PSI_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    if select:
        cmd += ["-k", select]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(EXT_MUTANTS))
def test_pins_reject_ext_mutant(name, tmp_path):
    old, new = EXT_MUTANTS[name]
    r = _run_mutant(old, new, tmp_path, EXT_PINS)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation pattern for {name} not found"
    mut = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mut)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-w", "-o", str(lib), str(csrc), "-lm"], check=True)
    env = dict(os.environ, PSI_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(RESIDUAL_MUTANTS))
def test_pins_reject_residual_mutant(name, tmp_path):
    old, new = RESIDUAL_MUTANTS[name]
    r = _run_mutant(old, new, tmp_path, RESIDUAL_PINS)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"
