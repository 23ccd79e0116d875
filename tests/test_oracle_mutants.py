"""The pins must catch plausible mistakes planted in the oracle.

Each mutant is a copy of oracle/gdn_oracle.c with one textual change (a
dropped term, a wrong sign, index or operand), built into a temporary
library on the CPU.  All pins run against it in a child process (a mutant
may read out of bounds); the child must fail.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

MUTANTS = {
    "prediction_not_decayed": ("p[j] = vt[j] - a * p[j]", "p[j] = vt[j] - p[j]"),
    "write_sign_flipped": ("a * Hs[i * V + j] + b * kt[i] * p[j]",
                           "a * Hs[i * V + j] - b * kt[i] * p[j]"),
    "prediction_uses_q": ("p[j] += Hs[i * V + j] * kt[i]", "p[j] += Hs[i * V + j] * qt[i]"),
    "state_not_decayed": ("Hs[i * V + j] = a * Hs[i * V + j] +", "Hs[i * V + j] = Hs[i * V + j] +"),
    "beta_dropped": ("+ b * kt[i] * p[j]", "+ kt[i] * p[j]"),
    "output_uses_k": ("ot[j] += Hs[i * V + j] * qt[i]", "ot[j] += Hs[i * V + j] * kt[i]"),
    "state_transposed": ("p[j] += Hs[i * V + j] * kt[i]", "p[j] += Hs[j * K + i] * kt[i]"),
    "gqa_mapping_modulo": ("const int h = hv / (HV / H);", "const int h = hv % H;"),
    "softplus_threshold_2": ("x > 20.0 ? x :", "x > 2.0 ? x :"),
    "gate_sign": ("g_out[t * HV + hv] = -exp(A_log[hv])", "g_out[t * HV + hv] = exp(A_log[hv])"),
    "gate_no_exp": ("g_out[t * HV + hv] = -exp(A_log[hv])", "g_out[t * HV + hv] = -(A_log[hv])"),
    "dt_bias_dropped": ("(dt_bias ? dt_bias[hv] : 0.0)", "0.0"),
    "scale_ignored": ("ot[j] *= J->scale;", "ot[j] *= 1.0;"),
    "h0_ignored": ("  if (J->h0)\n    memcpy", "  if (0)\n    memcpy"),
    "no_reset_between_sequences": ("for (int64_t t = J->bos[n];", "for (int64_t t = J->bos[0];"),
    "kda_bias_per_channel_only": ("dt_bias[(int64_t)h * D + d]", "dt_bias[d]"),
    "kda_bias_per_head_only": ("dt_bias[(int64_t)h * D + d]", "dt_bias[h]"),
    "kda_scale_not_exponentiated": ("const double head_scale = -exp(A_log[h]);",
                                    "const double head_scale = -A_log[h];"),
    "kda_rows_strided_by_D": ("const int64_t row = (t * H + h) * (int64_t)D;",
                              "const int64_t row = (h * T + t) * (int64_t)D;"),
    "bwd_dk_misses_prediction_path": ("dk[i] = b * acc_u + acc_p;", "dk[i] = b * acc_u;"),
    "bwd_dp_sign": ("acc_p += Hp[i * V + j] * (-a * du[j]);", "acc_p += Hp[i * V + j] * (a * du[j]);"),
    "bwd_state_grad_not_decayed": ("dH[i * V + j] = a * dH[i * V + j] + kt[i]",
                                   "dH[i * V + j] = dH[i * V + j] + kt[i]"),
    "bwd_da_misses_prediction": ("for (int j = 0; j < V; ++j) da -= p[j] * du[j];", ""),
    "bwd_dg_not_times_a": ("const double dg = a * da;", "const double dg = da;"),
    "bwd_softplus_slope_sign": ("1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))"),
    "bwd_dq_uses_previous_state": ("acc += Hs[i * V + j] * dot[j];", "acc += Hp[i * V + j] * dot[j];"),
    "bwd_gqa_first_head_only": ("for (int r = 0; r < G; ++r) {", "for (int r = 0; r < 1; ++r) {"),
    "bwd_dA_log_uses_dg_raw": ("dA_sum += dg * gl[s];", "dA_sum += dgr * gl[s];"),
    "bwd_dbeta_uses_v": ("dbeta += dH[i * V + j] * kt[i] * u[j];",
                         "dbeta += dH[i * V + j] * kt[i] * vt[j];"),
    "bwd_dht_ignored": ("  if (J->dht)\n    memcpy", "  if (0)\n    memcpy"),
    "bwd_output_scale_dropped": ("dH[i * V + j] += J->scale * qt[i] * dot[j];",
                                 "dH[i * V + j] += qt[i] * dot[j];"),
    "decay_is_exp_of_negative": ("const double a = exp(J->g[t * HV + hv]);",
                                 "const double a = exp(-J->g[t * HV + hv]);"),
}

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
lib = oracle.load(%r)
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except AssertionError as e:
        failed.append(pin.__name__)
    except Exception as e:
        failed.append(pin.__name__ + ":" + type(e).__name__)
print("FAILED_PINS", failed)
sys.exit(1 if failed else 0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %r" % old
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new, 1))
    lib = oracle_build.build(str(mut), str(tmp_path / "libmutant.so"), werror=False)
    code = CHILD % (ROOT, os.path.join(ROOT, "tests"), lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, "mutant %s passed every pin:\n%s%s" % (name, res.stdout,
                                                                      res.stderr[-2000:])


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness on an unmodified copy passes."""
    lib = oracle_build.build(oracle_build.SRC, str(tmp_path / "libcopy.so"))
    code = CHILD % (ROOT, os.path.join(ROOT, "tests"), lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr[-2000:]
