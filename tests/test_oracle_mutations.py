"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the
pins in test_oracle_pins.py catch every one of them."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dn_oracle.c")

# (name, old text, new text, which occurrence of old to replace)
MUTATIONS = [
    ("eps_outside_sqrt", "double inv = 1.0 / sqrt(ss + eps);", "double inv = 1.0 / (sqrt(ss) + eps);", 0),
    ("no_decay", "for (long e = 0; e < (long)dk * dv; ++e) S[e] *= alpha;", "(void)alpha;", 0),
    ("readout_before_update", "acc += S[(long)i * dv + j] * q[i];", "acc += (S[(long)i * dv + j] - k[i] * d[j]) * q[i];", 0),
    ("delta_sign", "d[j] = beta * (v[j] - kv);", "d[j] = beta * (v[j] + kv);", 0),
    ("beta_dropped", "d[j] = beta * (v[j] - kv);", "d[j] = (v[j] - kv);", 0),
    ("gqa_mapping", "const int g = h / group;", "const int g = h % Hk;", 0),
    ("conv_taps_reversed", "double a = (double)w[(long)c * K + (K - 1)] * u[c];", "double a = (double)w[(long)c * K] * u[c];", 0),
    ("silu_sign", "return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));", 0),
    ("gated_norm_sum_not_mean", "double inv = 1.0 / sqrt(ss / n + eps);", "double inv = 1.0 / sqrt(ss + eps);", 1),
    ("gate_dropped", "y[j] = (double)w[j] * o[j] * inv * dno_silu(z[j]);", "y[j] = (double)w[j] * o[j] * inv * z[j];", 0),
    ("norm_weight_dropped", "y[j] = (double)w[j] * o[j] * inv * dno_silu(z[j]);", "y[j] = o[j] * inv * dno_silu(z[j]);", 0),
    ("nibble_order", "int nib = (c & 1) ? (byte >> 4) : (byte & 15);", "int nib = (c & 1) ? (byte & 15) : (byte >> 4);", 0),
    ("nibble_unsigned", "return nib >= 8 ? nib - 16 : nib;", "return nib;", 0),
    ("gemv_int4_nibble_order", "const int lo = row[m] & 15, hi = row[m] >> 4;", "const int lo = row[m] >> 4, hi = row[m] & 15;", 0),
    ("gemv_int4_unsigned", "acc += (double)((lo ^ 8) - 8) * x[2 * m];", "acc += (double)lo * x[2 * m];", 0),
    ("row_scale_index", "y[r] = (double)s[r] * acc;", "y[r] = (double)s[0] * acc;", 0),
    ("history_order", "if (K > 1) memcpy(hist + (long)(K - 2) * C, u, sizeof(double) * C);", "if (K > 1) memcpy(hist, u, sizeof(double) * C);", 0),
    ("q_reads_k", "dno_l2norm(dk, c + (long)g * dk, d->eps_l2, qh);", "dno_l2norm(dk, c + QK + (long)g * dk, d->eps_l2, qh);", 0),
    ("v_wrong_head", "const double *v = c + 2 * QK + (long)h * dv;", "const double *v = c + 2 * QK + (long)g * dv;", 0),
    ("z_wrong_offset", "const double *z = u + C;", "const double *z = u + 2 * QK;", 0),
    ("prenorm_missing", "if (d->flags & DNO_X_RMSNORM)", "if (0)", 0),
    ("chain_broken", "memcpy(xin, o, sizeof(double) * B * D);", "(void)o;", 0),
    ("q_scale_ignored", "o[j] = q_scale * acc;", "o[j] = acc;", 0),
    ("per_key_decay_on_columns", "S[(long)i * dv + j] *= alpha[i];", "S[(long)i * dv + j] *= alpha[j % dk];", 0),
    ("per_key_alpha_head_index", "av[i] = (double)alpha[((long)b * Hv + h) * dk + i];",
     "av[i] = (double)alpha[((long)h * B + b) * dk + i];", 0),
    ("per_key_alpha_layer_stride", "const long aa = (d->flags & DNO_ALPHA_PER_KEY) ? ab * d->d_k : ab;",
     "const long aa = ab;", 0),
    ("gate_rows_swapped", "dno_gates(u[C + V + h], u[C + V + Hv + h],", "dno_gates(u[C + V + Hv + h], u[C + V + h],", 0),
    ("gate_head_shifted", "dno_gates(u[C + V + h], u[C + V + Hv + h],", "dno_gates(u[C + V + (h + 1) % Hv], u[C + V + Hv + (h + 1) % Hv],", 0),
    ("gate_param_head", "(double)W->a_log[h], (double)W->a_bias[h]", "(double)W->a_log[0], (double)W->a_bias[h]", 0),
    ("softplus_dropped", "*alpha = exp(-exp(a_log) * dno_softplus(a + a_bias));", "*alpha = exp(-exp(a_log) * (a + a_bias));", 0),
    ("a_log_not_exponentiated", "*alpha = exp(-exp(a_log) * dno_softplus(a + a_bias));", "*alpha = exp(-a_log * dno_softplus(a + a_bias));", 0),
    ("a_bias_sign", "*alpha = exp(-exp(a_log) * dno_softplus(a + a_bias));", "*alpha = exp(-exp(a_log) * dno_softplus(a - a_bias));", 0),
    ("beta_gate_sign", "*beta = 1.0 / (1.0 + exp(-b));", "*beta = 1.0 / (1.0 + exp(b));", 0),
    ("softplus_negative_branch", "log1p(exp(-fabs(y)))", "log1p(exp(-y))", 0),
]


def _mutate(src, old, new, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = src.index(old, idx + 1)
    return src[:idx] + new + src[idx + len(old):]


def test_every_mutation_site_exists():
    src = open(SRC).read()
    for name, old, new, occ in MUTATIONS:
        assert src.count(old) > occ, name


@pytest.mark.parametrize("name,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, occ, tmp_path):
    src = open(SRC).read()
    mutant = tmp_path / "mutant.c"
    mutant.write_text(_mutate(src, old, new, occ))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so), str(mutant), "-lm"])
    env = dict(os.environ, DN_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
