"""Each pin must catch plausible mistakes in the oracle (CPU only).

Every mutant below is a copy of oracle/tg_oracle.c with one planted mistake
(a dropped term, a wrong sign, a wrong index, a transposed operand, a
reversed tie rule, ...).  It is compiled into a temporary library and the
full pin set of tests/oracle_pins.py runs against it in a child process; at
least one pin must fail for every mutant.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (name, exact text in tg_oracle.c, replacement)
MUTANTS = [
    ("gate_drop_eps", "sqrt(sumsq / (double)d + eps)", "sqrt(sumsq / (double)d)"),
    ("gate_sum_not_mean", "sqrt(sumsq / (double)d + eps)", "sqrt(sumsq + eps)"),
    ("gate_drop_gamma", "u[i] = g * (x[i] / rms);", "u[i] = (x[i] / rms); (void)g;"),
    ("gate_silu_sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    ("gate_sigmoid_not_silu", "z / (1.0 + exp(-z))", "1.0 / (1.0 + exp(-z))"),
    ("gate_drop_b1", "double z = b1 ? b1[j] : 0.0;", "double z = 0.0;"),
    ("gate_drop_b2", "double s = b2;", "double s = 0.0;"),
    ("gate_w1_transposed", "z += wrow[i] * u[i];", "z += w1[i * h + j] * u[i]; (void)wrow;"),
    ("gate_scores_nonprunable", "if (!prunable[t]) {\n        scores[t] = 0.0;", "if (0) {\n        scores[t] = 0.0;"),
    ("select_ties_high_index", "return (a->t < b->t) ? -1 : (a->t > b->t) ? 1 : 0;",
     "return (a->t < b->t) ? 1 : (a->t > b->t) ? -1 : 0;"),
    ("select_nan_highest", "if (an != bn) return an ? 1 : -1;", "if (an != bn) return an ? -1 : 1;"),
    ("select_ascending", "if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
     "if (a->s > b->s) return 1;\n    if (a->s < b->s) return -1;"),
    ("select_drops_nonprunable", "if (!prunable[t]) keep[t] = 1;", "if (0) keep[t] = 1;"),
    ("select_one_short", "for (int64_t i = 0; i < keepP; ++i)", "for (int64_t i = 0; i + 1 < keepP; ++i)"),
    ("select_negative_nan_order", "const int an = isnan(a->s), bn = isnan(b->s);",
     "const int an = 0, bn = 0;"),
    ("gather_pos_is_rank", "pos_kept[r] = (int32_t)t;", "pos_kept[r] = (int32_t)r;"),
    ("gather_score_by_rank", "score_kept[r] = scores[t];", "score_kept[r] = scores[r];"),
    ("kv_gather_layer0_only", "cache + (l * T + (int64_t)kept_idx[r]) * row_bytes",
     "cache + ((int64_t)kept_idx[r]) * row_bytes"),
    ("kv_gather_by_rank", "cache + (l * T + (int64_t)kept_idx[r]) * row_bytes",
     "cache + (l * T + r) * row_bytes"),
    ("attn_causal_excludes_diag", "causal ? r + 1 : N", "causal ? r : N"),
    ("attn_bias_sign", "scale * dot + gain[hq] * key_score[c]", "scale * dot - gain[hq] * key_score[c]"),
    ("attn_qscale_dot_only", "z[c] = cr * (scale * dot + gain[hq] * key_score[c]);",
     "z[c] = cr * scale * dot + gain[hq] * key_score[c];"),
    ("attn_gqa_modulo", "const int64_t kv = hq / G;", "const int64_t kv = hq % Hkv;"),
    ("attn_lse_missing_max", "lse[hq * n_rows + i] = m + log(denom);", "lse[hq * n_rows + i] = log(denom);"),
    ("attn_no_scale", "z[c] = cr * (scale * dot", "z[c] = cr * (dot"),
    ("attn_gain_by_kv_head", "gain[hq] * key_score[c]", "gain[kv] * key_score[c]"),
    ("attn_no_normalise", "for (int64_t e = 0; e < D; ++e) o[e] /= denom;", ";"),
    ("attn_q_by_kv_head", "const double* qr = q + (r * Hq + hq) * D;", "const double* qr = q + (r * Hq + kv) * D;"),
    ("attn_v_from_first_head", "const double* vc = v + (c * Hkv + kv) * D;", "const double* vc = v + (c * Hkv) * D;"),
    ("bwd_delta_sign", "P[c] * (dZ[c] - delta)", "P[c] * (dZ[c] + delta)"),
    ("bwd_dq_no_qscale", "dq_r[e] += dz * c_r * scale * k_c[e];", "dq_r[e] += dz * scale * k_c[e];"),
    ("bwd_dk_no_scale", "dk_c[e] += dz * c_r * scale * q_r[e];", "dk_c[e] += dz * c_r * q_r[e];"),
    ("bwd_dv_uses_dz", "dv_c[e] += P[c] * do_r[e];", "dv_c[e] += dz * do_r[e];"),
    ("bwd_dscore_no_gain", "ds_part[kvh * N + c] += dz * c_r * gain[hq];",
     "ds_part[kvh * N + c] += dz * c_r;"),
    ("bwd_dgain_no_qscale", "dg += dz * c_r * key_score[c];", "dg += dz * key_score[c];"),
    ("bwd_causal_excludes_diag", "causal ? (r + 1) : N", "causal ? r : N"),
    ("bwd_no_normalise", "P[c] /= sum;", "(void)sum;"),
    ("bwd_dk_from_first_head", "double* dk_c = dk + (c * Hkv + kvh) * D;", "double* dk_c = dk + (c * Hkv) * D;"),
]

RUNNER = r"""
import sys, traceback
sys.path[:0] = [%r, %r]
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle(sys.argv[1])
failed = []
for pin in ALL_PINS:
    try:
        pin(orc)
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED:" + ",".join(failed))
""" % (ROOT, HERE)


def _run_mutant(args):
    name, old, new, tmpdir = args
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    msrc = src.replace(old, new)
    cpath = os.path.join(tmpdir, name + ".c")
    with open(cpath, "w") as f:
        f.write(msrc)
    lib = oracle.build(force=True, src=cpath, out=os.path.join(tmpdir, name + ".so"))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-c", RUNNER, lib], capture_output=True,
                       text=True, timeout=300, env=env)
    line = [l for l in p.stdout.splitlines() if l.startswith("FAILED:")]
    if p.returncode != 0 and not line:
        return name, ["<crashed rc=%d>" % p.returncode]
    return name, [x for x in line[0][len("FAILED:"):].split(",") if x]


def test_every_mutant_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [(n, o, r, tmp) for n, o, r in MUTANTS]
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = dict(ex.map(_run_mutant, jobs))
    survivors = [n for n, f in results.items() if not f]
    assert not survivors, "mutants that pass every pin: %s" % survivors
