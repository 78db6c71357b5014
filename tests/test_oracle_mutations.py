"""Planted mistakes in the oracle: each one must fail at least one of the
oracle's pins (tests/test_oracle_steps.py, tests/test_oracle_formats.py).

A mistake is a one-line edit of oracle/step5_oracle.c of the kind that is
easy to make and hard to see (a dropped term, a flipped sign, a wrong index
or operand, an off-by-one window, a reversed tie order, a wrong rounding).
Every mutant is compiled like the oracle itself into a temporary library and
the pins run against it in a child process (the oracle wrapper loads the
library named by STEP5_ORACLE_LIB); the unmutated source, built the same way,
must pass them. CPU only; the mutants and the control run in parallel.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "step5_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_steps.py"),
        os.path.join(ROOT, "tests", "test_oracle_formats.py")]

# (name, text in the source, replacement)
MUTANTS = [
    # number formats
    ("bf16_truncates", "u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    ("bf16_ties_away", "u += 0x7fffu + lsb;", "u += 0x8000u + 0u * lsb;"),
    ("e4m3_subnormal_scale", "ldexp((double)m, -9)", "ldexp((double)m, -8)"),
    ("e4m3_exponent_bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 6)"),
    ("e4m3_ties_to_odd", "else pick = (c & 1) ? c + 1 : c;", "else pick = (c & 1) ? c : c + 1;"),
    ("e4m3_rounds_down", "if (dlo < dhi) pick = c;", "if (dlo <= dhi + 1.0) pick = c;"),
    # exp
    ("exp_drops_ln2_low_part", "r = fmaf(-n, O_LN2_LO, r);", "r = fmaf(-n, 0.0f, r);"),
    ("exp_degree_6", "float p = c[7];\n  for (int k = 6;", "float p = c[6];\n  for (int k = 5;"),
    ("exp_truncates_n", "float n = nearbyintf(t);", "float n = truncf(t);"),
    # rotation
    ("rope_sign", "y[i] = ac - bs;", "y[i] = ac + bs;"),
    ("rope_partner", "b[i] = y[i + 16];", "b[i] = y[i + 15];"),
    ("rope_cos_sin_swapped",
     "float c = o_bf16_to_f32(cs_row[i]), s = o_bf16_to_f32(cs_row[16 + i]);",
     "float s = o_bf16_to_f32(cs_row[i]), c = o_bf16_to_f32(cs_row[16 + i]);"),
    # norms
    ("q_scale_w_not_1_plus_w", "float scale = 1.0f + w[i];", "float scale = w[i];"),
    ("q_mean_not_mean_square", "sq[i] = x[i] * x[i]; }", "sq[i] = x[i]; }"),
    ("k_no_bias", "y[i] = t + b[i];", "y[i] = t;"),
    ("k_no_mean", "d[i] = x[i] - mu;", "d[i] = x[i];"),
    ("k_unbiased_variance", "float var = o_sum64(d2) / 64.0f;", "float var = o_sum64(d2) / 63.0f;"),
    ("sum64_drops_a_run", "for (int c = 0; c < 8; ++c) s[c] = pair8(x + 8 * c);",
     "for (int c = 0; c < 8; ++c) s[c] = c == 7 ? 0.0f : pair8(x + 8 * c);"),
    # summary
    ("summary_softmax_of_minus_z", "e[t] = o_exp(z[t] - m);", "e[t] = o_exp(m - z[t]);"),
    ("summary_no_division", "float s = num / den;", "float s = num;"),
    ("summary_token_offset", "float num = e[0] * kp[0][dd];", "float num = e[0] * kp[1][dd];"),
    # scores
    ("score_no_relu", "if (!(t > 0.0f)) t = 0.0f;", "if (0) t = 0.0f;"),
    ("score_heads_interleaved", "q8[(r * idx_heads + g * hpg + hh) * IDX_DIM + d]",
     "q8[(r * idx_heads + hh * groups + g) * IDX_DIM + d]"),
    ("score_weight_of_head_in_group", "float term = t * w[g * hpg + hh];", "float term = t * w[hh];"),
    ("score_misses_last_candidate", "int64_t ncand = row_pos[r] / REGION;\n    const uint8_t* S",
     "int64_t ncand = row_pos[r] / REGION - 1;\n    const uint8_t* S"),
    # selection
    ("select_ties_by_larger_id", "return (a->id < b->id) ? -1 : (a->id > b->id);",
     "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    ("select_ascending_scores", "if (a->s > b->s) return -1;\n  if (a->s < b->s) return 1;",
     "if (a->s < b->s) return -1;\n  if (a->s > b->s) return 1;"),
    ("select_window_short", "int64_t ncand = row_pos[u / groups] / REGION;",
     "int64_t ncand = row_pos[u / groups] / REGION - 1;"),
    # attention
    ("attend_own_region_drops_p", "for (int64_t t = own0; t <= p; ++t)",
     "for (int64_t t = own0; t < p; ++t)"),
    ("attend_kv_head_modulo", "int h = (int)(u % q_heads), g = h / qpk;",
     "int h = (int)(u % q_heads), g = h % kv_heads;"),
    ("attend_no_scale", "lg[i] = scale * dot;", "lg[i] = dot;"),
    ("attend_region_7_tokens", "for (int t = 0; t < REGION; ++t) toks[ntok++]",
     "for (int t = 0; t < REGION - 1; ++t) toks[ntok++]"),
    # fused projection
    ("project_drops_last_k", "for (int64_t k = 0; k < hsize; ++k)\n        acc +=",
     "for (int64_t k = 0; k < hsize - 1; ++k)\n        acc +="),
    ("project_weight_transposed", "(double)o_bf16_to_f32(wn[k]);", "(double)o_bf16_to_f32(w[k * n_out + n]);"),
    ("project_first_row_only", "const uint16_t* hr = hidden + r * hsize;", "const uint16_t* hr = hidden;"),
    ("project_hidden_column_off_by_one", "acc += (double)o_bf16_to_f32(hr[k])",
     "acc += (double)o_bf16_to_f32(hr[k > 0 ? k - 1 : 0])"),
]

CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
          "-fopenmp", "-fPIC", "-shared", "-w"]


def _compile(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *CFLAGS, c, "-o", path, "-lm"], check=True)
    return path


def _pins(lib):
    env = dict(os.environ, STEP5_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("mutants"))
    base = open(SRC).read()
    jobs = {"control": base}
    for name, old, new in MUTANTS:
        assert base.count(old) == 1, (name, base.count(old))
        jobs[name] = base.replace(old, new)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        libs = dict(zip(jobs, ex.map(lambda kv: _compile(kv[1], os.path.join(d, kv[0] + ".so")),
                                     jobs.items())))
        res = dict(zip(libs, ex.map(_pins, libs.values())))
    return res


def test_control_passes_every_pin(outcomes):
    rc, log = outcomes["control"]
    assert rc == 0, log


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(outcomes, name):
    rc, log = outcomes[name]
    assert rc != 0, f"planted mistake '{name}' passed every pin"
