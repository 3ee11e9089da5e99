"""The oracle's pins must catch plausible mistakes.  Each case below plants one
mistake into a copy of the oracle's C source (a dropped term, a wrong sign,
constant or index), builds it on the CPU, runs the pin suite against it in a
fresh process, and requires at least one pin to fail.  CPU only."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gpt2_ref.c")

# (name, text to find, replacement, which occurrence (0-based))
MUTANTS = [
    ("ln_eps", "const double eps = 1e-5;", "const double eps = 1e-3;", 0),
    ("ln_unbiased_var", "v = v / C;", "v = v / (C - 1);", 0),
    ("ln_bwd_drop_xhat_term", "dx[c] += rstd[r] * (g - g_mean - xhat * gx_mean);",
     "dx[c] += rstd[r] * (g - g_mean);", 0),
    ("ln_bwd_db_times_xhat", "sb += dout[(i64)r * C + c];", "sb += dout[(i64)r * C + c] * xhat;", 0),
    ("att_no_scale_fwd", "double scale = 1.0 / sqrt((double)hd);", "double scale = 1.0;", 0),
    ("att_no_scale_bwd", "double scale = 1.0 / sqrt((double)hd);", "double scale = 1.0;", 1),
    ("att_mask_excludes_diagonal", "for (int u = 0; u <= t; u++) a[u] /= sum;",
     "for (int u = 0; u <= t; u++) a[u] = (u == t ? 0.0 : a[u] / (sum - a[t]));", 0),
    ("att_bwd_drop_softmax_term", "dp[u] = a[u] * (da[u] - dot);", "dp[u] = a[u] * da[u];", 0),
    ("att_bwd_dk_uses_k", "dk[d] += dp[u] * q[d] * scale;", "dk[d] += dp[u] * k[d] * scale;", 0),
    ("gelu_cubic_dropped", "out[i] = 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x)));",
     "out[i] = 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x)));", 0),
    ("gelu_bwd_factor3", "double dudx = k * (1.0 + 3.0 * 0.044715 * x * x);",
     "double dudx = k * (1.0 + 0.044715 * x * x);", 0),
    ("matmul_bwd_dinp_sign", "for (int i = 0; i < K; i++) dx[i] += d * wr[i];",
     "for (int i = 0; i < K; i++) dx[i] -= d * wr[i];", 0),
    ("matmul_fwd_bias_dropped", "out[(i64)r * OC + o] = (bias ? bias[o] : 0.0) + acc;",
     "out[(i64)r * OC + o] = acc;", 0),
    ("ce_bwd_sign", "(p[v] - (v == targets[r] ? 1.0 : 0.0)) / N", "(p[v] + (v == targets[r] ? 1.0 : 0.0)) / N", 0),
    ("ce_bwd_no_mean", "(p[v] - (v == targets[r] ? 1.0 : 0.0)) / N", "(p[v] - (v == targets[r] ? 1.0 : 0.0))", 0),
    ("residual_bwd_dropped", "d_r2[i] += d_r3[i];", "(void)0;", 0),
    ("encoder_bwd_wpe_sign", "gp[c] += d[c];", "gp[c] -= d[c];", 0),
    ("encoder_fwd_wrong_position", "const double *pe = wpe + (i64)t * C;",
     "const double *pe = wpe + (i64)(T - 1 - t) * C;", 0),
    ("adamw_no_bias_correction", "double mhat = m[i] / c1, vhat = v[i] / c2;",
     "double mhat = m[i], vhat = v[i];", 0),
    ("adamw_eps_inside_sqrt", "mhat / (sqrt(vhat) + eps) + wd * params[i]", "mhat / sqrt(vhat + eps) + wd * params[i]", 0),
    ("param_count_head_bias", "n[15] = C;               /* lnfb", "n[15] = C + 1;           /* lnfb", 0),
    ("act_set_drops_probs", "n[A_PROBS] = BT * s->V;", "n[A_PROBS] = 0;", 0),
    ("decode_cache_excludes_new_key", "for (int u = 0; u <= pos; u++) {\n                    const double *k",
     "for (int u = 0; u < pos + (pos == 0); u++) {\n                    const double *k", 0),
    ("decode_wrong_position_embedding", "PAR(M, params, 1) + (i64)pos * C, 1, 1, C);", "PAR(M, params, 1), 1, 1, C);",
     0),
    ("sampler_cdf_not_normalised", "cum += exp(z[v] - z[best]) / sum;", "cum += exp(z[v] - z[best]);", 0),
    ("bf16_seven_bits", "double r = rint(ldexp(m, 8));", "double r = rint(ldexp(m, 7));", 0),
    ("bf16_bias_sum_rounded", "sb += dout[(i64)r * OC + o];", "sb += d;", 0),
    ("bf16_weight_not_rounded", "if (rw) W = rw;", "(void)rw;", 0),
]

CHECK = r"""
import sys, traceback
import oracle
from tests import test_oracle_pins as P
checks = [
    lambda: P.test_num_parameters_matches_printed_header(oracle),
    lambda: P.test_num_activations_matches_printed_header(oracle),
    lambda: P.test_gradients_match_central_differences_every_element(oracle, 0),
    lambda: P.test_whole_model_matches_torch_float64(oracle, "fd0"),
    lambda: P.test_layers_match_torch_library(oracle),
    lambda: P.test_adamw_matches_torch_optimizer(oracle),
    lambda: P.test_adamw_first_step_closed_form(oracle),
    lambda: P.test_zero_embeddings_give_uniform_logits_and_ln_v(oracle),
    lambda: P.test_layernorm_statistics_before_affine(oracle),
    lambda: P.test_attention_special_cases(oracle),
    lambda: P.test_gelu_limits_and_exact_gelu_bound(oracle),
    lambda: P.test_encoder_backward_all_tokens_equal(oracle),
    lambda: P.test_decode_from_scratch_reproduces_the_full_forward(oracle, 0),
    lambda: P.test_decode_from_scratch_reproduces_the_full_forward(oracle, 1),
    lambda: P.test_sampler_is_argmax_or_the_cumulative_search(oracle),
    lambda: P.test_bf16_rounding_matches_closed_forms_and_torch(oracle),
    lambda: P.test_bf16_products_round_the_operands_only(oracle),
]
failed = 0
for c in checks:
    try:
        c()
    except Exception:
        failed += 1
print("FAILED_PINS", failed)
"""


def _replace_nth(text, old, new, n):
    idx = -1
    for _ in range(n + 1):
        idx = text.find(old, idx + 1)
        if idx < 0:
            return None
    return text[:idx] + new + text[idx + len(old):]


def _run(mutant, tmp):
    name, old, new, n = mutant
    src = open(SRC).read()
    mut = _replace_nth(src, old, new, n)
    assert mut is not None, f"mutation site for {name} not found"
    cpath = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib{name}.so")
    open(cpath, "w").write(mut)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-D_GNU_SOURCE",
                           "-o", so, cpath, "-lm"])
    env = dict(os.environ, GPT2_ORACLE_LIB=so, PYTHONPATH=ROOT, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", CHECK], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    return name, r


def test_unmodified_oracle_passes_the_check_script(oracle_lib):
    env = dict(os.environ, PYTHONPATH=ROOT, OMP_NUM_THREADS="1")
    env.pop("GPT2_ORACLE_LIB", None)
    r = subprocess.run([sys.executable, "-c", CHECK], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert "FAILED_PINS 0" in r.stdout, r.stdout + r.stderr


def test_every_planted_mistake_is_caught(oracle_lib):
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run(m, tmp), MUTANTS))
    missed = []
    for name, r in results:
        line = [l for l in r.stdout.splitlines() if l.startswith("FAILED_PINS")]
        # a crash also counts as caught, but the pins normally fail cleanly
        caught = r.returncode != 0 or (line and line[0] != "FAILED_PINS 0")
        if not caught:
            missed.append(name)
    assert not missed, f"planted mistakes no pin caught: {missed}"
