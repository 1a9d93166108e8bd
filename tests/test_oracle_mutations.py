"""The oracle's pins must be able to fail: plant one plausible mistake at a time
in a copy of oracle/moe_oracle.c (on the CPU), build it, and require that the
pin suite (tests/test_oracle.py) rejects every planted copy."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# name -> (text in the oracle source, planted replacement)
MUTANTS = {
    "drop_expert_bias2": ("y[o] += load(b2, (int64_t)e * H + o, dt);", "y[o] += 0.0;"),
    "silu_evaluated_as_gelu": ("p->act == 1 ?", "p->act == 99 ?"),
    "silu_wrong_sign": ("a / (1.0 + exp(-a))", "a / (1.0 + exp(a))"),
    "gelu_wrong_sign": ("0.5 * a * (1.0 + erf(a * M_SQRT1_2))", "0.5 * a * (1.0 - erf(a * M_SQRT1_2))"),
    "aux_without_E": ("*aux = (double)E * acc;", "*aux = acc;"),
    "tie_to_higher_index": ("if (best < 0 || l[e] > l[best]) best = e;",
                            "if (best < 0 || l[e] >= l[best]) best = e;"),
    "capacity_off_by_one": ("if (fill[e] < cap) {", "if (fill[e] <= cap) {"),
    "dropped_slot_still_added": ("if (pos[t * k + s] < 0) continue;", ""),
    "z_not_squared": ("acc += L[t] * L[t];", "acc += L[t];"),
    "w1_transposed": ("axpy_row(a, xr[i], W1, ((int64_t)e * H + i) * F, F, dt);",
                      "for (int j = 0; j < F; ++j) a[j] += xr[i] * "
                      "load(W1, (int64_t)e * H * F + (int64_t)j * H + i, dt);"),
    "no_renormalisation": ("topk_w[t * k + s] = pt[idx[s]] / S;", "topk_w[t * k + s] = pt[idx[s]];"),
    "lse_without_shift": ("L[t] = m + log(Z);", "L[t] = log(Z);"),
    "gate_bias_dropped": ("for (int e = 0; e < E; ++e) l[e] += load(bg, e, dt);", ";"),
    "offsets_shifted": ("offsets[e + 1] = offsets[e] + (int32_t)fill[e];",
                        "offsets[e + 1] = offsets[e] + (int32_t)fill[e] + (e == 0);"),
    "aux_counts_after_capacity": (
        "acc += ((double)c / (double)(T * k))",
        "acc += ((double)(c < orc_capacity(p) ? c : orc_capacity(p)) / (double)(T * k))"),
    "ec_ties_to_higher_token": (
        "if (best < 0 || logits[(g * G + i) * E + e] > logits[(g * G + best) * E + e])",
        "if (best < 0 || logits[(g * G + i) * E + e] >= logits[(g * G + best) * E + e])"),
    "ec_ranked_by_probs": (
        "if (best < 0 || logits[(g * G + i) * E + e] > logits[(g * G + best) * E + e])",
        "if (best < 0 || probs[(g * G + i) * E + e] > probs[(g * G + best) * E + e])"),
    "ec_capacity_floor": ("double c = ceil(cf * (double)group * (double)p->k / (double)p->E);",
                          "double c = floor(cf * (double)group * (double)p->k / (double)p->E);"),
    "ec_weights_unnormalised": ("probs[t * E + e] = exp(l[e] - m) / Z;",
                                "probs[t * E + e] = exp(l[e] - m);"),
    "ec_rows_group_major": ("const int64_t row = (e * ng + g) * C + j;",
                            "const int64_t row = (g * E + e) * C + j;"),
    "bwd_gelu_grad_without_density": (
        "+ a * exp(-0.5 * a * a) / sqrt(2.0 * M_PI);", ";"),
    "bwd_silu_grad_is_sigmoid": ("return s * (1.0 + a * (1.0 - s));", "return s;"),
    "bwd_renorm_without_mean": ("dp[idx[s]] += (dw[s] - sw) / S;", "dp[idx[s]] += dw[s] / S;"),
    "bwd_aux_without_E": ("g_aux * (double)E * ((double)r->counts[e]",
                          "g_aux * ((double)r->counts[e]"),
    "bwd_z_without_2": ("g_z * 2.0 * r->lse[t]", "g_z * r->lse[t]"),
    "bwd_softmax_not_centred": ("dl[e] = pt[e] * (dp[e] - pdp)", "dl[e] = pt[e] * dp[e]"),
    "bwd_dW2_from_pre_activation": ("const double h = act_val(p, a[j]);", "const double h = a[j];"),
    "bwd_dropped_slot_passes_gradient": (
        "                dw[s] = 0.0;\n                if (r.pos[t * k + s] < 0) continue;\n"
        "                const int e = r.idx[t * k + s];\n                double* a = A",
        "                dw[s] = 0.0;\n"
        "                const int e = r.idx[t * k + s];\n                double* a = A"),
    "slot_weights_swapped": ("const double w = topk_w[t * k + s];",
                             "const double w = topk_w[t * k + (k - 1 - s)];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    d = tmp_path / name
    d.mkdir()
    (d / "moe_oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ROOT, "oracle", "moe_oracle.h"), d / "moe_oracle.h")
    lib = d / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(d / "moe_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not slow", os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"planted mistake {name} survived the pins:\n{r.stdout[-2000:]}"
