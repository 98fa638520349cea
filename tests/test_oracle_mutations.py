"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/moe_oracle.c (on the CPU,
in a temporary directory), builds it, and runs the pin suite against that
copy through ORACLE_LIB; the suite has to fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = [
    ("bias_dropped", "if (bias) s += (double)bias[e];\n            logits[t * E + e] = (float)s;",
     "logits[t * E + e] = (float)s;"),
    ("router_transposed", "(double)wg[(int64_t)e * d + i];\n            if (bias)",
     "(double)wg[(int64_t)i * E + e];\n            if (bias)"),
    ("ties_to_higher_index", "return ia < ib;", "return ia > ib;"),
    ("softmax_sign", "z += exp((double)l[idx[t * k + j]] - top);", "z += exp(top - (double)l[idx[t * k + j]]);"),
    ("switch_renormalised", "for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - top);",
     "for (int32_t e = 0; e < k; ++e) z += exp((double)l[idx[t * k + e]] - top);"),
    ("capacity_off_by_one", "used[e] < capacity", "used[e] <= capacity"),
    ("capacity_not_per_group", "if (t % G == 0) memset", "if (t == 0) memset"),
    ("rows_descending", "int32_t r = used[e]++;", "int32_t r = offsets[e + 1] - 1 - (used[e]++ - offsets[e]);"),
    ("down_proj_transposed", "(double)w2[(int64_t)o * F + f]", "(double)w2[(int64_t)f * d + o]"),
    ("gate_up_swapped", "h[f] = act_silu(a) * b;", "h[f] = act_silu(b) * a;"),
    ("gelu_tanh_form", "return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));",
     "return 0.5 * z * (1.0 + tanh(0.7978845608028654 * (z + 0.044715 * z * z * z)));"),
    ("expert_bias2_dropped", "if (act != ACT_SWIGLU && b2) s += (double)b2[o];", ";"),
    ("combine_slot_weight", "double g = (double)w[t * k + j];", "double g = (double)w[t * k];"),
    ("shared_dropped", "if (Ys)\n            for (int32_t o = 0; o < d; ++o) y[t * d + o] += Ys[t * d + o];", ";"),
    ("ec_softmax_over_experts", "z += exp((double)logits[t * E + e] - m);", "z += exp((double)logits[t * E + e] - m) * (t < E);"),
    ("aux_without_E", "*aux = (double)E * a;", "*aux = a;"),
    ("zloss_not_squared", "zsum += lse * lse;", "zsum += lse;"),
    ("f_not_normalised_by_k", "f[e] /= (double)(T * k);", "f[e] /= (double)T;"),
    ("topk_capacity_without_k", "(double)tokens * (double)k / (double)E);\n    return c < min_capacity",
     "(double)tokens / (double)E);\n    return c < min_capacity"),
    ("min_capacity_ignored", "return c < min_capacity ? min_capacity : c;", "return c;"),
    ("softplus_as_relu", "const double sp = (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)));",
     "const double sp = (u > 0.0 ? u : 0.0);"),
    ("noise_projection_transposed", "u += (double)x[t * d + i] * (double)wn[(int64_t)e * d + i];",
     "u += (double)x[t * d + i] * (double)wn[(int64_t)i * E + e];"),
    ("ec_ties_to_higher_token", "if (best < 0 || ranks_before(logits[t * E + e], t, logits[best * E + e], best))",
     "if (best < 0 || logits[t * E + e] >= logits[best * E + e])"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name} no longer applies"
    mutated = tmp_path / "moe_oracle_mutated.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutated.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(mutated),
                           "-o", str(lib), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
