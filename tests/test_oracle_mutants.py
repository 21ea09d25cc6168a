"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pin battery catches every one of them.  The real oracle is never
modified: each mutant is a text edit of moe_oracle.c compiled to a temporary
library and exercised in a subprocess."""
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "silu_sign": ("return z / (1.0f + expf(-z));", "return z / (1.0f + expf(z));"),
    "silu_as_sigmoid": ("return z / (1.0f + expf(-z));", "return 1.0f / (1.0f + expf(-z));"),
    "bias_dropped": ("for (int e = 0; e < E; ++e) l[e] = l[e] + bias[e];",
                     "for (int e = 0; e < E; ++e) l[e] = l[e];"),
    "logit_first_term_dropped": ("for (int h = 0; h < H; ++h) {\n            const float xv",
                                 "for (int h = 1; h < H; ++h) {\n            const float xv"),
    "tie_rule_reversed": ("return (A->e < B->e) ? -1 : (A->e > B->e ? 1 : 0);",
                          "return (A->e > B->e) ? -1 : (A->e < B->e ? 1 : 0);"),
    "order_ascending": ("if (A->p > B->p) return -1;\n    if (A->p < B->p) return 1;",
                        "if (A->p < B->p) return -1;\n    if (A->p > B->p) return 1;"),
    "no_max_shift": ("z[e] = expf(lc[e] - m);", "z[e] = expf(lc[e]);"),
    "nan_not_masked": ("lc[e] = isnan(l[e]) ? -INFINITY : l[e];", "lc[e] = l[e];"),
    "softmax_denominator_short": ("for (int e = 0; e < E; ++e) S = S + z[e];",
                                  "for (int e = 1; e < E; ++e) S = S + z[e];"),
    "renorm_dropped": ("w[(size_t)t * k + j] = renorm ? order[j].p / s : order[j].p;",
                       "w[(size_t)t * k + j] = order[j].p;"),
    "renorm_sum_short": ("for (int j = 0; j < k; ++j) s = s + order[j].p;",
                         "for (int j = 0; j + 1 < k; ++j) s = s + order[j].p;"),
    "gate_up_swapped": ("a[i] = oref_silu(g) * u;", "a[i] = oref_silu(u) * g;"),
    "up_reads_gate": ("const float* wup = w_gu + (size_t)(I + i) * H;",
                      "const float* wup = w_gu + (size_t)i * H;"),
    "gate_last_term_dropped": ("for (int h = 0; h < H; ++h) {\n                    g = g + x[h]",
                               "for (int h = 0; h + 1 < H; ++h) {\n                    g = g + x[h]"),
    "down_transposed": ("acc = acc + a[i] * wd[i];", "acc = acc + a[i] * w_dn[(size_t)i * H + c];"),
    "down_first_term_dropped": ("for (int i = 0; i < I; ++i) acc = acc + a[i] * wd[i];",
                                "for (int i = 1; i < I; ++i) acc = acc + a[i] * wd[i];"),
    "combine_single_weight": ("s = s + w[(size_t)t * k + j] * y[",
                              "s = s + w[(size_t)t * k] * y["),
    "combine_drops_shared": ("out[(size_t)t * H + c] = shared ? shared[(size_t)t * H + c] + s : s;",
                             "out[(size_t)t * H + c] = s;"),
    "mx_emax_7": ("s = ex - 1 - 8;", "s = ex - 1 - 7;"),
    "mx_round_half_up": ("ldexp(nearbyint(ldexp(a, 3 - E)), E - 3)",
                         "ldexp(floor(ldexp(a, 3 - E) + 0.5), E - 3)"),
    "mx_no_saturation": ("if (r > 448.0) r = 448.0;", "if (r > 480.0) r = 480.0;"),
    "mx_scale_bias": ("scales[r * nb + b] = (uint8_t)(s + 127);",
                      "scales[r * nb + b] = (uint8_t)(s + 128);"),
    "mx_subnormal_spacing": ("if (E < -6) E = -6;\n    }", "if (E < -7) E = -7;\n    }"),
    "mx_sign_dropped": ("const uint8_t sign = signbit(v) ? 0x80 : 0x00;",
                        "const uint8_t sign = 0x00;"),
    "mx_dequant_scale_off": ("(int)scales[r * nb + i / 32] - 127", "(int)scales[r * nb + i / 32] - 126"),
    "mx_subnormal_decode": ("mag = ldexp((double)m, -9);", "mag = ldexp(8.0 + m, -10);"),
    "mx_zero_block_scale": ("int s = -127;\n            if (amax > 0.0)", "int s = 0;\n            if (amax > 0.0)"),
    "wfi_sum_short": ("if (e < 0 || e >= E) { bad = 1; break; }\n                s = s + z[e] / S;",
                      "if (e < 0 || e >= E) { bad = 1; break; }\n                if (j + 1 < k) s = s + z[e] / S;"),
    "wfi_renorm_dropped": ("w[(size_t)t * k + j] = renorm ? p / s : p;",
                           "w[(size_t)t * k + j] = p;"),
    "wfi_first_id_only": ("const float p = z[e] / S;", "const float p = z[ids[(size_t)t * k]] / S;"),
    "permute_unstable": ("for (int t = 0; t < T; ++t) {\n        for (int j = 0; j < k; ++j) {\n            const long a",
                         "for (int t = T - 1; t >= 0; --t) {\n        for (int j = 0; j < k; ++j) {\n            const long a"),
}

RUNNER = r"""
import json, sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
res = oracle_pins.run_all(oracle.Oracle({lib!r}))
print("RESULT" + json.dumps(res))
"""


def _battery(lib_path):
    cp = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib_path)],
                        capture_output=True, text=True, timeout=300)
    for line in cp.stdout.splitlines():
        if line.startswith("RESULT"):
            return json.loads(line[6:])
    return {"process": f"exit {cp.returncode}: {cp.stderr[-400:]}"}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


def test_unmodified_source_passes_battery(source, tmp_path):
    lib = oracle.build_from_source_text(source, str(tmp_path))
    res = _battery(lib)
    assert all(v is None for v in res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, name, tmp_path):
    find, repl = MUTANTS[name]
    assert source.count(find) == 1, f"mutation anchor for {name} not unique"
    lib = oracle.build_from_source_text(source.replace(find, repl), str(tmp_path))
    res = _battery(lib)
    failed = [k for k, v in res.items() if v is not None]
    assert failed, f"no pin caught mutant {name}"
