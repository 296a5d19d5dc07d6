"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutant is a copy of oracle/zs_oracle.c with one plausible mistake
(a dropped term, a wrong sign, index or slot, a swapped operand, a changed
summation order or precision), compiled with the same gcc flags into a temp
directory.  The pins in ``pins.py`` are then run against it; a mutant that
passes every pin would mean the pins cannot tell that mistake apart from the
intended arithmetic.
"""
import os
import subprocess
import sys

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "zs_oracle.c")

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("fwd_sign", "o[c] = o[c] + msg;", "o[c] = o[c] - msg;", 0),
    ("fwd_fma", "const float msg = w * rad[c];\n                    o[c] = o[c] + msg;",
     "o[c] = __builtin_fmaf(w, rad[c], o[c]);", 0),
    ("fwd_slot", "const float *rad = radial + (e * 3 + (l - 1)) * C;",
     "const float *rad = radial + (e * 3 + (3 - l)) * C;", 0),
    ("fwd_coupling_col", "const float w = coupling[e * ZS_ORACLE_ZONAL + (r - 1)];",
     "const float w = coupling[e * ZS_ORACLE_ZONAL + (15 - r)];", 0),
    ("fwd_drop_last_m", "for (int m = -l; m <= l; ++m) {\n                const int r = l * l + l + m;\n"
     "                const float w", "for (int m = -l; m < l; ++m) {\n                const int r = l * l + l + m;\n"
     "                const float w", 0),
    ("fwd_row_shift", "float *o = out + (n * ZS_ORACLE_ROWS + r) * C;",
     "float *o = out + (n * ZS_ORACLE_ROWS + r - 1) * C;", 0),
    ("fwd_neg_zero_init", "out[i] = 0.0f;", "out[i] = -0.0f;", 0),
    ("fwd_skip_first_edge", "for (int64_t e = 0; e < E; ++e) {\n        const int64_t n = dst[e];\n"
     "        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {\n            const float *rad",
     "for (int64_t e = 1; e < E; ++e) {\n        const int64_t n = dst[e];\n"
     "        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {\n            const float *rad", 0),
    ("fwd_reverse_edges", "for (int64_t e = 0; e < E; ++e) {\n        const int64_t n = dst[e];\n"
     "        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {\n            const float *rad",
     "for (int64_t e = E - 1; e >= 0; --e) {\n        const int64_t n = dst[e];\n"
     "        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {\n            const float *rad", 0),
    ("fwd64_sign", "o[c] = o[c] + w * (double)rad[c];", "o[c] = o[c] - w * (double)rad[c];", 0),
    ("nodes_slot", "const float *rad = radial + (e * 3 + (l - 1)) * C;",
     "const float *rad = radial + (e * 3 + (3 - l)) * C;", 1),
    ("bwd_radial_order", "for (int m = -l; m <= l; ++m) {\n                const int r = l * l + l + m;\n"
     "                const float p", "for (int m = l; m >= -l; --m) {\n                const int r = l * l + l + m;\n"
     "                const float p", 0),
    ("bwd_radial_wrong_col", "coupling[e * ZS_ORACLE_ZONAL + (r - 1)];\n                acc = acc + p;",
     "coupling[e * ZS_ORACLE_ZONAL + (r % 15)];\n                acc = acc + p;", 0),
    ("bwd_grad_row0", "const float p = grad_out[(n * ZS_ORACLE_ROWS + r) * C + c] *",
     "const float p = grad_out[(n * ZS_ORACLE_ROWS + r - 1) * C + c] *", 0),
    ("bwd_coupling_fp32_sum", "double s = 0.0;\n            for (int64_t c = 0; c < C; ++c)\n"
     "                s = s + (double)g[c] * (double)rad[c];\n            gc_row[r - 1] = (float)s;",
     "float s = 0.0f;\n            for (int64_t c = 0; c < C; ++c)\n"
     "                s = s + g[c] * rad[c];\n            gc_row[r - 1] = s;", 0),
    ("bwd_coupling_wrong_slot", "const float *rad = radial + (e * 3 + (l - 1)) * C;",
     "const float *rad = radial + (e * 3 + (l % 3)) * C;", 2),
    ("bwd_node_is_edge", "backward_one_edge_f32(grad_out, coupling, radial, e, dst[e], C,\n"
     "                              grad_coupling",
     "backward_one_edge_f32(grad_out, coupling, radial, e, e % N, C,\n"
     "                              grad_coupling", 0),
    ("bwd64_transpose", "(double)coupling[e * ZS_ORACLE_ZONAL + (r - 1)];\n                }\n"
     "                grad_radial", "(double)coupling[e * ZS_ORACLE_ZONAL + (15 - r)];\n                }\n"
     "                grad_radial", 0),
    ("csr_off_by_one", "rowptr[dst[e] + 1] += 1;", "rowptr[dst[e]] += 1;", 0),
    ("csr_unstable", "for (int64_t e = 0; e < E; ++e)          /* increasing e keeps ties stable */",
     "for (int64_t e = E - 1; e >= 0; --e)", 0),
    ("norm_grad_factor", "(float)(-0.5 * t * t * t * s)", "(float)(-1.0 * t * t * t * s)", 0),
    ("norm_grad_power", "(float)(-0.5 * t * t * t * s)", "(float)(-0.5 * t * t * s)", 0),
    ("norm_grad_unscaled", "grad_y[n * ZS_ORACLE_ROWS * C + i] * norm[n];",
     "grad_y[n * ZS_ORACLE_ROWS * C + i];", 0),
    ("norm_not_inverse", "norm[n] = 1.0f / root;", "norm[n] = root;", 0),
    ("norm_counts_edges", "norm[dst[e]] = norm[dst[e]] + env[e];",
     "norm[dst[e]] = norm[dst[e]] + 1.0f;", 0),
    ("norm_y_unscaled", "y[n * ZS_ORACLE_ROWS * C + i] = out[n * ZS_ORACLE_ROWS * C + i] * norm[n];",
     "y[n * ZS_ORACLE_ROWS * C + i] = out[n * ZS_ORACLE_ROWS * C + i];", 0),
    ("no_index_check", "if (dst[e] < 0 || dst[e] >= N)\n            return -3;",
     "if (dst[e] < 0 && dst[e] >= N)\n            return -3;", 0),
]


def _apply(src, old, new, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


_RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
orc = oracle.Oracle({lib!r})
caught = []
for pin in pins.ALL_PINS:
    try:
        pin(orc)
    except Exception as exc:
        caught.append(pin.__name__)
print("CAUGHT", " ".join(caught))
sys.exit(3 if caught else 0)
"""


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    mutated = _apply(src, old, new, occ)
    assert mutated != src
    c_path = tmp_path / f"{name}.c"
    c_path.write_text(mutated)
    lib = oracle.build(force=True, src=str(c_path), out=str(tmp_path / f"lib{name}.so"))
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests_dir), tests=tests_dir, lib=lib)
    # a separate process: a mutant that writes out of bounds may crash it,
    # which also counts as caught
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"mutant {name} passes every pin:\n{res.stdout}{res.stderr}"
