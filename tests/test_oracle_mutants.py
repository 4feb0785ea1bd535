"""Plant plausible mistakes in copies of oracle.c (on the CPU) and check that
every one of them fails at least one pin.  This shows the pins constrain each
part of the oracle: direction of A_w, operand roles, signs, the weight factor,
stability and column fill of the lowering, the scale S, and the degree plan."""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "forward_scatters_to_source": ("y[dst[j] * h + k] += t;", "y[src[j] * h + k] += t;"),
    "forward_gathers_destination": ("double t = (double)w[j] * (double)x[src[j] * h + k];",
                                    "double t = (double)w[j] * (double)x[dst[j] * h + k];"),
    "forward_drops_weight": ("double t = (double)w[j] * (double)x[src[j] * h + k];",
                             "double t = (double)x[src[j] * h + k];"),
    "forward_wrong_sign": ("y[dst[j] * h + k] += t;", "y[dst[j] * h + k] -= t;"),
    "forward_scale_signed": ("s[dst[j] * h + k] += fabs(t);", "s[dst[j] * h + k] += t;"),
    "input_grad_scatters_to_destination": ("dx[src[j] * h + k] += t;", "dx[dst[j] * h + k] += t;"),
    "input_grad_gathers_source": ("double t = (double)w[j] * (double)dy[dst[j] * h + k];\n            dx[src",
                                  "double t = (double)w[j] * (double)dy[src[j] * h + k];\n            dx[src"),
    "edge_grad_swapped_rows": ("double t = (double)x[src[j] * h + k] * (double)dy[dst[j] * h + k];\n            acc += t;\n            sa += fabs(t);\n        }\n        dw[j] = acc;",
                               "double t = (double)x[dst[j] * h + k] * (double)dy[src[j] * h + k];\n            acc += t;\n            sa += fabs(t);\n        }\n        dw[j] = acc;"),
    "edge_grad_bad_init": ("double acc = 0.0, sa = 0.0;\n        for (k = 0; k < h; k++) {\n            double t = (double)x[src[j] * h + k] * (double)dy[dst[j] * h + k];\n            acc += t;\n            sa += fabs(t);\n        }\n        dw[j] = acc;",
                           "double acc = 1.0, sa = 0.0;\n        for (k = 0; k < h; k++) {\n            double t = (double)x[src[j] * h + k] * (double)dy[dst[j] * h + k];\n            acc += t;\n            sa += fabs(t);\n        }\n        dw[j] = acc;"),
    "lower_unstable_descending": ("for (j = 0; j < e; j++) {               /* ascending COO ordinal       */",
                                  "for (j = e - 1; j >= 0; j--) {"),
    "lower_col_from_key": ("col[p] = other[j];", "col[p] = key[j];"),
    "lower_rowptr_unshifted": ("rowptr[key[j] + 1] += 1;", "rowptr[key[j]] += 1;"),
    "plan_ascending_classes": ("for (c = 32; c >= 0; c--) {", "for (c = 0; c <= 32; c++) {"),
    "plan_class_off_by_one": ("class_count[k] += 1;", "class_count[k > 0 ? k - 1 : 0] += 1;"),
    "softmax_no_max_shift": ("        row_sum[dst[j]] += exp((double)s[j] - row_max[dst[j]]);",
                             "        row_sum[dst[j]] += exp((double)s[j]);"),
    "softmax_over_source_rows": ("        alpha[j] = exp((double)s[j] - row_max[dst[j]]) / row_sum[dst[j]];",
                                 "        alpha[j] = exp((double)s[j] - row_max[dst[j]]) / row_sum[dst[j] > 0 ? dst[j] - 1 : 0];"),
    "softmax_backward_sign": ("        ds[j] = (double)alpha[j] * ((double)dalpha[j] - row_dot[dst[j]]);",
                              "        ds[j] = (double)alpha[j] * ((double)dalpha[j] + row_dot[dst[j]]);"),
    "normalize_mean_by_out_degree": ("            out[j] = (double)in[j] / din[dst[j]];",
                                     "            out[j] = (double)in[j] / dout[dst[j]];"),
    "normalize_sym_squared": ("            out[j] = (double)in[j] / sqrt(dout[src[j]] * din[dst[j]]);",
                              "            out[j] = (double)in[j] / (dout[src[j]] * din[dst[j]]);"),
    "normalize_sym_swapped_ends": ("            out[j] = (double)in[j] / sqrt(dout[src[j]] * din[dst[j]]);",
                                   "            out[j] = (double)in[j] / sqrt(dout[dst[j]] * din[src[j]]);"),
    "heads_weight_head_major": ("double t = (double)w[j * k + c / hh] * (double)in[other[j] * h + c];",
                                "double t = (double)w[(c / hh) * e + j] * (double)in[other[j] * h + c];"),
    "heads_interleaved_columns": ("double t = (double)w[j * k + c / hh] * (double)in[other[j] * h + c];",
                                  "double t = (double)w[j * k + c % k] * (double)in[other[j] * h + c];"),
    "heads_forward_roles_swapped": ("return heads_aggregate(n, e, h, k, dst, src, w, x, nr, rows, y, s);",
                                    "return heads_aggregate(n, e, h, k, src, dst, w, x, nr, rows, y, s);"),
    "heads_edge_grad_strided": ("for (c = q * hh; c < (q + 1) * hh; c++) {",
                                "for (c = q; c < h; c += k) {"),
    "heads_edge_grad_transposed_out": ("            dw[i * k + q] = acc;",
                                       "            dw[q * count + i] = acc;"),
    "softmax_heads_head_major": ("            alpha[j * k + q] = exp((double)s[j * k + q] - row_max[dst[j] * k + q])",
                                 "            alpha[j * k + q] = exp((double)s[q * e + j] - row_max[dst[j] * k + q])"),
    "softmax_heads_shared_row_max": ("            if ((double)s[j * k + q] > row_max[dst[j] * k + q])\n                row_max[dst[j] * k + q] = (double)s[j * k + q];",
                                     "            if ((double)s[j * k + q] > row_max[dst[j] * k])\n                row_max[dst[j] * k] = (double)s[j * k + q];"),
    "softmax_backward_heads_row_dot_without_head": ("            row_dot[dst[j] * k + q] += t;",
                                                    "            row_dot[dst[j] * k] += t;"),
    "softmax_backward_row_dot_unweighted": ("        row_dot[dst[j]] += (double)alpha[j] * (double)dalpha[j];",
                                            "        row_dot[dst[j]] += (double)dalpha[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so_path), str(c_path),
                    "-lm"], check=True)
    # Run the pins in a child process: a mutant that corrupts memory must not
    # take the test runner down with it (a crash also counts as caught).
    code = (
        "import sys, oracle\n"
        "from tests.oracle_pins import ALL_PINS\n"
        "failed = []\n"
        f"with oracle.using_library({str(so_path)!r}):\n"
        "    for pin in ALL_PINS:\n"
        "        try:\n"
        "            pin()\n"
        "        except Exception:\n"
        "            failed.append(pin.__name__)\n"
        "print(' '.join(failed))\n"
        "sys.exit(0 if failed else 3)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                          text=True, timeout=600)
    assert proc.returncode != 3, f"mutant {name} passed every pin"
