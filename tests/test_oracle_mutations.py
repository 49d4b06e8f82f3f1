"""Planted mistakes in the oracle must be caught by its pins.

Each case edits one plausible mistake into a copy of the oracle's C source
(dropped term, wrong sign, wrong index, transposed operand, broken rounding,
broken stability, a wrong MX scale index, exponent or bias, a dropped clamp,
term or slope of the clamped activation, an ignored, unsigned or wrongly indexed int8
token scale, and in the backward a wrong derivative sign, a dropped routing
weight, a transposed index or swapped gate/up rows), builds it, and runs the CPU pin tests against it in a
subprocess; the run must fail.  The product path is not involved.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = {
    "gate_up_swapped": ("e, d_e + r, c) * xv", "e, r, c) * xv"),
    "routing_weight_dropped": ("R(wt * y[n], f64)", "y[n]"),
    "silu_sign": ("expf((float)-g)", "expf((float)g)"),
    "w2_transposed": ("d_h, d_e, e, n, r)", "d_h, d_e, e, r, n)"),
    "requant_scale_240": ("amax / 448.0", "amax / 240.0"),
    "scatter_unstable": ("pos[p] = offsets[id] + seen[id];", "pos[p] = offsets[id] + counts[id] - 1 - seen[id];"),
    "no_padding": ("padded_offsets[e] + tiles * bm", "padded_offsets[e] + counts[e]"),
    "bf16_truncates": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "e4m3_bias_8": ("ex - 7)", "ex - 8)"),
    "first_slot_skipped": ("for (j = 0; j < k; ++j)", "for (j = 1; j < k; ++j)"),
    "x_scale_block_ignored": ("xs)[t * (d_h / QBLK) + c / QBLK]", "xs)[t * (d_h / QBLK)]"),
    "w_scale_col_block_ignored": ("* (cols / QBLK) + c / QBLK]", "* (cols / QBLK)]"),
    "mx_x_scale_block_ignored": ("xs)[t * (d_h / MXBLK) + c / MXBLK]", "xs)[t * (d_h / MXBLK)]"),
    "mx_w_scale_row_ignored": ("[(e * rows + r) * (cols / MXBLK) + c / MXBLK]", "[(e * rows) * (cols / MXBLK) + c / MXBLK]"),
    "mx_shared_exponent_off_by_one": ("b = ex - 1 - 8 + 127;", "b = ex - 8 + 127;"),
    "e8m0_bias_128": ("ldexp(1.0, (int)s - 127)", "ldexp(1.0, (int)s - 128)"),
    "act_gate_clamp_dropped": ("if (g > ACT_LIMIT) g = ACT_LIMIT;", ""),
    "act_up_lower_clamp_dropped": ("if (u < -ACT_LIMIT) u = -ACT_LIMIT;", ""),
    "act_plus_one_dropped": ("R(u + 1.0, f64)", "u"),
    "act_alpha_one": ("R((double)ACT_ALPHA * g, f64)", "g"),
    "int8_scale_ignored": ("((const int8_t*)x)[t * d_h + c] * ((const float*)xs)[t], f64)",
                           "((const int8_t*)x)[t * d_h + c], f64)"),
    "int8_read_unsigned": ("((const int8_t*)x)[t * d_h + c]", "((const uint8_t*)x)[t * d_h + c]"),
    "int8_scale_by_column": ("((const float*)xs)[t], f64)", "((const float*)xs)[c % 8], f64)"),
    "bwd_dsilu_sign": ("R(1.0 - sig, f64)", "R(1.0 + sig, f64)"),
    "bwd_routing_weight_dropped": ("double dh = R(wt * q[r], f64)", "double dh = q[r]"),
    "bwd_dw2_unweighted": ("double dy = R(wt * oracle_bf16_decode(dout[t * d_h + n]), f64);",
                           "double dy = oracle_bf16_decode(dout[t * d_h + n]);"),
    "bwd_dx_up_uses_gate_rows": ("R(du[r] * ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, d_e + r, c), f64)",
                                 "R(du[r] * ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, r, c), f64)"),
    "bwd_dw2_transposed_index": ("i = (e * d_h + n) * d_e + r;", "i = (e * d_h + r) * d_e + n;"),
    "bwd_dtopk_uses_dh": ("dsum = R(dsum + R(q[r] * h[r], f64), f64);", "dsum = R(dsum + R(wt * q[r] * h[r], f64), f64);"),
}

PIN_TESTS = ["tests/test_oracle_codecs.py", "tests/test_oracle_routing.py", "tests/test_oracle_forward.py",
             "tests/test_oracle_activation.py", "tests/test_oracle_backward.py"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", str(c),
                    "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
