"""Plants plausible mistakes in copies of the oracle and checks that the pins catch each.

Every mutant is a one-line textual change to oracle/conv_oracle.c, compiled
with gcc into a temporary library; the pin suite (test_oracle_pins.py) is then
run against it in a child process and must fail.  The real oracle is never
modified.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "conv_oracle.c")

MUTANTS = {
    "flipped_kernel": ("w_at(s, wt, co, kd, kh, kw, c)",
                       "w_at(s, wt, co, s->k_d - 1 - kd, s->k_h - 1 - kh, s->k_w - 1 - kw, c)"),
    "pad_sign": ("oh * s->s_h - s->p_h + kh", "oh * s->s_h + s->p_h + kh"),
    "stride_on_tap": ("ow * s->s_w - s->p_w + kw", "ow - s->p_w + kw * s->s_w"),
    "ceil_extent": ("return span / s + 1;", "return (span + s - 1) / s + 1;"),
    "drops_first_column": ("if (w < 0 || w >= s->w) return 0.0;", "if (w < 1 || w >= s->w) return 0.0;"),
    "drops_last_channel": ("for (int64_t c = 0; c < cg; ++c)", "for (int64_t c = 0; c < cg - 1; ++c)"),
    "transposed_weight_taps": ("(((co * s->k_d + kd) * s->k_h + kh) * s->k_w + kw)",
                               "(((co * s->k_d + kd) * s->k_w + kw) * s->k_h + kh)"),
    "row_decode_mixup": ("const int64_t oh = (m / ow_n) % oh_n;", "const int64_t oh = (m / oh_n) % oh_n;"),
    "float_accumulator": ("double acc = 0.0;", "float acc = 0.0f;"),
    "drops_depth_padding": ("if (d < 0 || d >= s->d) return 0.0;", "if (d >= s->d) return 0.0;"),
    # the variants: dilation, groups, asymmetric padding
    "dilation_ignored_along_w": ("ow * s->s_w - s->p_w + kw * s->e_w", "ow * s->s_w - s->p_w + kw"),
    "dilation_on_the_stride": ("od * s->s_d - s->p_d + kd * s->e_d", "od * s->s_d * s->e_d - s->p_d + kd"),
    "dilation_missing_in_extent": ("int64_t span = in + p + q - (e * (k - 1) + 1);",
                                   "int64_t span = in + p + q - k;"),
    "high_pad_taken_as_low": ("int64_t span = in + p + q - (e * (k - 1) + 1);",
                              "int64_t span = in + 2 * p - (e * (k - 1) + 1);"),
    "group_channel_offset_dropped": ("g * cg + c)", "c)"),
    "group_of_output_interleaved": ("const int64_t g = co / og;", "const int64_t g = co % s->groups;"),
    "filter_channel_stride_ungrouped": ("* (s->c_in / s->groups) + c]", "* s->c_in + c]"),
    # backward-data
    "bwd_no_divisibility_check": ("if (td < 0 || td % s->s_d != 0 || td / s->s_d >= od_n) continue;",
                                  "if (td < 0 || td / s->s_d >= od_n) continue;"),
    "bwd_forward_index_sign": ("const int64_t th = ih + s->p_h - kh * s->e_h;",
                               "const int64_t th = ih - s->p_h + kh * s->e_h;"),
    "bwd_output_group_ignored": ("for (int64_t co = g * og; co < (g + 1) * og; ++co)",
                                 "for (int64_t co = 0; co < og; ++co)"),
    "bwd_dilation_ignored": ("const int64_t tw = iw + s->p_w - kw * s->e_w;",
                             "const int64_t tw = iw + s->p_w - kw;"),
    "bwd_high_edge_off_by_one": ("td / s->s_d >= od_n", "td / s->s_d > od_n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "conv_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutated),
                    "-o", str(lib)], check=True)
    env = dict(os.environ, ORACLE_CONV_LIB=str(lib), OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout[-2000:]}"
