"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins in test_oracle_pins.py catch every one of them.

Each mutant is a one-line textual change of oracle/wanattn_oracle.c: a
flipped sign, a swapped index, a dropped term, a transposed operand, a wrong
segment width, an off-by-one in a mask.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "wanattn_oracle.c")

MUTANTS = {
    "rotation_sign": ("y[2 * c] = re * cr - im * ci;", "y[2 * c] = re * cr + im * ci;"),
    "pair_swapped": ("double re = x[2 * c], im = x[2 * c + 1];", "double im = x[2 * c], re = x[2 * c + 1];"),
    "omega_over_head_dim": ("orc_omega(theta, dims[a], k)", "orc_omega(theta, head_dim, k)"),
    "axis_width": ("dims[1] = 2 * s;", "dims[1] = 2 * s + 2;"),
    "decode_height": ("pos[1] = (n / W) % H;", "pos[1] = n % H;"),
    "causal_strict": ("return (fj / chunk_frames) <= (fi / chunk_frames);",
                      "return (fj / chunk_frames) < (fi / chunk_frames) || fj == fi;"),
    "scale_dropped": ("    s *= scale;\n", "\n"),
    "denominator_dropped": ("den += srow[j];", "den += 1.0;"),
    "value_is_key": ("out[e] += p * vmat[(size_t)j * head_dim + e];",
                     "out[e] += p * kmat[(size_t)j * head_dim + e];"),
    "keys_not_rotated": ("      if (t->rope) {\n        int pos[3];\n        orc_decode(j,",
                         "      if (0) {\n        int pos[3];\n        orc_decode(j,"),
    "kv_len_off_by_one": ("allowed[j] = (j < kvl)", "allowed[j] = (j <= kvl && j < nk)"),
    "offset_axis_mixup": ("pos[1] + h0, pos[2] + w0, theta);", "pos[1] + w0, pos[2] + w0, theta);"),
    "cross_rotated": ("  t.rope = 0;\n", "  t.rope = 1;\n"),
    "bf16_widening": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "max_starts_at_zero": ("double m = -INFINITY;", "double m = 0.0;"),
    "kv_keys_take_query_offset": ("pos[0] + t->kf0, pos[1] + t->kh0", "pos[0] + t->f0, pos[1] + t->kh0"),
    "kv_query_offset_dropped": ("  t.f0 = qf0;\n", "  t.f0 = 0;\n"),
    "ln_unbiased_variance": ("    var /= dim;\n", "    var /= (dim - 1);\n"),
    "modulation_sign": ("* (1.0 + (double)t->e1", "* (1.0 - (double)t->e1"),
    "rms_gamma_dropped": ("x[i] = x[i] * inv * bf16_value(g[i]);", "x[i] = x[i] * inv;"),
    "projection_bias_dropped": ("double acc = bf16_value(b[o]);", "double acc = 0.0;"),
    "jitter_head_off_by_one": ("t->head_theta ? t->head_theta[hd] : t->theta;",
                               "t->head_theta ? t->head_theta[(hd + 1) % t->heads] : t->theta;"),
    "jitter_ignored": ("t->head_theta ? t->head_theta[hd] : t->theta;",
                       "t->head_theta ? t->head_theta[0] : t->theta;"),
    "kv_jitter_one_base": ("h0, w0, 0.0, theta_heads,", "h0, w0, theta_heads[0], 0,"),
    "jitter_keys_unjittered": ("pos[1] + t->kh0, pos[2] + t->kw0, th);", "pos[1] + t->kh0, pos[2] + t->kw0, 1e4);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(lib),
                           str(mutated), "-lm"])
    env = dict(os.environ, WANATTN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
