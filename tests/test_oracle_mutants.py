"""Plant plausible mistakes in copies of the C oracle, on the CPU, and require
that the pins catch every one of them.  Each mutant runs in its own process,
so that a mutant which crashes cannot take the test run down with it (a crash
counts as caught)."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "das_oracle.c")

# (name, text in das_oracle.c, replacement): first occurrence only.
MUTANTS = [
    ("lse_drops_max", "lse[(size_t)b * Hq + h] = M + log(Z);", "lse[(size_t)b * Hq + h] = log(Z);"),
    ("exp_wrong_sign", "w[j] = exp(w[j] - M);", "w[j] = exp(w[j] + M);"),
    ("max_wrong_compare", "if (w[j] > M) M = w[j];", "if (w[j] < M) M = w[j];"),
    ("gqa_modulo_mapping", "const int g = h / G;", "const int g = h % Hkv;"),
    ("no_normalisation", "for (int d = 0; d < D; ++d) o[d] /= Z;", ""),
    ("batch_offset_dropped", "const uint16_t* kbase = k + ((size_t)b * Hkv + g)",
     "const uint16_t* kbase = k + ((size_t)0 * Hkv + g)"),
    ("scale_dropped", "return scale * dot;", "return dot;"),
    ("key_d_reversed", "dot += widen_bf16(qrow[d]) * widen_bf16(krow[d]);",
     "dot += widen_bf16(qrow[d]) * widen_bf16(krow[D - 1 - d]);"),
    ("value_rows_reversed", "const uint16_t* vrow = vbase + (size_t)j * D;\n        for (int d = 0; d < D; ++d) o[d] += w[j]",
     "const uint16_t* vrow = vbase + (size_t)(L - 1 - j) * D;\n        for (int d = 0; d < D; ++d) o[d] += w[j]"),
    ("value_weight_dropped", "o[d] += w[j] * vterm(widen_bf16(vrow[d]), absv);",
     "o[d] += vterm(widen_bf16(vrow[d]), absv);"),
    ("merge_lse_drops_max", "const double lse = mx + log(exp(a - mx) + exp(b - mx));",
     "const double lse = log(exp(a - mx) + exp(b - mx));"),
    ("merge_weights_swapped", "const double wa = exp(a - lse), wb = exp(b - lse);",
     "const double wa = exp(b - lse), wb = exp(a - lse);"),
    ("split_factor_wrong_sign", "exp(m_c[c] - M);", "exp(M - m_c[c]);"),
    ("split_sum_unscaled", "Lsum += f * l_c[c];", "Lsum += l_c[c];"),
    ("e4m3_bias_8", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3_subnormal_as_normal", "v = ldexp((double)m, -9);", "v = ldexp(1.0 + (double)m / 8.0, -6);"),
    ("e4m3_no_nan", "if (e == 15 && m == 7) return NAN;", ""),
    ("e4m3_mantissa_over_16", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 16.0, e - 7);"),
    ("fp8_k_scale_dropped", "(ks * e4m3[krow[d]])", "e4m3[krow[d]]"),
    ("fp8_v_scale_from_k", "vterm(vs * e4m3[vrow[d]], absv)", "vterm(ks * e4m3[vrow[d]], absv)"),
    ("fp8_scale_first_head", "const double ks = (double)k_scale[g]", "const double ks = (double)k_scale[0]"),
    ("int4_unsigned", "return n >= 8 ? n - 16 : n;", "return n;"),
    ("int4_high_nibble_first", "const int n = high ? (byte >> 4) : (byte & 15);",
     "const int n = high ? (byte & 15) : (byte >> 4);"),
    ("int4_sign_off_by_one", "return n >= 8 ? n - 16 : n;", "return n >= 8 ? n - 15 : n;"),
    ("int4_scale_per_head", "const double ks = (double)k_scale[slab + j];",
     "const double ks = (double)k_scale[slab];"),
    ("int4_v_scale_from_k", "const double vs = (double)v_scale[slab + j];",
     "const double vs = (double)k_scale[slab + j];"),
    ("int4_v_scale_row_shift", "const double vs = (double)v_scale[slab + j];",
     "const double vs = (double)v_scale[slab + (j + 1) % L];"),
    ("int4_byte_index", "dot += widen_bf16(qrow[d]) * (ks * (double)int4_value(krow[d / 2], d & 1));",
     "dot += widen_bf16(qrow[d]) * (ks * (double)int4_value(krow[d % row_bytes], d & 1));"),
    ("magnitude_without_abs", "return absv ? fabs(x) : x;", "return x;"),
    ("magnitude_always_abs", "return absv ? fabs(x) : x;", "return fabs(x);"),
    ("magnitude_int4_abs_of_code_only",
     "o[d] += w[j] * vterm(vs * (double)int4_value(vrow[d / 2], d & 1), absv);",
     "o[d] += w[j] * vs * vterm((double)int4_value(vrow[d / 2], d & 1), absv);"),
    ("split_chunk_off_by_one", "const int j1 = (j0 + chunk < L) ? j0 + chunk : L;",
     "const int j1 = (j0 + chunk < L) ? j0 + chunk - 1 : L;"),
]


def _run_mutant(tmp, name, old, new):
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found"
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as fh:
        fh.write(text.replace(old, new, 1))
    lib = oracle.build(src=path, out=os.path.join(tmp, name + ".so"))
    env = dict(os.environ, OMP_NUM_THREADS="2", PYTHONPATH=os.pathsep.join([HERE, os.path.dirname(HERE)]))
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                       capture_output=True, text=True, env=env, timeout=300)
    return name, r.returncode, (r.stdout + r.stderr)[-400:]


def test_unmutated_copy_passes_all_pins():
    with tempfile.TemporaryDirectory() as tmp:
        name, rc, out = _run_mutant(tmp, "identity", "return scale * dot;", "return scale * dot;")
    assert rc == 0, out


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            results = list(ex.map(lambda m: _run_mutant(tmp, *m), MUTANTS))
    missed = [(n, out) for n, rc, out in results if rc == 0]
    assert not missed, f"mistakes the pins did not catch: {missed}"
