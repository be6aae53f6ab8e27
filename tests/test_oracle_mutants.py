"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of oracle/moe_oracle.c
(a dropped term, a wrong sign, index, rounding mode or comparison), builds
it, and runs the oracle pin suite against that build in a subprocess.  The
suite must fail for every planted mistake.  Nothing here touches the GPU
library.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact text in the oracle, replacement); each text must occur once
MUTANTS = [
    ("replica_index", "1 + (i % n)", "1 + (k % n)"),
    ("prune_compare", "scores[f] < thr[k]", "scores[f] <= thr[k]"),
    ("mask1d_rule", "token_mask[i] && !token_mask[i - 1]", "!token_mask[i] && token_mask[i - 1]"),
    ("unstable_order", "for (int f = 0; f < N; ++f) {\n        if (act[f]) {",
     "for (int f = N - 1; f >= 0; --f) {\n        if (act[f]) {"),
    ("scan_short_total", "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = offsets[e] + counts[e] - (e == E - 1 && counts[e] > 0);"),
    ("histogram_drops_first", "counts[ids[f]] += 1;", "counts[ids[f]] += (f > 0);"),
    ("int8_truncate", "float r = (w != w) ? 0.0f : nearbyintf(w);",
     "float r = (w != w) ? 0.0f : truncf(w);"),
    ("int8_scale_direction", "*scale = 1.0f / d;", "*scale = d;"),
    ("int8_no_abs", "float a = fabsf(v[j]);\n        if (a > m)\n            m = a;\n    }\n    if (m == 0.0f) {",
     "float a = v[j];\n        if (a > m)\n            m = a;\n    }\n    if (m == 0.0f) {"),
    ("int8_dst_max", "float d = 127.0f / m;", "float d = 128.0f / m;"),
    ("mx_emax", "se = ilogbf(m) - 8;", "se = ilogbf(m) - 7;"),
    ("mx_scale_direction", "*scale_byte = (uint8_t)(se + 127);", "*scale_byte = (uint8_t)(127 - se);"),
    ("e4m3_no_saturation", "return s | 0x7E;", "return s | 0x7F;"),
    ("e4m3_ties_away", "int q = (int)nearbyintf(ldexpf(a, 3 - e));", "int q = (int)roundf(ldexpf(a, 3 - e));"),
    ("e4m3_bias", "(e + 7) * 8 + (q - 8)", "(e + 8) * 8 + (q - 8)"),
    ("bf16_ties_away", "r = ldexp(nearbyint(ldexp(a, -q)), q);", "r = ldexp(floor(ldexp(a, -q) + 0.5), q);"),
    ("shared_weight_one", "double w = shared_mode == 0 ? ws : 1.0;", "double w = 1.0;"),
    ("residual_dropped", "xf[h] += (double)bf16_value(residual[(size_t)i * H + h]);",
     "xf[h] += 0.0 * (double)bf16_value(residual[(size_t)i * H + h]);"),
    ("rms_mean_n_minus_1", "sqrt(ss / H + (double)eps)", "sqrt(ss / (H - 1) + (double)eps)"),
    ("eps_outside_sqrt", "1.0 / sqrt(ss / H + (double)eps)", "1.0 / (sqrt(ss / H) + (double)eps)"),
    ("gamma_dropped", "xf[h] * rstd * (double)bf16_value(gamma[h])", "xf[h] * rstd"),
    ("static_clamp_symmetric", "if (r < -128.0f)\n        r = -128.0f;",
     "if (r < -127.0f)\n        r = -127.0f;"),
    ("static_truncate", "    float r = nearbyintf(v);\n    if (r > 127.0f)",
     "    float r = truncf(v);\n    if (r > 127.0f)"),
    ("expert_row_of_column", "s = qscales[(size_t)e * H + j];",
     "s = qscales[(size_t)(f % K) * H + j];"),
    ("smoothing_dropped", "v[j] = qscales_kind == 0 ? bf16_value(xi[j]) : bf16_value(xi[j]) * s;",
     "v[j] = bf16_value(xi[j]);"),
    ("static_row_index", "s = qscales[j];", "s = qscales[H - 1 - j];"),
    ("swiglu_gate_up_swapped", "double g = bf16_value(row[j]), u = bf16_value(row[I + j]);",
     "double u = bf16_value(row[j]), g = bf16_value(row[I + j]);"),
    ("swiglu_sigmoid_sign", "a[j] = bf16_from_double(g / (1.0 + exp(-g)) * u);",
     "a[j] = bf16_from_double(g / (1.0 + exp(g)) * u);"),
    ("static_e4m3_nan_signed", "    if (v != v)\n        return 0x7F;\n    return e4m3_from_float(v);",
     "    return e4m3_from_float(v);"),
    ("static_e4m3_unscaled", "c[j] = e4m3_static_cast(v[j]);",
     "c[j] = e4m3_static_cast(bf16_value(xi[j]));"),
    ("pruned_weight_counted", "int r = assist[i * K + k];\n                if (r < 0)\n                    continue;\n                double s = scales[i * K + k];\n                ws += s;",
     "int r = assist[i * K + k];\n                double s = scales[i * K + k];\n                ws += s;\n                if (r < 0)\n                    continue;"),
    ("e4m3_decode_bias", "v = ldexp(8.0 + m, ef - 10);", "v = ldexp(8.0 + m, ef - 9);"),
    ("e4m3_decode_subnormal", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e8m0_bias", "ldexp(1.0, (int)c - 127)", "ldexp(1.0, (int)c - 128)"),
    ("gemm_act_scale_block", "a_sc[(size_t)r * nb + k / 32]", "a_sc[(size_t)r * nb + (k / 32 + 1) % nb]"),
    ("gemm_weight_scale_row", "wse[(size_t)n * nb + k / 32]", "wse[(size_t)(n / 2) * nb + k / 32]"),
    ("gemm_wrong_instance", "const uint8_t *we = w + (size_t)e * N * Kd;",
     "const uint8_t *we = w + (size_t)((e + 1) % E) * N * Kd;"),
    ("gemm_transposed_weights", "e4m3_value(we[(size_t)n * Kd + k])", "e4m3_value(we[(size_t)k * N + n])"),
    ("gemm_extra_row", "(size_t)e * N * nb;\n        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {",
     "(size_t)e * N * nb;\n        for (int r = offsets[e]; r <= offsets[e + 1] && r < rows; ++r) {"),
    ("i8_tile_index", "a_sc[(size_t)r * n_tiles + t]", "a_sc[(size_t)r * n_tiles + (t + 1) % n_tiles]"),
    ("i8_weight_scale_column", "w_sc[(size_t)e * N + n]", "w_sc[(size_t)e * N + (n + 1) % N]"),
    ("i8_tile_bounds", "for (int k = t * tl; k < (t + 1) * tl; ++k)",
     "for (int k = t * tl; k < (t + 1) * tl - 1; ++k)"),
    ("i8_unsigned_codes", "(int64_t)a[(size_t)r * Kd + k]", "(int64_t)(uint8_t)a[(size_t)r * Kd + k]"),
    ("i8_extra_row", "const int8_t *we = w + (size_t)e * N * Kd;\n        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {",
     "const int8_t *we = w + (size_t)e * N * Kd;\n        for (int r = offsets[e]; r <= offsets[e + 1] && r < rows; ++r) {"),
    ("i8_wrong_instance", "const int8_t *we = w + (size_t)e * N * Kd;",
     "const int8_t *we = w + (size_t)((e + 1) % E) * N * Kd;"),
]

PIN_FILES = ["tests/test_oracle_numbers.py", "tests/test_oracle_route.py",
             "tests/test_oracle_dispatch_combine.py", "tests/test_oracle_scaled.py",
             "tests/test_oracle_gemm.py", "tests/test_oracle_swiglu.py", "tests/test_golden.py"]


def _run_mutant(name, old, new, workdir):
    """Build the oracle with one planted mistake and run the pin suite on it;
    returns (pytest return code, tail of its output)."""
    src = open(obuild.SRC).read()
    if src.count(old) != 1:
        return -1, f"mutation site for {name} not unique/present"
    mut_src = os.path.join(workdir, f"moe_oracle_{name}.c")
    with open(mut_src, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, f"libmoe_oracle_{name}.so")
    obuild.build(src=mut_src, lib=lib)
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant's pin-suite run, several at a time (each is a subprocess)."""
    from concurrent.futures import ThreadPoolExecutor
    workdir = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {m[0]: ex.submit(_run_mutant, *m, workdir) for m in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, mutant_results):
    rc, out = mutant_results[name]
    assert rc != -1, out
    assert rc == 1, f"pins did not catch mutant {name}:\n{out}"
