"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of the oracle's C source, builds
it, and runs the oracle pin suite against that build in a subprocess: the
suite must fail.  Mistakes cover every step of the definition: the eps
placement, the mean's divisor, the square, the weight, the bfloat16 and
float16 rounding rules (ties, truncation, spacing, exponent bias, overflow),
the fused op's choice of normalised value, the saved rstd, and each term
of the backward, including the residual gradient of the fused op; for
LayerNorm, E4M3 and RMSNorm + RoPE, each step of their definitions (the RoPE
signs, the cos/sin roles, the pairing of each layout, the table row, and the
empty-table-row rule)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "addrms_oracle.c")
PINS = ["tests/test_oracle_bf16.py", "tests/test_oracle_fwd.py", "tests/test_oracle_bwd.py",
        "tests/test_oracle_layernorm.py", "tests/test_oracle_fp8.py", "tests/test_oracle_rope.py",
        "tests/test_oracle_mxfp4.py", "tests/test_oracle_f16.py"]

MUTANTS = {
    "eps_outside_root": ("1.0 / sqrt(ms + eps)", "1.0 / sqrt(ms) + eps"),
    "eps_dropped": ("1.0 / sqrt(ms + eps)", "1.0 / sqrt(ms)"),
    "divisor_n_minus_1": ("ss / (double)N", "ss / (double)(N > 1 ? N - 1 : 1)"),
    "abs_not_square": ("ss += h * h;", "ss += fabs(h);"),
    "weight_dropped": ("h * rs * load_elem(w, w_dt, j)", "h * rs"),
    "weight_wrong_index": ("h * rs * load_elem(w, w_dt, j)", "h * rs * load_elem(w, w_dt, N - 1 - j)"),
    "rstd_saved_inverted": ("store_elem(rstd, rstd_dt, i, rs);", "store_elem(rstd, rstd_dt, i, 1.0 / rs);"),
    "ties_away_from_zero": ("(fmod(lo / ulp, 2.0) == 0.0) ? lo : hi", "hi"),
    "truncating_round": ("if (a < mid)", "if (a < hi)"),
    "subnormal_spacing": ("ulp = 0x1p-133;", "ulp = 0x1p-134;"),
    "overflow_saturates": ("return (uint16_t)(sign | 0x7F80u);\n    f = (float)q;",
                           "q = bf16_max;\n    f = (float)q;"),
    "fused_normalises_x": ("return oracle_rmsnorm_fwd(res, res_dt,", "return oracle_rmsnorm_fwd(x, in_dt,"),
    "residual_subtracts": ("float s32 = xs + rs;", "float s32 = xs - rs;"),
    "bwd_sign_of_projection": ("rs * (g - xh * c)", "rs * (g + xh * c)"),
    "bwd_projection_not_averaged": ("c /= (double)N;", "c /= 1.0;"),
    "bwd_g_without_weight": ("double g = load_elem(dy, in_dt, i * N + j) * load_elem(w, w_dt, j);",
                             "double g = load_elem(dy, in_dt, i * N + j);"),
    "bwd_dx_without_weight": ("double g = d * load_elem(w, w_dt, j);", "double g = d;"),
    "bwd_dw_without_rstd": ("acc[j] += d * xh;", "acc[j] += d * load_elem(h, in_dt, i * N + j);"),
    "fused_bwd_drops_dres": ("rs * (g - xh * c) + extra);", "rs * (g - xh * c));"),
    "fused_bwd_subtracts_dres": ("rs * (g - xh * c) + extra);", "rs * (g - xh * c) - extra);"),
    "ln_unbiased_variance": ("double var = sq / (double)N;", "double var = sq / (double)(N > 1 ? N - 1 : 1);"),
    "ln_eps_outside_root": ("double rs = 1.0 / sqrt(var + eps);", "double rs = 1.0 / sqrt(var) + eps;"),
    "ln_no_centering": ("double d = load_elem(x, x_dt, i * N + j) - mu;", "double d = load_elem(x, x_dt, i * N + j);"),
    "ln_mean_divisor": ("double mu = sum / (double)N;", "double mu = sum / (double)(N + 1);"),
    "ln_bias_dropped": ("v += load_elem(b, w_dt, j);", "v += 0.0;"),
    "ln_bwd_no_mean_g": ("rs * (g - mg - xh * mgx)", "rs * (g - xh * mgx)"),
    "ln_bwd_no_projection": ("rs * (g - mg - xh * mgx)", "rs * (g - mg)"),
    "ln_db_weighted": ("ab[j] += d;", "ab[j] += g;"),
    "ln_dw_uncentred": ("aw[j] += d * xh;", "aw[j] += d * load_elem(x, in_dt, i * N + j) * rs;"),
    "ln_fused_bwd_drops_dres": ("rs * (g - mg - xh * mgx) + extra);", "rs * (g - mg - xh * mgx));"),
    "bwd_dx_missing_outer_rstd": ("rs * (g - xh * c)", "(g - xh * c)"),
}


# anchors that occur more than once: (old, new, which occurrence, count)
MUTANTS.update({
    "ln_bwd_g_without_weight": ("double g = load_elem(dy, in_dt, i * N + j) * load_elem(w, w_dt, j);",
                                "double g = load_elem(dy, in_dt, i * N + j);", 1, 2),
    "ln_bwd_dx_without_weight": ("double g = d * load_elem(w, w_dt, j);", "double g = d;", 1, 2),
})
for _k in ("bwd_g_without_weight", "bwd_dx_without_weight"):
    MUTANTS[_k] = MUTANTS[_k] + (0, 2)
# the ties and truncation anchors occur in the bfloat16, float16, E4M3 (and
# E2M1) converters, in that order
MUTANTS["ties_away_from_zero"] = MUTANTS["ties_away_from_zero"] + (0, 3)
MUTANTS["truncating_round"] = MUTANTS["truncating_round"] + (0, 4)
MUTANTS.update({
    "f16_ties_away_from_zero": ("(fmod(lo / ulp, 2.0) == 0.0) ? lo : hi", "hi", 1, 3),
    "f16_truncating_round": ("if (a < mid)", "if (a < hi)", 1, 4),
    "f16_subnormal_spacing": ("ulp = 0x1p-24;", "ulp = 0x1p-23;"),
    "f16_significand_bits": ("ulp = ldexp(1.0, e - 11);", "ulp = ldexp(1.0, e - 10);"),
    "f16_exponent_bias": ("const int field = e - 1 + 15;", "const int field = e - 1 + 16;"),
    "f16_overflow_saturates": ("if (q > f16_max)\n        return (uint16_t)(sign | 0x7C00u);",
                               "if (q > f16_max)\n        q = f16_max;"),
    "f16_decode_bias": ("ldexp(1.0 + (double)frac / 1024.0, field - 15)",
                        "ldexp(1.0 + (double)frac / 1024.0, field - 16)"),
    "f16_decode_subnormal_scale": ("m = ldexp((double)frac, -24);", "m = ldexp((double)frac, -25);"),
    "fp8_ties_up": ("(fmod(lo / ulp, 2.0) == 0.0) ? lo : hi", "hi", 2, 3),
    "fp8_truncating_round": ("if (a < mid)", "if (a < hi)", 2, 4),
    "fp4_truncating_round": ("if (a < mid)", "if (a < hi)", 3, 4),
    "fp8_subnormal_spacing": ("ulp = 0x1p-9;", "ulp = 0x1p-10;"),
    "fp8_ulp_exponent": ("ulp = ldexp(1.0, e - 4);", "ulp = ldexp(1.0, e - 5);"),
    "fp8_exponent_bias": ("int exp_field = (e - 1) + 7;", "int exp_field = (e - 1) + 8;"),
    "fp8_no_saturation": ("return (uint8_t)(sign | 0x7Eu); /* 448", "return (uint8_t)(sign | 0x7Fu); /* 448"),
    "fp8_scale_inverted": ("sc = (float)(amax / 448.0);", "sc = (float)(448.0 / amax);"),
    "fp8_quantises_unscaled": ("oracle_fp8e4m3_encode(y[j] / (double)sc);",
                               "oracle_fp8e4m3_encode(y[j]);"),
    "fp8_group_is_whole_row": ("const int64_t j0 = g * group, j1 = j0 + group < N ? j0 + group : N;",
                               "const int64_t j0 = g * group, j1 = N;"),
    "fp8_group_scale_index": ("scale[i * ngroups + g] = sc;", "scale[i + g] = sc;"),
    "fp8_group_amax_from_row_start": ("for (int64_t j = j0; j < j1; j++) {\n                double m",
                                      "for (int64_t j = 0; j < j1; j++) {\n                double m"),
    "fp4_ties_to_odd": ("code = (k % 2 == 0) ? k : k + 1; /* the even code */",
                        "code = (k % 2 == 1) ? k : k + 1;"),
    "fp4_saturates_to_4": ("if (a >= 6.0)\n        return (uint8_t)(sign | 0x7u);",
                           "if (a >= 6.0)\n        return (uint8_t)(sign | 0x6u);"),
    "mx_exponent_offset": ("E = (e2 - 1) - 2;", "E = (e2 - 1) - 1;"),
    "mx_scale_bias": ("scale[i * nb + b] = (uint8_t)(E + 127);",
                      "scale[i * nb + b] = (uint8_t)(E + 126);"),
    "mx_nibbles_swapped": ("(uint8_t)(codes[j - j0] | (codes[j + 1 - j0] << 4));",
                           "(uint8_t)(codes[j + 1 - j0] | (codes[j - j0] << 4));"),
    "mx_nan_block_scale": ("scale[i * nb + b] = 0xFF;", "scale[i * nb + b] = 0x00;"),
    "mx_zero_block_scale": ("int E = -127;", "int E = 0;"),
    "rope_first_sign": ("store_elem(y, y_dt, yo + ja, a * c - b * s);",
                        "store_elem(y, y_dt, yo + ja, a * c + b * s);"),
    "rope_second_sign": ("store_elem(y, y_dt, yo + jb, b * c + a * s);",
                         "store_elem(y, y_dt, yo + jb, b * c - a * s);"),
    "rope_cos_sin_swapped": ("const double c = (double)cos_t[p * half + i];\n"
                             "                const double s = (double)sin_t[p * half + i];",
                             "const double c = (double)sin_t[p * half + i];\n"
                             "                const double s = (double)cos_t[p * half + i];"),
    "rope_token_index_not_position": ("const int64_t p = pos[t];", "const int64_t p = t;"),
    "rope_layouts_swapped": ("const int64_t ja = interleaved ? 2 * i : i;\n"
                             "                const int64_t jb = interleaved ? 2 * i + 1 : i + half;",
                             "const int64_t ja = interleaved ? i : 2 * i;\n"
                             "                const int64_t jb = interleaved ? i + half : 2 * i + 1;"),
    "rope_half_pairs_adjacent": ("const int64_t jb = interleaved ? 2 * i + 1 : i + half;",
                                 "const int64_t jb = interleaved ? 2 * i + 1 : (i + 1) % D;"),
    "rope_out_of_range_not_nan": ("store_elem(y, y_dt, yo + j, NAN);",
                                  "store_elem(y, y_dt, yo + j, 0.0);"),
    "rope_norm_without_eps": ("oracle_rmsnorm_fwd(xh, x_dt, w, w_dt, n, OR_F64, NULL, OR_F32, 1, D, eps);",
                           "oracle_rmsnorm_fwd(xh, x_dt, w, w_dt, n, OR_F64, NULL, OR_F32, 1, D, 0.0);"),
})


FAMILY = [("f16_", "tests/test_oracle_f16.py"),
          ("fp4_", "tests/test_oracle_mxfp4.py"), ("mx_", "tests/test_oracle_mxfp4.py"),
          ("rope_", "tests/test_oracle_rope.py"), ("fp8", "tests/test_oracle_fp8.py"),
          ("ln_", "tests/test_oracle_layernorm.py"), ("bwd_", "tests/test_oracle_bwd.py"),
          ("fused_bwd", "tests/test_oracle_bwd.py"), ("fused_", "tests/test_oracle_fwd.py")]


def _plant(src: str, spec) -> str:
    old, new = spec[0], spec[1]
    which, count = (spec[2], spec[3]) if len(spec) > 2 else (0, 1)
    assert src.count(old) == count, f"anchor {old!r} occurs {src.count(old)} times"
    at = -1
    for _ in range(which + 1):
        at = src.index(old, at + 1)
    return src[:at] + new + src[at + len(old):]


def _run_mutant(name: str, workdir: str):
    """Build the oracle with one planted mistake and run the pin suite on it;
    returns (pytest's exit status, the tail of its output)."""
    src = open(SRC).read()
    mutant = os.path.join(workdir, f"{name}.c")
    with open(mutant, "w") as f:
        f.write(_plant(src, MUTANTS[name]))
    lib = os.path.join(workdir, f"lib{name}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", lib, mutant, "-lm"])
    env = dict(os.environ, ADDRMS_ORACLE_LIB=lib)
    # the whole pin suite, with the mutant's own family first (the suite stops
    # at its first failure, so the order changes only how soon)
    first = next((f for prefix, f in FAMILY if name.startswith(prefix)), None)
    pins = ([first] if first else []) + [f for f in PINS if f != first]
    run = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          *pins], cwd=ROOT, env=env, capture_output=True, text=True)
    return run.returncode, run.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every mutant's outcome, run a few at a time (each is its own process)."""
    import concurrent.futures as cf
    workdir = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        futs = {n: ex.submit(_run_mutant, n, workdir) for n in MUTANTS}
        return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_planted_mistake(name, outcomes):
    code, out = outcomes[name]
    assert code == 1, f"pins did not catch {name}:\n{out}"
