"""Pin strength: plant plausible mistakes in copies of the oracle (CPU only)
and check that the oracle's own pins in test_oracle.py reject every one.

Each mutant is oracle.c with one textual change, compiled to a temporary
library and loaded through ORACLE_LIB_PATH in a child pytest run.  Mutants
are chosen to stay in bounds (no mutant may crash the child).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    # HGEMM: k runs backwards in A only (a transposed/misindexed operand)
    "gemm_a_k_reversed": ("acc += g_h2d[A[i * lda + k]] * g_h2d[B[j * ldb + k]];",
                          "acc += g_h2d[A[i * lda + (K - 1 - k)]] * g_h2d[B[j * ldb + k]];"),
    # HGEMM: the beta·C term dropped from the full-matrix routine
    "gemm_beta_dropped": ("            if (beta != 0.0)\n                r += beta * cin_value(Cin, cin_dtype, i * ldc + j);\n            ref[i * ldr + j] = r;",
                          "            ref[i * ldr + j] = r;"),
    # HGEMM: alpha applied twice
    "gemm_alpha_squared": ("        double r = alpha * acc;\n            if (beta != 0.0)\n                r += beta * cin_value(Cin, cin_dtype, i * ldc + j);\n            ref[i * ldr + j]",
                           "        double r = alpha * alpha * acc;\n            if (beta != 0.0)\n                r += beta * cin_value(Cin, cin_dtype, i * ldc + j);\n            ref[i * ldr + j]"),
    # HGEMM: one term of the sum dropped
    "gemm_last_k_dropped": ("for (int64_t k = 0; k < K; ++k)\n                    acc += g_h2d[A[i * lda + k]]",
                            "for (int64_t k = 0; k + 1 < K; ++k)\n                    acc += g_h2d[A[i * lda + k]]"),
    # TRMM: diagonal term dropped
    "trmm_diag_dropped": ("for (int64_t k = i; k < n; ++k)\n                acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]",
                          "for (int64_t k = i + 1; k < n; ++k)\n                acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]"),
    # TRMM: strict upper triangle read
    "trmm_reads_upper": ("for (int64_t k = i; k < n; ++k)\n                acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]",
                         "for (int64_t k = 0; k < n; ++k)\n                acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]"),
    # TRMM: A used untransposed
    "trmm_A_not_transposed": ("acc += g_h2d[A[k + i * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]",
                              "acc += g_h2d[A[i + k * lda]] * g_h2d[B[k + j * ldb]];\n            ref[i + j * ldr]"),
    # TRSM: substitution term added instead of subtracted
    "trsm_sign": ("acc -= g_h2d[A[k + i * lda]] * x[k];", "acc += g_h2d[A[k + i * lda]] * x[k];"),
    # TRSM: division by the diagonal dropped
    "trsm_no_divide": ("x[i] = acc / g_h2d[A[i + i * lda]];", "x[i] = acc;"),
    # TRSM: A used untransposed (reads the strict upper triangle)
    "trsm_untransposed": ("acc -= g_h2d[A[k + i * lda]] * x[k];", "acc -= g_h2d[A[i + k * lda]] * x[k];"),
    # TRSM: alpha not applied
    "trsm_alpha_dropped": ("double acc = alpha * g_h2d[B[i + j * ldb]];", "double acc = g_h2d[B[i + j * ldb]];"),
    # TRSM: last row's term dropped from every sum
    "trsm_last_term_dropped": ("for (int64_t k = i + 1; k < n; ++k)\n                acc -= ",
                               "for (int64_t k = i + 1; k + 1 < n; ++k)\n                acc -= "),
    # fused epilogue: bias dropped
    "epi_bias_dropped": ("            if (bias)\n                t += (double)bias[j];\n", ""),
    # fused epilogue: ReLU threshold inverted
    "epi_relu_inverted": ("if (act == 1 && t < 0.0)", "if (act == 1 && t > 0.0)"),
    # fused epilogue: bias indexed by row instead of column
    "epi_bias_by_row": ("t += (double)bias[j];", "t += (double)bias[i % N];"),
    # bf16 fused epilogue: bias dropped
    "bf16_epi_bias_dropped": ("            if (bias != NULL)\n                v += (double)bias[j];\n", ""),
    # bf16 fused epilogue: ReLU threshold inverted
    "bf16_epi_relu_inverted": ("if (act == 1 && v < 0.0)", "if (act == 1 && v > 0.0)"),
    # bf16 fused epilogue: bias indexed by row instead of column
    "bf16_epi_bias_by_row": ("v += (double)bias[j];", "v += (double)bias[i % N];"),
    # bf16 fused epilogue: the beta·C term dropped
    "bf16_epi_beta_dropped": ("            if (beta != 0.0)\n                v += beta * cin_value(Cin, cin_dtype, i * ldc + j);\n", ""),
    # sampled fused definition: bias indexed by row instead of column
    "sampled_epi_bias_by_row": ("u += (double)bias[j];", "u += (double)bias[i % (j + 1)];"),
    # sampled fused definition: ReLU never applied
    "sampled_epi_relu_dropped": ("if (act == 1 && u < 0.0)", "if (act == 2 && u < 0.0)"),
    # sampled fused definition: bf16 operands decoded as fp16
    "sampled_epi_decoder_swapped": ("const double *dec = in_dtype == 2 ? g_b2d : g_h2d;",
                                    "const double *dec = g_h2d;"),
    # sampled fused definition: the beta·C term dropped
    "sampled_epi_beta_dropped": ("        if (beta != 0.0)\n            u += beta * cin_value(Cin, cin_dtype, i * ldc + j);\n", ""),
    # bf16 decoding: exponent bias off by one
    "bf16_decode_bias": ("v = ldexp((double)(128 + frac), expo - 134);", "v = ldexp((double)(128 + frac), expo - 133);"),
    # bf16 decoding: fraction field one bit short
    "bf16_decode_frac": ("const int frac = h & 0x7f;", "const int frac = h & 0x3f;"),
    # bf16 GEMM: B read at reversed k (a misindexed operand)
    "bf16_gemm_B_k_reversed": ("acc += g_b2d[A[i * lda + k]] * g_b2d[B[j * ldb + k]];",
                               "acc += g_b2d[A[i * lda + k]] * g_b2d[B[j * ldb + (K - 1 - k)]];"),
    # TRMM variants: the triangle test inverted for upper
    "trmm_variant_upper_inverted": ("const int stored = uplo == 0 ? r >= c : r <= c;",
                                    "const int stored = uplo == 0 ? r >= c : r < c;"),
    # TRMM variants: transposition ignored
    "trmm_variant_no_trans": ("const int64_t r = trans ? k : i, c = trans ? i : k;",
                              "const int64_t r = i, c = k;"),
    # fp16 decoding: subnormal scale off by one binade
    "decode_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    # fp16 decoding: exponent bias off by one
    "decode_bias": ("v = ldexp((double)(1024 + frac), expo - 25);", "v = ldexp((double)(1024 + frac), expo - 24);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name} does not apply"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new, 1))   # first occurrence: the full-matrix routine
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(lib),
                    str(mut), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_PATH=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"pins did not reject mutant {name}:\n{r.stdout[-2000:]}"
