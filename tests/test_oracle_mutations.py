"""Mutation check of the oracle's pins (CPU only).

Each case below plants one plausible mistake in a copy of
oracle/bsfp_oracle.c (a dropped term, a wrong sign, index, constant or tie
rule), builds it with the oracle's own flags, and runs the pin files named
for it against that build in a child pytest (BSFP_ORACLE_LIB points the
oracle's Python face at it).  The pins must fail: a mistake that every pin
lets through would be a hole in what pins the oracle.  The planted text must
occur exactly once in the source, so a change to the oracle that moves it
shows up here instead of silently testing nothing.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bsfp_oracle.c")

CODECS = "tests/test_oracle_codecs.py"
QUANT = "tests/test_oracle_quantize.py"
MATMUL = "tests/test_oracle_matmul.py"
VARIANTS = "tests/test_oracle_variants.py"
SR = "tests/test_oracle_sr.py"

# (name, text in the source, planted replacement, pin files expected to fail)
MUTANTS = [
    ("e2m1 ties to the odd code",
     "double d = fabs(a - bo_e2m1_decode(c));\n        if (d < bd || (d == bd && (c & 1) == 0))",
     "double d = fabs(a - bo_e2m1_decode(c));\n        if (d < bd || (d == bd && (c & 1) == 1))",
     [CODECS]),
    ("e2m1 drops the sign of zero",
     "return best | (signbit(v) ? 8 : 0);",
     "return best | ((v < 0.0f && best) ? 8 : 0);",
     [CODECS]),
    ("e4m3 saturates to NaN",
     "if (!(a <= 448.0)) return 0x7E;",
     "if (!(a <= 448.0)) return 0x7F;",
     [CODECS]),
    ("e4m3 ties to the odd code",
     "double d = fabs(a - bo_e4m3_decode(c));\n        if (d < bd || (d == bd && (c & 1) == 0))",
     "double d = fabs(a - bo_e4m3_decode(c));\n        if (d < bd || (d == bd && (c & 1) == 1))",
     [CODECS]),
    ("e8m0 bias off by one",
     "return ldexp(1.0, (code & 0xFF) - 127);",
     "return ldexp(1.0, (code & 0xFF) - 128);",
     [CODECS]),
    ("bf16 ties away from zero",
     "return (lo & 1) ? hi : lo;",
     "return hi;",
     [CODECS]),
    ("nvfp4 block scale without the factor 6",
     "float sf = bamax / six_g;",
     "float sf = bamax / g;",
     [QUANT]),
    ("nvfp4 decoded block scale without g",
     "d = (float)bo_e4m3_decode(S) * g;",
     "d = (float)bo_e4m3_decode(S);",
     [QUANT]),
    ("global scale from 448 * 4",
     "const float max_product = 448.0f * 6.0f;",
     "const float max_product = 448.0f * 4.0f;",
     [QUANT]),
    ("alpha as a quotient",
     "return g_x * g_w; }",
     "return g_x / g_w; }",
     [QUANT, MATMUL]),
    ("amax skips the last element",
     "float m = 0.0f;\n    for (int64_t i = 0; i < n; ++i) {",
     "float m = 0.0f;\n    for (int64_t i = 0; i + 1 < n; ++i) {",
     [QUANT]),
    ("mxfp4 exponent offset 3",
     "const int emax_e2m1 = 2;",
     "const int emax_e2m1 = 3;",
     [QUANT]),
    ("mxfp8 exponent offset 7",
     "const int emax_e4m3 = 8;",
     "const int emax_e4m3 = 7;",
     [VARIANTS]),
    ("affine step over 16 levels",
     "float step = range / 15.0f;",
     "float step = range / 16.0f;",
     [QUANT]),
    ("affine codes truncated",
     "float q = nearbyintf(t); /* round to nearest, ties to even */",
     "float q = floorf(t); /* round to nearest, ties to even */",
     [QUANT]),
    ("nibbles packed high first",
     "row_words[k / 8] |= (uint32_t)(code & 0xF) << (4 * (k % 8));",
     "row_words[k / 8] |= (uint32_t)(code & 0xF) << (4 * (7 - k % 8));",
     [QUANT]),
    ("affine variant dequantize with the wrong group index",
     "float s = bo_bf16_to_f32(s16[r * groups + k / G]);",
     "float s = bo_bf16_to_f32(s16[r * groups + k / 64]);",
     [VARIANTS]),
    ("affine variant dequantize subtracts the bias",
     "out[r * cols + k] = bo_bf16_from_f32(fmaf(s, (float)c, b));",
     "out[r * cols + k] = bo_bf16_from_f32(fmaf(s, (float)c, -b));",
     [VARIANTS]),
    ("matmul with k reversed in B",
     "double p = A[m * K + k] * B[n * K + k];",
     "double p = A[m * K + k] * B[n * K + (K - 1 - k)];",
     [MATMUL]),
    ("stochastic rounding compares the wrong way",
     "return (u < p ? lo + 1 : lo) | sign;",
     "return (u > p ? lo + 1 : lo) | sign;",
     [SR]),
]


def _build(src_text, out_dir):
    c = os.path.join(out_dir, "bsfp_oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    # the same flags as oracle/build.py; the header comes from oracle/
    so = os.path.join(out_dir, "liboracle_mut.so")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fopenmp", "-I", os.path.join(ROOT, "oracle"), c,
                    "-o", so, "-lm"], check=True, capture_output=True)
    return so


@pytest.mark.parametrize("name,old,new,files", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, files):
    src = open(SRC).read()
    assert src.count(old) == 1, f"planted text not found exactly once: {old!r}"
    so = _build(src.replace(old, new), str(tmp_path))
    env = dict(os.environ, BSFP_ORACLE_LIB=so, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    # exit status 1: tests ran and at least one failed (2-4 would be a
    # collection or usage error, which proves nothing)
    assert r.returncode == 1, (name, r.returncode, r.stdout[-2000:], r.stderr[-2000:])


def test_unmutated_copy_passes(tmp_path):
    """The same build route without a planted mistake passes the same pins."""
    so = _build(open(SRC).read(), str(tmp_path))
    env = dict(os.environ, BSFP_ORACLE_LIB=so, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", CODECS, QUANT, MATMUL, VARIANTS, SR],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
