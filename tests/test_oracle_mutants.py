"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle_pins.py catch every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, text in the oracle, replacement)
MUTANTS = [
    ("nibble order swapped", "(k % 2 == 0) ? (unsigned)(byte & 0x0Fu)",
     "(k % 2 == 1) ? (unsigned)(byte & 0x0Fu)"),
    ("no sign extension", "return (int)field - (field >= 8u ? 16 : 0);", "return (int)field;"),
    ("sign threshold 7", "field >= 8u ? 16 : 0", "field >= 7u ? 16 : 0"),
    ("sign threshold 9", "field >= 8u ? 16 : 0", "field > 8u ? 16 : 0"),
    ("last k term dropped",
     "for (int64_t k = 0; k < K; ++k)\n                sum += (int64_t)arow[k] * (int64_t)brow[k];",
     "for (int64_t k = 0; k + 1 < K; ++k)\n                sum += (int64_t)arow[k] * (int64_t)brow[k];"),
    ("wrong B row", "const int8_t *brow = b + n * K;",
     "const int8_t *brow = b + (n % (M > 0 ? M : 1)) * K;"),
    ("int32 accumulator", "int64_t sum = 0;\n            for", "int32_t sum = 0;\n            for"),
    ("pack nibbles swapped", "out[r * (K / 2) + j] = (uint8_t)(even | (odd << 4));",
     "out[r * (K / 2) + j] = (uint8_t)(odd | (even << 4));"),
    ("sampled w4a8 k order", "sum += (int64_t)arow[k] * int4_value(nibble_of(brow, k));",
     "sum += (int64_t)arow[k] * int4_value(nibble_of(brow, k ^ 1));"),
    ("sampled i4i4 drops k=0",
     "sum += (int64_t)int4_value(nibble_of(arow, k)) * int4_value(nibble_of(brow, k));",
     "sum += (int64_t)int4_value(nibble_of(arow, k)) * int4_value(nibble_of(brow, k)) * (k > 0);"),
    ("output transposed", "C[m * N + n] = (int32_t)sum;", "C[n * M + m] = (int32_t)sum;"),
    ("packed row stride", "const uint8_t *src = packed + r * (K / 2);",
     "const uint8_t *src = packed + r * K / 2 + (r > 0);"),
    ("range check removed", "if (sum < INT32_MIN || sum > INT32_MAX) bad = 1;", ";"),
]

# Mistakes in the scaled epilogue, caught by test_oracle_scaled.py.
SCALED_MUTANTS = [
    ("scales multiplied first", "volatile float y = t * scale_a[m];      /* binary32 multiply */\n"
     "            volatile float z = y * scale_b[n];",
     "volatile float y = scale_a[m] * scale_b[n];\n            volatile float z = y * t;"),
    ("ties away from zero", "const double r = rint(ax / q) * q;",
     "const double r = round(ax / q) * q;"),
    ("truncation", "const double r = rint(ax / q) * q;", "const double r = trunc(ax / q) * q;"),
    ("bf16 keeps 7 bits", "round_to_format(v, 8, -126,", "round_to_format(v, 7, -126,"),
    ("f16 no subnormals", "if (e < emin) e = emin;", ";"),
    ("f16 overflow at max", "if (ax >= limit || r > maxv)", "if (ax > maxv || r > maxv)"),
    ("scale_b index", "volatile float z = y * scale_b[n];", "volatile float z = y * scale_b[m % N];"),
]


# Mistakes in the fp8 (e4m3) oracle, caught by test_oracle_fp8.py.
FP8_MUTANTS = [
    ("e4m3 bias 8", "v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 11);"),
    ("e4m3 subnormal scale", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3 NaN code not special", "if (e == 15 && m == 7)\n        return NAN;", "if (0)\n        return NAN;"),
    ("e4m3 ties up", "if (dhi < dlo) return sign | (uint8_t)hi;", "if (dhi <= dlo) return sign | (uint8_t)hi;"),
    ("e4m3 no saturation", "if (ax >= 448.0) return sign | 0x7E;", "if (ax >= 464.0) return sign | 0x7F;"),
    ("fp8 last k dropped", "for (int64_t k = 0; k < K; ++k) {\n                const double p",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n                const double p"),
    ("fp8 abs sum signed", "sa += fabs(p);", "sa += p;"),
]


# Mistakes in the e5m2 oracle, caught by test_oracle_fp8_e5m2.py.
E5M2_MUTANTS = [
    ("e5m2 bias 16", "ldexp(4.0 + m, e - 17);\n    return s ? -v : v;",
     "ldexp(4.0 + m, e - 18);\n    return s ? -v : v;"),
    ("e5m2 integer bias", "*ie = e == 0 ? -16 : e - 17;", "*ie = e == 0 ? -16 : e - 16;"),
    ("e5m2 subnormal scale", "const double v = e == 0 ? ldexp((double)m, -16)",
     "const double v = e == 0 ? ldexp((double)m, -15)"),
    ("e5m2 overflow saturates", "if (ax >= 61440.0) return sign | 0x7C;", "if (ax >= 61440.0) return sign | 0x7B;"),
    ("e5m2 overflow early", "if (ax >= 61440.0) return sign | 0x7C;", "if (ax > 57344.0) return sign | 0x7C;"),
    ("e5m2 ties up", "if (dhi < dlo) return sign | (uint8_t)hi;\n    return sign | (uint8_t)((lo & 1) ? hi : lo);\n}\n\nint oracle_fp8_e5m2_encode",
     "if (dhi <= dlo) return sign | (uint8_t)hi;\n    return sign | (uint8_t)((lo & 1) ? hi : lo);\n}\n\nint oracle_fp8_e5m2_encode"),
    ("e5m2 sum in 2^-31 units", "<< (ea + eb + 32));", "<< (ea + eb + 31));"),
    ("e5m2 product sign lost", "const __int128 p = (__int128)(ia * ib)", "const __int128 p = (__int128)(ia * ib < 0 ? -ia * ib : ia * ib)"),
    ("e5m2 inf not special", "if (e == 31) return 0;                     /* infinity or NaN */", ";"),
]


# Mistakes in the per-K-block scaled product, caught by test_oracle_blockscaled.py.
BLOCKSCALED_MUTANTS = [
    ("block boundary off by one", "for (int64_t k = j * g; k < k1; ++k)",
     "for (int64_t k = j * g + (j > 0); k < k1 + (j + 1 < nb); ++k)"),
    ("last partial block dropped", "const int64_t nb = (K + g - 1) / g;\n    if (out == NULL",
     "const int64_t nb = K / g;\n    if (out == NULL"),
    ("scales multiplied first", "volatile float y = t * SFA[m * nb + j];    /* binary32 multiply */\n"
     "                volatile float z = y * SFB[n * nb + j];",
     "volatile float y = SFA[m * nb + j] * SFB[n * nb + j];\n                volatile float z = y * t;"),
    ("SFB indexed by the output row", "volatile float z = y * SFB[n * nb + j];",
     "volatile float z = y * SFB[(m % N) * nb + j];"),
    ("SFA of the next block", "volatile float y = t * SFA[m * nb + j];",
     "volatile float y = t * SFA[m * nb + (j + 1 < nb ? j + 1 : j)];"),
    ("accumulated in double", "volatile float acc = 0.0f;\n            for (int64_t j = 0; j < nb; ++j) {\n                const int64_t k1",
     "volatile double acc = 0.0;\n            for (int64_t j = 0; j < nb; ++j) {\n                const int64_t k1"),
    ("blocks added last to first", "for (int64_t j = 0; j < nb; ++j) {\n                const int64_t k1",
     "for (int64_t jj = 0; jj < nb; ++jj) {\n                const int64_t j = nb - 1 - jj;\n                const int64_t k1"),
    ("scales applied after the sum", "volatile float y = t * SFA[m * nb + j];    /* binary32 multiply */",
     "volatile float y = t * (j == 0 ? SFA[m * nb] : 1.0f);"),
]


@pytest.mark.parametrize("what,old,new,pins",
                         [m + ("tests/test_oracle_pins.py",) for m in MUTANTS] +
                         [m + ("tests/test_oracle_scaled.py",) for m in SCALED_MUTANTS] +
                         [m + ("tests/test_oracle_fp8.py",) for m in FP8_MUTANTS] +
                         [m + ("tests/test_oracle_fp8_e5m2.py",) for m in E5M2_MUTANTS] +
                         [m + ("tests/test_oracle_blockscaled.py",) for m in BLOCKSCALED_MUTANTS],
                         ids=[m[0] for m in MUTANTS + SCALED_MUTANTS + FP8_MUTANTS + E5M2_MUTANTS +
                              BLOCKSCALED_MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, what, old, new, pins):
    for d in ("oracle", "tests", "precision_integer_gemm_amd"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.hip", "*.o"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src = tmp_path / "oracle" / "lpgemm_oracle.c"
    text = src.read_text()
    assert old in text, f"mutation site for '{what}' not found"
    src.write_text(text.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", pins, "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch: {what}\n{r.stdout[-2000:]}"
