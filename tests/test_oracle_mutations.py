"""The oracle's pins must be strong enough to catch plausible mistakes in it.

Each case below plants one mistake in a copy of the oracle's C source -- a wrong rounding
mode, a dropped term, a wrong sign or index, swapped nibbles, a different bias or divisor --
compiles the copy, and runs every pin of tests/test_oracle_pins.py against it.  At least one
pin has to fail for every planted mistake.  (The unmodified oracle passes all of them; that is
tests/test_oracle_pins.py itself.)  CPU only.
"""
import inspect
from pathlib import Path

import pytest

import oracle
import test_oracle_pins as pins

SRC = Path(oracle.__file__).resolve().parent / "w4a16_oracle.c"

# (name, text in the oracle source, replacement): each text occurs exactly once.
MUTATIONS = [
    ("bf16 rounds half away from zero",
     "ldexp(1.0, e - 7); /* 8 significant bits */\n    const double r = nearbyint(",
     "ldexp(1.0, e - 7); /* 8 significant bits */\n    const double r = round("),
    ("bf16 keeps 9 significant bits", "ldexp(1.0, e - 7);", "ldexp(1.0, e - 8);"),
    ("fp16 keeps 10 significant bits", "ldexp(1.0, e - 10);", "ldexp(1.0, e - 9);"),
    ("nibbles packed in reverse order", "w |= (uint32_t)(q[j] & 0xF) << (4 * j);",
     "w |= (uint32_t)(q[j] & 0xF) << (4 * (7 - j));"),
    ("nibble k % 8 read from the wrong end", "return q[k % 8];", "return q[7 - k % 8];"),
    ("scale divides by 16 levels", "const float s = (hi - lo) / 15.0f;", "const float s = (hi - lo) / 16.0f;"),
    ("minimum taken from the maximum", "const uint16_t m_b = oracle_f32_to_bf16(lo);",
     "const uint16_t m_b = oracle_f32_to_bf16(hi);"),
    ("-0 minimum not canonicalised", "if (lo == 0.0f) lo = 0.0f; /* -0 becomes +0 */", ""),
    ("codes round half up", "const float t = rintf((w[j] - mf) / sf);",
     "const float t = floorf((w[j] - mf) / sf + 0.5f);"),
    ("codes from the exact (not the stored) scale", "const float t = rintf((w[j] - mf) / sf);",
     "const float t = rintf((w[j] - lo) / s);"),
    ("codes not clamped", "const int q = t < 0.0f ? 0 : (t > 15.0f ? 15 : (int)t);\n                const int64_t k",
     "const int q = (int)t & 15;\n                const int64_t k"),
    ("degenerate group keeps scale 0", "if (oracle_bf16_to_f32(s_b) == 0.0f) s_b = 0x3F80; /* 1.0 */",
     "if (oracle_bf16_to_f32(s_b) == 0.0f) s_b = 0x0080; /* tiny */"),
    ("dequant subtracts the minimum", "((float*)out)[n * K + k] = fmaf((float)q, s, m);",
     "((float*)out)[n * K + k] = fmaf((float)q, s, -m);"),
    ("exact weight subtracts the minimum",
     "    return (double)q * (double)oracle_bf16_to_f32(scales[(k / 128) * N + n]) +\n",
     "    return (double)q * (double)oracle_bf16_to_f32(scales[(k / 128) * N + n]) -\n"),
    ("matmul keeps only the last term",
     "acc += act_value(x, x_kind, m * K + k) * g128_weight_exact(codes, scales, mins, N, n, k);",
     "acc = act_value(x, x_kind, m * K + k) * g128_weight_exact(codes, scales, mins, N, n, k);"),
    ("activations read as the other 16-bit type",
     "return x_kind == 0 ? (double)oracle_bf16_to_f32(x[i]) : oracle_f16_to_f64(x[i]);",
     "return x_kind == 1 ? (double)oracle_bf16_to_f32(x[i]) : oracle_f16_to_f64(x[i]);"),
    ("Q4 bias 7 when encoding", "const float t = rintf(w[j] / sf) + 8.0f;", "const float t = rintf(w[j] / sf) + 7.0f;"),
    ("Q4 scale divides by 8", "const float s = a / 7.0f;", "const float s = a / 8.0f;"),
    ("Q4 nibbles swapped", "return (k % 2) ? (byte >> 4) : (byte & 0xF);", "return (k % 2) ? (byte & 0xF) : (byte >> 4);"),
    ("Q4 decode bias 7", "const float v = (float)(q - 8) * s;", "const float v = (float)(q - 7) * s;"),
    ("ZP codes round half to even", "const float tz = roundf(w[j] / sf) + zf;",
     "const float tz = rintf(w[j] / sf) + zf;"),
    ("ZP codes round the sum w/s + z", "const float tz = roundf(w[j] / sf) + zf;",
     "const float tz = roundf(w[j] / sf + zf + 0.25f);"),
    ("ZP zero point with the wrong sign", "float z = roundf(-lo / sf);", "float z = roundf(lo / sf);"),
    ("ZP zero point from the maximum", "float z = roundf(-lo / sf);", "float z = roundf(-hi / sf);"),
    ("ZP zero point rounded half to even", "float z = roundf(-lo / sf);", "float z = rintf(-lo / sf);"),
    ("ZP zero point not clamped", "if (z < -2048.0f) z = -2048.0f;", ""),
    ("ZP scale over 16 levels", "const float s_zp = (hi - lo) / 15.0f;", "const float s_zp = (hi - lo) / 16.0f;"),
    ("ZP words laid out [K/8][N]", "codes[n * (K / 8) + k / 8] |= (uint32_t)q << (4 * (k % 8));",
     "codes[(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));"),
    ("ZP nibble read from the wrong end", "return q[k & 7];", "return q[7 - (k & 7)];"),
    ("ZP decode adds the zero point",
     "return ((double)g128zp_code(codes, K, n, k) - oracle_f16_to_f64(zeros[gi])) * oracle_f16_to_f64(scales[gi]);",
     "return ((double)g128zp_code(codes, K, n, k) + oracle_f16_to_f64(zeros[gi])) * oracle_f16_to_f64(scales[gi]);"),
    ("W8 scale over 128 levels", "float s8 = a / 127.0f;", "float s8 = a / 128.0f;"),
    ("W8 codes round half to even", "const float r8 = roundf(w[k] / s8);", "const float r8 = rintf(w[k] / s8);"),
    ("W8 scale from the maximum, not the largest magnitude", "if (fabsf(w[k]) > a) a = fabsf(w[k]);",
     "if (w[k] > a) a = w[k];"),
    ("W8 exact decode drops the scale", "const double v = (double)codes[n * K + k] * (double)scales[n];",
     "const double v = (double)codes[n * K + k];"),
    ("W8 matmul reads codes as unsigned",
     "acc += act_value(x, x_kind, m * K + k) * ((double)codes[n * K + k] * (double)scales[n]);",
     "acc += act_value(x, x_kind, m * K + k) * ((double)(uint8_t)codes[n * K + k] * (double)scales[n]);"),
    ("ZP f32 decode ignores the zero point", "const float v = ((float)g128zp_code(codes, K, n, k) - z) * s;",
     "const float v = ((float)g128zp_code(codes, K, n, k)) * s;"),
    ("Q4 bf16 dequant rounds through fp16 first",
     "oracle_f32_to_bf16(v);\n            else if (kind == 2)\n                ((double*)out)[n * K + k] = (double)(q - 8)",
     "oracle_f32_to_bf16((float)oracle_f16_to_f64(oracle_f32_to_f16(v)));\n            else if (kind == 2)\n"
     "                ((double*)out)[n * K + k] = (double)(q - 8)"),
    ("Q4 fp16 dequant keeps only bf16 precision",
     "(K / 32) + k / 32]);\n            else\n                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v);",
     "(K / 32) + k / 32]);\n            else\n"
     "                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(oracle_bf16_to_f32(oracle_f32_to_bf16(v)));"),
    ("Q4 16-bit dequant kinds swapped",
     "oracle_f32_to_bf16(v);\n            else if (kind == 2)\n                ((double*)out)[n * K + k] = (double)(q - 8)",
     "oracle_f32_to_f16(v);\n            else if (kind == 2)\n                ((double*)out)[n * K + k] = (double)(q - 8)"),
    ("ZP bf16 dequant rounds through fp16 first",
     "oracle_f32_to_bf16(v);\n            else if (kind == 2)\n                ((double*)out)[n * K + k] = g128zp_weight_exact",
     "oracle_f32_to_bf16((float)oracle_f16_to_f64(oracle_f32_to_f16(v)));\n            else if (kind == 2)\n"
     "                ((double*)out)[n * K + k] = g128zp_weight_exact"),
    ("ZP fp16 dequant keeps only bf16 precision",
     "g128zp_weight_exact(codes, scales, zeros, K, n, k);\n            else\n"
     "                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v);",
     "g128zp_weight_exact(codes, scales, zeros, K, n, k);\n            else\n"
     "                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(oracle_bf16_to_f32(oracle_f32_to_bf16(v)));"),
    ("ZP fp16 dequant truncates instead of rounding",
     "g128zp_weight_exact(codes, scales, zeros, K, n, k);\n            else\n"
     "                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v);",
     "g128zp_weight_exact(codes, scales, zeros, K, n, k);\n            else\n"
     "                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(nextafterf(v, 0.0f));"),
    ("W4A8 activation codes truncate", "const float t8 = rintf(oracle_bf16_to_f32(row[k]) / a8);",
     "const float t8 = truncf(oracle_bf16_to_f32(row[k]) / a8);"),
    ("W4A8 activation scale over 128 levels", "float a8 = amax / 127.0f;", "float a8 = amax / 128.0f;"),
    ("W4A8 zero row keeps scale 0", "if (a8 == 0.0f) a8 = 1.0f; /* an all-zero row */", ""),
    ("W4A8 activation scale from the signed maximum", "if (fabsf(v) > amax) amax = fabsf(v);",
     "if (v > amax) amax = v;"),
    ("W4A8 group sum keeps the last code", "sum += q8;", "sum = q8;"),
    ("W4A8 group sums laid out [M][K/128]", "xsum[g * M + m] = (float)sum;", "xsum[m * G + g] = (float)sum;"),
    ("W4A8 product drops the activation scale",
     "acc += ((double)ascale[m] * (double)xq[m * K + k]) * g128_weight_exact(codes, scales, mins, N, n, k);",
     "acc += ((double)xq[m * K + k]) * g128_weight_exact(codes, scales, mins, N, n, k);"),
]

PIN_TESTS = [f for name, f in inspect.getmembers(pins, inspect.isfunction)
             if name.startswith("test_") and f.__module__ == pins.__name__]


def test_every_mutation_text_occurs_once():
    text = SRC.read_text()
    for name, old, _ in MUTATIONS:
        assert text.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path, monkeypatch):
    src = tmp_path / "mutant.c"
    src.write_text(SRC.read_text().replace(old, new))
    monkeypatch.setattr(oracle, "_lib", oracle.bind(oracle.compile_to(src, tmp_path / "libmutant.so")))
    caught = []
    for pin in PIN_TESTS:
        try:
            pin()
        except Exception as e:  # an assertion, or the oracle refusing its own output
            caught.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert caught, f"no pin catches the planted mistake: {name}"
