"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is oracle.c with one small textual change (a wrong offset or
sign, a reversed bit order, a wrong scale index, a dropped term, a different
rounding, a transposed output).  It is compiled into a temporary library and
the pin suite is run against it in a subprocess; the suite must fail.  This
runs on the CPU only and never touches the GPU library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "offset_minus3": ("double v = (double)(c - 4) * s;", "double v = (double)(c - 3) * s;"),
    "gemm_sign": ("double t = xv * (double)(c - 4) * s;", "double t = xv * (double)(4 - c) * s;"),
    "gemm_offset": ("double t = xv * (double)(c - 4) * s;", "double t = xv * (double)(c - 3) * s;"),
    "msb_first_codes": ("c |= stream_bit(row_words, 3 * k + b) << b;",
                        "c |= stream_bit(row_words, 3 * k + b) << (2 - b);"),
    "word_bit_reversed": ("row[j >> 5] |= 1u << (j & 31);", "row[j >> 5] |= 1u << (31 - (j & 31));"),
    "scale_index_64": ("double s = bf16_bits_to_double(scales[n * G + k / 128]);\n                double xv",
                       "double s = bf16_bits_to_double(scales[n * G + (k / 64) % G]);\n                double xv"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n                int c = code_at(row, k);",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n                int c = code_at(row, k);"),
    "round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "transposed_output": ("y[m * nrows + i] = acc;", "y[i * M + m] = acc;"),
    "w4c_msb_first_nibbles": ("(w4[n * W4 + k / 8] >> (4 * (k % 8)))", "(w4[n * W4 + k / 8] >> (4 * (7 - k % 8)))"),
    "w4c_word_index": ("(w4[n * W4 + k / 8] >> (4 * (k % 8)))", "(w4[n * W4 + k / 4 % W4] >> (4 * (k % 8)))"),
    "w4c_padding_bit_kept": ("int c = (int)(nibble & 7u);", "int c = (int)((nibble & 7u) | ((nibble >> 1) & 4u));"),
}


def _mutate(src: str, old: str, new: str) -> str:
    assert src.count(old) == 1, old
    return src.replace(old, new)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as fh:
        src = _mutate(fh.read(), old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(csrc), "-lm"], check=True)
    env = dict(os.environ, W3_ORACLE_LIB_UNDER_TEST=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
