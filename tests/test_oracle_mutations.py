"""Planted mistakes in the oracle must be caught by its pins.

Each case below edits one line of the oracle's C source (a dropped term, a
wrong sign, a wrong index or leading dimension, a wrong decoding, an unfused
multiply-add), compiles the edited copy into a temporary library, swaps it in
and runs the pin tests against it: at least one pin must fail.  Every edit keeps
all memory accesses in bounds.
"""
import os

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "tgemm_oracle.c")

# (name, exact text to replace (first occurrence), replacement)
MUTATIONS = [
    ("f32_drops_last_k",
     "for (int64_t k = 0; k < K; ++k) {\n            double a = (double)A[i * lda + k];",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            double a = (double)A[i * lda + k];"),
    ("bf16_skips_first_k",
     "for (int64_t k = 0; k < K; ++k) {\n            double a = bf16_bits_to_double",
     "for (int64_t k = 1; k < K; ++k) {\n            double a = bf16_bits_to_double"),
    ("f32_wrong_sign", "c[j] += p;", "c[j] -= p;"),
    ("f32_companion_not_abs", "s[j] += fabs(p);", "s[j] += p;"),
    ("f32_ldb_ignored", "const float *b = B + k * ldb;", "const float *b = B + k * N;"),
    ("i8_reversed_k", "int64_t a = (int64_t)A[i * lda + k];",
     "int64_t a = (int64_t)A[i * lda + (K - 1 - k)];"),
    ("i8_unsigned_decode", "int64_t a = (int64_t)A[i * lda + k];",
     "int64_t a = (int64_t)(uint8_t)A[i * lda + k];"),
    ("i8_last_column_dropped", "for (int64_t j = 0; j < N; ++j) c[j] += a * (int64_t)b[j];",
     "for (int64_t j = 0; j + 1 < N; ++j) c[j] += a * (int64_t)b[j];"),
    ("bf16_decode_extra_bit", "uint32_t u = (uint32_t)bits << 16;",
     "uint32_t u = ((uint32_t)bits << 16) | 0x8000u;"),
    ("bf16_lda_as_K", "double a = bf16_bits_to_double(A[i * lda + k]);",
     "double a = bf16_bits_to_double(A[i * K + k]);"),
    ("fma_chain_unfused", "for (int64_t j = 0; j < N; ++j) c[j] = fmaf(a, b[j], c[j]);",
     "for (int64_t j = 0; j < N; ++j) c[j] = c[j] + a * b[j];"),
    # the sampled (one dot product per position) functions
    ("f32_sampled_ldb_ignored", "double q = (double)A[i * lda + k] * (double)B[k * ldb + j];",
     "double q = (double)A[i * lda + k] * (double)B[k * N + j];"),
    ("f32_sampled_companion_not_abs", "            s += fabs(q);", "            s += q;"),
    ("bf16_sampled_drops_last_k",
     "for (int64_t k = 0; k < K; ++k) {\n            double q = bf16_bits_to_double(A[i * lda + k]) *",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            double q = bf16_bits_to_double(A[i * lda + k]) *"),
    ("bf16_sampled_ldb_ignored", "bf16_bits_to_double(B[k * ldb + j]);", "bf16_bits_to_double(B[k * N + j]);"),
    ("i8_sampled_lda_as_K", "c += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];",
     "c += (int64_t)A[i * K + k] * (int64_t)B[k * ldb + j];"),
    ("i8_sampled_ldb_ignored", "c += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];",
     "c += (int64_t)A[i * lda + k] * (int64_t)B[k * N + j];"),
    ("fma_chain_sampled_unfused", "c = fmaf(A[i * lda + k], B[k * ldb + j], c);",
     "c = c + A[i * lda + k] * B[k * ldb + j];"),
    ("fma_chain_sampled_ldb_ignored", "c = fmaf(A[i * lda + k], B[k * ldb + j], c);",
     "c = fmaf(A[i * lda + k], B[k * N + j], c);"),
]


def _pins():
    """The pin checks, as zero-argument callables."""
    out = []
    for dtype in ("f32", "bf16", "i8"):
        for shape in [(3, 4, 5), (5, 7, 9), (13, 31, 6), (1, 2, 3)]:
            out.append(lambda d=dtype, s=shape: pins.test_brute_force_exact(*s, d))
        out.append(lambda d=dtype: pins.test_identity(d))
        out.append(lambda d=dtype: pins.test_permutation_rows(d))
        out.append(lambda d=dtype: pins.test_all_ones_gives_K(d))
        out.append(lambda d=dtype: pins.test_rank1_known_sums(d))
        out.append(lambda d=dtype: pins.test_hadamard(d))
    out.append(pins.test_bf16_decoding_matches_torch_widening)
    out.append(pins.test_int8_extremes)
    out.append(lambda: pins.test_fma_chain_exact_emulation(3, 4, 50))
    out.append(pins.test_fma_chain_differs_from_unfused_rounding)
    for dtype in ("f32", "bf16", "i8"):
        out.append(lambda d=dtype: pins.test_sampled_brute_force_exact(d))
    out.append(pins.test_sampled_fma_chain_exact_emulation)
    return out


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path, monkeypatch):
    text = open(SRC).read()
    assert old in text, "mutation anchor not found: %s" % name
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(text.replace(old, new, 1))
    lib_path = oracle.compile_source(str(src), str(tmp_path / ("libmut_%s.so" % name)))
    monkeypatch.setattr(oracle, "_lib", oracle.bind(lib_path))
    failures = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, "no pin caught the planted mistake %s" % name
