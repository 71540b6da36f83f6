"""Pins for the CPU oracle, checked against facts that do not come from it.

The oracle computes the definition of C = A x B ("4.1 CUDA GEMM算子性能优化",
section 1.1).  Here it is checked against:
  * exact rational brute force (``fractions.Fraction``) on tiny shapes, with
    non-square, non-symmetric, row-padded operands so that a transposed
    operand, a wrong index or a wrong leading dimension changes the answer;
  * closed forms that hold at any size: identity, permutation, all-ones,
    rank-1 outer products, Sylvester-Hadamard, int8 extremes;
  * for the fp32 fma-chain variant, an exact emulation of single-precision
    fused multiply-add (rational arithmetic, round to nearest even);
  * torch's own bf16 -> fp32 widening, for the oracle's bf16 decoding.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_software_pipelined_amd import inputs


def _bf16_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _exact_product(A, B):
    """Exact C and S = sum |a b| as Fractions (A, B are float or int arrays)."""
    M, K = A.shape
    N = B.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    Af = [[Fraction(float(A[i, k])) if A.dtype.kind == "f" else Fraction(int(A[i, k]))
           for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B[k, j])) if B.dtype.kind == "f" else Fraction(int(B[k, j]))
           for j in range(N)] for k in range(K)]
    for i in range(M):
        for j in range(N):
            c = Fraction(0)
            s = Fraction(0)
            for k in range(K):
                p = Af[i][k] * Bf[k][j]
                c += p
                s += abs(p)
            C[i][j] = c
            S[i][j] = s
    return C, S


TINY = [(m, n, k) for m in (1, 2, 3) for n in (1, 2, 4) for k in (1, 3, 5)] + \
       [(5, 7, 9), (9, 4, 13), (13, 31, 6), (3, 33, 17), (7, 2, 31)]


@pytest.mark.parametrize("M,N,K", TINY)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_brute_force_exact(M, N, K, dtype):
    kind = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}[dtype]
    seed = 17 * M + 131 * N + 1009 * K
    # padded leading dimensions: a wrong lda/ldb reads the filler and fails
    A = inputs.operand(kind, M, K, seed, ld=K + 3)
    B = inputs.operand(kind, K, N, seed + 1, ld=N + 5)
    Af = A.float().numpy() if dtype == "bf16" else A.numpy()
    Bf = B.float().numpy() if dtype == "bf16" else B.numpy()
    Cx, Sx = _exact_product(Af, Bf)
    C, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    assert C.shape == (M, N)
    if dtype == "i8":
        assert C.dtype == np.int64
        for i in range(M):
            for j in range(N):
                assert int(C[i, j]) == Cx[i][j]
        return
    bound_rel = Fraction(K, 2 ** 52)
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - Cx[i][j])
            assert err <= bound_rel * Sx[i][j], (i, j, float(err))
            errs = abs(Fraction(float(S[i, j])) - Sx[i][j])
            assert errs <= bound_rel * Sx[i][j]


def test_bf16_decoding_matches_torch_widening():
    # A = 1x1 [1.0] makes C the decoded row of B; compare with torch's widening.
    B = inputs.operand("bf16_normal", 1, 4096, 99)
    one = torch.ones((1, 1), dtype=torch.bfloat16)
    C, S = oracle.gemm(_bf16_bits(one), _bf16_bits(B), "bf16")
    np.testing.assert_array_equal(C[0], B.float().numpy()[0].astype(np.float64))
    np.testing.assert_array_equal(S[0], np.abs(B.float().numpy()[0]).astype(np.float64))


def _as(dtype, x):
    """Integer-valued numpy array -> operand of the given type (exact)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return _bf16_bits(torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))
    return np.ascontiguousarray(x, dtype=np.int8)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_identity(dtype):
    n = 96
    rng = np.random.default_rng(5)
    B = rng.integers(-100, 100, size=(n, 70))
    C, _ = oracle.gemm(_as(dtype, np.eye(n)), _as(dtype, B), dtype)
    np.testing.assert_array_equal(C, B)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_permutation_rows(dtype):
    n = 64
    rng = np.random.default_rng(6)
    perm = rng.permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1
    B = rng.integers(-50, 50, size=(n, 33))
    C, _ = oracle.gemm(_as(dtype, P), _as(dtype, B), dtype)
    np.testing.assert_array_equal(C, B[perm])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_all_ones_gives_K(dtype):
    M, N, K = 17, 23, 4104
    C, S = oracle.gemm(_as(dtype, np.ones((M, K))), _as(dtype, np.ones((K, N))), dtype)
    assert (C == K).all()
    if S is not None:
        assert (S == K).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_rank1_known_sums(dtype):
    rng = np.random.default_rng(7)
    M, N, K = 40, 36, 300
    u = rng.integers(-4, 5, size=M)
    v = rng.integers(-4, 5, size=N)
    x = rng.integers(-1, 3, size=K)
    y = rng.integers(-1, 3, size=K)
    A = np.outer(u, x)
    B = np.outer(y, v)
    C, S = oracle.gemm(_as(dtype, A), _as(dtype, B), dtype)
    xy = int(np.dot(x, y))
    np.testing.assert_array_equal(C, np.outer(u, v) * xy)
    if S is not None:
        np.testing.assert_array_equal(S, np.abs(np.outer(u, v)) * int(np.dot(np.abs(x), np.abs(y))))


def _sylvester(p):
    H = np.array([[1]])
    for _ in range(p):
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_hadamard(dtype):
    H = _sylvester(7)            # 128 x 128, entries +-1
    n = H.shape[0]
    C, S = oracle.gemm(_as(dtype, H), _as(dtype, H.T.copy()), dtype)
    np.testing.assert_array_equal(C, n * np.eye(n))
    if S is not None:
        assert (S == n).all()


def test_int8_extremes():
    K = 4096
    lo = np.full((3, K), -128, dtype=np.int8)
    C, _ = oracle.gemm(lo, np.full((K, 5), -128, dtype=np.int8), "i8")
    assert (C == 16384 * K).all() and C[0, 0] == 67108864
    C, _ = oracle.gemm(lo, np.full((K, 5), 127, dtype=np.int8), "i8")
    assert (C == -16256 * K).all() and C[0, 0] == -66584576


def test_int8_results_fit_int32_at_largest_K():
    # |C| <= 128^2 * K; at K = 8192 that is 2^27 < 2^31
    assert 128 * 128 * 8192 < 2 ** 31


def _round_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp_exp = max(e, -126) - 23
    scaled = q / Fraction(2) ** ulp_exp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * Fraction(2) ** ulp_exp


def test_round_f32_helper_agrees_with_numpy_on_doubles():
    rng = np.random.default_rng(3)
    for x in rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, size=2000):
        assert float(_round_f32(Fraction(float(x)))) == float(np.float32(x))


@pytest.mark.parametrize("M,N,K", [(3, 4, 50), (5, 2, 129), (1, 7, 300)])
def test_fma_chain_exact_emulation(M, N, K):
    A = inputs.operand("f32_uniform", M, K, 11 * K, ld=K + 2).numpy()
    B = inputs.operand("f32_uniform", K, N, 13 * K).numpy()
    C = oracle.gemm_f32_fma_chain(A, B)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc = _round_f32(Fraction(float(A[i, k])) * Fraction(float(B[k, j])) + acc)
            assert C[i, j] == np.float32(float(acc)), (i, j)


def test_fma_chain_differs_from_unfused_rounding():
    # the fused chain must not be a separately rounded multiply then add:
    # find a case where the two differ and check the oracle takes the fused one
    A = inputs.operand("f32_uniform", 1, 400, 21).numpy()
    B = inputs.operand("f32_uniform", 400, 1, 22).numpy()
    fused = Fraction(0)
    unfused = np.float32(0)
    for k in range(400):
        fused = _round_f32(Fraction(float(A[0, k])) * Fraction(float(B[k, 0])) + fused)
        unfused = np.float32(unfused + np.float32(A[0, k] * B[k, 0]))
    assert np.float32(float(fused)) != unfused
    C = oracle.gemm_f32_fma_chain(A, B)
    assert C[0, 0] == np.float32(float(fused))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_sampled_matches_full(dtype):
    # both operands row-padded with a non-zero filler: a sampled function that
    # ignored lda or ldb would read the filler
    kind = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}[dtype]
    M, N, K = 67, 45, 130
    A = inputs.as_oracle_array(inputs.operand(kind, M, K, 1, ld=K + 8))
    B = inputs.as_oracle_array(inputs.operand(kind, K, N, 2, ld=N + 7))
    C, S = oracle.gemm(A, B, dtype)
    rng = np.random.default_rng(0)
    rows = np.concatenate([rng.integers(0, M, 200), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 200), [0, N - 1, 0, N - 1]])
    Cs, Ss = oracle.gemm_sampled(A, B, rows, cols, dtype)
    np.testing.assert_array_equal(Cs, C[rows, cols])
    if S is not None:
        np.testing.assert_array_equal(Ss, S[rows, cols])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_sampled_brute_force_exact(dtype):
    # the sampled functions on their own against exact rational sums, with
    # padded A and B (not only through the full oracle)
    kind = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}[dtype]
    M, N, K = 6, 9, 37
    A = inputs.operand(kind, M, K, 41, ld=K + 3)
    B = inputs.operand(kind, K, N, 42, ld=N + 5)
    Af = A.float().numpy() if dtype == "bf16" else A.numpy()
    Bf = B.float().numpy() if dtype == "bf16" else B.numpy()
    Cx, Sx = _exact_product(Af, Bf)
    rows = np.array([i for i in range(M) for _ in range(N)])
    cols = np.array([j for _ in range(M) for j in range(N)])
    Cs, Ss = oracle.gemm_sampled(inputs.as_oracle_array(A), inputs.as_oracle_array(B), rows, cols, dtype)
    bound_rel = Fraction(K, 2 ** 52)
    for p in range(rows.shape[0]):
        i, j = rows[p], cols[p]
        if dtype == "i8":
            assert int(Cs[p]) == Cx[i][j]
        else:
            assert abs(Fraction(float(Cs[p])) - Cx[i][j]) <= bound_rel * Sx[i][j], (i, j)
            assert abs(Fraction(float(Ss[p])) - Sx[i][j]) <= bound_rel * Sx[i][j], (i, j)


def test_sampled_fma_chain_matches_full():
    A = inputs.operand("f32_uniform", 20, 77, 3, ld=80).numpy()
    B = inputs.operand("f32_uniform", 77, 19, 4, ld=23).numpy()
    C = oracle.gemm_f32_fma_chain(A, B)
    rows = np.array([0, 19, 5, 7])
    cols = np.array([18, 0, 5, 11])
    Cs, _ = oracle.gemm_sampled(A, B, rows, cols, "f32", fma_chain=True)
    np.testing.assert_array_equal(Cs, C[rows, cols])


def test_sampled_fma_chain_exact_emulation():
    A = inputs.operand("f32_uniform", 3, 60, 5, ld=63).numpy()
    B = inputs.operand("f32_uniform", 60, 4, 6, ld=9).numpy()
    rows = np.array([0, 2, 1])
    cols = np.array([3, 0, 2])
    Cs, _ = oracle.gemm_sampled(A, B, rows, cols, "f32", fma_chain=True)
    for p in range(3):
        acc = Fraction(0)
        for k in range(60):
            acc = _round_f32(Fraction(float(A[rows[p], k])) * Fraction(float(B[k, cols[p]])) + acc)
        assert Cs[p] == np.float32(float(acc)), p


def test_K_zero_gives_zeros():
    C, S = oracle.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32), "f32")
    assert (C == 0).all() and (S == 0).all() and C.shape == (3, 4)


def test_rejects_mismatched_inner_dimension():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((3, 4), np.float32), np.zeros((5, 4), np.float32), "f32")
    with pytest.raises(ValueError):
        oracle.gemm_sampled(np.zeros((3, 4), np.float32), np.zeros((4, 4), np.float32),
                            [3], [0], "f32")
