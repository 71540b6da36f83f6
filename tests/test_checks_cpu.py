"""CPU: the input generator is deterministic per seed, and the parity gates
of tests/parity.py catch the mistakes they exist for.

The gate check is exercised on an fp32 result computed on the CPU from the
same operands (which must pass) and on copies with one planted mistake each:
a dropped K slice of 32 products (the pipeline's forgotten epilogue), one
element's sign, one NaN, and an int8 result off by one.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check
from tiled_software_pipelined_amd import inputs


@pytest.mark.parametrize("kind", sorted(inputs.KINDS))
def test_operands_are_deterministic_per_seed(kind):
    a = inputs.operand(kind, 33, 70, 12345)
    b = inputs.operand(kind, 33, 70, 12345)
    c = inputs.operand(kind, 33, 70, 12346)
    assert a.dtype == inputs.KINDS[kind]
    assert torch.equal(a, b)
    assert not torch.equal(a, c)
    # a padded view holds the same values, with a non-zero filler past each row
    p = inputs.operand(kind, 33, 70, 12345, ld=80)
    assert p.stride(0) == 80 and torch.equal(p, a)
    full = p.as_strided((33, 80), (80, 1))
    assert (full[:, 70:] != 0).all()


def test_operand_distributions():
    x = inputs.operand("bf16_normal", 256, 256, 1).float()
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    u = inputs.operand("f32_uniform", 256, 256, 2)
    assert float(u.min()) >= -1.0 and float(u.max()) < 1.0
    i = inputs.operand("i8_uniform", 256, 256, 3)
    assert int(i.min()) == -128 and int(i.max()) == 127


def _fp32_result(A, B):
    # fp32 accumulation in increasing k on the CPU: what a correct kernel gives
    return (A.float() @ B.float()).numpy()


def test_gates_pass_a_correct_fp32_accumulation_and_catch_planted_mistakes():
    M, N, K = 64, 48, 512
    A = inputs.operand("bf16_normal", M, K, 41)
    B = inputs.operand("bf16_normal", K, N, 42)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), "bf16")
    C = _fp32_result(A, B)
    ok, _ = check(C, C_ref, S, "bf16", K)
    assert ok
    # a dropped slice of 32 products (k in [256, 288)) on every element
    drop = (A[:, 256:288].float() @ B[256:288, :].float()).numpy()
    ok, _ = check(C - drop, C_ref, S, "bf16", K)
    assert not ok
    for plant in ("sign", "nan"):
        bad = C.copy()
        if plant == "sign":
            bad[3, 5] = -bad[3, 5]
        else:
            bad[3, 5] = np.nan
        ok, _ = check(bad, C_ref, S, "bf16", K)
        assert not ok, plant


def test_int8_gate_is_exact():
    A = inputs.operand("i8_uniform", 16, 64, 51)
    B = inputs.operand("i8_uniform", 64, 24, 52)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), "i8")
    C = (A.long() @ B.long()).numpy()
    assert check(C, C_ref, S, "i8", 64)[0]
    C[7, 9] += 1
    assert not check(C, C_ref, S, "i8", 64)[0]
