"""Tolerance gates for comparing GPU results with the oracle.

Gates (per output element), with S = sum_k |a_ik b_kj| from the oracle:
  int8 -> int32      : exact equality;
  bf16 -> fp32 accum : |C - C_ref| <= 4e-3 * S;
  fp32 (vector FMA)  : |C - C_ref| <= 1e-5 * S.
A NaN or Inf in C fails; where S = 0 the result must be exactly 0.

A second, tighter check guards against a dropped K slice, which on random
data can hide inside the bf16 gate: with fp32 accumulation every partial sum
is rounded with relative error <= 2^-24, so |C - C_ref| <= K * 2^-24 * S
bounds the error of any summation order (Higham's recursive-summation bound;
products of bf16 or fp32 pairs are exact or rounded once).  The check uses
2 (K + 16) 2^-24 S, which also admits truncating rather than rounding adds
inside a matrix-core instruction.  A kernel that loses a K slice of 16-64
products errs by about sqrt(16..64) / (0.64 K) of S on N(0,1) data, several
times that bound on most elements.
"""
from __future__ import annotations

import numpy as np

GATE = {"bf16": 4e-3, "f32": 1e-5}


def check(C, C_ref, S, dtype: str, K: int):
    """Return (ok, report) for GPU result C vs oracle (C_ref, S)."""
    C = np.asarray(C)
    if dtype == "i8":
        C_ref = np.asarray(C_ref)
        bad = C.astype(np.int64) != C_ref
        return (not bad.any()), {"mismatches": int(bad.sum())}
    C = C.astype(np.float64)
    finite = np.isfinite(C).all()
    err = np.abs(C - C_ref)
    gate = GATE[dtype] * S
    zero_s = S == 0
    ok_gate = bool(finite and (err <= gate).all() and (C[zero_s] == 0).all())
    bound = 2.0 * (K + 16) * 2.0 ** -24 * S
    ok_bound = bool(finite and (err <= bound + 0.0).all())
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(S > 0, err / np.where(S > 0, S, 1), 0.0)
    report = {
        "finite": bool(finite),
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "rms_rel": float(np.sqrt((rel ** 2).mean())) if rel.size else 0.0,
        "gate_ok": ok_gate,
        "order_bound_ok": ok_bound,
    }
    return ok_gate and ok_bound, report
