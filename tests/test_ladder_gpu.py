"""GPU: every rung of the ablation ladders against the oracle at the ladder's
size (4096^3), all outputs: int8 exactly, bf16 within the per-element gates,
fp32 bit for bit with the sequential fp32 fma chain.  Every matrix-core rung
and every tiled fp32 rung must also give the default plan's C bit for bit
(the SM80 ablation plan, section 1.3: variants may differ by exactly 0)."""
import numpy as np
import pytest
import torch

import oracle
from parity import check
from tiled_software_pipelined_amd import inputs, ladders

pytestmark = pytest.mark.gpu

tl = None
_ref = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global tl
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_software_pipelined_amd import lib
    tl = lib
    yield
    _ref.clear()


def _reference(dtype):
    """(A, B on the device, oracle C, S, fp32 chain or None, default plan's C)."""
    if dtype not in _ref:
        _ref.clear()
        w = inputs.workloads()[ladders.LADDER_WORKLOAD[dtype]]
        A_cpu, B_cpu = w.operands()
        print("oracle", w.name, flush=True)
        C_ref, S = oracle.gemm(inputs.as_oracle_array(A_cpu), inputs.as_oracle_array(B_cpu), dtype)
        chain = oracle.gemm_f32_fma_chain(A_cpu.numpy(), B_cpu.numpy()) if dtype == "f32" else None
        A, B = A_cpu.cuda(), B_cpu.cuda()
        out_dtype = torch.int32 if dtype == "i8" else torch.float32
        D = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda")
        tl.gemm(A, B, out=D)
        torch.cuda.synchronize()
        _ref[dtype] = (w, A, B, C_ref, S, chain, D)
    return _ref[dtype]


CASES = [(dt, r.label) for dt in ("bf16", "i8", "f32") for r in ladders.LADDERS[dt]]


@pytest.mark.parametrize("dtype,label", CASES)
def test_rung_against_oracle(dtype, label):
    w, A, B, C_ref, S, chain, D = _reference(dtype)
    rung = next(r for r in ladders.LADDERS[dtype] if r.label == label)
    v = None if rung.fields is None else tl.Variant(**rung.fields)
    code = {"f32": tl.F32, "bf16": tl.BF16, "i8": tl.I8}[dtype]
    name = tl.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N, v).name
    print(dtype, label, name, flush=True)
    C = torch.full_like(D, -7)
    tl.gemm(A, B, out=C, variant=v)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    ok, rep = check(Ch, C_ref, S, dtype, w.K)
    assert ok, (label, name, rep)
    if chain is not None:
        assert np.array_equal(Ch, chain), (label, name, int((Ch != chain).sum()))
    naive_bf16 = dtype == "bf16" and rung.fields is not None and rung.fields.get("kernel") == tl.KERNEL_NAIVE
    if not naive_bf16:
        assert torch.equal(C, D), (label, name)
