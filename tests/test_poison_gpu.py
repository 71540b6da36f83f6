"""GPU: the poisoned-slot debug kernels (TGEMM_LDS_XOR_POISON).

Each lane of such a kernel fills the 16 LDS bytes its next direct copy will
write with all-ones bytes and waits for that store before issuing the copy.
A read of a ring slot before its copy has landed, or after the copy of a
later slice into it has begun, then sees NaN (bf16) or -1 (int8) instead of
plausible stale data, and the oracle check fails loudly (a NaN anywhere
fails it).  These tests run every poisoned kernel over shapes with many K
slices (the steady state of the ring, where a slice's copy overwrites the
slot the previous round read), a K tail and ragged edges, and require the
oracle gates and bit-identity with the kernel's ordinary twin: the poison
writes must never reach a chunk whose copy has been issued.
"""
import pytest
import torch

import oracle
from parity import check
from tiled_software_pipelined_amd import inputs

pytestmark = pytest.mark.gpu

tl = None

KIND = {"bf16": "bf16_normal", "i8": "i8_uniform"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global tl
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_software_pipelined_amd import lib
    tl = lib
    yield


def _poisoned(code):
    return [v for v in tl.variants(code) if v.lds_layout == tl.LDS_XOR_POISON]


def _twin(v):
    t = tl.Variant(**v.as_dict())
    t.lds_layout = tl.LDS_XOR
    return t


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
# rows 16-byte aligned for both types (the poisoned kernels are direct-loader
# kernels); a ragged M, N tile edge and a K tail in the middle shape
@pytest.mark.parametrize("M,N,K", [(512, 528, 2048), (300, 272, 1008), (1024, 1024, 4096)])
def test_poisoned_ring_matches_oracle_and_twin(dtype, M, N, K):
    code = {"bf16": tl.BF16, "i8": tl.I8}[dtype]
    vs = _poisoned(code)
    assert vs, "no poisoned kernels compiled"
    A = inputs.operand(KIND[dtype], M, K, 700 + K)
    B = inputs.operand(KIND[dtype], K, N, 800 + K)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    Ad, Bd = A.cuda(), B.cuda()
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    for v in vs:
        C = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
        tl.gemm(Ad, Bd, out=C, variant=v)
        C2 = torch.full((M, N), -5, dtype=out_dtype, device="cuda")
        tl.gemm(Ad, Bd, out=C2, variant=_twin(v))
        torch.cuda.synchronize()
        name = tl.Plan(M, N, K, code, variant=v).name
        assert "poison" in name, name
        ok, rep = check(C.cpu().numpy(), C_ref, S, dtype, K)
        assert ok, (name, rep)
        assert torch.equal(C, C2), name
