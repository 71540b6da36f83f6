"""GPU: gemm_run_noalloc (the library's fixed device workspace) gives the
same C as gemm_run_ws with a caller workspace, bit for bit, on two calls in a
row (the second smaller), and rejects a repack larger than its array before
enqueueing anything.  Calls go through the C ABI."""
import pytest
import torch

from parity import check
from tiled_software_pipelined_amd import inputs

pytestmark = pytest.mark.gpu

tl = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global tl
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_software_pipelined_amd import lib
    tl = lib
    yield


def _padded(t, ld, off):
    """A device view of CPU operand t with row stride ld, starting `off`
    elements into a buffer of exactly the bytes it spans."""
    rows, cols = t.shape
    n = off + (rows - 1) * ld + cols
    buf = torch.zeros(n, dtype=t.dtype)
    view = buf[off:off + rows * ld - (ld - cols)].as_strided((rows, cols), (ld, 1)) if rows else buf[:0]
    view.copy_(t)
    d = buf.cuda()
    return d, d[off:].as_strided((rows, cols), (ld, 1))


def _case(dtype, M, N, K, lda, ldb, offa, offb, seed):
    kind = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}[dtype]
    code = {"f32": tl.F32, "bf16": tl.BF16, "i8": tl.I8}[dtype]
    A = inputs.operand(kind, M, K, seed)
    B = inputs.operand(kind, K, N, seed + 1)
    bufa, Ad = _padded(A, lda, offa)
    bufb, Bd = _padded(B, ldb, offb)
    plan = tl.Plan(M, N, K, code, lda, ldb, N)
    need = plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr())
    assert 0 < need <= tl.NOALLOC_MAX_BYTES, need
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    C_ws = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
    C_na = torch.full((M, N), -5, dtype=out_dtype, device="cuda")
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    stream = torch.cuda.current_stream().cuda_stream
    plan.run_ws_ptr(Ad.data_ptr(), Bd.data_ptr(), C_ws.data_ptr(), base, need, stream)
    plan.run_noalloc_ptr(Ad.data_ptr(), Bd.data_ptr(), C_na.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.equal(C_ws, C_na), (dtype, M, N, K)
    import oracle
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    ok, rep = check(C_na.cpu().numpy(), C_ref, S, dtype, K)
    assert ok, rep
    del bufa, bufb
    return need


def test_noalloc_matches_caller_workspace_twice():
    # fp32, whose kernels need aligned rows and so repack misaligned
    # operands: first call, B rows misaligned (ldb odd) and A at an odd
    # element offset; second call, smaller: both operands misaligned by
    # stride
    n1 = _case("f32", 1000, 1001, 1000, 1000, 1001, 3, 0, 71)
    n2 = _case("f32", 300, 257, 200, 203, 261, 0, 1, 73)
    assert n2 < n1


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_noalloc_reads_matrix_core_operands_in_place(dtype):
    # the matrix-core kernels read misaligned rows in place: no workspace,
    # gemm_run_noalloc is gemm_run, bit for bit
    M, N, K, lda, ldb = 300, 257, 200, 203, 261
    kind = {"bf16": "bf16_normal", "i8": "i8_uniform"}[dtype]
    bufa, Ad = _padded(inputs.operand(kind, M, K, 75), lda, 1)
    bufb, Bd = _padded(inputs.operand(kind, K, N, 76), ldb, 3)
    plan = tl.Plan(M, N, K, {"bf16": tl.BF16, "i8": tl.I8}[dtype], lda, ldb, N)
    assert plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr()) == 0
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    C0 = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
    C1 = torch.full((M, N), -5, dtype=out_dtype, device="cuda")
    plan.run_ptr(Ad.data_ptr(), Bd.data_ptr(), C0.data_ptr())
    plan.run_noalloc_ptr(Ad.data_ptr(), Bd.data_ptr(), C1.data_ptr())
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)
    del bufa, bufb


def test_noalloc_without_misaligned_operands_is_gemm_run():
    M, N, K = 512, 512, 256
    A = inputs.operand("bf16_normal", M, K, 81).cuda()
    B = inputs.operand("bf16_normal", K, N, 82).cuda()
    plan = tl.Plan(M, N, K, tl.BF16)
    assert plan.workspace_bytes(A.data_ptr(), B.data_ptr()) == 0
    C0 = torch.full((M, N), -7.0, device="cuda")
    C1 = torch.full((M, N), -5.0, device="cuda")
    plan.run_ptr(A.data_ptr(), B.data_ptr(), C0.data_ptr())
    plan.run_noalloc_ptr(A.data_ptr(), B.data_ptr(), C1.data_ptr())
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)


def test_noalloc_rejects_a_repack_beyond_its_array():
    # B (8192 x 4097 fp32) repacked to rows of 4128 elements: 135 MB > 64 MiB
    M, N, K = 1, 4097, 8192
    A = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    B = torch.zeros((K, N), dtype=torch.float32, device="cuda")
    plan = tl.Plan(M, N, K, tl.F32)
    need = plan.workspace_bytes(A.data_ptr(), B.data_ptr())
    assert need > tl.NOALLOC_MAX_BYTES
    C = torch.full((M, N), -7.0, device="cuda")
    with pytest.raises(tl.TgemmError) as e:
        plan.run_noalloc_ptr(A.data_ptr(), B.data_ptr(), C.data_ptr())
    assert e.value.code == -1 and str(need) in str(e.value)
    torch.cuda.synchronize()
    assert (C == -7.0).all()  # nothing was enqueued
