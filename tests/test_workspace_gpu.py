"""GPU: gemm_run_ws repacks operands whose rows are not 16-byte aligned into
the caller's workspace where the plan's kernel needs aligned rows (the fp32
kernels, and matrix-core plans whose B rows end in a partial 16-byte piece),
and gives the same product as gemm_run.  Plans whose kernels read rows of any
alignment (the direct-copy tiles, the thin kernel) need no workspace.

int8 and fp32 must agree bit for bit with gemm_run (exact / one fma chain
per output in increasing k on every kernel); bf16 too on shapes whose plans
give no columns to the thin kernel.  Every result is also checked against the
oracle.  A workspace smaller than gemm_workspace_bytes makes gemm_run_ws run
gemm_run's kernels; a misaligned workspace is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

import oracle
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


DT = {"f32": 0, "bf16": 1, "i8": 2}
KIND = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}
CE = {"f32": 4, "bf16": 8, "i8": 16}


def _exact_view(t, ld, off):
    """t on the GPU with row stride ld, `off` elements into a buffer that
    ends exactly at t's last element."""
    rows, cols = t.shape
    buf = torch.zeros(off + (rows - 1) * ld + cols, dtype=t.dtype)
    buf.as_strided((rows, cols), (ld, 1), off).copy_(t)
    return buf.cuda().as_strided((rows, cols), (ld, 1), off)


def _run(plan, Ad, Bd, M, N, dtype, ws=None, ws_bytes=0, ldc=None):
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    ldc = ldc or N
    big = torch.full((M, ldc), -7, dtype=out_dtype, device="cuda")
    C = big[:, :N]
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        plan.run_ptr(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), stream)
    else:
        plan.run_ws_ptr(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), ws, ws_bytes, stream)
    torch.cuda.synchronize()
    big = big.cpu()
    assert (big[:, N:] == -7).all(), "wrote outside the M x N window"
    return big[:, :N].clone()


def _workspace(nbytes):
    buf = torch.empty(nbytes + 512, dtype=torch.uint8, device="cuda")
    base = (buf.data_ptr() + 255) // 256 * 256
    return buf, base


CASES = [  # M, N, K, lda - K, ldb - N, A offset, B offset (elements)
    (300, 520, 200, 1, 1, 0, 0),
    (257, 208, 331, 0, 3, 0, 1),
    (130, 1000, 96, 2, 0, 1, 0),
    (512, 264, 517, 5, 7, 3, 5),
    (260, 333, 150, 2, 1, 1, 3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("case", CASES)
def test_workspace_matches_run_and_oracle(dtype, case):
    M, N, K, pa, pb, oa, ob = case
    A = inputs.operand(KIND[dtype], M, K, 91 + K)
    B = inputs.operand(KIND[dtype], K, N, 92 + N)
    lda, ldb = K + pa, N + pb
    Ad, Bd = _exact_view(A, lda, oa), _exact_view(B, ldb, ob)
    plan = tl.Plan(M, N, K, DT[dtype], lda, ldb, N)
    need = plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr())
    # fp32 kernels need aligned rows; the matrix-core plans read any in place
    assert (need > 0) == (dtype == "f32"), (need, plan.info().name)
    print("workspace", dtype, case, need, plan.info().name.decode(), flush=True)
    ref = _run(plan, Ad, Bd, M, N, dtype)
    buf, base = _workspace(need)
    got = _run(plan, Ad, Bd, M, N, dtype, base, need)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    ok, rep = check(got.numpy(), C_ref, S, dtype, K)
    assert ok, rep
    assert torch.equal(got, ref), (dtype, case)
    if need:
        # too small: gemm_run's kernels, same result
        small = _run(plan, Ad, Bd, M, N, dtype, base, need - 1)
        assert torch.equal(small, ref)
    del buf


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_workspace_reused_in_order_and_ldc(dtype):
    # two products share one workspace on one stream; C with a padded,
    # unaligned row stride
    M, N, K = 384, 393, 260
    A1 = inputs.operand(KIND[dtype], M, K, 95)
    B1 = inputs.operand(KIND[dtype], K, N, 96)
    A2 = inputs.operand(KIND[dtype], M, K, 97)
    B2 = inputs.operand(KIND[dtype], K, N, 98)
    lda, ldb = K + 1, N + 3
    plan = tl.Plan(M, N, K, DT[dtype], lda, ldb, N + 5)
    views = [(_exact_view(A1, lda, 0), _exact_view(B1, ldb, 0)), (_exact_view(A2, lda, 2), _exact_view(B2, ldb, 1))]
    need = max(plan.workspace_bytes(a.data_ptr(), b.data_ptr()) for a, b in views)
    buf, base = _workspace(need)
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    Cs = [torch.full((M, N + 5), -7, dtype=out_dtype, device="cuda") for _ in views]
    stream = torch.cuda.current_stream().cuda_stream
    for (a, b), c in zip(views, Cs):
        plan.run_ws_ptr(a.data_ptr(), b.data_ptr(), c.data_ptr(), base, need, stream)
    torch.cuda.synchronize()
    for (A, B), c in zip([(A1, B1), (A2, B2)], Cs):
        c = c.cpu()
        assert (c[:, N:] == -7).all()
        C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
        ok, rep = check(c[:, :N].numpy(), C_ref, S, dtype, K)
        assert ok, rep
    del buf


def test_workspace_must_be_256_byte_aligned():
    M, N, K = 64, 73, 33
    A = inputs.operand("f32_uniform", M, K, 99)
    B = inputs.operand("f32_uniform", K, N, 100)
    Ad, Bd = A.cuda(), B.cuda()
    plan = tl.Plan(M, N, K, 0, K, N, N)
    need = plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr())
    assert need > 0
    buf, base = _workspace(need + 256)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    with pytest.raises(tl.TgemmError) as e:
        plan.run_ws_ptr(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), base + 16, need, 0)
    assert e.value.code == -3
    torch.cuda.synchronize()
    del buf


def test_binding_uses_workspace_by_default():
    # the Python binding passes a workspace from torch's allocator where the
    # plan asks for one (here none: the direct-copy tiles read the unaligned
    # rows in place); with workspace=False never; same bits (no thin columns)
    M, N, K = 600, 776, 1030
    A = inputs.operand("bf16_normal", M, K, 101)
    B = inputs.operand("bf16_normal", K, N, 102)
    Ad, Bd = A.cuda(), B.cuda()  # K, N not multiples of 8: rows unaligned
    C1 = tl.gemm(Ad, Bd)
    C2 = tl.gemm(Ad, Bd, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), "bf16")
    ok, rep = check(C1.cpu().numpy(), C_ref, S, "bf16", K)
    assert ok, rep
    assert np.isfinite(C1.cpu().numpy()).all()


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("r", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("a_off", [0, 1])
def test_split_plan_reads_unaligned_rows_in_place(dtype, r, a_off):
    # 2048 x (2048 + r): 256 whole 128 x 128 tiles plus r columns for the
    # thin kernel.  B's rows (ldb = N + 1) are never 16-byte
    # aligned and, with a_off = 1, neither is A's pointer: every kernel reads
    # them in place, so the plan asks for no workspace and gemm_run_ws is
    # gemm_run.  The oracle's values (K = 264: a partial last slice).
    M, N, K = 2048, 2048 + r, 264
    A = inputs.operand(KIND[dtype], M, K, 300 + r)
    B = inputs.operand(KIND[dtype], K, N, 400 + r)
    lda, ldb = K + a_off, N + 1
    Ad, Bd = _exact_view(A, lda, a_off), _exact_view(B, ldb, 0)
    plan = tl.Plan(M, N, K, DT[dtype], lda, ldb, N)
    info = plan.info()
    print("split", dtype, r, a_off, info.name.decode(), info.rem_name.decode(), info.packed_name.decode(),
          flush=True)
    need = plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr())
    assert need == 0 and info.n_main == 2048 and info.rem_name
    buf, base = _workspace(need)
    got = _run(plan, Ad, Bd, M, N, dtype, base, need)
    ref = _run(plan, Ad, Bd, M, N, dtype)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    ok, rep = check(got.numpy(), C_ref, S, dtype, K)
    assert ok, rep
    if dtype == "i8":
        assert np.array_equal(got.numpy().astype(np.int64), C_ref)
    assert torch.equal(got, ref), (dtype, r, a_off)
    del buf
