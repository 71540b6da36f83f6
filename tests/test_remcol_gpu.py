"""GPU: products one column wider than a whole number of 256 x 256 tile
columns (N = 16 k * 256 + 1 with at least 16 tile columns) compute that last
column inside the main kernel's K loop (the kernel's twin that copies, with
every slice, the 4 bytes of each B row that end at the column).  Checked
against the oracle on every output: int8 bit for bit, bf16 within the
per-element bound; with K tails, ragged M, B and A rows of any alignment,
offset pointers, buffers that end at the operands' last byte, and a padded C
row stride whose padding must stay untouched."""
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


DT = {"bf16": 1, "i8": 2}
KIND = {"bf16": "bf16_normal", "i8": "i8_uniform"}


def _exact_view(t, ld, off):
    """t on the GPU with row stride ld, `off` elements into a buffer that
    ends exactly at t's last element."""
    rows, cols = t.shape
    buf = torch.zeros(off + (rows - 1) * ld + cols, dtype=t.dtype)
    buf.as_strided((rows, cols), (ld, 1), off).copy_(t)
    return buf.cuda().as_strided((rows, cols), (ld, 1), off)


# one round of 256 x 256 tiles (16 x 16) for the main part: the planner's
# choice for these shapes (K above the short-K limit)
CASES = [  # dtype, M, N, K, lda - K, ldb - N, A offset, B offset, ldc - N
    ("bf16", 4096, 4097, 1100, 0, 0, 0, 0, 0),    # K tail of 12, B rows unaligned, exact buffers
    ("bf16", 4000, 4097, 1090, 1, 0, 1, 0, 3),    # ragged M, A rows and pointer unaligned
    ("bf16", 4096, 4097, 1088, 0, 7, 0, 3, 1),    # no K tail, B at an odd element offset
    ("i8", 4096, 4097, 2100, 0, 0, 0, 0, 0),      # K tail of 52
    ("i8", 4000, 4097, 2176, 3, 5, 1, 2, 2),      # no K tail, every operand unaligned
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_%dx%dx%d" % c[:4])
def test_last_column_in_the_k_loop(case):
    dtype, M, N, K, pa, pb, oa, ob, pc = case
    lda, ldb, ldc = K + pa, N + pb, N + pc
    plan = tl.Plan(M, N, K, DT[dtype], lda, ldb, ldc)
    info = plan.info()
    print("remcol", case, info.name.decode(), info.rem_name.decode(), flush=True)
    assert info.n_main == N - 1 and info.rem_name == info.name + b"_remcol"
    A = inputs.operand(KIND[dtype], M, K, 500 + K)
    B = inputs.operand(KIND[dtype], K, N, 600 + K)
    Ad, Bd = _exact_view(A, lda, oa), _exact_view(B, ldb, ob)
    assert plan.workspace_bytes(Ad.data_ptr(), Bd.data_ptr()) == 0
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    big = torch.full((M, ldc), -7, dtype=out_dtype, device="cuda")
    plan.run_ptr(Ad.data_ptr(), Bd.data_ptr(), big.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    big = big.cpu()
    assert (big[:, N:] == -7).all(), "wrote outside the M x N window"
    got = big[:, :N].numpy()
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    ok, rep = check(got, C_ref, S, dtype, K)
    assert ok, rep
    if dtype == "i8":
        assert np.array_equal(got.astype(np.int64), C_ref)
    else:
        # the last column on its own: fp32 sums of exact bf16 products, at
        # most K roundings (two per dot of two), each within 2^-24 of a
        # partial sum bounded by S: |err| <= K 2^-24 S
        err = np.abs(got[:, -1].astype(np.float64) - C_ref[:, -1])
        assert (err <= K * 2.0 ** -24 * S[:, -1]).all(), float((err / np.maximum(S[:, -1], 1e-30)).max())


def test_last_column_matches_the_main_kernel_on_the_other_columns():
    # the twin's first N - 1 columns are the plain kernel's, bit for bit (the
    # extra work only adds the last column): compare with the product on
    # the first N - 1 columns alone
    M, N, K = 4096, 4097, 1100
    A = inputs.operand("bf16_normal", M, K, 701)
    B = inputs.operand("bf16_normal", K, N, 702)
    Ad, Bd = A.cuda(), B.cuda()
    C = tl.gemm(Ad, Bd, workspace=False)
    C_main = tl.gemm(Ad, Bd[:, :N - 1], workspace=False)
    torch.cuda.synchronize()
    assert tl.Plan(M, N - 1, K, tl.BF16, K, N, N - 1).info().name == tl.Plan(M, N, K, tl.BF16).info().name
    assert torch.equal(C[:, :N - 1], C_main)
