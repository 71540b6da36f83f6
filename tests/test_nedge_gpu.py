"""GPU: products whose N is not a whole number of 16-byte pieces, at sizes of
a few thousand (no split: the last tile column is wider than the thin
kernel's), on the direct loader: the piece of each B row that crosses N is
copied in place, pieces past N come from the row's last whole piece or the
tile's first column, and B's last row goes through the register tail when K
is a whole number of slices.  All outputs against the oracle (int8 exactly),
with B in exactly sized buffers (its last row ends the allocation), unaligned
strides and pointers, and a padded C whose padding must stay untouched."""
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
    rows, cols = t.shape
    buf = torch.zeros(off + (rows - 1) * ld + cols, dtype=t.dtype)
    buf.as_strided((rows, cols), (ld, 1), off).copy_(t)
    return buf.cuda().as_strided((rows, cols), (ld, 1), off)


CASES = [  # dtype, M, N, K, lda - K, ldb - N, B offset, ldc - N
    ("bf16", 2000, 2068, 2048, 0, 0, 0, 0),    # K a whole number of slices: B's last row in the tail
    ("bf16", 2048, 2068, 2052, 1, 3, 1, 2),    # K tail of 4, every stride unaligned
    ("i8", 2000, 2068, 2048, 0, 0, 0, 0),
    ("i8", 2048, 2075, 2176, 3, 0, 5, 1),      # 2075 = 16 * 129 + 11
    ("bf16", 4000, 4092, 4096, 0, 0, 0, 0),    # the 256 x 256 tile: last tile column 252 wide
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_%dx%dx%d" % c[:4])
def test_partial_last_piece_read_in_place(case):
    dtype, M, N, K, pa, pb, ob, pc = case
    lda, ldb, ldc = K + pa, N + pb, N + pc
    plan = tl.Plan(M, N, K, DT[dtype], lda, ldb, ldc)
    info = plan.info()
    print("nedge", case, info.name.decode(), flush=True)
    assert info.variant.loader == tl.LOADER_DIRECT and info.b_guarded == 1 and info.n_main == N
    A = inputs.operand(KIND[dtype], M, K, 800 + K)
    B = inputs.operand(KIND[dtype], K, N, 900 + K)
    Ad, Bd = _exact_view(A, lda, 0), _exact_view(B, ldb, ob)
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
