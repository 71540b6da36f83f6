"""GPU parity on seeded random products: shapes, row strides, pointer offsets
and the workspace switch drawn at random, each compared with the CPU oracle
element by element (int8 exact; bf16 and fp32 within the per-element gates of
tests/parity.py).

The shape classes follow the planner's branches: small products of every
kind, thin products (N <= 16), split plans (a tiled main part plus a
remainder of 1-16 columns), mid-size products on the tiled kernels, and
large ones with K > 512, a third of them one column past 16 x 16 tiles of
256 x 256 (the column computed inside the main K loop).  Each
operand sits at the end of a buffer sized to its last element, offset by up
to 7 elements from the buffer's start, so rows and pointers take every
alignment; C is written into a padded buffer whose padding must stay intact.
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
    from tiled_software_pipelined_amd import lib  # must load: there is no fallback
    tl = lib
    yield


KIND = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}
N_CASES = 100


def _case(i):
    """The i-th case: (dtype, M, N, K, pad_a, pad_b, pad_c, off_a, off_b, workspace)."""
    r = np.random.RandomState(1000 + i)
    dtype = ("bf16", "i8", "f32")[r.randint(3)]
    cls = i % 5
    if cls == 0:    # small
        M, N, K = r.randint(1, 300), r.randint(1, 300), r.randint(1, 300)
    elif cls == 1:  # thin
        M, N, K = r.randint(1, 3000), r.randint(1, 17), r.randint(1, 2000)
    elif cls == 2:  # split: 2048 or 4096 columns of whole tiles plus a remainder
        M, N, K = r.randint(1000, 4100), (2048, 4096)[r.randint(2)] + r.randint(1, 17), r.randint(1, 600)
    elif cls == 3:  # mid-size
        M, N, K = r.randint(200, 1100), r.randint(200, 1100), r.randint(1, 700)
    elif r.rand() < 0.34:  # 16 x 16 tiles of 256 x 256 and one column more
        M, N, K = r.randint(3841, 4097), 4097, r.randint(513, 1100)
    else:           # large, K > 512
        M, N, K = r.randint(2000, 4100), r.randint(2000, 4400), r.randint(513, 1100)
    pads = [0 if r.rand() < 0.4 else int(r.randint(1, 10)) for _ in range(3)]
    offs = [0 if r.rand() < 0.4 else int(r.randint(1, 8)) for _ in range(2)]
    return (dtype, M, N, K, pads[0], pads[1], pads[2], offs[0], offs[1], bool(r.rand() < 0.5))


def _device_view(t, ld, off):
    """t on the GPU with row stride ld, `off` elements into a buffer that ends
    exactly at its last element."""
    rows, cols = t.shape
    buf = torch.zeros(off + (rows - 1) * ld + cols, dtype=t.dtype)
    buf.as_strided((rows, cols), (ld, 1), off).copy_(t)
    return buf.cuda().as_strided((rows, cols), (ld, 1), off)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_product(i):
    dtype, M, N, K, pa, pb, pc, oa, ob, ws = c = _case(i)
    print("case", i, c, flush=True)
    A = inputs.operand(KIND[dtype], M, K, 5000 + 2 * i)
    B = inputs.operand(KIND[dtype], K, N, 5001 + 2 * i)
    Ad, Bd = _device_view(A, K + pa, oa), _device_view(B, N + pb, ob)
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    big = torch.full((M, N + pc), -7, dtype=out_dtype, device="cuda")
    tl.gemm(Ad, Bd, out=big[:, :N], workspace=ws)
    torch.cuda.synchronize()
    big = big.cpu()
    assert (big[:, N:] == -7).all(), "wrote outside the M x N window"
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    ok, rep = check(big[:, :N].numpy(), C_ref, S, dtype, K)
    assert ok, (c, rep)
