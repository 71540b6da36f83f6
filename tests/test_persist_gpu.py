"""GPU parity of the persistent kernel (TGEMM_KERNEL_PERSISTENT) through the C ABI.

Each workgroup walks several tiles with one copy ring and two accumulator
sets, and writes a tile's C block during the next tile's first slices.  What
can go wrong is the bookkeeping across tiles: which tile a workgroup takes
next, which slice the ring copies, which accumulator set is stored where and
when, the wait counts that let the stores stay in flight.  So every case
runs with grids that give each workgroup one tile, several tiles, an odd
number, unequal numbers (the tile count not a multiple of the grid), and
the XCD-major rank (grid a multiple of 8) as well as the plain one; every
output is compared with the oracle (int8 exactly, bf16 by the gate of
tests/parity.py) and with the tiled kernel bit for bit (the same matrix
instructions in the same K order).
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


DT = {"bf16": 1, "i8": 2}
KIND = {"bf16": "bf16_normal", "i8": "i8_uniform"}


def _persistent(dtype):
    return [v for v in tl.variants(DT[dtype]) if v.kernel == tl.KERNEL_PERSISTENT]


def _with(v, **kw):
    d = v.as_dict()
    d.update(kw)
    return tl.Variant(**d)


def _run(Ad, Bd, variant, C=None):
    M, N = Ad.shape[0], Bd.shape[1]
    out_dtype = torch.int32 if Ad.dtype == torch.int8 else torch.float32
    if C is None:
        C = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
    tl.gemm(Ad, Bd, out=C, variant=variant)
    torch.cuda.synchronize()
    return C


def _tiled(dtype):
    # the default 256 x 256 tiled kernel (swapped product, 16-byte stores):
    # the reference for bit-equality
    return tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, tile_k=64 if dtype == "bf16" else 128,
                      stages=2, loader=tl.LOADER_DIRECT, waves_m=2, waves_n=4)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_every_persistent_variant_every_grid(dtype):
    vs = _persistent(dtype)
    assert {v.c_slices for v in vs} == {4, 8}
    assert {(v.tile_m, v.tile_n) for v in vs} == {(256, 128), (128, 256)}
    bk = vs[0].tile_k
    # 768 x 1024: 24 tiles of either shape; K: the fewest slices the deeper
    # variant takes, then a longer K
    M, N = 768, 1024
    for K in (bk * 10, bk * 13):
        A = inputs.operand(KIND[dtype], M, K, 31 + K)
        B = inputs.operand(KIND[dtype], K, N, 37 + K)
        C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
        Ad, Bd = A.cuda(), B.cuda()
        ref_bits = _run(Ad, Bd, _tiled(dtype)).cpu()
        ok, rep = check(ref_bits.numpy(), C_ref, S, dtype, K)
        assert ok, ("tiled reference", rep)
        # grids: 1 (every tile on one workgroup), 3 (8 tiles each, plain
        # rank), 5 (5 or 4 tiles: unequal), 8 (3 each, XCD-major rank), 16
        # (XCD-major, 2 or 1 each), 0 (the device: one tile each)
        for v in vs:
            for wgs in (1, 3, 5, 8, 16, 0):
                vv = _with(v, workgroups=wgs)
                p = tl.plan_for(M, N, K, DT[dtype], K, N, N, vv)
                info = p.info()
                assert "persist" in info.name.decode()
                assert info.grid == (24 if wgs == 0 else wgs), (info.grid, wgs)
                print("  %s K=%d workgroups=%d" % (info.name.decode(), K, wgs), flush=True)
                C = _run(Ad, Bd, vv).cpu()
                ok, rep = check(C.numpy(), C_ref, S, dtype, K)
                assert ok, (info.name.decode(), K, wgs, rep)
                if dtype == "i8":
                    assert np.array_equal(C.numpy().astype(np.int64), C_ref)
                assert torch.equal(C, ref_bits), (info.name.decode(), K, wgs)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_persistent_c_rows_not_16_byte_aligned(dtype):
    # ldc = N + 1: 4-byte stores (more store instructions than the waits
    # count on), nothing outside the M x N window written
    v = _with(_persistent(dtype)[0], workgroups=5)
    M, N, K = 512, 512, v.tile_k * (v.c_slices + 2)
    A = inputs.operand(KIND[dtype], M, K, 41)
    B = inputs.operand(KIND[dtype], K, N, 43)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    big = torch.full((M, N + 1), -7, dtype=out_dtype, device="cuda")
    C = _run(A.cuda(), B.cuda(), v, C=big[:, :N])
    big = big.cpu()
    assert (big[:, N:] == -7).all(), "wrote outside the M x N window"
    ok, rep = check(big[:, :N].numpy(), C_ref, S, dtype, K)
    assert ok, rep


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_persistent_misaligned_operand_takes_the_fallback(dtype):
    # an A pointer one element past a 16-byte boundary: the plan runs its
    # register-staged fallback, with the same result
    v = _persistent(dtype)[0]
    M, N, K = 512, 512, v.tile_k * (v.c_slices + 2)
    A = inputs.operand(KIND[dtype], M, K, 47)
    B = inputs.operand(KIND[dtype], K, N, 53)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)
    store = torch.zeros(M * K + 16, dtype=A.dtype, device="cuda")
    Ad = store[1:1 + M * K].view(M, K)
    Ad.copy_(A.cuda())
    C = _run(Ad, B.cuda(), v).cpu()
    ok, rep = check(C.numpy(), C_ref, S, dtype, K)
    assert ok, rep


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_persistent_clocked_run(dtype):
    # the clock marks of every launched workgroup: start <= loop end <= end
    v = _with(_persistent(dtype)[0], workgroups=8)
    M, N, K = 768, 1024, v.tile_k * (v.c_slices + 2)
    A = inputs.operand(KIND[dtype], M, K, 59).cuda()
    B = inputs.operand(KIND[dtype], K, N, 61).cuda()
    p = tl.plan_for(M, N, K, DT[dtype], K, N, N, v)
    slots = p.clock_slots()
    assert slots >= tl.CLOCK_VALUES * 8
    clk = torch.zeros(slots, dtype=torch.int64, device="cuda")
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    C = torch.empty((M, N), dtype=out_dtype, device="cuda")
    p.run_clocked_ptr(A.data_ptr(), B.data_ptr(), C.data_ptr(), clk.data_ptr(), slots,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    c = clk.cpu().numpy().view("uint64").reshape(-1, tl.CLOCK_VALUES)[:8].astype(np.int64)
    assert (c[:, 0] <= c[:, 2]).all() and (c[:, 2] <= c[:, 4]).all()
    assert (c[:, 1] <= c[:, 3]).all() and (c[:, 3] <= c[:, 5]).all()
    assert (c[:, 1] > 0).all()
    assert torch.equal(C, _run(A, B, _tiled(dtype)))


def test_persistent_repeated_runs_identical():
    v = _persistent("bf16")[-1]
    M, N, K = 1024, 768, v.tile_k * (v.c_slices + 4)
    A = inputs.operand("bf16_normal", M, K, 67).cuda()
    B = inputs.operand("bf16_normal", K, N, 71).cuda()
    first = _run(A, B, _with(v, workgroups=7))
    for _ in range(3):
        assert torch.equal(_run(A, B, _with(v, workgroups=7)), first)
