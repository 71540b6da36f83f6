"""GPU parity: libtgemm (through its C ABI) against the CPU oracle.

Every case generates seeded operands on the CPU, runs the HIP kernel through
the C ABI, and compares with the oracle element by element on small, edge
and ragged shapes (the full-size workloads are compared in full in
test_fullsize_gpu.py).  Gates: int8 exact; bf16 and fp32 within
the per-element tolerances of tests/parity.py.  Integer-valued inputs must be
exact on every path, the fp32 kernels must equal the sequential fp32 fma chain
bit for bit, and all matrix-core variants (tile, stages, loader, layout,
workgroup order) must agree bit for bit, since pipelining only reorders loads.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check
from tiled_software_pipelined_amd import inputs

pytestmark = pytest.mark.gpu

tl = None  # the binding, loaded by the fixture below (it must load wherever a GPU is present)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    global tl
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_software_pipelined_amd import lib  # must load: there is no fallback
    tl = lib
    yield


DT = {"f32": 0, "bf16": 1, "i8": 2}
KIND = {"f32": "f32_uniform", "bf16": "bf16_normal", "i8": "i8_uniform"}


def _to_device(t):
    """Copy a (possibly row-padded) CPU operand to the GPU keeping its row stride."""
    rows, cols = t.shape
    ld = t.stride(0) if rows > 1 else cols
    if ld == cols or rows == 0 or cols == 0:
        return t.contiguous().cuda()
    big = torch.zeros((rows, ld), dtype=t.dtype)
    big.as_strided((rows, ld), (ld, 1)).copy_(t.as_strided((rows, ld), (ld, 1)))
    return big.cuda()[:, :cols]


def _run(A, B, variant=None, ldc=None):
    Ad, Bd = _to_device(A), _to_device(B)
    M, N = A.shape[0], B.shape[1]
    out_dtype = torch.int32 if A.dtype == torch.int8 else torch.float32
    if ldc is None or ldc == N:
        C = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
        tl.gemm(Ad, Bd, out=C, variant=variant)
        torch.cuda.synchronize()
        return C.cpu()
    big = torch.full((M, ldc), -7, dtype=out_dtype, device="cuda")
    C = big[:, :N]
    tl.gemm(Ad, Bd, out=C, variant=variant)
    torch.cuda.synchronize()
    big = big.cpu()
    assert (big[:, N:] == -7).all(), "wrote outside the M x N window"
    return big[:, :N]


def _oracle(A, B, dtype):
    return oracle.gemm(inputs.as_oracle_array(A), inputs.as_oracle_array(B), dtype)


def _assert_parity(C, A, B, dtype):
    C_ref, S = _oracle(A, B, dtype)
    ok, rep = check(C.numpy(), C_ref, S, dtype, A.shape[1])
    assert ok, rep
    return C_ref


def _variants(dtype, tiled_only=False):
    out = []
    for v in tl.variants(DT[dtype]):
        if tiled_only and v.kernel != tl.KERNEL_TILED:
            continue
        out.append(v)
    return out


def _vname(v):
    return "t%dx%dx%d_w%dx%d_s%d_l%d_y%d_a%d_f%d_st%d" % (v.tile_m, v.tile_n, v.tile_k, v.waves_m, v.waves_n,
                                                        v.stages, v.loader, v.lds_layout, v.access, v.frag,
                                                        v.store)


# ---------------------------------------------------------------- small shapes

@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_f32_256_style_full_check(dtype):
    M = N = K = 256
    A = inputs.operand(KIND[dtype], M, K, 11)
    B = inputs.operand(KIND[dtype], K, N, 12)
    _assert_parity(_run(A, B), A, B, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "i8", "f32"])
def test_every_variant_matches_oracle_and_each_other(dtype):
    # ragged in all three dimensions, several tiles, K tail, K < slice * stages
    for (M, N, K) in [(300, 520, 232), (129, 257, 40), (64, 64, 16)]:
        A = inputs.operand(KIND[dtype], M, K, M + K)
        B = inputs.operand(KIND[dtype], K, N, N + K)
        C_ref, S = _oracle(A, B, dtype)
        first_tiled = None
        for v in _variants(dtype):
            C = _run(A, B, variant=v)
            ok, rep = check(C.numpy(), C_ref, S, dtype, K)
            assert ok, (dtype, (M, N, K), _vname(v), rep)
            if v.kernel == tl.KERNEL_TILED:
                if first_tiled is None:
                    first_tiled = C
                elif dtype != "f32":
                    # one matrix-core K order for every tile / stage / loader / layout
                    assert torch.equal(C, first_tiled), (dtype, (M, N, K), _vname(v))


@pytest.mark.parametrize("dtype", ["bf16", "i8", "f32"])
@pytest.mark.parametrize("M,N", [(1, 1), (1, 129), (127, 1), (128, 128), (129, 127), (255, 257)])
@pytest.mark.parametrize("K", [1, 7, 8, 31, 33, 64, 96, 127, 128, 129])
def test_edge_shapes_default_plan(dtype, M, N, K):
    A = inputs.operand(KIND[dtype], M, K, 3 * M + K)
    B = inputs.operand(KIND[dtype], K, N, 5 * N + K)
    _assert_parity(_run(A, B), A, B, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_short_K_with_deep_rings(dtype):
    # fewer K slices than stages - 1: the prologue must not over-issue
    for v in _variants(dtype, tiled_only=True):
        for slices in (1, 2, 3):
            K = slices * v.tile_k
            A = inputs.operand(KIND[dtype], 200, K, 7 + K)
            B = inputs.operand(KIND[dtype], K, 300, 9 + K)
            C_ref, S = _oracle(A, B, dtype)
            ok, rep = check(_run(A, B, variant=v).numpy(), C_ref, S, dtype, K)
            assert ok, (_vname(v), K, rep)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_edge_K_across_ring_depths(dtype):
    # the K edge sweep on every direct-loader ring depth (1-4 and 8 slots,
    # the production 256 x 256 tile, the half tiles) with ragged M and N:
    # whole slices only, a partial last slice, fewer slices than the ring
    # rows 16-byte aligned (A padded to 64 elements per row) so that every
    # plan runs the requested direct-loader kernel
    M, N = 129, 272
    vs = [v for v in _variants(dtype, tiled_only=True)
          if v.loader == tl.LOADER_DIRECT and v.lds_layout == tl.LDS_XOR]
    assert {v.stages for v in vs} >= {1, 2, 3, 4, 8}
    for K in (1, 7, 8, 31, 32, 33, 64, 96, 127, 128, 4104):
        A = inputs.operand(KIND[dtype], M, K, 17 + K, ld=(K + 63) // 64 * 64)
        B = inputs.operand(KIND[dtype], K, N, 19 + K)
        C_ref, S = _oracle(A, B, dtype)
        first = None
        for v in vs:
            name = tl.Plan(M, N, K, DT[dtype], (K + 63) // 64 * 64, N, N, v).name
            assert "direct" in name, (name, K)
            C = _run(A, B, variant=v)
            ok, rep = check(C.numpy(), C_ref, S, dtype, K)
            assert ok, (_vname(v), K, rep)
            if first is None:
                first = C
            else:
                assert torch.equal(C, first), (_vname(v), K)


def test_fp32_equals_sequential_fma_chain_bitwise():
    for (M, N, K) in [(256, 256, 256), (130, 200, 77)]:
        A = inputs.operand("f32_uniform", M, K, 21 + K)
        B = inputs.operand("f32_uniform", K, N, 22 + K)
        ref = oracle.gemm_f32_fma_chain(A.numpy(), B.numpy())
        for v in _variants("f32"):
            C = _run(A, B, variant=v).numpy()
            assert np.array_equal(C, ref), (_vname(v), int((C != ref).sum()))


# ------------------------------------------------------ exact integer inputs

def _as_dtype(x, dtype):
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return {"f32": t, "bf16": t.to(torch.bfloat16), "i8": t.to(torch.int8)}[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_integer_valued_inputs_are_exact(dtype):
    rng = np.random.default_rng(1)
    # all-ones with the ragged K: C == K everywhere
    K = 4104
    C = _run(_as_dtype(np.ones((130, K)), dtype), _as_dtype(np.ones((K, 260)), dtype))
    assert (C == K).all()
    # rank-1 with known sums
    M, N, K = 257, 300, 520
    u, v = rng.integers(-4, 5, M), rng.integers(-4, 5, N)
    x, y = rng.integers(-1, 3, K), rng.integers(-1, 3, K)
    C = _run(_as_dtype(np.outer(u, x), dtype), _as_dtype(np.outer(y, v), dtype))
    assert (C.numpy() == np.outer(u, v) * int(np.dot(x, y))).all()
    # identity and a permutation
    n = 384
    B = rng.integers(-100, 100, size=(n, 200))
    assert (_run(_as_dtype(np.eye(n), dtype), _as_dtype(B, dtype)).numpy() == B).all()
    perm = rng.permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1
    assert (_run(_as_dtype(P, dtype), _as_dtype(B, dtype)).numpy() == B[perm]).all()


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_permutation_products_every_variant(dtype):
    # the one-hot lane-layout probe, for every matrix-core variant: with P and
    # Q permutation matrices each output of P Q holds exactly one product, so a
    # wrong fragment row / column, K position or output lane moves or drops a
    # 1 (n = 384: a whole and a ragged 256-wide tile, several slices)
    rng = np.random.default_rng(7)
    n = 384
    P = np.zeros((n, n))
    P[np.arange(n), rng.permutation(n)] = 1
    Q = np.zeros((n, n))
    Q[np.arange(n), rng.permutation(n)] = 1
    want = P @ Q
    for v in _variants(dtype, tiled_only=True):
        C = _run(_as_dtype(P, dtype), _as_dtype(Q, dtype), variant=v).numpy()
        assert (C == want).all(), _vname(v)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_hadamard(dtype):
    H = np.array([[1]])
    for _ in range(9):
        H = np.block([[H, H], [H, -H]])
    n = H.shape[0]  # 512
    C = _run(_as_dtype(H, dtype), _as_dtype(H.T.copy(), dtype)).numpy()
    assert (C == n * np.eye(n)).all()


def test_int8_extremes_at_full_K():
    K = 4096
    C = _run(torch.full((300, K), -128, dtype=torch.int8), torch.full((K, 260), -128, dtype=torch.int8))
    assert (C == 67108864).all()
    C = _run(torch.full((300, K), -128, dtype=torch.int8), torch.full((K, 260), 127, dtype=torch.int8))
    assert (C == -66584576).all()


# ------------------------------------------------ layouts and boundary cases

@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_padded_leading_dimensions(dtype):
    M, N, K = 200, 136, 96
    A = inputs.operand(KIND[dtype], M, K, 31, ld=K + 32)
    B = inputs.operand(KIND[dtype], K, N, 32, ld=N + 64)
    C = _run(A, B, ldc=N + 24)
    _assert_parity(C, A, B, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_unaligned_leading_dimensions_and_pointers(dtype):
    M, N, K = 150, 131, 101  # odd N and K: rows not 16-byte aligned
    A = inputs.operand(KIND[dtype], M, K, 41)
    B = inputs.operand(KIND[dtype], K, N, 42)
    _assert_parity(_run(A, B), A, B, dtype)
    # pointers aligned to the element but not to 16 bytes
    K2, N2 = 128, 256
    Aw = inputs.operand(KIND[dtype], M, K2 + 1, 43)
    Bw = inputs.operand(KIND[dtype], K2, N2 + 1, 44)
    A2, B2 = Aw[:, 1:], Bw[:, 1:]
    Ad = Aw.cuda()[:, 1:]
    Bd = Bw.cuda()[:, 1:]
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    C = torch.empty((M, N2), dtype=out_dtype, device="cuda")
    tl.gemm(Ad, Bd, out=C)
    torch.cuda.synchronize()
    _assert_parity(C.cpu(), A2, B2, dtype)


def _exact_device_view(t, ld, off):
    """t copied to the GPU with row stride ld, starting `off` elements into a
    buffer that ends exactly at t's last element."""
    rows, cols = t.shape
    buf = torch.zeros(off + (rows - 1) * ld + cols, dtype=t.dtype)
    buf.as_strided((rows, cols), (ld, 1), off).copy_(t)
    return buf.cuda().as_strided((rows, cols), (ld, 1), off)


def _run_views(Ad, Bd, variant):
    out_dtype = torch.int32 if Ad.dtype == torch.int8 else torch.float32
    C = torch.full((Ad.shape[0], Bd.shape[1]), -7, dtype=out_dtype, device="cuda")
    tl.gemm(Ad, Bd, out=C, variant=variant)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_shifted_loads_every_byte_offset(dtype):
    # Rows that are not 16-byte aligned go through pairs of aligned 16-byte
    # loads and a funnel shift.  Odd leading dimensions give consecutive rows
    # every byte offset (all 16 for int8, all 8 even ones for bf16); the
    # pointer offsets put the first and last pairs against the ends of
    # exactly sized buffers, where the checked form must fall back to element
    # loads.  K spans the first, interior, last and partial slices.  Every
    # register-staged variant must match the oracle and, bit for bit, itself
    # on 16-byte aligned copies of the same operands.
    ce = 8 if dtype == "bf16" else 16
    vs = [v for v in _variants(dtype, tiled_only=True)
          if v.loader == tl.LOADER_VGPR and v.access == tl.ACCESS_WIDE]
    assert vs
    for v in vs:
        M, N, K = 161, 208, 5 * v.tile_k + 3
        A = inputs.operand(KIND[dtype], M, K, 61 + K)
        B = inputs.operand(KIND[dtype], K, N, 62 + K)
        lda_al = (K + ce - 1) // ce * ce
        ref = _run_views(_exact_device_view(A, lda_al, 0), _exact_device_view(B, N, 0), v)
        _assert_parity(ref, A, B, dtype)
        # both operands misaligned; then B only and A only, by stride and by pointer
        for (lda, ldb, oa, ob) in [(K, N + 1, 0, 0), (K + 2, N + 3, 1, ce - 1), (lda_al, N, ce // 2, 1),
                                   (K + 1, N + ce + 1, ce - 1, ce // 2),
                                   (lda_al, N + 1, 0, 0), (lda_al, N, 0, 1), (lda_al, N + 3, 0, ce - 1),
                                   (K, N, 0, 0), (lda_al, N, 1, 0), (K + 2, N, ce - 1, 0)]:
            print("shifted", dtype, _vname(v), lda, ldb, oa, ob, flush=True)
            C = _run_views(_exact_device_view(A, lda, oa), _exact_device_view(B, ldb, ob), v)
            assert torch.equal(C, ref), (_vname(v), lda, ldb, oa, ob)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_shifted_loads_few_slices(dtype):
    # one, two and three whole slices (no interior slice, or one), with and
    # without a partial slice, on every register-staged variant
    ce = 8 if dtype == "bf16" else 16
    for v in _variants(dtype, tiled_only=True):
        if v.loader != tl.LOADER_VGPR or v.access != tl.ACCESS_WIDE:
            continue
        for K in (v.tile_k, v.tile_k + 5, 2 * v.tile_k, 2 * v.tile_k + 5, 3 * v.tile_k, 3 * v.tile_k + 5):
            M, N = 300, 520
            A = inputs.operand(KIND[dtype], M, K, 71 + K)
            B = inputs.operand(KIND[dtype], K, N, 72 + K)
            C_ref, S = _oracle(A, B, dtype)
            lda_al = (K + ce - 1) // ce * ce
            for (lda, ldb, oa, ob) in [(K + 1, N + 1, 1, ce - 1), (lda_al, N + 1, 0, 0), (K + 1, N, 0, 0)]:
                C = _run_views(_exact_device_view(A, lda, oa), _exact_device_view(B, ldb, ob), v)
                ok, rep = check(C.numpy(), C_ref, S, dtype, K)
                assert ok, (_vname(v), K, lda, ldb, oa, ob, rep)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("k_bytes", [384, 4160])
def test_streaming_and_plain_C_stores_agree(dtype, k_bytes):
    # C rows 128-byte aligned take non-temporal stores (on 256 x 256 tiles
    # only when K spans at least 4 KiB per row), others plain ones; both must
    # write the same values and nothing outside the M x N window
    M, N = 300, 256
    K = k_bytes // (1 if dtype == "i8" else 2)
    A = inputs.operand(KIND[dtype], M, K, 81)
    B = inputs.operand(KIND[dtype], K, N, 82)
    Ad, Bd = _to_device(A), _to_device(B)
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    ref = None
    for ldc, off in [(N, 0), (N + 1, 0), (N + 32, 0), (N, 1), (N + 5, 3)]:
        buf = torch.full((off + M * ldc + 64,), -7, dtype=out_dtype, device="cuda")
        C = buf.as_strided((M, N), (ldc, 1), off)
        tl.gemm(Ad, Bd, out=C)
        torch.cuda.synchronize()
        got = C.cpu().clone()
        mask = torch.ones(buf.numel(), dtype=torch.bool)
        mask.as_strided((M, N), (ldc, 1), off).fill_(False)
        assert (buf.cpu()[mask] == -7).all(), (ldc, off)
        if ref is None:
            ref = got
            _assert_parity(got, A, B, dtype)
        assert torch.equal(got, ref), (ldc, off)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_c_store_policies_agree(dtype):
    # the 256 x 256 tile at a short K (plain stores under AUTO) and a long
    # one (streaming): every policy writes the same bits, inside the window
    # only, on line-aligned and unaligned C
    M, N = 512, 512
    v = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, waves_n=4, loader=tl.LOADER_DIRECT)
    out_dtype = torch.int32 if dtype == "i8" else torch.float32
    try:
        for K in (256, 4160):
            A = inputs.operand(KIND[dtype], M, K, 83 + K)
            B = inputs.operand(KIND[dtype], K, N, 84 + K)
            Ad, Bd = _to_device(A), _to_device(B)
            ref = None
            for policy in (tl.C_STORES_AUTO, tl.C_STORES_STREAM, tl.C_STORES_PLAIN):
                tl.set_c_store_policy(policy)
                for ldc, off in [(N, 0), (N + 1, 0), (N, 1)]:
                    buf = torch.full((off + M * ldc + 64,), -7, dtype=out_dtype, device="cuda")
                    C = buf.as_strided((M, N), (ldc, 1), off)
                    tl.gemm(Ad, Bd, out=C, variant=v)
                    torch.cuda.synchronize()
                    got = C.cpu().clone()
                    mask = torch.ones(buf.numel(), dtype=torch.bool)
                    mask.as_strided((M, N), (ldc, 1), off).fill_(False)
                    assert (buf.cpu()[mask] == -7).all(), (K, policy, ldc, off)
                    if ref is None:
                        ref = got
                        _assert_parity(got, A, B, dtype)
                    assert torch.equal(got, ref), (K, policy, ldc, off)
    finally:
        tl.set_c_store_policy(tl.C_STORES_AUTO)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_thin_kernel(dtype):
    # N <= 16: the thin kernels (from 2 columns on the matrix cores, one
    # column on the vector ALUs), whatever the alignment; offset pointers
    # and K tails
    ce = 8 if dtype == "bf16" else 16
    for (M, N, K) in [(1, 1, 1), (5, 3, 7), (17, 16, 9), (33, 8, 1029), (1000, 1, 4104), (64, 16, 64),
                      (130, 5, 520)]:
        A = inputs.operand(KIND[dtype], M, K, 101 + K)
        B = inputs.operand(KIND[dtype], K, N, 102 + K)
        lda_al = (K + ce - 1) // ce * ce
        C_ref, S = _oracle(A, B, dtype)
        name = tl.plan_for(M, N, K, DT[dtype], K + 1, N + 3, N).info().name
        assert b"thin" in name and (b"thin_mma" in name) == (N >= 2), (M, N, K, name)
        for (lda, oa, ldb, ob) in [(lda_al, 0, N, 0), (K + 1, 1, N + 3, 1), (lda_al, ce - 1, N, 0), (K, 0, N, 0)]:
            C = _run_views(_exact_device_view(A, lda, oa), _exact_device_view(B, ldb, ob), None)
            ok, rep = check(C.numpy(), C_ref, S, dtype, K)
            assert ok, ((M, N, K), lda, oa, ldb, ob, rep)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_thin_kernel_rows_per_wave(dtype):
    # larger M: thin kernels with 2 and 4 rows of C per wave (the planner
    # keeps about 256 workgroups), M not a multiple of a workgroup's rows,
    # B's rows in 16-byte pieces that run into the next row (its last row by
    # element) and element by element, unaligned views on exact buffers
    cols = [(1, 3), (3, 3), (7, 7)] + ([(13, 13), (9, 11)] if dtype == "i8" else [])
    for (M, rows) in [(8200, 2), (16500, 4)]:
        for (N, ldb) in cols:
            K = 777
            name = tl.plan_for(M, N, K, DT[dtype], K + 1, ldb, N).info().name.decode()
            assert name.endswith("_r%d" % rows) and "thin" in name, (M, N, name)
            A = inputs.operand(KIND[dtype], M, K, 201 + N)
            B = inputs.operand(KIND[dtype], K, N, 202 + N)
            print("thin rows", dtype, M, N, K, ldb, name, flush=True)
            C = _run_views(_exact_device_view(A, K + 1, 1), _exact_device_view(B, ldb, 1), None)
            _assert_parity(C, A, B, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_split_plans(dtype):
    # the main tiled kernel on the first N - r columns, the thin kernel on
    # the last r, with aligned and unaligned B and exactly sized buffers
    for (M, N, K, ldb) in [(4096, 4097, 256, 4097), (4096, 4097, 256, 4112), (4095, 4100, 300, 4100)]:
        info = tl.plan_for(M, N, K, DT[dtype], K, ldb, N).info()
        assert info.n_main < N and b"thin" in info.rem_name, (M, N, K, ldb)
        A = inputs.operand(KIND[dtype], M, K, 111 + K)
        B = inputs.operand(KIND[dtype], K, N, 112 + K)
        print("split", dtype, M, N, K, ldb, info.name.decode(), flush=True)
        C = _run_views(_exact_device_view(A, K, 0), _exact_device_view(B, ldb, 0), None)
        _assert_parity(C, A, B, dtype)


def test_huge_leading_dimension():
    # lda = 8.5M bf16 (17 MB rows, a 4.35 GB A): the direct loader's 32-bit
    # per-lane offsets would wrap on a 256-row tile, so the plan takes the
    # register-staged kernel; only the first K columns of each row are set
    M, N, K, lda = 256, 256, 512, 8_500_000
    A = inputs.operand("bf16_normal", M, K, 97)
    B = inputs.operand("bf16_normal", K, N, 98)
    big = torch.empty((M, lda), dtype=torch.bfloat16, device="cuda")
    big[:, :K].copy_(A.cuda())
    Bd = B.cuda()
    C = torch.full((M, N), -7.0, dtype=torch.float32, device="cuda")
    req = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, tile_k=64, waves_n=4,
                     loader=tl.LOADER_DIRECT)
    assert tl.plan_for(M, N, K, tl.BF16, lda, N, N, req).info().variant.loader == tl.LOADER_VGPR
    tl.gemm(big[:, :K], Bd, out=C, variant=req)
    torch.cuda.synchronize()
    del big
    _assert_parity(C.cpu(), A, B, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_K_zero_writes_zeros(dtype):
    A = torch.zeros((70, 0), dtype=inputs.KINDS[KIND[dtype]])
    B = torch.zeros((0, 90), dtype=inputs.KINDS[KIND[dtype]])
    C = _run(A, B)
    assert (C == 0).all()


def test_workgroup_orders_agree_bitwise():
    A = inputs.operand("bf16_normal", 1024, 512, 51)
    B = inputs.operand("bf16_normal", 512, 2048, 52)
    base = None
    # 4 tile rows: groups of 4, 8 and 2^30 rows give the same order; the
    # largest must not wrap the group arithmetic (the run clamps it)
    for g in (tl.ORDER_ROW_MAJOR, 1, 2, 4, 8, 1 << 30):
        v = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, wg_group=g)
        C = _run(A, B, variant=v)
        if base is None:
            base = C
            _assert_parity(C, A, B, "bf16")
        assert torch.equal(C, base), g


def test_int8_largest_K_extremes_exact():
    # K = 131071, the largest K a plan takes: A = B = -128 gives 16384 K =
    # 2147467264 in every output, just below 2^31; A = -128, B = 127 gives
    # -16256 K (closed forms, and the exact int64 oracle agrees)
    K = 131071
    A = torch.full((64, K), -128, dtype=torch.int8)
    for bval, want in ((-128, 16384 * K), (127, -16256 * K)):
        B = torch.full((K, 64), bval, dtype=torch.int8)
        C = _run(A, B)
        assert (C.to(torch.int64) == want).all(), bval
        C_ref, _ = _oracle(A[:1], B[:, :1], "i8")
        assert int(C_ref[0, 0]) == want
