"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/tgemm.h declares, validates plans and picks variants."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")

tl = pytest.importorskip("tiled_software_pipelined_amd.lib")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("TGEMM")))


def test_header_declares_the_abi():
    names = _declared_functions()
    for n in ("gemm_plan", "gemm_run", "gemm_destroy"):
        assert n in names
    assert set(names) == set(tl.EXPORTS)


@pytest.mark.parametrize("name", _declared_functions())
def test_library_exports_symbol(name):
    lib = ctypes.CDLL(tl.LIB_PATH)
    assert hasattr(lib, name)


def test_version():
    assert "gfx950" in tl.version()


@pytest.mark.parametrize("args", [
    (-1, 4, 4, tl.F32, 4, 4, 4),          # negative M
    (4, 4, 4, 7, 4, 4, 4),                # unknown dtype
    (4, 4, 8, tl.BF16, 7, 4, 4),          # lda < K
    (4, 8, 4, tl.BF16, 4, 7, 8),          # ldb < N
    (4, 8, 4, tl.BF16, 4, 8, 7),          # ldc < N
    (4, 4, 200000, tl.I8, 200000, 4, 4),  # int8 K beyond exact int32 range
    (4, 4, 131072, tl.I8, 131072, 4, 4),  # 16384 * 131072 = 2^31 wraps int32
    (2 ** 31, 4, 4, tl.F32, 4, 4, 4),     # too large
])
def test_plan_rejects_invalid(args):
    with pytest.raises(tl.TgemmError):
        tl.Plan(*args)
    assert tl.last_error() != ""


def test_int8_largest_exact_K_is_accepted():
    # |C| <= 128 * 128 * K = 2147467264 < 2^31 at K = 131071
    assert 128 * 128 * 131071 < 2 ** 31 <= 128 * 128 * 131072
    assert tl.Plan(4, 4, 131071, tl.I8, 131071, 4, 4).K == 131071


def test_huge_workgroup_group_is_accepted():
    # any group of at least tiles_m rows gives one group of all tile rows;
    # the run clamps it (the GPU test checks the result)
    v = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=128, tile_n=128, wg_group=1 << 30)
    assert tl.Plan(512, 512, 64, tl.BF16, variant=v).info().variant.wg_group == 1 << 30


def test_plan_run_rejects_null_plan():
    assert tl._lib.gemm_run(None, None, None, None, None) == -2
    assert "NULL" in tl.last_error()


def test_occupancy_rejects_null_arguments():
    n = ctypes.c_int32(-1)
    assert tl._lib.gemm_kernel_occupancy(None, 0, ctypes.byref(n)) == -2 and n.value == -1
    p = tl.Plan(64, 64, 64, tl.BF16)
    assert tl._lib.gemm_kernel_occupancy(p._h, 0, None) == -2


def test_clock_slots_and_null_arguments():
    # host-only: the count covers the largest grid the plan may launch
    p = tl.Plan(4096, 4096, 4096, tl.BF16)
    assert p.clock_slots() == tl.CLOCK_VALUES * p.info().grid == 6 * 256
    q = tl.Plan(4096, 4096, 4096, tl.BF16, 4096, 4097, 4096)  # B rows unaligned: register-staged
    assert q.clock_slots() >= tl.CLOCK_VALUES * q.info().grid
    assert tl.Plan(0, 64, 64, tl.BF16).clock_slots() == 0
    assert tl.Plan(64, 64, 0, tl.BF16, 1, 64, 64).clock_slots() == 0
    assert tl._lib.gemm_clock_slots(None) == 0
    assert tl._lib.gemm_run_clocked(None, None, None, None, None, 0, None) == -2
    assert tl._lib.gemm_run_clocked(p._h, None, None, None, None, 0, None) == -2
    # nothing to clock: returns before touching the device
    assert tl._lib.gemm_run_clocked(tl.Plan(0, 64, 64, tl.BF16)._h, None, None, None, 8, 4, None) == -1


def test_clock_ghz_arithmetic():
    # two workgroups: 2.0e6 and 1.0e6 shader ticks over 1000 and 1000 real ticks (10 us each)
    c = [[0, 0, 1_500_000, 700, 2_000_000, 1000], [5, 7, 900_005, 907, 1_000_005, 1007]]
    assert abs(tl.clock_ghz(c) - 3.0e6 / 2000 * 0.1 / 1000 * 1000) < 1e-12
    assert abs(tl.clock_ghz([[0, 0, 100, 4, 240, 10]]) - 2.4) < 1e-12
    loop, store = tl.clock_split_us(c)
    assert list(loop) == [7.0, 9.0] and list(store) == [3.0, 1.0]


def test_run_with_empty_output_is_a_noop_without_device():
    # M = 0: nothing to do, returns before touching the device
    p = tl.Plan(0, 16, 16, tl.BF16)
    p.run_ptr(0, 0, 0)


def test_leading_dimension_of_views():
    import torch
    x = torch.zeros(6, 10)
    assert tl._ld(x, "A") == 10
    assert tl._ld(x[:, 2:7], "A") == 10      # padded rows: the row stride
    assert tl._ld(x[:1, :4], "A") == 4       # one row: its length
    with pytest.raises(ValueError):
        tl._ld(torch.zeros(8).expand(4, 8), "A")  # every row is the same memory
    with pytest.raises(ValueError):
        tl._ld(torch.zeros(20).as_strided((4, 8), (4, 1)), "A")  # rows overlap
    with pytest.raises(ValueError):
        tl._ld(x.t(), "A")                   # column-major
    with pytest.raises(ValueError):
        tl._ld(torch.zeros(2, 3, 4), "A")


def test_destroy_null_is_allowed():
    tl._lib.gemm_destroy(None)


@pytest.mark.parametrize("dtype", [tl.F32, tl.BF16, tl.I8])
def test_variants_enumerate(dtype):
    vs = tl.variants(dtype)
    assert len(vs) >= 3
    kinds = {v.kernel for v in vs}
    assert kinds == {tl.KERNEL_NAIVE, tl.KERNEL_TILED}
    for v in vs:
        p = tl.Plan(512, 512, 512, dtype, variant=v)
        got = p.info().variant
        for f in ("kernel", "tile_m", "tile_n", "tile_k", "stages", "loader", "lds_layout", "access", "frag",
                  "waves_m", "waves_n", "store"):
            assert getattr(got, f) == getattr(v, f)


def test_bad_variant_rejected():
    v = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=96)
    with pytest.raises(tl.TgemmError):
        tl.Plan(256, 256, 256, tl.BF16, variant=v)


def test_default_choice_by_shape():
    big = tl.Plan(4096, 4096, 4096, tl.BF16).info()
    assert (big.variant.tile_m, big.variant.tile_n, big.variant.tile_k) == (256, 256, 64)
    assert (big.variant.waves_m, big.variant.waves_n) == (2, 4)
    assert big.variant.loader == tl.LOADER_DIRECT and big.grid == 256
    mid = tl.Plan(2048, 2048, 512, tl.BF16).info()
    assert (mid.variant.tile_m, mid.variant.tile_n) == (128, 128) and mid.grid == 256
    assert mid.variant.stages == 4
    assert tl.Plan(2048, 2048, 256, tl.BF16).info().variant.stages == 3
    # 128 x 128 tiles filling a quarter of the CUs or fewer: 64 x 64
    for dtype in (tl.BF16, tl.I8):
        q = tl.Plan(1024, 1024, 4096, dtype).info()
        assert (q.variant.tile_m, q.variant.tile_n, q.variant.stages, q.grid) == (64, 64, 4, 256), dtype
    # one round of 256 x 256 tiles from K = 512 (int8: 1024); several rounds
    # at short K stay on 128 x 128
    for M, K, dt, edge in [(4096, 512, tl.BF16, 256), (4096, 256, tl.BF16, 128), (3072, 512, tl.BF16, 256),
                           (6144, 512, tl.BF16, 128), (4096, 1024, tl.I8, 256), (4096, 512, tl.I8, 128)]:
        assert tl.Plan(M, M, K, dt).info().variant.tile_m == edge, (M, K, dt)
    # 128 x 128 tiles filling at most half the CUs: half tiles, wide along the longer side
    for M, N, tile in [(512, 4096, (64, 128)), (4096, 512, (128, 64))]:
        v = tl.Plan(M, N, 4096, tl.BF16).info().variant
        assert (v.tile_m, v.tile_n, v.tile_k, v.stages) == tile + (32, 4), (M, N)
        v = tl.Plan(M, N, 4096, tl.I8).info().variant
        assert (v.tile_m, v.tile_n, v.tile_k, v.stages) == tile + (64, 4), (M, N)
    # int8 from K = 2048 only
    assert tl.Plan(512, 4096, 1024, tl.I8).info().variant.tile_m == 128
    assert tl.Plan(512, 4096, 1024, tl.BF16).info().variant.tile_m == 64
    # long K on the 128 x 128 tile: the deeper ring; on the 64 x 64 tile
    # 128-deep (int8 256) slices in 4 slots from K = 1024 bf16, 2048 int8, and
    # whole-slice fragment read-ahead at every K
    assert tl.Plan(2048, 2048, 4096, tl.BF16).info().variant.stages == 4
    for dtype, bk in ((tl.BF16, 128), (tl.I8, 256)):
        small = tl.Plan(512, 512, 4096, dtype).info().variant
        assert (small.tile_m, small.tile_k, small.stages, small.frag) == (64, bk, 4, tl.FRAG_SLICE), dtype
        assert tl.Plan(512, 512, 512, dtype).info().variant.stages == 3
        assert tl.Plan(512, 512, 512, dtype).info().variant.frag == tl.FRAG_SLICE
    assert (tl.Plan(512, 512, 1024, tl.BF16).info().variant.tile_k, tl.Plan(512, 512, 1024, tl.BF16).info().variant.stages) == (128, 4)
    assert (tl.Plan(512, 512, 1024, tl.I8).info().variant.tile_k, tl.Plan(512, 512, 1024, tl.I8).info().variant.stages) == (128, 3)
    # the larger tiles keep reading one K step ahead
    assert tl.Plan(2048, 2048, 4096, tl.BF16).info().variant.frag == tl.FRAG_REUSE
    small = tl.Plan(512, 512, 512, tl.BF16).info()
    assert (small.variant.tile_m, small.variant.tile_n) == (64, 64) and small.grid == 64
    # fp32: 64 x 64 tiles while 128 x 128 ones would give one per CU or fewer
    f = tl.Plan(256, 256, 256, tl.F32).info()
    assert (f.variant.tile_m, f.variant.tile_k, f.grid) == (64, 16, 16)
    assert tl.Plan(2048, 2048, 2048, tl.F32).info().variant.tile_m == 64
    f = tl.Plan(4096, 4096, 4096, tl.F32).info()
    assert (f.variant.tile_m, f.variant.tile_k, f.grid) == (128, 16, 1024)


def test_unaligned_rows_are_read_in_place():
    # ragged workload: B rows of 4097 bf16 = 8194 bytes are not 16-byte
    # aligned.  The direct loader's copies read 16 bytes from any byte
    # address, so the plan keeps the direct-loader kernel, unguarded.
    for dtype in (tl.BF16, tl.I8):
        info = tl.Plan(4095, 4097, 4104, dtype).info()
        assert info.b_guarded == 0 and info.a_guarded == 0
        assert info.variant.loader == tl.LOADER_DIRECT
        # split: the first 4096 columns on 256 x 256 tiles (one round of 256
        # workgroups; 4097 columns would need 272 of them, or 1056 of
        # 128 x 128), the last column in the same K loop (the kernel's twin)
        assert (info.variant.tile_m, info.variant.tile_n) == (256, 256)
        assert info.grid == 16 * 16 and info.n_main == 4096
        assert info.rem_name == info.name + b"_remcol"
    # rows and pointers of any alignment with whole 16-byte pieces per row
    info = tl.Plan(4096, 4096, 4096, tl.BF16, lda=4097, ldb=4097).info()
    assert info.variant.loader == tl.LOADER_DIRECT and info.a_guarded == 0 and info.b_guarded == 0
    # N not a whole number of 16-byte pieces (the last piece of a B row
    # crosses N): the direct loader reads that piece in place too (guarded:
    # B's last row through the register tail)
    for dtype in (tl.BF16, tl.I8):
        info = tl.Plan(150, 131, 101, dtype).info()
        assert info.variant.loader == tl.LOADER_DIRECT and info.b_guarded == 1, dtype
    # so does an explicit direct-loader request on N = 4097 (no split for
    # explicit variants)
    req = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, tile_k=64, waves_n=4,
                     loader=tl.LOADER_DIRECT)
    info = tl.Plan(4095, 4097, 4104, tl.BF16, variant=req).info()
    v = info.variant
    assert (v.loader, v.tile_m, v.tile_n, v.tile_k, v.waves_m, v.waves_n) == (tl.LOADER_DIRECT, 256, 256, 64, 2, 4)
    assert info.b_guarded == 1
    # fewer than one whole piece per row: not the direct loader
    for dtype in (tl.BF16, tl.I8):
        assert tl.Plan(150, 5, 101, dtype, variant=tl.Variant(kernel=tl.KERNEL_TILED, tile_m=64, tile_n=64,
                                                              loader=tl.LOADER_DIRECT)).info().variant.loader \
            == tl.LOADER_VGPR, dtype


def test_default_tile_follows_the_round_model():
    # measured (interleaved, bf16, K = 4096): 256 x 256 faster at 4096^2,
    # 5120^2 and 3072^2; 128 x 128 faster at 4096 x 4352 and 4096 x 4608
    # (272 / 288 big tiles: a second, nearly empty round)
    for (M, N, want) in [(4096, 4096, 256), (5120, 5120, 256), (3072, 3072, 256), (4096, 4352, 128),
                         (4096, 4608, 128)]:
        assert tl.Plan(M, N, 4096, tl.BF16).info().variant.tile_m == want, (M, N)
    # unaligned B rows: 4096^2 keeps the 256 x 256 direct-loader kernel
    big = tl.Plan(4096, 4096, 4096, tl.BF16, ldb=4097).info()
    assert big.b_guarded == 0 and big.variant.tile_m == 256 and big.variant.loader == tl.LOADER_DIRECT
    # 4096 x 4097 splits off its last column (272 big tiles or 1056 small
    # ones would need a second round) into the main kernel's K loop, with B
    # rows aligned or not
    for ldb in (4097, 4104):
        info = tl.Plan(4096, 4097, 4096, tl.BF16, ldb=ldb).info()
        assert info.b_guarded == 0 and info.variant.tile_m == 256 and info.n_main == 4096
        assert info.variant.loader == tl.LOADER_DIRECT and info.rem_name.endswith(b"_remcol")
    # three last columns: the thin kernel after the main part
    info = tl.Plan(4096, 4099, 4096, tl.BF16).info()
    assert info.n_main == 4096 and b"thin" in info.rem_name
    # fewer than 16 tile columns (a tile's rows would not all have a
    # workgroup for the last column): the thin kernel
    info = tl.Plan(8192, 2049, 4096, tl.BF16).info()
    assert info.n_main == 2048 and b"thin" in info.rem_name, info.rem_name
    # 4096 x 4352 leaves no thin remainder: no split
    info = tl.Plan(4096, 4352, 4096, tl.BF16).info()
    assert info.n_main == 4352 and info.rem_name == b""


def test_thin_products_use_the_thin_kernel():
    # N <= 16 (bf16, int8), whatever the rows' alignment: from 2 columns the
    # matrix-core thin kernel of the smallest width that covers N (bf16 4,
    # 8, 16; int8 8, 16), one column the vector one (its contiguous-column
    # twin exactly when ldb = 1); 17 columns and more the tiles
    for dtype in (tl.BF16, tl.I8):
        cases = [(1, 1, 1), (1, 5, 1), (7, 7, 8), (3, 64, 4 if dtype == tl.BF16 else 8), (9, 9, 16), (16, 32, 16),
                 (16, 17, 16), (8, 8, 8 if dtype == tl.BF16 else 8)]
        for N, ldb, width in cases:
            info = tl.Plan(4096, N, 4096, dtype, ldb=ldb).info()
            assert b"thin" in info.name and info.n_main == N, (dtype, N, ldb)
            assert (b"thin_mma" in info.name) == (N >= 2), info.name
            # rows per workgroup: 16 waves sharing 16 rows (matrix cores) or
            # holding one row each; the contiguous-column twin 4 waves of one row
            rows = 4 if (N, ldb) == (1, 1) else 16
            assert info.variant.tile_n == width and info.variant.tile_m == rows and info.grid == 4096 // rows
            assert info.name.endswith(b"_col") == ((N, ldb) == (1, 1))
        assert b"thin" not in tl.Plan(4096, 17, 4096, dtype, ldb=17).info().name
    # the matrix-core kernel's B pieces of NB columns must end within the
    # next row (NB <= ldb + N): a single column with ldb = 2 keeps the
    # vector kernel
    assert b"thin_n1" in tl.Plan(4096, 1, 4096, tl.BF16, ldb=2).info().name
    # fp32 keeps its one-fma-chain-per-output kernel
    assert b"thin" not in tl.Plan(4096, 4, 4096, tl.F32).info().name


@pytest.mark.parametrize("dtype", [tl.F32, tl.BF16, tl.I8])
def test_default_plan_exists_for_every_shape_class(dtype):
    # every branch of the default choice must name a compiled kernel, for
    # aligned and unaligned leading dimensions
    sizes = [1, 7, 64, 127, 128, 129, 512, 1000, 2048, 4095, 4096, 4097, 8192]
    for M in sizes:
        for N in sizes:
            for K in (1, 33, 1024, 1025, 4096, 4104, 8192):
                for pad in (0, 1):
                    tl.Plan(M, N, K, dtype, lda=K + pad, ldb=N + pad, ldc=N)


def test_huge_leading_dimension_leaves_the_direct_loader():
    # the direct loader's per-lane offsets are 32-bit: (BM-1)*lda*2 bytes
    # must fit.  lda = 8.5M bf16 overflows them on a 256-row tile.
    req = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=256, tile_n=256, tile_k=64, waves_n=4,
                     loader=tl.LOADER_DIRECT)
    assert tl.Plan(256, 256, 512, tl.BF16, variant=req).info().variant.loader == tl.LOADER_DIRECT
    v = tl.Plan(256, 256, 512, tl.BF16, lda=8_500_000, variant=req).info().variant
    assert v.loader == tl.LOADER_VGPR and (v.tile_m, v.tile_n) == (256, 256)
    # a huge ldb (B offsets reach (BK-1)*ldb)
    v = tl.Plan(4096, 4096, 4096, tl.BF16, ldb=40_000_000).info().variant
    assert v.loader == tl.LOADER_VGPR
    # the default plan of a small shape too
    v = tl.Plan(512, 512, 512, tl.BF16, lda=40_000_000).info().variant
    assert v.loader == tl.LOADER_VGPR
    # the whole-slice read-ahead is a schedule of the direct loader: the
    # register-staged fallback reads one K step ahead
    req = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=64, tile_n=64, tile_k=64, stages=8, frag=tl.FRAG_SLICE)
    assert tl.Plan(512, 512, 4096, tl.BF16, variant=req).info().variant.frag == tl.FRAG_SLICE
    v = tl.Plan(512, 512, 4096, tl.BF16, lda=40_000_000, variant=req).info().variant
    assert v.loader == tl.LOADER_VGPR and v.frag == tl.FRAG_REUSE


def test_lds_budget_of_stage_ring():
    # 128 x 128 x 32 bf16: 8 KiB of A + 8 KiB of B per stage (the SM80 ablation
    # plan's stage table, section 1.4): S = 2, 3, 4 -> 32, 48, 64 KiB
    for s, kib in ((2, 32), (3, 48), (4, 64)):
        v = tl.Variant(kernel=tl.KERNEL_TILED, tile_m=128, tile_n=128, tile_k=32, stages=s,
                       loader=tl.LOADER_DIRECT)
        assert tl.Plan(4096, 4096, 4096, tl.BF16, variant=v).info().lds_bytes == kib * 1024


def test_loads_per_stage_match_tile_bytes():
    info = tl.Plan(4096, 4096, 4096, tl.BF16).info()
    # 256 x 64 + 64 x 256 bf16 = 64 KiB per slice, 16 B per load per thread
    assert info.threads == 64 * info.variant.waves_m * info.variant.waves_n
    assert info.loads_per_stage == 65536 // info.threads // 16


def test_guard_follows_global_load_width_for_every_variant():
    # N = 257 leaves a partial 16-byte chunk at the end of every B row: every
    # tiled variant that loads B in chunks must guard B (found on the fp32
    # rung whose A-fragment access is narrow but whose B loads are 16 bytes)
    # (the fp32 rungs with 4-byte global loads read one element at a time,
    # each checked against N, and need no guard)
    for dtype in (tl.F32, tl.BF16, tl.I8):
        for v in tl.variants(dtype):
            info = tl.Plan(129, 257, 40, dtype, variant=v).info()
            if info.variant.kernel != tl.KERNEL_TILED:
                continue
            if dtype == tl.F32 and info.variant.access == tl.ACCESS_NARROW:
                assert info.b_guarded == 0, info.name.decode()
            else:
                assert info.b_guarded == 1, info.name.decode()


def _ru(x, m):
    return (x + m - 1) // m * m


@pytest.mark.parametrize("dtype,esz", [(tl.F32, 4), (tl.BF16, 2), (tl.I8, 1)])
def test_workspace_bytes(dtype, esz):
    # host-only: the addresses are numbers, nothing is dereferenced
    al = 1 << 20
    M, N, K = 4095, 4097, 4104
    p = tl.Plan(M, N, K, dtype, K, N, N)
    if dtype != tl.F32:
        # the matrix-core plans read rows and pointers of any alignment in
        # place: nothing to repack
        for a, b in ((al, al), (al + esz, al), (al, al + esz), (al + 1, al + 3)):
            assert p.workspace_bytes(a, b) == 0
        assert tl.Plan(1024, 1024, 512, dtype).workspace_bytes(al, al + esz) == 0
        return
    # fp32: repacked rows are rounded up to whole 128-byte lines
    bytes_a = _ru(M * _ru(K * esz, 128), 256)
    bytes_b = _ru(K * _ru(N * esz, 128), 256)
    a_al = (K * esz) % 16 == 0
    # leading dimensions: B rows (N = 4097) are never aligned; A rows at K = 4104 are for bf16 / fp32
    assert p.workspace_bytes(al, al) == (0 if a_al else bytes_a) + bytes_b
    # a pointer that is not 16-byte aligned adds its operand (its rows keep lda = K when aligned)
    assert p.workspace_bytes(al + esz, al) == (_ru(M * K * esz, 256) if a_al else bytes_a) + bytes_b
    q = tl.Plan(1024, 1024, 512, dtype)
    assert q.workspace_bytes(al, al) == 0
    assert q.workspace_bytes(al, al + esz) == _ru(512 * 1024 * esz, 256)
    # no repack for explicit variants, thin products, or empty work
    v = tl.variants(dtype)[0]
    assert tl.Plan(M, N, K, dtype, variant=v).workspace_bytes(al, al) == 0
    assert tl.Plan(4096, 9, 4096, dtype, 4096, 9, 9).workspace_bytes(al, al) == 0
    assert tl.Plan(64, 64, 0, dtype, 1, 64, 64).workspace_bytes(al + 1, al + 1) == 0
    assert tl.Plan(0, 64, 64, dtype).workspace_bytes(al + 1, al + 1) == 0


def test_run_ws_without_workspace_falls_back_to_run():
    # M = 0: both return before touching the device
    p = tl.Plan(0, 16, 16, tl.BF16)
    p.run_ws_ptr(0, 0, 0, 0, 0)


def test_ladders_select_distinct_kernels():
    # every rung of the ablation ladders resolves to its own kernel (no two
    # rungs time the same code), except where a rung repeats another on
    # purpose (A4 = R7s3: the fragment-read ladder ends on the 3-slot kernel)
    from tiled_software_pipelined_amd import inputs, ladders
    for dtype, rungs in ladders.LADDERS.items():
        code = {"f32": tl.F32, "bf16": tl.BF16, "i8": tl.I8}[dtype]
        w = inputs.workloads()[ladders.LADDER_WORKLOAD[dtype]]
        names = {}
        for r in rungs:
            v = None if r.fields is None else tl.Variant(**r.fields)
            names.setdefault(tl.Plan(w.M, w.N, w.K, code, variant=v).name, []).append(r.label)
        dup = {k: v for k, v in names.items() if len(v) > 1}
        assert all(set(v) == {"R7s3", "A4"} for v in dup.values()), dup
        for r in rungs:
            if r.base is not None:
                assert r.base in [x.label for x in rungs], r.label


def test_c_store_policy_setter():
    # process-wide; returns the previous policy, rejects unknown ones
    try:
        assert tl.set_c_store_policy(tl.C_STORES_PLAIN) == tl.C_STORES_AUTO
        assert tl.set_c_store_policy(tl.C_STORES_STREAM) == tl.C_STORES_PLAIN
        with pytest.raises(tl.TgemmError):
            tl.set_c_store_policy(7)
        assert tl.set_c_store_policy(tl.C_STORES_AUTO) == tl.C_STORES_STREAM
    finally:
        tl.set_c_store_policy(tl.C_STORES_AUTO)
