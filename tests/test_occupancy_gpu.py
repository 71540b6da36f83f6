"""GPU: gemm_kernel_occupancy reports the HIP runtime's workgroups per CU for
a plan's main kernel, consistent with the kernel's LDS per workgroup and the
160 KiB of LDS per compute unit."""
import pytest
import torch

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


@pytest.mark.parametrize("M,N,K,dt", [(4096, 4096, 4096, "BF16"), (4096, 4096, 4096, "I8"),
                                      (4096, 4096, 4096, "F32"), (256, 256, 256, "F32"),
                                      (1024, 1024, 4096, "BF16"), (512, 4096, 4096, "BF16")])
def test_occupancy_within_the_lds_bound(M, N, K, dt):
    p = tl.Plan(M, N, K, getattr(tl, dt))
    info = p.info()
    n = p.occupancy()
    assert 1 <= n <= 160 * 1024 // info.lds_bytes, (info.name, n)
    # at most 32 waves (8 per SIMD) on a compute unit
    assert n * ((info.threads + 63) // 64) <= 32, (info.name, n)


def test_default_large_tiles_fill_a_compute_unit_alone():
    # 256 x 256 tiles take 128 KiB of LDS: one workgroup per CU
    assert tl.Plan(4096, 4096, 4096, tl.BF16).occupancy() == 1
    assert tl.Plan(4096, 4096, 4096, tl.I8).occupancy() == 1


def test_packed_form_of_a_misaligned_plan():
    # fp32 with ldb = 4097: gemm_run runs the guarded kernel, gemm_run_ws the
    # same tile on the repacked operand; bf16 reads the rows in place and has
    # no repacked form
    p = tl.Plan(4095, 4097, 4104, tl.F32)
    assert p.info().packed_name
    assert p.occupancy(packed=False) >= 1 and p.occupancy(packed=True) >= 1
    assert tl.Plan(4095, 4097, 4104, tl.BF16).info().packed_name == b""
