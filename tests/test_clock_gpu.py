"""GPU: gemm_run_clocked writes the same C as gemm_run and, per workgroup of
the tiled kernel, start / K-loop-end / end readings of the shader-clock and
100 MHz real-time counters from which the run's mean shader clock and its
split into K loop and C write-back follow."""
import numpy as np
import pytest
import torch

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


# 4096 x 4096 x 512: the plan's kernel is a 256 x 256 tile, its fallback for
# unaligned rows a 128 x 128 one, so the buffer holds four times the rows the
# launch writes
CASES = [("bf16_normal", "BF16", 1024, 1024, 1024), ("i8_uniform", "I8", 512, 768, 1000),
         ("f32_uniform", "F32", 300, 260, 200), ("bf16_normal", "BF16", 4096, 4096, 4096),
         ("bf16_normal", "BF16", 4096, 4096, 512)]


@pytest.mark.parametrize("kind,dt,M,N,K", CASES)
def test_clocked_run_matches_and_reads_a_plausible_clock(kind, dt, M, N, K):
    A = inputs.operand(kind, M, K, 61).cuda()
    B = inputs.operand(kind, K, N, 62).cuda()
    out_dtype = torch.int32 if dt == "I8" else torch.float32
    p = tl.Plan(M, N, K, getattr(tl, dt))
    slots = p.clock_slots()
    # sized for the largest grid among the plan's kernels; with aligned
    # operands the main kernel runs and writes the first `grid` rows
    grid = p.info().grid
    assert slots >= tl.CLOCK_VALUES * grid and slots % tl.CLOCK_VALUES == 0
    C0 = torch.full((M, N), -7, dtype=out_dtype, device="cuda")
    C1 = torch.full((M, N), -5, dtype=out_dtype, device="cuda")
    clocks = torch.zeros(slots + tl.CLOCK_VALUES, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    p.run_ptr(A.data_ptr(), B.data_ptr(), C0.data_ptr(), stream)
    p.run_clocked_ptr(A.data_ptr(), B.data_ptr(), C1.data_ptr(), clocks.data_ptr(), slots, stream)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)
    c = clocks.cpu().numpy().view(np.uint64)
    assert (c[tl.CLOCK_VALUES * grid:] == 0).all()  # nothing past the launched grid's rows
    c = c[:tl.CLOCK_VALUES * grid].reshape(-1, tl.CLOCK_VALUES)
    # start <= K-loop end <= end, for both counters
    assert (c[:, 2] > c[:, 0]).all() and (c[:, 3] >= c[:, 1]).all()
    assert (c[:, 4] > c[:, 2]).all() and (c[:, 5] >= c[:, 3]).all() and (c[:, 5] > c[:, 1]).all()
    loop_us, store_us = tl.clock_split_us(c)
    assert (loop_us >= 0).all() and (store_us >= 0).all() and loop_us.sum() > 0
    ghz = tl.clock_ghz(c)
    assert 0.3 < ghz < 3.0, ghz


def test_short_clock_buffer_launches_nothing():
    M = N = K = 512
    A = inputs.operand("bf16_normal", M, K, 63).cuda()
    B = inputs.operand("bf16_normal", K, N, 64).cuda()
    p = tl.Plan(M, N, K, tl.BF16)
    C = torch.full((M, N), -7.0, device="cuda")
    clocks = torch.zeros(p.clock_slots(), dtype=torch.int64, device="cuda")
    with pytest.raises(tl.TgemmError):
        p.run_clocked_ptr(A.data_ptr(), B.data_ptr(), C.data_ptr(), clocks.data_ptr(), p.clock_slots() - 1)
    torch.cuda.synchronize()
    assert (C == -7.0).all() and (clocks == 0).all()


def test_thin_plans_have_nothing_to_clock():
    p = tl.Plan(1024, 4, 512, tl.BF16, 512, 5, 4)  # B rows not 16-byte aligned: the thin kernel
    assert "thin" in p.name and p.clock_slots() == 0
