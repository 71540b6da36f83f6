"""GPU: gemm_run / gemm_run_ws launches recorded into a HIP graph replay to
the eager result.

The library enqueues only its own kernels on the caller's stream (the K = 0
case uses a fill kernel, not a memset; the repack of gemm_run_ws is a copy
kernel into a workspace the binding takes from torch's allocator, which
serves captured allocations from the graph's own pool), so a captured
sequence of launches must reproduce the eager C on every replay.  Each
replay is preceded by eager work on the same buffers (overwriting C) and a
synchronisation, and checked against the eager result.
"""
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


CASES = [
    ("bf16_normal", 512, 384, 328, 0),    # 64 x 64 direct ring, K tail
    ("bf16_normal", 1024, 1024, 512, 0),  # 128 x 128 direct ring
    ("bf16_normal", 300, 257, 129, 1),    # unaligned rows and a partial last piece, read in place
    ("f32_uniform", 130, 77, 65, 1),      # fp32 unaligned rows: repack, or the guarded kernel
    ("i8_uniform", 520, 264, 1000, 0),
    ("f32_uniform", 200, 136, 96, 0),     # vector-FMA path
    ("bf16_normal", 70, 90, 0, 0),        # K = 0: the fill kernel
    ("bf16_normal", 4096, 4097, 256, 0),  # split plan (tiled + thin kernel), B rows unaligned
    ("i8_uniform", 2000, 9, 700, 1),      # thin kernel
]


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("kind,M,N,K,pad", CASES)
def test_graph_replay_matches_eager(kind, M, N, K, pad, workspace):
    A = inputs.operand(kind, M, K, 91 + K).cuda()
    Bw = inputs.operand(kind, K, N + pad, 92 + K).cuda()
    B = Bw[:, pad:] if pad else Bw
    out_dtype = torch.int32 if kind.startswith("i8") else torch.float32
    C = torch.empty((M, N), dtype=out_dtype, device="cuda")
    tl.gemm(A, B, out=C, workspace=workspace)
    torch.cuda.synchronize()
    eager = C.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(3):
            tl.gemm(A, B, out=C, workspace=workspace)
    for r in range(4):
        C.fill_(-3)  # eager work on the same output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), (kind, M, N, K, r)
