"""GPU parity at the workloads' own sizes: every output compared with the oracle.

Each workload (fp32 256^3 and 4096^3, bf16 4096^3, int8 4096^3, the ten bf16
sweep shapes, the ragged bf16 4095 x 4097 x 4104 and the 512 x 4096 x 4096
one-GPU share) runs through the C ABI in the launch configuration the
benchmark times, and all M x N outputs are compared with the oracle computed
once per workload: int8 exactly, bf16 and fp32 by the per-element gates of
tests/parity.py, and the fp32 kernels bit for bit with the sequential fp32
fma chain.  Besides the default plan, each workload also runs the kernels
whose speed the ladder and the sweep report on it: the 128 x 128 x 32 tile
at 2, 3 and 4 stages on bf16 4096^3, every loader / ring depth of the sweep
on every sweep shape, and on the ragged product the default plan with and
without a workspace (the same launch: its unaligned rows are read in place
and its last column is computed in the main K loop) and the register-staged
256 x 256 tile, which reads B's rows by shifted loads.  Every matrix-core
result of one workload must also be the same bit for bit (pipelining only
reorders loads: the "流水化 GPU 内核" skill, Step 5; the SM80 ablation plan,
section 1.3), but for the ragged product's last column, whose in-loop sum
takes another order.
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


def _variant(**kw):
    return tl.Variant(kernel=tl.KERNEL_TILED, **kw)


def _extra_variants(w):
    """(label, variant, workspace) of the kernels besides the default plan."""
    out = []
    if w.name == "bf16_4096" or w.name.startswith("bf16_sweep"):
        # the tile of the 4096^3 configuration at 2 / 3 / 4 stages (direct
        # loader), then the sweep's other loaders on the same tile
        for st in (2, 3, 4):
            out.append(("t128x128x32_direct_s%d" % st,
                        _variant(tile_m=128, tile_n=128, tile_k=32, stages=st, loader=tl.LOADER_DIRECT,
                                 waves_m=2, waves_n=2), False))
        out.append(("t128x128x32_vgpr_s2", _variant(tile_m=128, tile_n=128, tile_k=32, stages=2,
                                                     loader=tl.LOADER_VGPR, lds_layout=tl.LDS_XOR,
                                                     waves_m=2, waves_n=2), False))
        out.append(("t128x128x32_direct_s1", _variant(tile_m=128, tile_n=128, tile_k=32, stages=1,
                                                       loader=tl.LOADER_DIRECT, waves_m=2, waves_n=2), False))
    if w.name == "i8_4096":
        for st in (2, 3, 4):
            out.append(("t128x128x64_direct_s%d" % st,
                        _variant(tile_m=128, tile_n=128, tile_k=64, stages=st, loader=tl.LOADER_DIRECT,
                                 waves_m=2, waves_n=2), False))
    if w.name.startswith("bf16_ragged"):
        # B's rows (4097 bf16) are not 16-byte aligned: the default plan
        # reads them in place, workspace or not; the register-staged tile on
        # all 4097 columns reads them by shifted loads
        out.append(("default_in_place", None, False))
        out.append(("t256x256x64_vgpr_shift", _variant(tile_m=256, tile_n=256, tile_k=64, stages=2,
                                                       loader=tl.LOADER_VGPR, lds_layout=tl.LDS_XOR,
                                                       waves_m=2, waves_n=4), False))
    return out


def _run(w, A, B, variant, workspace):
    out_dtype = torch.int32 if w.dtype == "i8" else torch.float32
    C = torch.full((w.M, w.N), -7, dtype=out_dtype, device="cuda")
    tl.gemm(A, B, out=C, variant=variant, workspace=workspace)
    torch.cuda.synchronize()
    return C


NAMES = sorted(inputs.workloads())


@pytest.mark.parametrize("name", NAMES)
def test_workload_in_full(name):
    w = inputs.workloads()[name]
    A_cpu, B_cpu = w.operands()
    print("workload", name, "oracle ...", flush=True)
    C_ref, S = oracle.gemm(inputs.as_oracle_array(A_cpu), inputs.as_oracle_array(B_cpu), w.dtype)
    chain = oracle.gemm_f32_fma_chain(A_cpu.numpy(), B_cpu.numpy()) if w.dtype == "f32" else None
    A, B = A_cpu.cuda(), B_cpu.cuda()
    runs = [("default", None, True)] + _extra_variants(w)
    first = None
    for label, v, ws in runs:
        kname = tl.plan_for(w.M, w.N, w.K, {"f32": tl.F32, "bf16": tl.BF16, "i8": tl.I8}[w.dtype],
                            w.K, w.N, w.N, v).kernel_for(A.data_ptr(), B.data_ptr(), workspace=ws and v is None)
        print("  ", label, kname, flush=True)
        C = _run(w, A, B, v, ws)
        Ch = C.cpu().numpy()
        ok, rep = check(Ch, C_ref, S, w.dtype, w.K)
        assert ok, (name, label, kname, rep)
        if w.dtype == "i8":
            assert np.array_equal(Ch.astype(np.int64), C_ref), (name, label)
        if chain is not None:
            bad = int((Ch != chain).sum())
            assert bad == 0, (name, label, "differs from the fp32 fma chain at %d outputs" % bad)
        if w.dtype != "f32":
            # one matrix-core K order for every tile, ring depth and loader
            # (the ragged product's last column: the default plan sums it in
            # the main K loop in another order)
            n = w.N - 1 if name.startswith("bf16_ragged") else w.N
            if first is None:
                first = C
            else:
                assert torch.equal(C[:, :n], first[:, :n]), (name, label)
        del C


def test_ragged_reads_unaligned_rows_in_place():
    # B's rows (4097 bf16 = 8194 bytes) are not 16-byte aligned: the direct-
    # copy kernel reads them in place and computes the last column in its
    # own K loop, so the plan asks for no workspace and gemm_run_ws runs
    # exactly gemm_run's launch
    w = inputs.workloads()["bf16_ragged_4095x4097x4104"]
    A_cpu, B_cpu = w.operands()
    A, B = A_cpu.cuda(), B_cpu.cuda()
    p = tl.plan_for(w.M, w.N, w.K, tl.BF16, w.K, w.N, w.N)
    info = p.info()
    print("ragged plan:", info.name.decode(), info.rem_name.decode(), flush=True)
    assert info.rem_name == info.name + b"_remcol" and info.packed_name == b""
    assert p.workspace_bytes(A.data_ptr(), B.data_ptr()) == 0
    C_ws = _run(w, A, B, None, True)
    C_in = _run(w, A, B, None, False)
    assert torch.equal(C_ws, C_in)
