"""GPU: the rate probe executes the instructions its definition names.

The probe (tgemm_mfma_rate_probe, include/tgemm.h) sums every accumulator
register of each thread after `reps` iterations of 16 independent
matrix-core instructions (kinds 0, 1) or fp32 fma chains (kind 2).  With
small integer operands every product and sum is exact, so each thread's sum
is recomputed here from the operand bytes and the instruction's operand /
result lane layout: a dropped or repeated instruction, a wrong operand
register or a wrong layout changes it.
"""
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


def _operands(kind, workgroups, seed):
    """Small integers: bf16 / fp32 in [-3, 3], int8 in [-8, 8]; shape (threads, 8, H)."""
    g = np.random.default_rng(seed)
    threads = workgroups * 256
    if kind == 2:
        vals = g.integers(-3, 4, size=(threads, 8, 4)).astype(np.float32)
        return vals, torch.from_numpy(vals.reshape(-1).copy())
    if kind == 0:
        vals = g.integers(-3, 4, size=(threads, 8, 8)).astype(np.float32)
        bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # exact: small integers
        return vals, torch.from_numpy(bits.reshape(-1).view(np.int16).copy())
    vals = g.integers(-8, 9, size=(threads, 8, 16)).astype(np.int8)
    return vals.astype(np.int64), torch.from_numpy(vals.reshape(-1).copy())


def _expected(kind, vals, reps):
    """Per-thread sum of the 16 accumulators' registers after `reps` iterations
    (kind 2: of the 16 fma chains, acc_i = reps * x_i * y_i)."""
    if kind == 2:
        x = vals[:, 0:4, :].reshape(vals.shape[0], 16).astype(np.int64)
        y = vals[:, 4:8, :].reshape(vals.shape[0], 16).astype(np.int64)
        return (x * y).sum(axis=1) * reps
    H = 8 if kind == 0 else 16  # K elements per lane
    out = np.zeros(vals.shape[0], dtype=np.int64)
    lane = np.arange(64)
    rows = np.array([[8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)] for l in lane])
    cols = lane % 32
    for w0 in range(0, vals.shape[0], 64):
        wv = vals[w0:w0 + 64].astype(np.int64)
        total = np.zeros(64, dtype=np.int64)
        for i in range(16):
            a = wv[:, i & 3, :]         # (64 lanes, H)
            b = wv[:, 4 + ((i >> 2) & 3), :]
            A = np.concatenate([a[0:32], a[32:64]], axis=1)    # (32 rows, 2H): row m, k
            B = np.concatenate([b[0:32], b[32:64]], axis=1).T  # (2H, 32 cols)
            P = A @ B
            total += P[rows, cols[:, None]].sum(axis=1)
        out[w0:w0 + 64] = total * reps
    return out


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("reps", [0, 1, 3])
def test_rate_probe_checksum(kind, reps):
    wgs = 3
    vals, ops = _operands(kind, wgs, 100 + 10 * kind + reps)
    ops = ops.to("cuda:0")
    out = torch.full((wgs * 256,), -1, dtype=torch.int32, device="cuda:0")
    clocks = torch.full((2 * wgs,), -1, dtype=torch.int64, device="cuda:0")
    tl.mfma_rate_probe(kind, reps, ops, out, clocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    exp = _expected(kind, vals, reps)
    if kind in (0, 2):
        got = got.view(np.float32).astype(np.int64)
    else:
        exp = exp.astype(np.int32).astype(np.int64)
        got = got.astype(np.int64)
    np.testing.assert_array_equal(got, exp)
    clk = clocks.cpu().numpy()
    assert (clk >= 0).all()


def test_rate_probe_clock_ratio():
    """Shader-clock and real-time ticks over a long loop give a plausible clock."""
    wgs = 8
    _, ops = _operands(0, wgs, 7)
    ops = ops.to("cuda:0")
    out = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
    clocks = torch.empty(2 * wgs, dtype=torch.int64, device="cuda:0")
    tl.mfma_rate_probe(0, 2000, ops, out, clocks)
    torch.cuda.synchronize()
    clk = clocks.cpu().numpy().reshape(-1, 2)
    # 2000 iterations x 16 instructions x at least 32 cycles each
    assert (clk[:, 0] >= 2000 * 16 * 32).all()
    ghz = clk[:, 0] / clk[:, 1] * 0.1
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz


def test_rate_probe_rejects_bad_arguments():
    out = torch.empty(256, dtype=torch.int32, device="cuda:0")
    clocks = torch.empty(2, dtype=torch.int64, device="cuda:0")
    ops = torch.empty(256 * 8 * 8, dtype=torch.int16, device="cuda:0")
    with pytest.raises(Exception):
        tl.mfma_rate_probe(5, 1, ops, out, clocks)
    with pytest.raises(Exception):
        tl.mfma_rate_probe(0, -1, ops, out, clocks)
    with pytest.raises(ValueError):
        tl.mfma_rate_probe(0, 1, ops[:-8], out, clocks)


@pytest.mark.parametrize("kind", [3, 4])
def test_mix_probe_all_ones(kind):
    # all-ones bf16 operands: every matrix instruction adds K = 16 to each
    # accumulator value; 8 accumulators x 16 values, 2 K steps per iteration
    # -> every thread's sum is 128 x 16 x 2 x reps (exact in fp32)
    wgs, reps = 512, 40
    ops = torch.full((wgs * 256 * 8 * 8,), 1.0, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
    clocks = torch.empty(2 * wgs, dtype=torch.int64, device="cuda:0")
    tl.mfma_rate_probe(kind, reps, ops, out, clocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float32)
    assert (got == np.float32(128 * 16 * 2 * reps)).all(), got[:4]


def test_mix_probe_copies_do_not_change_the_sums():
    # random operands: kinds 3 and 4 read the same LDS bytes (the copies land
    # in a region no read touches), so their sums agree bit for bit
    wgs, reps = 512, 20
    ops = inputs.operand("bf16_normal", wgs * 256 * 8, 8, 91).reshape(-1).cuda()
    outs = []
    for kind in (3, 4):
        out = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
        clocks = torch.empty(2 * wgs, dtype=torch.int64, device="cuda:0")
        tl.mfma_rate_probe(kind, reps, ops, out, clocks)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])
    assert np.isfinite(outs[0].numpy().view(np.float32)).all()
