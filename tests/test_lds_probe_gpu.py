"""GPU: the LDS read-path probe reads exactly the bytes its definition names.

The probe (tgemm_lds_read_probe, include/tgemm.h) folds everything each
thread read into a 16-bit checksum; the XOR over a workgroup is recomputed
here from the fill pattern and the address formula, for each of the four
read instruction forms.  A wrong address, a dropped or repeated read, or a
result used before its read completed changes it.
"""
import numpy as np
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


WIDTH = {0: 4, 1: 8, 2: 16, 3: 8}  # bytes per lane of one instruction of each kind


def _expected_acc(kind, pattern, reps):
    """Each thread's checksum, from the fill pattern and the address formula."""
    i = np.arange(4096, dtype=np.uint64)
    lds = (((i * 2654435761) & 0xFFFFFFFF) ^ (i >> 7)).astype(np.uint32)
    t = np.arange(256)
    l, w = t % 64, t // 64
    W = WIDTH[kind]
    acc = np.zeros(256, dtype=np.uint32)
    for r in range(reps):
        f = np.zeros(256, dtype=np.uint32)
        if pattern == 0:
            for j in range(64 // W):
                dword = (w * 4096 + j * 64 * W + l * W) // 4
                for d in range(W // 4):
                    f ^= lds[dword + d]
        else:
            for c in range(4):
                row = (l & 31) + 32 * (c & 1)
                chunk = ((l >> 5) + 2 * (c >> 1) + 4 * ((r + w) & 3)) & 15
                dword = (row * 256 + (chunk ^ (row & 15)) * 16) // 4
                for d in range(4):
                    f ^= lds[dword + d]
        acc = (((acc << 1) | (acc >> 15)) & 0xFFFF) ^ ((f ^ (f >> 16)) & 0xFFFF)
    return acc


@pytest.mark.parametrize("pattern", [0, 1])
@pytest.mark.parametrize("kind", [0, 1, 2, 3])
@pytest.mark.parametrize("reps", [0, 1, 5, 12])
def test_probe_checksum(kind, pattern, reps):
    wgs = 6
    out = torch.full((wgs * 256,), -1, dtype=torch.int32, device="cuda")
    tl.lds_read_probe(kind, pattern, reps, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(wgs, 256)
    want = _expected_acc(kind, pattern, reps)
    for g in range(wgs):
        if kind != 3:
            assert np.array_equal(got[g], want), (kind, pattern, reps, g)
        else:
            # the transposing read moves 16-bit elements between the lanes of
            # a 16-lane group: compare each group's XOR
            gx = np.bitwise_xor.reduce(got[g].reshape(16, 16), axis=1)
            wx = np.bitwise_xor.reduce(want.reshape(16, 16), axis=1)
            assert np.array_equal(gx, wx), (kind, pattern, reps, g)
            if reps:
                assert not np.array_equal(got[g], want)  # it did transpose


def test_probe_rejects_bad_arguments():
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    for kind, pattern, reps in [(4, 0, 1), (-1, 0, 1), (0, 2, 1), (0, 0, -1)]:
        with pytest.raises(tl.TgemmError):
            tl.lds_read_probe(kind, pattern, reps, out)
