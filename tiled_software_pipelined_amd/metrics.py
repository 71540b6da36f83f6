"""Performance-model arithmetic used by the benchmark and the plan report.

Formulas from "4.1 CUDA GEMM算子性能优化" (CUDA GEMM operator optimisation):
throughput = 2MNK / time (section 1.3); arithmetic intensity = flops / bytes
and the compute/bandwidth balance point (section 2.1); naive-kernel intensity
(section 3.2); block-tile intensity (section 4.3).  The block-tile intensity
is the same quantity as the compute/load ratio of the "流水化 GPU 内核" skill,
Step 2, which picks the loader.  Stage bytes per LDS slot follow the stage
table of the SM80 ablation plan, section 1.4.
"""
from __future__ import annotations


def flops(M: int, N: int, K: int) -> int:
    """Work of one product: 2 M N K (one multiply and one add per term)."""
    return 2 * M * N * K


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    return flops(M, N, K) / seconds / 1e12


def algorithmic_bytes(M: int, N: int, K: int, esize_in: int, esize_out: int) -> int:
    """One read of A and B, one write of C."""
    return (M * K + K * N) * esize_in + M * N * esize_out


def balance_point(peak_flops: float, bandwidth_bytes: float) -> float:
    """Intensity (flop/byte) above which a kernel is compute-bound."""
    return peak_flops / bandwidth_bytes


def naive_intensity(K: int, esize: int) -> float:
    """One output per thread: 2K flops over a row of A and a column of B."""
    return 2.0 * K / (2.0 * K * esize)


def tile_intensity(BM: int, BN: int, BK: int, esize: int) -> float:
    """Flops per byte loaded for one BM x BN x BK slice (= BM BN / ((BM + BN) esize / 2))."""
    return 2.0 * BM * BN * BK / ((BM * BK + BK * BN) * esize)


def stage_bytes(BM: int, BN: int, BK: int, esize: int) -> int:
    """LDS bytes of one stage: the A slice (BM x BK) plus the B slice (BK x BN)."""
    return (BM * BK + BK * BN) * esize


def roofline_time(M: int, N: int, K: int, esize_in: int, esize_out: int, peak_flops: float,
                  bandwidth_bytes: float) -> float:
    """Lower bound on the time of one product: compute- or memory-bound."""
    return max(flops(M, N, K) / peak_flops,
               algorithmic_bytes(M, N, K, esize_in, esize_out) / bandwidth_bytes)
