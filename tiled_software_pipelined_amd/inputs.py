"""Seeded synthetic operands for the GEMM workloads.

This module only draws random numbers and lays them out in memory; it holds
none of the product's arithmetic.  Both the HIP path's tests/benchmark and the
CPU oracle's checks take their operands from here, so the two sides see the
same bytes.  It imports neither side.

Distributions follow the workloads the pages measure: square GEMMs with
entries i.i.d. N(0,1) rounded to bf16 (the bf16 4096^3 ablation of the SM80
cp.async / ldmatrix plan, section 1), fp32 entries uniform in [-1, 1), and
int8 entries uniform over [-128, 127].  No page fixes a seed or generator, so
each operand comes from its own CPU ``torch.Generator`` seeded with a stable
integer; bf16 values are the round-to-nearest-even image of fp32 draws.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# operand distribution -> torch dtype of the operand
KINDS = {
    "f32_uniform": torch.float32,
    "bf16_normal": torch.bfloat16,
    "bf16_uniform": torch.bfloat16,
    "i8_uniform": torch.int8,
}


def _draw(kind: str, rows: int, cols: int, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    if kind == "f32_uniform":
        return torch.rand((rows, cols), generator=g, dtype=torch.float32) * 2.0 - 1.0
    if kind == "bf16_uniform":
        u = torch.rand((rows, cols), generator=g, dtype=torch.float32) * 2.0 - 1.0
        return u.to(torch.bfloat16)
    if kind == "bf16_normal":
        return torch.randn((rows, cols), generator=g, dtype=torch.float32).to(torch.bfloat16)
    if kind == "i8_uniform":
        return torch.randint(-128, 128, (rows, cols), generator=g, dtype=torch.int8)
    raise ValueError("unknown operand kind %r" % kind)


def operand(kind: str, rows: int, cols: int, seed: int, ld: int | None = None) -> torch.Tensor:
    """A ``rows x cols`` CPU tensor; with ``ld > cols`` it is a row-padded view.

    Padding columns hold a fixed, non-zero filler so that a kernel that reads
    past a row's end gives a visibly wrong answer rather than a lucky zero.
    """
    x = _draw(kind, rows, cols, seed)
    if ld is None or ld == cols:
        return x.contiguous()
    if ld < cols:
        raise ValueError("leading dimension %d < row length %d" % (ld, cols))
    fill = 7 if kind == "i8_uniform" else 3.0
    big = torch.full((rows, ld), fill, dtype=x.dtype)
    big[:, :cols] = x
    return big[:, :cols]


def as_oracle_array(t: torch.Tensor) -> np.ndarray:
    """Numpy view of a CPU operand in the oracle's encoding (bf16 -> raw uint16 bits).

    Keeps the row stride of padded views.
    """
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass(frozen=True)
class Workload:
    """One GEMM problem: shape, operand distribution, seeds, leading dims."""
    name: str
    dtype: str           # "f32", "bf16" or "i8" (operand type)
    M: int
    N: int
    K: int
    kind: str            # operand distribution, a key of KINDS
    seed: int
    lda: int | None = None
    ldb: int | None = None

    def operands(self):
        A = operand(self.kind, self.M, self.K, 2 * self.seed + 1, self.lda)
        B = operand(self.kind, self.K, self.N, 2 * self.seed + 2, self.ldb)
        return A, B

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


SWEEP_MN = (512, 4096)
SWEEP_K = (256, 512, 1024, 4096, 8192)


def workloads() -> dict:
    """The measured problems, keyed by name."""
    w = {}
    w["f32_256"] = Workload("f32_256", "f32", 256, 256, 256, "f32_uniform", 1000)
    w["bf16_4096"] = Workload("bf16_4096", "bf16", 4096, 4096, 4096, "bf16_normal", 2000)
    w["i8_4096"] = Workload("i8_4096", "i8", 4096, 4096, 4096, "i8_uniform", 3000)
    for a, mn in enumerate(SWEEP_MN):
        for b, k in enumerate(SWEEP_K):
            name = "bf16_sweep_%dx%dx%d" % (mn, mn, k)
            w[name] = Workload(name, "bf16", mn, mn, k, "bf16_normal", 4000 + 10 * (5 * a + b))
    w["f32_4096"] = Workload("f32_4096", "f32", 4096, 4096, 4096, "f32_uniform", 5000)
    w["bf16_ragged_4095x4097x4104"] = Workload("bf16_ragged_4095x4097x4104", "bf16",
                                               4095, 4097, 4104, "bf16_uniform", 5100)
    # the ragged product's last column as a product of its own (a contiguous
    # 4104 x 1 B): the thin kernel, bound by one read of A
    w["bf16_thin_4095x1x4104"] = Workload("bf16_thin_4095x1x4104", "bf16", 4095, 1, 4104, "bf16_uniform", 5300)
    # eight columns of the same: the matrix-core thin kernel
    w["bf16_thin_4095x8x4104"] = Workload("bf16_thin_4095x8x4104", "bf16", 4095, 8, 4104, "bf16_uniform", 5400)
    # one GPU's share of bf16 4096^3 split over 8 GPUs by rows of A and C
    w["bf16_msplit_512x4096x4096"] = Workload("bf16_msplit_512x4096x4096", "bf16", 512, 4096, 4096,
                                              "bf16_normal", 5200)
    return w
