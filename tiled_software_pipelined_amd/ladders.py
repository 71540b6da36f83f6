"""The ablation ladders: one variable per rung, in the order the pages give.

"cp.async / ldmatrix 消融实验 —— 初步规划（SM80 专用）" (the SM80 ablation plan)
asks that every gain be attributed to one change (section 1.3, pitfall 1),
that the SIMT and the tensor-core ladders stay apart (section 1.5), and that
the LDS -> register ladder be run with the copy, the ring depth and the
swizzle held fixed (section 1.1, section 3 table 2).  The rungs follow
"4.1 CUDA GEMM算子性能优化" sections 3-10 (naive -> block tiling -> register
tiling -> 128-bit accesses -> conflict-free LDS -> double buffer ->
asynchronous multi-stage copy) on this GPU's instructions.

Each rung is (label, what changes against the rung named in `base`, the
variant fields that select it).  Fields absent from a rung's dict are left to
the plan (zero); `None` as the variant means the default plan.  Only data
lives here: bench.py times the rungs, tests/test_ladder_gpu.py checks each
against the oracle at the ladder's size.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Rung:
    label: str
    change: str
    fields: dict | None          # variant fields; None = the default plan
    base: str | None = None      # the rung this one changes one thing of (None: the previous rung)
    extra: dict = field(default_factory=dict)


def _mfma(tile_k: int) -> list:
    """The matrix-core ladder on the 128 x 128 tile (tile_k: 32 for bf16,
    64 for int8: the same 64 bytes per row of a slice), then the
    fragment-read ladder on the direct loader at 3 slots, then the
    production tile and the workgroup order."""
    t = dict(kernel=2, tile_m=128, tile_n=128, tile_k=tile_k, waves_m=2, waves_n=2)
    narrow = dict(t, stages=1, loader=1, lds_layout=1, access=2)
    return [
        Rung("R0", "naive: one thread per C element, no LDS (GEMM page 3.1)", dict(kernel=1)),
        Rung("R1", "LDS block tiling + matrix cores; 4-byte global loads, LDS writes and fragment reads; "
                   "fragments re-read for every matrix instruction (GEMM page 4)",
             dict(narrow, frag=2)),
        Rung("R2", "+ register (wave) tiling: each fragment read once per K step and reused (GEMM page 5-6)",
             dict(narrow, frag=1)),
        Rung("R3a", "+ 16-byte global loads and LDS writes (fragment reads stay 4-byte) (GEMM page 7.1-7.2)",
             dict(t, stages=1, loader=1, lds_layout=1, access=1, frag=1, frag_read=1)),
        Rung("R3b", "+ 16-byte A fragment reads and transposing B reads (SM80 plan 1.1: ldmatrix's analogue)",
             dict(t, stages=1, loader=1, lds_layout=1, access=1, frag=1, frag_read=4)),
        Rung("R4", "+ XOR-swizzled 16-byte chunks: conflict-free LDS (GEMM page 8.5, scheme 2)",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=4)),
        Rung("R4a", "R4 with the direct global->LDS copy but one slot: asynchronous copy without a second "
                    "buffer (SM80 plan 1.2)",
             dict(t, stages=1, loader=2, lds_layout=2, access=1, frag=1, frag_read=4), base="R4"),
        Rung("R5", "R4 + register-staged double buffer, 2 slots (GEMM page 9.3-9.5)",
             dict(t, stages=2, loader=1, lds_layout=2, access=1, frag=1, frag_read=4), base="R4"),
        Rung("R6", "+ direct global->LDS copies instead of the register-staged loads, 2 slots (GEMM page 10)",
             dict(t, stages=2, loader=2, lds_layout=2, access=1, frag=1, frag_read=4)),
        Rung("R7s3", "+ 3 slots (GEMM page 10.2: multi-stage)",
             dict(t, stages=3, loader=2, lds_layout=2, access=1, frag=1, frag_read=4)),
        Rung("R7s4", "+ 4 slots", dict(t, stages=4, loader=2, lds_layout=2, access=1, frag=1, frag_read=4)),
        # the LDS -> register ladder with the copy (direct), the ring (3 slots)
        # and the swizzle (XOR) fixed (SM80 plan 1.1 and 3, table 2)
        Rung("A1", "fragment reads: A 4 x ds_read_b32, B one element read per K value (direct, 3 slots, XOR)",
             dict(t, stages=3, loader=2, lds_layout=2, access=1, frag=1, frag_read=1), base="R7s3"),
        Rung("A2", "+ A 2 x ds_read_b64", dict(t, stages=3, loader=2, lds_layout=2, access=1, frag=1, frag_read=2)),
        Rung("A3", "+ A 1 x ds_read_b128", dict(t, stages=3, loader=2, lds_layout=2, access=1, frag=1, frag_read=3)),
        Rung("A4", "+ B by two transposing reads (ds_read_b64_tr_b16 / _tr_b8): R7s3",
             dict(t, stages=3, loader=2, lds_layout=2, access=1, frag=1, frag_read=4)),
        Rung("R8", "the default plan's tile (256 x 256, 8 waves, 2 slots) and XCD-aware workgroup order",
             None, base="R7s4"),
    ]


def _simt() -> list:
    """The fp32 (vector FMA) ladder on the 128 x 128 x 8 tile, then the
    direct-copy rungs and the production 16-deep slices."""
    t = dict(kernel=2, tile_m=128, tile_n=128, tile_k=8)
    q = dict(t, lds_layout=1, access=1, frag=1, lane_map=2, store=1)
    return [
        Rung("S0", "naive: one thread per C element, one fma chain each (GEMM page 3.1)", dict(kernel=1)),
        Rung("S1", "LDS block tiling, 128 x 128 x 8, 8 x 8 outputs per lane; 4-byte loads; both operands "
                   "read from LDS for every FMA (GEMM page 4)",
             dict(t, stages=1, loader=1, lds_layout=1, access=2, frag=2, frag_read=1, lane_map=1, store=2)),
        Rung("S2", "+ register tiling: the lane's 8 + 8 fragment values read once per k step (GEMM page 5)",
             dict(t, stages=1, loader=1, lds_layout=1, access=2, frag=1, frag_read=1, lane_map=1, store=2)),
        Rung("S3", "+ 16-byte global loads and LDS writes (GEMM page 7.1-7.2)",
             dict(t, stages=1, loader=1, lds_layout=1, access=1, frag=1, frag_read=1, lane_map=1, store=2)),
        Rung("S4", "+ A transposed in LDS: 16-byte fragment reads (GEMM page 7.3)",
             dict(t, stages=1, loader=1, lds_layout=1, access=1, frag=1, frag_read=3, lane_map=1, store=2)),
        Rung("S5", "+ padded rows of transposed A: conflict-free A writes (GEMM page 8.5, scheme 1)",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=1, store=2)),
        Rung("S6q", "+ 4 x 4 quarters per lane (GEMM page 7.4 and 8.5, scheme 4)",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=2, store=2)),
        Rung("S6z", "S5 + Z-order lanes instead (GEMM page 8.5, scheme 3)",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=3, store=2),
             base="S5"),
        Rung("S6zq", "S6q + Z-order lanes",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=4, store=2),
             base="S6q"),
        Rung("S7", "S6q + 16-byte C stores (coalesced write-back)",
             dict(t, stages=1, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=2, store=1),
             base="S6q"),
        Rung("S8", "+ register-staged double buffer, 2 slots (GEMM page 9.3-9.5)",
             dict(t, stages=2, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=2, store=1)),
        Rung("S8k", "S8 with A row-major, read as 16-byte pieces along K (the layout a direct copy gives)",
             dict(q, stages=2, loader=1, frag_read=5)),
        Rung("S9", "+ direct global->LDS copies of both operands, 2 slots (GEMM page 10)",
             dict(q, stages=2, loader=2, frag_read=5)),
        Rung("S10s3", "+ 3 slots (GEMM page 10.2: multi-stage)", dict(q, stages=3, loader=2, frag_read=5)),
        Rung("S10s4", "+ 4 slots", dict(q, stages=4, loader=2, frag_read=5)),
        Rung("P8", "S8 with 16-deep slices",
             dict(t, tile_k=16, stages=2, loader=1, lds_layout=2, access=1, frag=1, frag_read=3, lane_map=2,
                  store=1), base="S8"),
        Rung("P8z", "+ Z-order lanes: the default plan", None),
        Rung("P8k", "P8 with A row-major read along K", dict(q, tile_k=16, stages=2, loader=1, frag_read=5),
             base="P8"),
        Rung("P9", "+ direct copies, 2 slots", dict(q, tile_k=16, stages=2, loader=2, frag_read=5)),
        Rung("P10s3", "+ 3 slots", dict(q, tile_k=16, stages=3, loader=2, frag_read=5)),
        Rung("P10s4", "+ 4 slots", dict(q, tile_k=16, stages=4, loader=2, frag_read=5)),
    ]


LADDERS = {
    "bf16": _mfma(32),
    "i8": _mfma(64),
    "f32": _simt(),
}

# the workload each ladder runs on
LADDER_WORKLOAD = {"bf16": "bf16_4096", "i8": "i8_4096", "f32": "f32_4096"}


def base_of(rungs: list, i: int) -> int | None:
    """Index of the rung rung i is compared with (None for the first)."""
    b = rungs[i].base
    if b is None:
        return i - 1 if i > 0 else None
    return [r.label for r in rungs].index(b)
