"""Python binding of libtgemm (argument marshalling only).

Every step of the product runs in the HIP kernels of ``libtgemm.so``; this
module checks tensor arguments, caches plans and calls the C ABI of
``include/tgemm.h`` with raw device pointers and torch's current stream.
There is no CPU fallback: if the library is missing, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtgemm.so")

# dtype codes of the C ABI
F32, BF16, I8 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", I8: "i8"}

OK = 0
ERRORS = {-1: "TGEMM_E_ARG", -2: "TGEMM_E_NULL", -3: "TGEMM_E_ALIGN", -4: "TGEMM_E_ARCH",
          -5: "TGEMM_E_VARIANT", -6: "TGEMM_E_HIP"}

# variant field values (include/tgemm.h)
KERNEL_AUTO, KERNEL_NAIVE, KERNEL_TILED = 0, 1, 2
LOADER_VGPR, LOADER_DIRECT = 1, 2
LDS_PLAIN, LDS_XOR, LDS_XOR_POISON = 1, 2, 3
ACCESS_WIDE, ACCESS_NARROW = 1, 2
FRAG_REUSE, FRAG_PER_MMA, FRAG_SLICE = 1, 2, 3
STORE_VECTOR, STORE_SCALAR = 1, 2
COPY_BURST, COPY_SPREAD, COPY_LATE = 1, 2, 3
C_STORES_AUTO, C_STORES_STREAM, C_STORES_PLAIN = 0, 1, 2
READ_B32, READ_B64, READ_B128, READ_TR, READ_KVEC = 1, 2, 3, 4, 5
LANES_BLOCKS, LANES_QUARTERS, LANES_ZORDER, LANES_ZQUARTERS = 1, 2, 3, 4
ORDER_ROW_MAJOR = -1


class Variant(ctypes.Structure):
    """Mirror of ``tgemm_variant``; zero fields mean "default"."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "tile_m", "tile_n", "tile_k", "stages", "loader", "lds_layout", "access", "frag",
        "wg_group", "waves_m", "waves_n", "store", "copy_sched", "frag_read", "lane_map")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self):
        return "Variant(%s)" % ", ".join("%s=%d" % kv for kv in self.as_dict().items() if kv[1])


class PlanInfo(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("variant", Variant), ("grid", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("loads_per_stage", ctypes.c_int32), ("a_guarded", ctypes.c_int32),
                ("b_guarded", ctypes.c_int32), ("name", ctypes.c_char * 96), ("n_main", ctypes.c_int64),
                ("rem_name", ctypes.c_char * 96), ("packed_name", ctypes.c_char * 96),
                ("waves_per_simd", ctypes.c_int32)]


EXPORTS = ("gemm_plan", "gemm_plan_variant", "gemm_run", "gemm_destroy", "tgemm_last_error",
           "gemm_plan_get_info", "gemm_variant_count", "gemm_variant_get", "tgemm_version",
           "tgemm_lds_read_probe", "tgemm_mfma_rate_probe", "gemm_workspace_bytes", "gemm_run_ws",
           "gemm_kernel_occupancy", "gemm_clock_slots", "gemm_run_clocked", "gemm_run_noalloc",
           "tgemm_set_c_store_policy")


def _load():
    # Load torch first: its HIP runtime (libamdhip64, SONAME libamdhip64.so.7)
    # is then the one libtgemm binds to, so device memory, streams and the
    # kernel launches all belong to one runtime in this process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtgemm.so is not built (%s); run "
                          "`python -m tiled_software_pipelined_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.gemm_plan.argtypes = [i64, i64, i64, i32, i64, i64, i64]
    lib.gemm_plan.restype = vp
    lib.gemm_plan_variant.argtypes = [i64, i64, i64, i32, i64, i64, i64, ctypes.POINTER(Variant)]
    lib.gemm_plan_variant.restype = vp
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp]
    lib.gemm_run.restype = ctypes.c_int
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = None
    lib.tgemm_last_error.argtypes = []
    lib.tgemm_last_error.restype = ctypes.c_char_p
    lib.gemm_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.gemm_kernel_occupancy.argtypes = [vp, i32, ctypes.POINTER(i32)]
    lib.gemm_kernel_occupancy.restype = ctypes.c_int
    lib.gemm_clock_slots.argtypes = [vp]
    lib.gemm_clock_slots.restype = i64
    lib.gemm_run_clocked.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.gemm_run_clocked.restype = ctypes.c_int
    lib.gemm_plan_get_info.restype = ctypes.c_int
    lib.gemm_variant_count.argtypes = [i32]
    lib.gemm_variant_count.restype = ctypes.c_int
    lib.gemm_variant_get.argtypes = [i32, i32, ctypes.POINTER(Variant)]
    lib.gemm_variant_get.restype = ctypes.c_int
    lib.tgemm_version.argtypes = []
    lib.tgemm_version.restype = ctypes.c_char_p
    lib.tgemm_lds_read_probe.argtypes = [i32, i32, i32, i32, vp, vp]
    lib.tgemm_lds_read_probe.restype = ctypes.c_int
    lib.gemm_workspace_bytes.argtypes = [vp, vp, vp]
    lib.gemm_workspace_bytes.restype = i64
    lib.gemm_run_ws.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.gemm_run_ws.restype = ctypes.c_int
    lib.gemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
    lib.gemm_run_noalloc.restype = ctypes.c_int
    lib.tgemm_mfma_rate_probe.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.tgemm_mfma_rate_probe.restype = ctypes.c_int
    lib.tgemm_set_c_store_policy.argtypes = [i32]
    lib.tgemm_set_c_store_policy.restype = ctypes.c_int
    return lib


_lib = _load()


class TgemmError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s: %s" % (ERRORS.get(code, code), msg))
        self.code = code


def last_error() -> str:
    return _lib.tgemm_last_error().decode()


def set_c_store_policy(policy: int) -> int:
    """tgemm_set_c_store_policy: C_STORES_AUTO / _STREAM / _PLAIN for every
    later run in this process; returns the previous policy."""
    rc = _lib.tgemm_set_c_store_policy(int(policy))
    if rc < 0:
        raise TgemmError(rc, last_error())
    return rc


def version() -> str:
    return _lib.tgemm_version().decode()


LDS_PROBE_KINDS = ("ds_read_b32", "ds_read_b64", "ds_read_b128", "ds_read_b64_tr_b16")
LDS_PROBE_PATTERNS = ("linear", "swizzled")
LDS_PROBE_THREADS = 256


def lds_read_probe(kind: int, pattern: int, reps: int, out):
    """Launch the LDS read-path probe on the current stream: one workgroup
    per 256 entries of ``out`` (a uint32-compatible int32 GPU tensor)."""
    import torch
    if not out.is_cuda or out.dtype != torch.int32 or out.numel() % LDS_PROBE_THREADS or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 GPU tensor of 256 * workgroups entries")
    wgs = out.numel() // LDS_PROBE_THREADS
    stream = torch.cuda.current_stream(out.device).cuda_stream
    with torch.cuda.device(out.device):
        rc = _lib.tgemm_lds_read_probe(kind, pattern, reps, wgs, out.data_ptr(), stream)
    if rc != OK:
        raise TgemmError(rc, "tgemm_lds_read_probe(kind=%d, pattern=%d, reps=%d, workgroups=%d)" % (
            kind, pattern, reps, wgs))
    return out


# kinds of tgemm_mfma_rate_probe: the bare bf16 / int8 matrix instruction, the
# fp32 FMA, and the bf16 matrix stream of the default GEMM kernel with its LDS
# fragment reads, then also its direct global->LDS copies
RATE_PROBE_KINDS = ("bf16", "i8", "f32", "bf16_lds", "bf16_lds_dma")
RATE_PROBE_THREADS = 256
RATE_PROBE_OPS_PER_INST = {"bf16": 2 * 32 * 32 * 16, "i8": 2 * 32 * 32 * 32, "f32": 2 * 64,
                           "bf16_lds": 2 * 32 * 32 * 16, "bf16_lds_dma": 2 * 32 * 32 * 16}


def mfma_rate_probe(kind: int, reps: int, operands, out, clocks):
    """Launch the matrix-core rate probe on the current stream.

    operands: contiguous GPU tensor of workgroups * 256 * 8 16-byte entries
    (any dtype; its bytes are the operand registers), out: int32 GPU tensor
    of workgroups * 256 entries, clocks: int64 GPU tensor of 2 * workgroups
    entries (shader-clock and real-time ticks per workgroup)."""
    import torch
    if not out.is_cuda or out.dtype != torch.int32 or out.numel() % RATE_PROBE_THREADS or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 GPU tensor of 256 * workgroups entries")
    wgs = out.numel() // RATE_PROBE_THREADS
    if (not operands.is_cuda or not operands.is_contiguous()
            or operands.numel() * operands.element_size() != wgs * RATE_PROBE_THREADS * 8 * 16):
        raise ValueError("operands must be a contiguous GPU tensor of workgroups * 256 * 8 * 16 bytes")
    if not clocks.is_cuda or clocks.dtype != torch.int64 or clocks.numel() != 2 * wgs or not clocks.is_contiguous():
        raise ValueError("clocks must be a contiguous int64 GPU tensor of 2 * workgroups entries")
    stream = torch.cuda.current_stream(out.device).cuda_stream
    with torch.cuda.device(out.device):
        rc = _lib.tgemm_mfma_rate_probe(kind, reps, wgs, operands.data_ptr(), out.data_ptr(), clocks.data_ptr(),
                                        stream)
    if rc != OK:
        raise TgemmError(rc, "tgemm_mfma_rate_probe(kind=%d, reps=%d, workgroups=%d)" % (kind, reps, wgs))
    return out, clocks


def variants(dtype: int):
    """The variants compiled into the library for a dtype code."""
    out = []
    for i in range(_lib.gemm_variant_count(dtype)):
        v = Variant()
        if _lib.gemm_variant_get(dtype, i, ctypes.byref(v)) != OK:
            raise TgemmError(-1, last_error())
        out.append(v)
    return out


class Plan:
    """A ``tgemm_plan`` (host metadata only; never touches the GPU)."""

    def __init__(self, M, N, K, dtype, lda=None, ldb=None, ldc=None, variant: Variant | None = None):
        lda = K if lda is None else lda
        ldb = N if ldb is None else ldb
        ldc = N if ldc is None else ldc
        self.M, self.N, self.K, self.dtype = int(M), int(N), int(K), int(dtype)
        self.lda, self.ldb, self.ldc = int(lda), int(ldb), int(ldc)
        if variant is None:
            h = _lib.gemm_plan(M, N, K, dtype, lda, ldb, ldc)
        else:
            h = _lib.gemm_plan_variant(M, N, K, dtype, lda, ldb, ldc, ctypes.byref(variant))
        if not h:
            raise TgemmError(-1, last_error())
        self._h = h

    def info(self) -> PlanInfo:
        info = PlanInfo()
        rc = _lib.gemm_plan_get_info(self._h, ctypes.byref(info))
        if rc != OK:
            raise TgemmError(rc, last_error())
        return info

    @property
    def name(self) -> str:
        return self.info().name.decode()

    def kernel_for(self, A: int, B: int, workspace: bool = True) -> str:
        """Name of the main kernel that runs for operands at these addresses:
        the repacked plan's when the binding would use a workspace."""
        info = self.info()
        if workspace and self.workspace_bytes(A, B) > 0:
            return info.packed_name.decode()
        return info.name.decode()

    def occupancy(self, packed: bool = False) -> int:
        """Workgroups of the main kernel (packed: the repacked plan's) that one
        compute unit holds at once, from the HIP runtime's calculator (GPU only)."""
        n = ctypes.c_int32(0)
        rc = _lib.gemm_kernel_occupancy(self._h, 1 if packed else 0, ctypes.byref(n))
        if rc != OK:
            raise TgemmError(rc, last_error())
        return int(n.value)

    def clock_slots(self) -> int:
        """Values of the clock buffer gemm_run_clocked needs (0: nothing to clock)."""
        return int(_lib.gemm_clock_slots(self._h))

    def run_clocked_ptr(self, A: int, B: int, C: int, clocks: int, clocks_len: int, stream: int = 0) -> None:
        """gemm_run_clocked on raw device pointers."""
        rc = _lib.gemm_run_clocked(self._h, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(C),
                                   ctypes.c_void_p(clocks), clocks_len, ctypes.c_void_p(stream))
        if rc != OK:
            raise TgemmError(rc, last_error())

    def run_ptr(self, A: int, B: int, C: int, stream: int = 0) -> None:
        """Enqueue on raw device pointers (the caller keeps the buffers alive)."""
        rc = _lib.gemm_run(self._h, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(C),
                           ctypes.c_void_p(stream))
        if rc != OK:
            raise TgemmError(rc, last_error())

    def workspace_bytes(self, A: int, B: int) -> int:
        """Workspace bytes gemm_run_ws uses to repack misaligned operands at these
        addresses (0 where the plan's kernel reads them in place)."""
        return int(_lib.gemm_workspace_bytes(self._h, ctypes.c_void_p(A), ctypes.c_void_p(B)))

    def run_ws_ptr(self, A: int, B: int, C: int, ws: int, ws_bytes: int, stream: int = 0) -> None:
        """gemm_run_ws on raw device pointers (the caller keeps the buffers alive)."""
        rc = _lib.gemm_run_ws(self._h, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(C),
                              ctypes.c_void_p(ws), ws_bytes, ctypes.c_void_p(stream))
        if rc != OK:
            raise TgemmError(rc, last_error())

    def run_noalloc_ptr(self, A: int, B: int, C: int, stream: int = 0) -> None:
        """gemm_run_noalloc on raw device pointers: repacks misaligned operands
        into the library's fixed device array (no allocation)."""
        rc = _lib.gemm_run_noalloc(self._h, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(C),
                                   ctypes.c_void_p(stream))
        if rc != OK:
            raise TgemmError(rc, last_error())

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:  # module globals are gone at interpreter exit
            _lib.gemm_destroy(h)
            self._h = None


_cache: dict = {}
_cache_lock = threading.Lock()


def _torch_dtype_code(t):
    import torch
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s (float32, bfloat16, int8)" % t.dtype)
    return m[t.dtype]


def _ld(t, name):
    """Leading dimension (row stride in elements) of a row-major 2-D tensor.

    Rows must not overlap: a row stride below the row length (a broadcast or
    otherwise aliased view) would make the kernels read past the rows the
    tensor's storage holds, so it is rejected."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major with unit column stride" % name)
    if t.shape[0] > 1 and t.shape[1] > 0 and t.stride(0) < t.shape[1]:
        raise ValueError("%s has overlapping rows (row stride %d < %d columns); pass a contiguous copy"
                         % (name, t.stride(0), t.shape[1]))
    return max(int(t.stride(0)), int(t.shape[1]), 1) if t.shape[0] > 1 else max(int(t.shape[1]), 1)


CLOCK_VALUES = 6  # TGEMM_CLOCK_VALUES: values per workgroup written by gemm_run_clocked
NOALLOC_MAX_BYTES = 64 << 20  # TGEMM_NOALLOC_MAX_BYTES: the fixed workspace of gemm_run_noalloc


def clock_ghz(clocks) -> float:
    """Mean shader clock (GHz) of clocked runs: a host array of CLOCK_VALUES
    values per workgroup as gemm_run_clocked writes them (any number of runs
    stacked); shader ticks over 100 MHz real-time ticks from start to end,
    summed over workgroups."""
    import numpy as np
    c = np.asarray(clocks, dtype=np.uint64).reshape(-1, CLOCK_VALUES).astype(np.float64)
    shader = float((c[:, 4] - c[:, 0]).sum())
    real = float((c[:, 5] - c[:, 1]).sum())
    if real <= 0:
        raise ValueError("no real-time ticks recorded")
    return shader / real * 0.1


def clock_split_us(clocks):
    """Per workgroup of clocked runs: (K-loop microseconds, C write-back
    microseconds) from the real-time ticks (100 MHz), as two arrays."""
    import numpy as np
    c = np.asarray(clocks, dtype=np.uint64).reshape(-1, CLOCK_VALUES).astype(np.int64)
    return (c[:, 3] - c[:, 1]) * 0.01, (c[:, 5] - c[:, 3]) * 0.01


def plan_for(M, N, K, dtype, lda, ldb, ldc, variant: Variant | None = None) -> Plan:
    key = (M, N, K, dtype, lda, ldb, ldc, None if variant is None else tuple(variant.as_dict().items()))
    with _cache_lock:
        p = _cache.get(key)
        if p is None:
            p = Plan(M, N, K, dtype, lda, ldb, ldc, variant)
            _cache[key] = p
    return p


def gemm(A, B, out=None, variant: Variant | None = None, workspace: bool = True):
    """C = A @ B on the current CUDA/HIP stream.

    A: (M, K), B: (K, N) torch tensors on the GPU, both float32, both bfloat16
    or both int8, row-major (row stride may exceed the row length).  Returns
    C (M, N): float32 for float32/bfloat16 inputs, int32 for int8 inputs.
    ``out`` may be a preallocated row-major C (its row stride is used as ldc).
    Operands whose rows are not 16-byte aligned are read in place by the
    matrix-core kernels.  With ``workspace`` (default plans only), where the
    plan's kernel needs aligned rows (fp32) they are repacked into a device
    buffer taken from torch's allocator on the current stream (gemm_run_ws);
    otherwise a kernel that reads such rows in place runs (gemm_run).
    """
    import torch
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be GPU tensors")
    if A.device != B.device:
        raise ValueError("A and B must be on the same device (%s, %s)" % (A.device, B.device))
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    code = _torch_dtype_code(A)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    out_dtype = torch.int32 if code == I8 else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out must be a %s tensor of shape (%d, %d) on %s" % (out_dtype, M, N, A.device))
    lda, ldb, ldc = _ld(A, "A"), _ld(B, "B"), _ld(out, "out")
    p = plan_for(M, N, K, code, lda, ldb, ldc, variant)
    stream = torch.cuda.current_stream(A.device).cuda_stream
    with torch.cuda.device(A.device):
        need = p.workspace_bytes(A.data_ptr(), B.data_ptr()) if workspace and variant is None else 0
        if need > 0:
            # stream-ordered: the block returns to torch's pool for this
            # stream when `ws` is dropped, after the work queued here
            ws = torch.empty(need + 256, dtype=torch.uint8, device=A.device)
            base = (ws.data_ptr() + 255) // 256 * 256
            p.run_ws_ptr(A.data_ptr(), B.data_ptr(), out.data_ptr(), base, need, stream)
        else:
            p.run_ptr(A.data_ptr(), B.data_ptr(), out.data_ptr(), stream)
    return out
