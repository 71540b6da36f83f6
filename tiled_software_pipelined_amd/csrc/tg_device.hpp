// Device-side building blocks shared by the libtgemm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_args.hpp"

namespace tg {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define TG_LDS __attribute__((address_space(3)))

// Wait until at most N vector-memory instructions of this wave are still
// outstanding and every LDS access of this wave has completed, then meet the
// other waves of the workgroup at the barrier.  Written as one asm statement
// with a memory clobber so that the compiler neither moves LDS accesses
// across it nor widens it into vmcnt(0) (which the fenced __syncthreads()
// does and which would drain every stage in flight).  Waiting for the LDS
// reads matters: after the barrier another wave may start a copy into the
// slot those reads came from.
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit counter on gfx9");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for this wave's LDS writes, then barrier (register-staged loaders).
__device__ __forceinline__ void wait_lds_then_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait for every outstanding memory instruction of this wave, then barrier.
__device__ __forceinline__ void wait_all_then_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Clock marks of a workgroup (GemmArgs::clocks): the shader-clock counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime), read when
// the workgroup starts, when wave 0 leaves the K loop (before its C stores)
// and once every wave's memory instructions, the C stores included, have
// completed.  Thread 0 writes [start shader, start real, loop-end shader,
// loop-end real, end shader, end real] to clocks[CLOCK_VALUES * workgroup ..]
// with vector stores.

struct ClockMark {
    uint64_t c0 = 0, w0 = 0, c1 = 0, w1 = 0;
    __device__ __forceinline__ void start(const uint64_t* clocks) {
        if (clocks) {
            c0 = __builtin_amdgcn_s_memtime();
            w0 = __builtin_amdgcn_s_memrealtime();
        }
    }
    __device__ __forceinline__ void loop_end(const uint64_t* clocks) {
        if (clocks) {
            c1 = __builtin_amdgcn_s_memtime();
            w1 = __builtin_amdgcn_s_memrealtime();
        }
    }
    __device__ __forceinline__ void finish(uint64_t* clocks) const {
        if (clocks) {
            wait_all_then_barrier();
            const uint64_t c2 = __builtin_amdgcn_s_memtime();
            const uint64_t w2 = __builtin_amdgcn_s_memrealtime();
            if (threadIdx.x == 0) {
                uint64_t* p = clocks + CLOCK_VALUES * (uint64_t)blockIdx.x;
                p[0] = c0;
                p[1] = w0;
                p[2] = c1;
                p[3] = w1;
                p[4] = c2;
                p[5] = w2;
            }
        }
    }
};

// One 16-byte-per-lane copy global -> LDS that bypasses the registers
// (global_load_lds_dwordx4).  Lane l reads `base + voff` and its 16 bytes
// land at LDS byte `lds + 16 l`; `lds` and `base` must be wave-uniform.
// Issued from asm so that the compiler does not treat the LDS write as
// aliasing every later LDS read (it would otherwise wait for the copy to
// finish before each read and serialise the pipeline); completion is tracked
// explicitly with wait_vm_then_barrier.  M0 is written here: the kernels that
// use this issue every LDS copy through it and nothing else of theirs uses
// M0.  On gfx9-family chips a global/buffer load with LDS=1 that follows a
// scalar write of M0 needs one wait state in between, which the hardware
// does not insert and the compiler only inserts between instructions it
// emits itself, so the asm carries its own s_nop 0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(uint32_t lds, uint32_t voff, const void* base) {
    // make the wave-uniform operands scalar (they are, but the compiler may
    // not be able to prove it)
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(sl), "v"(voff), "s"(sb)
                 : "m0");
}
// The same copy, 4 bytes per lane: lane l's 4 bytes land at lds + 4 l.
__device__ __forceinline__ void copy4_to_lds(uint32_t lds, uint32_t voff, const void* base) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(sl), "v"(voff), "s"(sb)
                 : "m0");
}
#pragma clang diagnostic pop

// Bytes [sh, sh + 16) of the 32-byte pair x | y (x first in memory),
// 0 <= sh < 16: how a 16-byte piece at any byte offset is cut out of the
// two aligned 16-byte blocks that cover it.
__device__ __forceinline__ i32x4 funnel16(i32x4 x, i32x4 y, uint32_t sh) {
    // Named scalars, not an array: selects between elements of a local
    // array are turned into a dynamically indexed stack copy.
    const bool s8 = sh & 8, s4 = sh & 4;
    const uint32_t t0 = s8 ? x[2] : x[0], t1 = s8 ? x[3] : x[1], t2 = s8 ? y[0] : x[2];
    const uint32_t t3 = s8 ? y[1] : x[3], t4 = s8 ? y[2] : y[0], t5 = s8 ? y[3] : y[1];
    const uint32_t u0 = s4 ? t1 : t0, u1 = s4 ? t2 : t1, u2 = s4 ? t3 : t2;
    const uint32_t u3 = s4 ? t4 : t3, u4 = s4 ? t5 : t4;
    const uint32_t b = sh & 3;
    i32x4 out;
    out[0] = int32_t(__builtin_amdgcn_alignbyte(u1, u0, b));
    out[1] = int32_t(__builtin_amdgcn_alignbyte(u2, u1, b));
    out[2] = int32_t(__builtin_amdgcn_alignbyte(u3, u2, b));
    out[3] = int32_t(__builtin_amdgcn_alignbyte(u4, u3, b));
    return out;
}

// Guarded loads.  Written as `ok ? *p : 0`, the compiler turns the select
// into a branch around the load (a load is costly enough to skip), and every
// such branch ends with a wait for all of the wave's outstanding loads, so a
// run of guarded loads becomes a chain of memory round trips.  load_or_zero
// instead always loads once, from p or from a zero-filled device array,
// which keeps every load of the run in flight together.  The array is never
// written, and is not const, so that the compiler cannot fold its value
// back into a select.
// 16 bytes from any byte address.  gfx950 global loads take unaligned
// addresses (one global_load_dwordx4 either way); the copy keeps the
// compiler from assuming the 16-byte alignment of an i32x4 pointer.
__device__ __forceinline__ i32x4 load16(const void* p) {
    i32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

static __device__ __attribute__((aligned(16))) int32_t g_zeros[4];

template <class T>
__device__ __forceinline__ T load_or_zero(const T* p, bool ok) {
    static_assert(sizeof(T) <= sizeof(g_zeros), "at most 16 bytes");
    const T* src = ok ? p : reinterpret_cast<const T*>(g_zeros);
    T v;
    __builtin_memcpy(&v, src, sizeof(T));  // any alignment
    return v;
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup -> output tile.  The hardware hands workgroup b to XCD b mod 8;
// with wg_group > 0 the id is first re-ranked so that consecutive ids run on
// one XCD (and share its L2), then tiles are walked in groups of wg_group
// tile rows, column by column, so that one XCD's workgroups reuse the same
// A row panels and B column panels (the block-order effect on L2 hit rate of
// "4.1 CUDA GEMM算子性能优化", section 2.3).
__device__ __forceinline__ void tile_of_workgroup(const GemmArgs& g, int& tm, int& tn) {
    const int b = blockIdx.x;
    if (g.wg_group <= 0) {
        tm = b / g.tiles_n;
        tn = b - tm * g.tiles_n;
        return;
    }
    const int total = g.tiles_m * g.tiles_n;
    int r = b;
    if ((total & 7) == 0) r = (b & 7) * (total >> 3) + (b >> 3);
    const int per_group = g.wg_group * g.tiles_n;
    const int group = r / per_group;
    const int first_m = group * g.wg_group;
    const int rows = min(g.tiles_m - first_m, g.wg_group);
    const int in_group = r - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

}  // namespace tg
