// LDS read-path probe: the same bytes read from LDS through four instruction
// forms, to attribute the gain of wide fragment reads separately from the
// GEMM, where matrix-core time hides it ("4.1 CUDA GEMM算子性能优化",
// section 8: wide shared-memory reads and their bank behaviour; the
// "流水化 GPU 内核" skill: ldmatrix-style reads cut instructions, not bytes).
//
// Every workgroup fills a 16 KiB LDS block (64 rows of 256 bytes, one
// 64-bank window per row) with a fixed pattern, then each lane reads 64
// bytes per iteration as
//   kind 0: 16 x ds_read_b32        kind 1: 8 x ds_read_b64
//   kind 2:  4 x ds_read_b128       kind 3: 8 x ds_read_b64_tr_b16
// from one of two address patterns:
//   pattern 0 (linear): instruction j of a wave reads 64 consecutive
//     W-byte slots (W = its width), lane l the l-th - conflict-free for
//     every width, so the kinds differ by instruction form alone;
//   pattern 1 (swizzled): four 16-byte pieces in 256-byte rows whose
//     16-byte chunks are permuted by an XOR with the row index, the kind of
//     layout the GEMM's operands use; each piece is read as 16 / W
//     instructions.
// Each lane folds what it read into a 16-bit checksum, so that the host can
// check every read happened and returned the right bytes (the transposing
// read only permutes 16-bit elements within a 16-lane group; the XOR over a
// workgroup does not see the permutation).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tg_device.hpp"
#include "tgemm.h"

namespace tg {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_ROW = 256;
constexpr int PROBE_ROWS = 64;
constexpr int PROBE_DWORDS = PROBE_ROW * PROBE_ROWS / 4;

__device__ __forceinline__ uint32_t probe_pattern(uint32_t i) { return i * 2654435761u ^ (i >> 7); }

// pattern 1: byte address of 16-byte piece c (0..3) of lane l of wave w in
// iteration r
__device__ __forceinline__ uint32_t probe_addr(int l, int w, int r, int c) {
    const int row = (l & 31) + 32 * (c & 1);
    const int chunk = ((l >> 5) + 2 * (c >> 1) + 4 * ((r + w) & 3)) & 15;
    return row * PROBE_ROW + (chunk ^ (row & 15)) * 16;
}

__device__ __forceinline__ uint32_t fold16(uint32_t x) { return (x ^ (x >> 16)) & 0xffffu; }

template <int KIND, int PATTERN>
__global__ __launch_bounds__(PROBE_THREADS) void lds_read_probe(uint32_t* out, int reps) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[PROBE_DWORDS];
    for (int i = threadIdx.x; i < PROBE_DWORDS; i += PROBE_THREADS) lds[i] = probe_pattern(i);
    __syncthreads();
    const uint32_t base = (uint32_t)(uintptr_t)(TG_LDS char*)(lds);
    const int l = lane_id(), w = wave_id();
    // pattern 0: this lane's slot in the wave's 4 KiB quarter; instruction j
    // adds j * 64 * W (an immediate offset)
    constexpr int W = KIND == 0 ? 4 : KIND == 2 ? 16 : 8;
    const uint32_t lin = base + w * 4096 + l * W;
    uint32_t acc = 0;
    for (int r = 0; r < reps; ++r) {
        uint32_t a[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) a[c] = base + probe_addr(l, w, r, c);
        uint32_t f = 0;
        if constexpr (KIND == 0) {
            uint32_t v[16];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if constexpr (PATTERN == 0)
                        asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v[4 * c + d]) : "v"(lin), "n"(256 * (4 * c + d)));
                    else
                        asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v[4 * c + d]) : "v"(a[c]), "n"(4 * d));
                }
            // the wait names every result, so no use of one moves above it
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                           "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]),
                           "+v"(v[14]), "+v"(v[15]));
#pragma unroll
            for (int i = 0; i < 16; ++i) f ^= v[i];
        } else if constexpr (KIND == 2) {
            i32x4 v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (PATTERN == 0)
                    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v[c]) : "v"(lin), "n"(1024 * c));
                else
                    asm volatile("ds_read_b128 %0, %1" : "=v"(v[c]) : "v"(a[c]));
            }
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
            for (int c = 0; c < 4; ++c) f ^= uint32_t(v[c][0] ^ v[c][1] ^ v[c][2] ^ v[c][3]);
        } else {
            i32x2 v[8];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t ad = PATTERN == 0 ? lin : a[c];
                    if constexpr (KIND == 1) {
                        if constexpr (PATTERN == 0)
                            asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v[2 * c + h]) : "v"(ad), "n"(512 * (2 * c + h)));
                        else
                            asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v[2 * c + h]) : "v"(ad), "n"(8 * h));
                    } else {
                        if constexpr (PATTERN == 0)
                            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                                         : "=v"(v[2 * c + h])
                                         : "v"(ad), "n"(512 * (2 * c + h)));
                        else
                            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                                         : "=v"(v[2 * c + h])
                                         : "v"(ad), "n"(8 * h));
                    }
                }
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                           "+v"(v[7]));
#pragma unroll
            for (int i = 0; i < 8; ++i) f ^= uint32_t(v[i][0] ^ v[i][1]);
        }
        acc = (((acc << 1) | (acc >> 15)) & 0xffffu) ^ fold16(f);
    }
    out[(int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = acc;
}

// ---------------------------------------------------------------------------
// Matrix-core rate probe: the matrix-core instruction of each GEMM type
// issued back to back with no memory traffic, to measure the rate the chip
// sustains for given operand bits (the dense peak assumes the nominal clock;
// the clock the power budget allows depends on what the operands toggle).
//
// Each of the 4 waves of a workgroup loads 4 A and 4 B operand registers
// (16 bytes each) per lane, then runs `reps` iterations of 16 independent
// accumulators, acc[i] += mma(a[i % 4], b[(i / 4) % 4]).  Wave 0 records the
// shader-clock ticks (s_memtime) and the 100 MHz real-time ticks
// (s_memrealtime) around the loop; their ratio is the clock.
constexpr int RATE_THREADS = 256;
constexpr int RATE_ACC = 16;

template <int KIND>
__global__ __launch_bounds__(RATE_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_rate_probe(const i32x4* operands, uint32_t* out, uint64_t* clocks, int reps) {
    const int64_t t = (int64_t)blockIdx.x * RATE_THREADS + threadIdx.x;
    i32x4 a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a[q] = operands[t * 8 + q];
        b[q] = operands[t * 8 + 4 + q];
    }
    typedef typename std::conditional<KIND == 0, f32x16, i32x16>::type Acc;
    Acc acc[RATE_ACC];
#pragma unroll
    for (int i = 0; i < RATE_ACC; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < reps; ++it) {
#pragma unroll
        for (int i = 0; i < RATE_ACC; ++i) {
            if constexpr (KIND == 0)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i & 3]),
                                                                 __builtin_bit_cast(bf16x8, b[(i >> 2) & 3]),
                                                                 acc[i], 0, 0, 0);
            else
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i & 3], b[(i >> 2) & 3], acc[i], 0, 0, 0);
        }
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    // fold every accumulator register so that no matrix instruction is dead
    if constexpr (KIND == 0) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < RATE_ACC; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][r];
        out[t] = __builtin_bit_cast(uint32_t, s);
    } else {
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < RATE_ACC; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += (uint32_t)acc[i][r];
        out[t] = s;
    }
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

// The fp32 vector counterpart: 16 independent v_fmac_f32 chains per thread,
// every operand in a VGPR, acc[i] = fma(x[i], y[i], acc[i]) with x the 16
// floats of the thread's A registers and y those of its B registers.  Built
// for up to 8 waves per SIMD, so that the number of workgroups per compute
// unit sets how many waves share a SIMD.
__global__ __launch_bounds__(RATE_THREADS) __attribute__((amdgpu_waves_per_eu(1, 8)))
void fma_rate_probe(const i32x4* operands, uint32_t* out, uint64_t* clocks, int reps) {
    const int64_t t = (int64_t)blockIdx.x * RATE_THREADS + threadIdx.x;
    float x[16], y[16], acc[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 a = __builtin_bit_cast(f32x4, operands[t * 8 + q]);
        const f32x4 b = __builtin_bit_cast(f32x4, operands[t * 8 + 4 + q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[4 * q + e] = a[e];
            y[4 * q + e] = b[e];
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < reps; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = __builtin_fmaf(x[i], y[i], acc[i]);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[i];
    out[t] = __builtin_bit_cast(uint32_t, s);
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

// The bf16 matrix-core stream of the default 256 x 256 x 64 GEMM kernel
// with its on-chip data movement added step by step, no barrier and no C
// store: where the clock the power budget allows goes between the bare
// matrix instructions (mfma_rate_probe) and the GEMM.  Per wave and K step,
// as in that kernel's 128 x 64 wave tile: 8 matrix instructions on 4 A and 2
// B fragments; the next step's fragments are read from LDS meanwhile (4 x
// ds_read_b128 for A, 4 x ds_read_b64_tr_b16 for B, one read after each
// matrix instruction), so the matrix instructions consume LDS data.  DMA
// adds the direct global -> LDS copies at the kernel's rate, 8 per 32 matrix
// instructions per wave (2 per loop iteration), from the workgroup's operand
// bytes (L2-resident) into an LDS region the reads never touch.  One loop
// iteration is two K steps (16 matrix instructions, as in the rate probe).
constexpr int MIX_READ_BYTES = 16384;  // LDS the fragments are read from
constexpr int MIX_DMA_BYTES = 16384;   // LDS the copies land in

template <bool DMA>
__global__ __launch_bounds__(RATE_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_mix_probe(const i32x4* operands, uint32_t* out, uint64_t* clocks, int reps) {
    __shared__ __attribute__((aligned(1024))) char lds_raw[MIX_READ_BYTES + MIX_DMA_BYTES];
    TG_LDS char* lds = (TG_LDS char*)(lds_raw);
    const int64_t t = (int64_t)blockIdx.x * RATE_THREADS + threadIdx.x;
    const i32x4* wg_ops = operands + (int64_t)blockIdx.x * RATE_THREADS * 8;
    // the read region: the workgroup's first 16 KiB of operand bytes
    for (int i = threadIdx.x; i < MIX_READ_BYTES / 16; i += RATE_THREADS)
        *reinterpret_cast<TG_LDS i32x4*>(lds + 16 * i) = wg_ops[i];
    __syncthreads();
    const int lane = lane_id(), wave = wave_id();
    // lane offsets of the reads: A fragment f of step s at 1 KiB-aligned
    // rows of the read region (16 B per lane, conflict-free); B halves at
    // 8 B per lane
    const uint32_t rbase = (uint32_t)(uintptr_t)lds;
    const uint32_t dbase = rbase + MIX_READ_BYTES;
    i32x4 a[2][4], b[2][2];
#pragma unroll
    for (int f = 0; f < 4; ++f) a[0][f] = *reinterpret_cast<const TG_LDS i32x4*>(lds + 1024 * f + 16 * lane);
#pragma unroll
    for (int f = 0; f < 2; ++f) b[0][f] = *reinterpret_cast<const TG_LDS i32x4*>(lds + 4096 + 1024 * f + 16 * lane);
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const char* src = reinterpret_cast<const char*>(wg_ops);
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < reps; ++it) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int cur = st, nxt = st ^ 1;
            // the step's read window rotates through the region
            const uint32_t win = (uint32_t)(((it * 2 + st + 1) & 3) * 4096);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = k >> 1, j = k & 1;
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[cur][i]),
                                                                 __builtin_bit_cast(bf16x8, b[cur][j]), acc[k], 0,
                                                                 0, 0);
                if (k < 4) {
                    a[nxt][k] = *reinterpret_cast<const TG_LDS i32x4*>(lds + win + 1024 * k + 16 * lane);
                } else {
                    const int f = (k - 4) >> 1, h = (k - 4) & 1;
                    const TG_LDS char* pb = lds + ((win + 2048) & (MIX_READ_BYTES - 1)) + 1024 * f + 512 * h + 8 * lane;
                    const i32x2 v = __builtin_bit_cast(
                        i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS i16x4*)(pb)));
                    if (h == 0) {
                        b[nxt][f].x = v.x;
                        b[nxt][f].y = v.y;
                    } else {
                        b[nxt][f].z = v.x;
                        b[nxt][f].w = v.y;
                    }
                }
                if (DMA && (k == 3 || k == 7)) {
                    // copy (it * 4 + st * 2 + k / 4) of this wave: 1 KiB from the
                    // workgroup's operand bytes into the copy region
                    const int n = it * 4 + st * 2 + (k >> 2);
                    const uint32_t lds_dst = dbase + (uint32_t)(((n * 4 + wave) & 15) * 1024);
                    const uint32_t voff = (uint32_t)(((n * 4 + wave) & 31) * 1024 + 16 * lane);
                    copy16_to_lds(lds_dst, voff, src);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (DMA) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        }
    }
    if (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][r];
    out[t] = __builtin_bit_cast(uint32_t, sum);
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

}  // namespace tg

extern "C" int tgemm_lds_read_probe(int32_t kind, int32_t pattern, int32_t reps, int32_t workgroups, uint32_t* out,
                                    void* stream) {
    if (kind < 0 || kind > 3 || pattern < 0 || pattern > 1 || reps < 0 || workgroups < 1) return TGEMM_E_ARG;
    if (!out) return TGEMM_E_NULL;
    if ((uintptr_t)out % 4) return TGEMM_E_ALIGN;
    static void (*const fns[2][4])(uint32_t*, int) = {
        {tg::lds_read_probe<0, 0>, tg::lds_read_probe<1, 0>, tg::lds_read_probe<2, 0>, tg::lds_read_probe<3, 0>},
        {tg::lds_read_probe<0, 1>, tg::lds_read_probe<1, 1>, tg::lds_read_probe<2, 1>, tg::lds_read_probe<3, 1>}};
    void* args[] = {&out, &reps};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fns[pattern][kind]), dim3((unsigned)workgroups),
                                           dim3(tg::PROBE_THREADS), args, 0, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TGEMM_OK : TGEMM_E_HIP;
}

extern "C" int tgemm_mfma_rate_probe(int32_t kind, int32_t reps, int32_t workgroups, const void* operands,
                                     uint32_t* out, uint64_t* clocks, void* stream) {
    if (kind < 0 || kind > 4 || reps < 0 || workgroups < 1) return TGEMM_E_ARG;
    if (!operands || !out || !clocks) return TGEMM_E_NULL;
    if ((uintptr_t)operands % 16 || (uintptr_t)out % 4 || (uintptr_t)clocks % 8) return TGEMM_E_ALIGN;
    static void (*const fns[5])(const tg::i32x4*, uint32_t*, uint64_t*, int) = {
        tg::mfma_rate_probe<0>, tg::mfma_rate_probe<1>, tg::fma_rate_probe, tg::mfma_mix_probe<false>,
        tg::mfma_mix_probe<true>};
    const tg::i32x4* ops = static_cast<const tg::i32x4*>(operands);
    void* args[] = {&ops, &out, &clocks, &reps};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fns[kind]), dim3((unsigned)workgroups),
                                           dim3(tg::RATE_THREADS), args, 0, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TGEMM_OK : TGEMM_E_HIP;
}
