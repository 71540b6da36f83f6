// fp32 GEMM on the vector ALUs (no matrix cores): the register-tiled
// outer-product kernel of "4.1 CUDA GEMM算子性能优化", sections 4-9, laid out
// for 64-wide waves, with the switches of the SIMT ladder of the SM80
// cp.async / ldmatrix ablation plan (section 1.5.4: tiling -> A transposed in
// shared memory -> conflict-free layout -> coalesced write-back -> double
// buffer), one per template parameter:
//
//   TRANS_A   A slice stored transposed in LDS (As[k][m], section 7.3), so the
//             A fragment is two 16-byte reads instead of eight 4-byte reads
//             of rows BK*4 bytes apart;
//   QUARTERS  the conflict-free layout: each lane's 8 x 8 outputs split into
//             4 x 4 quarters 32 rows / columns apart (section 8.5's sub-block
//             split), so the 16-byte fragment reads of a wave cover 8
//             contiguous 16-byte words, and the rows of transposed A padded
//             (section 8's padding fix) so that the lanes writing one A row
//             of a slice land on different banks; off: one contiguous 8 x 8
//             block per lane, unpadded rows;
//   VEC_STORE C written as 16-byte row pieces (one instruction writes whole
//             128-byte row segments); off: one float per store;
//   STAGES    1: load slice, barrier, compute, barrier.  2: the
//             register-staged double buffer of section 9.5 (issue the loads of
//             slice t+1, compute slice t, store slice t+1 to the other
//             buffer, one barrier).
//
// Workgroup tile TILE x TILE (128, or 64 for grids too small to fill the
// compute units), K slice BK (8, or 16 in the default kernel), 256 threads =
// 4 waves in a 2 x 2 grid, each wave TILE/2 x TILE/2; lane l of a wave is
// (lr, lc) = (l / 8, l % 8) and owns TM x TM outputs, TM = TILE / 16.  The
// 64 x 64 tile spreads a product over four times the SIMDs of the 128 x 128
// one: on the vector ALUs a wave's time is set by its count of FMAs.
//
// Every C element is one fused multiply-add chain in increasing k, started
// from zero: acc = fma(a_ik, b_kj, acc).  The K tail is zero-filled, and
// fma(0, b, acc) = acc, so the result equals the sequential single-precision
// fma chain bit for bit in every variant.
#pragma once

#include "tg_device.hpp"

namespace tg {

template <int STAGES, bool TRANS_A, bool QUARTERS, bool VEC_STORE, int BK_ = 8, int TILE = 128, int TILE_N = TILE>
struct F32Gemm {
    static constexpr int BM = TILE, BN = TILE_N, BK = BK_, NT = 256;
    static constexpr int TM = BM / 16;        // outputs per lane along M
    static constexpr int TN = BN / 16;        // outputs per lane along N
    static constexpr int AQ = BK / 4;         // pieces per A row of a slice
    // Row stride of transposed A in floats.  The 4 k-rows of one A piece go
    // to rows kq .. kq+3; AQ lanes with the same m but kq = 0, 4, .. write
    // each of them.  Padding by 16 / AQ floats (at least 4, to keep 16-byte
    // reads aligned) moves consecutive kq a quarter (AQ = 4) or half (AQ = 2)
    // of the 64 banks apart: no conflicts for 8- and 16-deep slices, 2-way
    // for 32-deep ones.
    static constexpr int AS_LD = BM + ((TRANS_A && QUARTERS) ? (16 / AQ > 4 ? 16 / AQ : 4) : 0);
    static constexpr int A_BYTES = TRANS_A ? BK * AS_LD * 4 : BK * BM * 4;
    static constexpr int B_BYTES = BK * BN * 4;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * SLOT;
    static constexpr int PA = BK * BM / 4 / NT;  // 16-byte pieces of A per thread per slice
    static constexpr int PB = BK * BN / 4 / NT;  // and of B
    static constexpr int N_LD = PA + PB;
    static constexpr int BQ = BN / 4;         // pieces per B row of a slice
    static_assert(STAGES == 1 || STAGES == 2, "register-staged: 1 or 2 slots");
    static_assert((TM == 4 && TN == 4) || (TM == 8 && TN == 8) || (TM == 8 && TN == 16 && QUARTERS),
                  "lane blocks of 4 x 4, 8 x 8, or 8 x 16 in the quarter layout");
    static_assert(PA >= 1 && PB >= 1 && (BK * BM / 4) % NT == 0 && (BK * BN / 4) % NT == 0,
                  "whole pieces per thread");

    struct Staged {
        f32x4 a[PA], b[PB];
    };

    // Piece p = q NT + t (q < PER) of the slice: A[m0 + p / AQ][k0 + 4 (p % AQ) .. +3]
    // and B[k0 + p / BQ][n0 + 4 (p % BQ) .. +3].
    template <bool GA, bool GB>
    __device__ static __forceinline__ void load_t(Staged& r, const GemmArgs& g, int m0, int n0, int k0) {
        load_any(r, g, m0, n0, k0, GA, GB);
    }

    __device__ static __forceinline__ void load(Staged& r, const GemmArgs& g, int m0, int n0, int k0,
                                                bool guard_a, bool guard_b) {
        load_any(r, g, m0, n0, k0, guard_a, guard_b);
    }

    __device__ static __forceinline__ void load_any(Staged& r, const GemmArgs& g, int m0, int n0, int k0,
                                                    bool guard_a, bool guard_b) {
        const float* A = static_cast<const float*>(g.A);
        const float* B = static_cast<const float*>(g.B);
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int p = q * NT + threadIdx.x;
            const float* rowp = A + (int64_t)min(m0 + p / AQ, g.M - 1) * g.lda;
            const int kc = k0 + 4 * (p % AQ);
            if (!guard_a) {
                r.a[q] = *reinterpret_cast<const f32x4*>(rowp + kc);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) r.a[q][e] = kc + e < g.K ? rowp[kc + e] : 0.0f;
            }
        }
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            const int p = q * NT + threadIdx.x;
            const int gk = k0 + p / BQ;
            const int nc = n0 + 4 * (p % BQ);
            if (!guard_b) {
                r.b[q] = *reinterpret_cast<const f32x4*>(B + (int64_t)gk * g.ldb + min(nc, g.N - 4));
            } else {
                const float* rowp = B + (int64_t)min(gk, g.K - 1) * g.ldb;
#pragma unroll
                for (int e = 0; e < 4; ++e) r.b[q][e] = (gk < g.K && nc + e < g.N) ? rowp[nc + e] : 0.0f;
            }
        }
    }

    __device__ static __forceinline__ void store(TG_LDS char* slot, const Staged& r) {
        TG_LDS float* As = reinterpret_cast<TG_LDS float*>(slot);
        TG_LDS float* Bs = reinterpret_cast<TG_LDS float*>(slot + A_BYTES);
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int p = q * NT + threadIdx.x;
            const int row = p / AQ, kq = 4 * (p % AQ);
            if constexpr (TRANS_A) {
#pragma unroll
                for (int e = 0; e < 4; ++e) As[(kq + e) * AS_LD + row] = r.a[q][e];
            } else {
                *reinterpret_cast<TG_LDS f32x4*>(As + row * BK + kq) = r.a[q];
            }
        }
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            const int p = q * NT + threadIdx.x;
            *reinterpret_cast<TG_LDS f32x4*>(Bs + (p / BQ) * BN + 4 * (p % BQ)) = r.b[q];
        }
    }

    // Row (column) offset of this lane's fragment element i within the tile.
    // (With TM = 4 both forms are the lane's 4 contiguous rows.)
    __device__ static __forceinline__ int frag_off(int base, int idx, int i) {
        if constexpr (QUARTERS) return base + 4 * idx + (i & 3) + 32 * (i >> 2);
        else return base + TM * idx + i;
    }

    struct Frag {
        float a[TM], b[TN];
    };

    __device__ static __forceinline__ void read_frag(Frag& f, const TG_LDS char* slot, int k, int wm, int wn,
                                                     int lr, int lc) {
        const TG_LDS float* As = reinterpret_cast<const TG_LDS float*>(slot);
        const TG_LDS float* Bs = reinterpret_cast<const TG_LDS float*>(slot + A_BYTES);
        if constexpr (TRANS_A) {
            // rows frag_off(wm, lr, 4h .. 4h+3) are 4 contiguous for each h
#pragma unroll
            for (int h = 0; h < TM / 4; ++h) {
                const f32x4 a = *reinterpret_cast<const TG_LDS f32x4*>(As + k * AS_LD + frag_off(wm, lr, 4 * h));
                f.a[4 * h] = a.x; f.a[4 * h + 1] = a.y; f.a[4 * h + 2] = a.z; f.a[4 * h + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) f.a[i] = As[frag_off(wm, lr, i) * BK + k];
        }
#pragma unroll
        for (int h = 0; h < TN / 4; ++h) {
            const f32x4 b = *reinterpret_cast<const TG_LDS f32x4*>(Bs + k * BN + frag_off(wn, lc, 4 * h));
            f.b[4 * h] = b.x; f.b[4 * h + 1] = b.y; f.b[4 * h + 2] = b.z; f.b[4 * h + 3] = b.w;
        }
    }

    // End of one outer-product step: an empty asm that takes every
    // accumulator in and out and clobbers memory, so that this step's FMAs
    // stay before it, the next step's after it, and the LDS reads issued for
    // the step after next cannot be hoisted above it (neither the FMAs nor
    // plain LDS loads are ordered by a scheduling barrier alone).
    __device__ static __forceinline__ void step_fence(float (&c)[TM][TN]) {
        if constexpr (TN == 16) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                asm volatile(""
                             : "+v"(c[i][0]), "+v"(c[i][1]), "+v"(c[i][2]), "+v"(c[i][3]), "+v"(c[i][4]),
                               "+v"(c[i][5]), "+v"(c[i][6]), "+v"(c[i][7]), "+v"(c[i][8]), "+v"(c[i][9]),
                               "+v"(c[i][10]), "+v"(c[i][11]), "+v"(c[i][12]), "+v"(c[i][13]), "+v"(c[i][14]),
                               "+v"(c[i][15])
                             :
                             : "memory");
        } else if constexpr (TM == 8) {
#pragma unroll
            for (int i = 0; i < 8; i += 2)
                asm volatile(""
                             : "+v"(c[i][0]), "+v"(c[i][1]), "+v"(c[i][2]), "+v"(c[i][3]), "+v"(c[i][4]),
                               "+v"(c[i][5]), "+v"(c[i][6]), "+v"(c[i][7]), "+v"(c[i + 1][0]), "+v"(c[i + 1][1]),
                               "+v"(c[i + 1][2]), "+v"(c[i + 1][3]), "+v"(c[i + 1][4]), "+v"(c[i + 1][5]),
                               "+v"(c[i + 1][6]), "+v"(c[i + 1][7])
                             :
                             : "memory");
        } else {
            asm volatile(""
                         : "+v"(c[0][0]), "+v"(c[0][1]), "+v"(c[0][2]), "+v"(c[0][3]), "+v"(c[1][0]),
                           "+v"(c[1][1]), "+v"(c[1][2]), "+v"(c[1][3]), "+v"(c[2][0]), "+v"(c[2][1]),
                           "+v"(c[2][2]), "+v"(c[2][3]), "+v"(c[3][0]), "+v"(c[3][1]), "+v"(c[3][2]),
                           "+v"(c[3][3])
                         :
                         : "memory");
        }
    }

    // The slice's BK outer products, each lane's TM x TM block at a time.  The
    // fragments of step k+1 are read while the TM^2 FMAs of step k issue, and a
    // fence per step keeps the compiler from hoisting the reads of the whole
    // slice ahead (which took 219 registers and limited a SIMD to 2 waves).
    __device__ static __forceinline__ void compute(const TG_LDS char* slot, float (&c)[TM][TN], int wm, int wn,
                                                   int lr, int lc) {
        Frag f[2];
        read_frag(f[0], slot, 0, wm, wn, lr, lc);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            if (k + 1 < BK) read_frag(f[(k + 1) & 1], slot, k + 1, wm, wn, lr, lc);
            const Frag& x = f[k & 1];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) c[i][j] = __builtin_fmaf(x.a[i], x.b[j], c[i][j]);
            step_fence(c);
        }
    }

    __device__ static void run(const GemmArgs& g) {
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
        TG_LDS char* smem = (TG_LDS char*)(smem_raw);
        ClockMark clk;
        clk.start(g.clocks);
        int tm, tn;
        tile_of_workgroup(g, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int wave = wave_id(), lane = lane_id();
        const int lr = lane >> 3, lc = lane & 7;
        const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

        float c[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) c[i][j] = 0.0f;

        const int tiles = (g.K + BK - 1) / BK;
        const int full = g.K / BK;
        const bool ga = g.a_guard != 0, gb = g.b_guard != 0;
        if constexpr (STAGES == 1) {
            for (int t = 0; t < tiles; ++t) {
                Staged r;
                load(r, g, m0, n0, t * BK, ga || t >= full, gb || t >= full);
                store(smem, r);
                wait_lds_then_barrier();
                compute(smem, c, wm, wn, lr, lc);
                wait_lds_then_barrier();
            }
        } else {
            if (tiles > 0) {
                Staged r;
                load(r, g, m0, n0, 0, ga || full == 0, gb || full == 0);
                store(smem, r);
                wait_lds_then_barrier();
            }
            int t = 0;
            if (!ga && !gb) {
                // whole slices of aligned operands: no guarded paths in the loop
#pragma nounroll
                for (; t + 1 < full; ++t) {
                    Staged r;
                    load_t<false, false>(r, g, m0, n0, (t + 1) * BK);
                    compute(smem + (t & 1) * SLOT, c, wm, wn, lr, lc);
                    store(smem + ((t + 1) & 1) * SLOT, r);
                    wait_lds_then_barrier();
                }
            }
#pragma nounroll
            for (; t < tiles; ++t) {
                const int nxt = t + 1;
                Staged r;
                if (nxt < tiles) load(r, g, m0, n0, nxt * BK, ga || nxt >= full, gb || nxt >= full);
                compute(smem + (t & 1) * SLOT, c, wm, wn, lr, lc);
                if (nxt < tiles) store(smem + (nxt & 1) * SLOT, r);
                wait_lds_then_barrier();
            }
        }

        clk.loop_end(g.clocks);
        float* C = static_cast<float*>(g.C);
        const bool vec_ok = VEC_STORE && (m0 + BM <= g.M) && (n0 + BN <= g.N) && (g.ldc % 4 == 0) &&
                            ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = m0 + frag_off(wm, lr, i);
            if (vec_ok) {
                // columns frag_off(wn, lc, 4h .. 4h+3) are 4 contiguous for each h
#pragma unroll
                for (int h = 0; h < TN / 4; ++h)
                    *reinterpret_cast<f32x4*>(C + (int64_t)row * g.ldc + n0 + frag_off(wn, lc, 4 * h)) =
                        f32x4{c[i][4 * h], c[i][4 * h + 1], c[i][4 * h + 2], c[i][4 * h + 3]};
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + frag_off(wn, lc, j);
                    if (row < g.M && col < g.N) C[(int64_t)row * g.ldc + col] = c[i][j];
                }
            }
        }
        clk.finish(g.clocks);
    }
};

// One thread per C element, no LDS: the naive kernel of section 3.1 (the
// ladder's anchor).  fp32 accumulation as one fma chain in increasing k
// (int32 sums for int8).
template <int DT>
struct NaiveGemm {
    static constexpr int BM = 16, BN = 16, NT = 256;
    __device__ static void run(const GemmArgs& g) {
        int tm, tn;
        tile_of_workgroup(g, tm, tn);
        const int row = tm * BM + (threadIdx.x >> 4);
        const int col = tn * BN + (threadIdx.x & 15);
        if (row >= g.M || col >= g.N) return;
        if constexpr (DT == 0) {  // fp32
            const float* A = static_cast<const float*>(g.A) + (int64_t)row * g.lda;
            const float* B = static_cast<const float*>(g.B) + col;
            float acc = 0.0f;
            for (int k = 0; k < g.K; ++k) acc = __builtin_fmaf(A[k], B[(int64_t)k * g.ldb], acc);
            static_cast<float*>(g.C)[(int64_t)row * g.ldc + col] = acc;
        } else if constexpr (DT == 1) {  // bf16 bits
            const uint16_t* A = static_cast<const uint16_t*>(g.A) + (int64_t)row * g.lda;
            const uint16_t* B = static_cast<const uint16_t*>(g.B) + col;
            float acc = 0.0f;
            for (int k = 0; k < g.K; ++k) {
                const float a = __uint_as_float((uint32_t)A[k] << 16);
                const float b = __uint_as_float((uint32_t)B[(int64_t)k * g.ldb] << 16);
                acc = __builtin_fmaf(a, b, acc);
            }
            static_cast<float*>(g.C)[(int64_t)row * g.ldc + col] = acc;
        } else {  // int8
            const int8_t* A = static_cast<const int8_t*>(g.A) + (int64_t)row * g.lda;
            const int8_t* B = static_cast<const int8_t*>(g.B) + col;
            int32_t acc = 0;
            for (int k = 0; k < g.K; ++k) acc += (int32_t)A[k] * (int32_t)B[(int64_t)k * g.ldb];
            static_cast<int32_t*>(g.C)[(int64_t)row * g.ldc + col] = acc;
        }
    }
};

}  // namespace tg
