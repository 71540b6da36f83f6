// fp32 GEMM on the vector ALUs (no matrix cores): the register-tiled
// outer-product kernel of "4.1 CUDA GEMM算子性能优化", sections 4-10, laid
// out for 64-wide waves, with one switch per step of the SIMT ladder (the
// SM80 cp.async / ldmatrix ablation plan, section 1.5.4) in FLAGS:
//
//   F_NO_REUSE  block tiling alone (section 4): every FMA reads its two
//               operands from LDS; off: each k step reads the lane's TM + TN
//               fragment values into registers once and reuses them over the
//               TM x TN outer product (section 5, register tiling);
//   F_GLOBAL4   4-byte global loads and LDS writes; off: 16-byte (float4)
//               ones (section 7.1-7.2);
//   F_TRANS_A   A slice stored transposed in LDS (As[k][m], section 7.3), so
//               that the A fragment is 16-byte reads, and B's fragment too is
//               read 16 bytes at a time; off: A row-major, both fragments
//               read 4 bytes at a time;
//   F_PAD_A     the rows of transposed A padded so that the lanes writing one
//               A row of a slice land on different banks (section 8.5,
//               scheme 1);
//   F_QUARTERS  each lane's 8 x 8 outputs split into 4 x 4 quarters 32 rows /
//               columns apart (section 8.5, scheme 4, and the coordinate map
//               of section 7.4); off: one contiguous block per lane;
//   F_ZORDER    lanes placed on the wave's 8 x 8 grid in Z order (section 8.5,
//               scheme 3: each 16-lane group covers a 4 x 4 square of lane
//               positions instead of 2 rows of 8); off: row-major;
//   F_VEC_STORE C written as 16-byte row pieces; off: one float per store;
//   F_AKVEC     A row-major in LDS and read as 16-byte pieces along K (four
//               k steps at a time): the layout a copy that does not pass
//               through registers produces (it cannot transpose);
//   F_DIRECT    both operands copied global -> LDS with global_load_lds_dwordx4
//               (section 10, the asynchronous copy) through a ring of STAGES
//               slots: wait for slice t, barrier, issue slice t + STAGES - 1
//               into the slot slice t - 1 left, multiply slice t.
//   STAGES      register-staged: 1 (load slice, barrier, multiply, barrier) or
//               2 (section 9.5: issue the loads of slice t+1, multiply slice
//               t, store slice t+1 to the other buffer, one barrier); direct:
//               1 to 4 slots.
//
// Workgroup tile BM x BN (128 x 128, 64 x 64 for grids too small to fill the
// compute units, 128 x 256), K slice BK, 256 threads = 4 waves in a 2 x 2
// grid, each wave BM/2 x BN/2; lane (lr, lc) of the wave's 8 x 8 lane grid
// owns TM x TN outputs, TM = BM / 16, TN = BN / 16.
//
// Every C element is one fused multiply-add chain in increasing k, started
// from zero: acc = fma(a_ik, b_kj, acc).  The K tail is zero-filled, and
// fma(0, b, acc) = acc, so the result equals the sequential single-precision
// fma chain bit for bit in every variant.
#pragma once

#include "tg_device.hpp"

namespace tg {

enum F32Flags {
    F_TRANS_A = 1,
    F_QUARTERS = 2,
    F_VEC_STORE = 4,
    F_PAD_A = 8,
    F_NO_REUSE = 16,
    F_ZORDER = 32,
    F_GLOBAL4 = 64,
    F_AKVEC = 128,
    F_DIRECT = 256,
};

template <int STAGES, int FLAGS, int BK_ = 8, int TILE = 128, int TILE_N = TILE>
struct F32Gemm {
    static constexpr bool TRANS_A = FLAGS & F_TRANS_A, QUARTERS = FLAGS & F_QUARTERS;
    static constexpr bool VEC_STORE = FLAGS & F_VEC_STORE, PAD_A = FLAGS & F_PAD_A;
    static constexpr bool REUSE = !(FLAGS & F_NO_REUSE), ZORDER = FLAGS & F_ZORDER;
    static constexpr bool WIDE_G = !(FLAGS & F_GLOBAL4), AKVEC = FLAGS & F_AKVEC, DIRECT = FLAGS & F_DIRECT;
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
    static constexpr int AS_LD = BM + ((TRANS_A && PAD_A) ? (16 / AQ > 4 ? 16 / AQ : 4) : 0);
    static constexpr int A_BYTES = TRANS_A ? BK * AS_LD * 4 : BK * BM * 4;
    static constexpr int B_BYTES = BK * BN * 4;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * SLOT;
    static constexpr int PA = BK * BM / 4 / NT;  // 16-byte pieces of A per thread per slice
    static constexpr int PB = BK * BN / 4 / NT;  // and of B
    static constexpr int EA = BK * BM / NT;      // 4-byte elements of A per thread per slice
    static constexpr int EB = BK * BN / NT;
    static constexpr int N_LD = PA + PB;         // direct copies per thread (= per wave) per slice
    static constexpr int BQ = BN / 4;            // pieces per B row of a slice
    static_assert(DIRECT ? (STAGES >= 1 && STAGES <= 4) : (STAGES == 1 || STAGES == 2),
                  "register-staged: 1 or 2 slots; direct: 1 to 4");
    static_assert((TM == 4 && TN == 4) || (TM == 8 && TN == 8) || (TM == 8 && TN == 16 && QUARTERS),
                  "lane blocks of 4 x 4, 8 x 8, or 8 x 16 in the quarter layout");
    static_assert(PA >= 1 && PB >= 1 && (BK * BM / 4) % NT == 0 && (BK * BN / 4) % NT == 0,
                  "whole pieces per thread");
    static_assert(!PAD_A || TRANS_A, "padding is for the rows of transposed A");
    static_assert(!(TRANS_A && AKVEC), "A is either transposed or read along K");
    static_assert(!DIRECT || (AKVEC && WIDE_G && REUSE), "direct copies: 16-byte pieces, A row-major");
    static_assert(!AKVEC || (BK % 4 == 0 && REUSE), "A read four k steps at a time");
    static_assert(WIDE_G || !TRANS_A, "the narrow-load rungs keep A row-major");
    static_assert(REUSE || (!TRANS_A && !QUARTERS), "per-FMA reads: the block-tiling rung");
    static_assert(N_LD * (STAGES > 2 ? STAGES - 2 : 0) <= 63, "vmcnt range");

    struct Staged {
        f32x4 a[PA], b[PB];
        float ae[WIDE_G ? 1 : EA], be[WIDE_G ? 1 : EB];
    };

    // 16-byte pieces: piece p = q NT + t (q < PA) of the slice is
    // A[m0 + p / AQ][k0 + 4 (p % AQ) .. +3], and B[k0 + p / BQ][n0 + 4 (p % BQ) .. +3].
    // 4-byte elements (F_GLOBAL4): element p is A[m0 + p / BK][k0 + p % BK]
    // and B[k0 + p / BN][n0 + p % BN].
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
        if constexpr (!WIDE_G) {
#pragma unroll
            for (int q = 0; q < EA; ++q) {
                const int p = q * NT + threadIdx.x;
                const int kc = k0 + p % BK;
                const float* rowp = A + (int64_t)min(m0 + p / BK, g.M - 1) * g.lda;
                r.ae[q] = load_or_zero(rowp + kc, kc < g.K);
            }
#pragma unroll
            for (int q = 0; q < EB; ++q) {
                const int p = q * NT + threadIdx.x;
                const int gk = k0 + p / BN, nc = n0 + p % BN;
                r.be[q] = load_or_zero(B + (int64_t)gk * g.ldb + nc, gk < g.K && nc < g.N);
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int p = q * NT + threadIdx.x;
            const float* rowp = A + (int64_t)min(m0 + p / AQ, g.M - 1) * g.lda;
            const int kc = k0 + 4 * (p % AQ);
            if (!guard_a) {
                r.a[q] = *reinterpret_cast<const f32x4*>(rowp + kc);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) r.a[q][e] = load_or_zero(rowp + kc + e, kc + e < g.K);
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
                for (int e = 0; e < 4; ++e) r.b[q][e] = load_or_zero(rowp + nc + e, gk < g.K && nc + e < g.N);
            }
        }
    }

    __device__ static __forceinline__ void store(TG_LDS char* slot, const Staged& r) {
        TG_LDS float* As = reinterpret_cast<TG_LDS float*>(slot);
        TG_LDS float* Bs = reinterpret_cast<TG_LDS float*>(slot + A_BYTES);
        if constexpr (!WIDE_G) {
            // element p of a slice sits at float p of As[m][k] / Bs[k][n]
#pragma unroll
            for (int q = 0; q < EA; ++q) As[q * NT + threadIdx.x] = r.ae[q];
#pragma unroll
            for (int q = 0; q < EB; ++q) Bs[q * NT + threadIdx.x] = r.be[q];
            return;
        }
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

    // ---- direct copies (F_DIRECT): the slot holds A as [BM][BK] and B as
    // [BK][BN], both row-major, so copy q of a slice is the 16-byte piece q
    // of its region: lane l of copy i in wave w lands at (i NT + 64 w + l) 16.
    // Its global source, as a 32-bit byte offset from the slice's A / B base
    // (the host only picks these kernels when the offsets fit): A piece p ->
    // row p / AQ (clamped to M-1), column 4 (p % AQ); B piece p -> row p / BQ,
    // column 4 (p % BQ) clamped to the last whole piece of the row.
    struct DirectOffsets {
        uint32_t a[PA], b[PB];
    };

    __device__ static __forceinline__ void direct_offsets(DirectOffsets& o, const GemmArgs& g, int m0, int n0) {
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int p = q * NT + threadIdx.x;
            const int r = min(m0 + p / AQ, g.M - 1) - m0;
            o.a[q] = (uint32_t)(((int64_t)r * g.lda + 4 * (p % AQ)) * 4);
        }
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            const int p = q * NT + threadIdx.x;
            const int col = min(n0 + 4 * (p % BQ), g.N - 4) - n0;
            o.b[q] = (uint32_t)(((int64_t)(p / BQ) * g.ldb + col) * 4);
        }
    }

    __device__ static __forceinline__ void issue_direct(TG_LDS char* slot, const DirectOffsets& o, const char* abase,
                                                        const char* bbase, int wave) {
        const uint32_t lds = (uint32_t)(uintptr_t)slot;
#pragma unroll
        for (int i = 0; i < PA; ++i) copy16_to_lds(lds + (i * NT + wave * 64) * 16, o.a[i], abase);
#pragma unroll
        for (int i = 0; i < PB; ++i) copy16_to_lds(lds + A_BYTES + (i * NT + wave * 64) * 16, o.b[i], bbase);
    }

    // Wait until at most `ahead` slices' copies issued after the one needed
    // now are in flight, then barrier (the immediate selects among
    // compile-time instances).
    template <int AH>
    __device__ static __forceinline__ void wait_ahead(int ahead) {
        if constexpr (AH > 0) {
            if (ahead >= AH) {
                wait_vm_then_barrier<AH * N_LD>();
                return;
            }
            wait_ahead<AH - 1>(ahead);
        } else {
            wait_vm_then_barrier<0>();
        }
    }

    // Lane (lr, lc) on the wave's 8 x 8 lane grid: row-major, or Z order
    // (lr from lane bits 1, 3, 5 and lc from bits 0, 2, 4, so that each
    // 16-lane group covers a 4 x 4 square).
    __device__ static __forceinline__ void lane_pos(int lane, int& lr, int& lc) {
        if constexpr (ZORDER) {
            lr = ((lane >> 1) & 1) | ((lane >> 2) & 2) | ((lane >> 3) & 4);
            lc = (lane & 1) | ((lane >> 1) & 2) | ((lane >> 2) & 4);
        } else {
            lr = lane >> 3;
            lc = lane & 7;
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

    // The lane's fragment values of k step k: A rows frag_off(wm, lr, i) and
    // B columns frag_off(wn, lc, j).  With F_TRANS_A both come as 16-byte
    // pieces (4 consecutive rows / columns each); without it, one 4-byte read
    // per value (volatile, so that the compiler does not merge them).
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
#pragma unroll
            for (int h = 0; h < TN / 4; ++h) {
                const f32x4 b = *reinterpret_cast<const TG_LDS f32x4*>(Bs + k * BN + frag_off(wn, lc, 4 * h));
                f.b[4 * h] = b.x; f.b[4 * h + 1] = b.y; f.b[4 * h + 2] = b.z; f.b[4 * h + 3] = b.w;
            }
        } else {
            const volatile TG_LDS float* Av = As;
            const volatile TG_LDS float* Bv = Bs;
#pragma unroll
            for (int i = 0; i < TM; ++i) f.a[i] = Av[frag_off(wm, lr, i) * BK + k];
#pragma unroll
            for (int j = 0; j < TN; ++j) f.b[j] = Bv[k * BN + frag_off(wn, lc, j)];
        }
    }

    // F_AKVEC: the lane's A values of k steps 4 kk .. 4 kk + 3, one 16-byte
    // piece per row (a[i][d] = A[row_i][4 kk + d]).
    __device__ static __forceinline__ void read_a_kvec(f32x4 (&a)[TM], const TG_LDS char* slot, int kk, int wm,
                                                       int lr) {
        const TG_LDS float* As = reinterpret_cast<const TG_LDS float*>(slot);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = *reinterpret_cast<const TG_LDS f32x4*>(As + frag_off(wm, lr, i) * BK + 4 * kk);
    }

    __device__ static __forceinline__ void read_b(float (&b)[TN], const TG_LDS char* slot, int k, int wn, int lc) {
        const TG_LDS float* Bs = reinterpret_cast<const TG_LDS float*>(slot + A_BYTES);
#pragma unroll
        for (int h = 0; h < TN / 4; ++h) {
            const f32x4 v = *reinterpret_cast<const TG_LDS f32x4*>(Bs + k * BN + frag_off(wn, lc, 4 * h));
            b[4 * h] = v.x; b[4 * h + 1] = v.y; b[4 * h + 2] = v.z; b[4 * h + 3] = v.w;
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

    // The slice's BK outer products, each lane's TM x TN block at a time.  The
    // fragments of step k+1 are read while the TM x TN FMAs of step k issue,
    // and a fence per step keeps the compiler from hoisting the reads of the
    // whole slice ahead (which took 219 registers and limited a SIMD to 2
    // waves).  F_AKVEC: A's values of four k steps come from one 16-byte read
    // per row.  F_NO_REUSE: both operands of every FMA are read from LDS for
    // it.
    __device__ static __forceinline__ void compute(const TG_LDS char* slot, float (&c)[TM][TN], int wm, int wn,
                                                   int lr, int lc) {
        if constexpr (!REUSE) {
            const volatile TG_LDS float* As = reinterpret_cast<const volatile TG_LDS float*>(slot);
            const volatile TG_LDS float* Bs = reinterpret_cast<const volatile TG_LDS float*>(slot + A_BYTES);
#pragma unroll 1
            for (int k = 0; k < BK; ++k) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        c[i][j] = __builtin_fmaf(As[frag_off(wm, lr, i) * BK + k], Bs[k * BN + frag_off(wn, lc, j)],
                                                 c[i][j]);
            }
        } else if constexpr (AKVEC) {
#pragma unroll
            for (int kk = 0; kk < BK / 4; ++kk) {
                f32x4 a[TM];
                read_a_kvec(a, slot, kk, wm, lr);
                float b[2][TN];
                read_b(b[0], slot, 4 * kk, wn, lc);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if (d + 1 < 4) read_b(b[(d + 1) & 1], slot, 4 * kk + d + 1, wn, lc);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) c[i][j] = __builtin_fmaf(a[i][d], b[d & 1][j], c[i][j]);
                    step_fence(c);
                }
            }
        } else {
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
        int lr, lc;
        lane_pos(lane, lr, lc);
        const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

        float c[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) c[i][j] = 0.0f;

        const int tiles = (g.K + BK - 1) / BK;
        const int full = g.K / BK;
        const bool ga = g.a_guard != 0, gb = g.b_guard != 0;
        if constexpr (DIRECT) {
            // The ring: slices 0 .. STAGES-2 in flight before the loop.  In
            // iteration t: wait until slice t has landed (at most
            // min(STAGES-2, full-1-t) later slices still in flight) and
            // barrier, which also certifies that every wave is done with
            // slice t-1's slot; issue slice t + STAGES - 1 into that slot;
            // multiply slice t.  One slot: issue, wait, multiply, barrier.
            // The partial last slice follows through registers once the ring
            // has drained (the last wait is vmcnt(0)).
            DirectOffsets off;
            direct_offsets(off, g, m0, n0);
            const char* abase = static_cast<const char*>(g.A) + (int64_t)m0 * g.lda * 4;
            const char* bbase = static_cast<const char*>(g.B) + (int64_t)n0 * 4;
            const int64_t astep = (int64_t)BK * 4, bstep = (int64_t)BK * g.ldb * 4;
            auto issue_slice = [&](int sl) {
                issue_direct(smem + (sl % STAGES) * SLOT, off, abase + sl * astep, bbase + sl * bstep, wave);
            };
#pragma unroll
            for (int sl = 0; sl < STAGES - 1; ++sl)
                if (sl < full) issue_slice(sl);
            for (int t = 0; t < full; ++t) {
                if constexpr (STAGES == 1) {
                    issue_slice(t);
                    wait_all_then_barrier();
                } else {
                    wait_ahead<(STAGES > 2 ? STAGES - 2 : 0)>(min(STAGES - 2, full - 1 - t));
                    if (t + STAGES - 1 < full) issue_slice(t + STAGES - 1);
                }
                compute(smem + (t % STAGES) * SLOT, c, wm, wn, lr, lc);
                if constexpr (STAGES == 1) wait_lds_then_barrier();
            }
            if (full < tiles) {
                // no copy is in flight; the barrier keeps this slot's new
                // contents from landing while a wave still reads its old ones
                Staged r;
                load(r, g, m0, n0, full * BK, true, true);
                wait_lds_then_barrier();
                store(smem + (full % STAGES) * SLOT, r);
                wait_lds_then_barrier();
                compute(smem + (full % STAGES) * SLOT, c, wm, wn, lr, lc);
            }
        } else if constexpr (STAGES == 1) {
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
