// Thin-N GEMM (N <= THIN_N_MAX) for bf16 and int8: C = A x B when B has only
// a few columns - a matrix-vector product in all but name, and the narrow
// remainder of a split plan (the last N mod BN columns of a shape whose
// last tile column would otherwise add a nearly empty round of workgroups).
//
// A tiled kernel is the wrong shape here: a grid of M / 64 workgroups, each
// running the whole K loop alone on its compute unit, waits on one slice's
// loads at a time.  This kernel streams A once.  A workgroup owns BM rows of
// C (ROWS per wave) and walks K in chunks of KC = V x 512: the chunk is V
// sub-chunks of 512, and in each every lane takes 8 consecutive k, one
// 16-byte (bf16) or 8-byte (int8) load per row where the row is aligned,
// element loads otherwise.  The chunk's KC x NB block of B is loaded once per
// workgroup (element loads from clamped, valid addresses, zero past K and N)
// and shared through LDS.  The loads of chunk c+1 (A into registers, B into
// registers then LDS) are issued before chunk c is multiplied - the
// register-staged double buffer of the GEMM page, section 9 - and one
// barrier per chunk orders the LDS slots.  With so little arithmetic per
// byte each chunk costs about one memory round trip, so the V sub-chunks
// keep V times the bytes in flight and take K / KC round trips instead of
// K / 512.  The lanes' partial sums are added across the wave at the end.
//
// Products of two bf16 values are exact in fp32 and are summed in fp32;
// int8 products are summed exactly in int32.  The order of the fp32 sum
// differs from a single chain over k (per lane, then across lanes).
#pragma once

#include <type_traits>

#include "tg_device.hpp"

namespace tg {

template <int DT, int NB>  // DT 1: bf16 -> fp32, 2: int8 -> int32; NB: columns computed (>= N)
struct ThinGemm {
    static_assert(NB >= 1 && NB <= THIN_N_MAX && (NB & (NB - 1)) == 0, "NB: a power of two up to 16");
    typedef typename std::conditional<DT == 1, uint16_t, int8_t>::type T;
    typedef typename std::conditional<DT == 1, float, int32_t>::type Acc;
    static constexpr int NT = 256;
    static constexpr int ROWS = NB >= 16 ? 2 : 4;  // rows of C per wave (fewer for 16 columns: registers)
    static constexpr int BM = ROWS * (NT / 64);  // rows per workgroup
    static constexpr int BN = NB;
    static constexpr int ESZ = sizeof(T);
    static constexpr int KE = 8;                 // consecutive k per lane per sub-chunk
    static constexpr int V = NB <= 2 ? 4 : NB <= 8 ? 2 : 1;  // sub-chunks per chunk (registers)
    static constexpr int KS = 64 * KE;           // k per sub-chunk
    static constexpr int KC = V * KS;            // k per chunk
    // LDS: the chunk's B rows, NB elements each, as V x 64 runs of KE rows
    // (run r = sub-chunk r / 64, lane r % 64); every run is followed by 16
    // bytes of padding so that lanes reading their own rows at the same
    // offset fall on different banks
    static constexpr int LANE_ELEMS = KE * NB + 16 / ESZ;
    static constexpr int SLOT_ELEMS = V * 64 * LANE_ELEMS;
    static constexpr int BPT = KC * NB / NT;  // B elements each thread stages per chunk
    // with B rows in whole aligned 16-byte pieces: pieces per row, per thread
    static constexpr int BV = NB * ESZ >= 16 ? NB * ESZ / 16 : 0;
    static constexpr int BVPT = BV ? KC * BV / NT : 1;
    static constexpr int LDS_BYTES = 2 * SLOT_ELEMS * ESZ;
    typedef typename std::conditional<DT == 1, i32x4, i32x2>::type AVec;

    __device__ static __forceinline__ Acc widen(T v) {
        if constexpr (DT == 1) return __uint_as_float((uint32_t)v << 16);
        else return (int32_t)v;
    }

    // element e (a constant in the unrolled loops) of a lane's A piece
    __device__ static __forceinline__ Acc elem(const AVec& v, int e) {
        const uint32_t w = (uint32_t)v[e / (4 / ESZ)];
        if constexpr (DT == 1) return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
        else return (int32_t)(w << (24 - 8 * (e & 3))) >> 24;
    }

    __device__ static __forceinline__ Acc wave_sum(Acc v) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        return v;
    }

    // This lane's 8 elements of each of its rows at kv (zero past K): one
    // sub-chunk.
    __device__ static __forceinline__ void load_a(AVec (&av)[ROWS], const T* const (&rowp)[ROWS], int kv, int K,
                                                  bool a_wide) {
        if (a_wide && kv + KE <= K) {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) av[i] = *reinterpret_cast<const AVec*>(rowp[i] + kv);
        } else {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                union { AVec v; T e[KE]; } u;
#pragma unroll
                for (int e = 0; e < KE; ++e) {
                    const T x = rowp[i][min(kv + e, K - 1)];  // always a valid address
                    u.e[e] = kv + e < K ? x : T(0);
                }
                av[i] = u.v;
            }
        }
    }

    // This thread's share of the chunk's B block: element q*NT + tid is row
    // (q*NT + tid) / NB, column (q*NT + tid) % NB of the chunk.
    __device__ static __forceinline__ void load_b(T (&bv)[BPT], const GemmArgs& g, int kc0) {
        const T* B = static_cast<const T*>(g.B);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int k = kc0 + idx / NB, j = idx % NB;
            const T x = B[(int64_t)min(k, g.K - 1) * g.ldb + min(j, g.N - 1)];
            bv[q] = (k < g.K && j < g.N) ? x : T(0);
        }
    }

    // The same block in 16-byte pieces (B rows aligned, N a whole number of
    // pieces: N == NB); piece q*NT + tid is row (q*NT + tid) / BV.
    __device__ static __forceinline__ void load_b_vec(i32x4 (&bw)[BVPT], const GemmArgs& g, int kc0) {
        if constexpr (BV > 0) {
            const T* B = static_cast<const T*>(g.B);
#pragma unroll
            for (int q = 0; q < BVPT; ++q) {
                const int idx = q * NT + threadIdx.x;
                const int k = kc0 + idx / BV, p = idx % BV;
                const i32x4 x =
                    *reinterpret_cast<const i32x4*>(B + (int64_t)min(k, g.K - 1) * g.ldb + p * (16 / ESZ));
                bw[q] = k < g.K ? x : i32x4{0, 0, 0, 0};
            }
        }
    }

    __device__ static __forceinline__ void store_b_vec(TG_LDS T* slot, const i32x4 (&bw)[BVPT]) {
        if constexpr (BV > 0) {
#pragma unroll
            for (int q = 0; q < BVPT; ++q) {
                const int idx = q * NT + threadIdx.x;
                const int kk = idx / BV, p = idx % BV;
                *reinterpret_cast<TG_LDS i32x4*>(slot + (kk / KE) * LANE_ELEMS + (kk % KE) * NB + p * (16 / ESZ)) =
                    bw[q];
            }
        }
    }

    __device__ static __forceinline__ void store_b(TG_LDS T* slot, const T (&bv)[BPT]) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int kk = idx / NB, j = idx % NB;
            slot[(kk / KE) * LANE_ELEMS + (kk % KE) * NB + j] = bv[q];
        }
    }

    // Sub-chunk v of the chunk in `slot` times this lane's A elements of it.
    __device__ static __forceinline__ void multiply(Acc (&acc)[ROWS][NB], const AVec (&av)[ROWS],
                                                    const TG_LDS T* slot, int v, int lane) {
        const TG_LDS T* mine = slot + (v * 64 + lane) * LANE_ELEMS;
#pragma unroll
        for (int e = 0; e < KE; ++e) {
            Acc b[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) b[j] = widen(mine[e * NB + j]);
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const Acc a = elem(av[i], e);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if constexpr (DT == 1) acc[i][j] = __builtin_fmaf(a, b[j], acc[i][j]);
                    else acc[i][j] += a * b[j];
                }
            }
        }
    }

    __device__ static __forceinline__ void run(const GemmArgs& g) {
        __shared__ __attribute__((aligned(16))) T lds[2 * SLOT_ELEMS];
        TG_LDS T* slots = (TG_LDS T*)(lds);
        // B in 16-byte pieces when its rows allow it (b_guard == 0 means
        // aligned rows and pointer, and N a whole number of pieces); A in
        // 16-byte (int8: 8-byte) pieces when its rows are aligned
        const bool a_wide = g.a_guard == 0;
        if constexpr (BV > 0) {
            if (g.b_guard == 0) {
                if (a_wide) run_k<true, true>(g, slots);
                else run_k<true, false>(g, slots);
                return;
            }
        }
        if (a_wide) run_k<false, true>(g, slots);
        else run_k<false, false>(g, slots);
    }

    // The chunk's B block (zero past K and N) into `slot`.
    template <bool BVEC>
    __device__ static __forceinline__ void load_b_any(typename std::conditional<BVEC, i32x4[BVPT], T[BPT]>::type& r,
                                                      const GemmArgs& g, int kc0) {
        if constexpr (BVEC) load_b_vec(r, g, kc0);
        else load_b(r, g, kc0);
    }
    template <bool BVEC>
    __device__ static __forceinline__ void store_b_any(
        TG_LDS T* slot, const typename std::conditional<BVEC, i32x4[BVPT], T[BPT]>::type& r) {
        if constexpr (BVEC) store_b_vec(slot, r);
        else store_b(slot, r);
    }

    // WIDE: A rows are 16-byte (int8: 8-byte) aligned.  The whole chunks then
    // take one wide load per row and sub-chunk, all V sub-chunks of chunk c+1
    // in flight while chunk c is multiplied (each sub-chunk's registers are
    // refilled as soon as they are used); the partial last chunk, and every
    // chunk of unaligned rows, take element loads one sub-chunk at a time.
    template <bool BVEC, bool WIDE>
    __device__ static __forceinline__ void run_k(const GemmArgs& g, TG_LDS T* slots) {
        typedef typename std::conditional<BVEC, i32x4[BVPT], T[BPT]>::type BRegs;
        const T* A = static_cast<const T*>(g.A);
        const int lane = lane_id(), wave = wave_id();
        const int r0 = blockIdx.x * BM + wave * ROWS;
        const T* rowp[ROWS];
#pragma unroll
        for (int i = 0; i < ROWS; ++i) rowp[i] = A + (int64_t)min(r0 + i, g.M - 1) * g.lda;
        Acc acc[ROWS][NB];
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = Acc(0);

        const int chunks = (g.K + KC - 1) / KC;
        const int full = WIDE ? g.K / KC : 0;  // chunks on the wide path
        {
            BRegs b;
            load_b_any<BVEC>(b, g, 0);
            store_b_any<BVEC>(slots, b);
            wait_lds_then_barrier();
        }
        int c = 0;
        if (WIDE && full > 0) {
            AVec av[V][ROWS];
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int i = 0; i < ROWS; ++i)
                    av[v][i] = *reinterpret_cast<const AVec*>(rowp[i] + v * KS + lane * KE);
            for (; c < full; ++c) {
                const bool more_b = c + 1 < chunks, more_a = c + 1 < full;
                const TG_LDS T* cur = slots + (c & 1) * SLOT_ELEMS;
                const int k_next = (c + 1) * KC + lane * KE;
                BRegs b;
                if (more_b) load_b_any<BVEC>(b, g, (c + 1) * KC);
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    multiply(acc, av[v], cur, v, lane);
                    if (more_a) {
#pragma unroll
                        for (int i = 0; i < ROWS; ++i)
                            av[v][i] = *reinterpret_cast<const AVec*>(rowp[i] + k_next + v * KS);
                    }
                }
                if (more_b) store_b_any<BVEC>(slots + ((c + 1) & 1) * SLOT_ELEMS, b);
                wait_lds_then_barrier();
            }
        }
        for (; c < chunks; ++c) {
            const bool more_b = c + 1 < chunks;
            const TG_LDS T* cur = slots + (c & 1) * SLOT_ELEMS;
            BRegs b;
            if (more_b) load_b_any<BVEC>(b, g, (c + 1) * KC);
            // sub-chunks that start at or past K hold only zeros: skipped
            const int vs = min(V, (g.K - c * KC + KS - 1) / KS);
#pragma nounroll
            for (int v = 0; v < vs; ++v) {
                AVec t[ROWS];
                load_a(t, rowp, c * KC + v * KS + lane * KE, g.K, WIDE);
                multiply(acc, t, cur, v, lane);
            }
            if (more_b) store_b_any<BVEC>(slots + ((c + 1) & 1) * SLOT_ELEMS, b);
            wait_lds_then_barrier();
        }

        Acc* C = static_cast<Acc*>(g.C);
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const Acc s = wave_sum(acc[i][j]);
                if (lane == 0 && r0 + i < g.M && j < g.N) C[(int64_t)(r0 + i) * g.ldc + j] = s;
            }
    }
};

}  // namespace tg
