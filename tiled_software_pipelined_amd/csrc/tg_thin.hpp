// Thin-N GEMM on the vector ALUs for bf16 and int8: C = A x B when B has one
// column (or, int8, up to 4 whose rows are too short for the matrix-core
// thin kernel's 8-byte pieces) - a matrix-vector product in all but name,
// and the narrow remainder of a split plan (the last N mod BN columns of a
// shape whose last tile column would otherwise add a nearly empty round of
// workgroups).  Wider B goes to tg_thin_mfma.hpp.
//
// A tiled kernel is the wrong shape here: a grid of M / 64 workgroups, each
// running the whole K loop alone on its compute unit, waits on one slice's
// loads at a time.  This kernel streams A once.  A workgroup owns BM rows of
// C (ROWS per wave) and walks K in chunks of KC = V x 512: the chunk is V
// sub-chunks of 512, and in each every lane takes 8 consecutive k, one
// 16-byte (bf16) or 8-byte (int8) load per row at any alignment (element
// loads only where the 8 would cross K).  The chunk's KC x NB block of B is
// loaded once per workgroup, element by element from valid addresses (zero
// past K and N), and shared through LDS.  The loads of chunk c+1 (A into registers, B into
// registers then LDS) are issued before chunk c is multiplied - the
// register-staged double buffer of the GEMM page, section 9 - and one
// barrier per chunk orders the LDS slots.  With so little arithmetic per
// byte each chunk costs about one memory round trip, so the V sub-chunks
// keep V times the bytes in flight and take K / KC round trips instead of
// K / 512.  The lanes' partial sums are added across the wave at the end.
//
// Products of two bf16 values are exact in fp32 and are summed in fp32, two
// at a time (v_dot2c_f32_bf16); int8 products four at a time, exactly, in
// int32 (v_dot4c_i32_i8).  The order of the fp32 sum differs from a single
// chain over k (per lane in pairs, then across lanes).
#pragma once

#include <type_traits>

#include "tg_device.hpp"

namespace tg {

// DT 1: bf16 -> fp32, 2: int8 -> int32; NB: columns computed (>= N); ROWS_ /
// V_: rows of C per wave and sub-chunks per chunk (0: by NB); NT_: threads
// per workgroup
template <int DT, int NB, int ROWS_ = 0, int V_ = 0, int NT_ = 1024>
struct ThinGemm {
    static_assert(NB >= 1 && NB <= THIN_N_MAX && (NB & (NB - 1)) == 0, "NB: a power of two up to 16");
    typedef typename std::conditional<DT == 1, uint16_t, int8_t>::type T;
    static_assert(NB * sizeof(T) < 16, "B rows of whole 16-byte pieces: the matrix-core thin kernel");
    typedef typename std::conditional<DT == 1, float, int32_t>::type Acc;
    static constexpr int NT = NT_;
    static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
    // One row of C per wave, 16 waves per workgroup (one workgroup per CU at
    // 4 waves per SIMD): the chunk's B block is staged by 1024 threads, so
    // each holds few of its elements and 9 sub-chunks (K up to 4608 in one
    // memory round trip) fit the registers up to 4 columns (4095 x N x 4104
    // bf16, compact B: N = 2 8.8 us, 3 11.5, 8 15.3, 16 24.1 against 12.7,
    // 16.7, 21.2, 35.4 with 256 threads and 1-4 rows per wave; a strided
    // column, the remainder of a split plan: N = 1 11.4 against 21.8)
    static constexpr int ROWS = ROWS_ ? ROWS_ : 1;
    // waves per SIMD the kernel is compiled for
    static constexpr int WAVES = 4;
    static constexpr int BM = ROWS * (NT / 64);  // rows per workgroup
    static constexpr int BN = NB;
    static constexpr int ESZ = sizeof(T);
    static constexpr int KE = 8;                 // consecutive k per lane per sub-chunk
    // sub-chunks per chunk (registers: V x ROWS pieces of A per lane; 9 of 512
    // cover K up to 4608 in one chunk).  With more rows per wave (for M
    // large enough to keep ~256 workgroups) the registers hold fewer: 2
    // rows 4, 4 rows 2 (16384 x 3 x 4104 bf16 36.1 -> 31.4 us with 4 rows,
    // 8192 rows 19.3 -> 17.3 with 2)
    static constexpr int V = V_ ? V_ : ROWS == 1 ? 9 : ROWS == 2 ? 4 : 2;
    static constexpr int KS = 64 * KE;           // k per sub-chunk
    static constexpr int KC = V * KS;            // k per chunk
    // LDS: the chunk's B block as V x 64 runs of KE rows (run r = sub-chunk
    // r / 64, lane r % 64), each run column by column (the KE values of
    // column j at j KE), so that a lane reads a column as one 16-byte (int8:
    // 8-byte) piece whose dwords pair (quad) consecutive k like its piece of
    // A; runs are padded to an odd number of 16-byte pieces, so that the 16
    // lanes of one read fall on distinct banks
    static constexpr int RUN_PIECES = (KE * NB * ESZ + 15) / 16;
    static constexpr int LANE_ELEMS = (RUN_PIECES | 1) * 16 / ESZ;
    static constexpr int SLOT_ELEMS = V * 64 * LANE_ELEMS;
    static constexpr int BPT = (KC * NB + NT - 1) / NT;  // B elements each thread stages per chunk
    static constexpr int LDS_BYTES = 2 * SLOT_ELEMS * ESZ;
    typedef typename std::conditional<DT == 1, i32x4, i32x2>::type AVec;

    __device__ static __forceinline__ Acc wave_sum(Acc v) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        return v;
    }

    // This lane's 8 elements of each of its rows at kv (zero past K): one
    // sub-chunk.
    __device__ static __forceinline__ void load_a(AVec (&av)[ROWS], const T* const (&rowp)[ROWS], int kv, int K) {
        if (kv + KE <= K) {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) __builtin_memcpy(&av[i], rowp[i] + kv, sizeof(AVec));
        } else {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                union { AVec v; T e[KE]; } u;
#pragma unroll
                for (int e = 0; e < KE; ++e) u.e[e] = load_or_zero(rowp[i] + kv + e, kv + e < K);
                __builtin_amdgcn_sched_barrier(0);  // one piece's addresses live at a time
                av[i] = u.v;
            }
        }
    }

    // Is element / piece q*NT + tid of a chunk's B block one of its `total`?
    // (Every thread's is, but for the last round when NT does not divide it.)
    template <int TOTAL>
    __device__ static __forceinline__ bool in_block(int q, int idx) {
        return (q + 1) * NT <= TOTAL || idx < TOTAL;
    }

    // This thread's share of the chunk's B block: element q*NT + tid is row
    // (q*NT + tid) / NB, column (q*NT + tid) % NB of the chunk.
    __device__ static __forceinline__ void load_b(T (&bv)[BPT], const GemmArgs& g, int kc0) {
        const T* B = static_cast<const T*>(g.B);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int k = kc0 + idx / NB, j = idx % NB;
            bv[q] = load_or_zero(B + (int64_t)k * g.ldb + j, in_block<KC * NB>(q, idx) && k < g.K && j < g.N);
            // at most 8 of these 64-bit addresses live at a time; the loads
            // of all groups still overlap
            if ((q & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
    }

    __device__ static __forceinline__ void store_b(TG_LDS T* slot, const T (&bv)[BPT]) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int kk = idx / NB, j = idx % NB;
            if (in_block<KC * NB>(q, idx)) slot[(kk / KE) * LANE_ELEMS + j * KE + kk % KE] = bv[q];
        }
    }

    // Sub-chunk v of the chunk in `slot` times this lane's A elements of it:
    // per column one read of its KE values and KE/2 dot products of two bf16
    // pairs (int8: KE/4 of four-byte quads, exact) with the lane's piece of
    // each row of A.
    __device__ static __forceinline__ void multiply(Acc (&acc)[ROWS][NB], const AVec (&av)[ROWS],
                                                    const TG_LDS T* slot, int v, int lane) {
        const TG_LDS T* mine = slot + (v * 64 + lane) * LANE_ELEMS;
        constexpr int WORDS = (int)(sizeof(AVec) / 4);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const AVec b = *reinterpret_cast<const TG_LDS AVec*>(mine + j * KE);
#pragma unroll
            for (int i = 0; i < ROWS; ++i)
#pragma unroll
                for (int q = 0; q < WORDS; ++q) {
                    if constexpr (DT == 1)
                        acc[i][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)av[i][q]),
                                                                    __builtin_bit_cast(bf16x2, (uint32_t)b[q]),
                                                                    acc[i][j], false);
                    else
                        acc[i][j] = __builtin_amdgcn_sdot4(av[i][q], b[q], acc[i][j], false);
                }
        }
    }

    __device__ static __forceinline__ void run(const GemmArgs& g) { run_block(g, blockIdx.x); }

    // The rows of C of workgroup `block` (rows block * BM ..).  A lane's 8
    // elements of a row that lie inside K take one wide load (element loads
    // with zero fill otherwise).  Before the first wait, the chunk-0 loads of
    // B and then of every sub-chunk of A are all in flight; B is staged into
    // LDS (waiting only for its own loads, issued first), and each
    // sub-chunk's A registers are refilled with the next chunk's as soon as
    // they have been multiplied, while that chunk's B is staged into the
    // other slot: the register-staged double buffer of the GEMM page,
    // section 9, one barrier per chunk.  Sub-chunks that start at or past K
    // hold only zeros and are not multiplied.
    __device__ static __forceinline__ void run_block(const GemmArgs& g, int block) {
        __shared__ __attribute__((aligned(16))) T lds[2 * SLOT_ELEMS];
        TG_LDS T* slots = (TG_LDS T*)(lds);
        const T* A = static_cast<const T*>(g.A);
        const int lane = lane_id(), wave = wave_id();
        const int r0 = block * BM + wave * ROWS;
        const T* rowp[ROWS];
#pragma unroll
        for (int i = 0; i < ROWS; ++i) rowp[i] = A + (int64_t)min(r0 + i, g.M - 1) * g.lda;
        Acc acc[ROWS][NB];
#pragma unroll
        for (int i = 0; i < ROWS; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = Acc(0);

        const int chunks = (g.K + KC - 1) / KC;
        AVec av[V][ROWS];
        {
            T b[BPT];
            load_b(b, g, 0);
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (v * KS < g.K) load_a(av[v], rowp, v * KS + lane * KE, g.K);
            store_b(slots, b);
            wait_lds_then_barrier();
        }
        for (int c = 0; c < chunks; ++c) {
            const bool more = c + 1 < chunks;
            const TG_LDS T* cur = slots + (c & 1) * SLOT_ELEMS;
            T b[BPT];
            if (more) load_b(b, g, (c + 1) * KC);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (c * KC + v * KS < g.K) multiply(acc, av[v], cur, v, lane);
                if (more && (c + 1) * KC + v * KS < g.K)
                    load_a(av[v], rowp, (c + 1) * KC + v * KS + lane * KE, g.K);
            }
            if (more) store_b(slots + ((c + 1) & 1) * SLOT_ELEMS, b);
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
