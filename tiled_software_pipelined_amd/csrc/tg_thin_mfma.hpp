// Thin-N GEMM on the matrix cores (bf16 2 <= N <= 16, int8 2 <= N <= 16):
// C = A x B with B of a few columns, as 16 x 16 output blocks of
// v_mfma_f32_16x16x32_bf16 / v_mfma_i32_16x16x64_i8 whose columns past N are
// computed and dropped.
//
// The vector-ALU thin kernel (tg_thin.hpp) gives each lane a piece of one
// row of A and reads N pieces of B from LDS per piece of A; from a few
// columns on, those reads and the dot products bound it.  Here a wave owns
// 16 rows of A (RB blocks of 16 per workgroup) and one matrix instruction
// multiplies 64 bytes of each of them by a 64-byte deep, 16-column slice of
// B: one 16-byte read of A per lane and two transposing LDS reads of B per
// instruction, whatever N is.  The 16 waves of a workgroup split K: in chunk
// c, wave w takes the P consecutive matrix steps starting at step
// (c x 16 + w) x P, so its loads of a row are 64 x P contiguous bytes.  A
// goes from memory straight into registers (16 bytes per lane at any
// alignment; element loads with zero fill only where a piece would cross
// K), P x RB pieces per lane in flight, refilled with the next chunk's as
// soon as each is multiplied: the register-staged double buffer of the GEMM
// page, section 9.  B's chunk (KC rows of NB columns, the layout the
// transposing read takes: row-major, NB x esize bytes a row) is loaded by
// the whole workgroup as 8- or 16-byte pieces of each row at any alignment
// and written to one of two LDS slots; one barrier per chunk.  Columns N..NB-1
// of a row then hold the next row's first values, which reach only columns
// of C that are not stored; B's last row, whose pieces could run past the
// matrix, is loaded by element once, up front, and rows past K are zero.
// At the end the 16 waves' partial blocks are added in LDS in a fixed order.
//
// bf16 products are exact in fp32 and summed in fp32 (inside the matrix
// instruction, then across the 16 waves); int8 sums are exact in int32.
#pragma once

#include <type_traits>

#include "tg_device.hpp"

namespace tg {

// DT 1: bf16 -> fp32, 2: int8 -> int32.  NB: columns of B kept per row
// (>= N; 4, 8 or 16 bf16, 8 or 16 int8: 8 to 32 bytes); RB: 16-row blocks
// per workgroup; P: matrix steps per wave per chunk.
template <int DT, int NB, int RB, int P>
struct ThinMfma {
    typedef typename std::conditional<DT == 1, uint16_t, int8_t>::type T;
    typedef typename std::conditional<DT == 1, float, int32_t>::type Acc;
    typedef typename std::conditional<DT == 1, f32x4, i32x4>::type Acc4;
    static constexpr int ESZ = sizeof(T);
    static constexpr int NT = 1024;
    static constexpr int NW = NT / 64;
    static constexpr int WAVES = 4;            // waves per SIMD (one workgroup per compute unit)
    static constexpr int BM = 16 * RB;
    static constexpr int BN = NB;
    static constexpr int KSTEP = 64 / ESZ;     // k per matrix instruction (64 bytes of a row)
    static constexpr int KL = KSTEP / 4;       // k per lane per instruction (16 bytes)
    static constexpr int KC = NW * P * KSTEP;  // k per chunk
    static constexpr int ROWB = NB * ESZ;      // bytes of one B row in LDS
    static_assert(ROWB == 8 || ROWB == 16 || ROWB == 32, "B rows of 8, 16 or 32 bytes");
    static constexpr int PIECE = ROWB < 16 ? ROWB : 16;  // bytes per load of a B row
    static constexpr int PPR = ROWB / PIECE;             // pieces per row
    static constexpr int BPT = (KC * PPR + NT - 1) / NT;  // pieces each thread stages per chunk
    static constexpr int SLOT_BYTES = KC * ROWB;
    static constexpr int ZERO_OFF = 2 * SLOT_BYTES;      // 16 zero bytes for reads of columns past NB
    static constexpr int RED_BYTES = NW * RB * 256 * 4;  // the waves' partial blocks, at the end
    static constexpr int LDS_BYTES = 2 * SLOT_BYTES + 16 > RED_BYTES ? 2 * SLOT_BYTES + 16 : RED_BYTES;
    typedef typename std::conditional<PIECE == 16, i32x4, i32x2>::type BPiece;

    __device__ static __forceinline__ Acc4 mma(const i32x4& a, const i32x4& b, const Acc4& c) {
        if constexpr (DT == 1)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }

    // This lane's 16 bytes of each of its rows from k (zero past K).
    __device__ static __forceinline__ void load_a(i32x4 (&a)[RB], const T* const (&rowp)[RB], int k, int K) {
        // (k is the lane's own first element: the step's first plus KL (l/16))
        if (k + KL <= K) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) a[rb] = load16(rowp[rb] + k);
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                union { i32x4 v; T e[KL]; } u;
#pragma unroll
                for (int e = 0; e < KL; ++e) u.e[e] = load_or_zero(rowp[rb] + k + e, k + e < K);
                __builtin_amdgcn_sched_barrier(0);  // one piece's addresses live at a time
                a[rb] = u.v;
            }
        }
    }

    template <int TOTAL>
    __device__ static __forceinline__ bool in_block(int q, int idx) {
        return (q + 1) * NT <= TOTAL || idx < TOTAL;
    }

    // This thread's pieces of the chunk of B from row kc0: piece q*NT + tid
    // is row (q*NT + tid) / PPR.  Rows from K - 1 on are left zero here.
    __device__ static __forceinline__ void load_b(BPiece (&bp)[BPT], const GemmArgs& g, int kc0) {
        const char* B = static_cast<const char*>(g.B);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int k = kc0 + idx / PPR, pp = idx % PPR;
            bp[q] = load_or_zero(reinterpret_cast<const BPiece*>(B + (int64_t)k * g.ldb * ESZ + pp * PIECE),
                                 in_block<KC * PPR>(q, idx) && k < g.K - 1);
            if ((q & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
    }

    struct LastRow {
        BPiece v[PPR];
    };
    // B's last row, columns 0..NB-1, zero past N (element loads, once)
    __device__ static __forceinline__ LastRow load_last_row(const GemmArgs& g) {
        const T* B = static_cast<const T*>(g.B);
        union { LastRow r; T e[NB]; } u;
#pragma unroll
        for (int j = 0; j < NB; ++j) u.e[j] = load_or_zero(B + (int64_t)(g.K - 1) * g.ldb + j, j < g.N && g.K > 0);
        return u.r;
    }

    // kk_last: the chunk row that is B's last row (its pieces from `last`)
    __device__ static __forceinline__ void store_b(TG_LDS char* slot, const BPiece (&bp)[BPT], const LastRow& last,
                                                   int kk_last) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = q * NT + threadIdx.x;
            const int kk = idx / PPR, pp = idx % PPR;
            if (in_block<KC * PPR>(q, idx)) {
                // (selects, not an index: a private array indexed by a lane
                // value would be moved to LDS)
                BPiece lv = last.v[0];
#pragma unroll
                for (int t = 1; t < PPR; ++t)
                    if (pp == t) lv = last.v[t];
                *reinterpret_cast<TG_LDS BPiece*>(slot + kk * ROWB + pp * PIECE) = kk == kk_last ? lv : bp[q];
            }
        }
    }

    // The B operand of the matrix step whose first row in the slot is k0:
    // lane l holds column l%16 of the step's rows KL (l/16) .. +KL, as two
    // transposing reads of half that run each (in each 16-lane group, input
    // lane j points at 8 bytes of one row, output lane i receives column i
    // of the rows read).  Lanes whose 8 bytes lie past the row's NB columns
    // read the zero bytes.
    __device__ static __forceinline__ i32x4 read_b(const TG_LDS char* slot, const TG_LDS char* zero, int k0,
                                                   int lane) {
        const int grp = lane >> 4, j = lane & 15;
        i32x2 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if constexpr (ESZ == 2) {
                const int row = k0 + 8 * grp + 4 * hh + (j >> 2);
                const int cb = 8 * (j & 3);
                const TG_LDS char* p = cb < ROWB ? slot + row * ROWB + cb : zero;
                h[hh] = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS i16x4*)(p)));
            } else {
                const int row = k0 + 16 * grp + 8 * hh + (j >> 1);
                const int cb = 8 * (j & 1);
                const TG_LDS char* p = cb < ROWB ? slot + row * ROWB + cb : zero;
                h[hh] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((TG_LDS i32x2*)(p));
            }
        }
        return i32x4{h[0].x, h[0].y, h[1].x, h[1].y};
    }

    __device__ static __forceinline__ void run(const GemmArgs& g) {
        __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
        TG_LDS char* L = (TG_LDS char*)(lds);
        const int lane = lane_id(), wave = wave_id();
        const int m0 = blockIdx.x * BM;
        const T* A = static_cast<const T*>(g.A);
        // lane l reads row l%16 of each block, 16 bytes at KL (l/16) into a step
        const T* rowp[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) rowp[rb] = A + (int64_t)min(m0 + rb * 16 + (lane & 15), g.M - 1) * g.lda;
        const int kl = (lane >> 4) * KL;
        Acc4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = Acc4{0, 0, 0, 0};

        const int ksteps = (g.K + KSTEP - 1) / KSTEP;
        const int chunks = (g.K + KC - 1) / KC;
        i32x4 av[P][RB];
        const LastRow last = load_last_row(g);
        if (threadIdx.x == 0) *reinterpret_cast<TG_LDS i32x4*>(L + ZERO_OFF) = i32x4{0, 0, 0, 0};
        {
            BPiece bp[BPT];
            load_b(bp, g, 0);
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (wave * P + p < ksteps) load_a(av[p], rowp, (wave * P + p) * KSTEP + kl, g.K);
            store_b(L, bp, last, g.K - 1);
            wait_lds_then_barrier();
        }
        for (int c = 0; c < chunks; ++c) {
            const bool more = c + 1 < chunks;
            const TG_LDS char* cur = L + (c & 1) * SLOT_BYTES;
            BPiece bp[BPT];
            if (more) load_b(bp, g, (c + 1) * KC);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int s = (c * NW + wave) * P + p;  // matrix step (of the whole K)
                if (s < ksteps) {
                    const i32x4 b = read_b(cur, L + ZERO_OFF, (wave * P + p) * KSTEP, lane);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) acc[rb] = mma(av[p][rb], b, acc[rb]);
                }
                if (more && s + NW * P < ksteps) load_a(av[p], rowp, (s + NW * P) * KSTEP + kl, g.K);
            }
            if (more) store_b(L + ((c + 1) & 1) * SLOT_BYTES, bp, last, g.K - 1 - (c + 1) * KC);
            wait_lds_then_barrier();
        }

        // lane l holds rows 4 (l/16) .. +4, column l%16 of each block; the
        // last barrier above ended every read of B, so its slots take the
        // partial blocks
        TG_LDS Acc* red = reinterpret_cast<TG_LDS Acc*>(L);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                red[((wave * RB + rb) * 16 + 4 * (lane >> 4) + t) * 16 + (lane & 15)] = acc[rb][t];
        wait_lds_then_barrier();
        Acc* C = static_cast<Acc*>(g.C);
        for (int e = threadIdx.x; e < RB * 256; e += NT) {
            const int rb = e >> 8, r = (e >> 4) & 15, col = e & 15;
            Acc sum = Acc(0);
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[((w * RB + rb) * 16 + r) * 16 + col];
            const int row = m0 + rb * 16 + r;
            if (row < g.M && col < g.N) C[(int64_t)row * g.ldc + col] = sum;
        }
    }
};

}  // namespace tg
