// Matrix-core (MFMA) GEMM kernel family for gfx950: bf16 x bf16 -> fp32 and
// int8 x int8 -> int32.
//
// One workgroup computes one BM x BN tile of C.  Its waves form a
// WAVES_M x WAVES_N grid; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) block
// made of 32 x 32 matrix-core tiles ("4.1 CUDA GEMM算子性能优化", sections 4-6:
// block, warp and thread tiling, with the wave as the unit on this GPU).  The
// K loop walks BK-wide slices of A and B through a ring of STAGES LDS slots
// (same page, sections 9-10; the "流水化 GPU 内核" skill, Step 3: prologue,
// steady loop, epilogue):
//
//   prologue : start the loads of slices 0 .. STAGES-2; wait for slice 0
//   slice t  : multiply slice t out of LDS, one matrix-core K step at a time,
//              reading the fragments of the next K step ahead; inside the
//              last K step wait for slice t+1, barrier, start slice
//              t+STAGES into the slot slice t just left and read slice
//              t+1's first fragments
//
// so that the global->LDS copy of later slices overlaps the matrix-core work
// on slice t.  Tiles whose waves issue only one or two matrix instructions
// per K step read a whole slice's fragments one slice ahead instead
// (FR_SLICE, slice_ahead), with the slice's barrier in its first K step.
// Two loaders are built (the skill's Step 2 choice):
//   LD_VGPR   : 16-byte loads into registers, written to LDS after the
//               multiply of the current slice (register-staged double buffer,
//               GEMM page section 9.5);
//   LD_DIRECT : global_load_lds_dwordx4, which writes LDS without passing
//               through registers (the asynchronous copy of section 10).
//
// Operand fragments come from LDS with 16-byte reads (A, K-contiguous) and
// the gfx950 transposing reads ds_read_b64_tr_b16 / _tr_b8 (B, which is
// N-contiguous in memory but must be K-contiguous in each lane).  With
// LY_XOR the 16-byte chunks of every LDS row are permuted by an XOR of the
// row index so that the lanes of one read hit distinct banks (section 8.5).
//
// Edges: rows of A past M and columns of B past N are loaded from a clamped,
// valid address (they only feed C elements that are never stored); the last,
// partial K slice is loaded element by element with zero fill (the skill's
// pitfall list: boundary tiles need a guarded fallback).  The direct loader
// reads rows of any alignment (its copies take any byte address) and a B
// whose N is not a whole number of chunks (see direct_offsets); the
// register-staged loader reads unaligned rows in its SHIFT twins, each chunk
// funnel-shifted out of two aligned 16-byte loads.
#pragma once

#include "tg_device.hpp"

namespace tg {

struct TraitsBF16 {
    typedef uint16_t T;
    typedef float Out;
    typedef f32x4 Out4;
    typedef f32x16 Acc;
    static constexpr int ESZ = 2;
    static constexpr int MK = 16;  // K of one v_mfma_f32_32x32x16_bf16
    __device__ static __forceinline__ Acc mma(i32x4 a, i32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct TraitsI8 {
    typedef int8_t T;
    typedef int32_t Out;
    typedef i32x4 Out4;
    typedef i32x16 Acc;
    static constexpr int ESZ = 1;
    static constexpr int MK = 32;  // K of one v_mfma_i32_32x32x32_i8
    __device__ static __forceinline__ Acc mma(i32x4 a, i32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

// CST selects the C write-back: CST_MFMA stores from the matrix
// instruction's own output layout (4-byte stores, each instruction writing
// two 128-byte row segments); CST_SWAP computes C^T = B^T A^T instead (the
// operands of every matrix instruction swapped, same products in the same k
// order), which puts four consecutive columns of one C row in each lane, so
// that the write-back takes a quarter of the store instructions, 16 bytes
// each.
enum CStore { CST_MFMA = 0, CST_SWAP = 1 };

// How the operand fragments come out of LDS (the LDS -> register ladder of
// the SM80 ablation plan, section 1.1, on this GPU's instructions): the A
// fragment (16 bytes of one row per lane) as four 4-byte, two 8-byte or one
// 16-byte read; the B fragment (one column, K-contiguous per lane, from the
// N-contiguous LDS rows) as one element read per K value, or as two
// transposing ds_read_b64_tr_b16 / _tr_b8 reads.  RD_AUTO: RD_TR for 16-byte
// accesses, RD_B32 for the narrow rung.
enum FragRead { RD_AUTO = 0, RD_B32 = 1, RD_B64 = 2, RD_B128 = 3, RD_TR = 4 };

// SPREAD (direct loader): issue each slice's copies in two parts, the
// second spread over the K steps of the following slice, instead of all of
// them right after the slice's barrier (see N1 below).  LATE (direct
// loader, steady ring): the slice's barrier, and the copies and reads that
// follow it, come after half of the last K step's matrix instructions
// instead of after its second one (a measurement twin: the cores idle
// longer at the barrier, with everything else the same).
template <class Tr, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int LOADER,
          int LAYOUT, int ACCESS, int FRAG, int SHIFT = 0, int CST = CST_MFMA, bool SPREAD = false,
          int FREAD_ = RD_AUTO, bool REM = false, bool LATE = false>
struct MfmaGemm {
    typedef typename Tr::T T;
    typedef typename Tr::Out Out;
    typedef typename Tr::Out4 Out4;
    typedef typename Tr::Acc Acc;

    // one matrix instruction: acc += A-fragment x B-fragment (CST_SWAP:
    // acc^T += B-fragment^T x A-fragment^T, the transposed tile)
    __device__ static __forceinline__ Acc mma(i32x4 a, i32x4 b, Acc c) {
        if constexpr (CST == CST_SWAP) return Tr::mma(b, a, c);
        else return Tr::mma(a, b, c);
    }

    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int ESZ = Tr::ESZ;
    static constexpr int CE = 16 / ESZ;      // elements per 16-byte chunk
    static constexpr int KB = BK * ESZ;      // bytes of one A row of a slice
    static constexpr int CA = KB / 16;       // 16-byte chunks per A row
    static constexpr int NB = BN * ESZ;      // bytes of one B row of a slice
    static constexpr int CB = NB / 16;       // 16-byte chunks per B row
    static constexpr int A_BYTES = BM * KB;
    static constexpr int B_BYTES = BK * NB;
    // REM: the last column of C (the one past the grid's N) is computed in
    // the same K loop (see rem_slice): each slot also holds, for every B row
    // of the slice, the 4 bytes of that row that end at the column
    static constexpr int REM_BYTES = REM ? BK * 4 : 0;
    static constexpr int SLOT = A_BYTES + B_BYTES + REM_BYTES;
    static constexpr int LDS_BYTES = STAGES * SLOT;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int KSUB = BK / Tr::MK;  // matrix-core K steps per slice
    static constexpr int A_PER = BM * CA / NT;  // 16-byte A chunks per thread per slice
    static constexpr int B_PER = BK * CB / NT;
    static constexpr int N_LD = A_PER + B_PER;  // loads per thread (= per wave) per slice
    static constexpr bool XOR = LAYOUT == LY_XOR || LAYOUT == LY_XOR_POISON;
    static constexpr bool POISON = LAYOUT == LY_XOR_POISON;
    static constexpr bool WIDE = ACCESS == AC_WIDE;
    static constexpr int FREAD = FREAD_ != RD_AUTO ? FREAD_ : (WIDE ? RD_TR : RD_B32);
    static constexpr bool DIRECT = LOADER == LD_DIRECT;
    // narrow (4-byte) accesses
    static constexpr int A_DW = BM * KB / 4 / NT;  // A dwords per thread per slice
    static constexpr int B_DW = BK * NB / 4 / NT;

    static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "wave tile");
    static_assert(BK % Tr::MK == 0, "slice must hold whole matrix-core steps");
    static_assert((BM * CA) % NT == 0 && (BK * CB) % NT == 0, "even 16-byte split");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS per CU");
    static_assert(!DIRECT || WIDE, "direct loads move 16-byte chunks");
    static_assert(DIRECT || STAGES <= 2, "register-staged loader: 1 or 2 slots");
    static_assert(WIDE || (!XOR && !DIRECT), "narrow accesses use the plain layout");
    static_assert(FRAG != FR_PER_MMA || !WIDE, "per-instruction fragment reloads only on the narrow rung");
    static_assert(!LATE || (DIRECT && STAGES >= 2 && FRAG != FR_SLICE && !REM), "late barrier: the direct ring");
    static_assert(FRAG != FR_SLICE || (DIRECT && STAGES >= 2 && !SPREAD && !REM),
                  "whole-slice read-ahead: the plain direct-loader ring");
    static_assert(N_LD * (STAGES > 2 ? STAGES - 2 : 0) <= 63, "vmcnt range");
    static_assert(!POISON || (DIRECT && STAGES >= 2), "poisoned slots: the direct-loader ring");
    static_assert(SHIFT == 0 || (LOADER == LD_VGPR && WIDE), "shifted loads: register-staged, 16-byte chunks");
    static_assert(WIDE || FREAD == RD_B32, "the narrow rung reads 4 bytes at a time");
    static_assert(!REM || (DIRECT && STAGES == 2 && !SPREAD && CST == CST_MFMA && !POISON && BK % 64 == 0 &&
                           BK / 64 <= WAVES_M * WAVES_N && KB / 16 == 8),
                  "in-loop remainder column: the 2-slot direct ring, 8 chunks per A row");
    // Shifted chunks complete their pairs from the neighbouring lane after
    // the multiply when the staged registers are few (the extra block and
    // shift per chunk then fit); with more chunks per thread the pair is
    // loaded and shifted at load time instead, which needs no extra
    // registers across the multiply.
    static constexpr bool DEFER_SHIFT = A_PER + B_PER <= 4;

    // ---- LDS layout --------------------------------------------------------
    // A: row r of a slice at r*KB; its 16-byte chunks permuted by an XOR so
    // that the rows read by one 16-byte fragment read spread over the banks.
    // gfx950's LDS serves 64 banks x 4 bytes = one 256-byte window per cycle
    // (16 lanes of a 16-byte read): the 16 rows such a group reads must land
    // on 16 distinct 16-byte offsets of that window.  Rows that share one
    // window differ by their row offset; consecutive windows get distinct
    // XOR keys.
    static constexpr int LDS_WINDOW = 256;
    static constexpr int A_ROWS_PER_WIN = KB >= LDS_WINDOW ? 1 : LDS_WINDOW / KB;
    __device__ static __forceinline__ int a_chunk(int row, int c) {
        if constexpr (XOR) return c ^ ((row / A_ROWS_PER_WIN) & (CA - 1));
        else return c;
    }
    // B: row k at k*NB.  A transposing read covers (8/ESZ) consecutive rows
    // per 16-lane group, and each 32 lanes of it (one LDS pass of 256 bytes)
    // read 16/B_RPG chunks of each of those rows.  Rows that fall on the same
    // banks - every row, where a row fills a 256-byte window or more; rows
    // B_RPW apart, where B_RPW rows share a window - get distinct XOR keys in
    // the bits above those chunks, so the pass touches every bank once.
    static constexpr int B_RPG = 8 / ESZ;                   // rows per 16-lane group of one transposing read
    static constexpr int B_RPW = NB >= LDS_WINDOW ? 1 : LDS_WINDOW / NB;  // B rows per 256-byte window
    __device__ static __forceinline__ int b_chunk(int k, int c) {
        if constexpr (XOR) return c ^ ((((k % B_RPG) / B_RPW) * (16 / B_RPG)) & (CB - 1));
        else return c;
    }

    // ---- global loads --------------------------------------------------------
    enum { LM_ALIGNED = 0, LM_SHIFTED = 1, LM_SHIFTED_EDGE = 2, LM_ELEMENT = 3 };
    // the mode of a first or last whole slice
    static constexpr int edge_mode(int m) { return m == LM_SHIFTED ? LM_SHIFTED_EDGE : m; }
    // Elements [start, start + CE) of one row, zero where index >= limit.
    // The scheduling fence keeps the compiler from computing the addresses
    // of every chunk's element loads up front (64-bit each, they would not
    // fit in the registers); the loads of all chunks still overlap.
    __device__ static __forceinline__ i32x4 load_chunk_guarded(const T* rowp, int start, int limit) {
        union { i32x4 v; T e[CE]; } u;
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            const int idx = start + e;
            u.e[e] = load_or_zero(rowp + idx, idx < limit);
        }
        __builtin_amdgcn_sched_barrier(0);
        return u.v;
    }

    __device__ static __forceinline__ i32x4 funnel(i32x4 x, i32x4 y, uint32_t sh) { return funnel16(x, y, sh); }

    // The value of `v` in lane + 1 of the same 16-lane row (DPP row_shl:1);
    // lanes 15, 31, 47, 63 keep `own`.
    __device__ static __forceinline__ i32x4 from_right_lane(i32x4 v, i32x4 own) {
        i32x4 out;
#pragma unroll
        for (int d = 0; d < 4; ++d) out[d] = __builtin_amdgcn_update_dpp(own[d], v[d], 0x101, 0xf, 0xf, false);
        return out;
    }

    // 16 bytes starting at p, for an operand whose valid bytes are [beg, end)
    // and whose rows are not 16-byte aligned: the two aligned 16-byte blocks
    // that cover them are loaded and the wanted bytes funnel-shifted out of
    // the pair (2 wide loads and ~15 ALU operations instead of CE element
    // loads).  CHECK: where the pair would leave [beg, end) the chunk falls
    // back to element loads, zero past end.  Without CHECK the caller has
    // shown that the pair lies inside (see staged_loop).
    template <bool CHECK>
    __device__ static __forceinline__ i32x4 load_chunk_shifted(const T* p, uintptr_t beg, uintptr_t end) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        const uintptr_t lo = a & ~uintptr_t(15);
        if (!CHECK || (lo >= beg && lo + 32 <= end)) {
            const i32x4 x = *reinterpret_cast<const i32x4*>(lo);
            const i32x4 y = *reinterpret_cast<const i32x4*>(lo + 16);
            return funnel(x, y, uint32_t(a & 15));
        }
        union { i32x4 v; T e[CE]; } u;
#pragma unroll
        for (int e = 0; e < CE; ++e) u.e[e] = load_or_zero(p + e, a + (e + 1) * ESZ <= end);
        return u.v;
    }

    // Registers of one register-staged slice.  For LM_SHIFTED operands with
    // DEFER_SHIFT, `a` / `b` hold the low aligned block of each chunk's pair
    // and `*sh` its byte offset; the high block is the next chunk's low block, which lane + 1
    // holds, except in the lanes at the end of an operand row or of a
    // 16-lane DPP row: those load it into `ah` / `bh` themselves.  The funnel
    // shift happens in store_regs, after the multiply, so that the loads'
    // latency stays hidden behind it as in the aligned case.
    template <int MODE_A, int MODE_B>
    struct Staged {
        static constexpr bool SA = DEFER_SHIFT && MODE_A == LM_SHIFTED;
        static constexpr bool SB = DEFER_SHIFT && MODE_B == LM_SHIFTED;
        i32x4 a[WIDE ? A_PER : 1];
        i32x4 b[WIDE ? B_PER : 1];
        i32x4 ah[SA ? A_PER : 1];
        i32x4 bh[SB ? B_PER : 1];
        uint32_t ash[SA ? A_PER : 1];
        uint32_t bsh[SB ? B_PER : 1];
        int32_t ad[WIDE ? 1 : A_DW];
        int32_t bd[WIDE ? 1 : B_DW];
    };

    // does this lane load the high block of its shifted pair itself?
    __device__ static __forceinline__ bool own_high(int c, int chunks_per_row) {
        return c == chunks_per_row - 1 || (threadIdx.x & 15) == 15;
    }

    // Register-staged load of slice k0.  Per operand, a load mode:
    //   LM_ALIGNED : 16-byte loads (rows 16-byte aligned, N a multiple of CE);
    //   LM_SHIFTED : rows not 16-byte aligned, slice inside K: one aligned
    //                16-byte load per chunk, the pair completed from the
    //                neighbouring lane and funnel-shifted in store_regs (values
    //                at n >= N are whatever follows in memory; they only reach
    //                C columns that are never stored);
    //   LM_SHIFTED_EDGE : the same with a bounds check per pair, for the
    //                first and last whole slices;
    //   LM_ELEMENT : element loads with zero fill at k >= K (and n >= N for
    //                B): the partial last K slice.  In kernels that only
    //                see 16-byte aligned rows (no SHIFT bit for the operand)
    //                a chunk wholly inside K (and N) takes one 16-byte load.
    template <int MODE_A, int MODE_B>
    __device__ static __forceinline__ void load_regs(Staged<MODE_A, MODE_B>& r, const GemmArgs& g, int m0, int n0,
                                                     int k0) {
        const T* A = static_cast<const T*>(g.A);
        const T* B = static_cast<const T*>(g.B);
        const int tid = threadIdx.x;
        if constexpr (WIDE) {
            const uintptr_t a_beg = reinterpret_cast<uintptr_t>(A);
            const uintptr_t a_end = a_beg + ((int64_t)(g.M - 1) * g.lda + g.K) * ESZ;
            const uintptr_t b_beg = reinterpret_cast<uintptr_t>(B);
            const uintptr_t b_end = b_beg + ((int64_t)(g.K - 1) * g.ldb + g.N) * ESZ;
#pragma unroll
            for (int q = 0; q < A_PER; ++q) {
                const int p = q * NT + tid;
                const int row = p / CA, c = p % CA;
                const T* rowp = A + (int64_t)min(m0 + row, g.M - 1) * g.lda;
                const int kc = k0 + c * CE;
                if constexpr (MODE_A == LM_ALIGNED) {
                    r.a[q] = *reinterpret_cast<const i32x4*>(rowp + kc);
                } else if constexpr (MODE_A == LM_SHIFTED && !DEFER_SHIFT) {
                    r.a[q] = load_chunk_shifted<false>(rowp + kc, a_beg, a_end);
                } else if constexpr (MODE_A == LM_SHIFTED) {
                    const uintptr_t ad = reinterpret_cast<uintptr_t>(rowp + kc);
                    const uintptr_t lo = ad & ~uintptr_t(15);
                    r.a[q] = *reinterpret_cast<const i32x4*>(lo);
                    r.ash[q] = uint32_t(ad & 15);
                    r.ah[q] = i32x4{0, 0, 0, 0};
                    if (own_high(c, CA)) r.ah[q] = *reinterpret_cast<const i32x4*>(lo + 16);
                } else if constexpr (MODE_A == LM_SHIFTED_EDGE) {
                    r.a[q] = load_chunk_shifted<true>(rowp + kc, a_beg, a_end);
                } else if ((SHIFT & 1) == 0 && kc + CE <= g.K) {
                    // K tail, a chunk wholly inside K (rows of any alignment
                    // in the direct kernels)
                    r.a[q] = load16(rowp + kc);
                } else {
                    r.a[q] = load_chunk_guarded(rowp, kc, g.K);
                }
            }
#pragma unroll
            for (int q = 0; q < B_PER; ++q) {
                const int p = q * NT + tid;
                const int k = p / CB, c = p % CB;
                const int gk = k0 + k;
                const int nc = n0 + c * CE;
                const T* rowp = B + (int64_t)gk * g.ldb;
                if constexpr (MODE_B == LM_ALIGNED) {
                    r.b[q] = *reinterpret_cast<const i32x4*>(rowp + min(nc, g.N - CE));
                } else if constexpr (MODE_B == LM_SHIFTED && !DEFER_SHIFT) {
                    r.b[q] = load_chunk_shifted<false>(rowp + min(nc, g.N - 1), b_beg, b_end);
                } else if constexpr (MODE_B == LM_SHIFTED) {
                    const uintptr_t ad = reinterpret_cast<uintptr_t>(rowp + min(nc, g.N - 1));
                    const uintptr_t lo = ad & ~uintptr_t(15);
                    r.b[q] = *reinterpret_cast<const i32x4*>(lo);
                    r.bsh[q] = uint32_t(ad & 15);
                    r.bh[q] = i32x4{0, 0, 0, 0};
                    if (own_high(c, CB)) r.bh[q] = *reinterpret_cast<const i32x4*>(lo + 16);
                } else if constexpr (MODE_B == LM_SHIFTED_EDGE) {
                    r.b[q] = load_chunk_shifted<true>(rowp + min(nc, g.N - 1), b_beg, b_end);
                } else if ((SHIFT & 2) == 0 && gk < g.K && nc + CE <= g.N) {
                    // K tail, a whole chunk that lies inside K and N
                    r.b[q] = load16(rowp + nc);
                } else {
                    r.b[q] = gk < g.K ? load_chunk_guarded(rowp, nc, g.N) : i32x4{0, 0, 0, 0};
                }
            }
        } else {
            constexpr int EPD = 4 / ESZ;  // elements per dword
#pragma unroll
            for (int q = 0; q < A_DW; ++q) {
                const int p = q * NT + tid;
                const int row = p / (KB / 4), d = p % (KB / 4);
                const T* rowp = A + (int64_t)min(m0 + row, g.M - 1) * g.lda;
                const int kc = k0 + d * EPD;
                if constexpr (MODE_A == LM_ALIGNED) {
                    r.ad[q] = *reinterpret_cast<const int32_t*>(rowp + kc);
                } else {
                    union { int32_t v; T e[EPD]; } u;
#pragma unroll
                    for (int e = 0; e < EPD; ++e) u.e[e] = load_or_zero(rowp + kc + e, kc + e < g.K);
                    r.ad[q] = u.v;
                }
            }
#pragma unroll
            for (int q = 0; q < B_DW; ++q) {
                const int p = q * NT + tid;
                const int k = p / (NB / 4), d = p % (NB / 4);
                const int gk = k0 + k;
                const int nc = n0 + d * EPD;
                if constexpr (MODE_B == LM_ALIGNED) {
                    r.bd[q] = *reinterpret_cast<const int32_t*>(B + (int64_t)gk * g.ldb + min(nc, g.N - EPD));
                } else {
                    union { int32_t v; T e[EPD]; } u;
                    const T* rowp = B + (int64_t)gk * g.ldb;
#pragma unroll
                    for (int e = 0; e < EPD; ++e) u.e[e] = load_or_zero(rowp + nc + e, gk < g.K && nc + e < g.N);
                    r.bd[q] = u.v;
                }
            }
        }
    }

    // Shifted chunks: the high block comes from lane + 1 (the next chunk of
    // the same row: its low block starts 16 bytes later) unless this lane
    // loaded it.  Where lane + 1's column was clamped to N - 1, its block is
    // either the right one or this lane's own, and then every byte past this
    // lane's low block lies at a column >= N.
    template <int MODE_A, int MODE_B>
    __device__ static __forceinline__ void store_regs(TG_LDS char* slot, const Staged<MODE_A, MODE_B>& r) {
        const int tid = threadIdx.x;
        if constexpr (WIDE) {
#pragma unroll
            for (int q = 0; q < A_PER; ++q) {
                const int p = q * NT + tid;
                const int row = p / CA, c = p % CA;
                i32x4 v = r.a[q];
                if constexpr (Staged<MODE_A, MODE_B>::SA) {
                    const i32x4 nb = from_right_lane(r.a[q], r.ah[q]);
                    v = funnel(r.a[q], own_high(c, CA) ? r.ah[q] : nb, r.ash[q]);
                }
                *reinterpret_cast<TG_LDS i32x4*>(slot + row * KB + a_chunk(row, c) * 16) = v;
            }
#pragma unroll
            for (int q = 0; q < B_PER; ++q) {
                const int p = q * NT + tid;
                const int k = p / CB, c = p % CB;
                i32x4 v = r.b[q];
                if constexpr (Staged<MODE_A, MODE_B>::SB) {
                    const i32x4 nb = from_right_lane(r.b[q], r.bh[q]);
                    v = funnel(r.b[q], own_high(c, CB) ? r.bh[q] : nb, r.bsh[q]);
                }
                *reinterpret_cast<TG_LDS i32x4*>(slot + A_BYTES + k * NB + b_chunk(k, c) * 16) = v;
            }
        } else {
#pragma unroll
            for (int q = 0; q < A_DW; ++q)
                *reinterpret_cast<TG_LDS int32_t*>(slot + (q * NT + tid) * 4) = r.ad[q];
#pragma unroll
            for (int q = 0; q < B_DW; ++q)
                *reinterpret_cast<TG_LDS int32_t*>(slot + A_BYTES + (q * NT + tid) * 4) = r.bd[q];
        }
    }

    // Direct global->LDS copies.  Lane l of each instruction lands at
    // (wave base + 16 l), so the XOR layout is produced by choosing which
    // global chunk each lane fetches.  The per-lane byte offsets from the
    // slice's (wave-uniform) base address never change along K, so they are
    // computed once: A chunk q of this thread sits at row r, logical chunk c
    // -> r*lda + c*16 bytes from A's slice base (rows past M clamped to the
    // last row); B chunk q at row k, chunk c -> k*ldb + column bytes from B's
    // slice base, where a chunk that starts inside N is read where it is and
    // one that starts at or past N is clamped to the row's last whole chunk,
    // or to the tile's first column when that lies further right (its
    // columns are never stored).  With N not a whole number of chunks
    // the chunk that crosses N also reads past N, into the row's padding or
    // the next row: still inside B for every row but the last, which the
    // kernel never copies (run: the slice holding it goes through the
    // register tail).  The host only picks this loader when the offsets fit
    // in 32 bits and N is at least one chunk.
    struct DirectOffsets {
        uint32_t a[A_PER];
        uint32_t b[B_PER];
        uint32_t rem;  // REM: this lane's B row (wave * 64 + lane) of a slice, in bytes
    };

    __device__ static __forceinline__ void direct_offsets(DirectOffsets& o, const GemmArgs& g, int m0,
                                                          int n0) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int q = 0; q < A_PER; ++q) {
            const int p = q * NT + tid;
            const int row = p / CA, pc = p % CA;
            const int c = a_chunk(row, pc);  // XOR is its own inverse
            const int r = min(m0 + row, g.M - 1) - m0;
            o.a[q] = (uint32_t)((int64_t)r * g.lda * ESZ + c * 16);
        }
#pragma unroll
        for (int q = 0; q < B_PER; ++q) {
            const int p = q * NT + tid;
            const int k = p / CB, pc = p % CB;
            const int c = b_chunk(k, pc);
            const int nc = n0 + c * CE;
            // never left of the tile's first column: the offset is unsigned
            // (a tile column that starts within a chunk of N has no whole
            // chunk inside N, and N - CE lies left of it)
            const int col = (nc < g.N ? nc : max(g.N - CE, n0)) - n0;
            o.b[q] = (uint32_t)((int64_t)k * g.ldb * ESZ + col * ESZ);
        }
        o.rem = REM ? (uint32_t)((int64_t)(wave_id() * 64 + lane_id()) * g.ldb * ESZ) : 0u;
    }

    // Issue copy number i (0 <= i < N_LD) of one slice into `slot`.  Lane l
    // of the copy writes the 16 bytes at its wave's base + 16 l.  POISON
    // (debug): the lane first stores all-ones bytes there and waits for the
    // store, so until the copy lands the chunk reads as NaN (bf16) / -1
    // (int8); every lane poisons only the bytes its own copy overwrites.
    __device__ static __forceinline__ void issue_direct_one(int i, TG_LDS char* slot, const DirectOffsets& o,
                                                            const char* abase, const char* bbase,
                                                            int wave) {
        const uint32_t lds = (uint32_t)(uintptr_t)slot;
        const int off = i < A_PER ? (i * NT + wave * 64) * 16 : A_BYTES + ((i - A_PER) * NT + wave * 64) * 16;
        if constexpr (POISON) {
            *reinterpret_cast<TG_LDS i32x4*>(slot + off + lane_id() * 16) = i32x4{-1, -1, -1, -1};
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if (i < A_PER) copy16_to_lds(lds + off, o.a[i], abase);
        else copy16_to_lds(lds + off, o.b[i - A_PER], bbase);
    }

    __device__ static __forceinline__ void issue_direct(TG_LDS char* slot, const DirectOffsets& o,
                                                        const char* abase, const char* bbase, int wave) {
#pragma unroll
        for (int i = 0; i < N_LD; ++i) issue_direct_one(i, slot, o, abase, bbase, wave);
    }

    // ---- fragments -----------------------------------------------------------
    // A fragment of 32 x 32 tile row block at `row0`, K step s: lane l holds
    // row row0 + l%32, bytes [16 (l/32), +16) of the step's 32-byte K span:
    // one 16-byte read, or (RD_B64 / RD_B32) two 8-byte or four 4-byte reads
    // of the same bytes (volatile, so that they are not merged).
    __device__ static __forceinline__ i32x4 read_a(const TG_LDS char* slot, int row0, int s, int lane) {
        const int row = row0 + (lane & 31);
        const int c = 2 * s + (lane >> 5);
        const TG_LDS char* p = slot + row * KB + a_chunk(row, c) * 16;
        if constexpr (FREAD == RD_B32) {
            const volatile TG_LDS int32_t* q = reinterpret_cast<const volatile TG_LDS int32_t*>(p);
            return i32x4{q[0], q[1], q[2], q[3]};
        } else if constexpr (FREAD == RD_B64) {
            const volatile TG_LDS i32x2* q = reinterpret_cast<const volatile TG_LDS i32x2*>(p);
            const i32x2 lo = q[0], hi = q[1];
            return i32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
            return *reinterpret_cast<const TG_LDS i32x4*>(p);
        }
    }

    // B fragment of the 32-column block at `col0`, K step s: lane l holds
    // column col0 + l%32 and K rows s*MK + (MK/2)(l/32) + e.  Half h (0:
    // first, 1: second 8/ESZ K rows of the lane's run).  RD_TR: one
    // transposing read - in each 16-lane group, input lane j points at row
    // kb + j/(8/ESZ) and 8 bytes of columns; output lane i receives column
    // nb + i of 8/ESZ consecutive rows.  Otherwise 8/ESZ element reads of
    // the lane's own column (volatile, one per K row).
    __device__ static __forceinline__ i32x2 read_b_half(const TG_LDS char* bslot, int col0, int s, int lane,
                                                        int h) {
        if constexpr (FREAD == RD_TR) {
            const int grp = lane >> 4, j = lane & 15;
            const int nb = col0 + 16 * (grp & 1);
            if constexpr (ESZ == 2) {
                const int row = s * 16 + 8 * (grp >> 1) + (j >> 2) + 4 * h;
                const int byte = (nb + 4 * (j & 3)) * 2;
                const int c = byte >> 4, w = byte & 15;
                const TG_LDS char* p = bslot + row * NB + b_chunk(row, c) * 16 + w;
                return __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS i16x4*)(p)));
            } else {
                const int row = s * 32 + 16 * (grp >> 1) + (j >> 1) + 8 * h;
                const int byte = nb + 8 * (j & 1);
                const int c = byte >> 4, w = byte & 15;
                const TG_LDS char* p = bslot + row * NB + b_chunk(row, c) * 16 + w;
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32((TG_LDS i32x2*)(p));
            }
        } else {
            constexpr int PER = 8 / ESZ;  // K rows per half
            const int col = col0 + (lane & 31);
            const int kb = s * Tr::MK + (Tr::MK / 2) * (lane >> 5) + PER * h;
            const int c = col / CE, w = (col % CE) * ESZ;
            union { i32x2 v; T e[PER]; } u;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int row = kb + e;
                u.e[e] = *reinterpret_cast<const volatile TG_LDS T*>(bslot + row * NB + b_chunk(row, c) * 16 + w);
            }
            return u.v;
        }
    }

    __device__ static __forceinline__ i32x4 read_b(const TG_LDS char* bslot, int col0, int s, int lane) {
        const i32x2 lo = read_b_half(bslot, col0, s, lane, 0);
        const i32x2 hi = read_b_half(bslot, col0, s, lane, 1);
        return i32x4{lo.x, lo.y, hi.x, hi.y};
    }

    struct Frags {
        i32x4 a[FM];
        i32x4 b[FN];
    };

    __device__ static __forceinline__ void read_frags(Frags& f, const TG_LDS char* slot, int s, int wm0,
                                                      int wn0, int lane) {
#pragma unroll
        for (int i = 0; i < FM; ++i) f.a[i] = read_a(slot, wm0 + 32 * i, s, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = read_b(slot + A_BYTES, wn0 + 32 * j, s, lane);
    }

    // ---- interleaved K step (direct loader) -------------------------------
    // One K step issues its FM*FN matrix-core instructions one at a time and
    // puts the step's memory instructions (fragment reads for the next K
    // step, copies for a later slice) between them, fenced so the compiler
    // keeps the order: with one or two waves per SIMD little else keeps the
    // matrix core busy while a burst of LDS instructions is being issued.
    static constexpr int NM = FM * FN;      // matrix-core instructions per K step
    static constexpr int NR = FM + 2 * FN;  // LDS reads per K step (A: 1 each, B: 2 each)

    // Read number r of K step s of `slot` into f, in the order the matrix
    // instructions consume them: a0, b0 (two halves), ..., b(FN-1), a1, ...
    __device__ static __forceinline__ void read_op(Frags& f, const TG_LDS char* slot, int s, int r,
                                                   int wm0, int wn0, int lane) {
        if (r == 0) {
            f.a[0] = read_a(slot, wm0, s, lane);
        } else if (r <= 2 * FN) {
            const int j = (r - 1) >> 1, h = (r - 1) & 1;
            const i32x2 v = read_b_half(slot + A_BYTES, wn0 + 32 * j, s, lane, h);
            if (h == 0) {
                f.b[j].x = v.x;
                f.b[j].y = v.y;
            } else {
                f.b[j].z = v.x;
                f.b[j].w = v.y;
            }
        } else {
            const int i = r - 2 * FN;
            f.a[i] = read_a(slot, wm0 + 32 * i, s, lane);
        }
    }

    // Memory instructions [mem_begin(k), mem_begin(k+1)) follow matrix
    // instruction k when `total` of them are spread evenly over matrix
    // instructions first .. NM-1 (0 <= first < NM).
    __device__ static constexpr int mem_begin(int k, int first, int total) {
        return k <= first ? 0 : ((k - first) * total + (NM - first) - 1) / (NM - first);
    }

    // Where one slice's direct copies go: the LDS slot and the wave-uniform
    // A / B addresses of the slice.
    struct CopyTarget {
        TG_LDS char* slot;
        const char* ca;
        const char* cb;
        const char* cc;  // REM: the slice's B rows at the remainder column's dword
    };

    // Copies of slice u are issued in two parts.  Part 1, copies [0, N1),
    // follows the barrier in the last K step of slice u - STAGES (the
    // barrier that frees u's slot); part 2, copies [N1, N_LD), is spread
    // over K steps 0 .. KSUB-2 of slice u - STAGES + 1.  Without SPREAD
    // part 1 is every copy.  Either way the copies of a slice are issued
    // before any copy of a later one, so "at most n later slices in flight"
    // stays vmcnt(n N_LD).
    static constexpr int N1 = (SPREAD && KSUB > 1) ? (N_LD + KSUB - 1) / KSUB : N_LD;
    static constexpr int N2 = N_LD - N1;
    // first copy of part 2 issued in K step s (0 <= s <= KSUB-1)
    __device__ static constexpr int part2_begin(int s) { return KSUB > 1 ? N1 + (s * N2) / (KSUB - 1) : N_LD; }

    // ---- the remainder column (REM) ------------------------------------------
    // A product one column wider than a whole number of tiles (N = g.N + 1)
    // gets that last column from the same K loop instead of a second launch,
    // whose workgroups would each walk B's column, one cache line per row of
    // B.  With every slice, waves 0 .. BK/64 - 1 copy for each of the slice's
    // B rows the 4 bytes that end at the column (the column is their last
    // element, CPD elements per dword) into the slot's REM area, row k at
    // 4 k.  Workgroup (tm, tn) owns rows tn*16 .. tn*16+15 of its tile for
    // that column (the host only takes this path when the tile columns cover
    // every row: BM <= 16 tiles_n); in waves 0 and 1, lane 8 r + c takes row
    // 8 w + r and the c-th 16-byte chunk (CE values of k) of the slice's A
    // row, and multiplies it by the column's CE values with the packed dot
    // instructions (bf16 pairs into fp32, int8 quads into int32).  Each lane
    // keeps one partial sum over the K loop; the 8 lanes of a row are added
    // at the end.
    static constexpr int CPD = 4 / ESZ;  // elements per copied dword
    __device__ static __forceinline__ void issue_rem(TG_LDS char* slot, const DirectOffsets& o, const char* cc,
                                                     int wave) {
        if constexpr (REM) {
            if (wave < BK / 64) copy4_to_lds((uint32_t)(uintptr_t)(slot + A_BYTES + B_BYTES + wave * 256), o.rem, cc);
        }
    }

    // The column's dwords of rows k0 .. k0+BK-1 (the partial last slice):
    // element loads of any alignment, zero at k >= K.
    __device__ static __forceinline__ void fill_rem(TG_LDS char* slot, const GemmArgs& g, int k0, int wave,
                                                    int lane) {
        if constexpr (REM) {
            if (wave < BK / 64) {
                const int k = k0 + wave * 64 + lane;
                const char* p = static_cast<const char*>(g.B) + ((int64_t)k * g.ldb + g.N + 1 - CPD) * ESZ;
                uint32_t v = 0;
                if (k < g.K) __builtin_memcpy(&v, p, 4);
                *reinterpret_cast<TG_LDS uint32_t*>(slot + A_BYTES + B_BYTES + (wave * 64 + lane) * 4) = v;
            }
        }
    }

    // One slice's share of the remainder column for row `rt` of the tile.
    __device__ static __forceinline__ void rem_slice(const TG_LDS char* slot, Out& racc, int rt, int lane) {
        const int c = lane & 7;
        const i32x4 a = *reinterpret_cast<const TG_LDS i32x4*>(slot + rt * KB + a_chunk(rt, c) * 16);
        const TG_LDS i32x4* col = reinterpret_cast<const TG_LDS i32x4*>(slot + A_BYTES + B_BYTES + c * CE * 4);
        if constexpr (ESZ == 2) {
            // rows 8c .. 8c+7: the column is the high half of each dword;
            // pair rows 2p, 2p+1 into one dword and take a dot of two
            const i32x4 b0 = col[0], b1 = col[1];
            const uint32_t d[8] = {(uint32_t)b0.x, (uint32_t)b0.y, (uint32_t)b0.z, (uint32_t)b0.w,
                                   (uint32_t)b1.x, (uint32_t)b1.y, (uint32_t)b1.z, (uint32_t)b1.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t pr = __builtin_amdgcn_perm(d[2 * q + 1], d[2 * q], 0x07060302u);
                racc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)a[q]),
                                                       __builtin_bit_cast(bf16x2, pr), racc, false);
            }
        } else {
            // rows 16c .. 16c+15: the column is byte 3 of each dword; gather
            // rows 4q .. 4q+3 into one dword and take a dot of four
            uint32_t d[16];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const i32x4 b = col[h];
                d[4 * h] = (uint32_t)b.x;
                d[4 * h + 1] = (uint32_t)b.y;
                d[4 * h + 2] = (uint32_t)b.z;
                d[4 * h + 3] = (uint32_t)b.w;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = __builtin_amdgcn_perm(d[4 * q + 1], d[4 * q], 0x07030703u);
                const uint32_t hi = __builtin_amdgcn_perm(d[4 * q + 3], d[4 * q + 2], 0x07030703u);
                const uint32_t v = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                racc = __builtin_amdgcn_sdot4((int)a[q], (int)v, racc, false);
            }
        }
    }

    // Matrix step on `cur` with reads of (rslot, rs) into `nxt` interleaved.
    // BARRIER: before the reads, meet the other waves once this wave's slot
    // reads are done and at most `ahead` later slices' copies are in flight
    // (after matrix instruction BAR_K); then issue copies [DB, DE) of the
    // slice `ct` after the reads.
    template <bool READS, bool BARRIER, int DB, int DE>
    __device__ static __forceinline__ void kstep(Acc (&acc)[FM][FN], const Frags& cur, Frags& nxt,
                                                 const TG_LDS char* rslot, int rs, int ahead, const CopyTarget& ct,
                                                 const DirectOffsets& off, int wm0, int wn0, int lane, int wave) {
        // the barrier follows matrix instruction BAR_K; the memory
        // instructions start after it
        constexpr int BAR_K = (BARRIER && NM >= 8) ? (LATE ? NM / 2 : 1) : 0;
        static_assert(BAR_K < NM, "barrier inside the K step");
        static_assert(0 <= DB && DB <= DE && DE <= N_LD, "copy range");
        constexpr int NREAD = READS ? NR : 0;
        constexpr int TOTAL = NREAD + (DE - DB);
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const int i = k / FN, j = k % FN;
            acc[i][j] = mma(cur.a[i], cur.b[j], acc[i][j]);
            if (BARRIER && k == BAR_K) wait_slice(ahead);
#pragma unroll
            for (int m = mem_begin(k, BAR_K, TOTAL); m < mem_begin(k + 1, BAR_K, TOTAL); ++m) {
                if (m < NREAD) read_op(nxt, rslot, rs, m, wm0, wn0, lane);
                else issue_direct_one(DB + m - NREAD, ct.slot, off, ct.ca, ct.cb, wave);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (REM && BARRIER && DB == 0 && DE > 0) issue_rem(ct.slot, off, ct.cc, wave);
    }

    // K steps s .. KSUB-1 of one slice t from `cur_slot`.  PREV: issue part
    // 2 of the copies of slice t + STAGES - 1 (`prev`) over steps 0 ..
    // KSUB-2.  NEXT: slice t+1 exists (barrier in the last K step, then its
    // first fragments are read from `next_slot`); DMA: after that barrier
    // also issue part 1 of the copies of slice t + STAGES (`next`, into the
    // slot slice t leaves).
    template <int S, bool PREV, bool NEXT, bool DMA>
    __device__ static __forceinline__ void slice_steps(Acc (&acc)[FM][FN], Frags (&f)[2],
                                                       const TG_LDS char* cur_slot, const TG_LDS char* next_slot,
                                                       int ahead, const CopyTarget& prev, const CopyTarget& next,
                                                       const DirectOffsets& off, int wm0, int wn0, int lane,
                                                       int wave) {
        if constexpr (S + 1 < KSUB) {
            constexpr int DB = PREV ? part2_begin(S) : 0, DE = PREV ? part2_begin(S + 1) : 0;
            kstep<true, false, DB, DE>(acc, f[S & 1], f[(S + 1) & 1], cur_slot, S + 1, 0, prev, off, wm0, wn0,
                                       lane, wave);
            slice_steps<S + 1, PREV, NEXT, DMA>(acc, f, cur_slot, next_slot, ahead, prev, next, off, wm0, wn0,
                                                lane, wave);
        } else {
            kstep<NEXT, NEXT, 0, DMA ? N1 : 0>(acc, f[S & 1], f[(S + 1) & 1], next_slot, 0, ahead, next, off,
                                               wm0, wn0, lane, wave);
        }
    }

    template <bool PREV, bool NEXT, bool DMA>
    __device__ static __forceinline__ void slice_direct(Acc (&acc)[FM][FN], Frags (&f)[2],
                                                        const TG_LDS char* cur_slot, const TG_LDS char* next_slot,
                                                        int ahead, const CopyTarget& prev, const CopyTarget& next,
                                                        const DirectOffsets& off, int wm0, int wn0, int lane,
                                                        int wave) {
        slice_steps<0, PREV, NEXT, DMA>(acc, f, cur_slot, next_slot, ahead, prev, next, off, wm0, wn0, lane,
                                        wave);
    }

    // ---- whole-slice read-ahead (FR_SLICE) -------------------------------------
    // With one or two matrix instructions per K step (32 x 32 or 64 x 32
    // wave tiles), the instruction issued before a K step's fragment reads
    // is too short to cover their LDS latency, so every K step would wait
    // for its own reads.  Here F[s] holds K step s of the slice being
    // multiplied, and right after step s's matrix instructions the same
    // registers are refilled with step s of the next slice: each read is
    // issued a whole slice before its use.  The slice's one barrier follows
    // step 0's instructions.  By then this wave has read all of its slot
    // (that happened during the previous slice), so after the barrier no wave
    // reads the slot any more and the copy of slice t + STAGES may overwrite
    // it (DMA); and with the wait before it, every wave's copy of slice t+1
    // has landed, so slice t+1's fragments may be read (NEXT).  Copies of a
    // slice thus get STAGES - 1 slices to land, as in slice_direct.
    template <bool NEXT, bool DMA>
    __device__ static __forceinline__ void slice_ahead(Acc (&acc)[FM][FN], Frags (&F)[KSUB],
                                                       const TG_LDS char* next_slot, int ahead,
                                                       const CopyTarget& next, const DirectOffsets& off, int wm0,
                                                       int wn0, int lane, int wave) {
        static_assert(NEXT || !DMA, "copies follow the barrier");
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
#pragma unroll
            for (int k = 0; k < NM; ++k) {
                const int i = k / FN, j = k % FN;
                acc[i][j] = mma(F[s].a[i], F[s].b[j], acc[i][j]);
            }
            if constexpr (NEXT) {
                if (s == 0) wait_slice(ahead);
                read_frags(F[s], next_slot, s, wm0, wn0, lane);
            }
            if constexpr (DMA) {
                if (s == 0) issue_direct(next.slot, off, next.ca, next.cb, wave);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Matrix-core K steps of the partial last slice (K - full BK > 0 values).
    __device__ static __forceinline__ int tail_steps(const GemmArgs& g, int full) {
        return (g.K - full * BK + Tr::MK - 1) / Tr::MK;
    }

    // Multiply one slice held in `slot` into the accumulators.  With
    // fragment reuse the reads are software-pipelined one K step ahead
    // (register double buffer, "4.1 CUDA GEMM算子性能优化" section 9.2): the
    // fragments of step s+1 are requested before the matrix-core work of
    // step s, which hides the LDS latency behind it.  (The register-staged
    // loops and the K tail use this; the direct ring's steady state runs
    // slice_direct, which also interleaves the copies.)  `ksteps`: the K
    // steps that hold data (the partial last slice of a K that is not a
    // multiple of BK is zero past K: its remaining K steps would only add
    // zero products, so they are skipped).
    __device__ static __forceinline__ void compute(const TG_LDS char* slot, Acc (&acc)[FM][FN],
                                                   int wm0, int wn0, int lane, int ksteps = KSUB) {
        const TG_LDS char* bslot = slot + A_BYTES;
        if constexpr (FRAG != FR_PER_MMA) {
            Frags f[2];
            read_frags(f[0], slot, 0, wm0, wn0, lane);
#pragma unroll
            for (int s = 0; s < KSUB; ++s) {
                if (s >= ksteps) break;
                if (s + 1 < KSUB && s + 1 < ksteps) read_frags(f[(s + 1) & 1], slot, s + 1, wm0, wn0, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mma(f[s & 1].a[i], f[s & 1].b[j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
            if (s >= ksteps) break;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const i32x4 a = read_a(slot, wm0 + 32 * i, s, lane);
                    const i32x4 b = read_b(bslot, wn0 + 32 * j, s, lane);
                    acc[i][j] = mma(a, b, acc[i][j]);
                }
        }
    }

    // K loop of the register-staged loaders: the `full` whole slices with
    // MODE_A / MODE_B loads, then the partial last slice (if tiles > full)
    // with element loads.  STAGES == 1: load, store, barrier, multiply,
    // barrier.  STAGES == 2: the loads of slice t+1 are issued before the
    // multiply of slice t and written to the other slot after it, one barrier
    // per slice.
    //
    // Shifted pairs need no bounds check on the interior slices 1 .. full-2
    // (a slice is at least 64 bytes of a row, lda >= K, ldb >= N >= 1): an A
    // pair starts at k >= BK, so at least 64 bytes past A's first element,
    // and ends at most 16 bytes past its chunk, whose k < (full-1) BK, so
    // before the end of row m <= M-1 at K; a B pair lies in a row
    // BK <= k < K - BK, at least BK rows (64 bytes) from both ends of B.
    // Only the first and last whole slices take the checked form.
    template <int MODE_A, int MODE_B>
    __device__ static __forceinline__ void staged_loop(Acc (&acc)[FM][FN], TG_LDS char* smem, const GemmArgs& g,
                                                       int m0, int n0, int wm0, int wn0, int lane, int full,
                                                       int tiles) {
        constexpr int EA = edge_mode(MODE_A), EB = edge_mode(MODE_B);
        if constexpr (STAGES == 1) {
            for (int t = 0; t < full; ++t) {
                if (t == 0 || t == full - 1) {
                    Staged<EA, EB> r;
                    load_regs(r, g, m0, n0, t * BK);
                    store_regs(smem, r);
                } else {
                    Staged<MODE_A, MODE_B> r;
                    load_regs(r, g, m0, n0, t * BK);
                    store_regs(smem, r);
                }
                wait_lds_then_barrier();
                compute(smem, acc, wm0, wn0, lane);
                wait_lds_then_barrier();  // all reads done before the next overwrite
            }
            if (full < tiles) {
                Staged<LM_ELEMENT, LM_ELEMENT> r;
                load_regs(r, g, m0, n0, full * BK);
                store_regs(smem, r);
                wait_lds_then_barrier();
                compute(smem, acc, wm0, wn0, lane, tail_steps(g, full));
            }
        } else {
            if (full == 0) {
                if (tiles > 0) {
                    Staged<LM_ELEMENT, LM_ELEMENT> r;
                    load_regs(r, g, m0, n0, 0);
                    store_regs(smem, r);
                    wait_lds_then_barrier();
                    compute(smem, acc, wm0, wn0, lane, tail_steps(g, full));
                }
                return;
            }
            {
                Staged<EA, EB> r;
                load_regs(r, g, m0, n0, 0);
                store_regs(smem, r);
                wait_lds_then_barrier();
            }
            int t = 0;
            for (; t + 2 < full; ++t) {  // loads slices 1 .. full-2
                Staged<MODE_A, MODE_B> r;
                load_regs(r, g, m0, n0, (t + 1) * BK);
                compute(smem + (t & 1) * SLOT, acc, wm0, wn0, lane);
                store_regs(smem + ((t + 1) & 1) * SLOT, r);
                wait_lds_then_barrier();
            }
            if (t + 1 < full) {  // loads the last whole slice
                Staged<EA, EB> r;
                load_regs(r, g, m0, n0, (t + 1) * BK);
                compute(smem + (t & 1) * SLOT, acc, wm0, wn0, lane);
                store_regs(smem + ((t + 1) & 1) * SLOT, r);
                wait_lds_then_barrier();
                ++t;
            }
            if (full < tiles) {  // loads the partial slice
                Staged<LM_ELEMENT, LM_ELEMENT> r;
                load_regs(r, g, m0, n0, full * BK);
                compute(smem + (t & 1) * SLOT, acc, wm0, wn0, lane);
                store_regs(smem + ((t + 1) & 1) * SLOT, r);
                wait_lds_then_barrier();
                ++t;
            }
            compute(smem + (t & 1) * SLOT, acc, wm0, wn0, lane, full < tiles ? tail_steps(g, full) : KSUB);
        }
    }

    template <bool STREAM>
    __device__ static __forceinline__ void store_c(Out* C, const GemmArgs& g, const Acc (&acc)[FM][FN], int r0,
                                                   int c0, int lane, bool inside) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = r0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int col = c0 + 32 * j + (lane & 31);
                    if (inside || (row < g.M && col < g.N)) {
                        Out* dst = &C[(int64_t)row * g.ldc + col];
                        if constexpr (STREAM) __builtin_nontemporal_store(static_cast<Out>(acc[i][j][r]), dst);
                        else *dst = static_cast<Out>(acc[i][j][r]);
                    }
                }
    }

    // CST_SWAP write-back: register r of tile (i, j) in lane l holds row
    // 32 i + l%32, column 32 j + 8 (r/4) + 4 (l/32) + r%4, so registers
    // 4q .. 4q+3 are four consecutive columns of one row: one 16-byte store
    // where C's rows are 16-byte aligned and the tile lies inside C, element
    // stores otherwise.  Each instruction writes 32 bytes of each of 32 rows;
    // the four of one tile complete those rows' 128-byte segments, which the
    // L2 merges before they are written back (plain, not streaming, stores).
    __device__ static __forceinline__ void store_c_swapped(Out* C, const GemmArgs& g, const Acc (&acc)[FM][FN],
                                                           int r0, int c0, int lane, bool inside) {
        const bool vec = inside && (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = r0 + 32 * i + (lane & 31);
                    const int col = c0 + 32 * j + 8 * q + 4 * (lane >> 5);
                    Out* dst = &C[(int64_t)row * g.ldc + col];
                    if (vec) {
                        *reinterpret_cast<Out4*>(dst) = Out4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                             acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (row < g.M && col + e < g.N) dst[e] = static_cast<Out>(acc[i][j][4 * q + e]);
                    }
                }
    }

    // Wait until at most `ahead` slices' copies (issued after the one needed
    // next) are still in flight, then barrier.  The wait count is an
    // immediate, so the runtime `ahead` (0 .. STAGES-2) selects among
    // compile-time instances.
    template <int A>
    __device__ static __forceinline__ void wait_ahead(int ahead) {
        if constexpr (A > 0) {
            if (ahead >= A) {
                wait_vm_then_barrier<A * N_LD>();
                return;
            }
            wait_ahead<A - 1>(ahead);
        } else {
            wait_vm_then_barrier<0>();
        }
    }

    __device__ static __forceinline__ void wait_slice(int ahead) {
        wait_ahead<(STAGES > 2 ? STAGES - 2 : 0)>(ahead);
    }

    __device__ static __forceinline__ void run(const GemmArgs& g) {
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
        TG_LDS char* smem = (TG_LDS char*)(smem_raw);
        ClockMark clk;
        clk.start(g.clocks);

        const int lane = lane_id();
        const int wave = wave_id();
        int tm, tn;
        tile_of_workgroup(g, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int wm0 = (wave / WAVES_N) * WTM;
        const int wn0 = (wave % WAVES_N) * WTN;

        Acc acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

        const int tiles = (g.K + BK - 1) / BK;
        // slices with no K tail; for the direct copy, with B's rows ending in
        // a partial chunk (b_guard) and K a whole number of slices, all but
        // the last: that slice holds B's last row, whose chunk across N a
        // copy would read past the end of B, so it goes through the register
        // tail (element loads) like a partial slice
        const int full = g.K / BK - ((DIRECT && g.b_guard && g.K % BK == 0 && g.K > 0) ? 1 : 0);

        // REM: this lane's row of the remainder column and its partial sum
        Out racc = Out(0);
        const bool rem_rows = REM && wave < 2 && tn * 16 < BM;  // wave-uniform
        const int rt = tn * 16 + wave * 8 + (lane >> 3);
        auto rem_at = [&](const TG_LDS char* slot) {
            if constexpr (REM) {
                if (rem_rows) rem_slice(slot, racc, rt, lane);
            }
        };

        if constexpr (DIRECT) {
            DirectOffsets off;
            direct_offsets(off, g, m0, n0);
            // wave-uniform byte addresses of slice 0 of this tile's A rows / B columns
            const char* abase = static_cast<const char*>(g.A) + (int64_t)m0 * g.lda * ESZ;
            const char* bbase = static_cast<const char*>(g.B) + (int64_t)n0 * ESZ;
            const int64_t astep = (int64_t)BK * ESZ;          // A base advance per slice
            const int64_t bstep = (int64_t)BK * g.ldb * ESZ;  // B base advance per slice
            // REM: slice 0's B rows at the dword that ends at column g.N
            const char* cbase = static_cast<const char*>(g.B) + (int64_t)(g.N + 1 - CPD) * ESZ;
            auto issue_slice = [&](int sl) {
                issue_direct(smem + (sl % STAGES) * SLOT, off, abase + sl * astep, bbase + sl * bstep, wave);
                issue_rem(smem + (sl % STAGES) * SLOT, off, cbase + sl * bstep, wave);
            };
            if constexpr (STAGES == 1) {
                // One slot: the copy of slice t+1 may only start once every
                // wave has finished reading slice t, so nothing overlaps -
                // the asynchronous copy without a second buffer.
                for (int t = 0; t < full; ++t) {
                    issue_slice(t);
                    wait_all_then_barrier();
                    compute(smem, acc, wm0, wn0, lane);
                    wait_lds_then_barrier();
                }
                if (full < tiles) {
                    Staged<LM_ELEMENT, LM_ELEMENT> r;
                    load_regs(r, g, m0, n0, full * BK);
                    store_regs(smem, r);
                    wait_lds_then_barrier();
                    compute(smem, acc, wm0, wn0, lane, tail_steps(g, full));
                }
            } else if constexpr (FRAG == FR_SLICE) {
            // Prologue as below, then all of slice 0's fragments; slice t
            // reads slice t+1's fragments and starts slice t + STAGES.
            auto target = [&](int sl) {
                return CopyTarget{smem + (sl % STAGES) * SLOT, abase + sl * astep, bbase + sl * bstep,
                                  cbase + sl * bstep};
            };
            const CopyTarget none{smem, abase, bbase, cbase};
            Frags F[KSUB];
#pragma unroll
            for (int s = 0; s < STAGES - 1; ++s)
                if (s < full) issue_slice(s);
            if (full > 0) {
                wait_slice(min(STAGES - 2, full - 1));
                if (STAGES - 1 < full) issue_slice(STAGES - 1);
#pragma unroll
                for (int s = 0; s < KSUB; ++s) read_frags(F[s], smem, s, wm0, wn0, lane);
            }
            int t = 0;
            for (; t + STAGES < full; ++t)
                slice_ahead<true, true>(acc, F, smem + ((t + 1) % STAGES) * SLOT, STAGES - 2, target(t + STAGES),
                                        off, wm0, wn0, lane, wave);
            for (; t + 1 < full; ++t)
                slice_ahead<true, false>(acc, F, smem + ((t + 1) % STAGES) * SLOT, min(STAGES - 2, full - 2 - t),
                                         none, off, wm0, wn0, lane, wave);
            if (t < full) slice_ahead<false, false>(acc, F, smem, 0, none, off, wm0, wn0, lane, wave);
            if (full < tiles) {
                // K tail into slot full % STAGES.  Every wave passed the last
                // barrier (in slice full-2; with one full slice, the
                // prologue's), by which all had finished reading that slot,
                // and its wait drained the copies; the last slice reads no
                // LDS.
                Staged<LM_ELEMENT, LM_ELEMENT> r;
                load_regs(r, g, m0, n0, full * BK);
                store_regs(smem + (full % STAGES) * SLOT, r);
                wait_lds_then_barrier();
                compute(smem + (full % STAGES) * SLOT, acc, wm0, wn0, lane, tail_steps(g, full));
            }
            } else {
            // Prologue: slices 0 .. STAGES-2 in flight; once slice 0 is in
            // LDS (barrier), start slice STAGES-1 and read the fragments of
            // slice 0's first K step.
            Frags f[2];
#pragma unroll
            for (int s = 0; s < STAGES - 1; ++s)
                if (s < full) issue_slice(s);
            if (full > 0) {
                wait_slice(min(STAGES - 2, full - 1));
                if (STAGES - 1 < full) issue_slice(STAGES - 1);
                read_frags(f[0], smem, 0, wm0, wn0, lane);
            }
            // Steady state.  Slice t is multiplied from slot t % STAGES with
            // the fragment reads one K step ahead.  The single barrier of the
            // slice sits inside its last K step: by then this wave's reads of
            // the slot are complete, so after the barrier (a) no wave reads
            // the slot any more and the copy of slice t+STAGES may overwrite
            // it, and (b) every wave's copy of slice t+1 has landed, so the
            // first fragments of slice t+1 are read while the last K step of
            // slice t still runs on the matrix cores.
            // With SPREAD, part 2 of slice t + STAGES - 1's copies is issued
            // during slice t; slice STAGES - 1 was issued whole above.
            auto target = [&](int sl) {
                return CopyTarget{smem + (sl % STAGES) * SLOT, abase + sl * astep, bbase + sl * bstep,
                                  cbase + sl * bstep};
            };
            const CopyTarget none{smem, abase, bbase, cbase};
            int t = 0;
            if (STAGES < full) {
                rem_at(smem);
                slice_direct<false, true, true>(acc, f, smem, smem + SLOT, STAGES - 2, none, target(STAGES), off,
                                                wm0, wn0, lane, wave);
                for (t = 1; t + STAGES < full; ++t) {
                    rem_at(smem + (t % STAGES) * SLOT);
                    slice_direct<SPREAD, true, true>(acc, f, smem + (t % STAGES) * SLOT,
                                                     smem + ((t + 1) % STAGES) * SLOT, STAGES - 2,
                                                     target(t + STAGES - 1), target(t + STAGES), off, wm0, wn0,
                                                     lane, wave);
                }
                // the last slice whose part 2 is still to be issued
                // (t + STAGES == full, so t + 1 < full)
                if constexpr (SPREAD) {
                    slice_direct<true, true, false>(acc, f, smem + (t % STAGES) * SLOT,
                                                    smem + ((t + 1) % STAGES) * SLOT, STAGES - 2,
                                                    target(t + STAGES - 1), none, off, wm0, wn0, lane, wave);
                    ++t;
                }
            }
            for (; t + 1 < full; ++t) {
                rem_at(smem + (t % STAGES) * SLOT);
                slice_direct<false, true, false>(acc, f, smem + (t % STAGES) * SLOT, smem + ((t + 1) % STAGES) * SLOT,
                                                 min(STAGES - 2, full - 2 - t), none, none, off, wm0, wn0, lane,
                                                 wave);
            }
            if (t < full) {
                rem_at(smem + (t % STAGES) * SLOT);
                slice_direct<false, false, false>(acc, f, smem + (t % STAGES) * SLOT, smem, 0, none, none, off, wm0,
                                                  wn0, lane, wave);
            }
            if (full < tiles) {
                // K tail: element loads with zero fill into slot full % STAGES.
                // No copy is in flight (the last wait drained them) and every
                // wave passed the barrier that ended its reads of that slot.
                Staged<LM_ELEMENT, LM_ELEMENT> r;
                load_regs(r, g, m0, n0, full * BK);
                store_regs(smem + (full % STAGES) * SLOT, r);
                fill_rem(smem + (full % STAGES) * SLOT, g, full * BK, wave, lane);
                wait_lds_then_barrier();
                rem_at(smem + (full % STAGES) * SLOT);
                compute(smem + (full % STAGES) * SLOT, acc, wm0, wn0, lane, tail_steps(g, full));
            }
            }
        } else {
            // register-staged loaders: the kernel's own pair of load modes
            staged_loop<(SHIFT & 1) ? LM_SHIFTED : LM_ALIGNED, (SHIFT & 2) ? LM_SHIFTED : LM_ALIGNED>(
                acc, smem, g, m0, n0, wm0, wn0, lane, full, tiles);
        }

        // Epilogue: accumulators -> C.  Register r of tile (i, j) in lane l is
        // row 8 (r/4) + 4 (l/32) + r%4, column l%32 of that 32 x 32 tile, so
        // each store instruction writes two 128-byte row segments.  C is
        // written once and never re-read here: when its rows are 128-byte
        // aligned each segment is one whole cache line and, for a long K
        // loop (g.c_stream, set by the host), the stores are non-temporal;
        // otherwise ordinary stores, which drain a large C faster where the
        // write is a big share of the launch, and where every segment
        // straddles two lines let the L2 merge the halves before they reach
        // HBM (about 20 % faster than streaming the partial lines at 4096^3).
        clk.loop_end(g.clocks);
        Out* C = static_cast<Out*>(g.C);
        const bool inside = (m0 + BM <= g.M) && (n0 + BN <= g.N);
        if constexpr (CST == CST_SWAP) {
            store_c_swapped(C, g, acc, m0 + wm0, n0 + wn0, lane, inside);
        } else {
            if (g.c_stream) store_c<true>(C, g, acc, m0 + wm0, n0 + wn0, lane, inside);
            else store_c<false>(C, g, acc, m0 + wm0, n0 + wn0, lane, inside);
        }
        if constexpr (REM) {
            if (rem_rows) {
#pragma unroll
                for (int o = 1; o < 8; o <<= 1) racc += __shfl_xor(racc, o, 64);
                if ((lane & 7) == 0 && m0 + rt < g.M) C[(int64_t)(m0 + rt) * g.ldc + g.N] = racc;
            }
        }
        clk.finish(g.clocks);
    }
};

}  // namespace tg
