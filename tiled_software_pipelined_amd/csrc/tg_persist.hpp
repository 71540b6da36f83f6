// Persistent matrix-core GEMM whose C write-back overlaps the next tile's
// K loop (bf16 -> fp32, int8 -> int32).
//
// The tiled kernel of tg_mfma.hpp gives each workgroup one C tile and writes
// the tile only after its K loop: when the grid is one round of tiles (or
// K is short) every compute unit stores at the same moment and nothing
// overlaps the write.  The "流水化 GPU 内核" skill (Step 3: prologue, steady
// loop, epilogue) and "4.1 CUDA GEMM算子性能优化" (section 10: the
// asynchronous multi-stage copy) overlap the loads of later slices with the
// work on the current one; this kernel applies the same idea to the epilogue.
//
//   * One workgroup per compute unit loops over several tiles.  Round r of
//     the grid takes tiles [r G, r G + G) of the grouped tile order, each
//     XCD a contiguous run of them (the hardware hands workgroup b to XCD
//     b mod 8), so that the tiles one XCD works on at once share A row and
//     B column panels in its L2.
//   * The slices of all the workgroup's tiles form one stream: the direct
//     global->LDS copy ring (2 slots) runs on across tile boundaries, so a
//     new tile starts with its first slices already in LDS.
//   * Two accumulator sets alternate between tiles.  While tile j
//     accumulates into one set, the other set, tile j-1's finished C
//     block, is written out: CSL of tile j's first slices each issue
//     NSTORE / CSL of its 16-byte stores, interleaved with the matrix
//     instructions like the copies and the fragment reads.  Only the last
//     tile's write is left after the loop.
//
// Stores and loads share one in-order counter of outstanding vector memory
// instructions (vmcnt).  The ring's wait at the end of slice u needs the
// copies of slice u+1, which were issued at the end of slice u-1; the only
// memory instructions issued after them are slice u's stores, so the wait
// is vmcnt(stores of slice u) and the stores stay in flight.
//
// Scope: whole tiles only (M % BM, N % BN, K % BK all zero), 16-byte
// aligned operand rows (the direct loader), at least CSL + 2 slices per
// tile, so that no store slice is one of the stream's last two; the host
// checks all of it.  C is written with 16-byte stores when its rows are
// 16-byte aligned, else with 4-byte stores (more store instructions: the
// ring's waits then only wait longer).
#pragma once

#include "tg_mfma.hpp"

namespace tg {

template <class Tr, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int CSL>
struct PersistGemm {
    typedef MfmaGemm<Tr, BM, BN, BK, WAVES_M, WAVES_N, 2, LD_DIRECT, LY_XOR, AC_WIDE, FR_REUSE, 0, CST_SWAP> Base;
    typedef typename Base::Acc Acc;
    typedef typename Base::Out Out;
    typedef typename Base::Out4 Out4;
    typedef typename Base::Frags Frags;
    typedef typename Base::DirectOffsets DirectOffsets;
    typedef typename Base::CopyTarget CopyTarget;

    static constexpr int NT = Base::NT;
    static constexpr int ESZ = Base::ESZ;
    static constexpr int SLOT = Base::SLOT;
    static constexpr int LDS_BYTES = Base::LDS_BYTES;
    static constexpr int N_LD = Base::N_LD;
    static constexpr int FM = Base::FM, FN = Base::FN;
    static constexpr int NM = Base::NM, NR = Base::NR;
    static constexpr int KSUB = Base::KSUB;
    static constexpr int WTM = Base::WTM, WTN = Base::WTN;
    static constexpr int FREAD = Base::FREAD;
    static constexpr int NSTORE = FM * FN * 4;  // 16-byte stores per lane per tile
    static constexpr int SPS = NSTORE / CSL;    // stores per store slice
    static constexpr int MIN_SLICES = CSL + 2;  // slices per tile the kernel needs

    static_assert(NSTORE % CSL == 0, "whole stores per slice");
    static_assert(KSUB >= 2, "stores go in K steps 0 .. KSUB-2 of a slice");
    static_assert(SPS <= 63, "vmcnt range");

    // Where the previous tile's C block goes: lane l's first element
    // (row m0 + wm0 + l%32, column n0 + wn0 + 4 (l/32)) and C's row stride.
    struct StoreTarget {
        Out* p;
        int64_t ldc;
        bool vec;  // 16-byte stores (C rows 16-byte aligned)
    };

    // Store n (0 <= n < NSTORE) of a lane's tile: matrix tile (i, j) =
    // (n / (4 FN), (n / 4) % FN), registers 4q .. 4q+3 with q = n % 4: row
    // 32 i + l%32, columns 32 j + 8 q + 4 (l/32) .. +3 of the wave's block
    // (the swapped product's layout, as MfmaGemm::store_c_swapped).
    __device__ static __forceinline__ void store_one(const Acc (&acc)[FM][FN], const StoreTarget& st, int n) {
        const int i = n / (4 * FN), j = (n / 4) % FN, q = n % 4;
        Out* dst = st.p + (int64_t)(32 * i) * st.ldc + 32 * j + 8 * q;
        if (st.vec) {
            *reinterpret_cast<Out4*>(dst) =
                Out4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = static_cast<Out>(acc[i][j][4 * q + e]);
        }
    }

    // K steps S .. KSUB-1 of one slice from `cur`, fragment reads one step
    // ahead.  Stores [ST0, ST0 + NST) of `prev` are spread over steps 0 ..
    // KSUB-2.  NEXT: another slice follows: in the last step wait until only
    // this slice's NST stores may still be in flight (so the next slice's
    // copies have landed), barrier, read the next slice's first fragments
    // from `nxt`.  DMA: then issue the copies of the slice two ahead into
    // `ct` (the slot this slice leaves).
    template <int S, bool NEXT, bool DMA, int NST, int ST0>
    __device__ static __forceinline__ void steps(Acc (&acc)[FM][FN], const Acc (&prev)[FM][FN], Frags (&f)[2],
                                                 const TG_LDS char* cur, const TG_LDS char* nxt,
                                                 const CopyTarget& ct, const DirectOffsets& off,
                                                 const StoreTarget& st, int wm0, int wn0, int lane, int wave) {
        constexpr bool LAST = S == KSUB - 1;
        constexpr int SB = LAST ? 0 : ST0 + (S * NST) / (KSUB - 1);
        constexpr int SE = LAST ? 0 : ST0 + ((S + 1) * NST) / (KSUB - 1);
        constexpr bool READS = !LAST || NEXT;
        constexpr bool BARRIER = LAST && NEXT;
        constexpr int NCOPY = (LAST && DMA) ? N_LD : 0;
        constexpr int BAR_K = (BARRIER && NM >= 8) ? 1 : 0;
        constexpr int NREAD = READS ? NR : 0;
        constexpr int TOTAL = NREAD + NCOPY + (SE - SB);
        static_assert(!DMA || NEXT, "copies follow the barrier");
        const TG_LDS char* rslot = LAST ? nxt : cur;
        const int rs = LAST ? 0 : S + 1;
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const int i = k / FN, j = k % FN;
            acc[i][j] = Base::mma(f[S & 1].a[i], f[S & 1].b[j], acc[i][j]);
            if (BARRIER && k == BAR_K) wait_vm_then_barrier<NST>();
#pragma unroll
            for (int m = Base::mem_begin(k, BAR_K, TOTAL); m < Base::mem_begin(k + 1, BAR_K, TOTAL); ++m) {
                if (m < NREAD) Base::read_op(f[(S + 1) & 1], rslot, rs, m, wm0, wn0, lane);
                else if (m < NREAD + NCOPY) Base::issue_direct_one(m - NREAD, ct.slot, off, ct.ca, ct.cb, wave);
                else store_one(prev, st, SB + (m - NREAD - NCOPY));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!LAST)
            steps<S + 1, NEXT, DMA, NST, ST0>(acc, prev, f, cur, nxt, ct, off, st, wm0, wn0, lane, wave);
    }

    // The workgroup's walk over its tiles and its copy stream.
    struct Walk {
        int G, base, tiles;      // grid, the workgroup's first tile ordinal, its tile count
        int slices;              // slices per tile (K / BK)
        // copy stream: the next slice to copy
        int cj, cp;              // its tile (0 .. tiles-1) and slice within the tile
        const char* ca;          // wave-uniform A / B addresses of slice (cj, 0)
        const char* cb;
    };

    // Tile (tm, tn) of ordinal r of this workgroup: the tile order of
    // tile_of_workgroup (groups of wg_group tile rows, column by column) on
    // the index r G + (XCD-major rank of the workgroup).
    __device__ static __forceinline__ void tile_of(const GemmArgs& g, const Walk& w, int r, int& m0, int& n0) {
        const int v = r * w.G + w.base;
        int tm, tn;
        if (g.wg_group <= 0) {
            tm = v / g.tiles_n;
            tn = v - tm * g.tiles_n;
        } else {
            const int per_group = g.wg_group * g.tiles_n;
            const int group = v / per_group;
            const int first_m = group * g.wg_group;
            const int rows = min(g.tiles_m - first_m, g.wg_group);
            const int in_group = v - group * per_group;
            tm = first_m + in_group % rows;
            tn = in_group / rows;
        }
        m0 = tm * BM;
        n0 = tn * BN;
    }

    __device__ static __forceinline__ void copy_tile_bases(const GemmArgs& g, Walk& w) {
        int m0, n0;
        tile_of(g, w, w.cj, m0, n0);
        w.ca = static_cast<const char*>(g.A) + (int64_t)m0 * g.lda * ESZ;
        w.cb = static_cast<const char*>(g.B) + (int64_t)n0 * ESZ;
    }

    // The copy target of the stream's next slice, into `slot`; advances the
    // stream (the caller only asks while slices are left).
    __device__ static __forceinline__ CopyTarget next_copy(const GemmArgs& g, Walk& w, TG_LDS char* slot) {
        const CopyTarget t{slot, w.ca + (int64_t)w.cp * BK * ESZ, w.cb + (int64_t)w.cp * BK * g.ldb * ESZ};
        if (++w.cp == w.slices) {
            w.cp = 0;
            if (++w.cj < w.tiles) copy_tile_bases(g, w);
        }
        return t;
    }

    __device__ static __forceinline__ void zero(Acc (&acc)[FM][FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    }

    // One slice of the stream (u = its index, `total` slices in all): the
    // copies of slice u+2 go into slice u's slot.
    template <bool NEXT, bool DMA, int NST, int ST0>
    __device__ static __forceinline__ void slice(Acc (&acc)[FM][FN], const Acc (&prev)[FM][FN], Frags (&f)[2],
                                                 TG_LDS char* smem, int u, const GemmArgs& g, Walk& w,
                                                 const DirectOffsets& off, const StoreTarget& st, int wm0,
                                                 int wn0, int lane, int wave) {
        TG_LDS char* cur = smem + (u & 1) * SLOT;
        TG_LDS char* nxt = smem + ((u + 1) & 1) * SLOT;
        CopyTarget ct{cur, nullptr, nullptr};
        if constexpr (DMA) ct = next_copy(g, w, cur);
        steps<0, NEXT, DMA, NST, ST0>(acc, prev, f, cur, nxt, ct, off, st, wm0, wn0, lane, wave);
    }

    // Store slices c .. CSL-1 of a tile (unrolled: each writes its own
    // compile-time range of `prev`).  Never among the stream's last two
    // slices (slices per tile >= CSL + 2).
    template <int CS>
    __device__ static __forceinline__ void store_slices(Acc (&acc)[FM][FN], const Acc (&prev)[FM][FN],
                                                        Frags (&f)[2], TG_LDS char* smem, int& u,
                                                        const GemmArgs& g, Walk& w, const DirectOffsets& off,
                                                        const StoreTarget& st, int wm0, int wn0, int lane,
                                                        int wave) {
        if constexpr (CS < CSL) {
            slice<true, true, SPS, CS * SPS>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
            ++u;
            store_slices<CS + 1>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
        }
    }

    // One tile into `acc`; STORES: `prev` holds the previous tile, written
    // to `st` during the first CSL slices.
    template <bool STORES>
    __device__ static __forceinline__ void tile(Acc (&acc)[FM][FN], const Acc (&prev)[FM][FN], Frags (&f)[2],
                                                TG_LDS char* smem, int& u, int total, const GemmArgs& g, Walk& w,
                                                const DirectOffsets& off, const StoreTarget& st, int wm0,
                                                int wn0, int lane, int wave) {
        zero(acc);
        int p = 0;
        if constexpr (STORES) {
            store_slices<0>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
            p = CSL;
        }
        for (; p < w.slices; ++p, ++u) {
            if (u + 2 < total)
                slice<true, true, 0, 0>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
            else if (u + 1 < total)
                slice<true, false, 0, 0>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
            else
                slice<false, false, 0, 0>(acc, prev, f, smem, u, g, w, off, st, wm0, wn0, lane, wave);
        }
    }

    __device__ static __forceinline__ StoreTarget target_of(const GemmArgs& g, int m0, int n0, int wm0, int wn0,
                                                            int lane) {
        Out* C = static_cast<Out*>(g.C);
        const bool vec = (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
        return StoreTarget{C + (int64_t)(m0 + wm0 + (lane & 31)) * g.ldc + n0 + wn0 + 4 * (lane >> 5), g.ldc, vec};
    }

    __device__ static __forceinline__ void store_all(const Acc (&acc)[FM][FN], const StoreTarget& st) {
#pragma unroll
        for (int n = 0; n < NSTORE; ++n) store_one(acc, st, n);
    }

    __device__ static __forceinline__ void run(const GemmArgs& g) {
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
        TG_LDS char* smem = (TG_LDS char*)(smem_raw);
        ClockMark clk;
        clk.start(g.clocks);

        const int lane = lane_id();
        const int wave = wave_id();
        const int wm0 = (wave / WAVES_N) * WTM;
        const int wn0 = (wave % WAVES_N) * WTN;

        Walk w;
        w.G = gridDim.x;
        const int b = blockIdx.x;
        // XCD-major rank: the G/8 workgroups of one XCD take consecutive
        // ordinals of each round
        w.base = (w.G & 7) == 0 ? (b & 7) * (w.G >> 3) + (b >> 3) : b;
        const int ntiles = g.tiles_m * g.tiles_n;
        w.tiles = w.base < ntiles ? (ntiles - w.base + w.G - 1) / w.G : 0;
        w.slices = g.K / BK;
        const int total = w.tiles * w.slices;
        if (total > 0) {
            // whole tiles: every lane's copy offsets are those of tile (0, 0)
            DirectOffsets off;
            Base::direct_offsets(off, g, 0, 0);
            w.cj = 0;
            w.cp = 0;
            copy_tile_bases(g, w);
            Frags f[2];
            {
                // prologue: slices 0 and 1 (both in tile 0) in flight; wait
                // for slice 0 and read its first fragments
                const CopyTarget c0 = next_copy(g, w, smem);
                Base::issue_direct(c0.slot, off, c0.ca, c0.cb, wave);
                const CopyTarget c1 = next_copy(g, w, smem + SLOT);
                Base::issue_direct(c1.slot, off, c1.ca, c1.cb, wave);
                wait_vm_then_barrier<N_LD>();
                Base::read_frags(f[0], smem, 0, wm0, wn0, lane);
            }
            Acc acc0[FM][FN], acc1[FM][FN];
            int u = 0;
            int m0, n0;
            tile_of(g, w, 0, m0, n0);
            StoreTarget st = target_of(g, m0, n0, wm0, wn0, lane);
            tile<false>(acc0, acc1, f, smem, u, total, g, w, off, st, wm0, wn0, lane, wave);
            // tile j into acc1 while acc0 (tile j-1) is written, then tile
            // j+1 into acc0 while acc1 is written (one instance of each)
            bool last_in_acc1 = false;
            for (int j = 1; j < w.tiles; j += 2) {
                tile<true>(acc1, acc0, f, smem, u, total, g, w, off, st, wm0, wn0, lane, wave);
                tile_of(g, w, j, m0, n0);
                st = target_of(g, m0, n0, wm0, wn0, lane);
                if (j + 1 == w.tiles) {
                    last_in_acc1 = true;
                    break;
                }
                tile<true>(acc0, acc1, f, smem, u, total, g, w, off, st, wm0, wn0, lane, wave);
                tile_of(g, w, j + 1, m0, n0);
                st = target_of(g, m0, n0, wm0, wn0, lane);
            }
            clk.loop_end(g.clocks);
            if (last_in_acc1) store_all(acc1, st);
            else store_all(acc0, st);
        } else {
            clk.loop_end(g.clocks);
        }
        clk.finish(g.clocks);
    }
};

}  // namespace tg
