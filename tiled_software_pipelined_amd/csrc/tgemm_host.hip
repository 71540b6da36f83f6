// libtgemm host side: plans, variant registry, launch (the C ABI of
// include/tgemm.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tg_args.hpp"
#include "tg_pack.hpp"
#include "tgemm.h"

using tg::KernelEntry;

struct tgemm_plan {
    int64_t M, N, K, lda, ldb, ldc;
    int32_t dtype;
    const KernelEntry* entry;        // what runs when the operands allow it
    const KernelEntry* fallback[4];  // by misaligned operands (bit 0 A, bit 1 B); [0] = entry
    int32_t wg_group;
    int32_t a_guard, b_guard;     // leading-dimension based (pointer alignment is checked per run)
    int64_t n_main;               // columns the entry's grid covers (N unless split)
    tgemm_plan* rem;              // split plans: the last N - n_main columns (thin kernel), else NULL
    bool rem_fused;               // split plans with one last column: the entry's REM twin computes
                                  // it in the main K loop (`rem` is kept for a fallback kernel)
    tgemm_plan* packed;           // default plans: the same product on operands repacked with
                                  // 16-byte aligned rows (gemm_run_ws), else NULL
    int64_t lda_p, ldb_p;         // leading dimensions of `packed`
};

namespace {

thread_local std::string g_err;

void set_err(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

std::vector<KernelEntry> g_reg[3];
std::once_flag g_reg_once;

void add_entry(const KernelEntry& e) { g_reg[e.dtype].push_back(e); }

void init_registry() {
    std::call_once(g_reg_once, [] {
        tg::register_f32(add_entry);
        tg::register_bf16(add_entry);
        tg::register_i8(add_entry);
    });
}

int elem_size(int dtype) { return dtype == TGEMM_F32 ? 4 : dtype == TGEMM_BF16 ? 2 : 1; }

// Width of an entry's unguarded global loads (0: it only does element loads).
int access_bytes(const KernelEntry& e) { return e.gload_bytes; }

// Kernels whose 16-byte reads take any byte address: the direct loader (the
// global -> LDS copy reads 16 bytes from any address, at the full rate of an
// aligned one) and the thin kernel (plain 16-byte loads, which gfx950 serves
// at any address too).  Only element alignment of the pointers is needed.
bool any_alignment(const KernelEntry& e) { return e.loader == tg::LD_DIRECT || e.family == tg::FAM_THIN; }

// Leading-dimension checks: can every row of the operand be read with
// `bytes`-wide aligned accesses?  (Pointer alignment is checked at run time.)
void ld_guards(const KernelEntry& e, int64_t N, int64_t lda, int64_t ldb, int32_t* ga, int32_t* gb) {
    const int bytes = access_bytes(e);
    if (bytes == 0) {
        *ga = *gb = 0;
        return;
    }
    const int esz = elem_size(e.dtype);
    const int per = bytes / esz;  // elements per access
    if (e.family == tg::FAM_THIN) {
        // the matrix-core thin kernel reads pieces of e.bn columns from every
        // B row but the last (which it loads by element): they stay within
        // the matrix when e.bn <= ldb + N, reaching at most into the next
        // row (the vector one reads B by element)
        *ga = 0;
        *gb = e.thin_mma && e.bn > ldb + N;
        return;
    }
    if (any_alignment(e)) {
        // rows of any alignment; the last chunk of a B row must still end at N
        *ga = 0;
        *gb = N % per != 0 || N < per;
        return;
    }
    *ga = (lda * esz) % bytes != 0;
    *gb = (ldb * esz) % bytes != 0 || N % per != 0 || N < per;
}

// Does entry e need 16-byte aligned operand pointers?
bool needs_aligned_ptrs(const KernelEntry& e) { return access_bytes(e) != 0 && !any_alignment(e); }

// The direct loader addresses each lane's 16 bytes as a wave-uniform base
// plus a 32-bit byte offset from the slice's first row: up to (BM-1)*lda
// elements into A and (BK-1)*ldb + BN into B.  Larger leading dimensions
// need a register-staged kernel (64-bit addresses).
bool direct_fits(const KernelEntry& e, int64_t lda, int64_t ldb) {
    if (e.loader != tg::LD_DIRECT) return true;
    const int64_t esz = elem_size(e.dtype);
    const int64_t lim = INT64_C(0xffffffff);
    return ((int64_t)(e.bm - 1) * lda + e.bk) * esz <= lim && ((int64_t)(e.bk - 1) * ldb + e.bn) * esz <= lim;
}

bool field_ok(int want, int have) { return want == 0 || want == have; }

bool matches(const KernelEntry& e, const tgemm_variant& v) {
    if (v.kernel == TGEMM_KERNEL_NAIVE && e.family != tg::FAM_NAIVE) return false;
    if (v.kernel == TGEMM_KERNEL_TILED && e.family != tg::FAM_TILED) return false;
    return field_ok(v.tile_m, e.bm) && field_ok(v.tile_n, e.bn) && field_ok(v.tile_k, e.bk) &&
           field_ok(v.stages, e.stages) && field_ok(v.loader, e.loader) &&
           field_ok(v.lds_layout, e.layout) && field_ok(v.access, e.access) && field_ok(v.frag, e.frag) &&
           field_ok(v.waves_m, e.wm) && field_ok(v.waves_n, e.wn) && field_ok(v.store, e.store) &&
           field_ok(v.copy_sched, e.copy_sched) && field_ok(v.frag_read, e.frag_read) &&
           field_ok(v.lane_map, e.lane_map);
}

const KernelEntry* find_entry(int dtype, const tgemm_variant& v) {
    for (const KernelEntry& e : g_reg[dtype])
        if (e.listed && matches(e, v)) return &e;
    return nullptr;
}

// Can entry e run an N-column product whose operands need these guards (ga:
// A rows not 16-byte aligned, gb: B rows not aligned or N not a whole
// number of 16-byte pieces)?  The direct loader takes the partial piece of
// N but needs at least one whole piece per row.
bool accepts(const KernelEntry& e, bool ga, bool gb, int64_t N) {
    if (gb && e.loader == tg::LD_DIRECT && N * elem_size(e.dtype) < 16) return false;
    return (!ga || (e.shift_mask & 1)) && (!gb || (e.shift_mask & 2));
}

// Default choice for a shape.  Small problems (fewer than half a workgroup
// per compute unit on 256 x 256 tiles, or short K) take 128 x 128 and then
// 64 x 64 tiles.  Otherwise the 8-wave 256 x 256 tile and the 128 x 128 tile
// compete on a time model fitted to interleaved runs of both at six
// aligned shapes and two with unaligned B rows (within about 5 %), in units
// of one full round of 256 x 256 tiles:
//  - 256 x 256 (one workgroup per compute unit): whole rounds of 256
//    workgroups, plus a partial last round of f x 256 workgroups that
//    takes 0.62 + 0.38 f of a full one (the idle units leave clock and
//    memory bandwidth to the busy ones: measured 0.65 at f = 1/16, 0.82 at
//    f = 9/16);
//  - 128 x 128 (three per unit): ceil(tiles / 256) tiles on the busiest
//    unit, each `mid_tile` of a 256 x 256 round.
// So 4096 x 4096 keeps 256 x 256 (1 vs 4 x 0.33) and 4096 x 4352 (272 big
// tiles, 1088 small ones) takes 128 x 128 (1.64 vs 5 x 0.33).  Products
// of at most 16 columns (bf16, int8) take the thin kernels.  With
// `guarded` (the fallback choice for operands the direct loader cannot take:
// leading dimensions beyond its 32-bit offsets) the candidates are the
// register-staged tiles.  Short K also takes 128 x 128: with one
// round of 256 x 256 tiles every workgroup writes its C tile at the same
// moment, unoverlapped, and at short K that write is most of the work.
double big_rounds(int64_t tiles) {
    const int64_t full = tiles / 256, rest = tiles % 256;
    return (double)full + (rest ? 0.62 + 0.38 * (double)rest / 256.0 : 0.0);
}

// Time of entry e on an M x N grid in units of one full round of the
// 256 x 256 direct tile (the same model; register-staged rounds are 1.9
// times as long: 212 vs 112 us at 4096^3), or a negative value where the
// model does not apply (other tiles).
double model_rounds(const KernelEntry& e, int64_t M, int64_t N) {
    if (e.family != tg::FAM_TILED) return -1.0;
    const bool staged = e.loader == tg::LD_VGPR;
    const double round = staged ? 1.9 : 1.0;
    const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    if (e.bm == 256 && e.bn == 256) return round * big_rounds(tiles);
    if (e.bm == 128 && e.bn == 128) {
        const double mid = staged ? 0.26 : (e.dtype == TGEMM_I8 ? 0.31 : 0.325);
        return round * mid * (double)((tiles + 255) / 256);
    }
    return -1.0;
}

const KernelEntry* default_entry(int dtype, int64_t M, int64_t N, int64_t K, int64_t ldb, bool guarded) {
    tgemm_variant v{};
    v.kernel = TGEMM_KERNEL_TILED;
    auto wgs = [&](int t) { return ((M + t - 1) / t) * ((N + t - 1) / t); };
    if (dtype == TGEMM_F32) {
        // One 128 x 128 tile per compute unit or fewer: 64 x 64 tiles, four
        // times the workgroups.  A wave's time on the vector ALUs is its
        // count of FMAs, so spreading the product over more SIMDs is what
        // pays: 1024^3 60 vs 154 us, 256^3 17 vs 42, 2048^3 239 vs 308;
        // 4096^3 stays on 128 x 128 (1565 vs 1745).
        if (wgs(128) <= 256) v.tile_m = v.tile_n = 64;
        return find_entry(dtype, v);
    }
    v.access = TGEMM_ACCESS_WIDE;
    v.frag = TGEMM_FRAG_REUSE;
    v.lds_layout = TGEMM_LDS_XOR;
    v.waves_m = 2;
    const bool i8 = dtype == TGEMM_I8;
    if (N <= tg::THIN_N_MAX) {
        // a few columns: the thin kernel with the fewest columns that cover
        // N (a tile would leave each workgroup waiting on one slice at a
        // time, and compute mostly columns past N: 4096 x 1 x 4096 in 11 us
        // against 95 us register-staged; 4095 x 8 x 4104 bf16 7.2 us against
        // 19.5 on the direct loader, 16384 x 16 x 256 5.0 against 7.5; int8
        // x 16 x 256 loses 0.4-0.6 us at 512-4095 rows)
        // (one column: the contiguous-column twin exactly when ldb = 1).
        // Of the kernels of that width, the most rows per workgroup that
        // still give 256 workgroups (one per compute unit), else the fewest:
        // every workgroup stages all of B, and fewer, fuller workgroups
        // stage it less often (16384 x 8 x 4104 bf16: 36.7 us with 64 rows
        // against 45.8 with 16; 4095 rows keep 16: 11.7 against 15.8 with 32).
        // The matrix-core kernels first, for 2..16 columns whose B rows take
        // their NB-column pieces (NB <= ldb + N).
        const KernelEntry* best = nullptr;
        auto better = [&](const KernelEntry& e) {
            if (!best) return true;
            if (e.thin_mma != best->thin_mma) return e.thin_mma > best->thin_mma;
            if (e.bn != best->bn) return e.bn < best->bn;
            const bool fills = (M + e.bm - 1) / e.bm >= 256, best_fills = (M + best->bm - 1) / best->bm >= 256;
            return fills ? (!best_fills || e.bm > best->bm) : (!best_fills && e.bm < best->bm);
        };
        for (const KernelEntry& e : g_reg[dtype]) {
            if (e.family != tg::FAM_THIN || e.bn < N || (N == 1 && (e.thin_col != 0) != (ldb == 1))) continue;
            if (e.thin_mma && (N < 2 || e.bn > ldb + N)) continue;
            if (better(e)) best = &e;
        }
        if (best) return best;
    }
    const int64_t short_k = i8 ? 2048 : 1024;
    // one 128 x 128 tile per unit, relative to a round of 256 x 256 tiles, at
    // 4096^3: bf16 direct 146 / 4 us vs 113 us; int8 85 / 4 vs 68 us;
    // register-staged, B rows unaligned: 221 / 4 vs 212 us
    const double mid_tile = guarded ? 0.26 : (i8 ? 0.31 : 0.325);
    // Below short_k, a single round of 256 x 256 tiles (128 to 256 of them)
    // still wins from K = 512 (int8: 1024), where the K loop outweighs the
    // one unoverlapped C write: bf16 4096^2 x 512 26.0 vs 27.2 us (128 x 128,
    // 4 slots), x 1024 38.3 vs 41.6; 3072^2 x 512 19.8 vs 21.9; int8 4096^2 x
    // 1024 28.0 vs 30.9, x 2048 41.3 vs 47.3.  With more than one round
    // (6144^2 x 512: 68.1 vs 57.4) the 128 x 128 tiles overlap their writes.
    const int64_t one_round_k = i8 ? 1024 : 512;
    int pick;  // tile edge
    if (wgs(256) >= 128 && K > short_k)
        pick = big_rounds(wgs(256)) <= mid_tile * (double)((wgs(128) + 255) / 256) ? 256 : 128;
    else if (!guarded && wgs(256) >= 128 && wgs(256) <= 256 && K >= one_round_k)
        pick = 256;
    else if (!guarded && wgs(128) > 64 && wgs(128) <= 128 && K >= (i8 ? 2048 : 1024))
        pick = 96;  // a half tile, 128 x 64 or 64 x 128 (below)
    else if (wgs(128) > 64 || guarded)
        pick = 128;
    else
        pick = 64;  // a quarter of the CUs or fewer on 128 x 128 (1024^2 x 4096: 19.4 vs 32.7 us)
    if (pick == 96) {
        // 128 x 128 tiles would fill between a quarter and half of the
        // compute units; half tiles fill them (bf16 512 x 4096 x 4096: 64 x
        // 128 27.2 us vs 34.3; 1024 x 2048 x 2048: 128 x 64 15.3 vs 19.7;
        // 2048 x 1024 x 4096: 26.7-27.9 vs 33.2; equal at K = 1024.  int8
        // 512 x 4096 x 4096: 17.7 vs 20.3; 2048 x 1024 x 4096: 17.5 vs 20.7;
        // 1024 x 2048 x 2048: 12.2 vs 12.8; 12.3 vs 11.8 at K = 1024)
        tgemm_variant h = v;
        h.tile_m = N >= M ? 64 : 128;
        h.tile_n = N >= M ? 128 : 64;
        h.tile_k = i8 ? 64 : 32;
        h.waves_n = 2;
        h.stages = 4;
        h.loader = TGEMM_LOADER_DIRECT;
        if (const KernelEntry* e = find_entry(dtype, h)) return e;
        pick = 128;
    }
    v.tile_m = v.tile_n = pick;
    v.waves_n = pick == 256 ? 4 : 2;
    // 128 x 128 direct: a 4-slot ring from K = 512 for bf16 (4-13 % faster
    // than 3 slots at 2048^2 x 4096, 4096 x 4352 x 4096, 1024^2 x 8192 and
    // 2048^2 x 8192; 3-8 % at 2048^2 x 1024..2048, 6144^2 and 8192^2 x 512)
    // and from K = 1024 for int8 (2048^2 x 4096 24.3 vs 25.4 us, 6144^2 x
    // 1024 57.0 vs 60.9; equal at 2048^2 x 8192); 3 below
    v.stages = pick == 256 || guarded ? 2 : (pick == 128 && K >= (i8 ? 1024 : 512) ? 4 : 3);
    // 64 x 64 tiles (grids of about one workgroup per compute unit): each
    // wave issues one matrix instruction per K step, too short to cover the
    // next step's fragment reads, so the fragments of a whole slice are read
    // one slice ahead (graph replay, bf16, us, reads one step ahead -> one
    // slice ahead: 512^2 x 4096 19.0 -> 13.9, x 8192 33.3 -> 27.2, x 1024
    // 7.5 -> 6.6; 1024^2 x 4096 20.0 -> 17.8; 768^2 x 4096 18.6 -> 15.7; int8
    // 512^2 x 4096 11.2 -> 8.9, x 8192 18.5 -> 13.5).  From 1024 bf16 /
    // 2048 int8 values of K, 128-deep (int8 256) slices in 4 slots: half the
    // barriers per matrix instruction of 64-deep slices in 8 slots (the same
    // 128 KiB ring; bf16 512^2 x 1024 6.2 vs 6.6 us, x 2048 8.6 vs 8.8, x
    // 8192 25.5 vs 27.0, 768^2 x 4096 15.4 vs 15.9, 1024^2 x 4096 17.2 vs
    // 18.1, 512^2 x 4096 13.5 vs 13.3; int8 512^2 x 2048 6.2 vs 6.6, x 4096
    // 8.7 vs 9.0, 1024^2 x 4096 11.0 vs 11.7), 64-deep in 3 slots below
    // (512^2 x 512 5.1 vs 5.3 us with 8)
    if (pick == 64) {
        v.frag = TGEMM_FRAG_SLICE;
        if (K >= (i8 ? 2048 : 1024)) {
            v.tile_k = i8 ? 256 : 128;
            v.stages = 4;
        }
    }
    v.loader = guarded ? TGEMM_LOADER_VGPR : TGEMM_LOADER_DIRECT;
    return find_entry(dtype, v);
}

// The kernel that runs in place of e for operands whose rows are not
// 16-byte aligned (ga: A, gb: B): e itself if it can read them, else a
// register-staged kernel with shifted loads for just those operands
// (registry order puts A-only before B-only before both) with the same tile
// and wave grid, else the same tile, else the nearest tile in size.
const KernelEntry* guard_capable(const KernelEntry* e, bool ga, bool gb, int64_t N) {
    if (accepts(*e, ga, gb, N)) return e;
    for (int same_waves = 1; same_waves >= 0; --same_waves)
        for (const KernelEntry& c : g_reg[e->dtype])
            if (accepts(c, ga, gb, N) && c.family == e->family && c.bm == e->bm && c.bn == e->bn &&
                c.bk == e->bk && c.access == tg::AC_WIDE && c.stages == 2 &&
                (!same_waves || (c.wm == e->wm && c.wn == e->wn)))
                return &c;
    const KernelEntry* best = nullptr;
    int best_d = INT_MAX;
    for (const KernelEntry& c : g_reg[e->dtype])
        if (accepts(c, ga, gb, N) && c.family == tg::FAM_TILED && c.access == tg::AC_WIDE && c.stages == 2) {
            const int d = abs(c.bm - e->bm) + abs(c.bn - e->bn);
            if (d < best_d) {
                best = &c;
                best_d = d;
            }
        }
    return best;
}

void entry_to_variant(const KernelEntry& e, int32_t wg_group, tgemm_variant* v) {
    memset(v, 0, sizeof *v);
    v->kernel = e.family == tg::FAM_NAIVE ? TGEMM_KERNEL_NAIVE : TGEMM_KERNEL_TILED;
    v->tile_m = e.bm;
    v->tile_n = e.bn;
    v->tile_k = e.bk;
    v->stages = e.stages;
    v->loader = e.loader;
    v->lds_layout = e.layout;
    v->access = e.access;
    v->frag = e.frag;
    v->wg_group = wg_group;
    v->waves_m = e.wm;
    v->waves_n = e.wn;
    v->store = e.store;
    v->copy_sched = e.copy_sched;
    v->frag_read = e.frag_read;
    v->lane_map = e.lane_map;
}

// TGEMM_C_STORES_*: how the matrix-core kernels write C (tgemm_set_c_store_policy)
std::atomic<int> g_c_store_policy{TGEMM_C_STORES_AUTO};

// Per-device gfx950 check, cached.
std::mutex g_arch_mu;
int g_arch_ok[64];  // 0 unknown, 1 gfx950, -1 other

int check_arch() {
    int dev = 0;
    const hipError_t gerr = hipGetDevice(&dev);
    if (gerr != hipSuccess) {
        set_err("hipGetDevice failed: %s", hipGetErrorString(gerr));
        return TGEMM_E_HIP;
    }
    if (dev < 0 || dev >= 64) {
        set_err("device index %d out of range", dev);
        return TGEMM_E_ARCH;
    }
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            set_err("hipGetDeviceProperties failed");
            return TGEMM_E_HIP;
        }
        g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (g_arch_ok[dev] < 0) set_err("device %d is %s, libtgemm is built for gfx950 only", dev, prop.gcnArchName);
    }
    return g_arch_ok[dev] > 0 ? TGEMM_OK : TGEMM_E_ARCH;
}

__global__ void zero_fill_4byte(uint32_t* C, int M, int N, int64_t ldc) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / N, c = i - r * N;
        C[r * ldc + c] = 0u;
    }
}

}  // namespace

extern "C" {

const char* tgemm_version(void) { return "tgemm 0.1 (gfx950)"; }

const char* tgemm_last_error(void) { return g_err.c_str(); }

int tgemm_set_c_store_policy(int policy) {
    if (policy != TGEMM_C_STORES_AUTO && policy != TGEMM_C_STORES_STREAM && policy != TGEMM_C_STORES_PLAIN) {
        set_err("unknown C store policy %d", policy);
        return TGEMM_E_ARG;
    }
    return g_c_store_policy.exchange(policy);
}

}  // extern "C"

extern "C" void gemm_destroy(tgemm_plan* plan);

namespace {

// One plan for the whole M x N x K product (no split).
tgemm_plan* make_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, int64_t lda, int64_t ldb, int64_t ldc,
                      const tgemm_variant* variant, bool* is_default) {
    if (dtype != TGEMM_F32 && dtype != TGEMM_BF16 && dtype != TGEMM_I8) {
        set_err("unknown dtype %d", dtype);
        return nullptr;
    }
    if (M < 0 || N < 0 || K < 0) {
        set_err("negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
        return nullptr;
    }
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) {
        set_err("sizes must be below 2^31");
        return nullptr;
    }
    if (lda < 1 || ldb < 1 || ldc < 1 || lda < K || ldb < N || ldc < N) {
        set_err("leading dimensions too small: lda=%lld (K=%lld) ldb=%lld (N=%lld) ldc=%lld (N=%lld)",
                (long long)lda, (long long)K, (long long)ldb, (long long)N, (long long)ldc, (long long)N);
        return nullptr;
    }
    // int8: every |product| is at most 128 * 128 = 16384, so |C| <= 16384 K,
    // which stays below 2^31 (int32) for K <= 131071
    if (dtype == TGEMM_I8 && K > 131071) {
        set_err("int8: K=%lld may overflow the int32 accumulator (K <= 131071)", (long long)K);
        return nullptr;
    }
    tgemm_variant v{};
    if (variant) v = *variant;
    if (v.wg_group < -1) {
        set_err("wg_group must be -1, 0 or positive");
        return nullptr;
    }
    const KernelEntry* e = nullptr;
    bool default_plan = false;
    if (v.kernel == TGEMM_KERNEL_AUTO && v.tile_m == 0 && v.tile_n == 0 && v.tile_k == 0 && v.stages == 0 &&
        v.loader == 0 && v.lds_layout == 0 && v.access == 0 && v.frag == 0 && v.waves_m == 0 &&
        v.waves_n == 0 && v.store == 0 && v.copy_sched == 0 && v.frag_read == 0 && v.lane_map == 0) {
        e = default_entry(dtype, M, N, K, ldb, false);
        default_plan = true;
    } else {
        e = find_entry(dtype, v);
    }
    if (!e) {
        set_err("no compiled variant matches the request (see gemm_variant_get)");
        return nullptr;
    }
    if (!direct_fits(*e, lda, ldb)) {
        // leading dimensions too large for the direct loader's 32-bit
        // offsets: the register-staged kernel of the same tile, else the
        // register-staged default for the shape
        tgemm_variant r{};
        entry_to_variant(*e, 0, &r);
        r.loader = TGEMM_LOADER_VGPR;
        r.stages = 2;
        if (r.frag == TGEMM_FRAG_SLICE) r.frag = TGEMM_FRAG_REUSE;  // a direct-loader schedule
        r.store = 0;
        r.copy_sched = 0;
        r.frag_read = 0;
        r.lane_map = 0;
        r.wg_group = 0;
        const KernelEntry* rs = find_entry(dtype, r);
        e = rs ? rs : default_entry(dtype, M, N, K, ldb, true);
        if (!e || !direct_fits(*e, lda, ldb)) {
            set_err("no kernel addresses leading dimensions lda=%lld ldb=%lld", (long long)lda, (long long)ldb);
            return nullptr;
        }
    }
    // Kernels for every combination of misaligned operands (pointers are
    // only known per run); the leading dimensions fix which one this plan
    // starts from.  A default plan falls back to the default register-staged
    // choice for the shape, an explicit variant to its nearest relative.
    const KernelEntry* fb[4] = {e, nullptr, nullptr, nullptr};
    const KernelEntry* base = default_plan ? default_entry(dtype, M, N, K, ldb, true) : e;
    for (int m = 1; m < 4; ++m) {
        fb[m] = guard_capable(accepts(*e, m & 1, m & 2, N) ? e : base, m & 1, m & 2, N);
        if (!fb[m]) {
            set_err("variant %s has no fallback for unaligned operands", e->name);
            return nullptr;
        }
    }
    int32_t ga = 0, gb = 0;
    ld_guards(*e, N, lda, ldb, &ga, &gb);
    if (ga || gb) {
        e = fb[ga | (gb << 1)];
        ld_guards(*e, N, lda, ldb, &ga, &gb);
    }
    if (e->thin_mma && gb) {
        // the matrix-core thin kernel reads NB-column pieces of B's rows,
        // which with NB > ldb + N could run past the matrix (the planner
        // never picks it then)
        set_err("%s cannot read B with ldb=%lld", e->name, (long long)ldb);
        return nullptr;
    }
    const int64_t tiles_m = (M + e->bm - 1) / e->bm, tiles_n = (N + e->bn - 1) / e->bn;
    if (tiles_m * tiles_n > INT_MAX) {
        set_err("too many tiles");
        return nullptr;
    }
    tgemm_plan* p = new tgemm_plan;
    p->M = M;
    p->N = N;
    p->K = K;
    p->lda = lda;
    p->ldb = ldb;
    p->ldc = ldc;
    p->dtype = dtype;
    p->entry = e;
    for (int m = 0; m < 4; ++m) p->fallback[m] = m == 0 ? e : fb[m];
    // default: XCD-aware order grouped by 4 tile rows (measured ~4% faster
    // than row-major for 256 x 256 tiles at 4096^3, with less L2-miss traffic)
    p->wg_group = v.wg_group == 0 ? (e->family == tg::FAM_NAIVE ? -1 : 4) : v.wg_group;
    p->a_guard = ga;
    p->b_guard = gb;
    p->n_main = N;
    p->rem = nullptr;
    p->rem_fused = false;
    p->packed = nullptr;
    p->lda_p = lda;
    p->ldb_p = ldb;
    if (is_default) *is_default = default_plan;
    g_err.clear();
    return p;
}

}  // namespace

extern "C" {

// A default plan whose tile leaves a last column of at most THIN_N_MAX
// columns may split: the tiled kernel on the first N - r columns and the
// thin kernel on the last r, launched one after the other on the stream.
// It does when the time model gives the main part fewer rounds than the
// whole (4095 x 4097: 1056 tiles of 128 x 128, five on the busiest compute
// unit, against 256 tiles of 256 x 256 in one round plus one column).
static tgemm_plan* split_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, int64_t lda, int64_t ldb,
                              int64_t ldc, const tgemm_variant* variant, bool* default_out) {
    bool is_default = false;
    tgemm_plan* p = make_plan(M, N, K, dtype, lda, ldb, ldc, variant, &is_default);
    if (default_out) *default_out = is_default;
    if (!p || !is_default || dtype == TGEMM_F32 || K == 0 || M == 0) return p;
    const KernelEntry& e = *p->entry;
    const int64_t r = N % e.bn;
    if (e.family != tg::FAM_TILED || r == 0 || r > tg::THIN_N_MAX || N <= e.bn) return p;
    const double t_full = model_rounds(e, M, N);
    if (t_full < 0) return p;
    tgemm_plan* main = make_plan(M, N - r, K, dtype, lda, ldb, ldc, nullptr, nullptr);
    if (!main) {
        g_err.clear();
        return p;
    }
    const double t_main = model_rounds(*main->entry, M, N - r);
    if (t_main < 0 || t_main >= t_full) {
        gemm_destroy(main);
        return p;
    }
    tgemm_plan* rem = make_plan(M, r, K, dtype, lda, ldb, ldc, nullptr, nullptr);
    if (!rem) {
        gemm_destroy(main);
        g_err.clear();
        return p;
    }
    gemm_destroy(p);
    main->N = N;  // the user's shape; the grid covers n_main
    main->rem = rem;
    // one last column, and tile columns enough to give every row of a tile
    // to some workgroup (16 rows each): the main kernel's twin computes it
    // in its own K loop (bf16 4095 x 4097 x 4104: 125 us against 145 us for
    // the two launches, whose thin kernel walks B's column once per
    // workgroup)
    main->rem_fused = r == 1 && main->entry->rem_fn && 16 * ((N - r + main->entry->bn - 1) / main->entry->bn) >=
                                                           main->entry->bm;
    g_err.clear();
    return main;
}

// Leading dimension of a repacked operand: ld itself when its rows are
// already 16-byte aligned (then only a misaligned pointer forces the copy,
// and the plan keeps the caller's stride), else rows rounded up to whole
// 128-byte lines, so that no row segment of a slice straddles an extra
// cache line.  That matters most for A, whose rows a slice reads 64 to 128
// bytes at a time (bf16 4096 x 4096 x 4104: lda = 4104 119.6 us, lda = 4160
// 115.4 us); a repacked B of the ragged product gains nothing measurable.
static int64_t aligned_ld(int64_t ld, int64_t cols, int esz) {
    if ((ld * esz) % 16 == 0) return ld;
    return (cols * esz + 127) / 128 * 128 / esz;
}

// A default plan whose kernel needs aligned rows also carries the plan for
// the same product on operands repacked into 16-byte aligned rows
// (gemm_run_ws), when that plan runs a tiled kernel on more than THIN_N_MAX
// columns (for thinner products the product itself moves about as many
// bytes as the repack would).
tgemm_plan* gemm_plan_variant(int64_t M, int64_t N, int64_t K, int32_t dtype, int64_t lda, int64_t ldb,
                              int64_t ldc, const tgemm_variant* variant) {
    init_registry();
    bool is_default = false;
    tgemm_plan* p = split_plan(M, N, K, dtype, lda, ldb, ldc, variant, &is_default);
    if (!p || !is_default || M == 0 || N <= tg::THIN_N_MAX || K == 0) return p;
    // a kernel that reads rows of any alignment gains nothing from the copy
    // (bf16 4096^3 with ldb = 4097: 114 us in place against 121 us
    // repacked), and a copy leaves N as it is
    if (any_alignment(*p->entry)) return p;
    const int esz = elem_size(dtype);
    const int64_t lda_p = aligned_ld(lda, K, esz), ldb_p = aligned_ld(ldb, N, esz);
    tgemm_plan* q = split_plan(M, N, K, dtype, lda_p, ldb_p, ldc, nullptr, nullptr);
    if (!q || q->entry->family != tg::FAM_TILED) {
        gemm_destroy(q);
        g_err.clear();
        return p;
    }
    p->packed = q;
    p->lda_p = lda_p;
    p->ldb_p = ldb_p;
    g_err.clear();
    return p;
}

tgemm_plan* gemm_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, int64_t lda, int64_t ldb,
                      int64_t ldc) {
    return gemm_plan_variant(M, N, K, dtype, lda, ldb, ldc, nullptr);
}

void gemm_destroy(tgemm_plan* plan) {
    if (!plan) return;
    gemm_destroy(plan->rem);
    gemm_destroy(plan->packed);
    delete plan;
}

}  // extern "C"

namespace {

// gemm_run with an optional clock buffer for the main kernel's workgroups.
int run_impl(const tgemm_plan* p, const void* A, const void* B, void* C, uint64_t* clocks, int64_t clocks_len,
             void* stream) {
    if (!p) {
        set_err("NULL plan");
        return TGEMM_E_NULL;
    }
    if (p->M == 0 || p->N == 0) return TGEMM_OK;
    if (!C || (p->K > 0 && (!A || !B))) {
        set_err("NULL matrix pointer");
        return TGEMM_E_NULL;
    }
    const int esz = elem_size(p->dtype);
    if (((uintptr_t)A % esz) || ((uintptr_t)B % esz) || ((uintptr_t)C % 4)) {
        set_err("pointer not aligned to its element size");
        return TGEMM_E_ALIGN;
    }
    int rc = check_arch();
    if (rc != TGEMM_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->K == 0) {
        const int64_t total = p->M * p->N;
        const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
        hipLaunchKernelGGL(zero_fill_4byte, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(C),
                           (int)p->M, (int)p->N, p->ldc);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) {
            set_err("launch failed: %s", hipGetErrorString(err));
            return TGEMM_E_HIP;
        }
        return TGEMM_OK;
    }
    const KernelEntry* e = p->entry;
    int32_t ga = p->a_guard, gb = p->b_guard;
    const int bytes = access_bytes(*e);
    if (needs_aligned_ptrs(*e)) {
        if ((uintptr_t)A % bytes) ga = 1;
        if ((uintptr_t)B % bytes) gb = 1;
    }
    if (!accepts(*e, ga, gb, p->n_main)) {
        e = p->fallback[ga | (gb << 1)];
        int32_t fa = 0, fbg = 0;
        ld_guards(*e, p->n_main, p->lda, p->ldb, &fa, &fbg);
        const int fbytes = access_bytes(*e);
        const bool fptr = needs_aligned_ptrs(*e);
        ga = fa || (fptr && (uintptr_t)A % fbytes);
        gb = fbg || (fptr && (uintptr_t)B % fbytes);
        if (!accepts(*e, ga, gb, p->n_main)) {
            set_err("no kernel of this plan reads operands at these addresses");
            return TGEMM_E_ALIGN;
        }
    }
    tg::GemmArgs g{};  // every field zero, the clock buffer NULL, unless set below
    g.A = A;
    g.B = B;
    g.C = C;
    g.M = (int32_t)p->M;
    g.N = (int32_t)p->n_main;
    g.K = (int32_t)p->K;
    g.tiles_m = (int32_t)((p->M + e->bm - 1) / e->bm);
    g.tiles_n = (int32_t)((p->n_main + e->bn - 1) / e->bn);
    g.lda = p->lda;
    g.ldb = p->ldb;
    g.ldc = p->ldc;
    // any group of tiles_m rows or more gives the same order (one group of
    // every tile row); clamping keeps wg_group * tiles_n within the grid
    g.wg_group = p->wg_group > g.tiles_m ? g.tiles_m : p->wg_group;
    g.a_guard = ga;
    g.b_guard = gb;
    // Streaming (non-temporal) C stores where C's rows are whole cache lines.
    // The exception: 256 x 256 tiles with a short K loop, where every
    // workgroup writes its C at the same time and the write is a large share
    // of the launch; plain stores drain it faster there (graph replay, us,
    // streaming vs plain: bf16 4096^2 x 512 27.0 vs 26.3, x 1024 39.8 vs
    // 38.9, x 2048 64.5 vs 64.9, x 4096 114.4 vs 115.8; int8 x 1024 27.0 vs
    // 26.6, x 2048 40.8 vs 40.1, x 4096 66.0 vs 66.9; bf16 8192^2 x 512
    // 100.2 vs 99.5), so those stream from 4 KiB of K per row.  Smaller tiles
    // run in several rounds, one round's writes under the next one's loops,
    // and keep streaming (bf16 4096^2 x 256 on 128 x 128 tiles: 20.6 us
    // streaming, 22.1 plain).
    const bool big_tile = e->bm * e->bn >= 256 * 256;
    const bool lines = (uintptr_t)C % 128 == 0 && (p->ldc * 4) % 128 == 0;
    const int policy = g_c_store_policy.load(std::memory_order_relaxed);
    g.c_stream = policy == TGEMM_C_STORES_PLAIN ? 0
                 : policy == TGEMM_C_STORES_STREAM ? lines
                 : lines && (!big_tile || p->K * esz >= 4096);
    if (clocks && e->family == tg::FAM_TILED) {
        // the kernel that runs decides the count (a fallback's tile may differ)
        const int64_t need = tg::CLOCK_VALUES * (int64_t)g.tiles_m * g.tiles_n;
        if (need > clocks_len) {
            set_err("clock buffer holds %lld values, %s needs %lld", (long long)clocks_len, e->name,
                    (long long)need);
            return TGEMM_E_ARG;
        }
        g.clocks = clocks;
    }
    // the plan's own kernel computes the last column too (REM twin)
    const bool fused = p->rem_fused && e == p->entry;
    void* args[] = {&g};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fused ? e->rem_fn : e->fn),
                                           dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(e->threads), args, 0, s);
    if (err != hipSuccess) {
        set_err("launch of %s failed: %s", e->name, hipGetErrorString(err));
        return TGEMM_E_HIP;
    }
    if (p->rem && !fused)  // the last N - n_main columns, after the main part on the same stream
        return run_impl(p->rem, A, static_cast<const char*>(B) + p->n_main * esz,
                        static_cast<char*>(C) + p->n_main * 4, nullptr, 0, stream);
    return TGEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run(const tgemm_plan* p, const void* A, const void* B, void* C, void* stream) {
    return run_impl(p, A, B, C, nullptr, 0, stream);
}

int64_t gemm_clock_slots(const tgemm_plan* p) {
    if (!p || p->M == 0 || p->N == 0 || p->K == 0) return 0;
    // the largest grid among the kernels this plan may launch
    int64_t most = 0;
    for (int m = 0; m < 4; ++m) {
        const KernelEntry* e = m == 0 ? p->entry : p->fallback[m];
        if (!e || e->family != tg::FAM_TILED) continue;
        const int64_t n = tg::CLOCK_VALUES * ((p->M + e->bm - 1) / e->bm) * ((p->n_main + e->bn - 1) / e->bn);
        if (n > most) most = n;
    }
    return most;
}

int gemm_run_clocked(const tgemm_plan* p, const void* A, const void* B, void* C, uint64_t* clocks,
                     int64_t clocks_len, void* stream) {
    if (!p || !clocks) {
        set_err("NULL plan or clock buffer");
        return TGEMM_E_NULL;
    }
    const int64_t need = gemm_clock_slots(p);
    if (need == 0) {
        set_err("this plan runs no tiled kernel to clock");
        return TGEMM_E_ARG;
    }
    if ((uintptr_t)clocks % 8) {
        set_err("clock buffer not 8-byte aligned");
        return TGEMM_E_ALIGN;
    }
    return run_impl(p, A, B, C, clocks, clocks_len, stream);
}

// Which operands gemm_run_ws repacks for these pointers (bit 0 A, bit 1 B)
// and the workspace bytes that takes: an operand is repacked when its rows
// are not 16-byte aligned (leading dimension or pointer), each copy starting
// on a 256-byte boundary of the workspace.
static int64_t pack_need(const tgemm_plan* p, const void* A, const void* B, int* mask) {
    *mask = 0;
    if (!p || !p->packed || p->M == 0 || p->N == 0 || p->K == 0) return 0;
    const int esz = elem_size(p->dtype);
    const bool ma = (p->lda * esz) % 16 != 0 || (uintptr_t)A % 16 != 0;
    const bool mb = (p->ldb * esz) % 16 != 0 || (uintptr_t)B % 16 != 0;
    int64_t need = 0;
    if (ma) need += (p->M * p->lda_p * esz + 255) / 256 * 256;
    if (mb) need += (p->K * p->ldb_p * esz + 255) / 256 * 256;
    *mask = (ma ? 1 : 0) | (mb ? 2 : 0);
    return need;
}

int64_t gemm_workspace_bytes(const tgemm_plan* p, const void* A, const void* B) {
    int mask = 0;
    return pack_need(p, A, B, &mask);
}

int gemm_run_ws(const tgemm_plan* p, const void* A, const void* B, void* C, void* workspace,
                int64_t workspace_bytes, void* stream) {
    int mask = 0;
    const int64_t need = pack_need(p, A, B, &mask);
    if (need == 0 || !workspace || workspace_bytes < need) return gemm_run(p, A, B, C, stream);
    if ((uintptr_t)workspace % 256) {
        set_err("workspace not 256-byte aligned");
        return TGEMM_E_ALIGN;
    }
    if (!C || !A || !B) {
        set_err("NULL matrix pointer");
        return TGEMM_E_NULL;
    }
    const int esz = elem_size(p->dtype);
    if (((uintptr_t)A % esz) || ((uintptr_t)B % esz) || ((uintptr_t)C % 4)) {
        set_err("pointer not aligned to its element size");
        return TGEMM_E_ALIGN;
    }
    int rc = check_arch();
    if (rc != TGEMM_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const void* a = A;
    const void* b = B;
    if (mask & 1) {
        const tg::PackArgs pa{static_cast<const char*>(A), ws, p->M, p->K * esz, p->lda * esz, p->lda_p * esz};
        const hipError_t err = tg::launch_pack(pa, s);
        if (err != hipSuccess) {
            set_err("repack of A failed: %s", hipGetErrorString(err));
            return TGEMM_E_HIP;
        }
        a = ws;
        ws += (p->M * p->lda_p * esz + 255) / 256 * 256;
    }
    if (mask & 2) {
        const tg::PackArgs pb{static_cast<const char*>(B), ws, p->K, p->N * esz, p->ldb * esz, p->ldb_p * esz};
        const hipError_t err = tg::launch_pack(pb, s);
        if (err != hipSuccess) {
            set_err("repack of B failed: %s", hipGetErrorString(err));
            return TGEMM_E_HIP;
        }
        b = ws;
    }
    return gemm_run(p->packed, a, b, C, stream);
}

}  // extern "C"

namespace {

// The workspace of gemm_run_noalloc: a fixed device array, one per GPU the
// library runs on, held until the process ends.  Its name is a host-side
// stand-in, not a device address: host code only ever uses the address
// hipGetSymbolAddress returns for the current device (looked up on the
// entry point's first call on that device and kept per device).
static __device__ __align__(256) char scratch[TGEMM_NOALLOC_MAX_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device; NULL until looked up

int scratch_of_current_device(void** out) {
    int dev = 0;
    const hipError_t gerr = hipGetDevice(&dev);
    if (gerr != hipSuccess) {
        set_err("hipGetDevice failed: %s", hipGetErrorString(gerr));
        return TGEMM_E_HIP;
    }
    if (dev < 0 || dev >= 64) {
        set_err("device index %d out of range", dev);
        return TGEMM_E_ARCH;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr) {
            set_err("hipGetSymbolAddress of the fixed workspace failed on device %d: %s", dev,
                    hipGetErrorString(err));
            return TGEMM_E_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TGEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run_noalloc(const tgemm_plan* p, const void* A, const void* B, void* C, void* stream) {
    if (!p) {
        set_err("NULL plan");
        return TGEMM_E_NULL;
    }
    int mask = 0;
    const int64_t need = pack_need(p, A, B, &mask);
    if (need == 0) return gemm_run(p, A, B, C, stream);
    if (need > TGEMM_NOALLOC_MAX_BYTES) {
        set_err("repacking these operands needs %lld bytes of workspace; the fixed array of gemm_run_noalloc "
                "holds %lld (use gemm_run_ws with a caller workspace, or gemm_run)",
                (long long)need, (long long)TGEMM_NOALLOC_MAX_BYTES);
        return TGEMM_E_ARG;
    }
    int rc = check_arch();
    if (rc != TGEMM_OK) return rc;
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != TGEMM_OK) return rc;
    return gemm_run_ws(p, A, B, C, ws, need, stream);
}

int gemm_plan_get_info(const tgemm_plan* p, tgemm_plan_info* info) {
    if (!p || !info) {
        set_err("NULL plan or info");
        return TGEMM_E_NULL;
    }
    memset(info, 0, sizeof *info);
    const KernelEntry& e = *p->entry;
    info->M = p->M;
    info->N = p->N;
    info->K = p->K;
    info->lda = p->lda;
    info->ldb = p->ldb;
    info->ldc = p->ldc;
    info->dtype = p->dtype;
    entry_to_variant(e, p->wg_group, &info->variant);
    info->grid = (int32_t)(((p->M + e.bm - 1) / e.bm) * ((p->n_main + e.bn - 1) / e.bn));
    info->n_main = p->n_main;
    if (p->rem_fused) snprintf(info->rem_name, sizeof info->rem_name, "%s_remcol", e.name);
    else if (p->rem) snprintf(info->rem_name, sizeof info->rem_name, "%s", p->rem->entry->name);
    if (p->packed) snprintf(info->packed_name, sizeof info->packed_name, "%s", p->packed->entry->name);
    info->threads = e.threads;
    info->lds_bytes = e.lds_bytes;
    info->waves_per_simd = e.waves_per_simd;
    info->loads_per_stage = e.loads_per_stage;
    info->a_guarded = p->a_guard;
    info->b_guarded = p->b_guard;
    snprintf(info->name, sizeof info->name, "%s", e.name);
    return TGEMM_OK;
}

int gemm_kernel_occupancy(const tgemm_plan* p, int32_t packed, int32_t* workgroups_per_cu) {
    if (!p || !workgroups_per_cu) {
        set_err("NULL plan or output");
        return TGEMM_E_NULL;
    }
    const KernelEntry& e = (packed && p->packed) ? *p->packed->entry : *p->entry;
    int n = 0;
    const hipError_t err =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(e.fn), e.threads, 0);
    if (err != hipSuccess) {
        set_err("hipOccupancyMaxActiveBlocksPerMultiprocessor: %s", hipGetErrorString(err));
        return (int)err;
    }
    *workgroups_per_cu = n;
    return TGEMM_OK;
}

int gemm_variant_count(int32_t dtype) {
    init_registry();
    if (dtype < 0 || dtype > 2) return 0;
    int n = 0;
    for (const KernelEntry& e : g_reg[dtype]) n += e.listed;
    return n;
}

int gemm_variant_get(int32_t dtype, int32_t index, tgemm_variant* out) {
    init_registry();
    if (dtype >= 0 && dtype <= 2 && out && index >= 0) {
        int n = 0;
        for (const KernelEntry& e : g_reg[dtype])
            if (e.listed && n++ == index) {
                entry_to_variant(e, 0, out);
                return TGEMM_OK;
            }
    }
    set_err("bad dtype or index");
    return TGEMM_E_ARG;
}

}  // extern "C"
