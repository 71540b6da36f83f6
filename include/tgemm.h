/*
 * tgemm.h -- C ABI of libtgemm, a tiled, software-pipelined GEMM for AMD
 * MI355X (gfx950).
 *
 * Operation.  C = A x B, the general matrix product defined in
 * "4.1 CUDA GEMM算子性能优化" (CUDA GEMM operator optimisation), section 1.1:
 * A is M x K, B is K x N, C is M x N, 2*M*N*K flops (section 1.3).  All three
 * matrices are row-major with leading dimensions in elements, the indexing of
 * that page's naive kernel (section 3.1):
 *
 *     C[i*ldc + j] = sum_{k < K} A[i*lda + k] * B[k*ldb + j],  i < M, j < N.
 *
 * C is overwritten (no alpha/beta, no transposes).  Elements of C outside the
 * M x N window are never written.  K = 0 writes zeros; M = 0 or N = 0 does
 * nothing.  A and B must not overlap C.
 *
 * Types (operand -> output):
 *   TGEMM_F32  : float    x float    -> float   (fp32 vector fused multiply-add,
 *                one fma chain per output in increasing k)
 *   TGEMM_BF16 : bf16     x bf16     -> float   (matrix cores, fp32 accumulate)
 *   TGEMM_I8   : int8     x int8     -> int32   (matrix cores, exact int32
 *                accumulate; |C| <= 16384 K stays below 2^31 for every
 *                input while K <= 131071, the largest K a plan accepts)
 * bf16 operands are passed as their raw 16-bit patterns.
 *
 * The K loop is software-pipelined as the "流水化 GPU 内核" (pipelining GPU
 * kernels) skill, Step 3, and the GEMM page, sections 9-10, describe: tiles of
 * A and B move global -> LDS through a ring of 1-4 stages (8 for the
 * smallest tiles) while the matrix cores work on an earlier stage.
 *
 * Ownership.  The caller owns A, B, C and the stream.  The library allocates
 * no device memory.  gemm_run never copies or pads inputs; gemm_run_ws
 * copies misaligned operands into the workspace the caller passes.  A plan
 * holds only host metadata; it is immutable after creation, so one plan may
 * be run concurrently on several streams.
 *
 * Errors.  gemm_plan* return NULL and record a message (tgemm_last_error) on
 * invalid arguments.  gemm_run returns TGEMM_OK once the kernel is enqueued,
 * a negative TGEMM_E_* code for a rejected call (nothing is enqueued), or
 * TGEMM_E_HIP if the launch itself failed.  Faults during execution surface
 * at the caller's next synchronisation on the stream.  The error message is
 * thread-local.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tgemm_dtype {
    TGEMM_F32 = 0,
    TGEMM_BF16 = 1,
    TGEMM_I8 = 2
} tgemm_dtype;

#define TGEMM_OK 0
#define TGEMM_E_ARG (-1)     /* invalid argument (sizes, leading dims, dtype) */
#define TGEMM_E_NULL (-2)    /* NULL plan or matrix pointer with non-empty work */
#define TGEMM_E_ALIGN (-3)   /* pointer not aligned to its element size */
#define TGEMM_E_ARCH (-4)    /* current device is not gfx950 */
#define TGEMM_E_VARIANT (-5) /* requested variant not available for this plan */
#define TGEMM_E_HIP (-6)     /* HIP runtime call failed (message has detail) */

/* Kernel families (the steps of the optimisation ladder, one variable per
 * step, as the SM80 cp.async / ldmatrix ablation plan, section 1, and the
 * GEMM page, sections 3-10, order them). */
#define TGEMM_KERNEL_AUTO 0      /* let the plan choose (the default) */
#define TGEMM_KERNEL_NAIVE 1     /* one thread per C element, no LDS (section 3.1) */
#define TGEMM_KERNEL_TILED 2     /* LDS block tiling + register / matrix-core tiles */

/* Global -> LDS loaders (the "流水化 GPU 内核" skill, Step 2: register-staged
 * vs asynchronous copy). */
#define TGEMM_LOADER_VGPR 1      /* loads into registers, then ds_write */
#define TGEMM_LOADER_DIRECT 2    /* global_load_lds_dwordx4 straight into LDS */

/* LDS layouts (GEMM page, section 8.5). */
#define TGEMM_LDS_PLAIN 1
#define TGEMM_LDS_XOR 2          /* 16-byte chunk index XOR-swizzled by row; for the fp32
                                    kernels: the rows of transposed A padded (conflict-free
                                    A writes) */
#define TGEMM_LDS_XOR_POISON 3   /* debug form of TGEMM_LDS_XOR for the direct-loader ring:
                                    each lane fills the 16 LDS bytes a direct copy will
                                    write with all-ones bytes (bf16 NaN, int8 -1) and waits
                                    for that store before issuing the copy, so a read of a
                                    slot before its copy lands, or after the copy of a later
                                    slice began, puts NaN (bf16) or a wrong sum (int8) into
                                    C.  Same results as TGEMM_LDS_XOR when the ring is
                                    correct; slower.  Only chosen when requested. */

/* Access width of global loads and LDS writes (GEMM page, section 7:
 * 128-bit vector accesses); fragment reads have their own field below (the
 * narrow matrix-core rung reads 4 bytes at a time). */
#define TGEMM_ACCESS_WIDE 1      /* 16-byte accesses */
#define TGEMM_ACCESS_NARROW 2    /* 4-byte global loads / LDS accesses */

/* Register tiling (GEMM page, sections 5-6). */
#define TGEMM_FRAG_REUSE 1       /* each fragment read once per k step, reused across the wave tile */
#define TGEMM_FRAG_PER_MMA 2     /* both fragments re-read for every matrix-core instruction */
#define TGEMM_FRAG_SLICE 3       /* as REUSE, with a whole slice's fragments read one slice ahead (direct loader) */

/* C write-back (the SIMT ladder's coalesced write-back step). */
#define TGEMM_STORE_VECTOR 1     /* 16-byte row pieces */
#define TGEMM_STORE_SCALAR 2     /* one element per store */

/* When the direct loader issues a slice's copies (the skill's Step 3: the
 * copy of a later stage overlaps the compute of the current one). */
#define TGEMM_COPY_BURST 1       /* all of them right after the barrier that frees their slot */
#define TGEMM_COPY_SPREAD 2      /* part of them there, the rest spread over the K steps of the
                                    next slice (fewer memory instructions between any two
                                    matrix instructions; a shorter lead for the rest) */
#define TGEMM_COPY_LATE 3        /* as BURST, with the slice's barrier (and the copies and reads
                                    after it) half-way through the last K step's matrix
                                    instructions instead of after its second: a measurement
                                    twin of the 256 x 256 defaults */

/* How operand fragments are read out of LDS (the LDS -> register ladder of
 * the SM80 ablation plan, section 1.1).  Matrix-core kernels: the A fragment
 * (16 bytes of one row per lane) as four 4-byte, two 8-byte or one 16-byte
 * ds_read; the B fragment (one column per lane, K-contiguous, out of
 * N-contiguous LDS rows) by one element read per K value, or (TR) by two
 * transposing reads ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (int8).
 * fp32 kernels report B128 (A transposed in LDS, 16-byte reads) or B32. */
#define TGEMM_READ_B32 1         /* A: 4 x ds_read_b32; B: element reads */
#define TGEMM_READ_B64 2         /* A: 2 x ds_read_b64; B: element reads */
#define TGEMM_READ_B128 3        /* A: 1 x ds_read_b128; B: element reads */
#define TGEMM_READ_TR 4          /* A: 1 x ds_read_b128; B: 2 transposing reads (16-byte kernels' default) */
#define TGEMM_READ_KVEC 5        /* fp32: A row-major in LDS, 16-byte reads along K (4 k steps each) */

/* Which outputs a lane of the fp32 kernels owns (GEMM page, sections 7.4 and
 * 8.5); matrix-core kernels report BLOCKS. */
#define TGEMM_LANES_BLOCKS 1     /* one contiguous TM x TN block, lanes row-major on the wave's 8 x 8 grid */
#define TGEMM_LANES_QUARTERS 2   /* 4 x 4 quarters 32 rows / columns apart (scheme 4: sub-block split) */
#define TGEMM_LANES_ZORDER 3     /* contiguous blocks, lanes in Z order (scheme 3: each 16-lane group
                                    covers a 4 x 4 square of the lane grid) */
#define TGEMM_LANES_ZQUARTERS 4  /* both */

/* Workgroup order (GEMM page, section 2.3). */
#define TGEMM_ORDER_ROW_MAJOR (-1)

/* Variant description.  Zero-initialise and set the fields you want; a zero
 * field means "the plan's default" (every TGEMM_* value above is non-zero).  Only combinations the library was built
 * with are accepted (TGEMM_E_VARIANT otherwise; gemm_variant_count /
 * gemm_variant_get enumerate them). */
typedef struct tgemm_variant {
    int32_t kernel;     /* TGEMM_KERNEL_* */
    int32_t tile_m;     /* workgroup tile rows (BM) */
    int32_t tile_n;     /* workgroup tile columns (BN) */
    int32_t tile_k;     /* K step per stage (BK), in elements */
    int32_t stages;     /* LDS stages in the ring: 1 (no pipelining) .. 4, or 8 (64 x 64 tiles) */
    int32_t loader;     /* TGEMM_LOADER_* */
    int32_t lds_layout; /* TGEMM_LDS_* */
    int32_t access;     /* TGEMM_ACCESS_* */
    int32_t frag;       /* TGEMM_FRAG_* */
    int32_t wg_group;   /* TGEMM_ORDER_ROW_MAJOR, or g >= 1: XCD-aware order grouped by g tile rows */
    int32_t waves_m;    /* waves per workgroup along M */
    int32_t waves_n;    /* waves per workgroup along N */
    int32_t store;      /* TGEMM_STORE_*: fp32 kernels, and the matrix-core kernels' write-back
                           (SCALAR: 4-byte stores from the matrix instruction's output layout;
                           VECTOR: the operands of every matrix instruction swapped, C^T = B^T A^T,
                           so each lane holds four consecutive columns: 16-byte stores) */
    int32_t copy_sched; /* TGEMM_COPY_* (matrix-core direct loader; other kernels report BURST) */
    int32_t frag_read;  /* TGEMM_READ_* */
    int32_t lane_map;   /* TGEMM_LANES_* */
} tgemm_variant;

typedef struct tgemm_plan tgemm_plan;

/* Create a plan for an M x N x K product of the given type with the given
 * leading dimensions (elements).  Requires M, N, K >= 0, lda >= K, ldb >= N,
 * ldc >= N (each leading dimension >= 1).  Does not touch the device.  The
 * plan picks the variant for this shape (tile size by a measured time model
 * of the grid, ring depth by K) and, for each combination of operands whose
 * rows may turn out unaligned at run time, the kernel that reads them.
 * Returns NULL on error (tgemm_last_error says why). */
tgemm_plan* gemm_plan(int64_t M, int64_t N, int64_t K, int32_t dtype,
                      int64_t lda, int64_t ldb, int64_t ldc);

/* As gemm_plan, with an explicit variant (NULL = default).  Used by the
 * ablation harness to time one rung of the ladder. */
tgemm_plan* gemm_plan_variant(int64_t M, int64_t N, int64_t K, int32_t dtype,
                              int64_t lda, int64_t ldb, int64_t ldc,
                              const tgemm_variant* variant);

/* Enqueue C = A x B on `stream` (a hipStream_t; NULL = the null stream) on
 * the current HIP device.  A, B, C are device pointers (or any pointers the
 * device can access) aligned to their element size.  The matrix-core
 * kernels with the direct global->LDS loader (every bf16 / int8 default for
 * products wider than 16 columns) and the thin kernel read rows of any
 * alignment in place: gfx950's 16-byte reads and copies take any byte
 * address at the rate of aligned ones.  The others (fp32, register-staged
 * tiles) run, for a pointer that is element-aligned but not 16-byte aligned
 * or a leading dimension whose rows are not 16-byte aligned, a kernel that
 * reads that operand in shifted or element pieces (slower, same results);
 * so does a B narrower than one 16-byte piece per row (when no thin kernel
 * takes it), and a leading dimension too large for the direct loader's
 * 32-bit lane offsets (from the plan on).  A B whose N is not a whole number
 * of 16-byte pieces is read in place by the direct loader as well (its last
 * row, and a partial last slice, by element loads).  A default bf16 / int8
 * plan of at most 16 columns runs a thin kernel: from 2 columns on the
 * matrix cores (16 x 16 output blocks whose columns past N are computed and
 * dropped; B's rows read as pieces of 4 to 16 columns that may reach into
 * the next row), one column on the vector ALUs.  A default plan one column
 * wider than 16 or more whole 256 x 256 tile columns computes that column
 * in the main kernel's K loop; a few more columns go to a thin kernel after
 * the main launch.  Nothing outside [A, A + ((M-1)*lda + K) elements) or
 * the corresponding range of B is read.
 * C outside its M x N window is not written.  The launch is asynchronous:
 * execution errors surface at the stream's next synchronisation.  Returns
 * TGEMM_OK or a TGEMM_E_* code. */
int gemm_run(const tgemm_plan* plan, const void* A, const void* B, void* C,
             void* stream);

/* Free a plan (NULL is allowed). */
void gemm_destroy(tgemm_plan* plan);

/* Last error message of this thread ("" if none). */
const char* tgemm_last_error(void);

/* Run with a caller-owned device workspace.  Operands whose rows are not
 * 16-byte aligned (a leading dimension that is not a whole number of
 * 16-byte chunks, or a pointer that is not 16-byte aligned) are first copied
 * on `stream` into the workspace with 16-byte aligned rows (leading
 * dimension rounded up to whole 128-byte lines; each copy starts on a
 * 256-byte boundary; the padding columns are written as zero), then the
 * plan's product runs on the copies.  Only plans whose kernel reads such
 * rows slowly carry the repack (fp32 plans, and matrix-core plans that fall
 * back to a register-staged kernel); the direct-loader and thin kernels
 * read any alignment in place, and their plans ask for no workspace.
 * Padding the misaligned operand is the pages' remedy besides a guarded
 * narrow loader (the "流水化 GPU 内核" skill's pitfall list; the SM80
 * ablation plan, section 1.4, note 2).  The result meets the same accuracy
 * as gemm_run's; it is the same bit for bit wherever both paths use
 * matrix-core or fp32 tiles (every such kernel accumulates each output in
 * increasing k) or both use the thin kernel, and may differ in the last bits
 * on columns that only one path gives to the thin kernel.
 *
 * gemm_workspace_bytes returns the bytes this needs for these pointers: 0
 * when no operand is misaligned, for K, M or N = 0, and for plans that carry
 * no repack (explicit variants, products with N <= 16, which read their
 * operands about once anyway, and plans on kernels that read any
 * alignment).  gemm_run_ws behaves exactly like gemm_run
 * when that is 0, when `workspace` is NULL or when `workspace_bytes` is
 * smaller.  The workspace must be 256-byte aligned (TGEMM_E_ALIGN otherwise),
 * must not overlap A, B or C, and must stay allocated until the stream has
 * run the product; its contents are overwritten, so runs that share one
 * workspace must be ordered on one stream.  Returns as gemm_run. */
int64_t gemm_workspace_bytes(const tgemm_plan* plan, const void* A, const void* B);
int gemm_run_ws(const tgemm_plan* plan, const void* A, const void* B, void* C, void* workspace,
                int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gemm_run_ws
 * with the library's own fixed workspace instead of a caller one.  The
 * workspace is one device array of TGEMM_NOALLOC_MAX_BYTES bytes per GPU,
 * created with the library's code on that GPU and held until the process
 * ends; the call itself allocates nothing.  When gemm_workspace_bytes(plan,
 * A, B) is 0 this is gemm_run; when it is at most TGEMM_NOALLOC_MAX_BYTES
 * the misaligned operands are repacked into the array and the result is
 * gemm_run_ws's, bit for bit; larger needs are rejected with TGEMM_E_ARG
 * (nothing is enqueued; tgemm_last_error gives the bytes needed).  Every call
 * on one GPU shares that GPU's array and overwrites what it uses, so calls
 * that overlap on one GPU (other streams, other host threads) race: order
 * them on one stream.  Returns as gemm_run_ws. */
#define TGEMM_NOALLOC_MAX_BYTES (64LL << 20)
int gemm_run_noalloc(const tgemm_plan* plan, const void* A, const void* B, void* C, void* stream);

/* C store policy of the matrix-core kernels that write C from the matrix
 * instruction's layout, process-wide, for measurement (the GEMM page,
 * section 2: the write-back as part of the roofline).  AUTO, the default:
 * non-temporal stores where C's pointer and row stride are 128-byte aligned,
 * except for 256 x 256 tiles with under 4 KiB of K per row, whose launches
 * write all of C at once and drain it faster with plain stores.  STREAM:
 * non-temporal wherever C is 128-byte aligned.  PLAIN: ordinary stores.
 * The results are the same bits under every policy; only the write path
 * differs.  Read when a run is enqueued; set it between runs, not while
 * another host thread enqueues.  Returns the previous policy, or
 * TGEMM_E_ARG for an unknown one. */
#define TGEMM_C_STORES_AUTO 0
#define TGEMM_C_STORES_STREAM 1
#define TGEMM_C_STORES_PLAIN 2
int tgemm_set_c_store_policy(int policy);

/* What a plan will launch. */
typedef struct tgemm_plan_info {
    int64_t M, N, K, lda, ldb, ldc;
    int32_t dtype;
    tgemm_variant variant;   /* fully resolved (no zero/default fields) */
    int32_t grid;            /* workgroups launched */
    int32_t threads;         /* threads per workgroup */
    int32_t lds_bytes;       /* LDS per workgroup */
    int32_t loads_per_stage; /* global->LDS instructions per wave per stage */
    int32_t a_guarded;       /* A rows are not 16-byte aligned and the kernel needs them aligned: a
                                kernel with shifted loads reads A (pointers are checked per run);
                                0 for kernels that read any alignment */
    int32_t b_guarded;       /* the same for B, and whenever N is not a whole number of 16-byte
                                pieces (the last piece of a B row would cross N) */
    char name[96];           /* kernel name, e.g. "bf16_t256x256x64_w2x4_s2_direct_xor_wide_reuse" */
    int64_t n_main;          /* columns the kernel above covers: N, or for a split plan the first
                                N - r, the last r (<= 16) going to `rem_name` */
    char rem_name[96];       /* split plans: the kernel of the last columns ("<name>_remcol": the
                                last column in the main kernel's own K loop); else "" */
    char packed_name[96];    /* the kernel gemm_run_ws runs on repacked operands (its plan's
                                `name`); "" for plans that carry no repack */
    int32_t waves_per_simd;  /* occupancy the kernel is compiled for: its registers (VGPRs + AGPRs,
                                512 per SIMD lane) leave room for at least this many waves per SIMD */
} tgemm_plan_info;

/* Fill *info for `plan`.  Returns TGEMM_OK or TGEMM_E_NULL. */
int gemm_plan_get_info(const tgemm_plan* plan, tgemm_plan_info* info);

/* Shader clock of a run (a diagnostic: the matrix cores' rate scales with
 * the shader clock, which the power budget lowers under load).
 * gemm_run_clocked is gemm_run, except that every workgroup of the plan's
 * tiled kernel (matrix-core or fp32; a split plan's thin remainder is not
 * clocked) writes TGEMM_CLOCK_VALUES = 6 values to clocks[6 w .. 6 w + 5],
 * w its workgroup index: the shader-clock counter (s_memtime) and the
 * 100 MHz real-time counter (s_memrealtime) when it starts; both again when
 * its first wave leaves the K loop, before any C store; and both once all its
 * memory instructions, the C stores included, have completed.  Summed over
 * workgroups, (end - start shader ticks) / (end - start real ticks) x 100 MHz
 * is the mean shader clock of the run, and the middle pair splits each
 * workgroup's time into its K loop and its C write-back.  The C written is
 * the same as gemm_run's, bit for bit.
 * clocks: device memory owned by the caller, 8-byte aligned, clocks_len
 * values; gemm_clock_slots(plan) values always suffice (it is the largest
 * grid among the kernels the plan may launch, times 6; 0 for a plan that
 * launches no tiled kernel, including empty products).
 * Returns what gemm_run returns, or TGEMM_E_NULL (NULL plan or clocks),
 * TGEMM_E_ARG (nothing to clock, or clocks_len below what the launched
 * kernel needs: then nothing is launched) or TGEMM_E_ALIGN. */
#define TGEMM_CLOCK_VALUES 6
int64_t gemm_clock_slots(const tgemm_plan* plan);
int gemm_run_clocked(const tgemm_plan* plan, const void* A, const void* B, void* C, uint64_t* clocks,
                     int64_t clocks_len, void* stream);

/* Occupancy of a plan's main kernel (a diagnostic for profile summaries, not
 * needed to run a plan): *workgroups_per_cu receives how many of its
 * workgroups one compute unit holds at once, as the HIP runtime's occupancy
 * calculator gives it from the kernel's registers, LDS and threads.
 * packed = 0: the kernel gemm_run launches; packed = 1: the kernel gemm_run_ws
 * launches after repacking (the same one when the plan has no repacked
 * form).  Needs the current device to be the gfx950 GPU the plan runs on.
 * Returns TGEMM_OK, TGEMM_E_NULL for a NULL argument, or a positive
 * hipError_t from the runtime. */
int gemm_kernel_occupancy(const tgemm_plan* plan, int32_t packed, int32_t* workgroups_per_cu);

/* Enumerate the variants compiled into the library for `dtype`.
 * gemm_variant_count returns how many; gemm_variant_get copies the i-th one
 * (0 <= i < count) and returns TGEMM_OK, or TGEMM_E_ARG for a bad index. */
int gemm_variant_count(int32_t dtype);
int gemm_variant_get(int32_t dtype, int32_t index, tgemm_variant* out);

/* Library version string. */
const char* tgemm_version(void);

/* LDS read-path probe (a measurement harness, not part of the GEMM).
 * Launches `workgroups` workgroups of 256 threads on `stream`; each fills a
 * 16 KiB LDS block with pattern(i) = i * 2654435761 ^ (i >> 7) for dword i
 * (mod 2^32), then for `reps` iterations reads 64 bytes per lane through
 *   kind 0: 16 x ds_read_b32       kind 1: 8 x ds_read_b64
 *   kind 2:  4 x ds_read_b128      kind 3: 8 x ds_read_b64_tr_b16
 * at the addresses of
 *   pattern 0 (linear, conflict-free at every width): instruction j of lane
 *     l of wave w reads W bytes (W = its width) at w * 4096 + j * 64 W + l W;
 *   pattern 1 (256-byte rows, 16-byte chunks XOR-permuted by row): four 16-byte
 *     pieces, piece c of lane l of wave w in iteration r at
 *     row * 256 + ((chunk ^ (row & 15)) * 16), row = (l & 31) + 32 (c & 1),
 *     chunk = ((l >> 5) + 2 (c >> 1) + 4 ((r + w) & 3)) & 15, each read as
 *     16 / W instructions at increasing offsets.
 * Each thread keeps acc = rotl16(acc, 1) ^ fold16(XOR of the dwords it read
 * in the iteration), fold16(x) = (x ^ x >> 16) & 0xffff, and writes it to
 * out[workgroup * 256 + thread]; the XOR over one workgroup's 256 values
 * does not depend on the kind (the transposing read only moves 16-bit
 * elements between the lanes of a 16-lane group).  out: device memory of
 * workgroups * 256 uint32 values, owned by the caller.  Returns TGEMM_OK,
 * TGEMM_E_ARG (kind outside 0..3, pattern outside 0..1, reps < 0,
 * workgroups < 1), TGEMM_E_NULL, TGEMM_E_ALIGN (out not 4-byte aligned) or
 * TGEMM_E_HIP (launch failed). */
int tgemm_lds_read_probe(int32_t kind, int32_t pattern, int32_t reps, int32_t workgroups, uint32_t* out,
                         void* stream);

/* Matrix-core rate probe (a measurement harness, not part of the GEMM): the
 * rate at which the chip sustains the matrix-core instruction of a GEMM type
 * for given operand bits, with no memory traffic.  The dense peak of the
 * datasheet assumes the nominal clock; the clock the power budget allows
 * depends on the operands (the "4.1 CUDA GEMM算子性能优化" page, section 2:
 * the roofline's compute ceiling is the one to measure against).
 *   kind 0: v_mfma_f32_32x32x16_bf16 (32768 flops per wave instruction)
 *   kind 1: v_mfma_i32_32x32x32_i8   (65536 ops per wave instruction)
 *   kind 2: v_fmac_f32, the fp32 vector fused multiply-add (128 flops per
 *           wave instruction), the ALU of the fp32 path
 *   kind 3: the bf16 matrix stream of the default 256 x 256 x 64 GEMM
 *           kernel's 128 x 64 wave tile, with its LDS fragment reads: per K
 *           step 8 matrix instructions on 4 A and 2 B fragments while the
 *           next step's are read (4 ds_read_b128, 4 ds_read_b64_tr_b16, one
 *           after each matrix instruction) from 16 KiB of LDS filled with the
 *           workgroup's first 16 KiB of operand bytes; 2 K steps per
 *           iteration; no barrier, no memory traffic (32768 flops per
 *           matrix instruction)
 *   kind 4: kind 3 plus that kernel's direct global -> LDS copies, 2 per K
 *           step per wave (global_load_lds_dwordx4, 1 KiB each) from the
 *           workgroup's 32 KiB of operand bytes into another 16 KiB of LDS
 *           that no read touches
 * Launches `workgroups` workgroups of 256 threads (4 waves, one per SIMD
 * while workgroups <= 256 compute units) on `stream`.  Thread t (global
 * index workgroup * 256 + thread) loads operands[8t .. 8t+3] (16 bytes each)
 * as A registers a[0..3] and operands[8t+4 .. 8t+7] as B registers b[0..3],
 * then runs `reps` iterations of 16 independent accumulators,
 * acc[i] += mma(a[i % 4], b[(i / 4) % 4]), i = 0..15 (16 * reps matrix
 * instructions per wave).  Operand layout of one instruction: lane l holds
 * row (A) / column (B) l % 32 and K elements 8 (l / 32) .. +7 (bf16) or
 * 16 (l / 32) .. +15 (int8); accumulator register r of lane l is row
 * 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
 * out[t] = the sum of the thread's 256 accumulator registers (bf16: fp32
 * bits of a sum taken in increasing i, then r; int8: the int32 sum mod 2^32).
 * Kind 2 instead reads the same 128 bytes as 16 floats x[0..15] (A
 * registers) and y[0..15] (B registers) and runs `reps` iterations of
 * acc[i] = fma(x[i], y[i], acc[i]), i = 0..15, from acc = 0; out[t] = fp32
 * bits of acc[0] + ... + acc[15] summed in increasing i.  It is built for up
 * to 8 waves per SIMD: `workgroups` / 256 compute units sets the waves that
 * share a SIMD (up to 8 workgroups of 4 waves per unit).
 * clocks[2 w], clocks[2 w + 1]: shader-clock ticks (s_memtime) and 100 MHz
 * real-time ticks (s_memrealtime) that wave 0 of workgroup w spent in the
 * loop.  operands (workgroups * 256 * 8 16-byte entries), out (workgroups *
 * 256 uint32) and clocks (2 * workgroups uint64) are device memory owned by
 * the caller.  Kinds 3 and 4 are built for 2 waves per SIMD (2 workgroups
 * per compute unit at workgroups = 512); their out[t] = fp32 bits of the sum
 * of the thread's 128 accumulator values (the same for both kinds: the
 * copies land where no read looks).  Returns TGEMM_OK, TGEMM_E_ARG (kind
 * outside 0..4, reps < 0, workgroups < 1), TGEMM_E_NULL, TGEMM_E_ALIGN
 * (operands not 16-byte, out not 4-byte or clocks not 8-byte aligned) or
 * TGEMM_E_HIP (launch failed). */
int tgemm_mfma_rate_probe(int32_t kind, int32_t reps, int32_t workgroups, const void* operands, uint32_t* out,
                          uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
