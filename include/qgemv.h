/*
 * qgemv — block-scaled small-M decode GEMV for AMD Instinct MI355X (gfx950)
 *
 *     Y[M, N] = A[M, K] . dequant(W)[N, K]^T (+ bias[N]),   1 <= M <= 16 (up to
 *     QGEMV_MAX_ROWS rows run as chunks of 16),
 *
 * with A, Y and the optional bias in fp16 or bf16 and fp32 accumulation. The weight W is quantized
 * in blocks along K in one of four formats:
 *
 *   QGEMV_FMT_U4     4-bit unsigned codes, fp16 scale and 4-bit zero point per
 *                    block: w = s * (q - zp). Layout [N, K/bs, bs/2] bytes, two
 *                    codes per byte with the lower k in the low nibble.
 *                    ("[CUDA] Batched small-M GEMV for MatMulNBits (4-bit/8-bit)",
 *                    Description: the [N, blocks, blob] layout.)
 *   QGEMV_FMT_U8     8-bit unsigned codes, fp16 scale and 8-bit zero point per
 *                    block. Layout [N, K/bs, bs] bytes. ("[CUDA] MatMulNBits
 *                    8-bit: wide fp16 M=1 kernel for decode GEMVs", Description:
 *                    per-block scale and zero point, (q - zp) exact.)
 *   QGEMV_FMT_FP8    OCP E4M3FN codes, row-major [N, K] bytes, one fp32 scale per
 *                    block of bs consecutive k: w = s * e4m3(q). ("[CUDA]
 *                    Block-scaled MatMul decode GEMV", FP8 mma paragraph.)
 *   QGEMV_FMT_NVFP4  packed E2M1 codes [N, K/2] bytes (lower k in the low nibble),
 *                    one E4M3 scale byte per 16 consecutive k, one fp32 tensor
 *                    scale: w = t * e4m3(s) * e2m1(q). (Same page, FP4 mma
 *                    paragraph.)
 *
 * Scales are row-major [N, K/bs]: fp16 bit patterns for U4/U8, float32 for FP8,
 * E4M3 bytes for NVFP4. Zero points: U4 packs two per byte, even block in the low
 * nibble, ceil((K/bs)/2) bytes per column; U8 has one byte per block, [N, K/bs].
 * A NULL zero-point pointer means the midpoint 2^(bits-1). FP8 and NVFP4 take no
 * zero points.
 *
 * Optional bias: one value per output column, in the activation dtype, added in
 * fp32 to the product of every row before the single rounding to the output type
 * (after the NVFP4 tensor scale, which belongs to dequant(W)). The pages' tests
 * cover such a bias ("[CUDA] Block-scaled MatMul decode GEMV: tensor cores, packed
 * FP4 decode and M-tiling", reviewed-changes table; "[CUDA] Pin FP8 GEMV residency
 * for grids just past two blocks per SM", a timeline note on its tests). NULL means none.
 *
 * All pointers passed to qgemv_create, qgemv_run, qgemv_run_ws and qgemv_run_noalloc
 * are DEVICE pointers, owned by the caller. The handle keeps the weight pointers (not
 * copies) and the caller keeps them alive until qgemv_destroy. The library allocates
 * no device memory: the one kernel that needs scratch memory (the K split across
 * workgroups of qgemv_run_ws) takes it from the caller, or, through qgemv_run_noalloc,
 * from a fixed device array the library holds.
 *
 * Every call returns QGEMV_OK (0) or a positive status; nothing aborts, prints or
 * throws across this interface. Arguments are validated before anything is
 * launched.
 */
#ifndef QGEMV_H_
#define QGEMV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMV_ABI_VERSION 6
/* Rows one plan carries; a call with more runs them as chunks of this many. */
#define QGEMV_MAX_M 16
/* Rows one call accepts. */
#define QGEMV_MAX_ROWS 65536
/* Bytes of the library's own device scratch array that qgemv_run_noalloc uses in place
 * of a workspace (one copy per device, held until the process ends). */
#define QGEMV_NOALLOC_SCRATCH_BYTES (16u << 20)
/* Most launches qgemv_tune_candidates lists (and qgemv_tune times) for one M. */
#define QGEMV_TUNE_MAX_CANDIDATES 256

/* Weight formats. */
enum qgemv_format {
    QGEMV_FMT_U4 = 1,
    QGEMV_FMT_U8 = 2,
    QGEMV_FMT_FP8 = 3,
    QGEMV_FMT_NVFP4 = 4
};

/* Activation (and output) element type. */
enum qgemv_act_dtype {
    QGEMV_ACT_F16 = 1,
    QGEMV_ACT_BF16 = 2
};

/* Status codes. */
enum qgemv_status {
    QGEMV_OK = 0,
    QGEMV_E_NULL = 1,     /* a required pointer is NULL */
    QGEMV_E_SHAPE = 2,    /* M outside [1, QGEMV_MAX_ROWS], N < 1, K < 1 or K % block_size != 0 */
    QGEMV_E_BLOCK = 3,    /* block size not supported for the format */
    QGEMV_E_FORMAT = 4,   /* unknown format / dtype, or zero points given for FP8/NVFP4 */
    QGEMV_E_DEVICE = 5,   /* no usable device, or the device is not gfx950 */
    QGEMV_E_LAUNCH = 6,   /* the kernel launch reported an error */
    QGEMV_E_ARG = 7,      /* other invalid argument (struct size, flags, plan request) */
    QGEMV_E_ALLOC = 8,    /* host memory for the handle (or qgemv_tune's device buffer) could not be allocated */
    QGEMV_E_WORKSPACE = 9, /* qgemv_run_ws: the plan needs a workspace and none, or too small
                              or misaligned a one, was given */
    QGEMV_E_SCRATCH = 10   /* qgemv_run_noalloc: the plan needs more workspace than
                              QGEMV_NOALLOC_SCRATCH_BYTES */
};

/* Kernel families (qgemv_plan_info.family; also usable in QGEMV_FLAG_FORCE). */
enum qgemv_family {
    QGEMV_FAMILY_AUTO = 0,
    QGEMV_FAMILY_STREAM = 1,   /* vector kernel: wave per column group, fp32 dot products */
    QGEMV_FAMILY_MFMA = 2,     /* matrix-core kernel: 16-column tiles, rows in 4-row groups */
    QGEMV_FAMILY_GENERIC = 3   /* element-wise kernel for any shape / alignment */
};

/* Flags (qgemv_desc.flags). Bits 0..3: forced family (0 = automatic choice).
 * Bits 4..6: forced number of K parts split across workgroups by qgemv_run_ws (v ->
 * 2^(v-1): 1, 2, 4 or 8 parts, at most one per K step of the MFMA family; 0 =
 * automatic). Bit 7: the persistent streaming kernel loads block metadata per chunk
 * with narrow (8- and 16-bit) loads, never as one window per round (8-bit codes) or as
 * the aligned dwords that hold it (for A/B comparisons).
 * Bits 8..11: forced K split of the MFMA family (0 = automatic; otherwise 1, 2, 4 or
 * 8 waves share the K range of a column tile). Bits 12..14: waves per workgroup of the
 * persistent streaming kernel with several rows per pass (v -> 4v, v = 1..4; 0 =
 * automatic; capped at 8 with two columns per wave and at 12 for four rows of 4-bit
 * codes in 16-wide blocks, the most those fit without spilling registers). Bit 15:
 * keep persistent grids as the dispatcher sizes them, without the create-time cut to
 * the workgroups the kernel's registers leave resident per CU (for A/B comparisons).
 * Bit 16: never pick the MFMA family.
 * Bits 17/18: MFMA family never / always stages the activations in LDS (when they
 * fit); neither set = automatic. Bits 19/20: MFMA family never / always (when
 * eligible) streams the weights through the LDS DMA ring.
 * Streaming family at M = 1 (the persistent one-row kernel): bits 21..22 force the
 * columns per wave (1 -> 1, 2 -> 2, 3 -> 4), bits 23..24 the chunks per lane per
 * batch (1 -> 2, 2 -> 3, 3 -> 4), bits 25..27 the resident waves per CU the grid is
 * sized for (v -> 4v); 0 = automatic. Bit 28: use the non-persistent streaming kernel
 * at M = 1 as well. Bits 29..30: MFMA ring depth (register ring: 1 -> 4 slots, 2 -> 8;
 * DMA ring: 1 -> 2 slots per wave, 2 -> 3 where they fit in LDS; 0 = automatic). Bit 31: 16-wave workgroups for the one-row streaming kernel with one
 * column per wave (also chosen automatically when the columns fill 8 to 16 waves per
 * CU and neither bits 21..22 nor 25..27 are set). None of these changes a result's
 * bits except the family choice, the K split and the K parts; they exist for A/B
 * comparisons and tuning. */
#define QGEMV_FLAG_FAMILY_MASK 0x0000000Fu
#define QGEMV_FLAG_KPARTS_SHIFT 4
#define QGEMV_FLAG_KPARTS_MASK 0x00000070u
#define QGEMV_FLAG_STREAM_META_CHUNK 0x00000080u
#define QGEMV_FLAG_KSPLIT_SHIFT 8
#define QGEMV_FLAG_KSPLIT_MASK 0x00000F00u
#define QGEMV_FLAG_STREAM_NWG_SHIFT 12
#define QGEMV_FLAG_STREAM_NWG_MASK 0x00007000u
#define QGEMV_FLAG_NO_RESIDENCY_FIT 0x00008000u
#define QGEMV_FLAG_NO_MFMA 0x00010000u
#define QGEMV_FLAG_STAGE_A_OFF 0x00020000u
#define QGEMV_FLAG_STAGE_A_ON 0x00040000u
#define QGEMV_FLAG_RING_OFF 0x00080000u
#define QGEMV_FLAG_RING_ON 0x00100000u
#define QGEMV_FLAG_STREAM_CPW_SHIFT 21
#define QGEMV_FLAG_STREAM_CPW_MASK 0x00600000u
#define QGEMV_FLAG_STREAM_UNR_SHIFT 23
#define QGEMV_FLAG_STREAM_UNR_MASK 0x01800000u
#define QGEMV_FLAG_STREAM_WPC_SHIFT 25
#define QGEMV_FLAG_STREAM_WPC_MASK 0x0E000000u
#define QGEMV_FLAG_STREAM_CLASSIC 0x10000000u
#define QGEMV_FLAG_MFMA_DEPTH_SHIFT 29
#define QGEMV_FLAG_MFMA_DEPTH_MASK 0x60000000u
#define QGEMV_FLAG_STREAM_WIDE_WG 0x80000000u

/* Problem description. struct_size must be sizeof(qgemv_desc). */
typedef struct qgemv_desc {
    uint32_t struct_size;
    int32_t format;        /* enum qgemv_format */
    int32_t act_dtype;     /* enum qgemv_act_dtype, for A and Y */
    int32_t block_size;    /* U4/U8/FP8: 16, 32, 64, 128 or 256; NVFP4: 16 */
    int64_t N;             /* output columns (weight rows) */
    int64_t K;             /* reduction length */
    const void *W;         /* device: packed codes (layout above) */
    const void *scales;    /* device: block scales [N, K/bs] */
    const void *zero_points; /* device: zero points, or NULL */
    float tensor_scale;    /* NVFP4 tensor scale (multiplies); ignored otherwise */
    uint32_t flags;        /* QGEMV_FLAG_* */
    const void *bias;      /* device: [N] bias in the activation dtype, or NULL; kept by
                              the handle like the weight pointers (ABI version 2) */
} qgemv_desc;

/* What qgemv_plan / qgemv_select report about a launch. */
typedef struct qgemv_plan_info {
    int32_t family;          /* enum qgemv_family actually used */
    int32_t rows_per_pass;   /* rows of A carried by one pass over the weight */
    int32_t passes;          /* passes over the weight for this M (the matrix family's
                                passes are one launch each, in order, on the stream) */
    int32_t cols_per_wave;   /* output columns one wave owns at a time */
    int32_t ksplit;          /* waves of a workgroup sharing one column tile's K */
    int32_t waves_per_wg;    /* waves per workgroup */
    int64_t grid;            /* workgroups launched (qgemv_plan: a persistent grid cut at create to
                                the workgroups that stay resident at once; qgemv_select, which asks
                                no device, reports the grid before that cut) */
    int32_t lds_bytes;       /* dynamic LDS per workgroup */
    int32_t variant;         /* family-specific variant bits. MFMA: bit 0 = activations staged in
                                LDS, bit 1 = weights through the LDS DMA ring (4-step slots,
                                two per wave), bit 2 = three DMA-ring slots per wave, bit 3 =
                                8-slot register ring (else 4, or fewer where the registers do
                                not allow 4).
                                Streaming: bit 0 = persistent kernel (1, 2 or 4 rows per pass),
                                bits 1..2 = chunks per lane per batch (2 -> 2, 3 -> 3, 0 -> 4),
                                bit 3 = block metadata loaded as one window per round (8-bit
                                codes), bit 4 = as the aligned dwords that hold it (4-bit,
                                8-bit and NVFP4 codes, where the rows are whole dwords),
                                bit 5 = a grid of every column group, one per wave, instead
                                of a persistent grid (one row of 1-byte codes) */
    int32_t kparts;          /* K parts split across workgroups (1 = none; only qgemv_run_ws
                                splits, ABI version 3) */
    int32_t reserved;        /* 0 */
    int64_t workspace_bytes; /* device workspace this launch needs (0 without K parts) */
} qgemv_plan_info;

typedef struct qgemv_handle qgemv_handle;

/* Validate d, read the device's properties (device index, or -1 for the current
 * device), and return a handle in *out. The weight pointers are kept, not copied.
 * Environment overrides (QGEMV_FORCE_FAMILY, QGEMV_FORCE_KSPLIT, QGEMV_NO_MFMA) are
 * read here once, never per call; a switch set to 0, false, off or no is off. Every
 * launch the handle can make (M = 1..16, with and without a workspace, aligned or not)
 * is planned here too, so a run only looks its plan up. The pages' review fixes ask for
 * exactly this split: device properties passed to each instance instead of a
 * process-wide cached SM count, and kill switches parsed as booleans ("[CUDA]
 * Block-scaled MatMul decode GEMV: tensor cores, packed FP4 decode and M-tiling",
 * review fixes). The handle is plain host memory (QGEMV_E_ALLOC if it cannot be
 * allocated), owned by the caller until qgemv_destroy. Returns QGEMV_E_DEVICE for a
 * device that is not gfx950 and the descriptor's own status for an invalid d. */
int qgemv_create(qgemv_handle **out, const qgemv_desc *d, int device);

/* Enqueue Y[M, N] = A[M, K] . dequant(W)^T on hip_stream (a hipStream_t; NULL = the
 * default stream). A is [M, K] row-major and Y is [M, N] row-major, both device
 * pointers in the handle's activation dtype. Asynchronous: no host sync, no
 * allocation, no environment read. Safe to call concurrently on different streams
 * (only qgemv_tune changes a handle after create, and it must not overlap any other
 * call on it). The call must be made with the handle's device current.
 *
 * The kernels are built for M <= QGEMV_MAX_M (16) rows, the decode regime of the
 * pages. More rows, up to QGEMV_MAX_ROWS, run as chunks of 16 rows (the last one
 * shorter), one after another on the stream, each with the plan for 16 rows: each
 * chunk reads the whole weight again, so this serves short prefills rather than
 * replacing a GEMM. A row's bits do not depend on the chunk that carries it. (The
 * pages' batched small-M kernel falls back to another path past its M limit; "[CUDA]
 * Batched small-M GEMV for MatMulNBits (4-bit/8-bit)", Description.) */
int qgemv_run(const qgemv_handle *h, const void *A, void *Y, int M, void *hip_stream);

/* The same product, where the K range may also be split across workgroups: for N so
 * small that the column tiles, even with the K split inside a workgroup, leave
 * compute units idle, each of `kparts` workgroups takes one contiguous part of the
 * K steps of a tile group, writes its fp32 partial tile to the workspace, and the
 * last of them to finish (counted by an atomic counter per tile group) adds the
 * partials in fixed part order and writes Y. This follows the pages' opt-in split-K
 * GEMV with its global workspace, completion counters and last-block reduction in
 * fixed slice order ("[CUDA] MatMul: add an opt-in split-K GEMV", Kernel and
 * dispatch; review threads on the workspace's visibility), here for the quantized
 * formats. The order of the fp32 sums depends on (format, N, K, block size, flags)
 * and the device's compute-unit count, and on M where the activation rows of this M
 * do not fit in LDS: with tile groups for at most half the compute units the K range
 * is then cut in 2 parts; where instead the unsplit tile groups fill between an
 * eighth of the compute units and all of them, the split inside a workgroup is dropped
 * and 2 to 8 parts taken (one round of workgroups, more where this M's rows need them
 * to stage). Rows stay
 * bit-identical whatever tile carries them within a call. Across M they stay so only
 * when the flags force both the kernel family (the automatic choice takes the
 * streaming family at small M and the matrix family above it, and the two add in
 * different orders) and the part count; the bits can differ from qgemv_run's where
 * qgemv_run does not split (within the same error bound).
 *
 * workspace: device memory of at least qgemv_workspace_size(h, M) bytes, 256-byte
 * aligned, owned by the caller: completion counters, then fp32 partial tiles. Zero
 * the whole workspace once before its first use (hipMemset). Every run that
 * completes leaves all of it zero again (the last workgroup of a tile group resets
 * its counter with an atomic store and clears the partials it read), so later runs
 * need no clearing and one workspace can serve any handle and any M in turn. Runs
 * that overlap in time (on different streams) must not share a workspace. A plan
 * without K parts ignores the workspace (it may then be NULL). Returns
 * QGEMV_E_WORKSPACE when the plan needs a workspace and none, or too small or
 * misaligned a one, is given. */
int qgemv_run_ws(const qgemv_handle *h, const void *A, void *Y, int M, void *workspace,
                 size_t workspace_bytes, void *hip_stream);

/* qgemv_run_ws without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc. The same plans and kernels as qgemv_run_ws,
 * with the library's own device array of QGEMV_NOALLOC_SCRATCH_BYTES (16 MiB, one per
 * device, set up and zeroed when the first handle for that device is created, held
 * until the process ends) as the workspace; the result is bit-identical to
 * qgemv_run_ws's. The call allocates nothing and frees nothing. Returns
 * QGEMV_E_SCRATCH, before any launch, when the plan for M rows needs more workspace
 * than the array holds (qgemv_workspace_size reports the need; automatic plans on a
 * 256-CU device need at most 16 MiB: long rows over nearly 32768 columns at 16 rows,
 * in 8 K parts; 4 MiB elsewhere), and QGEMV_E_DEVICE when the array could not be
 * set up. Every completed call leaves the area it used zero again, which is how the
 * next call finds its counters. All calls on one device share the one array: calls
 * that overlap in time on one device (different streams, or threads) race on it and
 * must be serialized by the caller. The other arguments and the threading contract
 * are those of qgemv_run_ws. */
int qgemv_run_noalloc(const qgemv_handle *h, const void *A, void *Y, int M, void *hip_stream);

/* Bytes of workspace qgemv_run_ws needs for M rows (0 when its plan has no K parts).
 * Sized at M = QGEMV_MAX_M, a workspace serves every M. */
int qgemv_workspace_size(const qgemv_handle *h, int M, size_t *bytes);

/* The launch qgemv_run (with_workspace = 0) or qgemv_run_ws (with_workspace != 0)
 * would make for M rows (pointers as given at create; A and Y assumed 16-byte
 * aligned), written to *out (caller-owned): the kernel family, grid, K split, K parts
 * and workspace. It makes the dispatcher's choice visible, as the pages' tests check
 * which kernel a shape reaches and its fallback path ("[CUDA] MatMulNBits 8-bit: wide
 * fp16 M=1 kernel for decode GEMVs", review: which test shapes reach the new path).
 * Returns QGEMV_E_SHAPE for M outside [1, QGEMV_MAX_ROWS]. */
int qgemv_plan(const qgemv_handle *h, int M, int with_workspace, qgemv_plan_info *out);

/* Pure host selector, no device needed and no HIP call made: the plan for d at M rows
 * on a device with cu_count compute units, assuming 16-byte aligned pointers;
 * with_workspace as for qgemv_plan; *out is caller-owned. The pages test their
 * occupancy window the same way, as a pure predicate at a fixed SM count so that the
 * expectations do not move with the test machine ("[CUDA] Pin FP8 GEMV residency for
 * grids just past two blocks per SM", Tests). Returns QGEMV_E_ARG for cu_count < 1 and
 * the descriptor's status for an invalid d. */
int qgemv_select(const qgemv_desc *d, int M, int cu_count, int with_workspace, qgemv_plan_info *out);

/* What qgemv_tune measured and kept. */
typedef struct qgemv_tune_info {
    int32_t candidates;     /* distinct launches timed (the automatic one included) */
    int32_t rounds;         /* timing rounds; each times `reps` calls of every candidate */
    uint32_t chosen_flags;  /* flag bits, over the descriptor's, that give the kept launch
                               (0 = the automatic one); a handle created with them in
                               qgemv_desc.flags plans the same launch for this M */
    int32_t reserved;       /* 0 */
    double auto_us;         /* median time of the automatic launch's timed calls (each cold) */
    double chosen_us;       /* the same for the kept launch */
} qgemv_tune_info;

/* Pure host list, no device needed and no HIP call made: the flag sets that qgemv_tune
 * would time for d at M rows (1..QGEMV_MAX_M) on cu_count compute units (16-byte
 * aligned pointers assumed; with_workspace as for qgemv_plan). flags_out[0] is 0, the
 * automatic plan; each later entry, added to the descriptor's flags, gives a launch of
 * its own with the automatic plan's kernel family, K split and K parts, hence the same
 * order of every fp32 sum and the same result bits, only spread over waves and fetched
 * differently (streaming: columns per wave, chunks per batch, waves per workgroup,
 * grid, classic or persistent kernel, metadata loads; matrix family: activation
 * staging, register or LDS DMA ring, ring depth; either: the create-time residency
 * cut). Dimensions the descriptor's flags already fix are left as they are. Writes at
 * most max entries and their number to *count. Returns QGEMV_E_SHAPE for M outside
 * [1, QGEMV_MAX_M], QGEMV_E_ARG for cu_count < 1 or max < 1, and the descriptor's
 * status for an invalid d. */
int qgemv_tune_candidates(const qgemv_desc *d, int M, int cu_count, int with_workspace, uint32_t *flags_out,
                          int max, int *count);

/* Online choice of the launch for M rows (1..QGEMV_MAX_M), the per-shape profiling the
 * pages' reviewers ask for instead of thresholds tuned on one machine ("[CUDA] Batched
 * small-M GEMV for MatMulNBits (4-bit/8-bit)", review). Times every launch that
 * qgemv_tune_candidates lists for this handle's device (after the create-time
 * residency cut; launches that come out equal are timed once) on the caller's A, Y
 * and workspace, `rounds` rounds of `reps` calls each (0 for either: 5 and 10),
 * interleaved so that every candidate sees the same conditions, and keeps the launch
 * with the least median time per call in the handle, for qgemv_run (with_workspace
 * = 0) or qgemv_run_ws and qgemv_run_noalloc (with_workspace != 0), for the pointer
 * alignment that A and Y have. The automatic launch is kept unless another is faster
 * by more than 2%. Every launch listed gives the same bits, so results do not change;
 * only the time does. Calls with more than 16 rows use the 16-row plan and so follow a
 * tuning of M = 16.
 *
 * Every timed call is cold, as in a decode step, where each weight is read once per
 * token among many times the caches' size of others: before it, a read sweep over a
 * 512 MiB device buffer (twice MI355X's 256 MB last-level cache) evicts the weight,
 * and the call alone is timed between two HIP events. A, Y, workspace and
 * workspace_bytes are as for qgemv_run_ws (the workspace only when with_workspace != 0
 * and the plan has K parts); Y is written many times and holds the kept launch's
 * product on return. The call waits for its own work on hip_stream (HIP events) and
 * returns after it; it allocates the sweep buffer on the handle's device for its
 * duration and frees it before returning. It changes the handle: no other call on the
 * same handle may overlap it. *out (may be NULL) receives what was measured. Returns
 * QGEMV_E_SHAPE for M outside [1, QGEMV_MAX_M], QGEMV_E_WORKSPACE when the plan needs
 * a workspace that is not given, QGEMV_E_ALLOC when the sweep buffer cannot be
 * allocated, QGEMV_E_LAUNCH when a launch or an event fails (the handle keeps the plan
 * it had in each case). */
int qgemv_tune(qgemv_handle *h, const void *A, void *Y, int M, int with_workspace, void *workspace,
               size_t workspace_bytes, int rounds, int reps, void *hip_stream, qgemv_tune_info *out);

/* Release the handle (NULL is ignored). Does not touch the caller's buffers or wait
 * for launches in flight: the caller keeps the weight buffers alive until the work it
 * enqueued has finished. */
void qgemv_destroy(qgemv_handle *h);

/* Static English text for a status code (owned by the library, never freed). Every
 * entry point reports failure as a status instead of aborting or printing, as the
 * pages' launchers return an error status to the operator that then falls back
 * ("[CUDA] MatMulNBits 8-bit: wide fp16 M=1 kernel for decode GEMVs", Description:
 * the guarded dispatch and its fallback). */
const char *qgemv_status_str(int status);

/* ABI version of the loaded library (QGEMV_ABI_VERSION it was built with). */
int qgemv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H_ */
