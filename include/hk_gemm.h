/*
 * hk_gemm.h -- C ABI of libhkgemm.so: dense C = A * B^T on one MI355X (gfx950).
 *
 * The operation.  The GeekNews summary "HipKittens: fast and furious AMD
 * kernels" (section "Performance results") reports a GEMM kernel that is the
 * fastest in BF16 and in FP8; its companion "How to make AMD GPUs go brrr"
 * (section "Real kernel example") shows the BF16 GEMM hot loop.  Neither page
 * gives an interface, so this one is ours:
 *
 *     C[i*ldc + j] = bf16_rne( s * sum_{k<K} A[i*lda + k] * B[j*ldb + k] )
 *
 * for 0 <= i < M, 0 <= j < N, with FP32 accumulation.  A is M x K and B is
 * N x K, both row-major with K contiguous (so B is used transposed), C is
 * M x N row-major.  s = 1 for BF16 inputs, s = scale_a * scale_b for FP8.
 * hk_gemm_ex also takes either operand stored the other way round (K x M,
 * K x N: hk_layout below), which gives A * B, A^T * B^T and A^T * B.
 *
 * Element types.  BF16: 16-bit bfloat16 bit patterns.  FP8: OCP E4M3FN bytes
 * (bias 7, largest finite 448, S.1111.111 is NaN), one fp32 scale per tensor
 * passed by value.  The pages quote only an MXFP8 peak rate and no scaling
 * scheme; per-tensor scales are the plainest reading.  Block-scaled MXFP8 has
 * an entry point of its own (hk_gemm_mxfp8, below).  C is always bf16,
 * rounded to nearest even from the fp32 accumulator (times s for FP8).
 *
 * Ownership and ordering.  All pointers are device pointers owned by the
 * caller; the library never allocates or frees memory.  Every call only
 * enqueues work on `stream` (0 = the null stream) and returns; it never
 * synchronises.  Buffers must stay valid until that work has completed.
 * Calls are thread-safe; the library keeps only a per-device property cache.
 *
 * Errors.  Every function returns an hk_status and never aborts or throws.
 * Arguments are validated before any HIP call; invalid ones return
 * HK_ERROR_INVALID_VALUE and enqueue nothing: negative M, N or K; a NULL
 * pointer for an operand that would be read or written; lda < K or ldb < K
 * (when K > 0; lda < M or ldb < N for an operand stored K-strided); ldc < N;
 * an unknown dtype, schedule, grid order or layout; a
 * non-finite scale.  M == 0 or N == 0 is a no-op success.  K == 0 writes
 * zeros to C (the empty sum is +0).  A failure reported by the HIP runtime at
 * launch returns HK_ERROR_LAUNCH.  HK_ERROR_NOT_SUPPORTED is returned when an
 * explicitly requested schedule cannot run the given shape or alignment
 * (the automatic choice never returns it).
 */
#ifndef HK_GEMM_H
#define HK_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; 0 selects the null stream. */
typedef struct ihipStream_t *hk_stream_t;

typedef enum hk_status {
    HK_SUCCESS = 0,
    HK_ERROR_INVALID_VALUE = 1,
    HK_ERROR_NOT_SUPPORTED = 2,
    HK_ERROR_LAUNCH = 3
} hk_status;

typedef enum hk_dtype {
    HK_DTYPE_BF16 = 0,
    HK_DTYPE_FP8_E4M3 = 1,
    HK_DTYPE_MXFP8_E4M3 = 2  /* block-scaled FP8: hk_gemm_mxfp8 (hk_gemm_plan describes it) */
} hk_dtype;

/*
 * Intra-CU schedule ("How to make AMD GPUs go brrr", section "Intra-processor
 * scheduling: wave patterns"):
 *   PINGPONG8   8 waves per CU in two groups of four; while one group issues
 *               its matrix-core cluster the other issues its memory cluster,
 *               and they swap at workgroup barriers; persistent like
 *               INTERLEAVE4;
 *   INTERLEAVE4 4 waves per CU, each interleaving its own loads with its
 *               matrix-core instructions; persistent (one workgroup per CU
 *               walks its share of the output tiles);
 *   BASIC       a plain LDS-staged kernel with no alignment requirements,
 *               used for shapes or strides the fast schedules do not accept;
 *   INTERLEAVE8 8 waves per CU, each interleaving its own loads with its
 *               matrix-core instructions (BF16 only);
 *   SMALLTILE   128 x 128 tiles with four K stages in flight, for outputs
 *               too small to give every CU a 256 x 256 tile;
 *   PRODUCER_CONSUMER  4 waves that only load and 4 that only compute, 256 x
 *               128 tiles (BF16 only; the wave-specialised design the pages
 *               compare the ping-pong against, kept as an ablation).
 * AUTO, when the fast-path conditions hold (16-byte aligned A and B, K, lda
 * and ldb whole 16-byte chunks), picks SMALLTILE if the output has at most
 * one 256 x 256 tile per four compute units and INTERLEAVE4 (the fastest on
 * MI355X at large sizes for both dtypes) otherwise; else BASIC.
 */
typedef enum hk_schedule {
    HK_SCHEDULE_AUTO = 0,
    HK_SCHEDULE_PINGPONG8 = 1,
    HK_SCHEDULE_INTERLEAVE4 = 2,
    HK_SCHEDULE_BASIC = 3,
    HK_SCHEDULE_INTERLEAVE8 = 4,
    HK_SCHEDULE_SMALLTILE = 5,
    HK_SCHEDULE_PRODUCER_CONSUMER = 6
} hk_schedule;

/*
 * Workgroup-to-tile order ("How to make AMD GPUs go brrr", section
 * "Inter-processor scheduling: chiplet-aware approach"): the hardware deals
 * workgroups to the 8 chiplets (XCDs) round-robin, so the order decides what
 * each chiplet's L2 and the shared last-level cache can reuse.
 *   ROW_MAJOR  workgroup w computes tile (w / tiles_n, w % tiles_n);
 *   XCD        within each window of co-resident workgroups, the ones dealt
 *              to one chiplet get a compact block of output tiles, and the
 *              window as a whole covers a compact region (grouped order of
 *              group_m tile rows).
 * AUTO is XCD.
 */
typedef enum hk_grid_order {
    HK_GRID_AUTO = 0,
    HK_GRID_ROW_MAJOR = 1,
    HK_GRID_XCD = 2
} hk_grid_order;

/*
 * Storage of an operand.  The GeekNews summary "HipKittens: fast and furious
 * AMD kernels" (section "Real kernel example") lists mma_AtB among the tile
 * operations of the hot loops, i.e. products with a transposed operand; the
 * page fixes no global layout, so both are offered for each operand:
 *   K_CONTIGUOUS  A(i, k) = A[i*lda + k] (A stored M x K), B(j, k) =
 *                 B[j*ldb + k] (B stored N x K): the default, lda, ldb >= K;
 *   K_STRIDED     A(i, k) = A[k*lda + i] (A stored K x M, lda >= M),
 *                 B(j, k) = B[k*ldb + j] (B stored K x N, ldb >= N).
 * C = sum_k A(i, k) B(j, k) in every case: A K_STRIDED gives A^T-style
 * products, B K_STRIDED gives C = A * B with B as stored, and both give the
 * pages' A^T * B.  K_STRIDED runs on INTERLEAVE4 (BF16 and FP8 with
 * per-tensor scales; chosen by AUTO) or BASIC.  INTERLEAVE4 needs, per
 * K_STRIDED operand, 16-byte alignment, the stride and M (or N) in whole
 * 16-byte chunks (multiples of 8 for BF16, of 16 for FP8), and (K + 128)
 * rows (BF16) or (K + 256) rows (FP8) of stride below 2^31 bytes; the other
 * schedules, and MXFP8, return HK_ERROR_NOT_SUPPORTED for it.
 */
typedef enum hk_layout {
    HK_LAYOUT_K_CONTIGUOUS = 0,
    HK_LAYOUT_K_STRIDED = 1
} hk_layout;

/*
 * Repacking an operand whose rows straddle cache lines.  The fast schedules
 * fetch each operand row in 128-byte segments of K.  When a K-contiguous
 * operand's row stride in bytes is not a multiple of 128 (lda = 8200 BF16
 * elements is 16 400 bytes), every segment but one in eight spans two cache
 * lines, which doubles the lines the loads touch: measured on MI355X, the
 * BF16 8191 x 28670 x 8200 product ran 3212 us as given against 2611-2707 us
 * on the same values copied to a padded stride.  With a workspace, the call
 * first copies such an operand (all M or N rows, K elements each) to a
 * stride that is a whole number of cache lines (the row bytes rounded up to
 * a multiple of 1024, plus 1024 when that is a multiple of 8192), then runs
 * the product on the copy.  The result is bit-identical either way.
 *   REPACK_AUTO    repack when the product is large enough to pay for the
 *                  copy (M*N >= 4096*(M+N)) and the workspace suffices;
 *                  otherwise run on the operands as given;
 *   REPACK_NEVER   never;
 *   REPACK_ALWAYS  repack every straddling K-contiguous operand, whatever
 *                  the size (HK_ERROR_INVALID_VALUE if the workspace is too
 *                  small).
 * Repacking applies to the fast schedules only (not BASIC) and to
 * K-contiguous operands only; hk_gemm_workspace_size reports the bytes.
 */
typedef enum hk_repack {
    HK_REPACK_AUTO = 0,
    HK_REPACK_NEVER = 1,
    HK_REPACK_ALWAYS = 2
} hk_repack;

/*
 * Optional knobs for hk_gemm_ex.  Zero-initialise for the defaults.
 *
 * clock_stamps: NULL, or a caller-owned device buffer of 32 uint64_t (256
 * bytes, 16-byte aligned; misaligned is HK_ERROR_INVALID_VALUE) that records
 * the clocks of the launch.  The persistent kernels (INTERLEAVE4, PINGPONG8) write, for each
 * of the first 8 workgroups x (the first workgroup dealt to chiplet x; the
 * hardware deals workgroups to the 8 chiplets round-robin), the chiplet's
 * shader-clock counter and the constant-rate counter as the workgroup starts
 * (words 4x, 4x+1) and as it ends (words 4x+2, 4x+3).  The chiplet's mean
 * clock over the launch is then (word 4x+2 - word 4x) / (word 4x+3 - word
 * 4x+1) times the constant counter's rate, hk_wall_clock_khz().  Words of
 * workgroups that do not exist, and the whole buffer under any other
 * schedule, are left untouched.  The kernels and their results are the same
 * with or without it.
 *
 * workspace, workspace_bytes: NULL and 0, or a caller-owned device buffer
 * (256-byte aligned; otherwise HK_ERROR_INVALID_VALUE) the call may use for
 * repacked operands (hk_repack above).  Its contents on entry do not matter
 * and are not preserved; it must stay valid until the call's work has
 * completed on the stream, and two calls that may run at the same time need
 * two workspaces.
 *
 * scale_a_dev, scale_b_dev: NULL, or a caller-owned device fp32 (4-byte
 * aligned) that the kernel reads when it runs, in stream order, in place of
 * the by-value scale_a (scale_b).  FP8 per-tensor scales only: with BF16 a
 * non-NULL pointer is HK_ERROR_INVALID_VALUE, as is a misaligned one.  For
 * scales computed on the device (an amax reduction, delayed scaling) this
 * needs no copy to the host, and a captured HIP graph reads the values
 * current at each replay.  The product is s = a * b in fp32, the same
 * rounding as for by-value scales, so equal values give bit-identical C.
 * The host cannot check these values: a non-finite one makes C non-finite,
 * where a non-finite by-value scale is HK_ERROR_INVALID_VALUE (a by-value
 * scale that a pointer replaces is not checked).
 */
typedef struct hk_gemm_opts {
    int32_t schedule;    /* hk_schedule */
    int32_t grid_order;  /* hk_grid_order */
    int32_t group_m;     /* tile rows per group in the XCD order; 0 = default */
    int32_t window;      /* co-resident workgroups per window; 0 = CU count */
    int32_t layout_a;    /* hk_layout of A */
    int32_t layout_b;    /* hk_layout of B */
    uint64_t *clock_stamps; /* NULL, or 32 words of clock record (above) */
    void *workspace;        /* NULL, or device memory for repacked operands */
    int64_t workspace_bytes; /* its size in bytes */
    int32_t repack;      /* hk_repack */
    int32_t reserved;    /* must be zero */
    const float *scale_a_dev; /* NULL, or device fp32 read in place of scale_a */
    const float *scale_b_dev; /* NULL, or device fp32 read in place of scale_b */
} hk_gemm_opts;

/* What a call with these arguments would launch (filled by hk_gemm_plan). */
typedef struct hk_gemm_plan_info {
    int32_t schedule;      /* the schedule actually used */
    int32_t grid_order;    /* the order actually used */
    int32_t tile_m, tile_n, tile_k;  /* tile_k in elements */
    int32_t threads;       /* threads per workgroup */
    int64_t tiles_m, tiles_n;
    int64_t workgroups;    /* 1-D grid size */
    int32_t lds_bytes;
    int32_t group_m, window;
    char kernel_name[96];  /* device symbol, as profilers print it */
} hk_gemm_plan_info;

/* BF16 x BF16 -> BF16 (fp32 accumulate).  Default schedule and grid order. */
hk_status hk_gemm_bf16(const void *A, const void *B, void *C,
                       int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc,
                       hk_stream_t stream);

/* E4M3FN x E4M3FN -> BF16, C = scale_a * scale_b * (A * B^T). */
hk_status hk_gemm_fp8(const void *A, const void *B, void *C,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc,
                      float scale_a, float scale_b,
                      hk_stream_t stream);

/*
 * MXFP8: E4M3FN elements with one E8M0 scale per 32 consecutive K-elements
 * of a row (the block-scaled FP8 of the OCP Microscaling (MX) Formats
 * specification v1.0, the format of the 5.0 PF FP8 peak quoted in "How to
 * make AMD GPUs go brrr", section "AMD CDNA GPU structure"):
 *
 *     C[i*ldc + j] = bf16_rne( sum_{k<K} XA(i, k/32) A[i*lda + k] * XB(j, k/32) B[j*ldb + k] )
 *
 * with X(r, b) = 2^(x - 127) for the scale byte x = scales[r*ld_scales + b]
 * (x = 255 is NaN).  scales_a holds M rows of ceil(K/32) bytes with row stride
 * ld_scales_a, scales_b N rows with ld_scales_b (device pointers, caller-owned).
 * Invalid (HK_ERROR_INVALID_VALUE): a NULL scale pointer or ld_scales below
 * ceil(K/32) when K > 0, besides the checks of the other entry points.
 * Not supported (HK_ERROR_NOT_SUPPORTED; no fallback kernel): K not a multiple
 * of 32; A, B, scales_a or scales_b not 16-byte aligned; lda, ldb,
 * ld_scales_a or ld_scales_b not a multiple of 16; 256 rows of any of them
 * spanning 2^31 bytes or more.
 */
hk_status hk_gemm_mxfp8(const void *A, const void *B, void *C,
                        int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc,
                        const void *scales_a, const void *scales_b,
                        int64_t ld_scales_a, int64_t ld_scales_b,
                        hk_stream_t stream);

/* BF16 or FP8 with explicit options (opts may be NULL = defaults).
 * scale_a and scale_b are ignored for BF16; for FP8 either may instead be
 * read from device memory (opts->scale_a_dev, scale_b_dev).
 * HK_DTYPE_MXFP8_E4M3 is HK_ERROR_INVALID_VALUE here (it needs
 * hk_gemm_mxfp8's scale arrays). */
hk_status hk_gemm_ex(int32_t dtype,
                     const void *A, const void *B, void *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     float scale_a, float scale_b,
                     const hk_gemm_opts *opts, hk_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as hk_gemm_ex, with the repack workspace (hk_repack) taken from a
 * device array the library owns, HK_NOALLOC_SCRATCH_BYTES per GPU, held
 * from the first such call on a GPU until the process ends.  The call
 * allocates nothing and never synchronises.  opts->workspace must be NULL and
 * workspace_bytes 0 (HK_ERROR_INVALID_VALUE otherwise).  A call that would
 * use more than HK_NOALLOC_SCRATCH_BYTES (hk_gemm_workspace_size; the BF16
 * 8191 x 28670 x 8200 product needs 642 MB) returns HK_ERROR_NOT_SUPPORTED
 * and enqueues nothing; repack = HK_REPACK_NEVER runs it on the operands as
 * given.  Every call on one GPU shares that GPU's array: calls ordered on
 * one stream are safe, calls that may overlap on one GPU (other streams,
 * other host threads) race.  HK_ERROR_LAUNCH if the runtime cannot give the
 * array's device address.
 */
#define HK_NOALLOC_SCRATCH_BYTES ((int64_t)256 << 20)
hk_status hk_gemm_ex_noalloc(int32_t dtype,
                             const void *A, const void *B, void *C,
                             int64_t M, int64_t N, int64_t K,
                             int64_t lda, int64_t ldb, int64_t ldc,
                             float scale_a, float scale_b,
                             const hk_gemm_opts *opts, hk_stream_t stream);

/* Describe the launch hk_gemm_ex would make, without touching the GPU
 * beyond reading (once) the current device's CU count.  Pointers only
 * matter for their alignment and may be any value.  Returns the same
 * validation errors as hk_gemm_ex. */
hk_status hk_gemm_plan(int32_t dtype, const void *A, const void *B, const void *C,
                       int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc,
                       const hk_gemm_opts *opts, hk_gemm_plan_info *out);

/* Workspace bytes a hk_gemm_ex call with these arguments would use for
 * repacked operands (0 if it would repack nothing), assuming a workspace at
 * least that large; opts->workspace and workspace_bytes are ignored here.
 * Same validation as hk_gemm_plan; pointers only matter for alignment. */
hk_status hk_gemm_workspace_size(int32_t dtype, const void *A, const void *B, const void *C,
                                 int64_t M, int64_t N, int64_t K,
                                 int64_t lda, int64_t ldb, int64_t ldc,
                                 const hk_gemm_opts *opts, int64_t *bytes);

/* Host evaluation of the workgroup-to-tile map used on the device (the
 * same code), for tests and locality models.  For each p < count, maps
 * workgroup id wg[p] of a tiles_m x tiles_n grid to (tm[p], tn[p]).
 * nxcd is the number of chiplets workgroups are dealt over (8 on MI355X).
 * Returns HK_ERROR_INVALID_VALUE for ids outside [0, tiles_m*tiles_n) or
 * non-positive parameters. */
hk_status hk_grid_map(int32_t grid_order, int64_t tiles_m, int64_t tiles_n,
                      int32_t group_m, int32_t window, int32_t nxcd,
                      int64_t count, const int64_t *wg, int64_t *tm, int64_t *tn);

/* Rate of the constant-rate counter the clock record uses (the current
 * device's wall-clock rate attribute), in kHz; 0 if the runtime cannot say. */
int32_t hk_wall_clock_khz(void);

/* Static string for a status code ("HK_SUCCESS", ...). */
const char *hk_status_string(hk_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t hk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HK_GEMM_H */
