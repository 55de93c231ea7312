/*
 * skinny.h -- C ABI of the MI355X (gfx950) skinny BF16 decode projection.
 *
 *   out[M, N] = x[M, K] @ W[N, K]^T (+ residual[M, N]),   M = 1..64 tokens,
 *   BF16 (or FP16) in, fp32 accumulation, BF16 or fp32 out.
 *
 * The operation is the one the pages define for their decode GEMMs:
 * "out[M, N] = x[M, K] @ weight[N, K]^T" (class PreparedWarpSplitK, page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.warp_splitk")
 * and "x @ weight.T" (class Projection, page
 * "vllm.models.glm5next.nvidia.specialized_decode.gemm").  No bias is added;
 * out is overwritten.  skinny_run_ex can add a residual (the `residual` of
 * try_low_latency_gemm, page "vllm.models.kimi_k3.nvidia.low_latency_gemm")
 * and takes row pitches, and skinny_prepare_ex FP16 weights and pitched
 * weights (class PreparedProjection and matrix_view, page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.projection").
 *
 * Usage follows the pages' prepare-once / run-per-forward split: a prepared
 * object owns the weight and a per-token-count kernel choice that is fixed
 * before graph capture, and each forward resolves its kernel with a single
 * lookup ("vllm.models.kimi_k3.nvidia.low_latency_gemm", module docstring:
 * the {M: call} plan resolved at install time).
 *
 * Conventions for every entry point:
 *  - All data pointers (W, x, out) are DEVICE pointers on the device that is
 *    current when the plan is prepared.  The library never dereferences them
 *    on the host.
 *  - Matrices are row-major: W is [N][K], x is [M][K], out is [M][N].  The
 *    plain entry points take them packed (row pitch = column count); the _ex
 *    entry points take a row pitch (in elements) for each.
 *  - Every call returns a status; none aborts or throws.  After a failure,
 *    skinny_last_error() returns a thread-local text describing it.
 *  - A stream is passed as a hipStream_t cast to void*; NULL is the null
 *    stream of the current device.  A plan runs on streams of the device it
 *    was prepared on; the run calls check nothing about devices, so a
 *    stream of another device is the caller's error (the kernel would run
 *    there on addresses of the plan's device).
 */
#ifndef SKINNY_H
#define SKINNY_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct skinny_plan skinny_plan; /* opaque; one per prepared weight */

typedef enum {
    SKINNY_OUT_BF16 = 0, /* out is BF16, rounded to nearest even once */
    SKINNY_OUT_F32 = 1   /* out is fp32 (the accumulator, unrounded) */
} skinny_out_dtype;

typedef enum {
    SKINNY_IN_BF16 = 0, /* W and x are BF16 (v_dot2_f32_bf16, bf16 MFMA) */
    SKINNY_IN_F16 = 1   /* W and x are FP16 (v_dot2_f32_f16, f16 MFMA) */
} skinny_in_dtype;

typedef enum {
    SKINNY_OK = 0,
    SKINNY_ERR_INVALID_ARG = 1,   /* null pointer, N <= 0, K <= 0, bad enum/tactic */
    SKINNY_ERR_SHAPE = 2,         /* K % 8 != 0, or N * K too large */
    SKINNY_ERR_ALIGN = 3,         /* W or x not 16-byte aligned, out not element aligned */
    SKINNY_ERR_UNSUPPORTED_M = 4, /* M outside 1..64: caller falls back */
    SKINNY_ERR_DEVICE = 5,        /* no device, or the current device is not gfx950 */
    SKINNY_ERR_NOMEM = 6,         /* device or host allocation failed */
    SKINNY_ERR_HIP = 7            /* a HIP call failed (e.g. prepare during capture) */
} skinny_status;

/* Largest token count a plan serves. */
#define SKINNY_MAX_M 64

/* Kernel families. */
typedef enum {
    SKINNY_PATH_DOT2 = 0,  /* v_dot2_f32_bf16, token tiles 1/2/4/8; waves split K */
    SKINNY_PATH_MFMA = 1,  /* v_mfma_f32_16x16x32_bf16, tiles 16/32/64; waves split K */
    SKINNY_PATH_DOT2X = 2, /* retired (never the fastest on any measured shape); reserved */
    SKINNY_PATH_MFMAX = 3, /* v_mfma_f32_16x16x32_bf16, tiles 16/32/64; 16 rows per wave,
                              W re-laid out and x staged through LDS via registers;
                              unroll = 2: equal row ranges (a whole multiple of CUs / split
                              of them) instead of aligned 16 * waves row tiles */
    SKINNY_PATH_MFMAD = 4, /* retired (direct-to-LDS rings; slower than MFMAX/MFMAW); reserved */
    SKINNY_PATH_MFMAS = 5, /* retired (stream-K grid; slower than equal row ranges); reserved */
    SKINNY_PATH_MFMAR = 6, /* retired (the stream-K kernel on a data-parallel grid); reserved */
    SKINNY_PATH_MFMAK = 7, /* retired (in-workgroup K groups; overtaken by MFMAX/MFMAW); reserved */
    SKINNY_PATH_DOT2R = 8, /* the DOT2 kernels over equal row ranges of at most `rows` rows,
                              a whole multiple of CUs / split of them, so that every CU gets
                              the same number of (range, K split) workgroups */
    SKINNY_PATH_MFMAW = 9, /* tiles 16/32/64: equal row ranges of at most `rows` rows (a whole
                              multiple of CUs / split of them); every wave multiplies all
                              rows / 16 row groups of the range over every waves-th K stage,
                              W and x re-laid out through the wave's own LDS tiles, with no
                              barrier until the waves' partial sums are added in LDS */
    SKINNY_PATH_MFMA4 = 10,/* v_mfma_f32_4x4x4_16b_bf16, tiles 4/8/16/32: equal row ranges of at
                              most `rows` rows (a whole multiple of CUs / split of them); each of
                              the 16 blocks of the MFMA takes one 16-byte K chunk, so a plain
                              row-contiguous load of 4 rows (tokens) x 256 bytes becomes an
                              operand after one lane permutation -- no LDS in the K loop; waves
                              take every waves-th stage of 16 chunks; K parts meet in an
                              atomic-swap exchange */
    SKINNY_PATH_DOT2W = 11,/* v_dot2_f32_bf16, tiles 1/2/4/8: the MFMA4 kernel's stream (equal
                              row ranges of 4-row groups, waves on every waves-th 16-chunk
                              stage, row-contiguous loads straight into registers, each x load
                              serving every row group) with dot2 arithmetic per lane */
    SKINNY_PATH_MFMAT = 12 /* the 16-token MFMA kernel over token groups: mt = 32 or 64 is the
                              most tokens served; a run launches ceil(M / 16) groups of 16
                              tokens, each multiplying every row tile, so a weight too short
                              to fill the chip with row tiles gets groups x tiles workgroups
                              (it re-reads each tile from L2 once per group; enumerated only
                              for weights of at most 16 MiB) */
} skinny_path;

/*
 * One tactic: a kernel instance plus its launch shape.  The fields play the
 * roles of the pages' tactic fields -- the token tile (the padded token
 * count a tactic serves; "smallest tile >= m" in Projection.__init__), the
 * output rows per block ("outputs" of SkinnyGemmConfig; the 16- or 32-row
 * output tiles of the warp split-K page), loads in flight ("unroll"), and the
 * cross-block K split ("split K" of the split-K projection page's
 * (M tile, N tile, split K, stages) policies).
 */
typedef struct {
    int path;   /* skinny_path */
    int mt;     /* token tile: DOT2/DOT2R/DOT2X/DOT2W 1,2,4,8; MFMA4 4,8,16,32; MFMAT
                   32,64 (tokens served, in groups of 16); the other MFMA paths 16,32,64 */
    int rows;   /* weight rows per workgroup.  DOT2, DOT2R: 1..16 (mt*rows <= 64; for
                   DOT2R the most rows of a range); MFMA, MFMAT: 16,32,64; MFMAX: 16 * waves;
                   MFMAW: 16, 32 or
                   64 (the most rows of a range); MFMA4, DOT2W: 4 x (1, 2, 4, 7, 13 or
                   14), the most rows of a range (fewer row groups for the largest
                   token tiles) */
    int waves;  /* wavefronts per workgroup: 1,2,4,8 */
    int unroll; /* 16-byte weight loads per lane per row per pipeline stage: 1,2,4
                   (MFMAX: 1 = row tiles of 16 * waves rows, 2 = equal row ranges, its
                   stage is fixed at 32 chunks; MFMAW: 1 or 2 = stages of 8 or 16
                   chunks, two in flight, 3 or 4 = the same, one in flight; MFMA4,
                   DOT2W: stages of 16 chunks in flight, 2 or 3) */
    int split;  /* workgroups splitting K per row tile (1 = none), 1..16 (MFMAW 1..4,
                   MFMA4 and DOT2W 1..8); their fp32 partials meet in the plan's
                   workspace by agent-scope atomic swaps, one per value and tree
                   level (MFMAX, and MFMAW where each thread holds an even count
                   of values: one 64-bit swap per pair) */
} skinny_tactic;

/*
 * skinny_prepare -- build a plan for weight W [N][K] (BF16 bits, device).
 *
 * The install-time step of the pages: the module docstring of
 * "vllm.models.kimi_k3.nvidia.low_latency_gemm" resolves the static part of
 * the per-shape, per-token-count decision once into an {M: call} plan (and
 * its autotune_kda_qkvg tunes before graph capture); PreparedWarpSplitK's
 * constructor compiles one code per M and PreparedProjection.prepare one
 * kernel per batch (pages "...cutedsl.gemm.warp_splitk" and
 * "...cutedsl.gemm.projection") before any run.  Here the per-M choice is
 * measured on the chip, and the kernels are compiled into the library and
 * warmed.
 *
 * Validates the arguments, then looks up the process-wide tactic table for
 * (device, N, K, out_dtype); on a miss it times every legal tactic on the
 * device with cache-cold weight copies at its full token tile (each timing
 * replays a captured graph of back-to-back launches, as decode steps run
 * them, for at least 0.2 ms, so that a kernel of a few microseconds is not
 * timed at the host's launch rate), and each tactic of a 16-token or larger
 * tile once more at M = 8, where such tiles serve most of their token
 * counts; then times the few fastest whose tile is >= M (SKINNY_TUNE_REFINE
 * of them, default 4; 0 or 1 skips this pass), the two fastest of every tile
 * >= M and, for M < 16, the few fastest at M = 8, again at M itself and
 * keeps, for each M in 1..64, the fastest; then every tactic the
 * table uses is timed again at each M its tile serves, and the fastest kept;
 * finally, at M <= 8, the quickest v_dot2 tactic replaces the choice when it
 * is within SKINNY_TUNE_DOT2_MARGIN (relative, default 0.02, the run-to-run
 * spread of one tactic's timing; negative: off).
 *
 * A second table serves runs that add a residual, as select_kimi_k3_backend
 * keys its choice on has_residual (page "vllm.models.kimi_k3.nvidia.
 * low_latency_gemm"): the residual is read when a value is stored, after any
 * split-K exchange, which changes the ranking at some M.  For each M every
 * distinct tactic of the first table whose tile serves M is timed with a
 * residual, and the fastest replaces the first table's entry if it is faster
 * by more than SKINNY_TUNE_RESIDUAL_MARGIN (relative, default 0.01), or by
 * more than the dot2 margin where that entry is a v_dot2 tactic at M <= 8
 * (SKINNY_TUNE_RESIDUAL=0: the first table serves both).  Every tactic either table uses is launched once (warm-up) so
 * that nothing loads lazily under graph capture.  The split-K exchange
 * workspace is allocated here (zeroed: zero is an empty exchange node).
 *
 * Tuned tables can persist across processes: when the environment variable
 * SKINNY_TABLE_CACHE names a file, the tables for this chip (arch and CU
 * count) and shape are loaded from it instead of tuning (one line each, the
 * residual table's output type marked +res), and freshly tuned tables are
 * appended to it.  SKINNY_LOG=1 prints the chosen table, SKINNY_LOG=2 also
 * every candidate's time; SKINNY_TUNE_ITERS sets the timed launches per
 * candidate; SKINNY_XCD_REMAP=0 stops placing the split-K workgroups of a row
 * tile on one XCD (a plan-time setting, for testing the exchange across XCDs).
 * SKINNY_FORCE_TACTIC=path.mt.rows.waves.unroll.split (a table line's field
 * syntax) skips tuning and the table file: the plan runs that tactic for
 * every M <= mt and the 64-token MFMA tactic 1.64.16.1.1.1 above it, as
 * skinny_prepare_tactics_ex would; a malformed or illegal value is
 * SKINNY_ERR_INVALID_ARG before any device call.
 *
 * Synchronous.  Must not be called while the device is capturing a graph.
 * W is NOT copied: the plan keeps the pointer, W must stay allocated until
 * skinny_destroy, and its values may change between runs.  W is read-only.
 * Requires: N >= 1, K >= 8, K % 8 == 0, W 16-byte aligned, N * K < 2^31.
 * Thread-safe.
 */
skinny_status skinny_prepare(const void *W, int N, int K, skinny_out_dtype out_dtype,
                             skinny_plan **plan);

/*
 * skinny_prepare_tactics -- like skinny_prepare, but with the table given:
 * table[M - 1] is the tactic used for M tokens (M = 1..64), with or without a
 * residual, and must have a token tile >= M.  No timing is done; tactics are
 * validated and warmed.  Used to force a tactic (tests) or to load a table
 * tuned earlier.
 */
skinny_status skinny_prepare_tactics(const void *W, int N, int K, skinny_out_dtype out_dtype,
                                     const skinny_tactic *table, skinny_plan **plan);

/*
 * skinny_prepare_ex -- skinny_prepare for a weight with a row pitch and an
 * input type: W[n][k] is element n * ldw + k, ldw >= K, ldw % 8 == 0 (the
 * 16-byte row pitch PreparedProjection requires), and W (and every x run
 * with the plan) holds BF16 or FP16 values as in_dtype says.  Tables are
 * tuned and cached per (device, N, K, in_dtype, out_dtype) on packed
 * copies of W, and a pitched plan runs its packed shape's table.  Packed rows
 * stream fastest: on 6288x7168 and 7168x18432, rows padded by 128 B to
 * 4 KiB measured up to 9 % slower per call, and a 16-byte pad (rows that
 * start inside a 128-byte line) up to 51 % slower.  Errors as
 * skinny_prepare, plus
 * SKINNY_ERR_INVALID_ARG for a bad in_dtype and SKINNY_ERR_SHAPE for a bad
 * ldw.  skinny_prepare(W, N, K, od, plan) is
 * skinny_prepare_ex(W, N, K, K, SKINNY_IN_BF16, od, plan).
 */
skinny_status skinny_prepare_ex(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                skinny_out_dtype out_dtype, skinny_plan **plan);

/* skinny_prepare_tactics for a weight with a row pitch and an input type. */
skinny_status skinny_prepare_tactics_ex(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                        skinny_out_dtype out_dtype, const skinny_tactic *table,
                                        skinny_plan **plan);

/*
 * skinny_run_ex -- out[m][n] = sum_k x[m][k] W[n][k] (+ residual[m][n]) for
 * m < M, n < N, on `stream`, asynchronously; the fused-residual epilogue of
 * try_low_latency_gemm(x, weight, residual) when residual is not NULL.
 *
 * x[m][k] is element m * ldx + k (ldx >= K, ldx % 8 == 0, x 16-byte aligned,
 * the plan's input type).  out[m][n] is element m * ldo + n (ldo >= N).
 * residual (NULL for none) has the out type and element m * ldr + n
 * (ldr >= N); it is added in fp32 to the fp32 sum before the one rounding to
 * BF16.  residual may be out itself (with ldr == ldo: out += x W^T) but must
 * not otherwise overlap out.  Elements of out outside rows < M and columns
 * < N are not touched.  A run with a residual launches the plan's residual
 * table entry for M (skinny_plan_tactic_ex), one without it the other table's.
 * Everything else as skinny_run, which is
 * skinny_run_ex(plan, x, K, NULL, 0, out, N, M, stream).
 */
skinny_status skinny_run_ex(const skinny_plan *plan, const void *x, int ldx, const void *residual, int ldr,
                            void *out, int ldo, int M, void *stream);

/*
 * skinny_run -- out[0:M, :] = x[0:M, :] @ W^T on `stream`, asynchronously.
 *
 * One table lookup and one kernel launch; no allocation, synchronisation,
 * copy or host read of device memory, so it may be captured in a hipGraph.
 * x: [M][K] BF16 bits, 16-byte aligned.  out: [M][N], BF16 (2-byte aligned)
 * or fp32 (4-byte aligned) as prepared.  Rows of out at and beyond M, and all
 * other memory, are not touched; out is written, never read.
 * A plan holds one split-K workspace: the same plan must not run on two
 * streams concurrently.  Different plans may.
 * Errors: SKINNY_ERR_UNSUPPORTED_M for M outside 1..64 (the caller falls back,
 * as the pages' selectors return None), SKINNY_ERR_INVALID_ARG, SKINNY_ERR_ALIGN,
 * SKINNY_ERR_HIP if the launch is rejected.
 */
skinny_status skinny_run(const skinny_plan *plan, const void *x, void *out, int M, void *stream);

/*
 * skinny_run_static -- one product out = x W^T (+ residual) with a given
 * tactic and no plan, allocating nothing: for callers that cannot allocate
 * device (or host) memory where they run it -- code under graph capture,
 * tight serving loops, harnesses that forbid allocation.  The arguments are
 * those of skinny_prepare_tactics_ex (W, N, K, ldw, in_dtype, out_dtype, one
 * tactic whose token tile is >= M) and of skinny_run_ex (x ... stream), with
 * the same checks and status codes; the result is bit-identical to a plan
 * prepared with that tactic.
 *
 * A K-split tactic exchanges its partials through a device array the library
 * holds per GPU for the life of the process (SKINNY_STATIC_SCRATCH_BYTES);
 * a tactic that would need more returns SKINNY_ERR_SHAPE.  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (two
 * streams, say) race and must not be issued; calls in stream order are fine.
 * The first call on a device looks the array up (hipGetSymbolAddress) and
 * the first launch of a kernel loads its code, so make one call before graph
 * capture.  No warm-up, no tuning: the tactic is the caller's choice (for
 * example skinny_plan_tactic of a plan prepared earlier).
 */
#define SKINNY_STATIC_SCRATCH_BYTES (4 << 20)
skinny_status skinny_run_static(const void *W, int N, int K, int ldw, skinny_in_dtype in_dtype,
                                skinny_out_dtype out_dtype, const skinny_tactic *tactic, const void *x, int ldx,
                                const void *residual, int ldr, void *out, int ldo, int M, void *stream);

/* 1 if the plan serves M tokens (1 <= M <= 64), else 0 (Projection.supports). */
int skinny_supports(const skinny_plan *plan, int M);

/* The tactic the plan uses for M tokens. */
skinny_status skinny_plan_tactic(const skinny_plan *plan, int M, skinny_tactic *out);

/*
 * skinny_plan_tactic_ex -- the tactic the plan runs for M tokens with a
 * residual (has_residual != 0) or without one (skinny_plan_tactic); the
 * has_residual key of select_kimi_k3_backend on the low_latency_gemm page.
 * Errors as skinny_plan_tactic.
 */
skinny_status skinny_plan_tactic_ex(const skinny_plan *plan, int M, int has_residual, skinny_tactic *out);

/*
 * skinny_describe -- human-readable name of the plan's kernel for M tokens
 * and its launch shape, NUL-terminated in buf (truncated to len - 1 chars):
 * the entry of the {M: call} plan the low_latency_gemm module docstring
 * describes, a ProjectionSpec's "winning backend per token count".
 * SKINNY_ERR_INVALID_ARG for a NULL plan or buf or len = 0,
 * SKINNY_ERR_UNSUPPORTED_M for M outside 1..64.
 */
skinny_status skinny_describe(const skinny_plan *plan, int M, char *buf, size_t len);

/*
 * skinny_destroy -- free the plan and its split-K workspace.  The plan owns
 * its per-weight state as PreparedProjection owns its kernels and TMA maps
 * (page "...cutedsl.gemm.projection"); the weight stays the caller's.
 * Synchronises the plan's device first.  NULL is a no-op.
 */
void skinny_destroy(skinny_plan *plan);

/*
 * skinny_status_string -- static text for a status code ("unknown status"
 * for any other value).  The statuses stand for the pages' ValueErrors
 * (PreparedWarpSplitK's packed-BF16 and 32 B alignment checks,
 * PreparedProjection's dtype, pitch and prepared-batch checks) and for
 * select_kimi_k3_backend returning None "to fall back"
 * (SKINNY_ERR_UNSUPPORTED_M).
 */
const char *skinny_status_string(skinny_status s);

/*
 * skinny_last_error -- the text of the last failure on this thread ("" if
 * none), naming the offending argument and value the way the pages'
 * ValueError messages do.  Owned by the library; valid until the next
 * failing call on the same thread.
 */
const char *skinny_last_error(void);

/*
 * skinny_tactic_check -- SKINNY_OK if the tactic is a legal kernel instance and
 * launch shape for an [N][K] weight, else SKINNY_ERR_INVALID_ARG with the
 * reason in skinny_last_error().  Host only; no device call.
 */
skinny_status skinny_tactic_check(const skinny_tactic *t, int N, int K);

/*
 * skinny_enumerate_tactics -- the candidate tactics the tuner times for an
 * [N][K] weight.  Writes up to `cap` tactics to buf (buf may be NULL when cap
 * is 0) and returns the total count, or -1 on bad arguments.  Host only.
 */
int skinny_enumerate_tactics(int N, int K, skinny_tactic *buf, int cap);

/*
 * skinny_enumerate_tactics_ex -- the same for a device with `cus` compute
 * units (>= 1): the launch-shape rules (how many workgroups fill the chip,
 * how many equal row ranges a K split needs) depend on it.
 * skinny_enumerate_tactics is this with cus = 256 (an MI355X); the tuner
 * inside skinny_prepare uses the current device's count.  Host only.
 */
int skinny_enumerate_tactics_ex(int N, int K, int cus, skinny_tactic *buf, int cap);

/*
 * skinny_select_table -- the table rule.  Given `count` candidate tactics and
 * their measured times in microseconds (times[i] for cand[i]; a negative time
 * marks a candidate that could not run), fill table[M - 1] for M = 1..64 with
 * the fastest candidate whose token tile is >= M.  Ties go to the smaller
 * token tile, then the lower index.  Returns SKINNY_OK, or
 * SKINNY_ERR_INVALID_ARG if some M has no usable candidate.  Host only.
 */
skinny_status skinny_select_table(const skinny_tactic *cand, const double *times_us,
                                  int count, skinny_tactic *table);

/*
 * Measurement helpers (not part of the projection).  They put the projection's
 * timings in context: the decode-step cost the pages care about is streaming
 * the weight at HBM speed, so a bench compares against what a plain stream of
 * the same bytes achieves, and against the floor of an empty launch.
 *
 * skinny_probe_read -- read `bytes` bytes at `buf` (device, 16-byte aligned,
 * bytes % 16 == 0) with 16-byte nontemporal loads, one 64-lane workgroup per
 * 4 KiB with all four of its loads in flight, and write fp32 partial sums to
 * `sink` (device, skinny_probe_read_blocks() floats), so the loads cannot be
 * elided.  Asynchronous on `stream`.
 */
skinny_status skinny_probe_read(const void *buf, size_t bytes, float *sink, void *stream);

/* Floats skinny_probe_read may write to its sink. */
int skinny_probe_read_blocks(void);

/* skinny_probe_empty -- launch one empty 64-lane workgroup on `stream`. */
skinny_status skinny_probe_empty(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_H */
