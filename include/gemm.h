/*
 * gemm.h -- C ABI of an MI355X (gfx950) GEMM library:  D = alpha * A * B + beta * C
 *
 * The operation and the shape of the interface follow the pages this library
 * is built from:
 *   - "CUTLASS Python 接口全解析", section 2: a GEMM plan computes D = A*B + C;
 *     section 2.1: the plan binds element_A/B/C/D/accumulator and the layout at
 *     construction, and one plan runs problems of different shapes with the
 *     same types; section 2.2: compilation is separate from running;
 *     section 2.3: an elementwise activation (ReLU) fuses into the epilogue,
 *     and run() is asynchronous with an explicit synchronisation afterwards.
 *   - "CUTLASS Python接口", section 3.3: D = alpha * A * B + beta * C with an
 *     fp32 accumulator; section 4.3: automatic, persistent and grouped kernel
 *     schedules; section 7.1: descriptive errors instead of crashes.
 *   - "Python packages associated with CUTLASS", Overview: descriptive
 *     run-time errors and an enumeration of the configurations known to work;
 *     Current functionality: GEMM, fused elementwise epilogue (ReLU),
 *     stream-K work splitting, grouped GEMM.
 *   - "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL
 *     backend", section 5.1: FP8 matrix multiply as a scaled mm.
 *
 * Conventions shared by every call
 *   - Matrices are dense and packed. A is M x K, B is K x N, C and D are
 *     M x N. RowMajor means the last index is contiguous (X[r][c] at
 *     base[r * cols + c]); ColumnMajor means X[r][c] at base[r + c * rows].
 *     C and D share the plan's layout_C.
 *   - All data pointers are device pointers (hipMalloc'd memory or torch CUDA
 *     tensors on ROCm). The caller owns them and keeps them alive until the
 *     enqueued work has completed on `stream`.
 *   - `stream` is a hipStream_t passed as void*; NULL selects the null stream.
 *     Runs are asynchronous: they enqueue kernels and return. Synchronise the
 *     stream before reading D on the host.
 *   - Every call returns a gemm_status; on failure gemm_last_error() gives a
 *     descriptive, thread-local message. Arguments are validated before
 *     anything is enqueued, so a failed call has enqueued nothing. Faults in
 *     enqueued work surface at the caller's stream synchronisation.
 *   - Accumulation is always fp32 (element_accumulator must be GEMM_F32).
 *   - D may be the same pointer as C (in-place update). Any other overlap
 *     between D and A, B or C is undefined.
 *   - beta == 0: C is not read and may be NULL (NaN/Inf in C do not
 *     propagate). M == 0 or N == 0: nothing is enqueued, GEMM_OK.
 *     K == 0: D = epilogue(beta * C). Negative sizes: GEMM_INVALID_ARG.
 *   - Any pointer alignment and any size are accepted; operands whose base
 *     address or contiguous extent do not allow 16-byte vector loads run on a
 *     slower, scalar-load kernel with the same arithmetic contract.
 *   - A plan owns one device workspace (stream-K / split-K partial tiles and
 *     their arrival counters, the grouped descriptor table and tile queues)
 *     that every run
 *     call of the plan shares. A plan must therefore not run on two streams
 *     at once, for any run call: two overlapping runs of one plan race on
 *     the workspace (wrong D, counters left dirty). Create one plan per
 *     stream for concurrent work. Consecutive runs on one stream, or on
 *     different streams ordered by events, are fine.
 */
#ifndef MI355_GEMM_H
#define MI355_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_F32 = 0,
    GEMM_F16 = 1,
    GEMM_BF16 = 2,
    GEMM_F8_E4M3 = 3, /* OCP FP8 E4M3 (e4m3fn: bias 7, max 448, no Inf) */
    GEMM_F4_E2M1 = 4  /* OCP FP4 E2M1 (bias 1, max 6, no Inf/NaN), two per byte
                         along K, element 2t in the low nibble of byte t; only
                         as MX block-scaled elements (gemm_plan_run_mx) */
} gemm_dtype;

typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout;

/* Epilogue activation, applied to v = alpha*acc + beta*C (+ bias[n] with
 * gemm_plan_run_ex) and then rounded once, to nearest even, into element_D:
 * LINEAR keeps v; RELU gives max(v, +0) (NaN maps to +0); SIGMOID gives
 * 1/(1+exp(-v)); TANH gives tanh(v) ("CUTLASS Python 接口全解析" section 2.3;
 * "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL backend",
 * section 7: ReLU, Sigmoid and Tanh in the fused epilogue). SIGMOID and TANH
 * are evaluated in fp32 with the hardware exponential and reciprocal (a few
 * fp32 ulp; absolute error below 1e-7 near 0). */
typedef enum {
    GEMM_EPI_LINEAR = 0,
    GEMM_EPI_RELU = 1,
    GEMM_EPI_SIGMOID = 2,
    GEMM_EPI_TANH = 3
} gemm_epilogue;

typedef enum {
    GEMM_OK = 0,
    GEMM_INVALID_ARG = 1,     /* NULL/negative/inconsistent arguments */
    GEMM_UNSUPPORTED = 2,     /* type tuple or option not provided */
    GEMM_HIP_ERROR = 3,       /* a HIP runtime call failed */
    GEMM_OUT_OF_MEMORY = 4,   /* workspace allocation failed */
    GEMM_NOT_INITIALIZED = 5  /* NULL or destroyed plan */
} gemm_status;

/* Work schedule ("CUTLASS Python接口" section 4.3: auto / persistent /
 * grouped schedules; "Python packages associated with CUTLASS": stream-K). */
typedef enum {
    GEMM_SCHED_AUTO = 0,          /* heuristic: data-parallel, stream-K or hybrid */
    GEMM_SCHED_DATA_PARALLEL = 1, /* one work unit per output tile */
    GEMM_SCHED_STREAM_K = 2,      /* every tile's MAC iterations split evenly */
    GEMM_SCHED_HYBRID = 3,        /* whole waves data-parallel, the rest stream-K */
    GEMM_SCHED_SPLIT_K = 4        /* each tile cut into interleaved K units (skinny shapes) */
} gemm_schedule;

/* Output tile shape (rows of D x columns of D per workgroup). */
typedef enum {
    GEMM_TILE_AUTO = 0,
    GEMM_TILE_256x256 = 1,
    GEMM_TILE_128x128 = 2,
    GEMM_TILE_64x256 = 3,
    GEMM_TILE_32x256 = 4,
    GEMM_TILE_GENERIC = 5,  /* the scalar-load kernel, for any alignment */
    GEMM_TILE_WHOLEK = 6    /* 32x32 blocks, all of K loaded at once: small problems with
                               K <= 1024 (fp32, fp16, bf16); batch 1, no MX scales; a
                               problem it cannot take runs on the heuristic tile */
} gemm_tile;

typedef struct gemm_plan_s *gemm_plan_t;

/* Create a plan binding the element types, layouts and epilogue.
 * Supported (element_A, element_B, element_C, element_D, element_accumulator):
 *   (F32, F32, F32, F32, F32), (F16, F16, F16, F16, F32),
 *   (BF16, BF16, BF16, BF16, F32), (F8_E4M3, F8_E4M3, BF16, BF16, F32),
 *   (F4_E2M1, F4_E2M1, BF16, BF16, F32) -- the last for MXFP4 runs only
 *   (gemm_plan_run_mx; every other run call on it returns GEMM_UNSUPPORTED
 *   unless K == 0).
 * Others return GEMM_UNSUPPORTED naming the tuple. Makes no device call.
 * On success *out owns host memory until gemm_plan_destroy. */
gemm_status gemm_plan_create(gemm_plan_t *out, gemm_dtype element_a,
                             gemm_dtype element_b, gemm_dtype element_c,
                             gemm_dtype element_d, gemm_dtype element_acc,
                             gemm_layout layout_a, gemm_layout layout_b,
                             gemm_layout layout_c, gemm_epilogue epilogue);

/* Shorthand ("CUTLASS Python 接口全解析" section 2.1: one `element` and one
 * `layout` for every operand): element for A, B, C, D; F8_E4M3 is not
 * accepted here (its output type differs). Accumulator fp32. */
gemm_status gemm_plan_create_simple(gemm_plan_t *out, gemm_dtype element,
                                    gemm_layout layout, gemm_epilogue epilogue);

/* Release the plan and its device workspace. Waits for the last stream the
 * plan ran on before freeing device memory. NULL is a no-op. */
gemm_status gemm_plan_destroy(gemm_plan_t plan);

/* Override the heuristic choice of schedule and tile (for tuning and tests).
 * sk_grid > 0 caps the number of persistent workgroups (0 = automatic).
 * Host-only; no device call. */
gemm_status gemm_plan_set_config(gemm_plan_t plan, gemm_schedule schedule,
                                 gemm_tile tile, int32_t sk_grid);

/* Enqueue D = epilogue(alpha * A * B + beta * C) on `stream`.
 * For an F8 plan this is gemm_plan_run_scaled with unit scales. */
gemm_status gemm_plan_run(gemm_plan_t plan, const void *A, const void *B,
                          const void *C, void *D, int64_t M, int64_t N,
                          int64_t K, float alpha, float beta, void *stream);

/* gemm_plan_run for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, semantics and results contract as gemm_plan_run; it calls
 * no hipMalloc, hipFree or other allocating routine. The stream-K / split-K
 * partial tiles and arrival counters come from a static workspace compiled
 * into the library (32 MiB of partials and 16384 counters per device, held
 * by each device the library runs on until the process ends) instead of the
 * plan's: a stream-K grid or split-K factor is reduced until its partials
 * fit, and a hybrid schedule whose remainder would not spread over the grid
 * runs data-parallel, so results may differ from gemm_plan_run's in the
 * order of the fp32 sums only. A launch that still needs more partials or
 * counters than the workspace holds returns GEMM_UNSUPPORTED, naming both
 * sizes, and enqueues nothing.
 * The first call on each device initialises that device's workspace (it
 * clears the counters on `stream` and waits for them): it must not be
 * captured into a graph (GEMM_UNSUPPORTED if it is); later calls may be.
 * Every call on one device shares that device's workspace: two calls that
 * overlap in time on one device (two streams, or two host threads) race on
 * it and give wrong results. Order them, or use gemm_plan_run with one plan
 * per stream. */
gemm_status gemm_plan_run_noalloc(gemm_plan_t plan, const void *A, const void *B,
                                  const void *C, void *D, int64_t M, int64_t N,
                                  int64_t K, float alpha, float beta,
                                  void *stream);

/* FP8 with per-tensor scales ("Generating State-of-the-Art GEMMs ...",
 * section 5.1, scaled mm): D = epi(alpha * s_A * s_B * (A_q B_q) + beta * C).
 * scale_a / scale_b point to one fp32 each in device memory (NULL = 1.0);
 * they are read by the kernel, so they may be produced on the same stream.
 * Accepted by every plan; for non-F8 plans the scales multiply alpha too. */
gemm_status gemm_plan_run_scaled(gemm_plan_t plan, const void *A,
                                 const void *B, const void *C, void *D,
                                 int64_t M, int64_t N, int64_t K, float alpha,
                                 float beta, const float *scale_a,
                                 const float *scale_b, void *stream);

/* Fused bias ("CUTLASS Python接口", the BiasAdd-ReLU GEMM example:
 * Output = Activation(Input * Weight + Bias)):
 *   D = act(alpha * s_A * s_B * (A B) + beta * C + bias[n])
 * bias points to N elements of element_C (device memory, one value per
 * column of D, added to every row); NULL means no bias. scale_a / scale_b are
 * as in gemm_plan_run_scaled (NULL = 1.0). This is the general form of the
 * two calls above. */
gemm_status gemm_plan_run_ex(gemm_plan_t plan, const void *A, const void *B,
                             const void *C, void *D, const void *bias,
                             int64_t M, int64_t N, int64_t K, float alpha,
                             float beta, const float *scale_a,
                             const float *scale_b, void *stream);

/* MX block-scaled GEMM ("Generating State-of-the-Art GEMMs with
 * TorchInductor's CuteDSL backend", sections 5.1 and 5.2: MXFP8 among the
 * scaled GEMMs, with their own scale type, block size and layout; the format
 * itself is the OCP Microscaling v1.0 one). The plan must have the
 * (F8_E4M3, F8_E4M3, BF16, BF16, F32) tuple; A and B hold e4m3 elements in
 * the plan's layouts, and
 *   D = act(alpha * sum_k a(i,k) X_A(i,k/32) b(k,j) X_B(j,k/32) + beta*C + bias)
 * where mx_scale_a is M x (K/32) and mx_scale_b is N x (K/32) E8M0 bytes,
 * row-major whatever the operand layouts (scale row i belongs to row i of A,
 * scale row j to column j of B); an E8M0 byte e is 2^(e-127), 0xFF is NaN.
 * K must be a multiple of 32 (else GEMM_INVALID_ARG); the MFMA tile kernels
 * run when K % 128 == 0 and both scale arrays are 4-byte aligned, otherwise
 * the scalar kernel does. bias as in gemm_plan_run_ex. No per-tensor scales.
 * MXFP4 (the same section lists MXF4 beside MXFP8): on a (F4_E2M1, F4_E2M1,
 * BF16, BF16, F32) plan A and B hold OCP FP4 E2M1 elements packed two per
 * byte in their storage order (element 2t in the low nibble of byte t), the
 * scales and the formula unchanged; the MFMA tile kernels take A RowMajor
 * and B ColumnMajor (both packed along K) with K % 256 == 0, every other
 * case runs on the scalar kernel.
 * A NULL scale array with M, N, K > 0 gives GEMM_INVALID_ARG; a plan of
 * another type tuple gives GEMM_UNSUPPORTED. Buffers stay the caller's. */
gemm_status gemm_plan_run_mx(gemm_plan_t plan, const void *A, const void *B,
                             const void *C, void *D, const void *bias,
                             int64_t M, int64_t N, int64_t K, float alpha,
                             float beta, const uint8_t *mx_scale_a,
                             const uint8_t *mx_scale_b, void *stream);

/* Elementwise op between the epilogue value and an auxiliary tensor, and
 * the side of the activation it sits on (see gemm_plan_run_aux). */
typedef enum {
    GEMM_AUX_ADD = 0, /* y + X */
    GEMM_AUX_SUB = 1, /* y - X */
    GEMM_AUX_MUL = 2, /* y * X */
    GEMM_AUX_DIV = 3  /* y / X (IEEE fp32 division) */
} gemm_aux_op;

typedef enum {
    GEMM_AUX_BEFORE_ACT = 0, /* D = act(v op X)  */
    GEMM_AUX_AFTER_ACT = 1   /* D = act(v) op X  */
} gemm_aux_pos;

/* Auxiliary-tensor epilogue ("Generating State-of-the-Art GEMMs with
 * TorchInductor's CuteDSL backend", section 7: the epilogue-fusion kernels
 * load and store auxiliary tensors and apply elementwise add, multiply,
 * subtract and divide besides the ReLU / Sigmoid / Tanh activations).
 * With v = alpha * s_A * s_B * (A B) + beta * C + bias[n] (as in
 * gemm_plan_run_ex) and the plan's activation act:
 *   aux_pos = GEMM_AUX_BEFORE_ACT:  z = v op aux,  D = act(z)
 *   aux_pos = GEMM_AUX_AFTER_ACT:   z = v,         D = act(v) op aux
 * and aux_out, if not NULL, receives z (the activation's input), rounded
 * once to element_D. aux and aux_out are M x N in the plan's layout_C and
 * element_C / element_D types, device memory; aux NULL means no op (D =
 * act(v)), so aux_out alone stores the pre-activation value. All arithmetic
 * is fp32; division is IEEE (x / 0 gives Inf or NaN, not an error).
 * aux may be C, and aux_out may be aux (in place); aux_out equal to D gives
 * GEMM_INVALID_ARG, any other overlap with A, B, C or D is undefined. An
 * unknown aux_op or aux_pos gives GEMM_INVALID_ARG. Buffers stay the
 * caller's. */
gemm_status gemm_plan_run_aux(gemm_plan_t plan, const void *A, const void *B,
                              const void *C, void *D, const void *bias,
                              const void *aux, gemm_aux_op aux_op,
                              gemm_aux_pos aux_pos, void *aux_out, int64_t M,
                              int64_t N, int64_t K, float alpha, float beta,
                              const float *scale_a, const float *scale_b,
                              void *stream);

/* Batched GEMM ("CUTLASS Python接口", batched GEMM: batch_count and
 * batch_stride_A/B/C): batch_count problems of one shape M x N x K; problem b
 * reads A + b*stride_a, B + b*stride_b, C + b*stride_c and writes
 * D + b*stride_d (strides in elements of the operand's type, each operand in
 * the plan's layout). A stride of 0 shares that operand across the batch
 * (C too); stride_d must be at least M*N when batch_count > 1, so outputs do
 * not overlap. bias (N elements of the C/D type, or NULL), scale_a and
 * scale_b (device fp32 scalars, or NULL for 1.0) are shared by every problem,
 * with the meaning gemm_plan_run_ex gives them. All problems run in one
 * persistent launch over a batch-major tile space; batch entries whose
 * strides break the tile kernels' 16-byte alignment run one launch each.
 * batch_count == 0 is a no-op; a negative count or stride, or overlapping
 * outputs, give GEMM_INVALID_ARG; batch_count > 2^31 gives GEMM_UNSUPPORTED.
 * The caller keeps ownership of every buffer. */
gemm_status gemm_plan_run_batched(gemm_plan_t plan, const void *A, const void *B,
                                  const void *C, void *D, const void *bias,
                                  int64_t M, int64_t N, int64_t K,
                                  int64_t batch_count, int64_t stride_a,
                                  int64_t stride_b, int64_t stride_c,
                                  int64_t stride_d, float alpha, float beta,
                                  const float *scale_a, const float *scale_b,
                                  void *stream);

/* One problem of a grouped call; pointers follow the conventions above. */
typedef struct {
    int64_t M, N, K;
    const void *A;
    const void *B;
    const void *C; /* may be NULL when beta == 0 */
    void *D;
} gemm_problem;

/* Grouped GEMM ("Python packages associated with CUTLASS", Current
 * functionality): `count` independent problems with the plan's types,
 * layouts and epilogue, and shared alpha/beta, in one persistent launch.
 * `problems` is a host array, copied before the call returns (the caller may
 * free it at once). Problems with M, N or K == 0 follow the single-GEMM
 * rules. Workgroups take their first tile, then claim further tiles from
 * per-XCD queues (so problems of different K finish together), or, when all
 * problems need the same number of k-tiles (the same K up to the kernel's k
 * step), take every grid-th tile; results do not depend on which workgroup
 * ran a tile. The plan keeps a device copy of
 * the descriptor table and the queue words (zeroed by each launch for the
 * next): one plan must not run grouped calls on two streams at once. */
gemm_status grouped_gemm_run(gemm_plan_t plan, const gemm_problem *problems,
                             int32_t count, float alpha, float beta,
                             void *stream);

/* Describe, without any device call, the kernel and schedule a run of
 * M x N x K would use, as a short JSON object written into buf (NUL
 * terminated, truncated to len). num_cus = 0 assumes 256 compute units. */
gemm_status gemm_plan_describe(gemm_plan_t plan, int64_t M, int64_t N,
                               int64_t K, int32_t num_cus, char *buf,
                               int32_t len);

/* One timed configuration of gemm_plan_profile. */
typedef struct {
    gemm_schedule schedule; /* as launched (never AUTO) */
    gemm_tile tile;         /* as launched; GENERIC for the scalar-load kernel */
    int32_t sk_grid;        /* 0: automatic grid */
    int32_t grid;           /* workgroups launched */
    float us;               /* mean microseconds per run */
} gemm_config;

/* Kernel profiler ("CUTLASS Python接口", GemmProfiler: for a given size and
 * data type, run every kernel implementation of the library and report each
 * one's execution time). Runs every distinct (tile, schedule) launch this plan
 * can make for M x N x K on the caller's buffers and `stream`: one untimed
 * run, then `iters` back-to-back runs between two HIP events; blocks until
 * they finish. Writes up to max_results configurations, fastest first, to
 * `results` and their total count to *n_results (either may be NULL/0), and
 * records the fastest in the plan's configuration cache, which later runs of
 * exactly this M x N x K use whenever the plan has no gemm_plan_set_config
 * override (batched calls and MX runs keep the heuristics). Before a
 * launch is timed, its untimed run writes into a NaN-filled D whose copy is
 * compared with the first launch's result: the same elements non-finite,
 * the finite ones within 4 output ulp plus 1 % of the result's root mean
 * square (the launches differ only in the order of their fp32 sums). A
 * launch that disagrees makes the call fail with GEMM_HIP_ERROR naming it
 * and the first differing element, and nothing is cached. The check copies
 * D to host memory (2 * M * N output elements of host buffers). D is
 * overwritten (it holds the last run's result); D == C with beta != 0
 * gives GEMM_INVALID_ARG. iters outside [1, 100000] gives GEMM_INVALID_ARG.
 * Operands follow gemm_plan_run's rules. */
gemm_status gemm_plan_profile(gemm_plan_t plan, const void *A, const void *B,
                              const void *C, void *D, int64_t M, int64_t N,
                              int64_t K, float alpha, float beta, int32_t iters,
                              gemm_config *results, int32_t max_results,
                              int32_t *n_results, void *stream);

/* Exportable configuration cache ("Generating State-of-the-Art GEMMs with
 * TorchInductor's CuteDSL backend", roadmap: a portable, human-readable
 * format such as JSON for autotuned GEMM configurations, with import and
 * export calls, so tuning carries across runs and environments).
 * Export writes the plan's cache as JSON text: the format name and version,
 * the plan's element types and layouts, and one entry per tuned shape
 * {m, n, k, mx, schedule, tile, sk_grid, us}. *needed receives the size
 * including the terminating NUL; buf == NULL only queries it; a buffer
 * shorter than that gives GEMM_INVALID_ARG and writes nothing.
 * Import merges such a text into the plan's cache (an imported entry
 * replaces one of the same shape). Malformed text gives GEMM_INVALID_ARG, a
 * cache written for other element types or layouts GEMM_UNSUPPORTED; on any
 * error the cache is left unchanged. Host-only; no device call. */
gemm_status gemm_plan_cache_export(gemm_plan_t plan, char *buf, int32_t len,
                                   int32_t *needed);
gemm_status gemm_plan_cache_import(gemm_plan_t plan, const char *json);

/* Number of cached shapes (-1 for an invalid handle), and clearing. */
int32_t gemm_plan_cache_size(gemm_plan_t plan);
gemm_status gemm_plan_cache_clear(gemm_plan_t plan);

/* gemm_plan_describe for a gemm_plan_run_batched call of batch_count
 * problems of this shape (batch_count = 1 is gemm_plan_describe); "tiles"
 * then counts the tiles of the whole batch. batch_count outside [1, 2^31)
 * gives GEMM_INVALID_ARG. */
gemm_status gemm_plan_describe_batched(gemm_plan_t plan, int64_t M, int64_t N,
                                       int64_t K, int64_t batch_count,
                                       int32_t num_cus, char *buf, int32_t len);

/* Thread-local description of the last failure in this thread ("" if none). */
const char *gemm_last_error(void);

/* Static name of a status code. */
const char *gemm_status_string(gemm_status status);

/* Enumerate the supported type tuples ("Python packages associated with
 * CUTLASS", Overview: configurations known to work). */
int32_t gemm_supported_count(void);
gemm_status gemm_supported_get(int32_t index, gemm_dtype *element_a,
                               gemm_dtype *element_b, gemm_dtype *element_c,
                               gemm_dtype *element_d, gemm_dtype *element_acc);

/* Library version string. */
const char *gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355_GEMM_H */
