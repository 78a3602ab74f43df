/*
 * tgemm.h -- output-stationary tiled matrix multiply C = A @ B on MI355X (gfx950).
 *
 * The operation ("Reading a matrix multiply through its tiles", opening paragraph
 * and section "Keep one output tile resident"; Mojo GPU puzzles, "Tiled Matrix
 * Multiplication", section 3, which fixes it as A x B and not A x B^T):
 *
 *     C[i][j] = sum_{k < K} A[i][k] * B[k][j]      0 <= i < M, 0 <= j < N
 *
 * A is M x K, B is K x N, C is M x N, all row-major (the puzzle page's "row-major
 * layout for all tensors") with leading dimensions lda, ldb, ldc counted in
 * ELEMENTS. C is overwritten: no alpha/beta, no accumulate into C (each page
 * stores the finished accumulator tile exactly once). Each C tile's fp32 (int32
 * for the integer path) accumulator stays in registers for the whole reduction;
 * A and B K-tiles are staged through LDS; partial edge tiles are handled over
 * their actual row, column and reduction ranges ("Edge tiles still matter").
 *
 * Number formats (dtype): the inputs A and B share one format; the accumulator is
 * fp32 for 16-bit float inputs (Helion matmul page: the C tile is an fp32 zero
 * tile; "What fits in local storage?": FP16 inputs with FP32 accumulation) and
 * the result is rounded once, to nearest-even, into C's format. The integer path
 * sums in 32-bit two's complement and wraps modulo 2^32.
 *
 * Conventions shared by every entry point:
 *  - All pointers A, B, C are DEVICE pointers (memory of the current HIP device),
 *    owned by the caller; the library never frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream), owned by
 *    the caller. gemm_run only enqueues work and returns; it never synchronizes.
 *    Faults inside a launched kernel surface at the caller's next synchronization.
 *  - Argument errors are detected on the host BEFORE any HIP call and leave C
 *    untouched. No C++ exception crosses this interface.
 *  - C must not overlap A or B (not checked).
 *  - Any alignment of A, B, C and any leading dimension >= the row length is
 *    accepted. The 16-byte loads straight into LDS need A and B at even byte
 *    addresses (the 16x16x32 tile also needs 16-byte aligned A and B, leading
 *    dimensions and contiguous extents in multiples of 8 elements); otherwise a
 *    slower element-wise loader is used. gemm_plan reports which one applies.
 *  - Operands may also be supplied transposed (gemm_run_op).
 *  - A handle may be used by one host thread at a time.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tgemm_handle* gemm_handle_t;

/* The enumerations below are 32-bit integers in the ABI. Compiled as C++ (the library
 * itself) they have int32_t as their fixed underlying type, so that every int32 a C
 * caller may pass (an unknown dtype, say) is a value of the type, which the argument
 * checks then reject, and never a value outside the enumeration's range. */
#ifdef __cplusplus
#define TGEMM_ENUM_BASE : int32_t
#else
#define TGEMM_ENUM_BASE
#endif

/* Status codes (int32). */
typedef enum TGEMM_ENUM_BASE {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_ARG = 1,       /* null/negative/too-small argument, destroyed or null handle */
  GEMM_ERR_UNSUPPORTED_DTYPE = 2, /* dtype is not one of gemm_dtype_t */
  GEMM_ERR_NO_DEVICE = 3,         /* no HIP device visible */
  GEMM_ERR_ARCH = 4,              /* current device is not gfx950 */
  GEMM_ERR_HIP = 5,               /* a HIP runtime call or kernel launch failed */
  GEMM_ERR_OUT_OF_MEMORY = 6,     /* a host allocation, or a device workspace allocation, failed */
  GEMM_ERR_UNSUPPORTED_TILE = 7,  /* gemm_set_tile asked for a tile no kernel has, for this dtype */
  GEMM_ERR_SCRATCH_TOO_SMALL = 8  /* gemm_run_op_noalloc: the split-K partial tiles exceed its scratch */
} gemm_status_t;

/* Input/accumulator/output formats (int32). */
typedef enum TGEMM_ENUM_BASE {
  GEMM_I32_I32 = 0,   /* int32 in, int32 accumulate (wraps mod 2^32), int32 out */
  GEMM_F16_F32 = 1,   /* IEEE binary16 in, fp32 accumulate, fp32 out */
  GEMM_BF16_F32 = 2,  /* bfloat16 in, fp32 accumulate, fp32 out */
  GEMM_BF16_BF16 = 3, /* bfloat16 in, fp32 accumulate, bfloat16 out (round to nearest even) */
  GEMM_F16_F16 = 4    /* binary16 in, fp32 accumulate, binary16 out (round to nearest even) */
} gemm_dtype_t;

/* Operand forms (int32) for the *_op entry points: op(X) = X or X^T. */
typedef enum TGEMM_ENUM_BASE {
  GEMM_OP_N = 0, /* as given: A stored M x K (lda >= K), B stored K x N (ldb >= N) */
  GEMM_OP_T = 1  /* transposed: A stored K x M (lda >= M), B stored N x K (ldb >= K) */
} gemm_op_t;

/* The kernel configuration gemm_run would use for a call (see gemm_plan). */
typedef struct {
  int32_t tile_m, tile_n, tile_k; /* C tile rows/cols and K-step of one workgroup */
  int32_t threads;                /* threads per workgroup */
  int32_t vector_loads;           /* 1: 16-byte loads straight into LDS; 0: element-wise loader */
  int32_t kernel;                 /* 0 none (empty C), 1 zero fill (K = 0), 2 int32 VALU,
                                     3 one-wave 16x16x32 MFMA, 4 macro-tile MFMA */
  int64_t grid;                   /* C tiles (workgroups per K-slice) */
  int32_t lds_bytes;              /* LDS per workgroup */
  int32_t split_k;                /* K-slices: 1, or S > 1 when each tile's reduction is cut into S
                                     slices whose fp32 partial tiles a second kernel sums in slice order */
  int32_t stages;                 /* the macro-tile kernel's LDS pipeline: 2 (A loaded two K-steps ahead
                                     into two A stages, B three ahead into three B stages); 3 (A loaded
                                     three K-steps ahead into three A stages, B two ahead into two B
                                     stages) for the 256x256 tile when C has at most four tile columns
                                     and at least four times as many tile rows; or 4 (both loaded three
                                     K-steps ahead into four stages of each) when the launch has at most
                                     one workgroup per compute unit and its tiles are 64x64 or cut into
                                     K-slices; 2 for the 16x16x32 tile (two stages of each), 1 for the
                                     int32 kernel, 0 when nothing is launched */
  int32_t tail_split_k;           /* 0, or S > 1: the tiles of C rows [tail_m0, M) run after the others
                                     as a second launch of the same tile with S K-slices (fp32 partial
                                     tiles summed in slice order), so that they fill the compute units
                                     left idle by a last, partial round of tiles */
  int32_t tail_m0;                /* first C row of that tail (a multiple of tile_m; 0 without a tail) */
  int32_t repack;                 /* bit 0: A, bit 1: B is first copied into rows starting on 128-byte
                                     boundaries of the handle's workspace (an operand whose rows do
                                     not; see gemm_set_repack); 0 otherwise */
} gemm_plan_t;

/* Counts of one planned call (see gemm_model). Counts are held as doubles (exact
 * below 2^53). The byte counts follow the no-reuse traffic count of "Reading a
 * matrix multiply through its tiles" (section "Count the repeated reads"): every
 * C tile requests its A row panel and B column panel once per K-step, and C is
 * written once; over actual ranges at partial tiles ("Edge tiles still matter"),
 * since the kernels load nothing outside the matrices. */
typedef struct {
  double flops;            /* 2 M N K, the algorithmic operation count */
  double executed_flops;   /* multiply-adds x 2 the kernel executes, the zero padding of partial
                              tiles (to whole tile_m x tile_n x tile_k blocks) included */
  double bytes_a;          /* bytes of A the load schedule requests: M K ceil(N / tile_n) elements */
  double bytes_b;          /* bytes of B requested: K N ceil(M / tile_m) elements */
  double bytes_c;          /* bytes of C written: M N elements */
  double bytes_workspace;  /* split-K partial tiles written and read back, plus operands copied into
                              aligned rows (read and written once each); 0 without either */
  double compulsory_bytes; /* A and B read once, C written once */
  int64_t tiles;           /* C tiles */
  int64_t k_steps;         /* K-steps per tile over the whole K range: ceil(K / tile_k) */
  int64_t footprint_bytes; /* working set of "What fits in local storage?": an A tile and a B tile in
                              the input format plus the fp32 (int32) C tile */
  int64_t lds_bytes;       /* LDS per workgroup, all stages */
} gemm_model_t;

/* Create a handle on the CURRENT HIP device. Host-only: no device work is enqueued.
 * Returns GEMM_ERR_NO_DEVICE if no device is visible, GEMM_ERR_ARCH if the current
 * device is not gfx950, GEMM_ERR_INVALID_ARG if out is NULL. On success *out owns
 * the handle until gemm_destroy. */
gemm_status_t gemm_create(gemm_handle_t* out);

/* C = A @ B (see the top of this file). Enqueues on `stream` and returns.
 *   M, N, K    0 .. 2^30. M == 0 or N == 0: nothing is launched. K == 0: C is
 *              filled with zeros (the empty sum).
 *   A          device pointer, M x K, row stride lda >= max(K, 1) elements.
 *   B          device pointer, K x N, row stride ldb >= max(N, 1) elements.
 *   C          device pointer, M x N, row stride ldc >= max(N, 1) elements.
 *   A/B/C may be NULL only when the matrix has no elements.
 *   dtype      one of gemm_dtype_t; element sizes: 4 (i32), 2 (f16, bf16) for A/B;
 *              4 for *_F32 and I32 outputs, 2 for *_BF16 and *_F16 outputs.
 * Errors: GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED_DTYPE, GEMM_ERR_UNSUPPORTED_TILE
 * (a forced tile this dtype has no kernel for), GEMM_ERR_OUT_OF_MEMORY (a workspace),
 * GEMM_ERR_HIP (launch failed).
 * Split-K: with the automatic tile choice, a product whose C tiles fill at most half
 * of the GPU and whose K is long is computed in K-slices (gemm_plan reports split_k),
 * so is one round of 128x128 tiles with a still longer K (slices enough for two
 * workgroups per compute unit),
 * and a last, partly full round of tiles may run as a split-K tail (tail_split_k).
 * The fp32 partial tiles go to a device workspace owned by the handle; operand
 * copies into line-aligned rows (gemm_plan reports repack; see gemm_set_repack) go
 * to a second one. Each is allocated (hipMalloc) by the first call that needs it and
 * replaced by a larger one when a later call needs more; a replaced buffer is kept
 * (work enqueued or captured earlier may still use it) until gemm_destroy frees them
 * all. Such a call is the one case where gemm_run allocates device memory, and
 * hipMalloc may synchronize with the device. Calls on one handle that use a
 * workspace share it, so they must be ordered (one stream, or synchronized between
 * streams); use one handle per stream otherwise. Partial sums are added in a fixed
 * order, so results are reproducible run to run.
 * Stream capture: a call only enqueues kernels on `stream` (no memset, no
 * synchronization), so it may be captured into a HIP graph, provided the handle's
 * workspace is already large enough: a captured call that would have to allocate or
 * grow it fails (GEMM_ERR_OUT_OF_MEMORY or GEMM_ERR_HIP). Run the call once outside
 * the capture first. */
gemm_status_t gemm_run(gemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, void* C, int64_t ldc, gemm_dtype_t dtype, void* stream);

/* C = op(A) @ op(B) with either operand supplied transposed (Mojo GPU puzzles,
 * "Tiled Matrix Multiplication", the section on transposed loading: a transposed
 * operand is read through the same shared tile). op(A) is M x K and op(B) is K x N
 * whatever the storage:
 *   op_a == GEMM_OP_N: op(A)[i][k] = A[i * lda + k], lda >= max(K, 1);
 *   op_a == GEMM_OP_T: op(A)[i][k] = A[k * lda + i], lda >= max(M, 1) (A stored K x M);
 *   op_b == GEMM_OP_N: op(B)[k][j] = B[k * ldb + j], ldb >= max(N, 1);
 *   op_b == GEMM_OP_T: op(B)[k][j] = B[j * ldb + k], ldb >= max(K, 1) (B stored N x K).
 * C is M x N row-major as in gemm_run. Everything else (dtypes, tiles, split-K,
 * empty and K == 0 cases, errors, asynchrony) is as gemm_run, which is
 * gemm_run_op(GEMM_OP_N, GEMM_OP_N, ...). An op other than GEMM_OP_N/GEMM_OP_T ->
 * GEMM_ERR_INVALID_ARG. */
gemm_status_t gemm_run_op(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                          gemm_dtype_t dtype, void* stream);

/* gemm_run_op for callers that cannot allocate memory (code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it): the same
 * arguments, errors and results, and no allocation of any kind -- no hipMalloc,
 * hipFree or allocating library call, host or device. The split-K partial tiles go
 * to a fixed scratch array of 32 MiB in device memory (one per GPU, set up by
 * gemm_create on that GPU and held until the process ends) instead of the handle's
 * workspace: a call whose plan splits K into S slices needs S * M * N * 4 bytes of it
 * (gemm_plan reports split_k), and one that needs more returns
 * GEMM_ERR_SCRATCH_TOO_SMALL before anything is enqueued. Operands are never copied
 * into aligned rows here (the results do not depend on it), and a split-K tail runs
 * only if its partial tiles fit; otherwise the plan is gemm_run_op's. The scratch
 * array holds the last call's partial tiles; nothing in it needs to start at zero.
 * Every call on one GPU shares that GPU's array, so calls that may overlap on one
 * GPU (different streams, different handles, different host threads) race and must
 * be ordered by the caller. h must have been created on the device the call runs on. */
gemm_status_t gemm_run_op_noalloc(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N,
                                  int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                                  int64_t ldc, gemm_dtype_t dtype, void* stream);

/* Choose the fastest plan for one call's shape by measurement (the pages' Helion
 * page: the compiler tunes the tile size automatically). Runs every candidate --
 * each macro tile (256x256, 256x128, 128x128, 64x64) with K-slice counts up to 32,
 * the 256x256 tile also with A loaded three K-steps ahead (stages 3), the 4-stage
 * twins where they apply, and the 16x16x32 tile for outputs of up to
 * 2^20 elements; where an operand's rows are off 128-byte boundaries and the handle
 * leaves operand copies automatic (gemm_set_repack 0), each macro-tile candidate
 * also with every subset of those operands copied into aligned rows -- on the
 * caller's buffers on `stream`: one warm-up launch and
 * `iters` (1..1000) timed launches each, timed with HIP events; then the three
 * fastest and the automatic plan again, twice, in one order and its reverse (the
 * clock drifts under sustained load), and a candidate replaces the automatic plan
 * only if it is more than 1% faster over both. BLOCKS until the stream has run
 * them. C receives the product (every candidate computes it). The chosen candidate
 * is written to *best and kept in the handle for this shape
 * (op_a, op_b, M, N, K, dtype and whether 16-byte loads apply): later gemm_run /
 * gemm_run_op / gemm_plan calls on the handle with that shape use it. A forced tile
 * or K-slice count (gemm_set_tile, gemm_set_split_k) takes precedence over a tuned
 * plan; with one set, or for the integer path and empty products, nothing is
 * measured and *best is the plan gemm_run would use. Arguments as gemm_run_op;
 * errors: those of gemm_run_op, GEMM_ERR_INVALID_ARG for a bad handle, iters or
 * best, GEMM_ERR_HIP for a failing event call. */
gemm_status_t gemm_tune(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                        gemm_dtype_t dtype, void* stream, int32_t iters, gemm_plan_t* best);

/* Release a handle and its workspaces, replaced ones included (hipFree waits for work
 * still using them). NULL or an already destroyed handle -> GEMM_ERR_INVALID_ARG. */
gemm_status_t gemm_destroy(gemm_handle_t h);

/* Force the C tile (tm x tn) and K-step tk of later gemm_run calls on this handle;
 * (0, 0, 0) returns to the library's own choice. The pages' tiles are available:
 * 3x3x3 (and any tm*tn <= 1024 with a 64 KiB LDS budget) for int32 -- the Mojo
 * puzzle's 9x9 example; 16x16x32 for the float formats -- the traffic example of
 * "Count the repeated reads"; 64x64x64 -- "Edge tiles still matter". Float formats
 * also offer 128x128x64, 256x128x64 and 256x256x64. Whether a tile fits the dtype
 * is checked by gemm_run/gemm_plan (GEMM_ERR_UNSUPPORTED_TILE). Negative values or
 * a partial zero triple -> GEMM_ERR_INVALID_ARG. */
gemm_status_t gemm_set_tile(gemm_handle_t h, int32_t tm, int32_t tn, int32_t tk);

/* Force the number of K-slices S of later gemm_run calls on this handle that use
 * the macro-tile MFMA kernel (gemm_plan_t.kernel == 4); other kernels ignore it.
 * 0 returns to the library's choice (split only with automatic tiles, when the C
 * tiles fill at most half of the GPU, or one round of 128x128 tiles, and K is long),
 * 1 never splits, 2..64 ask for
 * S slices: each holds cdiv(nk, S) of the nk K-tiles, and S is lowered so that no
 * slice is empty (gemm_plan reports the count used). Split-K needs a workspace of
 * S * M * N * 4 bytes (see gemm_run). Out of range or a bad handle ->
 * GEMM_ERR_INVALID_ARG. */
gemm_status_t gemm_set_split_k(gemm_handle_t h, int32_t splits);

/* Operand copies into aligned rows, for later calls on this handle that use the
 * macro-tile MFMA kernel with 16-byte loads (gemm_plan_t.kernel == 4,
 * vector_loads == 1). An operand whose rows do not start on 128-byte boundaries
 * (base, or a leading dimension not a multiple of 64 elements) makes every 128-byte
 * row segment of a K-tile span two cache lines; copying it first (rows padded to a
 * multiple of 64 elements, in the handle's workspace) costs one read and one write. mode 0: the library's
 * choice (copy when the estimated time saved exceeds the copy's, and the copy is at
 * most 1 GiB); 1: copy every such operand; -1: never copy. The results do not
 * depend on the mode: the same kernels see the same values in the same order.
 * Other values or a bad handle -> GEMM_ERR_INVALID_ARG. */
gemm_status_t gemm_set_repack(gemm_handle_t h, int32_t mode);

/* Validate gemm_run's arguments without a handle and without any HIP call.
 * Returns exactly the status gemm_run would return for an argument error, or
 * GEMM_OK. */
gemm_status_t gemm_check_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, const void* C, int64_t ldc, gemm_dtype_t dtype);

/* gemm_check_args for gemm_run_op's arguments (operand forms as gemm_run_op). */
gemm_status_t gemm_check_args_op(gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K, const void* A,
                                 int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                                 gemm_dtype_t dtype);

/* The configuration gemm_run would use for these arguments on this handle
 * (honouring gemm_set_tile). Host-only. h may be NULL (then the automatic
 * choice is reported). Errors as gemm_check_args, plus GEMM_ERR_UNSUPPORTED_TILE. */
gemm_status_t gemm_plan(gemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        const void* B, int64_t ldb, const void* C, int64_t ldc, gemm_dtype_t dtype,
                        gemm_plan_t* out);

/* gemm_plan for gemm_run_op's arguments. */
gemm_status_t gemm_plan_op(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                           gemm_dtype_t dtype, gemm_plan_t* out);

/* The counts of gemm_model_t for a plan (from gemm_plan / gemm_plan_op, or any
 * plan_t filled by the caller with kernel 1..4 and positive tile sizes) and the
 * call's M, N, K and dtype. Host-only. Errors: GEMM_ERR_INVALID_ARG for null
 * pointers, negative sizes or an inconsistent plan, GEMM_ERR_UNSUPPORTED_DTYPE. */
gemm_status_t gemm_model(const gemm_plan_t* plan, int64_t M, int64_t N, int64_t K, gemm_dtype_t dtype,
                         gemm_model_t* out);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* gemm_status_string(gemm_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
