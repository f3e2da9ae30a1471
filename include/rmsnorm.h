/*
 * rmsnorm.h -- C ABI of librmsnorm_mi355x.so, the row RMSNorm forward for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (per row m of a row-major [M, N] matrix):
 *
 *     rstd[m] = 1 / sqrt( (1/N) * sum_j x[m,j]^2 + eps )
 *     y[m,j]  = x[m,j] * rstd[m] * (offset + w[j])
 *
 * Defined by "Rmsnorm Kernel Optimization", section "Overview" (the
 * normalisation: x over the root of the mean square plus eps, times the
 * weight) and by the kernel listing in the opening report of "Why cutile's
 * rmsnorm required full register" (the weight enters as offset + w, with
 * offset 0.0 for Llama-style and 1.0 for Gemma3-style models; the mean
 * divides by the true width N; eps and offset are fp32; the per-row
 * reciprocal root is written out for a backward pass; y is cast to the
 * input dtype once, at the end).  x and w are read as bf16, fp16 or fp32,
 * all arithmetic is fp32 ("Rmsnorm Kernel Optimization", Key Optimizations
 * and Common Pitfalls: the sum of squares must not run in the 16-bit type),
 * the root is the hardware reciprocal square root, and y is rounded to the
 * input dtype with round-to-nearest-even.  "Rmsnorm Kernel Optimization",
 * Verification, writes the operation over the last dimension of a tensor of
 * any rank: rmsnorm_fwd_ex takes such rows through a strided layout.
 *
 * Conventions shared by every entry point:
 *   - Pointers named x, w, y, rstd are DEVICE memory owned by the caller; the
 *     library never allocates, frees or synchronises.
 *   - x and y are contiguous row-major [M, N] of `dtype` (rmsnorm_fwd_ex: rows
 *     placed by an rmsnorm_layout_t); w is [N] of `dtype`; rstd is [M] fp32.
 *   - y == x (exactly the same pointer) is allowed and normalises in place;
 *     any other overlap of y with x or w, or of rstd with x, w or y, is
 *     rejected.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without waiting.  Faults during execution show up
 *     at the caller's next synchronisation, as usual for HIP.
 *   - Argument errors are detected on the host BEFORE any HIP call and are
 *     returned as a status; nothing is enqueued then.
 *   - Calls are thread-safe.  The only library state is a per-device cache of
 *     device properties and kernel occupancy, filled on first use.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x, w and y. */
typedef enum rmsnorm_dtype {
    RMSNORM_BF16 = 0,
    RMSNORM_FP16 = 1,
    RMSNORM_FP32 = 2     /* forward and backward; four elements per 16-byte vector */
} rmsnorm_dtype_t;

/* Status codes. */
typedef enum rmsnorm_status {
    RMSNORM_OK = 0,
    RMSNORM_ERR_NULL = 1,     /* a required pointer is NULL (M > 0) */
    RMSNORM_ERR_SHAPE = 2,    /* M < 0, N <= 0, M*N*4 bytes overflows int64, a bad layout,
                                 or a workspace that is too small */
    RMSNORM_ERR_DTYPE = 3,    /* dtype is not an rmsnorm_dtype_t value */
    RMSNORM_ERR_SCALAR = 4,   /* eps < 0 or non-finite, or offset non-finite */
    RMSNORM_ERR_OVERLAP = 5,  /* buffers overlap other than y == x */
    RMSNORM_ERR_HIP = 6,      /* a HIP runtime call failed (text: rmsnorm_last_error) */
    RMSNORM_ERR_DEVICE = 7,   /* current device is not gfx950 */
    RMSNORM_ERR_PLAN = 8      /* an explicit plan does not fit this call */
} rmsnorm_status_t;

/* Kernel families. */
typedef enum rmsnorm_variant {
    RMSNORM_VARIANT_AUTO = 0,    /* let the library choose (rmsnorm_plan_query) */
    RMSNORM_VARIANT_WAVE = 1,    /* one or more rows per 64-lane wavefront, no LDS */
    RMSNORM_VARIANT_BLOCK = 2,   /* one row per workgroup, cross-wave LDS reduce */
    RMSNORM_VARIANT_GENERIC = 3, /* any N and alignment: scalar I/O, row read twice */
    RMSNORM_VARIANT_SHIFTED = 4, /* rows not 16-byte aligned (N % 8 != 0, contiguous): one row
                                    per workgroup, aligned 16-byte chunks, shifted weights.
                                    Edge chunks are read whole (the aligned 16 bytes that hold
                                    row elements) and written element by element */
    RMSNORM_VARIANT_SHIFTED_WAVE = 5, /* the same chunks for short rows: a row per segment of
                                         lanes_per_row lanes (8, 16, 32, 64), row_slots slots per
                                         wave per trip, no LDS */
    RMSNORM_VARIANT_WIDE = 6     /* aligned rows wider than the block family holds: one row per
                                    workgroup in tiles of block_threads * vectors_per_lane
                                    vectors, squares summed in a first pass, the row read again
                                    (from the caches) to normalise.  Backward: one tile per
                                    row (dw of every vector in registers), c formed in a first
                                    pass, dx in a second that reads x and dy again */
} rmsnorm_variant_t;

/*
 * Launch plan: which kernel runs and how the rows are spread over the chip.
 *
 *   variant           RMSNORM_VARIANT_WAVE / _BLOCK / _GENERIC / _SHIFTED /
 *                     _SHIFTED_WAVE / _WIDE
 *   vec_elems         elements per lane access: 16 bytes' worth, 8 (bf16, fp16)
 *                     or 4 (fp32), for every family but GENERIC (1)
 *   lanes_per_row     WAVE: lanes sharing one row (4, 8, 16, 32 or 64);
 *                     SHIFTED_WAVE: 8, 16, 32 or 64; BLOCK, SHIFTED and
 *                     GENERIC: threads per row (= block_threads, or
 *                     block_threads / row_slots for a backward BLOCK plan)
 *   vectors_per_lane  16-byte vectors (SHIFTED, SHIFTED_WAVE: aligned chunks)
 *                     each lane holds per row; lanes_per_row * vectors_per_lane
 *                     * vec_elems >= N, and >= N + vec_elems - 1 for the
 *                     shifted families, whose rows straddle one more chunk
 *   row_slots         WAVE, SHIFTED_WAVE: row slots per wave per trip; a slot
 *                     is 64/lanes_per_row rows, and all of a trip's loads are
 *                     issued before its first reduction.  Backward BLOCK: rows
 *                     per workgroup per trip (1, 2 or 4; lanes_per_row =
 *                     block_threads / row_slots threads each).  1 otherwise
 *   block_threads     workgroup size (a multiple of 64, at most 1024)
 *   prefetch          WAVE, BLOCK, SHIFTED_WAVE: 1 = load the next trip's rows
 *                     before this trip's reduction (pays off when workgroups
 *                     loop);
 *                     SHIFTED: 1 = fetch the row's weights with its x and pass
 *                     neighbouring weight vectors between lanes, 0 = fetch them
 *                     after the row's reduction; 0 otherwise
 *   xcd_group         1 to 256: the rows of this many consecutive workgroups
 *                     run on one XCD (MI355X hands workgroup b to XCD b mod 8;
 *                     the workgroup index is permuted within windows of
 *                     8 * xcd_group workgroups).  1 leaves the order alone
 *   max_blocks_per_cu 0 = no cap; 2 to 32 = at most this many workgroups per
 *                     compute unit, enforced by giving each workgroup an
 *                     otherwise unused share of the unit's LDS (an occupancy
 *                     hint: fewer rows in flight per unit can stream faster)
 *   grid              workgroups launched.  When grid times the rows one
 *                     workgroup covers per trip is below M the workgroups
 *                     loop over rows (persistent grid) and keep offset + w
 *                     in registers across trips.  The automatic plan uses
 *                     one trip per workgroup, measured fastest on MI355X;
 *                     set grid = resident_grid for a persistent launch
 *   rows_per_trip     rows one workgroup covers per loop trip (derived)
 *   trips             loop trips of the busiest workgroup (derived)
 *   resident_grid     workgroups of this kernel the device holds at once:
 *                     compute units x resident workgroups per unit (derived)
 */
typedef struct rmsnorm_plan {
    int32_t variant;
    int32_t vec_elems;
    int32_t lanes_per_row;
    int32_t vectors_per_lane;
    int32_t row_slots;
    int32_t block_threads;
    int32_t prefetch;
    int32_t xcd_group;
    int32_t max_blocks_per_cu;
    int64_t grid;
    int64_t rows_per_trip;
    int64_t trips;
    int64_t resident_grid;
} rmsnorm_plan_t;

/*
 * Row RMSNorm forward: y and rstd from x and w, as defined at the top.
 *   x      [M, N] dtype, device      w    [N] dtype, device
 *   y      [M, N] dtype, device      rstd [M] fp32, device
 *   M >= 0 rows (M == 0 is a no-op returning RMSNORM_OK), N >= 1 columns
 *   eps    >= 0, finite, added to the mean of squares inside the root
 *   offset finite, added to every weight (0.0 Llama-style, 1.0 Gemma-style)
 *   dtype  rmsnorm_dtype_t
 *   stream hipStream_t (NULL = null stream)
 * The library picks the kernel (rmsnorm_plan_query).  Returns a status.
 */
int rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd,
                int64_t M, int64_t N, float eps, float offset, int dtype, void* stream);

/*
 * Placement of rows in memory for rmsnorm_fwd_ex: the M rows form
 * M / rows batches of `rows` rows; row m = b * rows + s (b the batch, s the
 * row in it) of x starts at element  b * x_batch_stride + s * x_row_stride
 * of x, and likewise for y.  A [B, S, N] tensor with strides (sB, sS, 1) is
 * rows = S, row stride sS, batch stride sB; a 2-D [M, N] view with row
 * stride ld is rows = 0 (one batch), row stride ld.  Strides count elements
 * and must be >= 0.  Rows of x may overlap (x is only read: a row stride 0
 * broadcasts one row); rows of y may not: y_row_stride >= N when a batch
 * has several rows, and across batches either y_batch_stride >=
 * (rows - 1) * y_row_stride + N (batch-major) or y_row_stride >=
 * (batches - 1) * y_batch_stride + N with y_batch_stride >= N (row-major
 * interleaved).  rows = 0 or rows >= M means one batch; otherwise M must
 * be a multiple of rows.  Violations: RMSNORM_ERR_SHAPE.  Batches run as
 * the launch grid's second dimension, and a plan (rmsnorm_plan_query_ex,
 * or the caller's) describes one batch of `rows` rows; batches whose
 * strides continue the row stride (batch stride = rows * row stride for
 * both x and y) are treated as one batch of M rows.  The 16-byte
 * kernels run when x, w and y are 16-byte aligned and every row starts
 * 16-byte aligned (row and batch strides times the element size multiples
 * of 16); N itself may be any width.  Otherwise the generic kernel runs.
 */
typedef struct rmsnorm_layout {
    int64_t rows;
    int64_t x_row_stride;
    int64_t x_batch_stride;
    int64_t y_row_stride;
    int64_t y_batch_stride;
} rmsnorm_layout_t;

/*
 * Same as rmsnorm_fwd but with an explicit launch plan (from
 * rmsnorm_plan_query, possibly edited: variant, lanes_per_row,
 * vectors_per_lane, row_slots, block_threads, prefetch, xcd_group,
 * max_blocks_per_cu and grid are honoured;
 * the derived fields are ignored).  Returns RMSNORM_ERR_PLAN, before any HIP
 * call, if the plan's kernel does not exist, does not cover N, or needs an
 * alignment the pointers lack.  For benchmarks and tests of each kernel.
 */
int rmsnorm_fwd_with_plan(const void* x, const void* w, void* y, float* rstd,
                          int64_t M, int64_t N, float eps, float offset, int dtype,
                          const rmsnorm_plan_t* plan, void* stream);

/*
 * The general forward: rmsnorm_fwd with
 *   layout  row placement of x and y (NULL = contiguous [M, N]);
 *   rstd    may be NULL (nothing is written: inference);
 *   plan    NULL = the library's plan (tuned or rule), else as in
 *           rmsnorm_fwd_with_plan.
 * y == x in place needs the same layout for both.  Overlap checks use each
 * operand's span, from its first row's start to its last row's end.
 */
int rmsnorm_fwd_ex(const void* x, const void* w, void* y, float* rstd,
                   int64_t M, int64_t N, float eps, float offset, int dtype,
                   const rmsnorm_layout_t* layout, const rmsnorm_plan_t* plan, void* stream);

/*
 * The plan rmsnorm_fwd would use for these sizes and pointers (only their
 * alignment is looked at; they may be NULL, which counts as aligned).  The
 * plan itself is host logic.  cu_count only feeds resident_grid: cu_count > 0
 * assumes that many compute units and the register-free bound of 2048
 * threads per unit, touching no HIP API; cu_count <= 0 asks the current
 * device (unit count and the kernel's occupancy).  Writes *out and returns a
 * status.
 */
int rmsnorm_plan_query(int64_t M, int64_t N, int dtype,
                       const void* x, const void* w, const void* y,
                       int32_t cu_count, rmsnorm_plan_t* out);

/* rmsnorm_plan_query for rmsnorm_fwd_ex's layouts (NULL = contiguous). */
int rmsnorm_plan_query_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                          const rmsnorm_layout_t* layout, int32_t cu_count, rmsnorm_plan_t* out);

/*
 * Compiled resources of the kernel a plan selects, read from the loaded code
 * object (needs a device).  Any of the outputs may be NULL.
 *   vgprs       vector registers per lane (arch + accumulation)
 *   sgprs       scalar registers per wave
 *   lds_bytes   static LDS per workgroup
 *   scratch     private (spill) bytes per lane; 0 means no spills
 */
int rmsnorm_plan_resources(const rmsnorm_plan_t* plan, int dtype,
                           int32_t* vgprs, int32_t* sgprs, int32_t* lds_bytes,
                           int32_t* scratch);

/*
 * The kernel instance rmsnorm_fwd_with_plan launches for a call over
 * contiguous [M, N] rows with these pointers (alignment only; they may be
 * NULL) and `plan` (NULL = the plan rmsnorm_fwd takes), and its resources.
 * It is the plan's instance, or an exact-width form: for a wave plan, the
 * wave layout without column masks, strided rows or loop, which serves
 * one-trip, one-batch launches over rows of exactly lanes_per_row *
 * vectors_per_lane vectors without XCD remap or prefetch (widths 128, 256,
 * 512, 1024 for 16-bit dtypes; 64 to 512 for fp32); for a 256-thread block
 * plan of 4 or 8 vectors per thread, one row per workgroup without guards,
 * which serves one-batch launches of exactly M workgroups over rows of
 * exactly 256 * vectors_per_lane vectors without prefetch (widths 8192 and
 * 16384 for 16-bit dtypes, 4096 for fp32).  rmsnorm_plan_resources reports
 * the plan's general instance.  Any output may be NULL; *kernel_name
 * is a static string.  Needs a device when vgprs, lds_bytes or scratch is
 * requested; a NULL plan is planned on the host (as rmsnorm_plan_query with
 * cu_count = 256).  RMSNORM_ERR_SHAPE for M == 0 (nothing is launched).
 */
int rmsnorm_fwd_kernel_query(int64_t M, int64_t N, int dtype, const void* x, const void* w,
                             const void* y, const rmsnorm_plan_t* plan, const char** kernel_name,
                             int32_t* vgprs, int32_t* lds_bytes, int32_t* scratch);

/*
 * ---------------------------------------------------------------------------
 * Backward.  The pages store rstd "for backward" ("Why cutile's rmsnorm
 * required full register", kernel listing) but give no formula; this one is
 * the derivative of the forward above.  With g_j = offset + w_j and
 * r = rstd[m] (the forward's output, taken as given):
 *
 *     c[m]    = (1/N) sum_j dy[m,j] g_j x[m,j]
 *     dx[m,k] = r (g_k dy[m,k] - r^2 c[m] x[m,k])
 *     dw[j]   = sum_m dy[m,j] x[m,j] r[m]
 *
 * fp32 arithmetic; x, w, dy, dx of `dtype`; rstd and dw fp32.
 *
 * Two passes on `stream`: a row pass over a grid of `plan.grid` workgroups
 * writes dx and one fp32 partial row of dw per workgroup into `workspace`,
 * then a column pass adds the partial rows in a fixed order into dw (so dw is
 * the same on every run).  The workspace is caller-owned device memory of at
 * least plan.grid * N * 4 bytes; its contents on entry do not matter and on
 * return are unspecified.
 * ---------------------------------------------------------------------------
 */

/*
 * Plan of the backward row pass (variant, lanes, vectors, slots, block
 * threads, grid as for the forward; grid is the number of partial rows).
 * x, dy, dx only inform the alignment check; w, not an argument here, is taken
 * as 16-byte aligned (as every device allocation is).  cu_count as for
 * rmsnorm_plan_query.  Host only unless cu_count <= 0.
 */
int rmsnorm_bwd_plan_query(int64_t M, int64_t N, int dtype, const void* x, const void* dy,
                           const void* dx, int32_t cu_count, rmsnorm_plan_t* out);

/* Workspace bytes rmsnorm_bwd needs for these sizes and pointers (host only). */
int rmsnorm_bwd_workspace_size(int64_t M, int64_t N, int dtype, const void* x, const void* dy,
                               const void* dx, int64_t* bytes);

/*
 * Completes and checks an explicit backward plan without launching anything
 * (the counterpart of rmsnorm_plan_validate): the derived fields (vec_elems,
 * lanes_per_row of block plans, rows_per_trip, trips) and resident_grid
 * (cu_count as for rmsnorm_plan_query) are filled into *out.  Returns
 * RMSNORM_ERR_PLAN exactly when rmsnorm_bwd_with_plan would reject the plan
 * for these sizes and pointers (contiguous rows; alignment only, they may be
 * NULL; w taken as 16-byte aligned).  Host only unless cu_count <= 0.
 */
int rmsnorm_bwd_plan_validate(int64_t M, int64_t N, int dtype, const void* x, const void* dy,
                              const void* dx, const rmsnorm_plan_t* plan, int32_t cu_count,
                              rmsnorm_plan_t* out);

/*
 * Row RMSNorm backward.
 *   x, dy   [M, N] dtype, device      w  [N] dtype, device
 *   rstd    [M] fp32, device (from rmsnorm_fwd)
 *   dx      [M, N] dtype, device; may be exactly dy (in place), no other overlap
 *   dw      [N] fp32, device (written, not accumulated into)
 *   offset  finite (as in the forward)
 *   workspace, workspace_bytes: see above (RMSNORM_ERR_SHAPE if too small)
 * M == 0 writes dw = 0.  Argument errors return before any HIP call.
 */
int rmsnorm_bwd(const void* x, const void* w, const void* dy, const float* rstd, void* dx,
                float* dw, int64_t M, int64_t N, float offset, int dtype, void* workspace,
                int64_t workspace_bytes, void* stream);

/* rmsnorm_bwd with an explicit row-pass plan (honoured fields as in
 * rmsnorm_fwd_with_plan, except xcd_group and max_blocks_per_cu, which must
 * be 1 and 0; prefetch 1 exists for the wave and block shapes that fit the
 * register budget with it, RMSNORM_ERR_PLAN otherwise).  The workspace must
 * hold plan.grid * N * 4 bytes. */
int rmsnorm_bwd_with_plan(const void* x, const void* w, const void* dy, const float* rstd,
                          void* dx, float* dw, int64_t M, int64_t N, float offset, int dtype,
                          const rmsnorm_plan_t* plan, void* workspace, int64_t workspace_bytes,
                          void* stream);

/*
 * rmsnorm_bwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, plan rule, results and errors as
 * rmsnorm_bwd over contiguous [M, N] rows, minus the workspace: the dw
 * partial rows go to a scratch array of RMSNORM_BWD_SCRATCH_BYTES (16 MiB)
 * that the library keeps in device memory, one per GPU, for the life of the
 * process.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Where the rule's grid needs more partial rows than fit
 * (grid * N * 4 > RMSNORM_BWD_SCRATCH_BYTES) the grid shrinks to fit and the
 * row pass loops, so dw may then differ from rmsnorm_bwd's in rounding only;
 * N > RMSNORM_BWD_SCRATCH_BYTES / 4 is rejected with RMSNORM_ERR_SHAPE before
 * any HIP call.  All calls on one GPU share its scratch: two calls that run at
 * the same time on one GPU (different streams, no ordering between them) race
 * and give wrong dw; calls ordered on one stream do not.  The first call on a
 * device looks the scratch address up (hipGetSymbolAddress) with that device
 * current; a failure there returns RMSNORM_ERR_HIP.
 */
#define RMSNORM_BWD_SCRATCH_BYTES (16 * 1024 * 1024)
int rmsnorm_bwd_noalloc(const void* x, const void* w, const void* dy, const float* rstd, void* dx,
                        float* dw, int64_t M, int64_t N, float offset, int dtype, void* stream);

/*
 * Row layout of the backward's x, dy and dx, as rmsnorm_layout_t for the
 * forward ("Rmsnorm Kernel Optimization", Verification: the operation runs
 * over the last dimension of a tensor of any rank).  Row m = b * rows + s
 * (s < rows) starts at element b * x_batch_stride + s * x_row_stride of x,
 * likewise of dy and dx; rstd stays [M] contiguous.  rows = 0 means M (one
 * batch).  dx's rows must be disjoint (batch-major or row-major interleaved,
 * as y in the forward), x's and dy's may overlap.  With several batches
 * M < 2^31.  Element strides, >= 0.
 */
typedef struct rmsnorm_bwd_layout {
    int64_t rows;
    int64_t x_row_stride;
    int64_t x_batch_stride;
    int64_t dy_row_stride;
    int64_t dy_batch_stride;
    int64_t dx_row_stride;
    int64_t dx_batch_stride;
} rmsnorm_bwd_layout_t;

/*
 * The general backward: rows placed by `layout` (NULL = contiguous [M, N]),
 * an optional explicit plan (NULL = the library's, as rmsnorm_bwd), the
 * workspace as above.  dx may be exactly dy with the same row and batch
 * strides (in place).  The 16-byte kernels (wave, block, wide) run when x, w,
 * dy and dx are 16-byte aligned, N is a multiple of vec_elems, every stride
 * keeps rows aligned and a row has at most 32768 16-bit or 24576 fp32
 * elements; the shifted kernels (RMSNORM_VARIANT_SHIFTED_WAVE up to 128
 * chunks, RMSNORM_VARIANT_SHIFTED up to 2048) when rows are not 16-byte
 * aligned but x, dy and dx sit equally far past a 16-byte boundary on every
 * row, w is 16-byte aligned and N >= 16; the generic kernel otherwise.
 * Errors as rmsnorm_bwd, plus RMSNORM_ERR_SHAPE for a bad layout.
 */
int rmsnorm_bwd_ex(const void* x, const void* w, const void* dy, const float* rstd, void* dx,
                   float* dw, int64_t M, int64_t N, float offset, int dtype,
                   const rmsnorm_bwd_layout_t* layout, const rmsnorm_plan_t* plan, void* workspace,
                   int64_t workspace_bytes, void* stream);

/* Plan and workspace bytes of rmsnorm_bwd_ex for these sizes, pointers
 * (alignment only; they may be NULL) and layout.  Host only unless
 * cu_count <= 0 (plan query). */
int rmsnorm_bwd_plan_query_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w,
                              const void* dy, const void* dx, const rmsnorm_bwd_layout_t* layout,
                              int32_t cu_count, rmsnorm_plan_t* out);
int rmsnorm_bwd_workspace_size_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w,
                                  const void* dy, const void* dx,
                                  const rmsnorm_bwd_layout_t* layout, int64_t* bytes);

/*
 * Completes and checks an explicit forward plan without launching anything:
 * the derived fields (vec_elems, rows_per_trip, trips) and resident_grid (as
 * in rmsnorm_plan_query, cu_count likewise) are filled into *out.  Returns
 * RMSNORM_ERR_PLAN exactly when rmsnorm_fwd_with_plan would reject the plan
 * for these sizes and pointers (alignment only; they may be NULL).
 */
int rmsnorm_plan_validate(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                          const rmsnorm_plan_t* plan, int32_t cu_count, rmsnorm_plan_t* out);

/*
 * Tuned dispatch (the measured counterpart of the planner's rules, for the
 * register-budget and occupancy choices the pages tune by hand: "Why cutile's
 * rmsnorm required full register", opening report and replies).
 *
 * rmsnorm_plan_set_tuned registers `plan` (fields as for
 * rmsnorm_fwd_with_plan) for calls with exactly these M, N and dtype:
 * rmsnorm_fwd and rmsnorm_plan_query then use it instead of their own rule
 * whenever it fits the call's pointers, and fall back to the rule otherwise.
 * The plan is validated here against 16-byte aligned pointers
 * (RMSNORM_ERR_PLAN if it does not fit, RMSNORM_ERR_SHAPE for M == 0);
 * registering a shape again replaces its plan.  The table is process-wide,
 * guarded by a lock, and holds copies (the caller keeps ownership of `plan`).
 * rmsnorm_plan_clear_tuned empties it; rmsnorm_plan_tuned_count returns its
 * size.  Host only.
 */
int rmsnorm_plan_set_tuned(int64_t M, int64_t N, int dtype, const rmsnorm_plan_t* plan);
int rmsnorm_plan_clear_tuned(void);
int rmsnorm_plan_tuned_count(void);

/* Static name of a status code ("RMSNORM_OK", ...); never NULL. */
const char* rmsnorm_status_string(int status);

/*
 * Detail text of the most recent failing call on the calling thread (for
 * RMSNORM_ERR_HIP it holds the HIP error string); "" if none.  The pointer
 * stays valid until the next library call on the same thread.
 */
const char* rmsnorm_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int rmsnorm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
