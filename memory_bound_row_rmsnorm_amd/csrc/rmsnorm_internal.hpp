// rmsnorm_internal.hpp -- what the kernel translation unit exports to the
// host dispatcher: a table of compiled kernel instances, all with one
// argument list, so the dispatcher launches any of them the same way.
#pragma once

#include <stdint.h>

namespace rmsnorm_impl {

// Every kernel takes exactly these arguments, in this order.
//   x, w, y : element buffers of the dtype (device), rstd : fp32 [M] (device)
//   M rows, N columns, inv_n = fp32(1/N), eps, offset
//   xcd_group: consecutive workgroups' worth of rows placed on one XCD (1 = none)
//   grid, threads : the launch's workgroup count and workgroup size, passed
//   here so the kernels read no launch geometry from the dispatch's hidden
//   arguments (a second scalar-memory round trip before the first row load)
//   (the fields the kernels need before their first row load come first, in
//   the 64 bytes the kernels' first scalar loads fetch together)
//   M is the rows of one batch; the launch's grid y dimension counts the
//   batches.  Row m of batch b of x starts at element b * x_bs + m * x_rs,
//   likewise for y, and its rstd is rstd[b * M + m].  rstd may be NULL (not
//   written).
struct KernelArgs {
    // the first 64 bytes: everything the first row load depends on
    const void* x;
    int64_t M;
    int64_t N;
    int64_t grid;
    int32_t threads;
    int32_t xcd_group;
    int32_t x_rsv;      // row stride of x in 16-byte vectors (vector kernels; < 2^31)
    int32_t y_rsv;      // row stride of y in 16-byte vectors
    int64_t x_bs;       // batch stride of x, elements
    const void* w;
    int64_t x_rs;       // row stride of x, elements (element-wise kernels)
    // the rest: needed after the loads are in flight
    void* y;
    float* rstd;
    int64_t y_rs;       // row stride of y, elements
    int64_t y_bs;       // batch stride of y, elements
    float inv_n;
    float eps;
    float offset;
};

// Arguments of every backward row-pass kernel.
//   x, w, dy : element buffers of the dtype (device); rstd : fp32 [M] (device)
//   dx : output rows of the dtype; partials : fp32 [grid, N] workspace rows
//   Row m (0 <= m < M) is row m % rows of batch m / rows; it starts at
//   element (m / rows) * x_bs + (m % rows) * x_rs of x, likewise for dy and
//   dx, and its rstd is rstd[m].  One batch: rows = M (no division).
struct BwdArgs {
    const void* x;
    const void* w;
    const void* dy;
    const float* rstd;
    void* dx;
    float* partials;
    int64_t M;
    int64_t N;
    int64_t grid;       // launch geometry, as in KernelArgs
    int32_t threads;
    float inv_n;
    float offset;
    int64_t rows;       // rows per batch; M < 2^31 when rows < M
    int64_t x_rs, dy_rs, dx_rs;   // row strides, elements
    int64_t x_bs, dy_bs, dx_bs;   // batch strides, elements
};

struct KernelEntry {
    int variant;           // rmsnorm_variant_t
    int dtype;             // rmsnorm_dtype_t
    int lanes_per_row;     // WAVE: 4/8/16/32/64; SHIFTED_WAVE: 8/16/32/64; others: 0 (= block size)
    int vectors_per_lane;  // WAVE, BLOCK: 16-byte vectors per lane per row; GENERIC: 0
    int row_slots;         // WAVE: slots per wave per trip; others 1
    bool prefetch;         // WAVE, BLOCK: next trip's rows loaded before this trip's reduction
    bool tails;            // handles N that is not a multiple of the vector (forward)
    const void* func;      // host stub of the __global__ function
    const char* name;
};

// The compiled instances (defined in rmsnorm_kernels.hip).
const KernelEntry* kernel_table(int* count);

// The exact-width wave form with this row segment shape and workgroup size,
// or nullptr.  It serves one-trip, one-batch, unremapped, non-prefetching
// launches of a wave plan over contiguous rows of exactly lanes * vpl
// vectors, with M below kExactMaxRows; its arguments are KernelArgs as for
// every forward kernel.
const KernelEntry* exact_wave_kernel(int dtype, int lanes, int vpl, int slots, int threads);
constexpr int64_t kExactMaxRows = (int64_t{1} << 31) - (int64_t{1} << 16);

// The exact-width block form with this many vectors per thread and
// workgroup size, or nullptr.  It holds one row of exactly threads * vpt
// vectors per workgroup and runs one trip over one batch of contiguous rows;
// block plans with vpt vectors per thread exist only through it.
const KernelEntry* exact_block_kernel(int dtype, int vpt, int threads);

// Backward row-pass instances and the column-pass kernel (rmsnorm_bwd_kernels.hip).
// The column pass takes (const float* partials, float* dw, int64_t G, int64_t N,
// int32_t vec4): vec4 = 1 when N % 4 == 0 and dw is 16-byte aligned.
const KernelEntry* bwd_kernel_table(int* count);
// split 16 or 64, cols (column groups per workgroup) 4 or 16: cols * split threads
const void* dw_reduce_kernel(int split, int cols);

// Device address of the current device's RMSNORM_BWD_SCRATCH_BYTES scratch
// array (rmsnorm_bwd_noalloc's dw partial rows), looked up once per device.
// Returns nullptr and sets *ptr, or returns the error text.
const char* bwd_scratch(void** ptr);

}  // namespace rmsnorm_impl
