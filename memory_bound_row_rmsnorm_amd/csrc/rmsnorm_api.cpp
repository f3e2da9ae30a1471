// rmsnorm_api.cpp -- host side of librmsnorm_mi355x.so: argument checks,
// launch planning and the C ABI declared in include/rmsnorm.h.
//
// Argument checks are pure host code and run before any HIP call, so a bad
// call never enqueues work.  Planning picks a kernel family and geometry from
// the row width (the pages' row-parallel design: one program per row, several
// rows per program when rows are short -- "Rmsnorm Kernel Optimization", Core
// Technique and Key Optimizations) and caps the grid at what the compute
// units hold at once (the static persistent grid of the cuTile listing in
// "Why cutile's rmsnorm required full register").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "../../include/rmsnorm.h"
#include "rmsnorm_internal.hpp"

using rmsnorm_impl::BwdArgs;
using rmsnorm_impl::KernelArgs;
using rmsnorm_impl::KernelEntry;

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr int kMaxDevices = 64;
constexpr int kWaveBlockThreads = 256;   // 4 waves per workgroup for the wave family, one row per slot
constexpr int kWaveBlockThreadsMultiRow = 128;   // 2 waves when a slot holds several rows
constexpr int kMaxThreadsPerCu = 2048;   // 4 SIMDs x 8 waves x 64 lanes
constexpr int kMaxXcdGroup = 256;        // largest xcd_group a plan takes

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

// ---------------------------------------------------------------------------
// Per-device cache: compute-unit count, architecture check, and occupancy of
// each (kernel, block size) the dispatcher has launched.
// ---------------------------------------------------------------------------
struct DeviceInfo {
    std::once_flag once;
    int status = RMSNORM_OK;
    std::string error;
    int cu_count = 0;
    int lds_per_cu = 0;
};

DeviceInfo g_devices[kMaxDevices];

int device_info(int* cu_count, int* lds_per_cu = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RMSNORM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(RMSNORM_ERR_DEVICE, "device ordinal out of range");
    DeviceInfo& d = g_devices[dev];
    std::call_once(d.once, [&d, dev]() {
        hipDeviceProp_t p;
        hipError_t err = hipGetDeviceProperties(&p, dev);
        if (err != hipSuccess) {
            d.status = RMSNORM_ERR_HIP;
            d.error = std::string("hipGetDeviceProperties: ") + hipGetErrorString(err);
            return;
        }
        if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) {
            d.status = RMSNORM_ERR_DEVICE;
            d.error = std::string("librmsnorm_mi355x is built for gfx950, device is ") + p.gcnArchName;
            return;
        }
        d.cu_count = p.multiProcessorCount;
        d.lds_per_cu = static_cast<int>(p.maxSharedMemoryPerMultiProcessor);
    });
    if (d.status != RMSNORM_OK) return fail(d.status, d.error);
    *cu_count = d.cu_count;
    if (lds_per_cu) *lds_per_cu = d.lds_per_cu;
    return RMSNORM_OK;
}

std::mutex g_occ_mu;
std::map<std::tuple<int, const void*, int>, int> g_occ;  // (device, kernel, threads) -> blocks per CU

// Workgroups of `threads` threads of kernel `func` one CU holds at once.
int occupancy(const void* func, int threads, int* blocks) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RMSNORM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    const auto key = std::make_tuple(dev, func, threads);
    std::lock_guard<std::mutex> lock(g_occ_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) {
        *blocks = it->second;
        return RMSNORM_OK;
    }
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, func, threads, 0);
    if (e != hipSuccess)
        return fail(RMSNORM_ERR_HIP,
                    std::string("hipOccupancyMaxActiveBlocksPerMultiprocessor: ") + hipGetErrorString(e));
    if (n < 1) n = 1;
    g_occ.emplace(key, n);
    *blocks = n;
    return RMSNORM_OK;
}

// ---------------------------------------------------------------------------
// Argument checks (host only).
// ---------------------------------------------------------------------------
bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

int elem_size(int dtype) { return dtype == RMSNORM_FP32 ? 4 : 2; }
int elems_per_vector(int dtype) { return 16 / elem_size(dtype); }

// Forward and backward calls take all three dtypes.
int check_shape_dtype(int64_t M, int64_t N, int dtype) {
    if (M < 0) return fail(RMSNORM_ERR_SHAPE, "M must be >= 0");
    if (N <= 0) return fail(RMSNORM_ERR_SHAPE, "N must be >= 1");
    if (M > 0 && N > INT64_MAX / 4 / M) return fail(RMSNORM_ERR_SHAPE, "M*N*4 bytes overflows int64");
    if (dtype != RMSNORM_BF16 && dtype != RMSNORM_FP16 && dtype != RMSNORM_FP32)
        return fail(RMSNORM_ERR_DTYPE, "dtype must be RMSNORM_BF16, RMSNORM_FP16 or RMSNORM_FP32");
    return RMSNORM_OK;
}

// Row layout of x and y in elements, normalised: `rows` rows per batch,
// M / rows batches.  Contiguous [M, N] is one batch with row stride N.
struct Layout {
    int64_t rows;
    int64_t x_rs, x_bs, y_rs, y_bs;
    int64_t batches(int64_t M) const { return rows > 0 ? M / rows : 0; }
    // elements from the first element of row 0 to one past the last element of the last row
    int64_t x_span(int64_t M, int64_t N) const { return span(M, N, x_rs, x_bs); }
    int64_t y_span(int64_t M, int64_t N) const { return span(M, N, y_rs, y_bs); }
    int64_t span(int64_t M, int64_t N, int64_t rs, int64_t bs) const {
        if (M == 0) return 0;
        return (batches(M) - 1) * bs + (rows - 1) * rs + N;
    }
};

Layout contiguous_layout(int64_t M, int64_t N) { return Layout{M > 0 ? M : 1, N, M * N, N, M * N}; }

// Checks a caller's layout and normalises it.  y's rows must not overlap one
// another (the kernels write them concurrently): either batch-major
// (y_batch_stride >= (rows - 1) * y_row_stride + N) or row-major interleaved
// (y_row_stride >= (batches - 1) * y_batch_stride + N), with y_row_stride >= N
// when a batch has several rows.  x's rows may overlap (x is only read).
int normalise_layout(const rmsnorm_layout_t* L, int64_t M, int64_t N, Layout* out) {
    if (!L) {
        *out = contiguous_layout(M, N);
        return RMSNORM_OK;
    }
    if (L->rows < 0) return fail(RMSNORM_ERR_SHAPE, "layout rows must be >= 0");
    if (L->x_row_stride < 0 || L->x_batch_stride < 0 || L->y_row_stride < 0 || L->y_batch_stride < 0)
        return fail(RMSNORM_ERR_SHAPE, "layout strides must be >= 0");
    Layout o;
    o.rows = (L->rows == 0 || L->rows >= M) ? (M > 0 ? M : 1) : L->rows;
    if (M > 0 && M % o.rows != 0) return fail(RMSNORM_ERR_SHAPE, "M must be a multiple of layout rows");
    o.x_rs = L->x_row_stride;
    o.y_rs = L->y_row_stride;
    const int64_t B = M > 0 ? M / o.rows : 1;
    o.x_bs = B > 1 ? L->x_batch_stride : 0;
    o.y_bs = B > 1 ? L->y_batch_stride : 0;
    const int64_t lim = INT64_MAX / 4;
    if (o.rows > 1 && o.y_rs < N) return fail(RMSNORM_ERR_SHAPE, "y rows overlap: y_row_stride < N");
    if (o.x_rs > lim / (o.rows > 1 ? o.rows : 1) || o.y_rs > lim / (o.rows > 1 ? o.rows : 1) ||
        o.x_bs > lim / B || o.y_bs > lim / B)
        return fail(RMSNORM_ERR_SHAPE, "layout spans overflow int64");
    if (B > 1) {
        const bool batch_major = o.y_bs >= (o.rows - 1) * o.y_rs + N;
        const bool interleaved = o.y_rs >= (B - 1) * o.y_bs + N && o.y_bs >= N;
        if (!batch_major && !interleaved) return fail(RMSNORM_ERR_SHAPE, "y rows overlap across batches");
    }
    if (o.x_span(M, N) > lim || o.y_span(M, N) > lim) return fail(RMSNORM_ERR_SHAPE, "layout spans overflow int64");
    if (B > 1 && o.x_bs == o.rows * o.x_rs && o.y_bs == o.rows * o.y_rs) {
        // batches that continue each other's row stride are one batch
        o.rows = M;
        o.x_bs = 0;
        o.y_bs = 0;
    }
    *out = o;
    return RMSNORM_OK;
}

int check_args(const void* x, const void* w, const void* y, const float* rstd, int64_t M, int64_t N,
               float eps, float offset, int dtype, const Layout& L, bool rstd_optional = false) {
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    if (M > 0 && (!x || !w || !y || (!rstd && !rstd_optional)))
        return fail(RMSNORM_ERR_NULL, rstd_optional ? "x, w and y must be non-NULL" : "x, w, y and rstd must be non-NULL");
    if (!std::isfinite(eps) || eps < 0.0f) return fail(RMSNORM_ERR_SCALAR, "eps must be finite and >= 0");
    if (!std::isfinite(offset)) return fail(RMSNORM_ERR_SCALAR, "offset must be finite");
    if (M == 0) return RMSNORM_OK;
    const int64_t es = elem_size(dtype);
    const int64_t xb = L.x_span(M, N) * es, yb = L.y_span(M, N) * es, wb = N * es, rb = M * 4;
    const bool same_layout = L.x_rs == L.y_rs && L.x_bs == L.y_bs;
    if (x == y ? !same_layout : ranges_overlap(x, xb, y, yb))
        return fail(RMSNORM_ERR_OVERLAP, "y overlaps x (in place needs y == x with the same layout)");
    if (ranges_overlap(y, yb, w, wb)) return fail(RMSNORM_ERR_OVERLAP, "y overlaps w");
    if (rstd && (ranges_overlap(rstd, rb, x, xb) || ranges_overlap(rstd, rb, y, yb) || ranges_overlap(rstd, rb, w, wb)))
        return fail(RMSNORM_ERR_OVERLAP, "rstd overlaps x, y or w");
    return RMSNORM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The 16-byte kernels need 16-byte aligned x, w and y and row (and batch)
// strides that keep every row 16-byte aligned; N itself may be anything (a
// final partial vector moves element by element).
bool vector_ok(const void* x, const void* w, const void* y, int dtype, const Layout& L, int64_t M) {
    const int64_t es = elem_size(dtype);
    // with one row per batch the row stride is never applied
    const bool rows_ok = L.rows <= 1 || ((L.x_rs * es) % 16 == 0 && (L.y_rs * es) % 16 == 0 &&
                                         L.x_rs * es / 16 < INT32_MAX && L.y_rs * es / 16 < INT32_MAX);
    const bool batches_ok = L.batches(M) <= 1 || ((L.x_bs * es) % 16 == 0 && (L.y_bs * es) % 16 == 0);
    return aligned16(x) && aligned16(w) && aligned16(y) && rows_ok && batches_ok;
}

// What a call's pointers and layout allow: the 16-byte kernels (every row
// 16-byte aligned), or the shifted kernel (rows of x and y equally far past a
// 16-byte boundary on every row: the same layout and equally aligned bases;
// w 16-byte aligned).
struct Access {
    bool vec;
    bool shifted;
    bool contiguous;   // one batch of rows N elements apart (or a single row), x and y alike
};

Access access_of(const void* x, const void* w, const void* y, int dtype, const Layout& L, int64_t M, int64_t N) {
    const uintptr_t es = static_cast<uintptr_t>(elem_size(dtype));
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
    const bool same_layout = L.x_rs == L.y_rs && (L.batches(M) <= 1 || L.x_bs == L.y_bs);
    Access a;
    a.vec = vector_ok(x, w, y, dtype, L, M);
    a.shifted = !a.vec && aligned16(w) && xa % es == 0 && ya % es == 0 && xa % 16 == ya % 16 && same_layout;
    a.contiguous = L.batches(M) <= 1 && (M <= 1 || L.rows <= 1 || (L.x_rs == N && L.y_rs == N));
    return a;
}

// ---------------------------------------------------------------------------
// Kernel lookup.
// ---------------------------------------------------------------------------
const KernelEntry* find_kernel(int variant, int dtype, int lanes, int vpl, int slots, bool prefetch) {
    int n = 0;
    const KernelEntry* t = rmsnorm_impl::kernel_table(&n);
    for (int i = 0; i < n; ++i) {
        const KernelEntry& k = t[i];
        if (k.variant != variant || k.dtype != dtype || k.prefetch != prefetch) continue;
        if ((variant == RMSNORM_VARIANT_WAVE || variant == RMSNORM_VARIANT_SHIFTED_WAVE) &&
            (k.lanes_per_row != lanes || k.vectors_per_lane != vpl || k.row_slots != slots))
            continue;
        if ((variant == RMSNORM_VARIANT_BLOCK || variant == RMSNORM_VARIANT_SHIFTED || variant == RMSNORM_VARIANT_WIDE) &&
            k.vectors_per_lane != vpl)
            continue;
        return &k;
    }
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A dispatch holds fewer than 2^32 work-items per grid dimension (the packet's
// grid size is 32 bits) and fewer than 2^31 workgroups: the largest grid of
// `threads`-thread workgroups one launch takes.  Larger row counts loop.
int64_t grid_limit(int threads) {
    const int64_t by_items = ((int64_t{1} << 32) - 1) / (threads > 0 ? threads : 1);
    return by_items < 0x7FFFFFFF ? by_items : 0x7FFFFFFF;
}

int check_grid(const rmsnorm_plan_t* p) {
    if (p->grid < 1 || p->grid > 0x7FFFFFFF) return fail(RMSNORM_ERR_PLAN, "grid must be in [1, 2^31)");
    if (p->grid > grid_limit(p->block_threads))
        return fail(RMSNORM_ERR_PLAN, "grid * block_threads must stay below 2^32 work-items");
    return RMSNORM_OK;
}

// The instance a launch of plan p with kernel k runs: an exact-width form
// when the call fits it, k otherwise.  Both need a non-prefetching plan, one
// batch of contiguous rows of exactly (segment or workgroup) * vectors
// vectors, one trip, and row numbers of the whole grid below 2^31.  The
// wave form also needs no XCD remap and fewer than kExactMaxRows rows and
// keeps the plan's segment shape and workgroup size; the block form (256
// threads x 4 or 8 vectors) needs a grid of exactly M workgroups and keeps
// the plan's XCD groups and cap.  M is the
// rows of one batch, `batches` the batch count.  Host only.
const KernelEntry* launch_instance(const KernelEntry* k, const rmsnorm_plan_t* p, int64_t M, int64_t N, int dtype,
                                   const Layout& L, int64_t batches) {
    if (k->prefetch || batches != 1) return k;
    if (k->variant != RMSNORM_VARIANT_WAVE && k->variant != RMSNORM_VARIANT_BLOCK) return k;
    if (M > 1 && (L.x_rs != N || L.y_rs != N)) return k;
    const int64_t covered = p->grid * p->rows_per_trip;
    if (covered < M || covered >= (int64_t{1} << 31)) return k;
    const int64_t epv = elems_per_vector(dtype);
    if (k->variant == RMSNORM_VARIANT_BLOCK) {
        // a workgroup per row and no more: the block form has no guard for rows past M
        if (covered != M || N != static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * epv) return k;
        const KernelEntry* e = rmsnorm_impl::exact_block_kernel(dtype, p->vectors_per_lane, p->block_threads);
        return e ? e : k;
    }
    if (p->xcd_group != 1 || M >= rmsnorm_impl::kExactMaxRows) return k;
    if (N != static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv) return k;
    const KernelEntry* e = rmsnorm_impl::exact_wave_kernel(dtype, p->lanes_per_row, p->vectors_per_lane,
                                                           p->row_slots, p->block_threads);
    return e ? e : k;
}

// Fill the derived fields and check the plan against the call (`vec`: the
// call's pointers and strides suit the 16-byte kernels).  Host only.
int finish_plan(rmsnorm_plan_t* p, int64_t M, int64_t N, int dtype, Access acc, const KernelEntry** kernel) {
    const bool vec = acc.vec;
    if (p->block_threads < 64 || p->block_threads > 1024 || p->block_threads % 64 != 0)
        return fail(RMSNORM_ERR_PLAN, "block_threads must be a multiple of 64 in [64, 1024]");
    if (check_grid(p) != RMSNORM_OK) return RMSNORM_ERR_PLAN;
    if (p->xcd_group < 1 || p->xcd_group > kMaxXcdGroup)
        return fail(RMSNORM_ERR_PLAN, "xcd_group must be in [1, " + std::to_string(kMaxXcdGroup) + "]");
    if (p->max_blocks_per_cu != 0 && (p->max_blocks_per_cu < 2 || p->max_blocks_per_cu > 32))
        return fail(RMSNORM_ERR_PLAN, "max_blocks_per_cu must be 0 or in [2, 32]");
    const KernelEntry* k = nullptr;
    if (p->variant == RMSNORM_VARIANT_GENERIC) {
        p->vec_elems = 1;
        p->lanes_per_row = p->block_threads;
        p->vectors_per_lane = 0;
        p->row_slots = 1;
        p->prefetch = 0;
        p->rows_per_trip = 1;
        k = find_kernel(RMSNORM_VARIANT_GENERIC, dtype, 0, 0, 1, false);
    } else if (p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_BLOCK) {
        if (!vec)
            return fail(RMSNORM_ERR_PLAN, "16-byte kernels need 16-byte aligned x, w and y and 16-byte aligned rows");
        const int epv = elems_per_vector(dtype);
        p->vec_elems = epv;
        if (p->prefetch != 0 && p->prefetch != 1) return fail(RMSNORM_ERR_PLAN, "prefetch must be 0 or 1");
        if (p->variant == RMSNORM_VARIANT_WAVE) {
            k = find_kernel(RMSNORM_VARIANT_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, p->row_slots,
                            p->prefetch != 0);
            if (k) {
                const int64_t cap = static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv;
                if (cap < N) return fail(RMSNORM_ERR_PLAN, "wave plan does not cover N");
                p->rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
            }
        } else {
            p->row_slots = 1;
            p->lanes_per_row = p->block_threads;
            k = find_kernel(RMSNORM_VARIANT_BLOCK, dtype, 0, p->vectors_per_lane, 1, p->prefetch != 0);
            if (!k && p->prefetch == 0) {
                // shapes only the exact-width block form holds: one batch of contiguous rows of
                // exactly block_threads * vectors_per_lane vectors, one trip
                const KernelEntry* e = rmsnorm_impl::exact_block_kernel(dtype, p->vectors_per_lane, p->block_threads);
                if (e) {
                    if (!acc.contiguous || N != static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * epv)
                        return fail(RMSNORM_ERR_PLAN, "this block shape runs only over one batch of contiguous rows of "
                                                      "exactly block_threads * vectors_per_lane vectors");
                    if (p->grid != M)
                        return fail(RMSNORM_ERR_PLAN, "this block shape runs one trip: grid must equal M");
                    k = e;
                }
            }
            if (k) {
                const int64_t cap = static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * epv;
                if (cap < N) return fail(RMSNORM_ERR_PLAN, "block plan does not cover N");
                p->rows_per_trip = 1;
            }
        }
    } else if (p->variant == RMSNORM_VARIANT_SHIFTED) {
        if (!acc.shifted)
            return fail(RMSNORM_ERR_PLAN, "the shifted kernel needs x and y equally aligned with the same layout, "
                                          "16-byte aligned w, and rows that are not 16-byte aligned");
        const int epv = elems_per_vector(dtype);
        p->vec_elems = epv;
        p->row_slots = 1;
        p->lanes_per_row = p->block_threads;
        p->rows_per_trip = 1;
        if (p->prefetch != 0 && p->prefetch != 1) return fail(RMSNORM_ERR_PLAN, "prefetch must be 0 or 1");
        k = find_kernel(RMSNORM_VARIANT_SHIFTED, dtype, 0, p->vectors_per_lane, 1, p->prefetch != 0);
        if (k && static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * epv < N + epv - 1)
            return fail(RMSNORM_ERR_PLAN, "shifted plan does not cover N");
    } else if (p->variant == RMSNORM_VARIANT_WIDE) {
        if (!vec)
            return fail(RMSNORM_ERR_PLAN, "16-byte kernels need 16-byte aligned x, w and y and 16-byte aligned rows");
        p->vec_elems = elems_per_vector(dtype);
        p->row_slots = 1;
        p->lanes_per_row = p->block_threads;
        p->rows_per_trip = 1;
        if (p->prefetch != 0) return fail(RMSNORM_ERR_PLAN, "the wide kernel has no prefetching form");
        k = find_kernel(RMSNORM_VARIANT_WIDE, dtype, 0, p->vectors_per_lane, 1, false);
    } else if (p->variant == RMSNORM_VARIANT_SHIFTED_WAVE) {
        if (!acc.shifted)
            return fail(RMSNORM_ERR_PLAN, "the shifted kernels need x and y equally aligned with the same layout, "
                                          "16-byte aligned w, and rows that are not 16-byte aligned");
        const int epv = elems_per_vector(dtype);
        p->vec_elems = epv;
        if (p->prefetch != 0 && p->prefetch != 1) return fail(RMSNORM_ERR_PLAN, "prefetch must be 0 or 1");
        if (p->lanes_per_row != 8 && p->lanes_per_row != 16 && p->lanes_per_row != 32 && p->lanes_per_row != 64)
            return fail(RMSNORM_ERR_PLAN, "shifted wave plans take 8, 16, 32 or 64 lanes per row");
        k = find_kernel(RMSNORM_VARIANT_SHIFTED_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, p->row_slots,
                        p->prefetch != 0);
        if (k && static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv < N + epv - 1)
            return fail(RMSNORM_ERR_PLAN, "shifted wave plan does not cover N");
        p->rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
    } else {
        return fail(RMSNORM_ERR_PLAN, "unknown variant");
    }
    if (!k) return fail(RMSNORM_ERR_PLAN, "no compiled kernel for this plan");
    if (!k->tails && N % p->vec_elems != 0)
        return fail(RMSNORM_ERR_PLAN, "this kernel has no tail path: N must be a multiple of vec_elems");
    p->trips = M > 0 ? ceil_div(ceil_div(M, p->rows_per_trip), p->grid) : 0;
    if (kernel) *kernel = k;
    return RMSNORM_OK;
}

// Vectors per lane the block and wave families are compiled for (more would
// not fit the 128 VGPRs a 1024-thread workgroup allows without spilling).
constexpr int kWaveSlots[] = {8, 4, 2, 1};
constexpr int64_t kMaxVectors = 1024LL * 6;       // widest row the 16-byte kernels hold, in vectors
constexpr int64_t kMaxShiftedChunks = 1024LL * 4;  // widest row the shifted kernel holds, in chunks
// vectors per thread per tile of the wide kernel (4096 x 40968 bf16: 134.5 us
// with 1024 x 2, 140.1 us with 1024 x 4, 373.7 us generic)
constexpr int kWideVectors = 2;
constexpr int64_t kMaxShiftedWaveChunks = 64 * 2;  // widest row the shifted wave kernel holds, in chunks
constexpr int kShiftedWaveSlots = 4;               // slots per wave per trip of the shifted wave plans
// Unaligned rows shorter than this take the generic kernel.  The shifted wave
// kernel is ahead of it down to short rows (262144 x 36 bf16: 61.3 against
// 66.9 us; 262144 x 100 bf16: 62.2 against 89.5 us).
constexpr int64_t kMinShiftedWaveN = 16;
constexpr int64_t kWaveBytesInFlight = 4096;      // row bytes one wave loads per trip
constexpr int64_t kHalfWaveRowsMinRows = 16384;   // rows from which 64-vector rows take 32-lane segments
constexpr int64_t kWaveBytesInFlightMultiRow = 2048;   // the same when a slot holds several rows
constexpr int64_t kXcdGroupBytes = 128 * 1024;    // consecutive row bytes per XCD (block family)
constexpr int64_t kXcdGroupBytesLarge = 1024 * 1024;   // the same for batches beyond the Infinity Cache
constexpr int64_t kInfinityCacheBytes = 256LL * 1024 * 1024;
constexpr int64_t kBytesInFlightPerCu = 64 * 1024; // row bytes resident per compute unit (block family)
constexpr int kMinBlocksPerCu = 3;                 // the occupancy cap never goes below this

// Choose family and geometry (host only; no device needed).  A row is
// nvec = ceil(N / EPV) 16-byte vectors (EPV = 8 for bf16/fp16, 4 for fp32).
// Rules measured on MI355X with inputs cold in HBM:
//  * rows of at most 128 vectors: the wave family, 4/8/16/32/64 lanes per
//    row so that a row segment is one 16-byte vector per lane (two at 128),
//    and enough rows per wave for about 4 KiB of loads per trip (2 KiB in
//    2-wave workgroups when a slot holds several rows of 8 to 32 lanes);
//  * longer rows: the block family with 256 threads up to 1536 vectors and
//    1024 beyond, each thread holding ceil(nvec / threads) vectors;
//  * pointers or row strides that are not 16-byte aligned, or a row wider
//    than 6144 vectors: the generic kernel;
//  * one trip per workgroup (grid = row groups): launching every row group
//    measured faster than a grid of resident workgroups looping over rows on
//    every shape tried;
//  * block family: consecutive rows grouped on one XCD, about 128 KiB per
//    group (xcd_group 16 at 6000-byte rows), or about 1 MiB per group when
//    one batch of x exceeds the 256 MB Infinity Cache (xcd_group 64 at 16 KiB
//    rows, 128 at 8 KiB, 32 at 32 KiB); and at most about 64 KiB of rows, but
//    never fewer than 3 workgroups, resident per compute unit
//    (max_blocks_per_cu 4 at 16 KiB rows, 3 at 24 KiB; 3 for the exact-width
//    forms).  With the block family's kernel the 128 KiB groups were 5-6%
//    faster than none on 32768 x 8192 at a favourable placement of y
//    relative to x, but the rate then followed that placement over a 10%
//    range (165-181 us); 1 MiB groups hold 167-169 us (the exact-width form)
//    at every placement measured, and lift the median over placements by
//    1-3.5% at 4 KiB to 32 KiB rows.
//    Below 256 MB the placement does not matter and 128 KiB groups lead
//    (8192 x 3000: 18.1 us against 18.7 with 384 KiB groups).  A cap of 2 at
//    24 KiB rows left 512-thread workgroups at 193 us on 21840 x 12288,
//    against 173 us with 3.
int choose_plan(int64_t M, int64_t N, int dtype, Access acc, rmsnorm_plan_t* p) {
    std::memset(p, 0, sizeof(*p));
    const bool vec = acc.vec;
    const int64_t es = elem_size(dtype);
    const int64_t nvec = ceil_div(N, elems_per_vector(dtype));
    const int64_t nchunks = ceil_div(N + elems_per_vector(dtype) - 1, elems_per_vector(dtype));
    if (!vec && acc.shifted && N >= kMinShiftedWaveN && nchunks <= kMaxShiftedWaveChunks) {
        // a row per segment of the fewest lanes (8, 16, 32, 64) that hold its
        // chunks, 4-wave workgroups; four slots per wave, two with 8- and
        // 16-lane rows (262144 x 257 bf16: 73 us, against 97 us with one row
        // per 64-thread workgroup and 163 us generic; 16384 x 1001 bf16: 14.4
        // us with four slots against 16.0 us with two; 262144 x 100 bf16: 28.0
        // us with 16-lane rows and two slots, 29.7 with four, 61.5 with a row
        // per wave; 262144 x 36 bf16: 16.1 us with 8-lane rows, 22.4 with 16)
        p->variant = RMSNORM_VARIANT_SHIFTED_WAVE;
        p->lanes_per_row = nchunks <= 8 ? 8 : (nchunks <= 16 ? 16 : (nchunks <= 32 ? 32 : 64));
        p->vectors_per_lane = static_cast<int>(ceil_div(nchunks, p->lanes_per_row));
        p->block_threads = kWaveBlockThreads;
        p->row_slots = p->lanes_per_row <= 16 ? 2 : kShiftedWaveSlots;
    } else if (!vec && acc.shifted && nchunks > kMaxShiftedWaveChunks && nchunks <= kMaxShiftedChunks) {
        // one row per workgroup: the fewest threads (64 to 1024) that hold the
        // row's chunks with at most 3 per thread (32768 x 8191 bf16: 194 us with
        // 512 x 3 against 305 us with 1024 x 2; 8192 x 3001 bf16: 20.0 us with
        // 128 x 3 against 26.2 us with 256 x 2)
        p->variant = RMSNORM_VARIANT_SHIFTED;
        p->row_slots = 1;
        p->block_threads = 64;
        while (p->block_threads < 1024 && nchunks > 3LL * p->block_threads) p->block_threads *= 2;
        p->vectors_per_lane = static_cast<int>(ceil_div(nchunks, p->block_threads));
    } else if (!vec) {
        p->variant = RMSNORM_VARIANT_GENERIC;
        p->block_threads = N >= 1024 ? 256 : (N >= 256 ? 128 : 64);
        p->row_slots = 1;
    } else if (nvec > kMaxVectors) {
        // rows wider than the registers of a 1024-thread workgroup hold: two
        // passes over 1024 x 2 vector tiles
        p->variant = RMSNORM_VARIANT_WIDE;
        p->block_threads = 1024;
        p->vectors_per_lane = kWideVectors;
        p->row_slots = 1;
    } else if (nvec <= 128) {
        p->variant = RMSNORM_VARIANT_WAVE;
        p->lanes_per_row = nvec <= 4 ? 4 : (nvec <= 8 ? 8 : (nvec <= 16 ? 16 : (nvec <= 32 ? 32 : 64)));
        p->vectors_per_lane = static_cast<int>(ceil_div(nvec, p->lanes_per_row));
        // Several rows per 64-lane slot (N <= 256): 2 KiB of loads per wave in
        // 2-wave workgroups measured best (262144 x 128: 23.4 against 24.0 us
        // with 4 KiB in 4-wave workgroups; 262144 x 64: 12.6 us with 8-lane
        // rows, 13.5 with 16), and 4 KiB with 4-lane rows (262144 x 32: 6.4 us
        // with four slots, 7.1 with two, 11.0 with 16-lane rows); one row per
        // slot: 4 KiB, 4 waves.
        const bool multi_row = p->lanes_per_row < 64;
        p->block_threads = multi_row ? kWaveBlockThreadsMultiRow : kWaveBlockThreads;
        const int64_t budget = (multi_row && p->lanes_per_row > 4) ? kWaveBytesInFlightMultiRow : kWaveBytesInFlight;
        const int64_t per_slot = N * es * (64 / p->lanes_per_row);
        p->row_slots = 1;
        for (int s : kWaveSlots) {
            if (s * per_slot <= budget &&
                find_kernel(RMSNORM_VARIANT_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, s, false)) {
                p->row_slots = s;
                break;
            }
        }
        // Rows of exactly 64 vectors, 16384 rows or more: half-wave rows, 2 vectors per lane, 4
        // slots (8 rows and 8 KiB per wave, 32 rows per workgroup, 512 workgroups or more).
        // Measured on MI355X at 16384 x 512 bf16 with inputs cold in HBM, exact-width forms in
        // one process: 5.97-5.98 us against 6.13-6.21 us for 64-lane rows with 4 slots (4 KiB
        // per wave), where a copy of the same bytes with 8 KiB per wave and stores back to back
        // took 5.94-5.97 us.  With few rows the longer waves cost more than they save: 64 x 512
        // took 2.97 us in 2 workgroups against 2.37 us in 4 with 64-lane rows.
        if (N == 64 * elems_per_vector(dtype) && M >= kHalfWaveRowsMinRows &&
            find_kernel(RMSNORM_VARIANT_WAVE, dtype, 32, 2, 4, false)) {
            p->lanes_per_row = 32;
            p->vectors_per_lane = 2;
            p->row_slots = 4;
        }
    } else {
        p->variant = RMSNORM_VARIANT_BLOCK;
        p->row_slots = 1;
        // 256 threads up to 4 vectors each, 512 up to 3, then 1024-thread
        // workgroups (4096 x 10240 bf16: 29.7 us with 512 x 3 against 30.2 us
        // with 256 x 5; 4096 x 12288 bf16: 35.3 us with 512 x 3, where six
        // 16-bit vectors per thread have no compiled kernel)
        p->block_threads = nvec <= 256 * 4 ? 256 : (nvec <= 512 * 3 ? 512 : 1024);
        p->vectors_per_lane = static_cast<int>(ceil_div(nvec, p->block_threads));
        // contiguous 16-bit rows of exactly 16384 elements, one trip: the exact-width block
        // form, 256 threads x 8 vectors (4096 x 16384 fp16: 44.7 us against 47.4 us with
        // 1024 x 2)
        if (acc.contiguous && N == 256 * 8 * elems_per_vector(dtype) && M <= grid_limit(256) &&
            rmsnorm_impl::exact_block_kernel(dtype, 8, 256)) {
            p->block_threads = 256;
            p->vectors_per_lane = 8;
        }
        // rows wider than the compiled instances hold (or a ragged width the
        // widest ones have no tail path for) take the wide kernel
        const KernelEntry* k = find_kernel(RMSNORM_VARIANT_BLOCK, dtype, 0, p->vectors_per_lane, 1, false);
        if (!k) k = rmsnorm_impl::exact_block_kernel(dtype, p->vectors_per_lane, p->block_threads);
        if (!k || (!k->tails && N % elems_per_vector(dtype) != 0)) {
            p->variant = RMSNORM_VARIANT_WIDE;
            p->block_threads = 1024;
            p->vectors_per_lane = kWideVectors;
        }
    }
    int64_t rows_per_trip = 1;
    if (p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_SHIFTED_WAVE)
        rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
    const int64_t need = M > 0 ? ceil_div(M, rows_per_trip) : 1;
    p->grid = std::min(need, grid_limit(p->block_threads));
    p->xcd_group = 1;
    p->max_blocks_per_cu = 0;
    if (p->variant == RMSNORM_VARIANT_BLOCK || p->variant == RMSNORM_VARIANT_SHIFTED ||
        p->variant == RMSNORM_VARIANT_WIDE) {
        // about 128 KiB (1 MiB beyond the Infinity Cache) of consecutive rows per XCD: the
        // nearest power of two rows, at least 8 (on 8192 x 3000 bf16, groups of 16 rows took
        // 18.06 us and of 32 rows 18.30, where 12, 20 or 24 rows took 20.7-21.2 us)
        const int64_t row_bytes = N * es;
        const int64_t target = M * row_bytes >= kInfinityCacheBytes ? kXcdGroupBytesLarge : kXcdGroupBytes;
        int g = 8;
        while (g < kMaxXcdGroup && row_bytes * g * 3 < target * 2) g *= 2;
        p->xcd_group = g;
        // about 64 KiB of rows in flight per compute unit, at least 3 workgroups
        int64_t cap = kBytesInFlightPerCu / row_bytes;
        if (cap < kMinBlocksPerCu) cap = kMinBlocksPerCu;
        if (cap < kMaxThreadsPerCu / p->block_threads) p->max_blocks_per_cu = static_cast<int>(cap);
        // the exact-width block forms (launch_instance): at most 3 workgroups per CU
        // (4096 x 16384 fp16, 256 x 8: 45.9 us against 46.2 with 4, 46.7 with 5, 47.0
        // uncapped, 47.8 with 2; 32768 x 8192 bf16, 256 x 4: 166.6-168.7 us over eight
        // placements of y, against 170.0 with 4 and 175.5 with 2)
        if (p->variant == RMSNORM_VARIANT_BLOCK && acc.contiguous && p->block_threads == 256 &&
            N == static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * elems_per_vector(dtype) &&
            p->grid == M && rmsnorm_impl::exact_block_kernel(dtype, p->vectors_per_lane, p->block_threads))
            p->max_blocks_per_cu = 3;
    }
    p->prefetch = 0;
    if (p->variant == RMSNORM_VARIANT_SHIFTED) {
        // weights fetched with the row and passed between lanes up to 256
        // threads (8192 x 3001 bf16: 20.0 against 22.0 us), after the
        // reduction above (32768 x 8191 bf16: 194 against 210 us)
        p->prefetch = p->block_threads <= 256 ? 1 : 0;
    } else if (p->variant != RMSNORM_VARIANT_GENERIC && p->grid < need &&
        find_kernel(p->variant, dtype,
                    p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_SHIFTED_WAVE
                        ? p->lanes_per_row : 0,
                    p->vectors_per_lane, p->row_slots, true))
        p->prefetch = 1;
    return RMSNORM_OK;
}

// Workgroups of the plan's kernel the device holds at once.  cu_count > 0:
// that many units at the register-free bound of 2048 threads per unit, host
// only; otherwise the current device's unit count times the kernel's
// occupancy.  Either way no more than the plan's max_blocks_per_cu per unit.
int resident_grid(const rmsnorm_plan_t* p, const KernelEntry* k, int cu_count, int64_t* out) {
    int cu = cu_count, bpc = 0;
    if (cu > 0) {
        bpc = kMaxThreadsPerCu / p->block_threads;
    } else {
        int st = device_info(&cu);
        if (st != RMSNORM_OK) return st;
        st = occupancy(k->func, p->block_threads, &bpc);
        if (st != RMSNORM_OK) return st;
    }
    if (p->max_blocks_per_cu > 0 && bpc > p->max_blocks_per_cu) bpc = p->max_blocks_per_cu;
    *out = static_cast<int64_t>(cu) * bpc;
    return RMSNORM_OK;
}

// Launch one plan over every batch of the layout: grid (plan.grid, batches),
// at most kMaxGridY batches per launch, each launch's pointers moved to its
// first batch.  M here is the rows of one batch.
constexpr int64_t kMaxGridY = 65535;

int launch(const KernelEntry* k, const rmsnorm_plan_t* p, const void* x, const void* w, void* y,
           float* rstd, int64_t M, int64_t N, float eps, float offset, int dtype, const Layout& L,
           int64_t batches, int lds_per_cu, void* stream) {
    k = launch_instance(k, p, M, N, dtype, L, batches);
    // occupancy cap: (cap + 1) workgroups of this much LDS do not fit a unit
    size_t dyn_lds = 0;
    if (p->max_blocks_per_cu > 0 && lds_per_cu > 0)
        dyn_lds = static_cast<size_t>(lds_per_cu / (p->max_blocks_per_cu + 1) + 1);
    const int64_t es = elem_size(dtype);
    for (int64_t b0 = 0; b0 < batches; b0 += kMaxGridY) {
        const int64_t nb = std::min(batches - b0, kMaxGridY);
        KernelArgs a;
        a.x = static_cast<const char*>(x) + b0 * L.x_bs * es;
        a.w = w;
        a.y = static_cast<char*>(y) + b0 * L.y_bs * es;
        a.rstd = rstd != nullptr ? rstd + b0 * M : nullptr;
        a.M = M;
        a.N = N;
        a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
        a.eps = eps;
        a.offset = offset;
        a.xcd_group = p->xcd_group;
        a.grid = p->grid;
        a.threads = p->block_threads;
        a.x_rs = L.x_rs;
        a.y_rs = L.y_rs;
        a.x_bs = L.x_bs;
        a.y_bs = L.y_bs;
        // the vector kernels' row strides in 16-byte vectors (checked to fit 31 bits by vector_ok)
        const int64_t epv = elems_per_vector(dtype);
        a.x_rsv = L.rows <= 1 ? 0 : static_cast<int32_t>(L.x_rs / epv);   // unused with one row per batch
        a.y_rsv = L.rows <= 1 ? 0 : static_cast<int32_t>(L.y_rs / epv);
        void* args[] = {&a};
        hipError_t e = hipLaunchKernel(k->func, dim3(static_cast<unsigned>(p->grid), static_cast<unsigned>(nb)),
                                       dim3(static_cast<unsigned>(p->block_threads)), args, dyn_lds,
                                       static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(RMSNORM_ERR_HIP, std::string("hipLaunchKernel(") + k->name + "): " + hipGetErrorString(e));
    }
    return RMSNORM_OK;
}


// ---------------------------------------------------------------------------
// Backward: argument checks, planning, launch.
// ---------------------------------------------------------------------------
constexpr int64_t kBwdMaxVectors = 1024LL * 2;      // widest row the block and shifted kernels hold, in vectors
constexpr int kBwdWideThreads = 1024;
// vectors per thread the wide backward kernel is compiled for (dw of more
// would not fit 128 VGPRs without spilling)
int bwd_wide_max_vectors(int dtype) { return dtype == RMSNORM_FP32 ? 6 : 4; }
constexpr int kBwdWaveThreads = 1024;                // 16 waves share one LDS reduction of dw
constexpr int64_t kBwdMaxLds = 64 * 1024;
constexpr int64_t kBwdPlanCus = 256;                 // compute units the backward plan assumes
constexpr int64_t kBwdPlanWaves = kBwdPlanCus * 16;  // row-pass waves aimed for: 16 per unit
constexpr int64_t kBwdShortShiftedWaves = kBwdPlanWaves * 4;  // the same for several shifted rows per wave
constexpr int64_t kBwdPartialsGeneric = 1024;        // row-pass grid cap of the generic family
constexpr int kBwdWaveSlots[] = {4, 2, 1};
// Unaligned rows shorter than this take the generic kernel.
constexpr int64_t kBwdMinShiftedN = 16;
constexpr int64_t kBwdMaxShiftedWaveChunks = 128;  // two chunks per lane of a 64-lane segment

const KernelEntry* find_bwd_kernel(int variant, int dtype, int lanes, int vpl, int slots, bool prefetch) {
    int n = 0;
    const KernelEntry* t = rmsnorm_impl::bwd_kernel_table(&n);
    for (int i = 0; i < n; ++i) {
        const KernelEntry& k = t[i];
        if (k.variant != variant || k.dtype != dtype || k.prefetch != prefetch) continue;
        if ((variant == RMSNORM_VARIANT_WAVE || variant == RMSNORM_VARIANT_SHIFTED_WAVE) &&
            (k.lanes_per_row != lanes || k.vectors_per_lane != vpl || k.row_slots != slots))
            continue;
        if ((variant == RMSNORM_VARIANT_BLOCK || variant == RMSNORM_VARIANT_SHIFTED || variant == RMSNORM_VARIANT_WIDE) &&
            k.vectors_per_lane != vpl)
            continue;
        if (variant == RMSNORM_VARIANT_BLOCK && k.row_slots != slots) continue;
        return &k;
    }
    return nullptr;
}

int64_t bwd_wave_lds(const rmsnorm_plan_t* p, int64_t N) {
    return static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * N * 4;
}

// Dynamic LDS of the block row pass: with R rows per workgroup, the dw
// partials of slots 1 .. R - 1 (VPT vectors of vec_elems floats per thread).
int64_t bwd_block_lds(const rmsnorm_plan_t* p, int dtype) {
    if (p->row_slots <= 1) return 0;
    return static_cast<int64_t>(p->block_threads / p->row_slots) * (p->row_slots - 1) * p->vectors_per_lane *
           elems_per_vector(dtype) * 4;
}

// Dynamic LDS of the shifted row pass: with three chunks per thread, each
// thread's dw column vectors (vectors_per_lane of vec_elems floats); none
// with fewer, which keep dw in registers.
int64_t bwd_shifted_lds(const rmsnorm_plan_t* p, int dtype) {
    if (p->vectors_per_lane < 3) return 0;
    return static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * elems_per_vector(dtype) * 4;
}

// Row layout of x, dy and dx for the backward, normalised as the forward's:
// `rows` rows per batch, strides in elements.
struct BwdLayout {
    int64_t rows;
    int64_t x_rs, x_bs, dy_rs, dy_bs, dx_rs, dx_bs;
    int64_t batches(int64_t M) const { return rows > 0 ? M / rows : 0; }
    int64_t span(int64_t M, int64_t N, int64_t rs, int64_t bs) const {
        if (M == 0) return 0;
        return (batches(M) - 1) * bs + (rows - 1) * rs + N;
    }
    int64_t x_span(int64_t M, int64_t N) const { return span(M, N, x_rs, x_bs); }
    int64_t dy_span(int64_t M, int64_t N) const { return span(M, N, dy_rs, dy_bs); }
    int64_t dx_span(int64_t M, int64_t N) const { return span(M, N, dx_rs, dx_bs); }
};

BwdLayout contiguous_bwd_layout(int64_t M, int64_t N) {
    return BwdLayout{M > 0 ? M : 1, N, M * N, N, M * N, N, M * N};
}

// Checks and normalises a backward layout.  dx's rows must not overlap one
// another (batch-major or row-major interleaved, as the forward's y); x's
// and dy's rows may (they are only read).  Several batches need M < 2^31
// (the kernels split a row index with one 32-bit division).
int normalise_bwd_layout(const rmsnorm_bwd_layout_t* L, int64_t M, int64_t N, BwdLayout* out) {
    if (!L) {
        *out = contiguous_bwd_layout(M, N);
        return RMSNORM_OK;
    }
    if (L->rows < 0) return fail(RMSNORM_ERR_SHAPE, "layout rows must be >= 0");
    const int64_t strides[6] = {L->x_row_stride, L->x_batch_stride, L->dy_row_stride,
                                L->dy_batch_stride, L->dx_row_stride, L->dx_batch_stride};
    for (int64_t v : strides)
        if (v < 0) return fail(RMSNORM_ERR_SHAPE, "layout strides must be >= 0");
    BwdLayout o;
    o.rows = (L->rows == 0 || L->rows >= M) ? (M > 0 ? M : 1) : L->rows;
    if (M > 0 && M % o.rows != 0) return fail(RMSNORM_ERR_SHAPE, "M must be a multiple of layout rows");
    const int64_t B = M > 0 ? M / o.rows : 1;
    o.x_rs = L->x_row_stride;
    o.dy_rs = L->dy_row_stride;
    o.dx_rs = L->dx_row_stride;
    o.x_bs = B > 1 ? L->x_batch_stride : 0;
    o.dy_bs = B > 1 ? L->dy_batch_stride : 0;
    o.dx_bs = B > 1 ? L->dx_batch_stride : 0;
    const int64_t lim = INT64_MAX / 4;
    const int64_t r1 = o.rows > 1 ? o.rows : 1;
    if (o.x_rs > lim / r1 || o.dy_rs > lim / r1 || o.dx_rs > lim / r1 || o.x_bs > lim / B || o.dy_bs > lim / B ||
        o.dx_bs > lim / B)
        return fail(RMSNORM_ERR_SHAPE, "layout spans overflow int64");
    if (o.rows > 1 && o.dx_rs < N) return fail(RMSNORM_ERR_SHAPE, "dx rows overlap: dx_row_stride < N");
    if (B > 1) {
        const bool batch_major = o.dx_bs >= (o.rows - 1) * o.dx_rs + N;
        const bool interleaved = o.dx_rs >= (B - 1) * o.dx_bs + N && o.dx_bs >= N;
        if (!batch_major && !interleaved) return fail(RMSNORM_ERR_SHAPE, "dx rows overlap across batches");
    }
    if (o.x_span(M, N) > lim || o.dy_span(M, N) > lim || o.dx_span(M, N) > lim)
        return fail(RMSNORM_ERR_SHAPE, "layout spans overflow int64");
    if (B > 1 && o.x_bs == o.rows * o.x_rs && o.dy_bs == o.rows * o.dy_rs && o.dx_bs == o.rows * o.dx_rs) {
        o.rows = M;     // batches that continue each other's row stride are one batch
        o.x_bs = o.dy_bs = o.dx_bs = 0;
    }
    if (o.rows < M && M >= (int64_t{1} << 31))
        return fail(RMSNORM_ERR_SHAPE, "a backward layout with several batches takes M < 2^31 rows");
    *out = o;
    return RMSNORM_OK;
}

int check_bwd_args(const void* x, const void* w, const void* dy, const float* rstd, const void* dx,
                   const float* dw, int64_t M, int64_t N, float offset, int dtype, const BwdLayout& L) {
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    if (!dw) return fail(RMSNORM_ERR_NULL, "dw must be non-NULL");
    if (M > 0 && (!x || !w || !dy || !rstd || !dx))
        return fail(RMSNORM_ERR_NULL, "x, w, dy, rstd and dx must be non-NULL");
    if (!std::isfinite(offset)) return fail(RMSNORM_ERR_SCALAR, "offset must be finite");
    const int64_t es = elem_size(dtype);
    const int64_t xb = L.x_span(M, N) * es, yb = L.dy_span(M, N) * es, ob = L.dx_span(M, N) * es;
    const int64_t wb = N * es, rb = M * 4, db = N * 4;
    if (M > 0) {
        const bool same_layout = L.dx_rs == L.dy_rs && L.dx_bs == L.dy_bs;
        if (ranges_overlap(dx, ob, x, xb)) return fail(RMSNORM_ERR_OVERLAP, "dx overlaps x");
        if (dx == dy ? !same_layout : ranges_overlap(dx, ob, dy, yb))
            return fail(RMSNORM_ERR_OVERLAP, "dx overlaps dy (in place needs dx == dy with the same layout)");
        if (ranges_overlap(dx, ob, w, wb) || ranges_overlap(dx, ob, rstd, rb) || ranges_overlap(dx, ob, dw, db))
            return fail(RMSNORM_ERR_OVERLAP, "dx overlaps w, rstd or dw");
        if (ranges_overlap(dw, db, x, xb) || ranges_overlap(dw, db, dy, yb) || ranges_overlap(dw, db, w, wb) ||
            ranges_overlap(dw, db, rstd, rb))
            return fail(RMSNORM_ERR_OVERLAP, "dw overlaps an input");
    }
    return RMSNORM_OK;
}

// The 16-byte backward kernels: N a multiple of the vector, 16-byte aligned
// x, w, dy and dx, strides that keep every row aligned, rows they hold (the
// wide kernel's widest).
bool bwd_vector_ok(const void* x, const void* w, const void* dy, const void* dx, int dtype, const BwdLayout& L,
                   int64_t M, int64_t N) {
    const int64_t es = elem_size(dtype);
    const int64_t epv = elems_per_vector(dtype);
    const bool rows_ok = (L.x_rs * es) % 16 == 0 && (L.dy_rs * es) % 16 == 0 && (L.dx_rs * es) % 16 == 0;
    const bool batches_ok = L.batches(M) <= 1 ||
                            ((L.x_bs * es) % 16 == 0 && (L.dy_bs * es) % 16 == 0 && (L.dx_bs * es) % 16 == 0);
    return N % epv == 0 && N / epv <= int64_t{kBwdWideThreads} * bwd_wide_max_vectors(dtype) && aligned16(x) &&
           aligned16(w) && aligned16(dy) && aligned16(dx) && rows_ok && batches_ok;
}

// The shifted backward kernel: x, dy and dx the same distance past a 16-byte
// boundary on every row (equally aligned bases, strides that differ by whole
// 16-byte vectors), w 16-byte aligned, rows of at most 2048 chunks, and not
// the 16-byte kernels' case.
bool bwd_shifted_ok(const void* x, const void* w, const void* dy, const void* dx, int dtype, const BwdLayout& L,
                    int64_t M, int64_t N, bool vec) {
    if (vec) return false;
    const int64_t es = elem_size(dtype);
    const int64_t epv = elems_per_vector(dtype);
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(dy),
                    oa = reinterpret_cast<uintptr_t>(dx);
    const uintptr_t ue = static_cast<uintptr_t>(es);
    if (xa % ue != 0 || ya % ue != 0 || oa % ue != 0 || xa % 16 != ya % 16 || xa % 16 != oa % 16) return false;
    auto same_phase = [&](int64_t s1, int64_t s2) { return ((s1 - s2) * es) % 16 == 0; };
    const bool rows_ok = L.rows <= 1 || (same_phase(L.x_rs, L.dy_rs) && same_phase(L.x_rs, L.dx_rs));
    const bool batches_ok = L.batches(M) <= 1 || (same_phase(L.x_bs, L.dy_bs) && same_phase(L.x_bs, L.dx_bs));
    return aligned16(w) && rows_ok && batches_ok && ceil_div(N + epv - 1, epv) <= kBwdMaxVectors;
}

int check_workspace(const void* ws, int64_t ws_bytes, int64_t need, const void* x, const void* w,
                    const void* dy, const float* rstd, const void* dx, const float* dw, int64_t M, int64_t N,
                    int dtype, const BwdLayout& L) {
    if (need == 0) return RMSNORM_OK;
    if (!ws) return fail(RMSNORM_ERR_NULL, "workspace must be non-NULL");
    if (ws_bytes < need)
        return fail(RMSNORM_ERR_SHAPE, "workspace holds " + std::to_string(ws_bytes) + " bytes, plan needs " +
                                           std::to_string(need));
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return fail(RMSNORM_ERR_PLAN, "workspace must be 16-byte aligned");
    const int64_t es = elem_size(dtype);
    if (ranges_overlap(ws, need, x, L.x_span(M, N) * es) || ranges_overlap(ws, need, dy, L.dy_span(M, N) * es) ||
        ranges_overlap(ws, need, dx, L.dx_span(M, N) * es) ||
        ranges_overlap(ws, need, w, N * es) || ranges_overlap(ws, need, rstd, M * 4) ||
        ranges_overlap(ws, need, dw, N * 4))
        return fail(RMSNORM_ERR_OVERLAP, "workspace overlaps an argument");
    return RMSNORM_OK;
}

const char* const kBwdVecNeeds =
    "16-byte kernels need N a multiple of vec_elems, at most 4096 vectors (6144 with fp32), 16-byte aligned x, "
    "w, dy and dx, and strides that keep rows aligned";

int finish_bwd_plan(rmsnorm_plan_t* p, int64_t M, int64_t N, int dtype, bool vec, bool shifted,
                    const KernelEntry** kernel) {
    if (p->block_threads < 64 || p->block_threads > 1024 || p->block_threads % 64 != 0)
        return fail(RMSNORM_ERR_PLAN, "block_threads must be a multiple of 64 in [64, 1024]");
    if (check_grid(p) != RMSNORM_OK) return RMSNORM_ERR_PLAN;
    if (p->prefetch != 0 && p->prefetch != 1) return fail(RMSNORM_ERR_PLAN, "prefetch must be 0 or 1");
    if (p->xcd_group != 1 || p->max_blocks_per_cu != 0)
        return fail(RMSNORM_ERR_PLAN, "backward plans take xcd_group 1 and max_blocks_per_cu 0");
    const bool pf = p->prefetch != 0;
    const KernelEntry* k = nullptr;
    if (p->variant == RMSNORM_VARIANT_GENERIC) {
        p->vec_elems = 1;
        p->lanes_per_row = p->block_threads;
        p->vectors_per_lane = 0;
        p->row_slots = 1;
        p->rows_per_trip = 1;
        k = pf ? nullptr : find_bwd_kernel(RMSNORM_VARIANT_GENERIC, dtype, 0, 0, 1, false);
    } else if (p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_BLOCK) {
        const int epv = elems_per_vector(dtype);
        if (!vec)
            return fail(RMSNORM_ERR_PLAN, kBwdVecNeeds);
        p->vec_elems = epv;
        if (p->variant == RMSNORM_VARIANT_WAVE) {
            k = find_bwd_kernel(RMSNORM_VARIANT_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, p->row_slots, pf);
            if (k) {
                if (static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv < N)
                    return fail(RMSNORM_ERR_PLAN, "wave plan does not cover N");
                if (bwd_wave_lds(p, N) > kBwdMaxLds)
                    return fail(RMSNORM_ERR_PLAN, "wave plan needs more than 64 KiB of LDS for dw partials");
                p->rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
            }
        } else {
            // row_slots rows per workgroup (0 reads as 1), block_threads / row_slots threads each
            if (p->row_slots <= 1) p->row_slots = 1;
            if (p->row_slots != 2 && p->row_slots != 4 && p->row_slots != 1)
                return fail(RMSNORM_ERR_PLAN, "backward block plans take 1, 2 or 4 rows per workgroup");
            if (p->block_threads % (64 * p->row_slots) != 0)
                return fail(RMSNORM_ERR_PLAN, "block_threads must give each of the row_slots rows whole waves");
            p->lanes_per_row = p->block_threads / p->row_slots;
            k = find_bwd_kernel(RMSNORM_VARIANT_BLOCK, dtype, 0, p->vectors_per_lane, p->row_slots, pf);
            if (k) {
                if (static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv < N)
                    return fail(RMSNORM_ERR_PLAN, "block plan does not cover N");
                if (bwd_block_lds(p, dtype) > kBwdMaxLds)
                    return fail(RMSNORM_ERR_PLAN, "block plan needs more than 64 KiB of LDS for its slots' dw");
                p->rows_per_trip = p->row_slots;
            }
        }
    } else if (p->variant == RMSNORM_VARIANT_WIDE) {
        if (!vec) return fail(RMSNORM_ERR_PLAN, kBwdVecNeeds);
        p->vec_elems = elems_per_vector(dtype);
        p->row_slots = 1;
        p->lanes_per_row = p->block_threads;
        p->rows_per_trip = 1;
        k = find_bwd_kernel(RMSNORM_VARIANT_WIDE, dtype, 0, p->vectors_per_lane, 1, pf);
        if (k && static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * p->vec_elems < N)
            return fail(RMSNORM_ERR_PLAN, "wide plan does not cover N");
    } else if (p->variant == RMSNORM_VARIANT_SHIFTED) {
        if (!shifted)
            return fail(RMSNORM_ERR_PLAN, "the shifted backward kernel needs x, dy and dx equally far past a 16-byte "
                                          "boundary on every row, 16-byte aligned w, rows that are not 16-byte "
                                          "aligned, and at most 2048 chunks");
        const int epv = elems_per_vector(dtype);
        p->vec_elems = epv;
        p->row_slots = 1;
        p->lanes_per_row = p->block_threads;
        p->rows_per_trip = 1;
        k = find_bwd_kernel(RMSNORM_VARIANT_SHIFTED, dtype, 0, p->vectors_per_lane, 1, pf);
        if (k && static_cast<int64_t>(p->block_threads) * p->vectors_per_lane * epv < N + epv - 1)
            return fail(RMSNORM_ERR_PLAN, "shifted plan does not cover N");
        if (k && bwd_shifted_lds(p, dtype) > kBwdMaxLds)
            return fail(RMSNORM_ERR_PLAN, "shifted plan needs more than 64 KiB of LDS for dw");
    } else if (p->variant == RMSNORM_VARIANT_SHIFTED_WAVE) {
        if (!shifted)
            return fail(RMSNORM_ERR_PLAN, "the shifted backward kernels need x, dy and dx equally far past a 16-byte "
                                          "boundary on every row, 16-byte aligned w, rows that are not 16-byte "
                                          "aligned, and at most 2048 chunks");
        const int epv = elems_per_vector(dtype);
        p->vec_elems = epv;
        if (p->lanes_per_row != 8 && p->lanes_per_row != 16 && p->lanes_per_row != 32 && p->lanes_per_row != 64)
            return fail(RMSNORM_ERR_PLAN, "shifted wave plans take 8, 16, 32 or 64 lanes per row");
        k = find_bwd_kernel(RMSNORM_VARIANT_SHIFTED_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane,
                            p->row_slots, pf);
        if (k) {
            if (static_cast<int64_t>(p->lanes_per_row) * p->vectors_per_lane * epv < N + epv - 1)
                return fail(RMSNORM_ERR_PLAN, "shifted wave plan does not cover N");
            if (bwd_wave_lds(p, N) > kBwdMaxLds)
                return fail(RMSNORM_ERR_PLAN, "wave plan needs more than 64 KiB of LDS for dw partials");
            p->rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
        }
    } else {
        return fail(RMSNORM_ERR_PLAN, "unknown variant");
    }
    if (!k) return fail(RMSNORM_ERR_PLAN, "no compiled backward kernel for this plan");
    p->trips = M > 0 ? ceil_div(ceil_div(M, p->rows_per_trip), p->grid) : 0;
    if (kernel) *kernel = k;
    return RMSNORM_OK;
}

// Backward plan: the forward's families and widths and a persistent row
// pass (rows off a 16-byte boundary: the shifted family, at most 2 chunks per
// thread).  Its grid G, the number of dw partial rows, is the smallest of: the
// rows' trips (one trip per workgroup), enough workgroups for 16 waves on
// each of 256 compute units, and 3M/32, which keeps the workspace's write
// and read within 1/8 of the row pass's 6MN bytes.  The next trip is loaded
// ahead when a workgroup makes more than one and the grid leaves at most one
// workgroup per unit: its barriers then stall the whole unit, which the early
// loads cover; with two or more workgroups per unit they cover each other,
// and the extra registers of the prefetching form cost more than they hide.
int choose_bwd_plan(int64_t M, int64_t N, bool vec_ok, bool shifted_ok, int dtype, rmsnorm_plan_t* p) {
    std::memset(p, 0, sizeof(*p));
    p->xcd_group = 1;
    const int64_t epv = elems_per_vector(dtype);
    const int64_t shifted_chunks = ceil_div(N + epv - 1, epv);
    if (!vec_ok && shifted_ok && N >= kBwdMinShiftedN && shifted_chunks <= kBwdMaxShiftedWaveChunks) {
        // a row per segment of the fewest lanes (8, 16, 32, 64) that hold its
        // chunks, one chunk per lane up to 64 chunks, then two per lane of a
        // 64-lane wave.  One slot, except a row of one chunk per lane in a
        // 64-lane wave: two (262144 x 257 bf16: 118 us, against 138 us with
        // one; 65536 x 300 bf16: 35.3 against 38.9 us).  Several rows per
        // wave: one slot, against four before (262144 x 36 bf16: 36.6 against
        // 39.4 us; 262144 x 130 fp16: 67.4 against 76.3 us), with the larger
        // grid below.  Two chunks per lane: 16384 x 513 bf16 19.0 us, against
        // 19.8 with two slots and 33.5 with a 128-thread workgroup per row.
        // No prefetching form is taken: with the rows of a trip loaded
        // together it gained nothing.
        p->variant = RMSNORM_VARIANT_SHIFTED_WAVE;
        p->block_threads = kBwdWaveThreads;
        p->lanes_per_row = shifted_chunks <= 8 ? 8 : (shifted_chunks <= 16 ? 16 : (shifted_chunks <= 32 ? 32 : 64));
        p->vectors_per_lane = shifted_chunks <= 64 ? 1 : 2;
        p->row_slots = (p->lanes_per_row == 64 && p->vectors_per_lane == 1) ? 2 : 1;
    } else if (!vec_ok && shifted_ok && N >= kBwdMinShiftedN) {
        // one row per workgroup of the fewest threads (up to 1024) that hold
        // the row with at most 2 chunks per thread (8192 x 3001 bf16: 47.5 us
        // with 256 x 2, 46.6 with 512 x 1; 16384 x 1002 fp32: 44.0 us with
        // 128 x 2, 45.6 with 256 x 1).  Rows of 1025 to 1536 chunks would
        // leave up to half of 1024 x 2 idle: with rows enough for two
        // 512-thread workgroups per CU, 512 x 3 (32768 x 8191 bf16: 366 us
        // against 456 us; 4096 x 4097 fp32, 384 workgroups: 52.6 against 47.8)
        const int64_t nchunks = ceil_div(N + epv - 1, epv);
        int64_t per_thread = 2;
        if (nchunks > 1024 && nchunks <= 1536 && 3 * M / 32 >= 512 &&
            find_bwd_kernel(RMSNORM_VARIANT_SHIFTED, dtype, 0, 3, 1, false))
            per_thread = 3;
        p->variant = RMSNORM_VARIANT_SHIFTED;
        p->row_slots = 1;
        p->block_threads = 64;
        while (p->block_threads < 1024 && nchunks > per_thread * p->block_threads) p->block_threads *= 2;
        p->vectors_per_lane = static_cast<int>(ceil_div(nchunks, p->block_threads));
    } else if (!vec_ok) {
        p->variant = RMSNORM_VARIANT_GENERIC;
        p->block_threads = N >= 1024 ? 256 : (N >= 256 ? 128 : 64);
        p->row_slots = 1;
    } else if (N / epv <= 128) {
        const int64_t nvec = N / epv;
        p->variant = RMSNORM_VARIANT_WAVE;
        p->block_threads = kBwdWaveThreads;
        // the fewest lanes (8, 16, 32, 64) that hold the row: 262144 x 40 bf16
        // 16.7 us with 8-lane rows, 19.7 with 16; 262144 x 32 bf16 14.8 us,
        // against 16.3 with 4-lane rows and 19.1 with 16
        p->lanes_per_row = nvec <= 8 ? 8 : (nvec <= 16 ? 16 : (nvec <= 32 ? 32 : 64));
        p->vectors_per_lane = static_cast<int>(ceil_div(nvec, p->lanes_per_row));
        const int64_t per_slot = N * elem_size(dtype) * (64 / p->lanes_per_row);
        p->row_slots = 1;
        // A row per 64-lane wave: one row per trip, the next trip's loads
        // issued ahead (16384 x 512: 13.5 us against 15.0 us with four rows
        // per wave loaded up front in one trip).  Shorter rows: several
        // slots (flat within 3% on 262144 x 128).
        for (int sl : kBwdWaveSlots) {
            if (p->lanes_per_row < 64 && sl * per_slot <= kWaveBytesInFlight &&
                find_bwd_kernel(RMSNORM_VARIANT_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, sl, false)) {
                p->row_slots = sl;
                break;
            }
        }
    } else if (N / epv <= kBwdMaxVectors) {
        const int64_t nvec = N / epv;
        p->variant = RMSNORM_VARIANT_BLOCK;
        p->row_slots = 1;
        p->block_threads = nvec <= 512 ? 256 : (nvec <= 1024 ? 512 : 1024);
        p->vectors_per_lane = static_cast<int>(ceil_div(nvec, p->block_threads));
        // Rows of 256 threads go four to a 1024-thread workgroup: one workgroup
        // per CU with the next trip's rows loaded ahead, and a quarter of the
        // partial rows (8192 x 3000 bf16: 31.1 us against 34.7 us with 768
        // single-row workgroups; 16384 x 2048: 38.5 against 40.0).  Rows of
        // 512 threads stay one to a workgroup (32768 x 8192: 269-280 us two
        // to a workgroup against 265 us).
        if (p->block_threads == 256 && find_bwd_kernel(RMSNORM_VARIANT_BLOCK, dtype, 0, p->vectors_per_lane, 4, true)) {
            p->row_slots = 4;
            p->block_threads = 1024;
        }
    } else {
        // rows wider than x and dy can stay in registers: two passes over the row
        p->variant = RMSNORM_VARIANT_WIDE;
        p->row_slots = 1;
        p->block_threads = kBwdWideThreads;
        p->vectors_per_lane = static_cast<int>(ceil_div(N / epv, kBwdWideThreads));
    }
    int64_t rows_per_trip = 1;
    if (p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_SHIFTED_WAVE)
        rows_per_trip = static_cast<int64_t>(p->block_threads / 64) * (64 / p->lanes_per_row) * p->row_slots;
    if (p->variant == RMSNORM_VARIANT_BLOCK) rows_per_trip = p->row_slots;
    const int64_t need = M > 0 ? ceil_div(M, rows_per_trip) : 1;
    int64_t cap = kBwdPartialsGeneric;
    if (p->variant != RMSNORM_VARIANT_GENERIC) {
        // several short rows per wave off a 16-byte boundary: each row's
        // shifts are lane arithmetic, which more waves in flight hide, and
        // the partial rows are short (at most 249 16-bit elements).  Half as
        // many with 8-lane rows, which hold twice the rows per wave
        // (262144 x 36 bf16: 25.4 us at G = 512, 26.6 at 1024).
        const bool short_shifted = p->variant == RMSNORM_VARIANT_SHIFTED_WAVE && p->lanes_per_row < 64;
        int64_t waves = short_shifted ? kBwdShortShiftedWaves : kBwdPlanWaves;
        if (short_shifted && p->lanes_per_row == 8) waves /= 2;
        cap = waves / (p->block_threads / 64);
        const int64_t traffic_cap = std::max<int64_t>(3 * M / 32, 1);
        cap = std::min(cap, traffic_cap);
    }
    p->grid = std::min(need, cap);
    // past one workgroup per CU, whole CUs' worth: a grid of 384 leaves half
    // the CUs with one workgroup and half with two (4096 x 4096 fp32: 41.5 us
    // at G = 384, 39.0 at 256 with the next row loaded ahead)
    if (p->grid > kBwdPlanCus && p->grid < need) p->grid -= p->grid % kBwdPlanCus;
    const bool ahead = need > p->grid && p->grid <= kBwdPlanCus;
    if (ahead && p->variant == RMSNORM_VARIANT_WAVE &&
        find_bwd_kernel(RMSNORM_VARIANT_WAVE, dtype, p->lanes_per_row, p->vectors_per_lane, p->row_slots, true))
        p->prefetch = 1;
    if (ahead && (p->variant == RMSNORM_VARIANT_BLOCK || p->variant == RMSNORM_VARIANT_SHIFTED) &&
        find_bwd_kernel(p->variant, dtype, 0, p->vectors_per_lane, p->variant == RMSNORM_VARIANT_BLOCK ? p->row_slots : 1,
                        true))
        p->prefetch = 1;
    return RMSNORM_OK;
}

int launch_bwd(const KernelEntry* k, const rmsnorm_plan_t* p, const void* x, const void* w, const void* dy,
               const float* rstd, void* dx, float* dw, int64_t M, int64_t N, float offset, const BwdLayout& L,
               void* workspace, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t G = 0;
    if (M > 0) {
        BwdArgs a;
        a.x = x;
        a.w = w;
        a.dy = dy;
        a.rstd = rstd;
        a.dx = dx;
        a.partials = static_cast<float*>(workspace);
        a.M = M;
        a.N = N;
        a.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
        a.offset = offset;
        a.grid = p->grid;
        a.threads = p->block_threads;
        a.rows = L.rows;
        a.x_rs = L.x_rs;
        a.dy_rs = L.dy_rs;
        a.dx_rs = L.dx_rs;
        a.x_bs = L.x_bs;
        a.dy_bs = L.dy_bs;
        a.dx_bs = L.dx_bs;
        void* args[] = {&a};
        const bool wave = p->variant == RMSNORM_VARIANT_WAVE || p->variant == RMSNORM_VARIANT_SHIFTED_WAVE;
        size_t lds = wave ? static_cast<size_t>(bwd_wave_lds(p, N)) : 0;
        if (p->variant == RMSNORM_VARIANT_SHIFTED) lds = static_cast<size_t>(bwd_shifted_lds(p, k->dtype));
        if (p->variant == RMSNORM_VARIANT_BLOCK) lds = static_cast<size_t>(bwd_block_lds(p, k->dtype));
        hipError_t e = hipLaunchKernel(k->func, dim3(static_cast<unsigned>(p->grid)),
                                       dim3(static_cast<unsigned>(p->block_threads)), args, lds, s);
        if (e != hipSuccess)
            return fail(RMSNORM_ERR_HIP, std::string("hipLaunchKernel(") + k->name + "): " + hipGetErrorString(e));
        G = p->grid;
    }
    const float* partials = static_cast<const float*>(workspace);
    int64_t Nn = N;
    int32_t vec4 = (N % 4 == 0 && aligned16(dw)) ? 1 : 0;
    void* rargs[] = {&partials, &dw, &G, &Nn, &vec4};
    const int64_t groups = vec4 ? N / 4 : N;        // column groups
    // 4 groups per workgroup up to 256 groups (more workgroups share the reads), 16 above
    const int cols = groups <= 256 ? 4 : 16;
    const int64_t blocks = std::min(ceil_div(groups, cols), grid_limit(cols * 64));   // more loop in the kernel
    // 64-way splits once there are enough partial rows to share
    const int split = G >= 128 ? 64 : 16;
    hipError_t e = hipLaunchKernel(rmsnorm_impl::dw_reduce_kernel(split, cols), dim3(static_cast<unsigned>(blocks)),
                                   dim3(static_cast<unsigned>(cols * split)),
                                   rargs, 0, s);
    if (e != hipSuccess) return fail(RMSNORM_ERR_HIP, std::string("hipLaunchKernel(rmsnorm_dw_reduce): ") + hipGetErrorString(e));
    return RMSNORM_OK;
}

// Every backward entry point: checks, plan (the caller's or the rule),
// workspace check, launch of the row pass and the column pass.
int bwd_common(const void* x, const void* w, const void* dy, const float* rstd, void* dx, float* dw, int64_t M,
               int64_t N, float offset, int dtype, const rmsnorm_bwd_layout_t* layout, const rmsnorm_plan_t* plan,
               void* ws, int64_t ws_bytes, void* stream) {
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    BwdLayout L;
    st = normalise_bwd_layout(layout, M, N, &L);
    if (st != RMSNORM_OK) return st;
    st = check_bwd_args(x, w, dy, rstd, dx, dw, M, N, offset, dtype, L);
    if (st != RMSNORM_OK) return st;
    const bool vec = bwd_vector_ok(x, w, dy, dx, dtype, L, M, N);
    const bool shifted = bwd_shifted_ok(x, w, dy, dx, dtype, L, M, N, vec);
    rmsnorm_plan_t p;
    if (plan) p = *plan;
    else choose_bwd_plan(M, N, vec, shifted, dtype, &p);
    const KernelEntry* k = nullptr;
    st = finish_bwd_plan(&p, M, N, dtype, vec, shifted, &k);
    if (st != RMSNORM_OK) return st;
    const int64_t need = M > 0 ? p.grid * N * 4 : 0;
    st = check_workspace(ws, ws_bytes, need, x, w, dy, rstd, dx, dw, M, N, dtype, L);
    if (st != RMSNORM_OK) return st;
    int cu = 0;
    st = device_info(&cu);
    if (st != RMSNORM_OK) return st;
    return launch_bwd(k, &p, x, w, dy, rstd, dx, dw, M, N, offset, L, ws, stream);
}

// Plan and workspace of a backward call, host only (no pointers needed
// beyond their alignment).
int bwd_plan_for(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* dy, const void* dx,
                 const rmsnorm_bwd_layout_t* layout, rmsnorm_plan_t* p, const KernelEntry** k) {
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    BwdLayout L;
    st = normalise_bwd_layout(layout, M, N, &L);
    if (st != RMSNORM_OK) return st;
    const bool vec = bwd_vector_ok(x, w, dy, dx, dtype, L, M, N);
    const bool shifted = bwd_shifted_ok(x, w, dy, dx, dtype, L, M, N, vec);
    choose_bwd_plan(M, N, vec, shifted, dtype, p);
    return finish_bwd_plan(p, M, N, dtype, vec, shifted, k);
}

// ---------------------------------------------------------------------------
// Tuned dispatch: plans measured for exact (M, N, dtype) shapes, registered by
// the caller (for instance from a tuning run), take precedence over the
// heuristic in rmsnorm_fwd and rmsnorm_plan_query.  A tuned plan that does not
// fit a call's pointers (alignment) falls back to the heuristic.
// ---------------------------------------------------------------------------
std::mutex g_tuned_mu;
std::map<std::tuple<int64_t, int64_t, int>, rmsnorm_plan_t> g_tuned;
std::atomic<int> g_tuned_count{0};

bool tuned_plan(int64_t M, int64_t N, int dtype, rmsnorm_plan_t* out) {
    if (g_tuned_count.load(std::memory_order_acquire) == 0) return false;
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    const auto it = g_tuned.find(std::make_tuple(M, N, dtype));
    if (it == g_tuned.end()) return false;
    *out = it->second;
    return true;
}

int select_plan(int64_t M, int64_t N, int dtype, Access acc, rmsnorm_plan_t* p, const KernelEntry** k) {
    rmsnorm_plan_t t;
    if (tuned_plan(M, N, dtype, &t) && finish_plan(&t, M, N, dtype, acc, k) == RMSNORM_OK) {
        *p = t;
        return RMSNORM_OK;
    }
    g_last_error.clear();
    int st = choose_plan(M, N, dtype, acc, p);
    if (st == RMSNORM_OK) st = finish_plan(p, M, N, dtype, acc, k);
    return st;
}

// Every forward entry point: checks, plan (the caller's, a tuned one, or the
// rule), launch.
int fwd_common(const void* x, const void* w, void* y, float* rstd, int64_t M, int64_t N, float eps,
               float offset, int dtype, const rmsnorm_layout_t* layout, const rmsnorm_plan_t* plan,
               bool plan_required, bool rstd_optional, void* stream) {
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    Layout L;
    st = normalise_layout(layout, M, N, &L);
    if (st != RMSNORM_OK) return st;
    st = check_args(x, w, y, rstd, M, N, eps, offset, dtype, L, rstd_optional);
    if (st != RMSNORM_OK) return st;
    if (plan_required && !plan) return fail(RMSNORM_ERR_NULL, "plan must be non-NULL");
    const Access acc = access_of(x, w, y, dtype, L, M, N);
    const int64_t Mb = M > 0 ? L.rows : 0;    // plans cover one batch
    rmsnorm_plan_t p;
    const KernelEntry* k = nullptr;
    if (plan) {
        p = *plan;
        st = finish_plan(&p, Mb, N, dtype, acc, &k);
        if (st != RMSNORM_OK || M == 0) return st;
    } else {
        if (M == 0) return RMSNORM_OK;
        st = select_plan(Mb, N, dtype, acc, &p, &k);
        if (st != RMSNORM_OK) return st;
    }
    int cu = 0, lds = 0;
    st = device_info(&cu, &lds);  // gfx950 check, unit count and LDS (cached per device)
    if (st != RMSNORM_OK) return st;
    return launch(k, &p, x, w, y, rstd, Mb, N, eps, offset, dtype, L, L.batches(M), lds, stream);
}

}  // namespace

extern "C" {

int rmsnorm_fwd(const void* x, const void* w, void* y, float* rstd, int64_t M, int64_t N, float eps,
                float offset, int dtype, void* stream) {
    g_last_error.clear();
    return fwd_common(x, w, y, rstd, M, N, eps, offset, dtype, nullptr, nullptr, false, false, stream);
}

int rmsnorm_fwd_with_plan(const void* x, const void* w, void* y, float* rstd, int64_t M, int64_t N,
                          float eps, float offset, int dtype, const rmsnorm_plan_t* plan, void* stream) {
    g_last_error.clear();
    return fwd_common(x, w, y, rstd, M, N, eps, offset, dtype, nullptr, plan, true, false, stream);
}

int rmsnorm_fwd_ex(const void* x, const void* w, void* y, float* rstd, int64_t M, int64_t N, float eps,
                   float offset, int dtype, const rmsnorm_layout_t* layout, const rmsnorm_plan_t* plan,
                   void* stream) {
    g_last_error.clear();
    return fwd_common(x, w, y, rstd, M, N, eps, offset, dtype, layout, plan, false, true, stream);
}

int rmsnorm_plan_query_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                          const rmsnorm_layout_t* layout, int32_t cu_count, rmsnorm_plan_t* out) {
    g_last_error.clear();
    if (!out) return fail(RMSNORM_ERR_NULL, "out must be non-NULL");
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    Layout L;
    st = normalise_layout(layout, M, N, &L);
    if (st != RMSNORM_OK) return st;
    rmsnorm_plan_t p;
    const KernelEntry* k = nullptr;
    st = select_plan(M > 0 ? L.rows : 0, N, dtype, access_of(x, w, y, dtype, L, M, N), &p, &k);
    if (st == RMSNORM_OK) st = resident_grid(&p, k, cu_count, &p.resident_grid);
    if (st != RMSNORM_OK) return st;
    *out = p;
    return RMSNORM_OK;
}

int rmsnorm_plan_query(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                       int32_t cu_count, rmsnorm_plan_t* out) {
    return rmsnorm_plan_query_ex(M, N, dtype, x, w, y, nullptr, cu_count, out);
}

int rmsnorm_plan_validate(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                          const rmsnorm_plan_t* plan, int32_t cu_count, rmsnorm_plan_t* out) {
    g_last_error.clear();
    if (!plan || !out) return fail(RMSNORM_ERR_NULL, "plan and out must be non-NULL");
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    rmsnorm_plan_t p = *plan;
    const KernelEntry* k = nullptr;
    st = finish_plan(&p, M, N, dtype, access_of(x, w, y, dtype, contiguous_layout(M, N), M, N), &k);
    if (st == RMSNORM_OK) st = resident_grid(&p, k, cu_count, &p.resident_grid);
    if (st != RMSNORM_OK) return st;
    *out = p;
    return RMSNORM_OK;
}

int rmsnorm_fwd_kernel_query(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* y,
                             const rmsnorm_plan_t* plan, const char** kernel_name, int32_t* vgprs,
                             int32_t* lds_bytes, int32_t* scratch) {
    g_last_error.clear();
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    if (M == 0) return fail(RMSNORM_ERR_SHAPE, "M == 0 launches nothing");
    const Layout L = contiguous_layout(M, N);
    const Access acc = access_of(x, w, y, dtype, L, M, N);
    rmsnorm_plan_t p;
    if (plan) {
        p = *plan;
    } else {
        st = rmsnorm_plan_query(M, N, dtype, x, w, y, 256, &p);
        if (st != RMSNORM_OK) return st;
    }
    const KernelEntry* k = nullptr;
    st = finish_plan(&p, M, N, dtype, acc, &k);
    if (st != RMSNORM_OK) return st;
    k = launch_instance(k, &p, M, N, dtype, L, 1);
    if (kernel_name) *kernel_name = k->name;
    if (vgprs || lds_bytes || scratch) {
        hipFuncAttributes attr;
        hipError_t e = hipFuncGetAttributes(&attr, k->func);
        if (e != hipSuccess) return fail(RMSNORM_ERR_HIP, std::string("hipFuncGetAttributes: ") + hipGetErrorString(e));
        if (vgprs) *vgprs = attr.numRegs;
        if (lds_bytes) *lds_bytes = static_cast<int32_t>(attr.sharedSizeBytes);
        if (scratch) *scratch = static_cast<int32_t>(attr.localSizeBytes);
    }
    return RMSNORM_OK;
}

int rmsnorm_plan_resources(const rmsnorm_plan_t* plan, int dtype, int32_t* vgprs, int32_t* sgprs,
                           int32_t* lds_bytes, int32_t* scratch) {
    g_last_error.clear();
    if (!plan) return fail(RMSNORM_ERR_NULL, "plan must be non-NULL");
    if (dtype != RMSNORM_BF16 && dtype != RMSNORM_FP16 && dtype != RMSNORM_FP32)
        return fail(RMSNORM_ERR_DTYPE, "bad dtype");
    const KernelEntry* k = nullptr;
    const bool pf = plan->prefetch != 0;
    if (plan->variant == RMSNORM_VARIANT_GENERIC) k = find_kernel(RMSNORM_VARIANT_GENERIC, dtype, 0, 0, 1, false);
    else if (plan->variant == RMSNORM_VARIANT_BLOCK) {
        k = find_kernel(RMSNORM_VARIANT_BLOCK, dtype, 0, plan->vectors_per_lane, 1, pf);
        if (!k && !pf) k = rmsnorm_impl::exact_block_kernel(dtype, plan->vectors_per_lane, plan->block_threads);
    }
    else if (plan->variant == RMSNORM_VARIANT_SHIFTED)
        k = find_kernel(RMSNORM_VARIANT_SHIFTED, dtype, 0, plan->vectors_per_lane, 1, pf);
    else if (plan->variant == RMSNORM_VARIANT_WIDE)
        k = find_kernel(RMSNORM_VARIANT_WIDE, dtype, 0, plan->vectors_per_lane, 1, false);
    else if (plan->variant == RMSNORM_VARIANT_SHIFTED_WAVE)
        k = find_kernel(RMSNORM_VARIANT_SHIFTED_WAVE, dtype, plan->lanes_per_row, plan->vectors_per_lane,
                        plan->row_slots, pf);
    else if (plan->variant == RMSNORM_VARIANT_WAVE)
        k = find_kernel(RMSNORM_VARIANT_WAVE, dtype, plan->lanes_per_row, plan->vectors_per_lane, plan->row_slots, pf);
    if (!k) return fail(RMSNORM_ERR_PLAN, "no compiled kernel for this plan");
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, k->func);
    if (e != hipSuccess) return fail(RMSNORM_ERR_HIP, std::string("hipFuncGetAttributes: ") + hipGetErrorString(e));
    if (vgprs) *vgprs = attr.numRegs;
    if (sgprs) *sgprs = -1;  // not exposed by hipFuncGetAttributes
    if (lds_bytes) *lds_bytes = static_cast<int32_t>(attr.sharedSizeBytes);
    if (scratch) *scratch = static_cast<int32_t>(attr.localSizeBytes);
    return RMSNORM_OK;
}


// The queries without a w argument take w as 16-byte aligned (as every device
// allocation is); only its alignment informs a plan.
const void* const kAssumedW = reinterpret_cast<const void*>(uintptr_t{256});

int rmsnorm_bwd_plan_query(int64_t M, int64_t N, int dtype, const void* x, const void* dy, const void* dx,
                           int32_t cu_count, rmsnorm_plan_t* out) {
    return rmsnorm_bwd_plan_query_ex(M, N, dtype, x, kAssumedW, dy, dx, nullptr, cu_count, out);
}

int rmsnorm_bwd_plan_query_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* dy,
                              const void* dx, const rmsnorm_bwd_layout_t* layout, int32_t cu_count,
                              rmsnorm_plan_t* out) {
    g_last_error.clear();
    if (!out) return fail(RMSNORM_ERR_NULL, "out must be non-NULL");
    rmsnorm_plan_t p;
    const KernelEntry* k = nullptr;
    int st = bwd_plan_for(M, N, dtype, x, w, dy, dx, layout, &p, &k);
    if (st == RMSNORM_OK) st = resident_grid(&p, k, cu_count, &p.resident_grid);
    if (st != RMSNORM_OK) return st;
    *out = p;
    return RMSNORM_OK;
}

int rmsnorm_bwd_plan_validate(int64_t M, int64_t N, int dtype, const void* x, const void* dy, const void* dx,
                              const rmsnorm_plan_t* plan, int32_t cu_count, rmsnorm_plan_t* out) {
    g_last_error.clear();
    if (!plan || !out) return fail(RMSNORM_ERR_NULL, "plan and out must be non-NULL");
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    BwdLayout L;
    st = normalise_bwd_layout(nullptr, M, N, &L);
    if (st != RMSNORM_OK) return st;
    const bool vec = bwd_vector_ok(x, kAssumedW, dy, dx, dtype, L, M, N);
    const bool shifted = bwd_shifted_ok(x, kAssumedW, dy, dx, dtype, L, M, N, vec);
    rmsnorm_plan_t p = *plan;
    const KernelEntry* k = nullptr;
    st = finish_bwd_plan(&p, M, N, dtype, vec, shifted, &k);
    if (st == RMSNORM_OK) st = resident_grid(&p, k, cu_count, &p.resident_grid);
    if (st != RMSNORM_OK) return st;
    *out = p;
    return RMSNORM_OK;
}

int rmsnorm_bwd_workspace_size(int64_t M, int64_t N, int dtype, const void* x, const void* dy, const void* dx,
                               int64_t* bytes) {
    return rmsnorm_bwd_workspace_size_ex(M, N, dtype, x, kAssumedW, dy, dx, nullptr, bytes);
}

int rmsnorm_bwd_workspace_size_ex(int64_t M, int64_t N, int dtype, const void* x, const void* w, const void* dy,
                                  const void* dx, const rmsnorm_bwd_layout_t* layout, int64_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(RMSNORM_ERR_NULL, "bytes must be non-NULL");
    rmsnorm_plan_t p;
    const KernelEntry* k = nullptr;
    const int st = bwd_plan_for(M, N, dtype, x, w, dy, dx, layout, &p, &k);
    if (st != RMSNORM_OK) return st;
    *bytes = M > 0 ? p.grid * N * 4 : 0;
    return RMSNORM_OK;
}

int rmsnorm_bwd(const void* x, const void* w, const void* dy, const float* rstd, void* dx, float* dw, int64_t M,
                int64_t N, float offset, int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    g_last_error.clear();
    return bwd_common(x, w, dy, rstd, dx, dw, M, N, offset, dtype, nullptr, nullptr, workspace, workspace_bytes,
                      stream);
}

int rmsnorm_bwd_with_plan(const void* x, const void* w, const void* dy, const float* rstd, void* dx, float* dw,
                          int64_t M, int64_t N, float offset, int dtype, const rmsnorm_plan_t* plan,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!plan) {
        const int st = check_shape_dtype(M, N, dtype);
        return st != RMSNORM_OK ? st : fail(RMSNORM_ERR_NULL, "plan must be non-NULL");
    }
    return bwd_common(x, w, dy, rstd, dx, dw, M, N, offset, dtype, nullptr, plan, workspace, workspace_bytes,
                      stream);
}

int rmsnorm_bwd_ex(const void* x, const void* w, const void* dy, const float* rstd, void* dx, float* dw, int64_t M,
                   int64_t N, float offset, int dtype, const rmsnorm_bwd_layout_t* layout,
                   const rmsnorm_plan_t* plan, void* workspace, int64_t workspace_bytes, void* stream) {
    g_last_error.clear();
    return bwd_common(x, w, dy, rstd, dx, dw, M, N, offset, dtype, layout, plan, workspace, workspace_bytes,
                      stream);
}

int rmsnorm_bwd_noalloc(const void* x, const void* w, const void* dy, const float* rstd, void* dx, float* dw,
                        int64_t M, int64_t N, float offset, int dtype, void* stream) {
    g_last_error.clear();
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    const BwdLayout L = contiguous_bwd_layout(M, N);
    st = check_bwd_args(x, w, dy, rstd, dx, dw, M, N, offset, dtype, L);
    if (st != RMSNORM_OK) return st;
    constexpr int64_t kScratch = RMSNORM_BWD_SCRATCH_BYTES;
    if (N > kScratch / 4)
        return fail(RMSNORM_ERR_SHAPE, "rmsnorm_bwd_noalloc holds one fp32 partial row of N columns in its " +
                                           std::to_string(kScratch) + "-byte scratch: N must be at most " +
                                           std::to_string(kScratch / 4));
    const bool vec = bwd_vector_ok(x, w, dy, dx, dtype, L, M, N);
    const bool shifted = bwd_shifted_ok(x, w, dy, dx, dtype, L, M, N, vec);
    rmsnorm_plan_t p;
    choose_bwd_plan(M, N, vec, shifted, dtype, &p);
    // the rule's plan, with no more partial rows than the scratch holds (the row pass loops instead)
    p.grid = std::min<int64_t>(p.grid, kScratch / (N * 4));
    const KernelEntry* k = nullptr;
    st = finish_bwd_plan(&p, M, N, dtype, vec, shifted, &k);
    if (st != RMSNORM_OK) return st;
    int cu = 0;
    st = device_info(&cu);
    if (st != RMSNORM_OK) return st;
    void* scratch = nullptr;
    if (M > 0) {
        const char* err = rmsnorm_impl::bwd_scratch(&scratch);
        if (err) return fail(RMSNORM_ERR_HIP, std::string("scratch: ") + err);
    }
    return launch_bwd(k, &p, x, w, dy, rstd, dx, dw, M, N, offset, L, scratch, stream);
}

int rmsnorm_plan_set_tuned(int64_t M, int64_t N, int dtype, const rmsnorm_plan_t* plan) {
    g_last_error.clear();
    if (!plan) return fail(RMSNORM_ERR_NULL, "plan must be non-NULL");
    int st = check_shape_dtype(M, N, dtype);
    if (st != RMSNORM_OK) return st;
    if (M == 0) return fail(RMSNORM_ERR_SHAPE, "a tuned plan needs M > 0");
    rmsnorm_plan_t p = *plan;
    const KernelEntry* k = nullptr;
    st = finish_plan(&p, M, N, dtype, access_of(nullptr, nullptr, nullptr, dtype, contiguous_layout(M, N), M, N),
                     &k);  // aligned pointers
    if (st != RMSNORM_OK) return st;
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    g_tuned[std::make_tuple(M, N, dtype)] = p;
    g_tuned_count.store(static_cast<int>(g_tuned.size()), std::memory_order_release);
    return RMSNORM_OK;
}

int rmsnorm_plan_clear_tuned(void) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lock(g_tuned_mu);
    g_tuned.clear();
    g_tuned_count.store(0, std::memory_order_release);
    return RMSNORM_OK;
}

int rmsnorm_plan_tuned_count(void) { return g_tuned_count.load(std::memory_order_acquire); }

const char* rmsnorm_status_string(int status) {
    switch (status) {
        case RMSNORM_OK: return "RMSNORM_OK";
        case RMSNORM_ERR_NULL: return "RMSNORM_ERR_NULL";
        case RMSNORM_ERR_SHAPE: return "RMSNORM_ERR_SHAPE";
        case RMSNORM_ERR_DTYPE: return "RMSNORM_ERR_DTYPE";
        case RMSNORM_ERR_SCALAR: return "RMSNORM_ERR_SCALAR";
        case RMSNORM_ERR_OVERLAP: return "RMSNORM_ERR_OVERLAP";
        case RMSNORM_ERR_HIP: return "RMSNORM_ERR_HIP";
        case RMSNORM_ERR_DEVICE: return "RMSNORM_ERR_DEVICE";
        case RMSNORM_ERR_PLAN: return "RMSNORM_ERR_PLAN";
        default: return "RMSNORM_ERR_UNKNOWN";
    }
}

const char* rmsnorm_last_error(void) { return g_last_error.c_str(); }

int rmsnorm_version(void) { return kVersion; }

}  // extern "C"
