// rmsnorm_kernels.hip -- row RMSNorm forward kernels for gfx950 (MI355X).
//
// Per row m:  rstd[m] = rsqrt(sum_j x[m,j]^2 * (1/N) + eps)
//             y[m,j]  = x[m,j] * rstd[m] * (offset + w[j])
// ("Rmsnorm Kernel Optimization", Overview and Core Technique; "Why cutile's
// rmsnorm required full register", kernel listing of the opening report).
//
// All arithmetic is fp32; x, w and y are bf16, fp16 or fp32 (a 16-byte
// vector holds D::EPV = 8 or 4 elements).  Rows may be strided, in one or
// more batches (the grid's y dimension); a width that is not a multiple of
// EPV ends in a tail vector moved element by element; rstd may be NULL.
// The families:
//
//  * rmsnorm_wave   -- a row lives in a segment of 4, 8, 16, 32 or 64 lanes of
//    one wavefront, each lane holding VPL 16-byte vectors of it; a wave carries
//    SLOTS x (64 / LANES) rows per trip and issues every load of the trip
//    before its first reduction.  Reductions are DPP and v_readlane only, no
//    LDS.  Several rows per wave for small hidden sizes follows "Rmsnorm
//    Kernel Optimization", Key Optimizations.
//  * rmsnorm_block  -- one row per workgroup per trip, each thread holding VPT
//    16-byte vectors; wave sums meet in LDS behind one barrier per trip
//    (double-buffered partials).  For large N.
//  * rmsnorm_wave_exact, rmsnorm_block_exact -- one-trip forms of the two
//    above for contiguous rows of exactly their width, with the geometry fixed
//    at compile time; launches switch to them wherever a call fits.
//  * rmsnorm_wide   -- aligned rows wider than the block family holds, in tiles.
//  * rmsnorm_shifted, rmsnorm_shifted_wave -- rows that do not start 16-byte
//    aligned (contiguous rows with N % EPV != 0): aligned 16-byte chunks,
//    per-row shifted weights, element-wise edges.
//  * rmsnorm_generic -- any N and any alignment, element accesses, the row
//    read a second time (from cache) to normalise.  Correctness fallback.
//
// Except for the exact forms, each family loops over rows with a grid stride,
// so a grid smaller than the row count is a persistent grid that keeps
// offset + w in registers across trips (the static persistent schedule of the
// cuTile listing, re-expressed for wave64 and the 256-CU chip).  Columns at or past N are never loaded or
// stored: loads there yield zero and contribute nothing to the sum of
// squares, the padding rule of the same listing.
#include "rmsnorm_device.hpp"
#include "rmsnorm_internal.hpp"
#include "../../include/rmsnorm.h"

using namespace rmsnorm_dev;
using rmsnorm_impl::KernelArgs;

namespace {

// x and y are touched once per call: non-temporal loads and stores stream
// them, so they neither evict w nor sit dirty in L2 until the end-of-kernel
// write-back.  Measured on MI355X with inputs cold in HBM, streaming both is
// the fastest or tied on every shape tried (by 4% on 16384 x 512, where the
// kernel is short).  w is read by every row and keeps the default policy.
constexpr bool kStreamX = true;
constexpr bool kStreamY = true;

__device__ __forceinline__ u32x4 load_x(const u32x4* p) {
    if constexpr (kStreamX) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ __forceinline__ void store_y(u32x4* p, u32x4 v) {
    if constexpr (kStreamY) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// rstd goes out after the row's y stores, non-temporally.  Measured on MI355X
// at 16384 x 512, storing it before y made the compiler wait for the first
// rows' loads before issuing the rest (6.6 against 6.3 us per launch).
__device__ __forceinline__ void store_rstd(float* p, float v) { __builtin_nontemporal_store(v, p); }

template <class D, int VPL>
__device__ __forceinline__ float sum_squares(const u32x4 (&d)[VPL]) {
    float ss = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        float f[D::EPV];
        D::widen(d[v], f);
#pragma unroll
        for (int e = 0; e < D::EPV; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
    }
    return ss;
}

// offset + w for the EPV columns of one 16-byte weight vector (fp32, as the
// listing forms offset + w after widening w).
template <class D>
__device__ __forceinline__ void widen_weights(float (&we)[D::EPV], const u32x4 q, float offset) {
    float f[D::EPV];
    D::widen(q, f);
#pragma unroll
    for (int e = 0; e < D::EPV; ++e) we[e] = offset + f[e];
}

template <class D>
__device__ __forceinline__ u32x4 normalise(const u32x4 q, const float (&we)[D::EPV], float r) {
    float f[D::EPV];
    D::widen(q, f);
#pragma unroll
    for (int e = 0; e < D::EPV; ++e) f[e] = (f[e] * r) * we[e];
    return D::narrow(f);
}

constexpr u32x4 kZero = {0u, 0u, 0u, 0u};

// Batches of rows run as the grid's y dimension: batch b = blockIdx.y starts
// b * bs elements into x and y and b * M entries into rstd, and its rows are
// rs elements apart (no division anywhere).  The first batch (every launch
// without batches) skips the offset arithmetic.
__device__ __forceinline__ int64_t batch() { return static_cast<int64_t>(blockIdx.y); }

template <class T>
__device__ __forceinline__ T* batch_base(T* p, int64_t stride) {
    return __builtin_expect(blockIdx.y == 0, 1) ? p : p + batch() * stride;
}

// The last vector of a row whose width is not a multiple of EPV holds only
// `tail` elements: they move one element at a time, so nothing past column
// N - 1 is read or written (the bytes there may belong to something else).
template <class D>
__device__ __forceinline__ u32x4 load_tail(const u32x4* p, int tail) {
    typedef typename D::elem_t E;
    const E* q = reinterpret_cast<const E*>(p);
    E e[D::EPV];
#pragma unroll
    for (int i = 0; i < D::EPV; ++i) e[i] = i < tail ? q[i] : E(0);
    return __builtin_bit_cast(u32x4, e);
}

template <class D>
__device__ __forceinline__ void store_tail(u32x4* p, u32x4 v, int tail) {
    typedef typename D::elem_t E;
    E* q = reinterpret_cast<E*>(p);
    const auto e = __builtin_bit_cast(E __attribute__((ext_vector_type(D::EPV))), v);
#pragma unroll
    for (int i = 0; i < D::EPV; ++i)
        if (i < tail) q[i] = e[i];
}

// Strides arrive in elements (never negative); the 16-byte kernels step in
// vectors.
template <class D>
__device__ __forceinline__ int64_t vectors(int64_t elems) {
    return static_cast<int64_t>(static_cast<uint64_t>(elems) / D::EPV);
}

// Vector c of a row: full vectors below nfull; with TAIL, also the tail
// vector at nfull (instances without TAIL run only when N % EPV == 0).
template <class D, bool STREAM, bool TAIL>
__device__ __forceinline__ u32x4 load_vec(const u32x4* row, int c, int nfull, int tail) {
    if (c < nfull) return STREAM ? load_x(row + c) : row[c];
    if constexpr (TAIL) {
        if (__builtin_expect(tail != 0, 0) && c == nfull) return load_tail<D>(row + c, tail);
    }
    return kZero;
}

template <class D, bool TAIL>
__device__ __forceinline__ void store_vec(u32x4* row, int c, int nfull, int tail, u32x4 v) {
    if (c < nfull) {
        store_y(row + c, v);
    } else if constexpr (TAIL) {
        if (__builtin_expect(tail != 0, 0) && c == nfull) store_tail<D>(row + c, v, tail);
    }
}

// The dispatcher hands workgroup b to XCD b mod 8 (MI355X has 8 XCDs, each
// with its own L2).  With group g > 1 the workgroup index is remapped inside
// windows of 8 * g workgroups so that XCD x serves g consecutive row groups,
// (b mod 8) * g + (b / 8) mod g within the window: a transpose of the window,
// so every index in [0, G) is still used exactly once (a tail shorter
// than a window keeps its own order).  Consecutive rows then share an L2 and
// reach HBM as longer runs of neighbouring addresses.  Measured on MI355X:
// groups of about 128 KiB of rows shorten the 32768 x 8192 forward by 4-5% at
// a favourable placement of y relative to x but leave its rate following that
// placement over a 10% range; groups of about 1 MiB hold it at every
// placement measured (the planner's choice for batches beyond the 256 MB
// Infinity Cache).
// (32-bit arithmetic: grids stay below 2^31 workgroups and windows below 2^12.)
__device__ __forceinline__ int64_t grouped_block(int g, int64_t G) {
    const uint32_t b = blockIdx.x;
    if (__builtin_expect(g <= 1, 1)) return b;
    const uint32_t ug = static_cast<uint32_t>(g);
    const uint32_t span = 8u * ug;
    const uint32_t full = (static_cast<uint32_t>(G) / span) * span;
    if (b >= full) return b;
    return (b / span) * span + (b % 8u) * ug + (b / 8u) % ug;
}

}  // namespace

// ---------------------------------------------------------------------------
// Wave family.
//
// Lane l of a wave serves row segment l / LANES and, in it, the 16-byte
// vectors v * LANES + l % LANES, v < VPL (consecutive lanes touch
// consecutive 16-byte chunks: fully coalesced).  A trip covers SLOTS slots of
// 64 / LANES rows each, all loads issued before the first reduction.  The
// weights are loaded after the first trip's rows, so the two latencies
// overlap instead of adding up.  With PREFETCH the next trip's rows are
// loaded before this trip's reduction.
// ---------------------------------------------------------------------------
template <class D, int LANES, int VPL, int SLOTS, bool PREFETCH, bool TAIL>
__global__ __launch_bounds__(1024) void rmsnorm_wave(KernelArgs a) {
    constexpr int SEG = 64 / LANES;       // rows per slot
    constexpr int ROWS = SEG * SLOTS;     // rows per wave per trip
    const int64_t M = a.M;
    const u32x4* __restrict__ x = batch_base(static_cast<const u32x4*>(a.x), vectors<D>(a.x_bs));
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = batch_base(static_cast<u32x4*>(a.y), vectors<D>(a.y_bs));
    const int nfull = static_cast<int>(static_cast<uint64_t>(a.N) / D::EPV);
    const int tail = static_cast<int>(static_cast<uint64_t>(a.N) % D::EPV);
    const int x_rs = a.x_rsv, y_rs = a.y_rsv;   // vectors (32-bit: one short multiply per row)
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int wpb = a.threads >> 6;
    // the wave's index is the same in all its lanes: keep it in a scalar register
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t nwaves = a.grid * wpb;
    int64_t g = grouped_block(a.xcd_group, a.grid) * wpb + wid;
    // No early exit for waves past the last row: every access below is masked
    // by row < M, and without the branch the compiler fetches all the kernel
    // arguments the first loads need in one batch of scalar loads.

    auto load_trip = [&](u32x4 (&d)[SLOTS][VPL], int64_t gg) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            const u32x4* xr = x + row * x_rs;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                d[s][v] = (row < M && c < nfull) ? load_x(xr + c) : kZero;
            }
        }
        // tail vectors: a pass of their own, skipped as a whole when N % EPV == 0
        if constexpr (TAIL) {
            if (__builtin_expect(tail != 0, 0)) {
#pragma unroll
                for (int s = 0; s < SLOTS; ++s) {
                    const int64_t row = gg * ROWS + seg + s * SEG;
#pragma unroll
                    for (int v = 0; v < VPL; ++v)
                        if (row < M && v * LANES + li == nfull) d[s][v] = load_tail<D>(x + row * x_rs + nfull, tail);
                }
            }
        }
    };

    u32x4 d[SLOTS][VPL];
    load_trip(d, g);
    float we[VPL][D::EPV];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        widen_weights<D>(we[v], load_vec<D, false, TAIL>(w, c, nfull, tail), a.offset);
    }

    // reductions, then every y store of the trip, then its rstd stores
    auto finish_trip = [&](const u32x4 (&dd)[SLOTS][VPL], int64_t gg) {
        float r[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const float ss = segment_allreduce<LANES>(sum_squares<D, VPL>(dd[s]));
            r[s] = rsq(__builtin_fmaf(ss, a.inv_n, a.eps));
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            u32x4* yr = y + row * y_rs;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                if (row < M) store_vec<D, TAIL>(yr, c, nfull, tail, normalise<D>(dd[s][v], we[v], r[s]));
            }
        }
        if (a.rstd != nullptr) {
            float* rstd = a.rstd + batch() * M;
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
                const int64_t row = gg * ROWS + seg + s * SEG;
                if (li == 0 && row < M) store_rstd(rstd + row, r[s]);
            }
        }
    };

    // Without prefetching, a wave with one trip (every wave of the planned
    // launches) runs straight through: the loop below would let the compiler
    // move the next trip's loads in among this trip's stores.
    if constexpr (!PREFETCH) {
        if ((g + nwaves) * ROWS >= M) {
            finish_trip(d, g);
            return;
        }
    }
    for (;;) {
        const int64_t gn = g + nwaves;
        const bool more = gn * ROWS < M;
        u32x4 dn[SLOTS][VPL];
        if constexpr (PREFETCH) {
            if (more) load_trip(dn, gn);
        }
        finish_trip(d, g);
        if (!more) break;
        g = gn;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
#pragma unroll
                for (int v = 0; v < VPL; ++v) d[s][v] = dn[s][v];
        } else {
            load_trip(d, g);
        }
    }
}

// ---------------------------------------------------------------------------
// Exact-width wave form: the wave family's lane layout for the launches its
// rule makes most often -- contiguous rows of exactly LANES * VPL vectors, one
// batch, one trip per wave, WPB waves per workgroup, no XCD remap -- without
// what only other calls need: no per-lane column masks (every lane's vectors
// lie inside the row), a compile-time row stride and workgroup size, 32-bit
// row numbers (the dispatcher sends M below 2^31 - 2^16 only), no loop.
// The wave index stays per lane (a scalar one turns each slot's row test into
// a branch around its load), and the wave's ROWS consecutive rstd values go
// out in one store (up to 16 rows; the 64 rows of a 4-lane wave are gathered
// at two instructions a row, so there each slot stores its own: 262144 x 32
// bf16 took 7.04 us with the gather, 6.09-6.11 us without).  Measured on
// MI355X at 16384 x 512 bf16 with inputs cold in HBM, in timing copies on one
// box in one process: 6.22-6.25 us against 6.31-6.34 us for the same kernel
// with a scalar wave index, a runtime workgroup size and one rstd store per
// slot, and 6.39 us for the general wave instance.
// ---------------------------------------------------------------------------
template <class D, int LANES, int VPL, int SLOTS, int WPB>
__global__ __launch_bounds__(WPB * 64) void rmsnorm_wave_exact(KernelArgs a) {
    constexpr int SEG = 64 / LANES;       // rows per slot
    constexpr int ROWS = SEG * SLOTS;     // rows per wave: rows r0 .. r0 + ROWS - 1
    constexpr int RV = LANES * VPL;       // vectors per row, and the row stride
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = static_cast<u32x4*>(a.y);
    const int M = static_cast<int>(a.M);
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int r0 = (static_cast<int>(blockIdx.x) * WPB + static_cast<int>(threadIdx.x >> 6)) * ROWS;

    u32x4 d[SLOTS][VPL];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const int row = r0 + seg + s * SEG;
        const u32x4* xr = x + static_cast<int64_t>(row) * RV + li;
#pragma unroll
        for (int v = 0; v < VPL; ++v) d[s][v] = row < M ? load_x(xr + v * LANES) : kZero;
    }
    float we[VPL][D::EPV];
#pragma unroll
    for (int v = 0; v < VPL; ++v) widen_weights<D>(we[v], w[v * LANES + li], a.offset);

    float r[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const float ss = segment_allreduce<LANES>(sum_squares<D, VPL>(d[s]));
        r[s] = rsq(__builtin_fmaf(ss, a.inv_n, a.eps));
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const int row = r0 + seg + s * SEG;
        u32x4* yr = y + static_cast<int64_t>(row) * RV + li;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (row < M) store_y(yr + v * LANES, normalise<D>(d[s][v], we[v], r[s]));
    }
    if (a.rstd != nullptr) {
        if constexpr (ROWS <= 16) {
            // lane j < ROWS stores row r0 + j: slot j / SEG of segment j % SEG,
            // whose value every lane of that segment holds (read from its first lane)
            float rv = 0.0f;
#pragma unroll
            for (int j = 0; j < ROWS; ++j) {
                const float rj = SEG == 1 ? r[j] : readlane(r[j / SEG], (j % SEG) * LANES);
                rv = lane == j ? rj : rv;
            }
            if (lane < ROWS && r0 + lane < M) store_rstd(a.rstd + r0 + lane, rv);
        } else {
            // many rows per wave (4-lane rows): gathering them costs two
            // instructions a row; each slot's first lanes store its SEG
            // consecutive rows instead
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
                const int row = r0 + seg + s * SEG;
                if (li == 0 && row < M) store_rstd(a.rstd + row, r[s]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Block family.
//
// Thread t of a workgroup of T threads holds the 16-byte vectors v * T + t,
// v < VPT, of one row.  Wave sums meet in LDS: one barrier per row, with the
// partials double-buffered so the next row's writes cannot race this row's
// reads (a wave can be at most one barrier ahead of another).  With PREFETCH
// the next row is loaded before this row's reduction.
// ---------------------------------------------------------------------------
template <class D, int VPT, bool PREFETCH, bool TAIL>
__global__ __launch_bounds__(1024) void rmsnorm_block(KernelArgs a) {
    __shared__ float part[2][16];
    const int64_t M = a.M;
    const u32x4* __restrict__ x = batch_base(static_cast<const u32x4*>(a.x), vectors<D>(a.x_bs));
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = batch_base(static_cast<u32x4*>(a.y), vectors<D>(a.y_bs));
    const int nfull = static_cast<int>(static_cast<uint64_t>(a.N) / D::EPV);
    const int tail = static_cast<int>(static_cast<uint64_t>(a.N) % D::EPV);
    const int x_rs = a.x_rsv, y_rs = a.y_rsv;   // vectors (32-bit: one short multiply per row)
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;
    int64_t row = grouped_block(a.xcd_group, a.grid);
    // no early exit for workgroups past the last row (see the wave family):
    // their loads and stores are masked instead

    auto load_row = [&](u32x4 (&d)[VPT], int64_t rr) {
        const u32x4* xr = x + rr * x_rs;
        const bool live = rr < M;
#pragma unroll
        for (int v = 0; v < VPT; ++v) d[v] = (live && v * nt + tid < nfull) ? load_x(xr + v * nt + tid) : kZero;
        if constexpr (TAIL) {
            if (__builtin_expect(tail != 0, 0)) {
#pragma unroll
                for (int v = 0; v < VPT; ++v)
                    if (live && v * nt + tid == nfull) d[v] = load_tail<D>(xr + nfull, tail);
            }
        }
    };

    u32x4 d[VPT];
    load_row(d, row);
    float we[VPT][D::EPV];
#pragma unroll
    for (int v = 0; v < VPT; ++v) widen_weights<D>(we[v], load_vec<D, false, TAIL>(w, v * nt + tid, nfull, tail), a.offset);

    // the row's reduction (wave butterfly, then the waves' sums through LDS),
    // every y store, then rstd
    auto finish_row = [&](const u32x4 (&dd)[VPT], int64_t rr, int pp) {
        const float ss = segment_allreduce<64>(sum_squares<D, VPT>(dd));
        if (lane == 0) part[pp][wid] = ss;
        __syncthreads();
        float tot = part[pp][0];
        for (int i = 1; i < nw; ++i) tot += part[pp][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
        if (rr < M) {
            u32x4* yr = y + rr * y_rs;
#pragma unroll
            for (int v = 0; v < VPT; ++v) store_vec<D, TAIL>(yr, v * nt + tid, nfull, tail, normalise<D>(dd[v], we[v], r));
            if (tid == 0 && a.rstd != nullptr) store_rstd(a.rstd + batch() * M + rr, r);
        }
    };

    // one row per workgroup (the planned launches): straight through
    if constexpr (!PREFETCH) {
        if (row + a.grid >= M) {
            finish_row(d, row, 0);
            return;
        }
    }
    int par = 0;
    for (;;) {
        const int64_t next = row + a.grid;
        const bool more = next < M;
        u32x4 dn[VPT];
        if constexpr (PREFETCH) {
            if (more) load_row(dn, next);
        }
        finish_row(d, row, par);
        if (!more) break;
        row = next;
        par ^= 1;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) d[v] = dn[v];
        } else {
            load_row(d, row);
        }
    }
}

// ---------------------------------------------------------------------------
// Exact-width block form: one row of exactly T * VPT vectors per workgroup,
// contiguous rows in one batch, one trip (a grid of exactly M), the block family's
// XCD row placement.  The weights stay packed and are widened at use, so 8
// vectors per thread fit in 128 VGPRs at four 256-thread workgroups per CU,
// where the block family's fp32 weights would need 64 more registers.  With
// no row loop, no column mask and no branch around a load, all of a thread's
// loads issue back to back and the arithmetic starts as each vector lands.
// Measured on MI355X with inputs cold in HBM, at most 3 workgroups per CU:
// 4096 x 16384 fp16 (256 x 8) 44.7 us, against 47.4 us for 1024 x 2 block
// plans and 47.0 us for 512 x 4; 32768 x 8192 bf16 (256 x 4) 167.2-167.9 us
// on three boxes, where the block family's 256 x 4 at its best cap of 4 took
// 169.1-169.9 us (the exact form at 4 per CU: 170.0 us).  Launches switch to
// it wherever the call fits (launch_instance).
// ---------------------------------------------------------------------------
template <class D, int VPT, int T>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(4))) void rmsnorm_block_exact(KernelArgs a) {
    constexpr int NW = T / 64;
    constexpr int RV = T * VPT;           // vectors per row, and the row stride
    __shared__ float part[NW];
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = static_cast<u32x4*>(a.y);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    // The grid is exactly M workgroups (launch_instance and finish_plan send
    // no other), so every workgroup owns a row and no load or store needs a
    // guard.  Every load is unconditional: a load under a branch made the
    // compiler wait for the first vector before issuing the other fifteen
    // loads of the row, and a row-liveness guard cost 0.35 % at 32768 x 8192.
    const int64_t row = grouped_block(a.xcd_group, a.grid);
    const u32x4* xr = x + row * RV + tid;
    u32x4 d[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) d[v] = load_x(xr + v * T);
    u32x4 wq[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) wq[v] = w[v * T + tid];
    // nothing that uses a loaded value moves above this point
    __builtin_amdgcn_sched_barrier(0);

    const float ss = segment_allreduce<64>(sum_squares<D, VPT>(d));
    if (lane == 0) part[wid] = ss;
    __syncthreads();
    float tot = part[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) tot += part[i];
    const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
    u32x4* yr = y + row * RV + tid;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        float we[D::EPV];
        widen_weights<D>(we, wq[v], a.offset);
        store_y(yr + v * T, normalise<D>(d[v], we, r));
    }
    if (tid == 0 && a.rstd != nullptr) store_rstd(a.rstd + row, r);
}

// ---------------------------------------------------------------------------
// Wide family: aligned rows wider than the block family's registers hold.
// One row per workgroup per trip, in tiles of T * VPT vectors.  A first pass
// sums the squares tile by tile with cached loads; after the workgroup's
// reduction a second pass reads the row again (from the caches: a trip's
// rows, a few hundred KiB per compute unit, stay within the 256 MB Infinity
// Cache), normalises and stores it.  HBM still sees each element of x read
// once and of y written once.
// ---------------------------------------------------------------------------
template <class D, int VPT>
__global__ __launch_bounds__(1024) void rmsnorm_wide(KernelArgs a) {
    __shared__ float part[2][16];
    const int64_t M = a.M;
    const u32x4* __restrict__ x = batch_base(static_cast<const u32x4*>(a.x), vectors<D>(a.x_bs));
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = batch_base(static_cast<u32x4*>(a.y), vectors<D>(a.y_bs));
    const int nfull = static_cast<int>(static_cast<uint64_t>(a.N) / D::EPV);
    const int tail = static_cast<int>(static_cast<uint64_t>(a.N) % D::EPV);
    const int nvec = nfull + (tail != 0 ? 1 : 0);
    const int x_rs = a.x_rsv, y_rs = a.y_rsv;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;
    const int tile = nt * VPT;

    int par = 0;
    for (int64_t row = grouped_block(a.xcd_group, a.grid); row < M; row += a.grid) {
        const u32x4* xr = x + row * x_rs;
        float ss = 0.0f;
        for (int t0 = 0; t0 < nvec; t0 += tile) {
            u32x4 d[VPT];
#pragma unroll
            for (int v = 0; v < VPT; ++v) d[v] = load_vec<D, false, true>(xr, t0 + v * nt + tid, nfull, tail);
            ss += sum_squares<D, VPT>(d);
        }
        ss = segment_allreduce<64>(ss);
        if (lane == 0) part[par][wid] = ss;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
        u32x4* yr = y + row * y_rs;
        for (int t0 = 0; t0 < nvec; t0 += tile) {
            u32x4 d[VPT], wq[VPT];
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int c = t0 + v * nt + tid;
                d[v] = load_vec<D, true, true>(xr, c, nfull, tail);
                wq[v] = load_vec<D, false, true>(w, c, nfull, tail);
            }
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                float we[D::EPV];
                widen_weights<D>(we, wq[v], a.offset);
                store_vec<D, true>(yr, t0 + v * nt + tid, nfull, tail, normalise<D>(d[v], we, r));
            }
        }
        if (tid == 0 && a.rstd != nullptr) store_rstd(a.rstd + batch() * M + row, r);
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Shifted family: rows that do not start on a 16-byte boundary (contiguous
// rows of N elements with N % EPV != 0 start a different number of elements
// past one on every row).  One row per workgroup per trip.  The row is read
// as the aligned 16-byte chunks that cover it: with `al` the row start's
// distance in elements past a boundary, chunk c holds row elements
// c * EPV - al .. c * EPV - al + EPV - 1.  Every chunk, the two edge chunks
// included, is loaded whole; the edge chunks' elements outside the row (the
// neighbouring rows', or bytes next to the tensor inside the same aligned 16
// bytes, so on a page the row's own elements share) are set to zero before
// use and are never written: edge chunks are stored element by element.
// The weights of chunk c are w vectors c - 1 and c funnel-shifted by
// EPV - al elements (v_alignbyte on the packed words).  w is 16-byte
// aligned, and its last vector is read whole in the same way.
//
// WPRE picks when the weights are fetched.  false: both vectors after the
// row's reduction (registers stay free for loads in flight: faster with 512
// and 1024 threads).  true: vector c with the row's loads, vector c - 1 from
// the lane below (DPP wave shift) or, for lane 0, from the last lane of the
// wave below through LDS (faster with up to 256 threads, where a row has
// fewer waves to hide the weights' latency behind).
// x and y must sit the same distance past a boundary on every row.  The
// funnel, mask and edge-store helpers are in rmsnorm_device.hpp.
// ---------------------------------------------------------------------------
template <class D, int VPT, bool WPRE>
__global__ __launch_bounds__(1024) void rmsnorm_shifted(KernelArgs a) {
    typedef typename D::elem_t E;
    constexpr int EPV = D::EPV;
    __shared__ float part[2][16];
    __shared__ u32x4 top[WPRE ? 2 : 1][WPRE ? VPT : 1][16];   // each wave's last lane's weights (WPRE)
    const int64_t M = a.M;
    const int n = static_cast<int>(a.N);      // at most 4096 chunks: 32-bit element indices
    const E* xb = static_cast<const E*>(a.x) + batch() * a.x_bs;
    E* yb = static_cast<E*>(a.y) + batch() * a.y_bs;
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const int nvec_w = (n + EPV - 1) / EPV;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    auto wvec = [&](int k) -> u32x4 { return (k >= 0 && k < nvec_w) ? w[k] : kZero; };

    int par = 0;
    for (int64_t row = grouped_block(a.xcd_group, a.grid); row < M; row += a.grid) {
        const E* xr = xb + row * a.x_rs;
        E* yr = yb + row * a.y_rs;
        // distance past a 16-byte boundary, in elements; the same for y
        const int al = __builtin_amdgcn_readfirstlane(
            static_cast<int>((reinterpret_cast<uintptr_t>(xr) & 15u) / sizeof(E)));
        const u32x4* xc = reinterpret_cast<const u32x4*>(xr - al);
        u32x4* yc = reinterpret_cast<u32x4*>(yr - al);
        const int nch = (al + n + EPV - 1) / EPV;

        u32x4 d[VPT];
        u32x4 wv[WPRE ? VPT : 1];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            d[v] = c < nch ? load_x(xc + c) : kZero;
            if constexpr (WPRE) wv[v] = wvec(c);
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int j0 = (v * nt + tid) * EPV - al;
            if (j0 < 0 || j0 + EPV > n) d[v] = keep_row<D>(d[v], j0, n);
        }
        if constexpr (WPRE) {
            if (lane == 63) {
#pragma unroll
                for (int v = 0; v < VPT; ++v) top[par][v][wid] = wv[v];
            }
        }
        const float ss = segment_allreduce<64>(sum_squares<D, VPT>(d));
        if (lane == 0) part[par][wid] = ss;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            u32x4 wc;
            if constexpr (WPRE) {
                wc = wv[v];
                if (al != 0) {
                    // vector c - 1: the lane below's, or for lane 0 the last lane's of
                    // the wave below (of the last wave, one vector back, for wave 0)
                    u32x4 below = kZero;
                    if (lane == 0 && c > 0) below = wid > 0 ? top[par][v][wid - 1] : top[par][v > 0 ? v - 1 : 0][nw - 1];
                    wc = funnel<D>(from_lane_below(wv[v], below), wc, EPV - al);
                }
            }
            if (c < nch) {
                if constexpr (!WPRE) wc = al == 0 ? wvec(c) : funnel<D>(wvec(c - 1), wvec(c), EPV - al);
                float we[EPV];
                widen_weights<D>(we, wc, a.offset);
                const u32x4 o = normalise<D>(d[v], we, r);
                const int j0 = c * EPV - al;
                if (j0 < 0 || j0 + EPV > n) store_edge<D>(yc + c, o, j0, n);
                else store_y(yc + c, o);
            }
        }
        if (tid == 0 && a.rstd != nullptr) store_rstd(a.rstd + batch() * M + row, r);
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Shifted wave family: the shifted kernel's chunk scheme for short rows, a
// row per segment of LANES lanes (8, 16, 32 or 64; at most LANES * VPL chunks),
// SLOTS slots of 64 / LANES rows per wave per trip, no LDS and no barrier.
// With 64 lanes a row's distance past a 16-byte boundary is uniform in its
// wave and the weights are shifted by a branch on it; with several rows per
// wave every lane shifts by its own row's distance.  The weights do not
// depend on the row: each lane fetches w vectors c - 1 and c of its chunks
// once, after the first trip's rows, and shifts them for each row.
// ---------------------------------------------------------------------------
template <class D, int LANES, int VPL, int SLOTS, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_shifted_wave(KernelArgs a) {
    typedef typename D::elem_t E;
    constexpr int EPV = D::EPV;
    constexpr int SEG = 64 / LANES;       // rows per slot
    constexpr int ROWS = SEG * SLOTS;     // rows per wave per trip
    const int64_t M = a.M;
    const int n = static_cast<int>(a.N);      // at most LANES * VPL chunks
    const E* xb = static_cast<const E*>(a.x) + batch() * a.x_bs;
    E* yb = static_cast<E*>(a.y) + batch() * a.y_bs;
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const int nvec_w = (n + EPV - 1) / EPV;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int wpb = a.threads >> 6;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t nwaves = a.grid * wpb;
    int64_t g = grouped_block(a.xcd_group, a.grid) * wpb + wid;

    // rows past the end keep an in-range address and load nothing
    auto row_of = [&](int64_t gg, int s) -> int64_t { return gg * ROWS + seg + s * SEG; };
    auto offset_of = [&](int64_t row) -> int {
        const E* xr = xb + (row < M ? row : 0) * a.x_rs;
        const int al = static_cast<int>((reinterpret_cast<uintptr_t>(xr) & 15u) / sizeof(E));
        if constexpr (LANES == 64) return __builtin_amdgcn_readfirstlane(al);
        else return al;
    };
    auto load_trip = [&](u32x4 (&d)[SLOTS][VPL], int64_t gg) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = row_of(gg, s);
            const int al = offset_of(row);
            const int nch = (al + n + EPV - 1) / EPV;
            const u32x4* xc = reinterpret_cast<const u32x4*>(xb + (row < M ? row : 0) * a.x_rs - al);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                d[s][v] = (row < M && c < nch) ? load_x(xc + c) : kZero;
            }
        }
    };

    u32x4 d[SLOTS][VPL];
    load_trip(d, g);
    u32x4 wlo[VPL], whi[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        wlo[v] = (c >= 1 && c - 1 < nvec_w) ? w[c - 1] : kZero;
        whi[v] = c < nvec_w ? w[c] : kZero;
    }

    auto finish_trip = [&](u32x4 (&dd)[SLOTS][VPL], int64_t gg) {
        float r[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int al = offset_of(row_of(gg, s));
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int j0 = (v * LANES + li) * EPV - al;
                if (j0 < 0 || j0 + EPV > n) dd[s][v] = keep_row<D>(dd[s][v], j0, n);
            }
            const float ss = segment_allreduce<LANES>(sum_squares<D, VPL>(dd[s]));
            r[s] = rsq(__builtin_fmaf(ss, a.inv_n, a.eps));
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = row_of(gg, s);
            const int al = offset_of(row);
            const int nch = (al + n + EPV - 1) / EPV;
            u32x4* yc = reinterpret_cast<u32x4*>(yb + (row < M ? row : 0) * a.y_rs - al);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                if (row < M && c < nch) {
                    u32x4 wc;
                    if constexpr (LANES == 64) wc = al == 0 ? whi[v] : funnel<D>(wlo[v], whi[v], EPV - al);
                    else wc = funnel_lane<D>(wlo[v], whi[v], EPV - al);
                    float we[EPV];
                    widen_weights<D>(we, wc, a.offset);
                    const u32x4 o = normalise<D>(dd[s][v], we, r[s]);
                    const int j0 = c * EPV - al;
                    if (j0 < 0 || j0 + EPV > n) store_edge<D>(yc + c, o, j0, n);
                    else store_y(yc + c, o);
                }
            }
        }
        if (a.rstd != nullptr) {
            float* rstd = a.rstd + batch() * M;
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
                const int64_t row = row_of(gg, s);
                if (li == 0 && row < M) store_rstd(rstd + row, r[s]);
            }
        }
    };

    if constexpr (!PREFETCH) {
        if ((g + nwaves) * ROWS >= M) {
            finish_trip(d, g);
            return;
        }
    }
    for (;;) {
        const int64_t gn = g + nwaves;
        const bool more = gn * ROWS < M;
        u32x4 dn[SLOTS][VPL];
        if constexpr (PREFETCH) {
            if (more) load_trip(dn, gn);
        }
        finish_trip(d, g);
        if (!more) break;
        g = gn;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
#pragma unroll
                for (int v = 0; v < VPL; ++v) d[s][v] = dn[s][v];
        } else {
            load_trip(d, g);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic family: any N, any element alignment, any strides.  x and y may be
// the same buffer with the same layout: every element is read and then
// written by the same thread, and the sum of squares of a row is complete
// (barrier) before any of it is written.
// ---------------------------------------------------------------------------
template <class D>
__global__ __launch_bounds__(1024) void rmsnorm_generic(KernelArgs a) {
    typedef typename D::elem_t E;
    __shared__ float part[2][16];
    const int64_t M = a.M;
    const E* x = static_cast<const E*>(a.x) + batch() * a.x_bs;
    const E* __restrict__ w = static_cast<const E*>(a.w);
    E* y = static_cast<E*>(a.y) + batch() * a.y_bs;
    const int64_t N = a.N;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    int par = 0;
    for (int64_t row = grouped_block(a.xcd_group, a.grid); row < M; row += a.grid) {
        const E* xr = x + row * a.x_rs;
        E* yr = y + row * a.y_rs;
        float ss = 0.0f;
        for (int64_t j = tid; j < N; j += nt) {
            const float f = D::one(xr[j]);
            ss = __builtin_fmaf(f, f, ss);
        }
        ss = segment_allreduce<64>(ss);
        if (lane == 0) part[par][wid] = ss;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
        for (int64_t j = tid; j < N; j += nt) {
            yr[j] = D::round1((D::one(xr[j]) * r) * (a.offset + D::one(w[j])));
        }
        if (tid == 0 && a.rstd != nullptr) store_rstd(a.rstd + batch() * M + row, r);
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Instance table.
// ---------------------------------------------------------------------------
#define RMS_WAVE_T(D, DT, L, V, S, P, T)                                                      \
    {RMSNORM_VARIANT_WAVE, DT, L, V, S, P, T,                                                     \
     reinterpret_cast<const void*>(&rmsnorm_wave<D, L, V, S, P, T>),                              \
     "rmsnorm_wave<" #D "," #L "," #V "," #S "," #P "," #T ">"}
#define RMS_WAVE(D, DT, L, V, S, P) RMS_WAVE_T(D, DT, L, V, S, P, true)
#define RMS_WAVE2(D, DT, L, V, S) RMS_WAVE(D, DT, L, V, S, false), RMS_WAVE(D, DT, L, V, S, true)
#define RMS_BLOCK_T(D, DT, V, P, T)                                                            \
    {RMSNORM_VARIANT_BLOCK, DT, 0, V, 1, P, T,                                                    \
     reinterpret_cast<const void*>(&rmsnorm_block<D, V, P, T>),                                   \
     "rmsnorm_block<" #D "," #V "," #P "," #T ">"}
#define RMS_BLOCK(D, DT, V, P) RMS_BLOCK_T(D, DT, V, P, true)
#define RMS_BLOCK2(D, DT, V) RMS_BLOCK(D, DT, V, false), RMS_BLOCK(D, DT, V, true)
#define RMS_WIDE(D, DT, V)                                                                     \
    {RMSNORM_VARIANT_WIDE, DT, 0, V, 1, false, true,                                              \
     reinterpret_cast<const void*>(&rmsnorm_wide<D, V>), "rmsnorm_wide<" #D "," #V ">"}
#define RMS_SHIFTED_P(D, DT, V, P)                                                             \
    {RMSNORM_VARIANT_SHIFTED, DT, 0, V, 1, P, true,                                               \
     reinterpret_cast<const void*>(&rmsnorm_shifted<D, V, P>), "rmsnorm_shifted<" #D "," #V "," #P ">"}
#define RMS_SHIFTED(D, DT, V) RMS_SHIFTED_P(D, DT, V, false), RMS_SHIFTED_P(D, DT, V, true)
#define RMS_SHIFTED_WAVE_P(D, DT, L, V, S, P)                                                  \
    {RMSNORM_VARIANT_SHIFTED_WAVE, DT, L, V, S, P, true,                                          \
     reinterpret_cast<const void*>(&rmsnorm_shifted_wave<D, L, V, S, P>),                         \
     "rmsnorm_shifted_wave<" #D "," #L "," #V "," #S "," #P ">"}
#define RMS_SHIFTED_WAVE(D, DT, L, V, S)                                                       \
    RMS_SHIFTED_WAVE_P(D, DT, L, V, S, false), RMS_SHIFTED_WAVE_P(D, DT, L, V, S, true)
// Only instances that fit 128 VGPRs (the budget of a 1024-thread workgroup)
// without scratch are compiled.  The widest forms leave out the tail path
// (last argument false), which they have no registers for: they serve
// widths that are a multiple of the vector.  Six vectors per lane fit only
// for fp32.
#define RMS_FAMILY(D, DT)                                                                      \
    RMS_WAVE2(D, DT, 4, 1, 1), RMS_WAVE2(D, DT, 4, 1, 2), RMS_WAVE2(D, DT, 4, 1, 4),            \
    RMS_WAVE2(D, DT, 8, 1, 1), RMS_WAVE2(D, DT, 8, 1, 2), RMS_WAVE2(D, DT, 8, 1, 4),            \
    RMS_WAVE2(D, DT, 16, 1, 1), RMS_WAVE2(D, DT, 16, 1, 2), RMS_WAVE2(D, DT, 16, 1, 4),         \
    RMS_WAVE2(D, DT, 32, 1, 1), RMS_WAVE2(D, DT, 32, 1, 2), RMS_WAVE2(D, DT, 32, 1, 4),         \
    RMS_WAVE_T(D, DT, 32, 2, 4, false, false),                                                  \
    RMS_WAVE2(D, DT, 64, 1, 1), RMS_WAVE2(D, DT, 64, 1, 2), RMS_WAVE2(D, DT, 64, 1, 4),         \
    RMS_WAVE_T(D, DT, 64, 1, 8, false, false), RMS_WAVE_T(D, DT, 64, 1, 8, true, false),        \
    RMS_WAVE2(D, DT, 64, 2, 1), RMS_WAVE2(D, DT, 64, 2, 2), RMS_WAVE_T(D, DT, 64, 2, 4, false, false), \
    RMS_WAVE2(D, DT, 64, 3, 1), RMS_WAVE_T(D, DT, 64, 3, 2, false, false), RMS_WAVE(D, DT, 64, 3, 2, true), \
    RMS_WAVE2(D, DT, 64, 4, 1), RMS_WAVE2(D, DT, 64, 5, 1),                                     \
    RMS_BLOCK2(D, DT, 1), RMS_BLOCK2(D, DT, 2), RMS_BLOCK2(D, DT, 3), RMS_BLOCK2(D, DT, 4),     \
    RMS_BLOCK(D, DT, 5, false),                                                                 \
    RMS_WIDE(D, DT, 2), RMS_WIDE(D, DT, 4),                                                     \
    RMS_SHIFTED(D, DT, 1), RMS_SHIFTED(D, DT, 2), RMS_SHIFTED(D, DT, 3), RMS_SHIFTED(D, DT, 4),   \
    RMS_SHIFTED_WAVE(D, DT, 8, 1, 1), RMS_SHIFTED_WAVE(D, DT, 8, 1, 2), RMS_SHIFTED_WAVE(D, DT, 8, 1, 4), \
    RMS_SHIFTED_WAVE(D, DT, 16, 1, 1), RMS_SHIFTED_WAVE(D, DT, 16, 1, 2), RMS_SHIFTED_WAVE(D, DT, 16, 1, 4), \
    RMS_SHIFTED_WAVE(D, DT, 32, 1, 1), RMS_SHIFTED_WAVE(D, DT, 32, 1, 2), RMS_SHIFTED_WAVE(D, DT, 32, 1, 4), \
    RMS_SHIFTED_WAVE(D, DT, 64, 1, 1), RMS_SHIFTED_WAVE(D, DT, 64, 1, 2), RMS_SHIFTED_WAVE(D, DT, 64, 1, 4), \
    RMS_SHIFTED_WAVE(D, DT, 64, 2, 1), RMS_SHIFTED_WAVE(D, DT, 64, 2, 2),                         \
    RMS_SHIFTED_WAVE_P(D, DT, 64, 2, 4, false),                                                  \
    {RMSNORM_VARIANT_GENERIC, DT, 0, 0, 1, false, true,                                         \
     reinterpret_cast<const void*>(&rmsnorm_generic<D>), "rmsnorm_generic<" #D ">"}

namespace rmsnorm_impl {

static const KernelEntry kTable[] = {
    RMS_FAMILY(BF16, RMSNORM_BF16),
    RMS_FAMILY(FP16, RMSNORM_FP16),
    RMS_FAMILY(F32, RMSNORM_FP32),
    RMS_BLOCK_T(F32, RMSNORM_FP32, 6, false, false),   // six vectors per thread: fp32 only (no widening
    RMS_WAVE_T(F32, RMSNORM_FP32, 64, 6, 1, false, false),   // registers)
};

const KernelEntry* kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

// The exact-width wave forms: the shapes and workgroup sizes the wave rule
// picks for rows of exactly 4, 8, 16, 32, 64 and 128 vectors (32 to 1024
// 16-bit elements; 16 to 512 fp32 ones).
struct ExactEntry {
    KernelEntry k;
    int threads;
};
#define RMS_WAVE_EXACT(D, DT, L, V, S, W)                                                      \
    {{RMSNORM_VARIANT_WAVE, DT, L, V, S, false, false,                                            \
      reinterpret_cast<const void*>(&rmsnorm_wave_exact<D, L, V, S, W>),                           \
      "rmsnorm_wave_exact<" #D "," #L "," #V "," #S "," #W ">"},                                   \
     (W) * 64}
#define RMS_EXACT_FAMILY(D, DT)                                                                \
    RMS_WAVE_EXACT(D, DT, 4, 1, 4, 2), RMS_WAVE_EXACT(D, DT, 8, 1, 2, 2),                       \
    RMS_WAVE_EXACT(D, DT, 16, 1, 2, 2), RMS_WAVE_EXACT(D, DT, 32, 1, 2, 2),                     \
    RMS_WAVE_EXACT(D, DT, 64, 1, 4, 4), RMS_WAVE_EXACT(D, DT, 64, 2, 2, 4),                     \
    RMS_WAVE_EXACT(D, DT, 32, 2, 4, 4)

static const ExactEntry kExactTable[] = {
    RMS_EXACT_FAMILY(BF16, RMSNORM_BF16),
    RMS_EXACT_FAMILY(FP16, RMSNORM_FP16),
    RMS_EXACT_FAMILY(F32, RMSNORM_FP32),
};

// The exact-width block forms: 256 threads x 8 vectors (16-bit rows of 16384
// elements) and 256 threads x 4 vectors (16-bit rows of 8192, fp32 rows of 4096).
#define RMS_BLOCK_EXACT(D, DT, V, T)                                                           \
    {RMSNORM_VARIANT_BLOCK, DT, 0, V, 1, false, false,                                            \
     reinterpret_cast<const void*>(&rmsnorm_block_exact<D, V, T>),                                \
     "rmsnorm_block_exact<" #D "," #V "," #T ">"}

static const ExactEntry kExactBlockTable[] = {
    {RMS_BLOCK_EXACT(BF16, RMSNORM_BF16, 8, 256), 256},
    {RMS_BLOCK_EXACT(FP16, RMSNORM_FP16, 8, 256), 256},
    {RMS_BLOCK_EXACT(BF16, RMSNORM_BF16, 4, 256), 256},
    {RMS_BLOCK_EXACT(FP16, RMSNORM_FP16, 4, 256), 256},
    {RMS_BLOCK_EXACT(F32, RMSNORM_FP32, 4, 256), 256},
};

const KernelEntry* exact_block_kernel(int dtype, int vpt, int threads) {
    for (const ExactEntry& e : kExactBlockTable)
        if (e.k.dtype == dtype && e.k.vectors_per_lane == vpt && e.threads == threads) return &e.k;
    return nullptr;
}

const KernelEntry* exact_wave_kernel(int dtype, int lanes, int vpl, int slots, int threads) {
    for (const ExactEntry& e : kExactTable)
        if (e.k.dtype == dtype && e.k.lanes_per_row == lanes && e.k.vectors_per_lane == vpl &&
            e.k.row_slots == slots && e.threads == threads)
            return &e.k;
    return nullptr;
}

}  // namespace rmsnorm_impl
