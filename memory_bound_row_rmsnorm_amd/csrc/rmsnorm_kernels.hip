// rmsnorm_kernels.hip -- row RMSNorm forward kernels for gfx950 (MI355X).
//
// Per row m:  rstd[m] = rsqrt(sum_j x[m,j]^2 * (1/N) + eps)
//             y[m,j]  = x[m,j] * rstd[m] * (offset + w[j])
// ("Rmsnorm Kernel Optimization", Overview and Core Technique; "Why cutile's
// rmsnorm required full register", kernel listing of the opening report).
//
// All arithmetic is fp32; x, w and y are bf16 or fp16.  Three families:
//
//  * rmsnorm_wave   -- a row lives in a segment of 16, 32 or 64 lanes of one
//    wavefront, each lane holding VPL 16-byte vectors of it; a wave carries
//    SLOTS x (64 / LANES) rows per trip and issues every load of the trip
//    before its first reduction.  Reductions are DPP and v_readlane only, no
//    LDS.  Several rows per wave for small hidden sizes follows "Rmsnorm
//    Kernel Optimization", Key Optimizations.
//  * rmsnorm_block  -- one row per workgroup per trip, each thread holding VPT
//    16-byte vectors; wave sums meet in LDS behind one barrier per trip
//    (double-buffered partials).  For large N.
//  * rmsnorm_generic -- any N and any alignment, 2-byte accesses, the row read
//    a second time (from cache) to normalise.  Correctness fallback.
//
// Each family loops over rows with a grid stride, so a grid smaller than the
// row count is a persistent grid that keeps offset + w in registers across
// trips (the static persistent schedule of the cuTile listing, re-expressed
// for wave64 and the 256-CU chip).  Columns at or past N are never loaded or
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
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = D::lo(d[v][k]);
            const float b = D::hi(d[v][k]);
            ss = __builtin_fmaf(a, a, ss);
            ss = __builtin_fmaf(b, b, ss);
        }
    }
    return ss;
}

// offset + w for the 8 columns of one 16-byte weight vector (fp32, as the
// listing forms offset + w after widening w).
template <class D>
__device__ __forceinline__ void widen_weights(float (&we)[8], const u32x4 q, float offset) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        we[2 * k] = offset + D::lo(q[k]);
        we[2 * k + 1] = offset + D::hi(q[k]);
    }
}

template <class D>
__device__ __forceinline__ u32x4 normalise(const u32x4 q, const float (&we)[8], float r) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o[k] = D::pack((D::lo(q[k]) * r) * we[2 * k], (D::hi(q[k]) * r) * we[2 * k + 1]);
    }
    return o;
}

constexpr u32x4 kZero = {0u, 0u, 0u, 0u};

// The dispatcher hands workgroup b to XCD b mod 8 (MI355X has 8 XCDs, each
// with its own L2).  With group g > 1 the workgroup index is remapped inside
// windows of 8 * g workgroups so that XCD x serves g consecutive row groups,
// (b mod 8) * g + (b / 8) mod g within the window: a transpose of the window,
// so every index in [0, G) is still used exactly once (a tail shorter
// than a window keeps its own order).  Consecutive rows then share an L2 and
// reach HBM as longer runs of neighbouring addresses; measured on MI355X it
// shortens the 32768 x 8192 forward by 4-5%.
// (32-bit arithmetic: grids stay below 2^31 workgroups and windows below 2^10.)
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
template <class D, int LANES, int VPL, int SLOTS, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_wave(KernelArgs a) {
    constexpr int SEG = 64 / LANES;       // rows per slot
    constexpr int ROWS = SEG * SLOTS;     // rows per wave per trip
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = static_cast<u32x4*>(a.y);
    float* __restrict__ rstd = a.rstd;
    const int64_t M = a.M;
    const int nvec = static_cast<int>(a.N >> 3);
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int wpb = a.threads >> 6;
    // the wave's index is the same in all its lanes: keep it in a scalar register
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t nwaves = a.grid * wpb;
    int64_t g = grouped_block(a.xcd_group, a.grid) * wpb + wid;
    if (g * ROWS >= M) return;

    auto load_trip = [&](u32x4 (&d)[SLOTS][VPL], int64_t gg) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            const u32x4* xr = x + row * nvec;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                d[s][v] = (row < M && c < nvec) ? load_x(xr + c) : kZero;
            }
        }
    };

    u32x4 d[SLOTS][VPL];
    load_trip(d, g);
    float we[VPL][8];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        widen_weights<D>(we[v], c < nvec ? w[c] : kZero, a.offset);
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
            u32x4* yr = y + row * nvec;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                if (row < M && c < nvec) store_y(yr + c, normalise<D>(dd[s][v], we[v], r[s]));
            }
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            if (li == 0 && row < M) store_rstd(rstd + row, r[s]);
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
// Block family.
//
// Thread t of a workgroup of T threads holds the 16-byte vectors v * T + t,
// v < VPT, of one row.  Wave sums meet in LDS: one barrier per row, with the
// partials double-buffered so the next row's writes cannot race this row's
// reads (a wave can be at most one barrier ahead of another).  With PREFETCH
// the next row is loaded before this row's reduction.
// ---------------------------------------------------------------------------
template <class D, int VPT, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_block(KernelArgs a) {
    __shared__ float part[2][16];
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = static_cast<u32x4*>(a.y);
    float* __restrict__ rstd = a.rstd;
    const int64_t M = a.M;
    const int nvec = static_cast<int>(a.N >> 3);
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;
    int64_t row = grouped_block(a.xcd_group, a.grid);
    if (row >= M) return;

    auto load_row = [&](u32x4 (&d)[VPT], int64_t rr) {
        const u32x4* xr = x + rr * nvec;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            d[v] = c < nvec ? load_x(xr + c) : kZero;
        }
    };

    u32x4 d[VPT];
    load_row(d, row);
    float we[VPT][8];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        widen_weights<D>(we[v], c < nvec ? w[c] : kZero, a.offset);
    }

    // the row's reduction (wave butterfly, then the waves' sums through LDS),
    // every y store, then rstd
    auto finish_row = [&](const u32x4 (&dd)[VPT], int64_t rr, int pp) {
        const float ss = segment_allreduce<64>(sum_squares<D, VPT>(dd));
        if (lane == 0) part[pp][wid] = ss;
        __syncthreads();
        float tot = part[pp][0];
        for (int i = 1; i < nw; ++i) tot += part[pp][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
        u32x4* yr = y + rr * nvec;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            if (c < nvec) store_y(yr + c, normalise<D>(dd[v], we[v], r));
        }
        if (tid == 0) store_rstd(rstd + rr, r);
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
// Generic family: any N, any 2-byte alignment.  x and y may be the same
// buffer: every element is read and then written by the same thread, and the
// sum of squares of a row is complete (barrier) before any of it is written.
// ---------------------------------------------------------------------------
template <class D>
__global__ __launch_bounds__(1024) void rmsnorm_generic(KernelArgs a) {
    __shared__ float part[2][16];
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* __restrict__ w = static_cast<const uint16_t*>(a.w);
    uint16_t* y = static_cast<uint16_t*>(a.y);
    const int64_t M = a.M;
    const int64_t N = a.N;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    int par = 0;
    for (int64_t row = grouped_block(a.xcd_group, a.grid); row < M; row += a.grid) {
        const uint16_t* xr = x + row * N;
        uint16_t* yr = y + row * N;
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
        if (tid == 0) store_rstd(a.rstd + row, r);
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Instance table.
// ---------------------------------------------------------------------------
#define RMS_WAVE(D, DT, L, V, S, P)                                                           \
    {RMSNORM_VARIANT_WAVE, DT, L, V, S, P,                                                        \
     reinterpret_cast<const void*>(&rmsnorm_wave<D, L, V, S, P>),                                 \
     "rmsnorm_wave<" #D "," #L "," #V "," #S "," #P ">"}
#define RMS_WAVE2(D, DT, L, V, S) RMS_WAVE(D, DT, L, V, S, false), RMS_WAVE(D, DT, L, V, S, true)
#define RMS_BLOCK(D, DT, V, P)                                                                  \
    {RMSNORM_VARIANT_BLOCK, DT, 0, V, 1, P, reinterpret_cast<const void*>(&rmsnorm_block<D, V, P>), \
     "rmsnorm_block<" #D "," #V "," #P ">"}
#define RMS_BLOCK2(D, DT, V) RMS_BLOCK(D, DT, V, false), RMS_BLOCK(D, DT, V, true)
// Only instances that fit 128 VGPRs (the budget of a 1024-thread workgroup)
// without scratch are compiled.
#define RMS_FAMILY(D, DT)                                                                      \
    RMS_WAVE2(D, DT, 16, 1, 1), RMS_WAVE2(D, DT, 16, 1, 2), RMS_WAVE2(D, DT, 16, 1, 4),         \
    RMS_WAVE2(D, DT, 32, 1, 1), RMS_WAVE2(D, DT, 32, 1, 2), RMS_WAVE2(D, DT, 32, 1, 4),         \
    RMS_WAVE2(D, DT, 64, 1, 1), RMS_WAVE2(D, DT, 64, 1, 2), RMS_WAVE2(D, DT, 64, 1, 4),         \
    RMS_WAVE2(D, DT, 64, 1, 8),                                                                 \
    RMS_WAVE2(D, DT, 64, 2, 1), RMS_WAVE2(D, DT, 64, 2, 2), RMS_WAVE(D, DT, 64, 2, 4, false),   \
    RMS_WAVE2(D, DT, 64, 3, 1), RMS_WAVE2(D, DT, 64, 3, 2),                                     \
    RMS_WAVE2(D, DT, 64, 4, 1), RMS_WAVE2(D, DT, 64, 5, 1), RMS_WAVE(D, DT, 64, 6, 1, false),   \
    RMS_BLOCK2(D, DT, 1), RMS_BLOCK2(D, DT, 2), RMS_BLOCK2(D, DT, 3), RMS_BLOCK2(D, DT, 4),     \
    RMS_BLOCK2(D, DT, 5), RMS_BLOCK(D, DT, 6, false),                                           \
    {RMSNORM_VARIANT_GENERIC, DT, 0, 0, 1, false,                                               \
     reinterpret_cast<const void*>(&rmsnorm_generic<D>), "rmsnorm_generic<" #D ">"}

namespace rmsnorm_impl {

static const KernelEntry kTable[] = {
    RMS_FAMILY(BF16, RMSNORM_BF16),
    RMS_FAMILY(FP16, RMSNORM_FP16),
};

const KernelEntry* kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

}  // namespace rmsnorm_impl
