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

template <class D>
__device__ __forceinline__ void load_weights(float (&we)[8], const u32x4* w, int c, bool ok, float offset) {
    if (ok) {
        const u32x4 q = w[c];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            we[2 * k] = offset + D::lo(q[k]);
            we[2 * k + 1] = offset + D::hi(q[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) we[k] = 0.0f;
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

}  // namespace

// ---------------------------------------------------------------------------
// Wave family.
// ---------------------------------------------------------------------------
template <class D, int LANES, int VPL, int SLOTS>
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
    const int wpb = blockDim.x >> 6;
    // the wave's index is the same in all its lanes: keep it in a scalar register
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t wave0 = static_cast<int64_t>(blockIdx.x) * wpb + wid;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * wpb;

    float we[VPL][8];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        load_weights<D>(we[v], w, c, c < nvec, a.offset);
    }

    for (int64_t g = wave0; g * ROWS < M; g += nwaves) {
        const int64_t row0 = g * ROWS + seg;
        u32x4 d[SLOTS][VPL];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = row0 + s * SEG;
            const u32x4* xr = x + row * nvec;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                if (row < M && c < nvec) d[s][v] = xr[c];
                else d[s][v] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        float r[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const float ss = segment_allreduce<LANES>(sum_squares<D, VPL>(d[s]));
            r[s] = rsq(__builtin_fmaf(ss, a.inv_n, a.eps));
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = row0 + s * SEG;
            if (li == 0 && row < M) rstd[row] = r[s];
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = row0 + s * SEG;
            u32x4* yr = y + row * nvec;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                if (row < M && c < nvec) yr[c] = normalise<D>(d[s][v], we[v], r[s]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Block family.
// ---------------------------------------------------------------------------
template <class D, int VPT>
__global__ __launch_bounds__(1024) void rmsnorm_block(KernelArgs a) {
    __shared__ float part[2][16];
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    u32x4* __restrict__ y = static_cast<u32x4*>(a.y);
    float* __restrict__ rstd = a.rstd;
    const int64_t M = a.M;
    const int nvec = static_cast<int>(a.N >> 3);
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    float we[VPT][8];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        load_weights<D>(we[v], w, c, c < nvec, a.offset);
    }

    int par = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        u32x4 d[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            if (c < nvec) d[v] = x[row * nvec + c];
            else d[v] = u32x4{0u, 0u, 0u, 0u};
        }
        const float ss = segment_allreduce<64>(sum_squares<D, VPT>(d));
        if (lane == 0) part[par][wid] = ss;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r = rsq(__builtin_fmaf(tot, a.inv_n, a.eps));
        if (tid == 0) rstd[row] = r;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            if (c < nvec) y[row * nvec + c] = normalise<D>(d[v], we[v], r);
        }
        par ^= 1;
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
    const int nt = blockDim.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    int par = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
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
        if (tid == 0) a.rstd[row] = r;
        for (int64_t j = tid; j < N; j += nt) {
            yr[j] = D::round1((D::one(xr[j]) * r) * (a.offset + D::one(w[j])));
        }
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Instance table.
// ---------------------------------------------------------------------------
#define RMS_WAVE(D, DT, L, V, S)                                                           \
    {RMSNORM_VARIANT_WAVE, DT, L, V, S, reinterpret_cast<const void*>(&rmsnorm_wave<D, L, V, S>), \
     "rmsnorm_wave<" #D "," #L "," #V "," #S ">"}
#define RMS_WAVE_SLOTS4(D, DT, L, V) \
    RMS_WAVE(D, DT, L, V, 1), RMS_WAVE(D, DT, L, V, 2), RMS_WAVE(D, DT, L, V, 4), RMS_WAVE(D, DT, L, V, 8)
#define RMS_BLOCK(D, DT, V)                                                                  \
    {RMSNORM_VARIANT_BLOCK, DT, 0, V, 1, reinterpret_cast<const void*>(&rmsnorm_block<D, V>), \
     "rmsnorm_block<" #D "," #V ">"}
#define RMS_FAMILY(D, DT)                                                                      \
    RMS_WAVE_SLOTS4(D, DT, 16, 1), RMS_WAVE_SLOTS4(D, DT, 32, 1), RMS_WAVE_SLOTS4(D, DT, 64, 1), \
    RMS_WAVE(D, DT, 64, 2, 1), RMS_WAVE(D, DT, 64, 2, 2), RMS_WAVE(D, DT, 64, 2, 4),            \
    RMS_WAVE(D, DT, 64, 3, 1), RMS_WAVE(D, DT, 64, 3, 2),                                       \
    RMS_WAVE(D, DT, 64, 4, 1), RMS_WAVE(D, DT, 64, 4, 2),                                       \
    RMS_WAVE(D, DT, 64, 5, 1), RMS_WAVE(D, DT, 64, 6, 1),                                      \
    RMS_BLOCK(D, DT, 1), RMS_BLOCK(D, DT, 2), RMS_BLOCK(D, DT, 3), RMS_BLOCK(D, DT, 4),         \
    RMS_BLOCK(D, DT, 5), RMS_BLOCK(D, DT, 6),                                                   \
    {RMSNORM_VARIANT_GENERIC, DT, 0, 0, 1, reinterpret_cast<const void*>(&rmsnorm_generic<D>),  \
     "rmsnorm_generic<" #D ">"}

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
