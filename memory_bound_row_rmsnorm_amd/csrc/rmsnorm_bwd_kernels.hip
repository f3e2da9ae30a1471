// rmsnorm_bwd_kernels.hip -- row RMSNorm backward for gfx950 (MI355X).
//
// The pages keep the forward's per-row rstd "for backward" ("Why cutile's
// rmsnorm required full register", kernel listing) but give no formula.
// Differentiating y_j = x_j r (offset + w_j), r = (mean_j x_j^2 + eps)^(-1/2):
//
//     g_j      = offset + w_j
//     c[m]     = (1/N) sum_j dy[m,j] g_j x[m,j]
//     dx[m,k]  = r (g_k dy[m,k] - r^2 c[m] x[m,k])
//     dw[j]    = sum_m dy[m,j] x[m,j] r[m]
//
// All arithmetic is fp32; x, w, dy and dx are bf16, fp16 or fp32 (D: eight
// 16-bit or four fp32 elements per 16-byte vector), rstd and dw fp32.
//
// Two passes.  The row pass runs a grid of G workgroups that loop over rows
// (a persistent grid: each workgroup keeps its columns' share of dw in
// registers across all of its rows) and writes one fp32 partial row of dw
// per workgroup to a workspace [G, N].  The column pass sums the G partial
// rows in a fixed order, so dw does not depend on timing.  The row pass has
// the forward's two shapes: rows inside 8/16/32/64-lane wave segments for
// N <= 1024 (partials of the segments and waves that share columns are
// added in LDS at the end), and one row per workgroup for larger N (each
// thread owns distinct columns, so its partial goes straight out).  A
// generic kernel takes any N and alignment.
#include "rmsnorm_device.hpp"
#include "rmsnorm_internal.hpp"
#include "../../include/rmsnorm.h"

#include <mutex>

using namespace rmsnorm_dev;
using rmsnorm_impl::BwdArgs;

namespace {

constexpr u32x4 kZero = {0u, 0u, 0u, 0u};

__device__ __forceinline__ u32x4 stream_load(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void stream_store(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// sum over this lane's D::EPV columns of one vector of dy * g * x
template <class D>
__device__ __forceinline__ float dot_dgx(const u32x4 dq, const u32x4 xq, const float (&g)[D::EPV], float acc) {
    float d[D::EPV], xv[D::EPV];
    D::widen(dq, d);
    D::widen(xq, xv);
#pragma unroll
    for (int k = 0; k < D::EPV; ++k) acc = __builtin_fmaf(d[k] * g[k], xv[k], acc);
    return acc;
}

// dx for one vector, and dw partials += dy * x * r
template <class D>
__device__ __forceinline__ u32x4 grad_vector(const u32x4 dq, const u32x4 xq, const float (&g)[D::EPV], float r,
                                             float r2c, float (&dwp)[D::EPV]) {
    float d[D::EPV], xv[D::EPV], o[D::EPV];
    D::widen(dq, d);
    D::widen(xq, xv);
#pragma unroll
    for (int k = 0; k < D::EPV; ++k) {
        o[k] = r * (g[k] * d[k] - r2c * xv[k]);
        dwp[k] = __builtin_fmaf(d[k] * xv[k], r, dwp[k]);
    }
    return D::narrow(o);
}

// offset + w widened from one packed 16-byte weight vector, at the point of
// use (the block family keeps w packed: 4 VGPRs per vector instead of 8)
template <class D>
__device__ __forceinline__ void widen_g(float (&g)[D::EPV], const u32x4 q, float offset) {
    D::widen(q, g);
#pragma unroll
    for (int k = 0; k < D::EPV; ++k) g[k] = offset + g[k];
}

// Element offsets of row m of x, dy and dx (see BwdArgs): one 32-bit
// division when the rows form several batches, none otherwise.
struct RowOff {
    int64_t x, dy, dx;
};

__device__ __forceinline__ RowOff row_offsets(const BwdArgs& a, int64_t m) {
    if (a.rows >= a.M) return {m * a.x_rs, m * a.dy_rs, m * a.dx_rs};
    const uint32_t b = static_cast<uint32_t>(m) / static_cast<uint32_t>(a.rows);
    const int64_t s = static_cast<int64_t>(static_cast<uint32_t>(m) - b * static_cast<uint32_t>(a.rows));
    const int64_t bb = b;
    return {bb * a.x_bs + s * a.x_rs, bb * a.dy_bs + s * a.dy_rs, bb * a.dx_bs + s * a.dx_rs};
}

// 16-byte vector at element offset off (a multiple of EPV in the vector kernels)
template <class D, class T>
__device__ __forceinline__ T* vec_at(T* base, int64_t off) {
    return base + static_cast<uint64_t>(off) / D::EPV;
}

}  // namespace

// ---------------------------------------------------------------------------
// Row pass, wave family (N <= 1024).  Lane layout as in the forward wave
// kernel.  With PREFETCH the next trip's rows are loaded before this trip's
// reductions and stores (worth it when a wave makes more than one trip).
// Dynamic LDS: (waves per workgroup) x (64 / LANES) x N floats.
// ---------------------------------------------------------------------------
template <class D, int LANES, int VPL, int SLOTS, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_wave(BwdArgs a) {
    extern __shared__ float lds_part[];
    constexpr int SEG = 64 / LANES;
    constexpr int ROWS = SEG * SLOTS;
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const u32x4* __restrict__ dy = static_cast<const u32x4*>(a.dy);
    const float* __restrict__ rstd = a.rstd;
    u32x4* __restrict__ dx = static_cast<u32x4*>(a.dx);
    const int64_t M = a.M;
    const int N = static_cast<int>(a.N);
    const int nvec = N / D::EPV;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int wpb = a.threads >> 6;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t nwaves = a.grid * wpb;

    float g[VPL][D::EPV];
    float dwp[VPL][D::EPV];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        widen_g<D>(g[v], c < nvec ? w[c] : kZero, a.offset);
#pragma unroll
        for (int k = 0; k < D::EPV; ++k) dwp[v][k] = 0.0f;
    }

    auto load_trip = [&](u32x4 (&xd)[SLOTS][VPL], u32x4 (&dd)[SLOTS][VPL], float (&r)[SLOTS], int64_t gg) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            const bool live = row < M;
            const RowOff o = row_offsets(a, live ? row : 0);
            const u32x4* xr = vec_at<D>(x, o.x);
            const u32x4* dr = vec_at<D>(dy, o.dy);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                xd[s][v] = (live && c < nvec) ? stream_load(xr + c) : kZero;
                dd[s][v] = (live && c < nvec) ? stream_load(dr + c) : kZero;
            }
            r[s] = live ? rstd[row] : 0.0f;
        }
    };

    int64_t gi = static_cast<int64_t>(blockIdx.x) * wpb + wid;
    u32x4 xd[SLOTS][VPL], dd[SLOTS][VPL];
    float r[SLOTS];
    if (PREFETCH && gi * ROWS < M) load_trip(xd, dd, r, gi);
    while (gi * ROWS < M) {
        const int64_t gn = gi + nwaves;
        u32x4 xn[SLOTS][VPL], dn[SLOTS][VPL];
        float rn[SLOTS];
        if constexpr (PREFETCH) {
            if (gn * ROWS < M) load_trip(xn, dn, rn, gn);
        } else {
            load_trip(xd, dd, r, gi);
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            float t = 0.0f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) t = dot_dgx<D>(dd[s][v], xd[s][v], g[v], t);
            const float cm = segment_allreduce<LANES>(t) * a.inv_n;
            const float r2c = r[s] * r[s] * cm;
            const int64_t row = gi * ROWS + seg + s * SEG;
            u32x4* out = vec_at<D>(dx, row_offsets(a, row < M ? row : 0).dx);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                const u32x4 o = grad_vector<D>(dd[s][v], xd[s][v], g[v], r[s], r2c, dwp[v]);
                if (row < M && c < nvec) stream_store(out + c, o);
            }
        }
        gi = gn;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
                    xd[s][v] = xn[s][v];
                    dd[s][v] = dn[s][v];
                }
                r[s] = rn[s];
            }
        }
    }

    // partials of all segments of all waves cover the same columns: add them
    // in a fixed order through LDS, then one partial row per workgroup
    float* mine = lds_part + static_cast<int64_t>(wid * SEG + seg) * N;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        if (c < nvec) {
#pragma unroll
            for (int k = 0; k < D::EPV; ++k) mine[c * D::EPV + k] = dwp[v][k];
        }
    }
    __syncthreads();
    const int parts = wpb * SEG;
    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * N;
    for (int col = threadIdx.x; col < N; col += a.threads) {
        float acc = lds_part[col];
        for (int i = 1; i < parts; ++i) acc += lds_part[static_cast<int64_t>(i) * N + col];
        dst[col] = acc;
    }
}

// ---------------------------------------------------------------------------
// Row pass, block family (N > 1024): R rows per workgroup per trip, one per
// slot of T = threads / R threads, thread t of a slot holding vectors
// v * T + t of its row (with PREFETCH the next trip's rows are loaded before
// this trip's reductions); c is reduced across each slot's waves through LDS
// (double buffered, one barrier per trip); each thread's dw partial covers
// its own columns.  With one slot it is written straight to the workspace;
// with several, the slots' partials of the same columns are added in LDS in
// slot order first, so a workgroup still writes one partial row: R times
// fewer partial rows for the column pass at the same waves per CU.
// Dynamic LDS: (R - 1) x VPT x T x EPV floats.
// ---------------------------------------------------------------------------
template <class D, int VPT, bool PREFETCH, int R>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_block(BwdArgs a) {
    constexpr int EPV = D::EPV;
    __shared__ float part[2][16];
    extern __shared__ float lds_slot[];          // R > 1: [R - 1][VPT][EPV][T], slots 1 .. R - 1
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const u32x4* __restrict__ dy = static_cast<const u32x4*>(a.dy);
    const float* __restrict__ rstd = a.rstd;
    u32x4* __restrict__ dx = static_cast<u32x4*>(a.dx);
    const int64_t M = a.M;
    const int nvec = static_cast<int>(a.N / EPV);
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int T = nt / R;                        // threads per row
    const int q = R == 1 ? 0 : tid / T;          // slot
    const int t = R == 1 ? tid : tid - q * T;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wps = T >> 6;                      // waves per slot

    u32x4 wpk[VPT];                              // packed weights of this thread's vectors
    float dwp[VPT][EPV];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * T + t;
        wpk[v] = c < nvec ? w[c] : kZero;
#pragma unroll
        for (int k = 0; k < EPV; ++k) dwp[v][k] = 0.0f;
    }

    // the row of this slot in trip g; rows past the end load zeros and store nothing
    auto load_row = [&](u32x4 (&xd)[VPT], u32x4 (&dd)[VPT], float& r, int64_t g) {
        const int64_t rr = g * R + q;
        const bool live = rr < M;
        const RowOff o = row_offsets(a, live ? rr : 0);
        const u32x4* xr = vec_at<D>(x, o.x);
        const u32x4* dr = vec_at<D>(dy, o.dy);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * T + t;
            xd[v] = (live && c < nvec) ? stream_load(xr + c) : kZero;
            dd[v] = (live && c < nvec) ? stream_load(dr + c) : kZero;
        }
        r = live ? rstd[rr] : 0.0f;
    };

    int par = 0;
    int64_t g = blockIdx.x;
    u32x4 xd[VPT], dd[VPT];
    float r = 0.0f;
    if (PREFETCH && g * R < M) load_row(xd, dd, r, g);
    while (g * R < M) {
        const int64_t next = g + a.grid;
        u32x4 xn[VPT], dn[VPT];
        float rn = 0.0f;
        if constexpr (PREFETCH) {
            if (next * R < M) load_row(xn, dn, rn, next);
        } else {
            load_row(xd, dd, r, g);
        }
        float tsum = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float gw[EPV];
            widen_g<D>(gw, wpk[v], a.offset);
            tsum = dot_dgx<D>(dd[v], xd[v], gw, tsum);
        }
        tsum = segment_allreduce<64>(tsum);
        if (lane == 0) part[par][wid] = tsum;
        __syncthreads();
        float tot = part[par][q * wps];
        for (int i = 1; i < wps; ++i) tot += part[par][q * wps + i];
        const float r2c = r * r * (tot * a.inv_n);
        const int64_t row = g * R + q;
        u32x4* out = vec_at<D>(dx, row_offsets(a, row < M ? row : 0).dx);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * T + t;
            float gw[EPV];
            widen_g<D>(gw, wpk[v], a.offset);
            const u32x4 o = grad_vector<D>(dd[v], xd[v], gw, r, r2c, dwp[v]);
            if (row < M && c < nvec) stream_store(out + c, o);
        }
        par ^= 1;
        g = next;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                xd[v] = xn[v];
                dd[v] = dn[v];
            }
            r = rn;
        }
    }

    if constexpr (R > 1) {
        // slots 1 .. R - 1 hand their partials to slot 0, which adds them in slot order
        if (q > 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v)
#pragma unroll
                for (int k = 0; k < EPV; ++k) lds_slot[(((q - 1) * VPT + v) * EPV + k) * T + t] = dwp[v][k];
        }
        __syncthreads();
        if (q > 0) return;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
            for (int k = 0; k < EPV; ++k)
                for (int s2 = 1; s2 < R; ++s2) dwp[v][k] += lds_slot[(((s2 - 1) * VPT + v) * EPV + k) * T + t];
    }
    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * a.N;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * T + t;
        if (c < nvec) {
#pragma unroll
            for (int k = 0; k < EPV; ++k) dst[c * EPV + k] = dwp[v][k];
        }
    }
}

// ---------------------------------------------------------------------------
// Row pass, wide family: aligned rows too wide for x and dy to stay in a
// 1024-thread workgroup's registers next to dw (more than 2 vectors per
// thread).  One row per workgroup per trip, thread t owning vectors v * T + t
// as in the block family, but x and dy are not held: the first pass reads
// them (cached loads) and forms c, the second reads them again, from the
// caches (one row per compute unit in flight, at most 160 KiB of x and dy),
// and writes dx.  Each thread keeps dw for its VPT column vectors in
// registers across its rows.  dx may be dy: each element is read, then
// written, by one thread.
// ---------------------------------------------------------------------------
template <class D, int VPT>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_wide(BwdArgs a) {
    __shared__ float part[2][16];
    const u32x4* __restrict__ x = static_cast<const u32x4*>(a.x);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const u32x4* dy = static_cast<const u32x4*>(a.dy);
    const float* __restrict__ rstd = a.rstd;
    u32x4* dx = static_cast<u32x4*>(a.dx);
    const int64_t M = a.M;
    const int nvec = static_cast<int>(a.N / D::EPV);
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;

    u32x4 wq[VPT];
    float dwp[VPT][D::EPV];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        wq[v] = c < nvec ? w[c] : kZero;
#pragma unroll
        for (int k = 0; k < D::EPV; ++k) dwp[v][k] = 0.0f;
    }

    int par = 0;
    for (int64_t row = blockIdx.x; row < M; row += a.grid) {
        const RowOff o = row_offsets(a, row);
        const u32x4* xr = vec_at<D>(x, o.x);
        const u32x4* dr = vec_at<D>(dy, o.dy);
        const float r = rstd[row];
        float t = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            if (c < nvec) {
                float g[D::EPV];
                widen_g<D>(g, wq[v], a.offset);
                t = dot_dgx<D>(dr[c], xr[c], g, t);
            }
        }
        t = segment_allreduce<64>(t);
        if (lane == 0) part[par][wid] = t;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r2c = r * r * (tot * a.inv_n);
        u32x4* out = vec_at<D>(dx, o.dx);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            if (c < nvec) {
                float g[D::EPV];
                widen_g<D>(g, wq[v], a.offset);
                const u32x4 xq = stream_load(xr + c);
                const u32x4 dq = stream_load(dr + c);
                stream_store(out + c, grad_vector<D>(dq, xq, g, r, r2c, dwp[v]));
            }
        }
        par ^= 1;
    }

    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * a.N;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        if (c < nvec) {
#pragma unroll
            for (int k = 0; k < D::EPV; ++k) dst[c * D::EPV + k] = dwp[v][k];
        }
    }
}

// ---------------------------------------------------------------------------
// Row pass, shifted family: rows that do not start on a 16-byte boundary (N
// not a multiple of the vector, or bases past a boundary), one row per
// workgroup per trip, thread t holding chunks v * T + t.  The row is read as
// the aligned 16-byte chunks that cover it, as in the forward's shifted
// kernel (edge chunks read whole, their elements outside the row set to zero,
// stored element by element); c and dx are computed chunk by chunk with the
// weights funnel-shifted into the chunk frame.
//
// dw cannot be kept in the chunk frame: which columns a chunk holds moves with
// each row's distance `al` past a boundary.  Each thread keeps column vector
// c instead (columns c * EPV .. c * EPV + EPV - 1 on every row), whose
// products dy * x lie in chunk c from position al on and in chunk c + 1 below
// al.  Chunk c + 1's products come from the lane above (DPP wave shift) or,
// for a wave's last lane, from the next wave's first lane (the first wave's,
// one slot on, for the last wave) through LDS, written before the row's
// barrier.  The elements of w's last vector past the row are set to zero, so
// the weights of the masked elements are finite and add nothing to c.
// With PREFETCH the next row is loaded before this row's reduction.  x, dy
// and dx must sit the same distance past a boundary on every row; dx may be
// dy (in place: every element is read, then written, by one thread, and the
// neighbouring rows' elements of an edge chunk are read but never used).
// Dynamic LDS: none up to two chunks per thread; with three, each thread's
// dw column vectors (threads x 3 x EPV floats).
// ---------------------------------------------------------------------------
// acc[i] += r * (element i + al of the concatenation (cur, nxt)), for the
// wave-uniform al of one row: one branch, constant register indices.
template <int EPV>
__device__ __forceinline__ void add_columns(float (&acc)[EPV], const float (&cur)[EPV], const float (&nxt)[EPV],
                                            int al, float r) {
    switch (al) {
#define RMS_COLUMN_CASE(A)                                                                           \
        case A:                                                                                      \
            if constexpr (A < EPV) {                                                                 \
                _Pragma("unroll") for (int i = 0; i < EPV; ++i)                                      \
                    acc[i] = __builtin_fmaf(i + A < EPV ? cur[i + A] : nxt[i + A - EPV], r, acc[i]); \
            }                                                                                        \
            break;
        RMS_COLUMN_CASE(0) RMS_COLUMN_CASE(1) RMS_COLUMN_CASE(2) RMS_COLUMN_CASE(3)
        RMS_COLUMN_CASE(4) RMS_COLUMN_CASE(5) RMS_COLUMN_CASE(6) RMS_COLUMN_CASE(7)
#undef RMS_COLUMN_CASE
        default:
            break;
    }
}

template <class D, int VPT, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_shifted(BwdArgs a) {
    typedef typename D::elem_t E;
    constexpr int EPV = D::EPV;
    constexpr int H = EPV / 4;                   // float4 quarters of a column vector
    // Up to two chunks per thread, dw and both weight vectors of each chunk
    // stay in registers.  Three do not fit 128 VGPRs that way: then dw lives
    // in LDS (each thread reads and writes only its own columns) and w's
    // vector c - 1 comes from the lane below.
    constexpr bool LDS_DW = VPT >= 3;
    constexpr int VR = LDS_DW ? 1 : VPT;         // chunk sets held in registers (wlo, dwp)
    __shared__ float part[2][16];
    __shared__ float first[2][VPT][16][EPV];     // each wave's first lane's products dy * x
    __shared__ u32x4 wtop[LDS_DW ? VPT : 1][16]; // each wave's last lane's w vector, per chunk set
    extern __shared__ float4 lds_dw[];           // LDS_DW: [VPT][H][threads], each thread's dw columns
    const E* x = static_cast<const E*>(a.x);
    const E* dy = static_cast<const E*>(a.dy);
    E* dx = static_cast<E*>(a.dx);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const float* __restrict__ rstd = a.rstd;
    const int64_t M = a.M;
    const int n = static_cast<int>(a.N);         // at most 2048 chunks: 32-bit element indices
    const int nvec_w = (n + EPV - 1) / EPV;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = nt >> 6;

    // w vectors c - 1 and c of each chunk c (the same on every row); with
    // LDS_DW vector c - 1 comes from the lane below, or for a wave's first
    // lane from the last lane of the wave below (of the last wave, one chunk
    // set back, for wave 0)
    auto wvec = [&](int k) -> u32x4 {
        if (k < 0 || k >= nvec_w) return kZero;
        return k == nvec_w - 1 ? keep_row<D>(w[k], k * EPV, n) : w[k];
    };
    u32x4 whi[VPT], wlo[VR];
    float dwp[VR][EPV];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        whi[v] = wvec(c);
        if constexpr (LDS_DW) {
            if (lane == 63) wtop[v][wid] = whi[v];
#pragma unroll
            for (int h = 0; h < H; ++h) lds_dw[(v * H + h) * nt + tid] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        } else {
            wlo[v] = wvec(c - 1);
#pragma unroll
            for (int k = 0; k < EPV; ++k) dwp[v][k] = 0.0f;
        }
    }
    if constexpr (LDS_DW) __syncthreads();
    // offset + w in the chunk frame of a row al elements past a boundary
    auto weights = [&](float (&g)[EPV], int v, int al) {
        u32x4 q = whi[v];
        if (al != 0) {
            u32x4 lo;
            if constexpr (LDS_DW) {
                u32x4 below = kZero;
                if (lane == 0) {
                    if (wid > 0) below = wtop[v][wid - 1];
                    else if (v > 0) below = wtop[v > 0 ? v - 1 : 0][nw - 1];
                }
                lo = from_lane_below(whi[v], below);
            } else {
                lo = wlo[v < VR ? v : 0];
            }
            q = funnel<D>(lo, whi[v], EPV - al);
        }
        widen_g<D>(g, q, a.offset);
    };

    auto load_row = [&](u32x4 (&xd)[VPT], u32x4 (&dd)[VPT], float& r, int& al, int64_t rr) {
        const RowOff o = row_offsets(a, rr);
        al = __builtin_amdgcn_readfirstlane(
            static_cast<int>((reinterpret_cast<uintptr_t>(x + o.x) & 15u) / sizeof(E)));
        const u32x4* xc = reinterpret_cast<const u32x4*>(x + o.x - al);
        const u32x4* dc = reinterpret_cast<const u32x4*>(dy + o.dy - al);
        const int nch = (al + n + EPV - 1) / EPV;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            xd[v] = c < nch ? stream_load(xc + c) : kZero;
            dd[v] = c < nch ? stream_load(dc + c) : kZero;
        }
        r = rstd[rr];
    };

    int par = 0;
    int64_t row = blockIdx.x;
    u32x4 xd[VPT], dd[VPT];
    float r = 0.0f;
    int al = 0;
    if (PREFETCH && row < M) load_row(xd, dd, r, al, row);
    while (row < M) {
        const int64_t next = row + a.grid;
        u32x4 xn[VPT], dn[VPT];
        float rn = 0.0f;
        int aln = 0;
        if constexpr (PREFETCH) {
            if (next < M) load_row(xn, dn, rn, aln, next);
        } else {
            load_row(xd, dd, r, al, row);
        }
        const int nch = (al + n + EPV - 1) / EPV;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int j0 = (v * nt + tid) * EPV - al;
            if (j0 < 0 || j0 + EPV > n) {
                xd[v] = keep_row<D>(xd[v], j0, n);
                dd[v] = keep_row<D>(dd[v], j0, n);
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                float d[EPV], xv[EPV];
                D::widen(dd[v], d);
                D::widen(xd[v], xv);
#pragma unroll
                for (int k = 0; k < EPV; ++k) first[par][v][wid][k] = d[k] * xv[k];
            }
        }
        float t = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float g[EPV];
            weights(g, v, al);
            t = dot_dgx<D>(dd[v], xd[v], g, t);
        }
        t = segment_allreduce<64>(t);
        if (lane == 0) part[par][wid] = t;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r2c = r * r * (tot * a.inv_n);
        u32x4* oc = reinterpret_cast<u32x4*>(dx + row_offsets(a, row).dx - al);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = v * nt + tid;
            float g[EPV], d[EPV], xv[EPV], o[EPV], p[EPV], pn[EPV];
            weights(g, v, al);
            D::widen(dd[v], d);
            D::widen(xd[v], xv);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                o[k] = r * (g[k] * d[k] - r2c * xv[k]);
                p[k] = d[k] * xv[k];
            }
            if (c < nch) {
                const u32x4 ov = D::narrow(o);
                const int j0 = c * EPV - al;
                if (j0 < 0 || j0 + EPV > n) store_edge<D>(oc + c, ov, j0, n);
                else stream_store(oc + c, ov);
            }
            // chunk c + 1's products
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                float up = 0.0f;
                if (wid + 1 < nw) up = first[par][v][wid + 1][k];
                else if (v + 1 < VPT) up = first[par][v + 1 < VPT ? v + 1 : 0][0][k];
                pn[k] = from_lane_above(p[k], up);
            }
            if constexpr (LDS_DW) {
                float acc[EPV];
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const float4 q = lds_dw[(v * H + h) * nt + tid];
                    acc[4 * h] = q.x;
                    acc[4 * h + 1] = q.y;
                    acc[4 * h + 2] = q.z;
                    acc[4 * h + 3] = q.w;
                }
                add_columns<EPV>(acc, p, pn, al, r);
#pragma unroll
                for (int h = 0; h < H; ++h)
                    lds_dw[(v * H + h) * nt + tid] =
                        make_float4(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
            } else {
                add_columns<EPV>(dwp[v < VR ? v : 0], p, pn, al, r);
            }
        }
        par ^= 1;
        row = next;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                xd[v] = xn[v];
                dd[v] = dn[v];
            }
            r = rn;
            al = aln;
        }
    }

    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * n;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = v * nt + tid;
        if (c < nvec_w) {
            float e[EPV];
#pragma unroll
            for (int h = 0; h < H; ++h) {
                if constexpr (LDS_DW) {
                    const float4 q = lds_dw[(v * H + h) * nt + tid];
                    e[4 * h] = q.x;
                    e[4 * h + 1] = q.y;
                    e[4 * h + 2] = q.z;
                    e[4 * h + 3] = q.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) e[4 * h + j] = dwp[v < VR ? v : 0][4 * h + j];
                }
            }
#pragma unroll
            for (int k = 0; k < EPV; ++k)
                if (c * EPV + k < n) dst[c * EPV + k] = e[k];
        }
    }
}

// ---------------------------------------------------------------------------
// Row pass, shifted wave family: short rows off a 16-byte boundary (at most
// VPL * LANES chunks) with a row per segment of LANES lanes (8, 16, 32 or 64; two
// chunks per lane only with 64) and SLOTS slots of 64 / LANES rows per wave
// per trip; lane li of a segment holds chunks v * LANES + li of its row and
// keeps column vectors v * LANES + li of dw.  As in the shifted kernel the
// weights are funnel-shifted into each row's chunk frame and the products of
// chunk c + 1 come from the lane above; a segment's last lane takes them from
// its first lane's next chunk, or has none past the last chunk (its column
// vector's upper elements then lie past the row).  With 64 lanes a row's
// shift is uniform in its wave and both shifts branch on it; with several rows per wave every lane shifts by its own
// row's distance past a boundary (funnel_lane for the weights, a three-stage
// select for the products).  No barrier until the end, where the partials of
// the segments and waves are added in LDS in a fixed order, as in the wave
// family.  Dynamic LDS: (waves per workgroup) x (64 / LANES) x N floats.
// ---------------------------------------------------------------------------
// add_columns() for a shift that differs between lanes: the pair (cur, nxt)
// shifted down by al elements in stages of 4, 2 and 1 (whole-vector selects
// between a value and its shuffle, so the pair stays in registers), then
// acc[i] += r * element i.
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void add_columns_lane(float (&acc)[8], const float (&cur)[8], const float (&nxt)[8],
                                                 int al, float r) {
    f32x16 W = {cur[0], cur[1], cur[2], cur[3], cur[4], cur[5], cur[6], cur[7],
                nxt[0], nxt[1], nxt[2], nxt[3], nxt[4], nxt[5], nxt[6], nxt[7]};
    const f32x16 S4 = __builtin_shufflevector(W, W, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 15, 15, 15, 15);
    W = (al & 4) ? S4 : W;
    const f32x16 S2 = __builtin_shufflevector(W, W, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 15, 15);
    W = (al & 2) ? S2 : W;
    const f32x16 S1 = __builtin_shufflevector(W, W, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 15);
    W = (al & 1) ? S1 : W;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(W[i], r, acc[i]);
}

__device__ __forceinline__ void add_columns_lane(float (&acc)[4], const float (&cur)[4], const float (&nxt)[4],
                                                 int al, float r) {
    f32x8 W = {cur[0], cur[1], cur[2], cur[3], nxt[0], nxt[1], nxt[2], nxt[3]};
    const f32x8 S2 = __builtin_shufflevector(W, W, 2, 3, 4, 5, 6, 7, 7, 7);
    W = (al & 2) ? S2 : W;
    const f32x8 S1 = __builtin_shufflevector(W, W, 1, 2, 3, 4, 5, 6, 7, 7);
    W = (al & 1) ? S1 : W;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(W[i], r, acc[i]);
}

template <class D, int LANES, int VPL, int SLOTS, bool PREFETCH>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_shifted_wave(BwdArgs a) {
    static_assert(VPL == 1 || LANES == 64, "two chunks per lane only with a row per wave");
    typedef typename D::elem_t E;
    constexpr int EPV = D::EPV;
    constexpr int SEG = 64 / LANES;
    constexpr int ROWS = SEG * SLOTS;
    extern __shared__ float lds_part[];
    const E* x = static_cast<const E*>(a.x);
    const E* dy = static_cast<const E*>(a.dy);
    E* dx = static_cast<E*>(a.dx);
    const u32x4* __restrict__ w = static_cast<const u32x4*>(a.w);
    const float* __restrict__ rstd = a.rstd;
    const int64_t M = a.M;
    const int n = static_cast<int>(a.N);
    const int nvec_w = (n + EPV - 1) / EPV;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LANES;
    const int li = lane % LANES;
    const int wpb = a.threads >> 6;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t nwaves = a.grid * wpb;

    // lane li of a segment holds chunks v * LANES + li, v < VPL, and keeps
    // column vector v * LANES + li of dw
    auto wvec = [&](int k) -> u32x4 {
        if (k < 0 || k >= nvec_w) return kZero;
        return k == nvec_w - 1 ? keep_row<D>(w[k], k * EPV, n) : w[k];
    };
    u32x4 wlo[VPL], whi[VPL];
    float dwp[VPL][EPV];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        wlo[v] = wvec(v * LANES + li - 1);
        whi[v] = wvec(v * LANES + li);
#pragma unroll
        for (int k = 0; k < EPV; ++k) dwp[v][k] = 0.0f;
    }

    // distance of row m's start past a 16-byte boundary, in elements
    auto shift_of = [&](const E* p) -> int {
        const int s = static_cast<int>((reinterpret_cast<uintptr_t>(p) & 15u) / sizeof(E));
        if constexpr (LANES == 64) return __builtin_amdgcn_readfirstlane(s);
        else return s;
    };
    auto load_trip = [&](u32x4 (&xd)[SLOTS][VPL], u32x4 (&dd)[SLOTS][VPL], float (&r)[SLOTS], int (&al)[SLOTS],
                         int64_t gg) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gg * ROWS + seg + s * SEG;
            const bool live = row < M;
            const RowOff o = row_offsets(a, live ? row : 0);
            const int as = shift_of(x + o.x);
            const int nch = (as + n + EPV - 1) / EPV;
            const u32x4* xc = reinterpret_cast<const u32x4*>(x + o.x - as);
            const u32x4* dc = reinterpret_cast<const u32x4*>(dy + o.dy - as);
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int c = v * LANES + li;
                xd[s][v] = (live && c < nch) ? stream_load(xc + c) : kZero;
                dd[s][v] = (live && c < nch) ? stream_load(dc + c) : kZero;
            }
            r[s] = live ? rstd[row] : 0.0f;
            al[s] = as;
        }
    };

    int64_t gi = static_cast<int64_t>(blockIdx.x) * wpb + wid;
    u32x4 xd[SLOTS][VPL], dd[SLOTS][VPL];
    float r[SLOTS];
    int al[SLOTS];
    if (PREFETCH && gi * ROWS < M) load_trip(xd, dd, r, al, gi);
    while (gi * ROWS < M) {
        const int64_t gn = gi + nwaves;
        u32x4 xn[SLOTS][VPL], dn[SLOTS][VPL];
        float rn[SLOTS];
        int aln[SLOTS];
        if constexpr (PREFETCH) {
            if (gn * ROWS < M) load_trip(xn, dn, rn, aln, gn);
        } else {
            load_trip(xd, dd, r, al, gi);
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int64_t row = gi * ROWS + seg + s * SEG;
            const bool live = row < M;
            const int as = al[s];
            u32x4 xv4[VPL], dv4[VPL];
            float g[VPL][EPV];
            float t = 0.0f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int j0 = (v * LANES + li) * EPV - as;
                xv4[v] = xd[s][v];
                dv4[v] = dd[s][v];
                if (j0 < 0 || j0 + EPV > n) {
                    xv4[v] = keep_row<D>(xv4[v], j0, n);
                    dv4[v] = keep_row<D>(dv4[v], j0, n);
                }
                if constexpr (LANES == 64) widen_g<D>(g[v], funnel<D>(wlo[v], whi[v], EPV - as), a.offset);
                else widen_g<D>(g[v], funnel_lane<D>(wlo[v], whi[v], EPV - as), a.offset);
                t = dot_dgx<D>(dv4[v], xv4[v], g[v], t);
            }
            const float cm = segment_allreduce<LANES>(t) * a.inv_n;
            const float rs = r[s];
            const float r2c = rs * rs * cm;
            const int nch = (as + n + EPV - 1) / EPV;
            float p[VPL][EPV];
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                float d[EPV], xv[EPV], o[EPV];
                D::widen(dv4[v], d);
                D::widen(xv4[v], xv);
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    o[k] = rs * (g[v][k] * d[k] - r2c * xv[k]);
                    p[v][k] = d[k] * xv[k];
                }
                const int c = v * LANES + li;
                if (live && c < nch) {
                    u32x4* oc = reinterpret_cast<u32x4*>(dx + row_offsets(a, row).dx - as);
                    const u32x4 ov = D::narrow(o);
                    const int j0 = c * EPV - as;
                    if (j0 < 0 || j0 + EPV > n) store_edge<D>(oc + c, ov, j0, n);
                    else stream_store(oc + c, ov);
                }
            }
            // chunk c + 1's products: the lane above's, or for a segment's last
            // lane the first lane's next chunk (none past the last chunk)
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                float pn[EPV];
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    float wrap = 0.0f;
                    if constexpr (VPL > 1) {
                        if (v + 1 < VPL)
                            wrap = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                __builtin_bit_cast(int, p[v + 1 < VPL ? v + 1 : 0][k]), 0));
                    }
                    const float up = from_lane_above(p[v][k], wrap);
                    pn[k] = (LANES < 64 && li == LANES - 1) ? 0.0f : up;
                }
                if constexpr (LANES == 64) add_columns<EPV>(dwp[v], p[v], pn, as, rs);
                else add_columns_lane(dwp[v], p[v], pn, as, rs);
            }
        }
        gi = gn;
        if constexpr (PREFETCH) {
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) {
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
                    xd[s][v] = xn[s][v];
                    dd[s][v] = dn[s][v];
                }
                r[s] = rn[s];
                al[s] = aln[s];
            }
        }
    }

    // every segment of every wave holds column vectors 0 .. VPL * LANES - 1:
    // add them in a fixed order through LDS, then one partial row per workgroup
    float* mine = lds_part + static_cast<int64_t>(wid * SEG + seg) * n;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int c = v * LANES + li;
        if (c < nvec_w) {
#pragma unroll
            for (int k = 0; k < EPV; ++k)
                if (c * EPV + k < n) mine[c * EPV + k] = dwp[v][k];
        }
    }
    __syncthreads();
    const int parts = wpb * SEG;
    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * n;
    for (int col = threadIdx.x; col < n; col += a.threads) {
        float acc = lds_part[col];
        for (int i = 1; i < parts; ++i) acc += lds_part[static_cast<int64_t>(i) * n + col];
        dst[col] = acc;
    }
}

// ---------------------------------------------------------------------------
// Row pass, generic (any N and alignment): one row per workgroup per trip,
// element-wide accesses, the row read twice (c first, then dx), and the
// workgroup's partial row of dw updated in the workspace in place (each
// workgroup owns its own partial row, so no other workgroup touches it).
// dx may be the same buffer as dy: each element is read, then written, by
// the same thread, after the barrier that completes c.
// ---------------------------------------------------------------------------
template <class D>
__global__ __launch_bounds__(1024) void rmsnorm_bwd_generic(BwdArgs a) {
    __shared__ float part[2][16];
    typedef typename D::elem_t E;
    const E* x = static_cast<const E*>(a.x);
    const E* __restrict__ w = static_cast<const E*>(a.w);
    const E* dy = static_cast<const E*>(a.dy);
    E* dx = static_cast<E*>(a.dx);
    const int64_t M = a.M;
    const int64_t N = a.N;
    const int tid = threadIdx.x;
    const int nt = a.threads;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;
    float* dst = a.partials + static_cast<int64_t>(blockIdx.x) * N;
    for (int64_t j = tid; j < N; j += nt) dst[j] = 0.0f;

    int par = 0;
    for (int64_t row = blockIdx.x; row < M; row += a.grid) {
        const RowOff o = row_offsets(a, row);
        const E* xr = x + o.x;
        const E* dr = dy + o.dy;
        E* out = dx + o.dx;
        const float r = a.rstd[row];
        float t = 0.0f;
        for (int64_t j = tid; j < N; j += nt)
            t = __builtin_fmaf(D::one(dr[j]) * (a.offset + D::one(w[j])), D::one(xr[j]), t);
        t = segment_allreduce<64>(t);
        if (lane == 0) part[par][wid] = t;
        __syncthreads();
        float tot = part[par][0];
        for (int i = 1; i < nw; ++i) tot += part[par][i];
        const float r2c = r * r * (tot * a.inv_n);
        for (int64_t j = tid; j < N; j += nt) {
            const float d = D::one(dr[j]), xv = D::one(xr[j]);
            const float gj = a.offset + D::one(w[j]);
            dst[j] = __builtin_fmaf(d * xv, r, dst[j]);
            out[j] = D::round1(r * (gj * d - r2c * xv));
        }
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Column pass: dw[j] = sum over the G partial rows.  A workgroup covers COLS
// column groups (of 4 columns, or of 1) and splits the G partial rows SPLIT
// ways: thread (s, q) adds rows s, s + SPLIT, s + 2 SPLIT, ... of group q in
// that order; the SPLIT sub-sums then meet in LDS in a fixed order (groups of
// 8 in order, then the groups in order), so dw is the same on every run and
// for either COLS.  SPLIT = 64 gives every thread few rows: the partial rows
// were just written from other XCDs' caches, and each sequential round of
// loads costs a trip to memory.  COLS trades workgroups for width: measured
// on MI355X after a kernel that writes the partial rows, 4 groups per
// workgroup (256 threads) are faster up to 256 groups (G = 256, N = 512: 2.50
// against 2.88 us; N = 1024: 2.90 against 3.14 us) and 16 (1024 threads)
// above (N = 2048: 3.46 against 3.68 us; G = 512, N = 8192: 9.29 against
// 14.75 us).  With vec4 (N % 4 == 0 and dw 16-byte aligned; the workspace
// always is) columns move as float4, otherwise one column per lane of a group.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float4 add4(float4 a, const float4 b) {
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
    return a;
}

template <int SPLIT, int COLS>
__global__ __launch_bounds__(COLS * SPLIT) void rmsnorm_dw_reduce(const float* __restrict__ partials,
                                                                float* __restrict__ dw, int64_t G, int64_t N,
                                                                int32_t vec4) {
    static_assert(SPLIT == 16 || SPLIT == 64, "split 16 or 64");
    __shared__ float4 red[SPLIT][COLS];
    const int q = threadIdx.x % COLS;
    const int sp = threadIdx.x / COLS;
    // column blocks of COLS groups; a grid smaller than the blocks loops over
    // them (the same count in every thread of a workgroup: the barriers stay
    // uniform)
    const int64_t groups = vec4 ? N / 4 : N;
    const int64_t nblocks = (groups + COLS - 1) / COLS;
    for (int64_t cb = blockIdx.x; cb < nblocks; cb += gridDim.x) {
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const int64_t c = vec4 ? (cb * COLS + q) * 4 : cb * COLS + q;
        if (c < N) {
            if (vec4) {
#pragma unroll 4
                for (int64_t i = sp; i < G; i += SPLIT)
                    acc = add4(acc, *reinterpret_cast<const float4*>(partials + i * N + c));
            } else {
#pragma unroll 4
                for (int64_t i = sp; i < G; i += SPLIT) acc.x += partials[i * N + c];
            }
        }
        red[sp][q] = acc;
        __syncthreads();
        constexpr int GROUPS = SPLIT / 8;    // 2 or 8 groups of 8 sub-sums
        if (sp < GROUPS) {      // group sp reads and then overwrites only its own slots
            float4 t = red[sp * 8][q];
            for (int k = 1; k < 8; ++k) t = add4(t, red[sp * 8 + k][q]);
            red[sp * 8][q] = t;
        }
        __syncthreads();
        if (sp == 0 && c < N) {
            float4 t = red[0][q];
            for (int k = 1; k < GROUPS; ++k) t = add4(t, red[k * 8][q]);
            if (vec4) *reinterpret_cast<float4*>(dw + c) = t;
            else dw[c] = t.x;
        }
        __syncthreads();    // the next block's partial sums overwrite red
    }
}

// ---------------------------------------------------------------------------
// Instance table.
// ---------------------------------------------------------------------------
#define RMS_BWD_WAVE(D, DT, L, V, S, P)                                                        \
    {RMSNORM_VARIANT_WAVE, DT, L, V, S, P, false,                                                     \
     reinterpret_cast<const void*>(&rmsnorm_bwd_wave<D, L, V, S, P>),                          \
     "rmsnorm_bwd_wave<" #D "," #L "," #V "," #S "," #P ">"}
#define RMS_BWD_WAVE2(D, DT, L, V, S) RMS_BWD_WAVE(D, DT, L, V, S, false), RMS_BWD_WAVE(D, DT, L, V, S, true)
#define RMS_BWD_BLOCK_R(D, DT, V, R, P)                                                        \
    {RMSNORM_VARIANT_BLOCK, DT, 0, V, R, P, false,                                                    \
     reinterpret_cast<const void*>(&rmsnorm_bwd_block<D, V, P, R>),                            \
     "rmsnorm_bwd_block<" #D "," #V "," #P "," #R ">"}
#define RMS_BWD_BLOCK(D, DT, V, P) RMS_BWD_BLOCK_R(D, DT, V, 1, P)
#define RMS_BWD_WIDE(D, DT, V)                                                                 \
    {RMSNORM_VARIANT_WIDE, DT, 0, V, 1, false, false,                                                 \
     reinterpret_cast<const void*>(&rmsnorm_bwd_wide<D, V>), "rmsnorm_bwd_wide<" #D "," #V ">"}
#define RMS_BWD_SHIFTED(D, DT, V, P)                                                           \
    {RMSNORM_VARIANT_SHIFTED, DT, 0, V, 1, P, false,                                                  \
     reinterpret_cast<const void*>(&rmsnorm_bwd_shifted<D, V, P>),                             \
     "rmsnorm_bwd_shifted<" #D "," #V "," #P ">"}
#define RMS_BWD_SHIFTED_WAVE_V(D, DT, L, V, S, P)                                              \
    {RMSNORM_VARIANT_SHIFTED_WAVE, DT, L, V, S, P, false,                                             \
     reinterpret_cast<const void*>(&rmsnorm_bwd_shifted_wave<D, L, V, S, P>),                  \
     "rmsnorm_bwd_shifted_wave<" #D "," #L "," #V "," #S "," #P ">"}
#define RMS_BWD_SHIFTED_WAVE(D, DT, L, S, P) RMS_BWD_SHIFTED_WAVE_V(D, DT, L, 1, S, P)
#define RMS_BWD_SHIFTED_WAVE2(D, DT, L, S)                                                     \
    RMS_BWD_SHIFTED_WAVE(D, DT, L, S, false), RMS_BWD_SHIFTED_WAVE(D, DT, L, S, true)
// Only instances that fit 128 VGPRs without scratch: the block family holds
// at most two vectors of x and dy per thread (rows up to 1024 x 2 vectors:
// 16384 16-bit or 8192 fp32 elements), and the widest wave shapes, the
// 4-slot shifted wave shapes and the two-slot shifted wave shape of two
// chunks per lane have no prefetching form.  The wide family holds dw for up
// to 4 vectors per thread (rows up to 32768 16-bit elements), 6 with fp32
// (24576 elements).
#define RMS_BWD_FAMILY(D, DT)                                                                  \
    RMS_BWD_WAVE2(D, DT, 4, 1, 1), RMS_BWD_WAVE2(D, DT, 4, 1, 2),                              \
    RMS_BWD_WAVE2(D, DT, 8, 1, 1), RMS_BWD_WAVE2(D, DT, 8, 1, 2),                              \
    RMS_BWD_WAVE2(D, DT, 16, 1, 1), RMS_BWD_WAVE2(D, DT, 16, 1, 2),                            \
    RMS_BWD_WAVE2(D, DT, 32, 1, 1), RMS_BWD_WAVE2(D, DT, 32, 1, 2),                            \
    RMS_BWD_WAVE2(D, DT, 64, 1, 1), RMS_BWD_WAVE2(D, DT, 64, 1, 2),                            \
    RMS_BWD_WAVE(D, DT, 64, 1, 4, false), RMS_BWD_WAVE2(D, DT, 64, 2, 1),                      \
    RMS_BWD_WAVE(D, DT, 64, 2, 2, false),                                                      \
    RMS_BWD_BLOCK(D, DT, 1, false), RMS_BWD_BLOCK(D, DT, 1, true),                             \
    RMS_BWD_BLOCK(D, DT, 2, false), RMS_BWD_BLOCK(D, DT, 2, true),                             \
    RMS_BWD_BLOCK_R(D, DT, 1, 2, false), RMS_BWD_BLOCK_R(D, DT, 1, 2, true),                   \
    RMS_BWD_BLOCK_R(D, DT, 2, 2, false), RMS_BWD_BLOCK_R(D, DT, 2, 2, true),                   \
    RMS_BWD_BLOCK_R(D, DT, 1, 4, false), RMS_BWD_BLOCK_R(D, DT, 1, 4, true),                   \
    RMS_BWD_BLOCK_R(D, DT, 2, 4, false), RMS_BWD_BLOCK_R(D, DT, 2, 4, true),                   \
    RMS_BWD_WIDE(D, DT, 3), RMS_BWD_WIDE(D, DT, 4),                                            \
    RMS_BWD_SHIFTED(D, DT, 1, false), RMS_BWD_SHIFTED(D, DT, 1, true),                         \
    RMS_BWD_SHIFTED(D, DT, 2, false), RMS_BWD_SHIFTED(D, DT, 2, true),                         \
    RMS_BWD_SHIFTED(D, DT, 3, false),                                                          \
    RMS_BWD_SHIFTED_WAVE2(D, DT, 8, 1), RMS_BWD_SHIFTED_WAVE2(D, DT, 8, 2),                     \
    RMS_BWD_SHIFTED_WAVE2(D, DT, 16, 1), RMS_BWD_SHIFTED_WAVE2(D, DT, 16, 2),                   \
    RMS_BWD_SHIFTED_WAVE(D, DT, 16, 4, false), RMS_BWD_SHIFTED_WAVE2(D, DT, 32, 1),             \
    RMS_BWD_SHIFTED_WAVE2(D, DT, 32, 2), RMS_BWD_SHIFTED_WAVE(D, DT, 32, 4, false),             \
    RMS_BWD_SHIFTED_WAVE2(D, DT, 64, 1), RMS_BWD_SHIFTED_WAVE2(D, DT, 64, 2),                   \
    RMS_BWD_SHIFTED_WAVE(D, DT, 64, 4, false),                                                 \
    RMS_BWD_SHIFTED_WAVE_V(D, DT, 64, 2, 1, false), RMS_BWD_SHIFTED_WAVE_V(D, DT, 64, 2, 1, true), \
    RMS_BWD_SHIFTED_WAVE_V(D, DT, 64, 2, 2, false),                                            \
    {RMSNORM_VARIANT_GENERIC, DT, 0, 0, 1, false, false,                                              \
     reinterpret_cast<const void*>(&rmsnorm_bwd_generic<D>), "rmsnorm_bwd_generic<" #D ">"}

namespace rmsnorm_impl {

static const KernelEntry kBwdTable[] = {
    RMS_BWD_FAMILY(BF16, RMSNORM_BF16),
    RMS_BWD_FAMILY(FP16, RMSNORM_FP16),
    RMS_BWD_FAMILY(F32, RMSNORM_FP32),
    RMS_BWD_WIDE(F32, RMSNORM_FP32, 5), RMS_BWD_WIDE(F32, RMSNORM_FP32, 6),
};

const KernelEntry* bwd_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kBwdTable) / sizeof(kBwdTable[0]));
    return kBwdTable;
}

// The dw partial rows of rmsnorm_bwd_noalloc, which takes no workspace: a
// file-scope device array of RMSNORM_BWD_SCRATCH_BYTES that every GPU the
// library runs on holds for the life of the process (zero-filled when the
// code object loads; the row pass overwrites every partial row it uses before
// the column pass reads it, so nothing needs clearing between calls).  On the
// host `scratch` names a stand-in, not a device address: kernels get the
// address bwd_scratch() looked up for the current device.
static __device__ __align__(256) float scratch[RMSNORM_BWD_SCRATCH_BYTES / 4];

namespace {
constexpr int kScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void* ptr = nullptr;
};
ScratchSlot g_scratch[kScratchDevices];
}  // namespace

const char* bwd_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hipGetErrorString(e);
    if (dev < 0 || dev >= kScratchDevices) return "device ordinal out of range";
    ScratchSlot& s = g_scratch[dev];
    // once per device, with that device current (it is: dev is the calling thread's device)
    std::call_once(s.once, [&s]() { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess) return hipGetErrorString(s.err);
    if (s.ptr == nullptr) return "hipGetSymbolAddress returned no address for the scratch array";
    *ptr = s.ptr;
    return nullptr;
}

const void* dw_reduce_kernel(int split, int cols) {
    if (split == 64) return cols == 4 ? reinterpret_cast<const void*>(&rmsnorm_dw_reduce<64, 4>)
                                      : reinterpret_cast<const void*>(&rmsnorm_dw_reduce<64, 16>);
    return cols == 4 ? reinterpret_cast<const void*>(&rmsnorm_dw_reduce<16, 4>)
                     : reinterpret_cast<const void*>(&rmsnorm_dw_reduce<16, 16>);
}

}  // namespace rmsnorm_impl
