// rmsnorm_device.hpp -- gfx950 device helpers for the row RMSNorm kernels:
// 16-byte vector I/O, bf16/fp16 <-> fp32 conversion, and wave64 reductions
// that leave every lane of a row segment with bit-identical sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsnorm_dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Element formats.  A 16-byte vector holds EPV elements: eight 16-bit ones,
// two per 32-bit word with the low half first (the memory order of a
// little-endian row), or four fp32 ones.  widen() is exact; narrow() and
// round1() round to nearest even and keep subnormals (the compiler emits the
// hardware converts: v_cvt_pk_bf16_f32 on gfx950 for bf16, v_cvt_f16_f32 for
// fp16, both honouring the round-to-nearest-even mode; no round-toward-zero
// packing instruction is used).  fp32 needs no conversion at all.
// ---------------------------------------------------------------------------
template <class D>
struct Packed16 {
    static constexpr int EPV = 8;
    typedef uint16_t elem_t;
    static __device__ __forceinline__ void widen(const u32x4 q, float (&f)[EPV]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = D::lo(q[k]);
            f[2 * k + 1] = D::hi(q[k]);
        }
    }
    static __device__ __forceinline__ u32x4 narrow(const float (&f)[EPV]) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = D::pack(f[2 * k], f[2 * k + 1]);
        return o;
    }
};

struct BF16 : Packed16<BF16> {
    static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
    static __device__ __forceinline__ float one(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        f32x2 f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    static __device__ __forceinline__ uint16_t round1(float a) {
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    }
};

struct FP16 : Packed16<FP16> {
    static __device__ __forceinline__ float lo(uint32_t u) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
    }
    static __device__ __forceinline__ float hi(uint32_t u) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
    static __device__ __forceinline__ float one(uint16_t u) {
        return (float)__builtin_bit_cast(_Float16, u);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        f32x2 f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    }
    static __device__ __forceinline__ uint16_t round1(float a) {
        return __builtin_bit_cast(uint16_t, (_Float16)a);
    }
};

struct F32 {
    static constexpr int EPV = 4;
    typedef uint32_t elem_t;
    static __device__ __forceinline__ void widen(const u32x4 q, float (&f)[EPV]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(q[k]);
    }
    static __device__ __forceinline__ u32x4 narrow(const float (&f)[EPV]) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(f[k]);
        return o;
    }
    static __device__ __forceinline__ float one(uint32_t u) { return __uint_as_float(u); }
    static __device__ __forceinline__ uint32_t round1(float a) { return __float_as_uint(a); }
};

// ---------------------------------------------------------------------------
// Cross-lane sums.  A DPP "row" is 16 lanes.  The butterfly below swaps
// partners (neighbours, pairs, mirrored quads, mirrored half-rows), so both
// partners add the same two values and every lane of the row ends with the
// same bits: a + b == b + a exactly in IEEE arithmetic.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

enum : int {
    DPP_QUAD_SWAP1 = 0xB1,    // quad_perm [1,0,3,2]
    DPP_QUAD_SWAP2 = 0x4E,    // quad_perm [2,3,0,1]
    DPP_ROW_MIRROR = 0x140,   // lane i <-> 15 - i within the row
    DPP_HALF_MIRROR = 0x141,  // lane i <-> 7 - i within each half-row
};

// Sum over each aligned group of LANES (4, 8 or 16) lanes, in butterfly
// stages of 2, 4, 8 and 16 lanes; every lane of a group ends with the same
// bits (each stage adds two equal-valued partials, and a + b == b + a).
template <int LANES = 16>
__device__ __forceinline__ float row16_allreduce(float v) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "a DPP row holds groups of 4, 8 or 16 lanes");
    v += dpp_mov<DPP_QUAD_SWAP1>(v);
    v += dpp_mov<DPP_QUAD_SWAP2>(v);
    if constexpr (LANES >= 8) v += dpp_mov<DPP_HALF_MIRROR>(v);
    if constexpr (LANES >= 16) v += dpp_mov<DPP_ROW_MIRROR>(v);
    return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over each aligned group of LANES lanes (4, 8, 16, 32 or 64); every lane
// of a group receives the same value.  Groups wider than a DPP row combine
// the row sums through scalar registers (v_readlane), so no LDS and no
// LDS-unit permutes are involved.
template <int LANES>
__device__ __forceinline__ float segment_allreduce(float v) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64,
                  "segment must be 4, 8, 16, 32 or 64 lanes");
    v = row16_allreduce<(LANES < 16 ? LANES : 16)>(v);
    if constexpr (LANES == 32) {
        const float s01 = readlane(v, 0) + readlane(v, 16);
        const float s23 = readlane(v, 32) + readlane(v, 48);
        v = ((threadIdx.x & 63) < 32) ? s01 : s23;
    } else if constexpr (LANES == 64) {
        v = (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
    }
    return v;
}

// Hardware reciprocal square root (v_rsq_f32, about 1 ulp).
__device__ __forceinline__ float rsq(float v) { return __builtin_amdgcn_rsqf(v); }

// ---------------------------------------------------------------------------
// Rows that do not start on a 16-byte boundary.  Such a row is read as the
// aligned 16-byte chunks that cover it; with `al` the row start's distance
// past a boundary in elements, chunk c holds row elements c * EPV - al ..
// c * EPV - al + EPV - 1.  The helpers below shift packed vectors between that
// chunk frame and the frame of the (16-byte aligned) weights, mask the edge
// chunks, and store an edge chunk's own elements.
// ---------------------------------------------------------------------------
// Words k .. k + 3 of the 8-word concatenation (lo, hi) starting `sh`
// elements in (0 < sh <= EPV), for the wave-uniform sh of one row.
template <class D>
__device__ __forceinline__ u32x4 funnel(const u32x4 lo, const u32x4 hi, int sh) {
    constexpr int EPW = 4 / static_cast<int>(sizeof(typename D::elem_t));   // elements per word
    const uint32_t W[9] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3], 0u};
    const int q = sh / EPW;                                                 // whole words
    const uint32_t r = static_cast<uint32_t>((sh % EPW) * sizeof(typename D::elem_t));   // bytes
    u32x4 o;
    switch (q) {    // q is the same in every lane: one branch, constant register indices
#define RMS_FUNNEL_CASE(Q)                                                                   \
        case Q:                                                                              \
            for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_alignbyte(W[k + Q + 1], W[k + Q], r); \
            break;
        RMS_FUNNEL_CASE(0) RMS_FUNNEL_CASE(1) RMS_FUNNEL_CASE(2) RMS_FUNNEL_CASE(3)
#undef RMS_FUNNEL_CASE
        default:
            o = hi;
            break;
    }
    return o;
}

// funnel() for a shift that differs between lanes (rows of several segments
// in one wave): words k .. k + 3 of (lo, hi) from `sh` elements in, the word
// offset picked per lane by selects instead of a branch.
template <class D>
__device__ __forceinline__ u32x4 funnel_lane(const u32x4 lo, const u32x4 hi, int sh) {
    constexpr int EPW = 4 / static_cast<int>(sizeof(typename D::elem_t));
    const uint32_t W[9] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3], 0u};
    const int q = sh / EPW;                                                 // 0 .. 4
    const uint32_t r = static_cast<uint32_t>((sh % EPW) * sizeof(typename D::elem_t));
    uint32_t A[5];      // A[k] = W[k + q]
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        uint32_t t = W[k];
#pragma unroll
        for (int j = 1; j <= 4; ++j)
            if (k + j <= 8) t = q == j ? W[k + j] : t;
        A[k] = t;
    }
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_alignbyte(A[k + 1], A[k], r);
    return o;
}

// A chunk holding row elements j0 .. j0 + EPV - 1 with those outside
// 0 .. n - 1 set to zero.
template <class D>
__device__ __forceinline__ u32x4 keep_row(u32x4 v, int j0, int n) {
    constexpr int EPW = 4 / static_cast<int>(sizeof(typename D::elem_t));
    const int lo = -j0, hi = n - j0;    // kept: lo <= i < hi
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (EPW == 2) {
            const uint32_t m = ((2 * k >= lo && 2 * k < hi) ? 0x0000FFFFu : 0u) |
                               ((2 * k + 1 >= lo && 2 * k + 1 < hi) ? 0xFFFF0000u : 0u);
            v[k] &= m;
        } else {
            v[k] = (k >= lo && k < hi) ? v[k] : 0u;
        }
    }
    return v;
}

// The row's own elements of an edge chunk, stored one at a time.
template <class D>
__device__ __forceinline__ void store_edge(u32x4* p, u32x4 v, int j0, int n) {
    typedef typename D::elem_t E;
    E* q = reinterpret_cast<E*>(p);
    const auto e = __builtin_bit_cast(E __attribute__((ext_vector_type(D::EPV))), v);
#pragma unroll
    for (int i = 0; i < D::EPV; ++i)
        if (j0 + i >= 0 && j0 + i < n) q[i] = e[i];
}

// Each lane's v from the lane below (DPP wave_shr:1); lane 0 takes `lane0`.
__device__ __forceinline__ u32x4 from_lane_below(const u32x4 v, const u32x4 lane0) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        o[k] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(lane0[k]), static_cast<int>(v[k]),
                                                                 0x138, 0xF, 0xF, false));
    return o;
}

// Each lane's v from the lane above (DPP wave_shl:1); lane 63 takes `lane63`.
__device__ __forceinline__ float from_lane_above(const float v, const float lane63) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, lane63),
                                                                 __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
}

}  // namespace rmsnorm_dev
