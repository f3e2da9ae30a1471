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

__device__ __forceinline__ float row16_allreduce(float v) {
    v += dpp_mov<DPP_QUAD_SWAP1>(v);
    v += dpp_mov<DPP_QUAD_SWAP2>(v);
    v += dpp_mov<DPP_HALF_MIRROR>(v);
    v += dpp_mov<DPP_ROW_MIRROR>(v);
    return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over each aligned group of LANES lanes (16, 32 or 64); every lane of a
// group receives the same value.  Row sums are combined through scalar
// registers (v_readlane), so no LDS and no LDS-unit permutes are involved.
template <int LANES>
__device__ __forceinline__ float segment_allreduce(float v) {
    static_assert(LANES == 16 || LANES == 32 || LANES == 64, "segment must be 16, 32 or 64 lanes");
    v = row16_allreduce(v);
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

}  // namespace rmsnorm_dev
