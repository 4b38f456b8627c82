// ssd_common.h -- device helpers shared by the gfx950 SSD kernels.
//
// Matrix-core fragments follow the CDNA4 MFMA lane layout for the 16x16
// tiles used here (lane l, row/column index l % 16, k-group g = l / 16):
//   16x16x32 (f16, bf16): A[m = l%16][k = 8g .. 8g+7], B[k = 8g .. 8g+7][n = l%16]
//   16x16x4  (f32)      : A[m = l%16][k = g],          B[k = g][n = l%16]
//   accumulator (both)  : D[m = 4g + r][n = l%16], r = 0..3
// Only the pairing of k slots between A and B matters to the product, so a
// kernel may assign any set of reduction indices to a lane's k slots as long
// as both operands use the same assignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage: upper 16 bits of an fp32

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) through the hardware base-2 exponential: exp(x) = 2^(x log2 e).
// Results below the fp32 normal range flush to zero, which is exact enough
// for decay factors (they multiply values of order one).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Input element loads: bf16 bit patterns or fp32, returned as fp32 (exact).
__device__ __forceinline__ float load_in(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_in(const float *p) { return *p; }

// Eight consecutive inputs as fp32 (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const bf16_t *p, float v[8])
{
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float v[8])
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Pack two fp32 values into one 32-bit word of two fp16 halves (RNE).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    f16x2 h = {static_cast<f16>(lo), static_cast<f16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
}

// Per-input-type traits: the matrix-core operand types a kernel uses.
//  - bf16 inputs: GEMMs over raw inputs run on bf16 (exact operands); GEMMs
//    with a computed operand run on fp16 (11-bit significand) so that the
//    rounding of the computed operand stays near 2^-12 relative.
//  - fp32 inputs: every GEMM runs on the fp32 matrix path (16x16x4).
template <typename TIn> struct Traits;
template <> struct Traits<bf16_t> {
    static constexpr bool kF32 = false;
    typedef f16 op_t;      // computed-operand element in LDS
    typedef bf16_t raw_t;  // raw-input element in LDS
};
template <> struct Traits<float> {
    static constexpr bool kF32 = true;
    typedef float op_t;
    typedef float raw_t;
};

__device__ __forceinline__ f16 to_op(float v, f16 *) { return static_cast<f16>(v); }
__device__ __forceinline__ float to_op(float v, float *) { return v; }

}  // namespace ssd
