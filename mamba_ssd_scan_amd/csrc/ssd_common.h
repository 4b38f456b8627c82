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

#include <type_traits>

namespace ssd {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage: upper 16 bits of an fp32
// storage: OCP fp8 e4m3 ("fn"): a sign bit, 4 exponent bits (bias 7) and 3 mantissa bits;
// exponent 15 with mantissa 7 is NaN and there are no infinities (largest finite: 448)
struct fp8_t {
    uint8_t v;
};

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) through the hardware base-2 exponential: exp(x) = 2^(x log2 e).
// Results below the fp32 normal range flush to zero, which is exact enough
// for decay factors (they multiply values of order one).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Four e4m3 values (byte k of w is element k) as four fp16 values, exactly (every e4m3 value
// is an fp16 value).  A byte's exponent and mantissa bits are moved to the positions fp16
// keeps them in, which reads the value scaled by 2^-8 (the exponent biases differ by 8; e4m3
// subnormals land on fp16 subnormals with the same scale); one packed fp16 multiply by 2^8
// undoes the scale.  The NaN codes become fp16 NaN (a rare branch).  Result: elements 0, 1 in
// .x, 2, 3 in .y (low half first).
__device__ __forceinline__ uint32_t f8x2_placed_to_f16x2(uint32_t t)
{
    // t: the two bytes in the high byte of each 16-bit half
    const uint32_t h = (t & 0x80008000u) | ((t >> 1) & 0x3f803f80u);
    const f16x2 v = __builtin_bit_cast(f16x2, h) * f16x2{(f16)256.0f, (f16)256.0f};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint2 f8x4_to_f16x4(uint32_t w)
{
    uint2 r;
    r.x = f8x2_placed_to_f16x2(__builtin_amdgcn_perm(0u, w, 0x010c000cu));  // bytes 0, 1 -> high bytes of each half
    r.y = f8x2_placed_to_f16x2(__builtin_amdgcn_perm(0u, w, 0x030c020cu));  // bytes 2, 3
    const uint32_t nan = ((w & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;  // bit 7 of a byte: its code is NaN
    if (__builtin_expect(nan != 0u, 0)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (nan & (0x80u << (8 * k))) {
                uint32_t &word = k < 2 ? r.x : r.y;
                const int sh = 16 * (k & 1);
                const uint32_t sign = ((w >> (8 * k)) & 0x80u) << 8;
                word = (word & ~(0xffffu << sh)) | ((0x7e00u | sign) << sh);
            }
        }
    }
    return r;
}
// Eight e4m3 values (8 bytes) as an fp16 operand (16 bytes).
__device__ __forceinline__ uint4 f8x8_to_f16x8(uint2 w)
{
    const uint2 a = f8x4_to_f16x4(w.x), b = f8x4_to_f16x4(w.y);
    return make_uint4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ float fp8_to_f32(uint8_t v)
{
    const uint2 h = f8x4_to_f16x4((uint32_t)v);
    return static_cast<float>(__builtin_bit_cast(f16x2, h.x)[0]);
}

// Input element loads: bf16 bit patterns, e4m3 codes or fp32, returned as fp32 (exact).
__device__ __forceinline__ float load_in(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_in(const fp8_t *p) { return fp8_to_f32(p->v); }
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
__device__ __forceinline__ void load8(const fp8_t *p, float v[8])
{
    const uint4 h = f8x8_to_f16x8(*reinterpret_cast<const uint2 *>(p));
    const f16x8 f = __builtin_bit_cast(f16x8, h);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = static_cast<float>(f[k]);
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

// Options of the model-adjacent entry points (all off by default):
//  - dt_bias / dt_softplus: the step size the recurrence uses is softplus(dt + bias)
//    instead of the given dt ("Mamba-Family State-Space Model Kernels on a Programmable
//    CGLA", Sec. III-A: dt comes out of the in-projection as a raw channel);
//  - z: output gate, y <- y * z * sigmoid(z) (z is the in-projection's gate channel);
//  - y_bf16: y is stored as bf16 (round to nearest even) instead of fp32.
struct SsdOpts {
    const float *dt_bias;
    int dt_softplus;
    const void *z;
    int y_bf16;
    unsigned *sync;  // per-(b, h) counters of a launch that runs Step-3 inside the chunk scan
    // The prefill's control words: ctl[1] is the give-up word (set when a bounded wait between
    // workgroups gave up; cleared by the prefill's first launch).  nullptr: none.
    unsigned *ctl;
    // Bound of every wait between workgroups: 0 = the default; n > 0 = n - 1 polls (1: give up
    // at once, which only a test of the give-up path asks for).
    unsigned spin;
    // Nonzero: the prefill's X is too large to stay in the Infinity Cache from the first launch
    // to the chunk scan, and the launches that stream it read it with the kStream policy.
    int stream_x;
};
// Polls a bounded wait makes: the default bound, or the one SsdOpts::spin asks for.
constexpr unsigned kSpinLimit = 1u << 22;
__host__ __device__ __forceinline__ unsigned spin_polls(unsigned spin) { return spin ? spin - 1u : kSpinLimit; }
// One counter per 256 bytes, so that the heads' counters sit in different lines.
constexpr int kSyncStride = 64;

// dt as the recurrence uses it, for a token inside the sequence (fp32), with the head's
// bias already read
__device__ __forceinline__ float dt_effective_b(float d, float bias, int softplus)
{
    d += bias;
    if (softplus) d = d > 20.f ? d : log1pf(expf(d));  // log(1 + e^d); past 20 it equals d in fp32
    return d;
}
__device__ __forceinline__ float dt_effective(float d, const SsdOpts &o, int h)
{
    return dt_effective_b(d, o.dt_bias ? o.dt_bias[h] : 0.f, o.dt_softplus);
}
// z * sigmoid(z), through the hardware base-2 exponential and reciprocal (about 1 ulp
// each); for z below about -88, exp(-z) overflows to inf and the result is -0
__device__ __forceinline__ float silu(float v)
{
    return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * kLog2e));
}
// fp32 -> bf16, round to nearest even: gfx950's packed conversion (two values per
// instruction; the first lands in the low half)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) { return (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu); }

// the value of the lane next to this one (lanes 2k and 2k+1 swap), through a DPP quad
// permutation (1, 0, 3, 2): a VALU operation, no LDS round trip
__device__ __forceinline__ float swap_adjacent_lanes(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, true));
}

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
//  - e4m3 inputs: as bf16, with the raw inputs widened to fp16 (exact) and GEMMs over
//    them on fp16; dt (and the gate z) stay bf16.
template <typename TIn> struct Traits;
template <> struct Traits<bf16_t> {
    static constexpr bool kF32 = false;
    typedef f16 op_t;      // computed-operand element in LDS
    typedef bf16_t raw_t;  // raw-input element in LDS
    typedef bf16_t dt_t;   // storage of dt and z
};
template <> struct Traits<fp8_t> {
    static constexpr bool kF32 = false;
    typedef f16 op_t;
    typedef f16 raw_t;     // widened when staged
    typedef bf16_t dt_t;
};
template <> struct Traits<float> {
    static constexpr bool kF32 = true;
    typedef float op_t;
    typedef float raw_t;
    typedef float dt_t;
};

__device__ __forceinline__ f16 to_op(float v, f16 *) { return static_cast<f16>(v); }
__device__ __forceinline__ float to_op(float v, float *) { return v; }

// Buffer resource over [base, base + bytes): raw buffer loads take 32-bit byte
// offsets (one VGPR instead of a 64-bit address) and return zeros at or past
// `bytes`, which zero-fills ragged chunk tails without branches.  The config
// word is the gfx9-family raw-buffer setting (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a buffer access: 0 (the default), or kStream: non-temporal, for data read
// once per launch that cannot stay in the Infinity Cache until it is read again, so that it
// does not displace what the next launch reads back.
constexpr int kStream = 2;
template <int CP = 0> __device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP));
}

// Eight consecutive raw input elements held in registers between a global
// load and the LDS write that consumes them (software prefetch).
template <typename TIn> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
    // element offset `e` inside the buffer resource `r`
    template <int CP = 0> __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t e)
    {
        v = buf_load16<CP>(r, 2u * e);
    }
    __device__ __forceinline__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void store(bf16_t *dst) const { *reinterpret_cast<uint4 *>(dst) = v; }
    __device__ __forceinline__ void to_f32(float f[8]) const
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(w[k] << 16);
            f[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p)
    {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    template <int CP = 0> __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t e)
    {
        a = __builtin_bit_cast(float4, buf_load16<CP>(r, 4u * e));
        b = __builtin_bit_cast(float4, buf_load16<CP>(r, 4u * e + 16u));
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void store(float *dst) const
    {
        reinterpret_cast<float4 *>(dst)[0] = a;
        reinterpret_cast<float4 *>(dst)[1] = b;
    }
    __device__ __forceinline__ void to_f32(float f[8]) const
    {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

template <int CP = 0> __device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CP));
}
template <> struct Raw8<fp8_t> {
    uint2 v;
    __device__ __forceinline__ void load(const fp8_t *p) { v = *reinterpret_cast<const uint2 *>(p); }
    template <int CP = 0> __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t e)
    {
        v = buf_load8<CP>(r, e);
    }
    __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
    // widened to fp16 when staged (Traits<fp8_t>::raw_t)
    __device__ __forceinline__ void store(f16 *dst) const { *reinterpret_cast<uint4 *>(dst) = f8x8_to_f16x8(v); }
    __device__ __forceinline__ void to_f32(float f[8]) const
    {
        const f16x8 h = __builtin_bit_cast(f16x8, f8x8_to_f16x8(v));
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = static_cast<float>(h[k]);
    }
};

// Store two fp32 values as an adjacent pair of operand elements (4 or 8 bytes).
__device__ __forceinline__ void store_pair(f16 *dst, float lo, float hi)
{
    *reinterpret_cast<uint32_t *>(dst) = pack_f16x2(lo, hi);
}
__device__ __forceinline__ void store_pair(float *dst, float lo, float hi)
{
    *reinterpret_cast<float2 *>(dst) = make_float2(lo, hi);
}

// Eight bf16 bit patterns (as stored) to an fp16 matrix-core operand.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(bf16x8 v)
{
    const uint4 u = __builtin_bit_cast(uint4, v);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    f16x8 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[2 * k] = static_cast<f16>(__uint_as_float(w[k] << 16));
        h[2 * k + 1] = static_cast<f16>(__uint_as_float(w[k] & 0xFFFF0000u));
    }
    return h;
}

// Eight raw inputs held in a bf16x8 register as loaded (bf16: all 16 bytes; e4m3: the low
// 8 bytes) as an fp16 matrix-core operand.
template <typename TIn> __device__ __forceinline__ f16x8 held_to_f16x8(bf16x8 v)
{
    if constexpr (std::is_same<TIn, fp8_t>::value) {
        const uint4 u = __builtin_bit_cast(uint4, v);
        return __builtin_bit_cast(f16x8, f8x8_to_f16x8(make_uint2(u.x, u.y)));
    } else {
        return bf16x8_to_f16x8(v);
    }
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives four b16 values: value r is element (i % 4) of the
// four-element run addressed by lane 4r + i/4 of the same group.  If lane q
// of group g addresses row k0 + 4g + q/4, column m0 + 4(q % 4) of a row-major
// [k][m] tile, lane i therefore receives rows k0 + 4g + r of column m0 + i:
// a matrix-core operand slice whose reduction index runs down the LDS rows,
// read without storing the tile transposed.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ f16x4 lds_read_tr16(const f16 *p)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(f16x4, v);
}

// Address of this lane's run for lds_read_tr16 on a row-major tile of row
// pitch `ld` elements: rows k0 + 4g + q/4 (g = lane / 16, q = lane % 16),
// columns m0 + 4 (q % 4).
__device__ __forceinline__ int tr16_offset(int lane, int k0, int m0, int ld)
{
    const int g = lane >> 4, q = lane & 15;
    return (k0 + 4 * g + (q >> 2)) * ld + m0 + 4 * (q & 3);
}

// Direct-to-LDS buffer loads (gfx950): every lane reads 16 (or 4) bytes at byte
// offset `off` of the buffer resource and the wavefront writes them to LDS at
// `lds + 16 * lane` (or `lds + 4 * lane`) (the LDS address must be wave-uniform).  Out-of-range reads
// deliver zeros.  The load counts in the wavefront's vector-memory counter like any other.
typedef __attribute__((address_space(3))) void lds_void;
template <int CP = 0> __device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, (int)off, 0, 0, CP);
}
template <int CP = 0> __device__ __forceinline__ void buf_load_lds4(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 4, (int)off, 0, 0, CP);
}

// Eight raw inputs converted to fp16 and packed into 16 bytes (one LDS store).
template <typename TIn>
__device__ __forceinline__ uint4 raw8_to_f16x8(const Raw8<TIn> &r, float scale = 1.f)
{
    float f[8];
    r.to_f32(f);
    uint4 w;
    w.x = pack_f16x2(f[0] * scale, f[1] * scale);
    w.y = pack_f16x2(f[2] * scale, f[3] * scale);
    w.z = pack_f16x2(f[4] * scale, f[5] * scale);
    w.w = pack_f16x2(f[6] * scale, f[7] * scale);
    return w;
}

}  // namespace ssd
