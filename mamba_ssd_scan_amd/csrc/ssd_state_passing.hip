// ssd_state_passing.hip -- Step-3: inter-chunk recurrence of the state.
//
// The state entering chunk c+1 is the state entering chunk c, decayed by the
// chunk's total decay exp(dA_cum[c][Q-1]), plus the chunk's own state S_c
// ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec.
// III-A and IV-C: Step-3 is sequential across chunks; A_c is diagonal, so
// the per-chunk update of the [P, N] state is a per-head scalar scale plus an
// add, not a dense matrix-vector product).
//
// HBM-bound: each thread owns four consecutive state elements of one (b, h)
// and walks the chunks in order, reading S_c and writing the entering state in
// place (16-byte coalesced accesses for fp32 states, 8-byte for the fp16 states
// of bf16 inputs; the carry itself is fp32).  The loads of the next kUnroll
// chunks are issued before any of their results is needed, so many loads are
// in flight per thread while the dependent scale-add chain runs.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kPassThreads = 64;
constexpr int kUnroll = 16;

// Four consecutive stored state elements <-> fp32 (the carry is always fp32).
__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const f16 *p)
{
    const f16x4 v = *reinterpret_cast<const f16x4 *>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
__device__ __forceinline__ void store4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
__device__ __forceinline__ void store4(f16 *p, float4 v)
{
    uint2 u;
    u.x = pack_f16x2(v.x, v.y);
    u.y = pack_f16x2(v.z, v.w);
    *reinterpret_cast<uint2 *>(p) = u;
}

// The carry is rounded to fp32 by every step and only then to the stored type: an empty
// asm statement over the fresh carry keeps the compiler from fusing the step's
// multiply-add with the next store's conversion into one instruction that rounds
// straight to fp16 (the chunk scan's own Step-3 stores exactly these values).
__device__ __forceinline__ void carry_fp32(float4 &v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// T: element type of the chunk / entering states in memory (fp32, or fp16 for bf16 inputs)
template <typename T>
__global__ __launch_bounds__(kPassThreads) void state_passing_kernel(
    T *__restrict__ states, const float *__restrict__ acum, const float *init,
    float *fin, int H, int nc, int Q, int PN4)
{
    const int e = blockIdx.x * kPassThreads + threadIdx.x;  // group of 4 elements inside one [P, N] state
    const int h = blockIdx.y, b = blockIdx.z;
    if (e >= PN4) return;
    const size_t bh = (size_t)b * H + h;
    float4 run = init ? reinterpret_cast<const float4 *>(init)[bh * PN4 + e] : make_float4(0.f, 0.f, 0.f, 0.f);
    T *st = states + (bh * nc * (size_t)PN4 + e) * 4;
    const float *ac = acum + bh * nc * (size_t)Q + (Q - 1);

    int c = 0;
    for (; c + kUnroll <= nc; c += kUnroll) {
        float4 s[kUnroll];
        float dec[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            s[k] = load4(st + (size_t)(c + k) * PN4 * 4);
            dec[k] = ac[(size_t)(c + k) * Q];
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            store4(st + (size_t)(c + k) * PN4 * 4, run);
            const float r = exp_fast(dec[k]);
            run.x = fmaf(r, run.x, s[k].x);
            run.y = fmaf(r, run.y, s[k].y);
            run.z = fmaf(r, run.z, s[k].z);
            run.w = fmaf(r, run.w, s[k].w);
            carry_fp32(run);
        }
    }
    for (; c < nc; ++c) {
        const float4 s = load4(st + (size_t)c * PN4 * 4);
        store4(st + (size_t)c * PN4 * 4, run);
        const float r = exp_fast(ac[(size_t)c * Q]);
        run.x = fmaf(r, run.x, s.x);
        run.y = fmaf(r, run.y, s.y);
        run.z = fmaf(r, run.z, s.z);
        run.w = fmaf(r, run.w, s.w);
        carry_fp32(run);
    }
    if (fin) reinterpret_cast<float4 *>(fin)[bh * PN4 + e] = run;
}

hipError_t launch_state_passing(void *states, const float *acum, const float *init, float *fin,
                                const Dims &d, hipStream_t s)
{
    const int PN4 = d.P * d.N / 4;
    dim3 grid((PN4 + kPassThreads - 1) / kPassThreads, d.H, d.B);
    if (d.half())
        launch_kernel("state_passing_kernel", state_passing_kernel<f16>, grid, kPassThreads, s,
                      static_cast<f16 *>(states), acum, init, fin, d.H, d.nc, d.Q, PN4);
    else
        launch_kernel("state_passing_kernel", state_passing_kernel<float>, grid, kPassThreads, s,
                      static_cast<float *>(states), acum, init, fin, d.H, d.nc, d.Q, PN4);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_state_kernel(float *__restrict__ dst,
                                                         const float *__restrict__ src, size_t n4)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    reinterpret_cast<float4 *>(dst)[i] =
        src ? reinterpret_cast<const float4 *>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_fill_state(float *dst, const float *src, size_t n, hipStream_t s)
{
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    if (dst == src) return hipSuccess;
    launch_kernel("fill_state_kernel", fill_state_kernel, dim3((unsigned)((n4 + 255) / 256)), 256, s, dst, src,
                  n4);
    return hipGetLastError();
}

}  // namespace ssd
