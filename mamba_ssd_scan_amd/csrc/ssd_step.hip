// ssd_step.hip -- fused single-token decode update of the recurrent state.
//
// For every (b, h): H <- exp(dt A_h) H + (dt x) B^T, then y = H C + D_h x,
// with the [P, N] fp32 state read once and written once in place ("Compiler-
// First State Space Duality and Portable O(1) Autoregressive Caching for
// Inference", abstract: cached decode carries the state across tokens, cost
// independent of the sequence length; "Mamba-Family State-Space Model Kernels
// on a Programmable CGLA", Sec. III-A: the recurrent-state update).
//
// Optional model-adjacent work (see SsdOpts): dt = softplus(dt + bias), the z gate
// and bf16 storage of y.
//
// HBM-bound (0.5 flop per byte).  One 256-thread workgroup per (b, h).  A row
// p of the state (N floats) is covered by N/4 adjacent lanes holding one
// float4 each (rounded up to a power of two lanes), so every access is a 16-byte
// coalesced load or store; up to 16 of a thread's rows are loaded before any is
// updated so the loads are in flight together.  The dot product with C is reduced across the row's lanes
// with cross-lane shuffles.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int NQ>
__global__ __launch_bounds__(256) void step_kernel(float *__restrict__ state, const TIn *__restrict__ x,
                                                   const TIn *__restrict__ dt, const float *__restrict__ A,
                                                   const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
                                                   const float *__restrict__ D, void *__restrict__ y,
                                                   SsdOpts opt, int H, int G, int P, int N, int sx, int sbc,
                                                   int sdt, int sz)
{
    // inputs: batch entry b of x, B/C, dt and z starts sx, sbc, sdt and sz elements after
    // entry b - 1 (dense: H P, G N, H, H P); y is dense.  NQ lanes (a power of two, at least
    // N/4) cover a state row; lanes past the row's N/4 float4s hold zeros and store nothing.
    constexpr int RP = 256 / NQ;  // rows per pass of the workgroup
    constexpr int MB = 16;        // passes whose rows are in flight together
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int g = h / (H / G);
    const int q = threadIdx.x % NQ;
    const int r0 = threadIdx.x / NQ;
    const int N4 = N >> 2;  // float4s per state row
    const bool on = q < N4;

    const float dtv = dt_effective(load_in(dt + (size_t)b * sdt + h), opt, h);
    const float r = exp_fast(dtv * A[h]);
    const float Dh = D ? D[h] : 0.f;
    float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {0.f, 0.f, 0.f, 0.f};
    if (on) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bv[k] = load_in(Bm + (size_t)b * sbc + (size_t)g * N + 4 * q + k);
            cv[k] = load_in(Cm + (size_t)b * sbc + (size_t)g * N + 4 * q + k);
        }
    }
    float4 *st = reinterpret_cast<float4 *>(state) + (size_t)bh * P * N4;

    for (int pb = 0; pb < P; pb += RP * MB) {
        float4 s[MB];
        float xs[MB];
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int p = pb + r0 + k * RP;
            if (p < P) {
                if (on) s[k] = st[p * N4 + q];
                xs[k] = load_in(x + (size_t)b * sx + (size_t)h * P + p);
            }
        }
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int p = pb + r0 + k * RP;
            if (p < P) {  // uniform across the NQ lanes of a row
                const float u = dtv * xs[k];
                float part = 0.f;
                if (on) {
                    float4 v = s[k];
                    v.x = fmaf(r, v.x, u * bv[0]);
                    v.y = fmaf(r, v.y, u * bv[1]);
                    v.z = fmaf(r, v.z, u * bv[2]);
                    v.w = fmaf(r, v.w, u * bv[3]);
                    st[p * N4 + q] = v;
                    part = v.x * cv[0] + v.y * cv[1] + v.z * cv[2] + v.w * cv[3];
                }
#pragma unroll
                for (int off = NQ / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
                if (q == 0) {
                    float out = part + Dh * xs[k];
                    if (opt.z) out *= silu(load_in(static_cast<const TIn *>(opt.z) + (size_t)b * sz + (size_t)h * P + p));
                    if (opt.y_bf16)
                        static_cast<uint16_t *>(y)[(size_t)bh * P + p] = f32_to_bf16_rne(out);
                    else
                        static_cast<float *>(y)[(size_t)bh * P + p] = out;
                }
            }
        }
    }
}

template <typename TIn>
static hipError_t launch_step_t(float *state, const void *x, const void *dt, const float *A,
                                const void *Bm, const void *Cm, const float *D, void *y,
                                const SsdOpts &o, const Dims &d, hipStream_t s)
{
    if (d.N % 4 != 0 || d.N > 256 || d.P > 256) return hipErrorInvalidValue;
    const dim3 grid(d.B * d.H);
    const TIn *xx = static_cast<const TIn *>(x), *dd = static_cast<const TIn *>(dt);
    const TIn *bb = static_cast<const TIn *>(Bm), *cc = static_cast<const TIn *>(Cm);
    const int n4 = d.N / 4;
#define SSD_STEP(NQ) \
    step_kernel<TIn, NQ><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.N, d.sx, d.sbc, d.sdt, d.sz)
    if (n4 <= 4) SSD_STEP(4);
    else if (n4 <= 8) SSD_STEP(8);
    else if (n4 <= 16) SSD_STEP(16);
    else if (n4 <= 32) SSD_STEP(32);
    else SSD_STEP(64);
#undef SSD_STEP
    return hipGetLastError();
}

hipError_t launch_step(float *state, const void *x, const void *dt, const float *A, const void *Bm,
                       const void *Cm, const float *D, void *y, const SsdOpts &o, const Dims &d, hipStream_t s)
{
    return d.bf16 ? launch_step_t<bf16_t>(state, x, dt, A, Bm, Cm, D, y, o, d, s)
                  : launch_step_t<float>(state, x, dt, A, Bm, Cm, D, y, o, d, s);
}

}  // namespace ssd
