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
// HBM-bound (0.5 flop per byte).  One 256-thread workgroup per (b, h) (step_heads_kernel, the
// built widths N = 32, 64, 128), or per part of its rows when there are fewer heads than
// compute units or the width is another one (step_kernel).  A row
// p of the state (N floats) is covered by N/4 adjacent lanes holding one
// float4 each (rounded up to a power of two lanes), so every access is a 16-byte
// coalesced load or store; up to 16 of a thread's rows are loaded before any is
// updated so the loads are in flight together.  The dot product with C is reduced across the row's lanes
// with cross-lane shuffles.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

// One workgroup per (b, h), all of its rows: the batched decode at the built state widths.
template <typename TIn, int N>
__global__ __launch_bounds__(256) void step_heads_kernel(float *__restrict__ state, const TIn *__restrict__ x,
                                                   const typename Traits<TIn>::dt_t *__restrict__ dt,
                                                   const float *__restrict__ A,
                                                   const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
                                                   const float *__restrict__ D, void *__restrict__ y,
                                                   SsdOpts opt, int H, int G, int P, int sx, int sbc, int sdt,
                                                   int sz)
{
    // inputs: batch entry b of x, B/C, dt and z starts sx, sbc, sdt and sz elements after
    // entry b - 1 (dense: H P, G N, H, H P); y is dense
    constexpr int NQ = N / 4;          // lanes per state row (8, 16 or 32)
    constexpr int RP = 256 / NQ;       // rows per pass of the workgroup
    constexpr int MAXIT = 128 / RP > 0 ? 128 / RP : 1;  // P <= 128
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int g = h / (H / G);
    const int q = threadIdx.x % NQ;
    const int r0 = threadIdx.x / NQ;

    const float dtv = dt_effective(load_in(dt + (size_t)b * sdt + h), opt, h);
    const float r = exp_fast(dtv * A[h]);
    const float Dh = D ? D[h] : 0.f;
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bv[k] = load_in(Bm + (size_t)b * sbc + (size_t)g * N + 4 * q + k);
        cv[k] = load_in(Cm + (size_t)b * sbc + (size_t)g * N + 4 * q + k);
    }
    float4 *st = reinterpret_cast<float4 *>(state) + (size_t)bh * P * NQ;

    float4 s[MAXIT];
    float xs[MAXIT];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int p = r0 + k * RP;
        if (p < P) {
            s[k] = st[p * NQ + q];
            xs[k] = load_in(x + (size_t)b * sx + (size_t)h * P + p);
        }
    }
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int p = r0 + k * RP;
        if (p < P) {  // uniform across the NQ lanes of a row
            const float u = dtv * xs[k];
            float4 v = s[k];
            v.x = fmaf(r, v.x, u * bv[0]);
            v.y = fmaf(r, v.y, u * bv[1]);
            v.z = fmaf(r, v.z, u * bv[2]);
            v.w = fmaf(r, v.w, u * bv[3]);
            st[p * NQ + q] = v;
            float part = v.x * cv[0] + v.y * cv[1] + v.z * cv[2] + v.w * cv[3];
#pragma unroll
            for (int off = NQ / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
            if (q == 0) {
                float out = part + Dh * xs[k];
                if (opt.z) out *= silu(load_in(static_cast<const typename Traits<TIn>::dt_t *>(opt.z) + (size_t)b * sz + (size_t)h * P + p));
                if (opt.y_bf16)
                    static_cast<uint16_t *>(y)[(size_t)bh * P + p] = f32_to_bf16_rne(out);
                else
                    static_cast<float *>(y)[(size_t)bh * P + p] = out;
            }
        }
    }
}

// Any state width (N a multiple of 4 up to 256) and P up to 256, rows [p0, p1) of a head per
// workgroup.
template <typename TIn, int NQ, bool FULL>
__global__ __launch_bounds__(256) void step_kernel(float *__restrict__ state, const TIn *__restrict__ x,
                                                   const typename Traits<TIn>::dt_t *__restrict__ dt,
                                                   const float *__restrict__ A,
                                                   const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
                                                   const float *__restrict__ D, void *__restrict__ y,
                                                   SsdOpts opt, int H, int G, int P, int N, int sx, int sbc,
                                                   int sdt, int sz, int splits, int rows_per_wg)
{
    // inputs: batch entry b of x, B/C, dt and z starts sx, sbc, sdt and sz elements after
    // entry b - 1 (dense: H P, G N, H, H P); y is dense.  NQ lanes (a power of two, at least
    // N/4) cover a state row; lanes past the row's N/4 float4s hold zeros and store nothing.
    constexpr int RP = 256 / NQ;  // rows per pass of the workgroup
    constexpr int MB = 16;        // passes whose rows are in flight together
    // workgroup: rows [p0, p1) of the state of (b, h); a head's rows are split over `splits`
    // workgroups when there are few heads (batch-1 decode), else one workgroup takes them all
    const int bh = blockIdx.x / splits, part = blockIdx.x % splits;
    const int b = bh / H, h = bh % H;
    const int p0 = part * rows_per_wg, p1 = min(P, p0 + rows_per_wg);
    const int g = h / (H / G);
    const int q = threadIdx.x % NQ;
    const int r0 = threadIdx.x / NQ;
    // float4s per state row: FULL (N / 4 == NQ, every built size) makes it a constant
    const int N4 = FULL ? NQ : (N >> 2);
    const bool on = FULL || q < N4;

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

    for (int pb = p0; pb < p1; pb += RP * MB) {
        float4 s[MB];
        float xs[MB];
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int p = pb + r0 + k * RP;
            if (p < p1) {
                if (on) s[k] = st[p * N4 + q];
                xs[k] = load_in(x + (size_t)b * sx + (size_t)h * P + p);
            }
        }
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int p = pb + r0 + k * RP;
            if (p < p1) {  // uniform across the NQ lanes of a row
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
                    if (opt.z) out *= silu(load_in(static_cast<const typename Traits<TIn>::dt_t *>(opt.z) + (size_t)b * sz + (size_t)h * P + p));
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
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    const TIn *xx = static_cast<const TIn *>(x);
    const typename Traits<TIn>::dt_t *dd = static_cast<const typename Traits<TIn>::dt_t *>(dt);
    const TIn *bb = static_cast<const TIn *>(Bm), *cc = static_cast<const TIn *>(Cm);
    const int n4 = d.N / 4;
    const int nq = n4 <= 4 ? 4 : n4 <= 8 ? 8 : n4 <= 16 ? 16 : n4 <= 32 ? 32 : 64;
    const int rp = 256 / nq;  // rows per pass of one workgroup
    // With fewer heads than compute units, split each head's rows (whole passes) over up to
    // P / rp workgroups, as long as there are no more workgroups than compute units.
    const long heads = (long)d.B * d.H;
    int splits = 1;
    const int max_splits = (d.P + rp - 1) / rp;
    while (splits < max_splits && heads * splits * 2 <= ncu) splits *= 2;
    if (splits > max_splits) splits = max_splits;
    const int rows = ((d.P + splits - 1) / splits + rp - 1) / rp * rp;
    splits = (d.P + rows - 1) / rows;
    const dim3 grid((unsigned)(heads * splits));
    if (splits == 1 && d.P <= 128 && (d.N == 32 || d.N == 64 || d.N == 128)) {
        // the batched decode: one workgroup per head
        switch (d.N) {
        case 32: step_heads_kernel<TIn, 32><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.sx, d.sbc, d.sdt, d.sz); break;
        case 64: step_heads_kernel<TIn, 64><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.sx, d.sbc, d.sdt, d.sz); break;
        default: step_heads_kernel<TIn, 128><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.sx, d.sbc, d.sdt, d.sz); break;
        }
        return hipGetLastError();
    }
#define SSD_STEP(NQ)                                                                                                 \
    do {                                                                                                              \
        if (n4 == NQ)                                                                                                  \
            step_kernel<TIn, NQ, true><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.N,   \
                                                            d.sx, d.sbc, d.sdt, d.sz, splits, rows);                    \
        else                                                                                                           \
            step_kernel<TIn, NQ, false><<<grid, 256, 0, s>>>(state, xx, dd, A, bb, cc, D, y, o, d.H, d.G, d.P, d.N,  \
                                                             d.sx, d.sbc, d.sdt, d.sz, splits, rows);                   \
    } while (0)
    switch (nq) {
    case 4: SSD_STEP(4); break;
    case 8: SSD_STEP(8); break;
    case 16: SSD_STEP(16); break;
    case 32: SSD_STEP(32); break;
    default: SSD_STEP(64); break;
    }
#undef SSD_STEP
    return hipGetLastError();
}

hipError_t launch_step(float *state, const void *x, const void *dt, const float *A, const void *Bm,
                       const void *Cm, const float *D, void *y, const SsdOpts &o, const Dims &d, hipStream_t s)
{
    if (d.in == kInFp8) return launch_step_t<fp8_t>(state, x, dt, A, Bm, Cm, D, y, o, d, s);
    return d.in == kInBf16 ? launch_step_t<bf16_t>(state, x, dt, A, Bm, Cm, D, y, o, d, s)
                           : launch_step_t<float>(state, x, dt, A, Bm, Cm, D, y, o, d, s);
}

}  // namespace ssd
