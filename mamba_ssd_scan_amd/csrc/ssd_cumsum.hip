// ssd_cumsum.hip -- Step-0: per-chunk inclusive cumulative decay.
//
// For chunk c of head h, a_t = dt_t * A_h and dA_cum[i] = sum_{k<=i} a_{cQ+k}
// ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec.
// III-A: the sequence is cut into chunks of Q tokens; the decay is a
// diagonal, per-head scalar).  The scan restarts at every chunk, which keeps
// the fp32 cancellation in dA_cum[i] - dA_cum[j] bounded by one chunk.
//
// One 64-lane wavefront per (b, h, c): each lane scans Q/64 consecutive
// tokens serially (1 for Q < 64), then the lane totals are combined with a
// wavefront-wide Hillis-Steele scan over cross-lane shuffles.  The kernel
// also regroups dt into [B, H, nc, Q] so that the chunk kernels read it with
// unit stride.  Tokens past seqlen act as dt = 0 (neutral: no decay, no input).
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn>
__global__ __launch_bounds__(64) void chunk_cumsum_kernel(const TIn *__restrict__ dt,
                                                          const float *__restrict__ A,
                                                          float *__restrict__ acum,
                                                          float *__restrict__ dtc, int L, int H,
                                                          int Q, int nc)
{
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int per = Q > 64 ? Q / 64 : 1;  // tokens per lane: 1, 2 or 4
    const float Ah = A[h];

    float part[4], dts[4];
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        part[k] = 0.f;
        dts[k] = 0.f;
        if (k < per) {
            const int i = lane * per + k;
            const long t = (long)c * Q + i;
            float d = 0.f;
            if (i < Q && t < L) d = load_in(dt + ((size_t)b * L + t) * H + h);
            dts[k] = d;
            run += d * Ah;
            part[k] = run;
        }
    }
    // inclusive scan of the lane totals across the wavefront
    float incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;

    const size_t base = (((size_t)b * H + h) * nc + c) * Q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * per + k;
        if (k < per && i < Q) {
            acum[base + i] = excl + part[k];
            dtc[base + i] = dts[k];
        }
    }
}

hipError_t launch_chunk_cumsum(const void *dt, const float *A, float *acum, float *dtc,
                               const Dims &d, hipStream_t s)
{
    dim3 grid(d.nc, d.H, d.B);
    if (d.half())  // dt is bf16 beside bf16 and fp8 inputs
        launch_kernel("chunk_cumsum_kernel", chunk_cumsum_kernel<bf16_t>, grid, 64, s,
                      static_cast<const bf16_t *>(dt), A, acum, dtc, d.L, d.H, d.Q, d.nc);
    else
        launch_kernel("chunk_cumsum_kernel", chunk_cumsum_kernel<float>, grid, 64, s,
                      static_cast<const float *>(dt), A, acum, dtc, d.L, d.H, d.Q, d.nc);
    return hipGetLastError();
}

}  // namespace ssd
