// ssd_chunk_state.hip -- Step-2: the state each chunk leaves from a zero start.
//
//   S_c[p, n] = sum_j w_j x_j[p] B_j[n],   w_j = exp(dA_cum[Q-1] - dA_cum[j]) dt_j
//
// i.e. S_c = (X_c * w)^T B_c, a [P, Q] x [Q, N] contraction over the chunk's
// time axis.  The chunked method needs it to hand state from chunk to chunk
// ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec.
// III-A: the recurrent state links the chunks; Step-3 consumes these states).
//
// One 256-thread workgroup (4 wavefronts) per (b, h, c).  The chunk is
// streamed through LDS in blocks of JB tokens, stored transposed ([P][JB]
// and [N][JB]) so that each lane reads its reduction slots as one 16-byte LDS
// load.  The decay weight is folded into X while staging; the weighted X is
// a computed operand, so with bf16 inputs both operands go to the matrix
// cores as fp16 (B converts exactly), accumulating in fp32.  Each wavefront
// owns every fourth 16x16 output tile.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int P, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(const TIn *__restrict__ x,
                                                          const TIn *__restrict__ Bm,
                                                          const float *__restrict__ acum,
                                                          const float *__restrict__ dtc,
                                                          float *__restrict__ states, int L, int H,
                                                          int G, int Q, int nc)
{
    typedef Traits<TIn> Tr;
    typedef typename Tr::op_t op_t;
    constexpr bool F32 = Tr::kF32;
    constexpr int JB = F32 ? 32 : 64;       // tokens per staged block
    constexpr int LDX = JB + (F32 ? 4 : 8); // row length of the transposed tiles
    constexpr int TN = N / 16, NT = (P / 16) * TN;
    constexpr int TPW = (NT + 3) / 4;       // output tiles per wavefront
    __shared__ op_t xs[P * LDX];            // (X * w)^T
    __shared__ op_t bs[N * LDX];            // B^T

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const float *ac = acum + bhc * Q;
    const float *dd = dtc + bhc * Q;
    const float aend = ac[Q - 1];
    const long tc = (long)c * Q;

    f32x4 acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = zero4();

    for (int j0 = 0; j0 < Q; j0 += JB) {
        // ---- stage (X * w)^T: one unit = two consecutive tokens x eight channels
        constexpr int XG = P / 8;
        for (int u = tid; u < (JB / 2) * XG; u += 256) {
            const int jp = u / XG, pg = u % XG;
            const int j = j0 + 2 * jp;
            float v0[8], v1[8], w0 = 0.f, w1 = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) v0[k] = v1[k] = 0.f;
            if (j < Q && tc + j < L) {
                load8(x + (((size_t)b * L + tc + j) * H + h) * P + 8 * pg, v0);
                w0 = exp_fast(aend - ac[j]) * dd[j];
            }
            if (j + 1 < Q && tc + j + 1 < L) {
                load8(x + (((size_t)b * L + tc + j + 1) * H + h) * P + 8 * pg, v1);
                w1 = exp_fast(aend - ac[j + 1]) * dd[j + 1];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                op_t *dst = &xs[(8 * pg + k) * LDX + 2 * jp];
                if constexpr (F32) {
                    *reinterpret_cast<float2 *>(dst) = make_float2(v0[k] * w0, v1[k] * w1);
                } else {
                    *reinterpret_cast<uint32_t *>(dst) = pack_f16x2(v0[k] * w0, v1[k] * w1);
                }
            }
        }
        // ---- stage B^T
        constexpr int BG = N / 8;
        for (int u = tid; u < (JB / 2) * BG; u += 256) {
            const int jp = u / BG, ng = u % BG;
            const int j = j0 + 2 * jp;
            float v0[8], v1[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v0[k] = v1[k] = 0.f;
            if (j < Q && tc + j < L) load8(Bm + (((size_t)b * L + tc + j) * G + g) * N + 8 * ng, v0);
            if (j + 1 < Q && tc + j + 1 < L) load8(Bm + (((size_t)b * L + tc + j + 1) * G + g) * N + 8 * ng, v1);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                op_t *dst = &bs[(8 * ng + k) * LDX + 2 * jp];
                if constexpr (F32) {
                    *reinterpret_cast<float2 *>(dst) = make_float2(v0[k], v1[k]);
                } else {
                    *reinterpret_cast<uint32_t *>(dst) = pack_f16x2(v0[k], v1[k]);
                }
            }
        }
        __syncthreads();

        // ---- contraction over this block's tokens, 32 at a time
        for (int ks = 0; ks < JB && j0 + ks < Q; ks += 32) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int t = wave + 4 * tt;
                if (t < NT) {
                    const int pt = t / TN, nt = t % TN;
                    const op_t *xa = &xs[(pt * 16 + li) * LDX + ks];
                    const op_t *ba = &bs[(nt * 16 + li) * LDX + ks];
                    if constexpr (F32) {
#pragma unroll
                        for (int s = 0; s < 8; ++s) acc[tt] = mfma16x16x4_f32(xa[4 * s + lg], ba[4 * s + lg], acc[tt]);
                    } else {
                        const f16x8 a = *reinterpret_cast<const f16x8 *>(xa + 8 * lg);
                        const f16x8 bb = *reinterpret_cast<const f16x8 *>(ba + 8 * lg);
                        acc[tt] = mfma16x16x32_f16(a, bb, acc[tt]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- write S_c [P][N]: lane holds rows p = 16 pt + 4 lg + r of column n = 16 nt + li
    float *out = states + bhc * P * N;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int t = wave + 4 * tt;
        if (t < NT) {
            const int pt = t / TN, nt = t % TN;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(size_t)(pt * 16 + 4 * lg + r) * N + nt * 16 + li] = acc[tt][r];
        }
    }
}

template <typename TIn, int P>
static hipError_t launch_cs_n(const void *x, const void *Bm, const float *acum, const float *dtc,
                              float *states, const Dims &d, hipStream_t s)
{
    const dim3 grid(d.nc, d.H, d.B);
    const TIn *xx = static_cast<const TIn *>(x), *bb = static_cast<const TIn *>(Bm);
    switch (d.N) {
    case 32: chunk_state_kernel<TIn, P, 32><<<grid, 256, 0, s>>>(xx, bb, acum, dtc, states, d.L, d.H, d.G, d.Q, d.nc); break;
    case 64: chunk_state_kernel<TIn, P, 64><<<grid, 256, 0, s>>>(xx, bb, acum, dtc, states, d.L, d.H, d.G, d.Q, d.nc); break;
    case 128: chunk_state_kernel<TIn, P, 128><<<grid, 256, 0, s>>>(xx, bb, acum, dtc, states, d.L, d.H, d.G, d.Q, d.nc); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_cs_t(const void *x, const void *Bm, const float *acum, const float *dtc,
                              float *states, const Dims &d, hipStream_t s)
{
    switch (d.P) {
    case 32: return launch_cs_n<TIn, 32>(x, Bm, acum, dtc, states, d, s);
    case 64: return launch_cs_n<TIn, 64>(x, Bm, acum, dtc, states, d, s);
    case 128: return launch_cs_n<TIn, 128>(x, Bm, acum, dtc, states, d, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_state(const void *x, const void *Bm, const float *acum, const float *dtc,
                              float *states, const Dims &d, hipStream_t s)
{
    return d.bf16 ? launch_cs_t<bf16_t>(x, Bm, acum, dtc, states, d, s)
                  : launch_cs_t<float>(x, Bm, acum, dtc, states, d, s);
}

}  // namespace ssd
