// ssd_chunk_gemm1.hip -- Step-1 GEMM1: the C.B^T products of every chunk.
//
//   G_c[i, j] = C_i . B_j      (chunk-local tokens, j <= i, reduction over the state dim N)
//
// Sources: "Mamba-Family State-Space Model Kernels on a Programmable CGLA",
// Sec. III-A (Step-1 GEMM1 forms C.B^T over the state dimension; B and C come
// from the in-projection once per token, shared by the heads that read them).
// G depends on (batch, group, chunk) but not on the head, so it is formed once
// here and read by the chunk-scan kernel of every head of the group, instead
// of being recomputed per head.
//
// Output layout ("fragment order"; fp16 for bf16 inputs, whose matrix-core
// operands downstream are fp16, and fp32 for fp32 inputs): for row tile t (rows 16t .. 16t+15)
// and 32-column step s = 0 .. t/2 (columns 32s .. 32s+31), 64 lanes x 8 values;
// lane l (li = l % 16, lg = l / 16) holds G[16t + li][32s + 4lg + r] at r and
// G[16t + li][32s + 16 + 4lg + r] at 4 + r, for r = 0..3 -- the accumulator
// layout of two 16x16 matrix-core tiles of G^T, which is also a row slice of
// the GEMM2 operand.  Steps are numbered tile after tile: tile t starts at
// step T(t) = sum_{t' < t} (t'/2 + 1), i.e. T(2m) = m(m+1), T(2m+1) = (m+1)^2,
// and a chunk of Q tokens holds T(Q/16) steps.  Entries above the diagonal
// (and rows or columns past the sequence) are zero or unused.
#include "ssd_common.h"
#include "ssd_gemm1_body.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int N, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_gemm1_kernel(const TIn *__restrict__ Bm,
                                                              const TIn *__restrict__ Cm,
                                                              void *__restrict__ cb, int L, int G, int Q,
                                                              int nc)
{
    typedef Gemm1Chunk<TIn, N, NW, 16 * NW> K;
    __shared__ __align__(16) unsigned char smem[K::kLdsBytes];
    K::run(Bm, Cm, cb, L, G, G * N, Q, nc, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// Steps of 32 columns per chunk of q tokens (T(q/16) above).
int gemm1_steps_per_chunk(int q)
{
    const int nt = q / 16, m = nt / 2;
    return (nt & 1) ? (m + 1) * (m + 1) : m * (m + 1);
}

template <typename TIn>
static hipError_t launch_gemm1_t(const void *Bm, const void *Cm, void *cb, const Dims &d, hipStream_t s)
{
    const dim3 grid(d.nc, d.G, d.B);
    const TIn *bb = static_cast<const TIn *>(Bm), *cc = static_cast<const TIn *>(Cm);
#define SSD_G1_LAUNCH(NN, NWV) \
    launch_kernel("chunk_gemm1_kernel", chunk_gemm1_kernel<TIn, NN, NWV>, grid, 64 * NWV, s, bb, cc, cb, d.L, \
                  d.G, d.Q, d.nc)
#define SSD_G1_BY_Q(NN)          \
    if (d.Q == 256)              \
        SSD_G1_LAUNCH(NN, 16);   \
    else if (d.Q == 128)         \
        SSD_G1_LAUNCH(NN, 8);    \
    else                         \
        SSD_G1_LAUNCH(NN, 4)
    switch (d.N) {
    case 32: SSD_G1_BY_Q(32); break;
    case 64: SSD_G1_BY_Q(64); break;
    case 128: SSD_G1_BY_Q(128); break;
    case 256: SSD_G1_BY_Q(256); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_G1_BY_Q
#undef SSD_G1_LAUNCH
    return hipGetLastError();
}

hipError_t launch_chunk_gemm1(const void *Bm, const void *Cm, void *cb, const Dims &d, hipStream_t s)
{
    if (d.in == kInFp8) return launch_gemm1_t<fp8_t>(Bm, Cm, cb, d, s);
    return d.in == kInBf16 ? launch_gemm1_t<bf16_t>(Bm, Cm, cb, d, s) : launch_gemm1_t<float>(Bm, Cm, cb, d, s);
}

}  // namespace ssd
