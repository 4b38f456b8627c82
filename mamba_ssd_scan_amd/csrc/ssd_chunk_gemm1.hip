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
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int N, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_gemm1_kernel(const TIn *__restrict__ Bm,
                                                              const TIn *__restrict__ Cm,
                                                              void *__restrict__ cb, int L, int G, int Q,
                                                              int nc)
{
    typedef Traits<TIn> Tr;
    typedef typename Tr::raw_t raw_t;
    constexpr bool F32 = Tr::kF32;
    constexpr int ROWS = 16 * NW;               // chunk rows held in LDS (>= Q)
    constexpr int LDB = N + (F32 ? 4 : 8);      // row pitch: 16 rows read together hit distinct banks
    constexpr int KS = F32 ? N / 4 : N / 32;    // k steps over the state dim
    constexpr int NT = 64 * NW;
    __shared__ raw_t bs[ROWS * LDB];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const long tc = (long)c * Q;
    const int nt = Q >> 4;
    int t;  // row tile: the four wavefronts of a SIMD take tiles {s, 7-s, 8+s, 15-s}
    if (nt == NW && NW >= 8) {
        const int s = wave & 3, k = wave >> 2;
        t = 8 * (k >> 1) + ((k & 1) ? 7 - s : s);
    } else {
        t = wave < nt ? wave : -1;
    }
    const int ibase = 16 * t;

    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const size_t row0 = ((size_t)b * L + tc) * G + g;  // (token, group) row of the chunk's first token
    const uint32_t bytes = (uint32_t)(((vrows - 1) * G + 1) * N * sizeof(TIn));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bm + row0 * N, bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + row0 * N, bytes);

    // C rows of this wavefront's tile (the GEMM1^T B operand), kept in registers
    bf16x8 cbf[F32 ? 1 : KS];
    float cf[F32 ? KS : 1];
    {
        const uint32_t row = (uint32_t)((ibase + li) * G * N);
        if constexpr (F32) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                cf[ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(4u * (row + ks * 4 + lg)), 0, 0));
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cbf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
        }
    }
    // B rows of the whole chunk -> LDS (rows past the chunk or the sequence read as
    // zeros); a fixed trip count keeps every load in flight before the first store
    constexpr int BU = ROWS * (N / 8), BPT = (BU + NT - 1) / NT;
    Raw8<TIn> bv[BPT];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const int u = tid + k * NT;
        if (u < BU) bv[k].load(rb, (uint32_t)((u / (N / 8)) * G * N + 8 * (u % (N / 8))));
    }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const int u = tid + k * NT;
        if (u < BU) bv[k].store(&bs[(u / (N / 8)) * LDB + 8 * (u % (N / 8))]);
    }
    __syncthreads();
    if (t < 0) return;

    const int Tt = (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);
    const int spc = (nt & 1) ? ((nt >> 1) + 1) * ((nt >> 1) + 1) : (nt >> 1) * ((nt >> 1) + 1);
    const size_t slice0 = (((size_t)b * G + g) * nc + c) * (size_t)spc + Tt;  // this tile's first slice
    const int ns = (ibase + 15) / 32 + 1;
    for (int s = 0; s < ns; ++s) {
        const int jb = 32 * s;
        const bool has1 = jb + 16 <= ibase + 15;  // second 16-column half not entirely above the diagonal
        f32x4 d0 = zero4(), d1 = zero4();
        if constexpr (F32) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) d0 = mfma16x16x4_f32(bs[(jb + li) * LDB + ks * 4 + lg], cf[ks], d0);
            if (has1) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) d1 = mfma16x16x4_f32(bs[(jb + 16 + li) * LDB + ks * 4 + lg], cf[ks], d1);
            }
        } else {
            const raw_t *b0 = &bs[(jb + li) * LDB + 8 * lg];
            if (has1) {
                bf16x8 a0[KS], a1[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    a0[ks] = *reinterpret_cast<const bf16x8 *>(b0 + ks * 32);
                    a1[ks] = *reinterpret_cast<const bf16x8 *>(b0 + 16 * LDB + ks * 32);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    d0 = mfma16x16x32_bf16(a0[ks], cbf[ks], d0);
                    d1 = mfma16x16x32_bf16(a1[ks], cbf[ks], d1);
                }
            } else {
                bf16x8 a0[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a0[ks] = *reinterpret_cast<const bf16x8 *>(b0 + ks * 32);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) d0 = mfma16x16x32_bf16(a0[ks], cbf[ks], d0);
            }
        }
        if constexpr (F32) {
            float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(cb) + ((slice0 + s) * 64 + lane) * 8);
            o[0] = make_float4(d0[0], d0[1], d0[2], d0[3]);
            o[1] = make_float4(d1[0], d1[1], d1[2], d1[3]);
        } else {
            uint4 w;
            w.x = pack_f16x2(d0[0], d0[1]);
            w.y = pack_f16x2(d0[2], d0[3]);
            w.z = pack_f16x2(d1[0], d1[1]);
            w.w = pack_f16x2(d1[2], d1[3]);
            *reinterpret_cast<uint4 *>(static_cast<f16 *>(cb) + ((slice0 + s) * 64 + lane) * 8) = w;
        }
    }
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
    chunk_gemm1_kernel<TIn, NN, NWV><<<grid, 64 * NWV, 0, s>>>(bb, cc, cb, d.L, d.G, d.Q, d.nc)
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
    default: return hipErrorInvalidValue;
    }
#undef SSD_G1_BY_Q
#undef SSD_G1_LAUNCH
    return hipGetLastError();
}

hipError_t launch_chunk_gemm1(const void *Bm, const void *Cm, void *cb, const Dims &d, hipStream_t s)
{
    return d.bf16 ? launch_gemm1_t<bf16_t>(Bm, Cm, cb, d, s) : launch_gemm1_t<float>(Bm, Cm, cb, d, s);
}

}  // namespace ssd
