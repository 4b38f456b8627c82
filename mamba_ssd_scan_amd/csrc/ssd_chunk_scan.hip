// ssd_chunk_scan.hip -- Step-1 (intra-chunk) + Step-4 (off-diagonal) + skip.
//
// For token i of chunk c (chunk-local index), with the chunk's cumulative
// decay a = dA_cum and the state H_enter entering the chunk:
//
//   y_i = sum_{j<=i} (C_i . B_j) exp(a_i - a_j) dt_j x_j     Step-1: GEMM1 over N,
//                                                            Hadamard mask, GEMM2 over j
//       + exp(a_i) H_enter C_i                               Step-4: off-diagonal
//       + D_h x_i                                            skip
//
// Sources: "Mamba-Family State-Space Model Kernels on a Programmable CGLA",
// Sec. III-A and IV-B (Step-1 = GEMM1, element-wise mask of R, GEMM2; a
// fused mask+GEMM2 removes a round trip per chunk) and "Mambalaya: Einsum-
// Based Fusion Optimizations on State-Space Models", Fig. 2-5 (fusing
// consecutive Einsums removes the inter-Einsum traffic).  Here GEMM1, the
// mask, GEMM2, the off-diagonal product and the skip term are fused in one
// kernel: the score tile never leaves registers.
//
// Work split: one 256-thread workgroup per (b, h, c, block of IB = min(64, Q)
// rows); each wavefront owns 16 rows.  Per 32-column step it computes two
// 16x16 tiles of G^T = B C^T on the matrix cores (bf16 inputs are exact
// operands), which leaves every lane holding one row i and four columns j of
// G per tile -- exactly a row-slice of the GEMM2 A operand once the same
// column order is used for the X operand.  The mask/decay/dt scaling is
// applied in registers and the result is rounded to fp16 for GEMM2 (bf16
// would round the computed scores to 2^-9, too coarse for the error budget).
// B and X blocks of 64 tokens are staged in LDS (X transposed); the entering
// state is staged once as fp16.  Columns above the diagonal are skipped.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
    const float *__restrict__ acum, const float *__restrict__ dtc, const float *__restrict__ hen,
    const float *__restrict__ D, float *__restrict__ y, int L, int H, int G, int Q, int nc)
{
    typedef Traits<TIn> Tr;
    typedef typename Tr::op_t op_t;
    typedef typename Tr::raw_t raw_t;
    constexpr bool F32 = Tr::kF32;
    constexpr int JB = F32 ? 32 : 64;        // tokens per staged block
    constexpr int PADR = F32 ? 4 : 8;
    constexpr int LDB = N + PADR;            // B rows [JB][N] (raw inputs)
    constexpr int LDX = JB + PADR;           // X^T rows [P][JB] (operand type)
    constexpr int LDH = N + PADR;            // H_enter rows [P][N] (fp16), bf16 inputs only
    constexpr int TP = P / 16;
    constexpr int KS = F32 ? N / 4 : N / 32; // k steps over the state dim
    __shared__ raw_t bs[JB * LDB];
    __shared__ op_t xs[P * LDX];
    __shared__ op_t hs[F32 ? 1 : P * LDH];
    __shared__ float acs[256], dts[256];

    const int IB = Q < 64 ? Q : 64;
    const int nib = Q / IB;
    const int ib = nib - 1 - (int)(blockIdx.x % nib);  // heavier row blocks first
    const int c = blockIdx.x / nib;
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;  // first token of the chunk

    for (int i = tid; i < Q; i += 256) {
        acs[i] = acum[bhc * Q + i];
        dts[i] = dtc[bhc * Q + i];
    }
    const float *hp = hen + bhc * P * N;
    if constexpr (!F32) {
        for (int u = tid; u < P * N / 8; u += 256) {
            const int row = u / (N / 8), cg = u % (N / 8);
            const float4 a = *reinterpret_cast<const float4 *>(hp + row * N + 8 * cg);
            const float4 bq = *reinterpret_cast<const float4 *>(hp + row * N + 8 * cg + 4);
            uint4 w;
            w.x = pack_f16x2(a.x, a.y);
            w.y = pack_f16x2(a.z, a.w);
            w.z = pack_f16x2(bq.x, bq.y);
            w.w = pack_f16x2(bq.z, bq.w);
            *reinterpret_cast<uint4 *>(&hs[row * LDH + 8 * cg]) = w;
        }
    }

    // This wavefront's 16 rows; lane feeds row `irow` to GEMM1^T and the off-diagonal product.
    const bool active = wave < IB / 16;
    const int ibase = ib * IB + wave * 16;
    const int irow = ibase + li;
    const long ti = tc + irow;
    const bool row_ok = active && irow < Q && ti < L;
    const TIn *crow = Cm + (((size_t)b * L + (row_ok ? ti : 0)) * G + g) * N;

    // C fragments: raw (GEMM1) and operand-typed (off-diagonal) copies
    bf16x8 cb[F32 ? 1 : KS];
    f16x8 ch[F32 ? 1 : KS];
    float cf[F32 ? KS : 1];
    if constexpr (F32) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) cf[ks] = row_ok ? crow[ks * 4 + lg] : 0.f;
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok) u = *reinterpret_cast<const uint4 *>(crow + ks * 32 + 8 * lg);
            cb[ks] = __builtin_bit_cast(bf16x8, u);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ch[ks][2 * k] = static_cast<f16>(__uint_as_float(w[k] << 16));
                ch[ks][2 * k + 1] = static_cast<f16>(__uint_as_float(w[k] & 0xFFFF0000u));
            }
        }
    }
    __syncthreads();

    f32x4 acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();

    // ---- Step-4: exp(a_i) * (C_i . H_enter[p, :])
    if (active) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                if constexpr (F32) {
                    acc[pt] = mfma16x16x4_f32(cf[ks], hp[(pt * 16 + li) * N + ks * 4 + lg], acc[pt]);
                } else {
                    const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                    acc[pt] = mfma16x16x32_f16(ch[ks], hf, acc[pt]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ibase + 4 * lg + r;
            const float e = exp_fast(acs[i < Q ? i : Q - 1]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= e;
        }
    }

    // ---- Step-1: causal blocks of columns j < end of this row block
    const int iend = ib * IB + IB;
    const float ai = acs[irow < Q ? irow : Q - 1];
    for (int j0 = 0; j0 < iend; j0 += JB) {
        __syncthreads();  // the previous block is no longer read
        for (int u = tid; u < JB * (N / 8); u += 256) {
            const int jr = u / (N / 8), cg = u % (N / 8);
            const int j = j0 + jr;
            raw_t *dst = &bs[jr * LDB + 8 * cg];
            const bool ok = j < Q && tc + j < L;
            const TIn *src = Bm + (((size_t)b * L + (ok ? tc + j : 0)) * G + g) * N + 8 * cg;
            if constexpr (F32) {
                float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bq = a;
                if (ok) {
                    a = reinterpret_cast<const float4 *>(src)[0];
                    bq = reinterpret_cast<const float4 *>(src)[1];
                }
                reinterpret_cast<float4 *>(dst)[0] = a;
                reinterpret_cast<float4 *>(dst)[1] = bq;
            } else {
                *reinterpret_cast<uint4 *>(dst) = ok ? *reinterpret_cast<const uint4 *>(src) : make_uint4(0, 0, 0, 0);
            }
        }
        constexpr int XG = P / 8;
        for (int u = tid; u < (JB / 2) * XG; u += 256) {
            const int jp = u / XG, pg = u % XG;
            const int j = j0 + 2 * jp;
            float v0[8], v1[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v0[k] = v1[k] = 0.f;
            if (j < Q && tc + j < L) load8(x + (((size_t)b * L + tc + j) * H + h) * P + 8 * pg, v0);
            if (j + 1 < Q && tc + j + 1 < L) load8(x + (((size_t)b * L + tc + j + 1) * H + h) * P + 8 * pg, v1);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                op_t *dst = &xs[(8 * pg + k) * LDX + 2 * jp];
                if constexpr (F32) {
                    *reinterpret_cast<float2 *>(dst) = make_float2(v0[k], v1[k]);
                } else {
                    *reinterpret_cast<uint32_t *>(dst) = pack_f16x2(v0[k], v1[k]);
                }
            }
        }
        __syncthreads();
        if (!active) continue;

        for (int js = 0; js < JB; js += 32) {
            const int jb = j0 + js;
            if (jb > ibase + 15) break;                 // whole step above the diagonal
            const bool has1 = jb + 16 <= ibase + 15;    // second 16-column tile not all masked
            // GEMM1^T: d0 = G^T[jb .. jb+15][rows], d1 = G^T[jb+16 .. jb+31][rows]
            f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (F32) {
                    d0 = mfma16x16x4_f32(bs[(js + li) * LDB + ks * 4 + lg], cf[ks], d0);
                    if (has1) d1 = mfma16x16x4_f32(bs[(js + 16 + li) * LDB + ks * 4 + lg], cf[ks], d1);
                } else {
                    const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&bs[(js + li) * LDB + ks * 32 + 8 * lg]);
                    d0 = mfma16x16x32_bf16(a0, cb[ks], d0);
                    if (has1) {
                        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(&bs[(js + 16 + li) * LDB + ks * 32 + 8 * lg]);
                        d1 = mfma16x16x32_bf16(a1, cb[ks], d1);
                    }
                }
            }
            // Hadamard: causal mask, decay exp(a_i - a_j) and dt_j, in registers.
            // Lane holds G[irow][jb + 4 lg + r] (d0) and G[irow][jb + 16 + 4 lg + r] (d1).
            float r0[4], r1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jb + 4 * lg + r;
                const int jc = j < Q ? j : Q - 1;
                r0[r] = (j <= irow) ? d0[r] * exp_fast(ai - acs[jc]) * dts[jc] : 0.f;
                const int j1 = j + 16;
                const int j1c = j1 < Q ? j1 : Q - 1;
                r1[r] = (has1 && j1 <= irow) ? d1[r] * exp_fast(ai - acs[j1c]) * dts[j1c] : 0.f;
            }
            // GEMM2: k slots of lane group lg are columns {jb+4lg+r, jb+16+4lg+r}
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                const op_t *xr = &xs[(pt * 16 + li) * LDX + js + 4 * lg];
                if constexpr (F32) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(r0[r], xr[r], acc[pt]);
                    if (has1) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(r1[r], xr[16 + r], acc[pt]);
                    }
                } else {
                    f16x8 a;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a[r] = static_cast<f16>(r0[r]);
                        a[4 + r] = static_cast<f16>(r1[r]);
                    }
                    const f16x4 lo = *reinterpret_cast<const f16x4 *>(xr);
                    const f16x4 hi = *reinterpret_cast<const f16x4 *>(xr + 16);
                    const f16x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[pt] = mfma16x16x32_f16(a, bx, acc[pt]);
                }
            }
        }
    }

    // ---- epilogue: skip term and store; lane holds rows ibase + 4 lg + r, column 16 pt + li
    if (active) {
        const float Dh = D ? D[h] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ibase + 4 * lg + r;
            const long t = tc + i;
            if (i < Q && t < L) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const size_t idx = (((size_t)b * L + t) * H + h) * P + pt * 16 + li;
                    y[idx] = acc[pt][r] + Dh * load_in(x + idx);
                }
            }
        }
    }
}

template <typename TIn, int P>
static hipError_t launch_scan_n(const void *x, const void *Bm, const void *Cm, const float *acum,
                                const float *dtc, const float *hen, const float *D, float *y,
                                const Dims &d, hipStream_t s)
{
    const int nib = d.Q < 64 ? 1 : d.Q / 64;
    const dim3 grid(d.nc * nib, d.H, d.B);
    const TIn *xx = static_cast<const TIn *>(x), *bb = static_cast<const TIn *>(Bm),
              *cc = static_cast<const TIn *>(Cm);
    switch (d.N) {
    case 32: chunk_scan_kernel<TIn, P, 32><<<grid, 256, 0, s>>>(xx, bb, cc, acum, dtc, hen, D, y, d.L, d.H, d.G, d.Q, d.nc); break;
    case 64: chunk_scan_kernel<TIn, P, 64><<<grid, 256, 0, s>>>(xx, bb, cc, acum, dtc, hen, D, y, d.L, d.H, d.G, d.Q, d.nc); break;
    case 128: chunk_scan_kernel<TIn, P, 128><<<grid, 256, 0, s>>>(xx, bb, cc, acum, dtc, hen, D, y, d.L, d.H, d.G, d.Q, d.nc); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_scan_t(const void *x, const void *Bm, const void *Cm, const float *acum,
                                const float *dtc, const float *hen, const float *D, float *y,
                                const Dims &d, hipStream_t s)
{
    switch (d.P) {
    case 32: return launch_scan_n<TIn, 32>(x, Bm, Cm, acum, dtc, hen, D, y, d, s);
    case 64: return launch_scan_n<TIn, 64>(x, Bm, Cm, acum, dtc, hen, D, y, d, s);
    case 128: return launch_scan_n<TIn, 128>(x, Bm, Cm, acum, dtc, hen, D, y, d, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_scan(const void *x, const void *Bm, const void *Cm, const float *acum,
                             const float *dtc, const float *h_enter, const float *D, float *y,
                             const Dims &d, hipStream_t s)
{
    return d.bf16 ? launch_scan_t<bf16_t>(x, Bm, Cm, acum, dtc, h_enter, D, y, d, s)
                  : launch_scan_t<float>(x, Bm, Cm, acum, dtc, h_enter, D, y, d, s);
}

}  // namespace ssd
