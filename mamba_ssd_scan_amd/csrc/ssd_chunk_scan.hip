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
// Work split: one workgroup per (b, h, c) covering the whole chunk, so the
// entering state and X are read from memory once, and one wavefront per
// 16-row tile (16 wavefronts for Q = 256).  The four wavefronts that share a
// SIMD take tiles {s, 7-s, 8+s, 15-s}, which balances the causal triangle
// across the SIMDs.  Per 32-column step a wavefront computes two 16x16 tiles
// of G^T = B C^T on the matrix cores (bf16 inputs are exact operands), which
// leaves every lane holding one row i and four columns j of G per tile -- a
// row-slice of the GEMM2 A operand once the X operand uses the same column
// order.  The mask/decay/dt scaling is applied in registers and the result is
// rounded to fp16 for GEMM2 (bf16 would round the computed scores to 2^-9,
// too coarse for the error budget).  B and X are streamed through LDS in
// blocks of JB tokens, both row-major as they arrive from memory; the GEMM2
// operand, whose reduction index is the token, is read with the transposing
// LDS read (fp32 inputs store X transposed instead).  The blocks are
// double-buffered: the global loads of block k+1 are issued into registers
// before block k is computed and written to the other LDS buffer afterwards,
// so one barrier per block suffices and memory latency overlaps the matrix
// work.  Columns above the diagonal are skipped.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int P, int N, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_scan_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
    const float *__restrict__ acum, const float *__restrict__ dtc, const float *__restrict__ hen,
    const float *__restrict__ D, float *__restrict__ y, int L, int H, int G, int Q, int nc)
{
    typedef Traits<TIn> Tr;
    typedef typename Tr::op_t op_t;
    typedef typename Tr::raw_t raw_t;
    constexpr bool F32 = Tr::kF32;
    constexpr int JB = F32 ? 32 : 64;        // tokens per staged block
    constexpr int LDB = N + (F32 ? 4 : 8);   // B rows [JB][N] (raw inputs)
    // X block: bf16 inputs keep it row-major [JB][P + 16] (fp16) and read the GEMM2
    // operand with the transposing LDS read; fp32 inputs store it transposed [P][JB + 4].
    constexpr int LDX = F32 ? JB + 4 : P + 16;
    constexpr int XSZ = F32 ? P * LDX : JB * LDX;
    constexpr int LDH = N + 8;               // H_enter rows [P][N] (fp16), bf16 inputs only
    constexpr int TP = P / 16;
    constexpr int KS = F32 ? N / 4 : N / 32; // k steps over the state dim
    constexpr int NT = 64 * NW;              // threads per workgroup
    constexpr int BU = JB * (N / 8), BPT = (BU + NT - 1) / NT;       // B block: one row x 8 channels
    constexpr int XR = F32 ? 2 : 1;                                  // X rows per staging unit
    constexpr int XU = (JB / XR) * (P / 8), XPT = (XU + NT - 1) / NT;
    constexpr int HU = F32 ? 1 : P * N / 8, HPT = (HU + NT - 1) / NT;  // entering state
    __shared__ raw_t bs[2][JB * LDB];
    __shared__ op_t xs[2][XSZ];
    __shared__ op_t hs[F32 ? 1 : P * LDH];
    // chunk tables, padded past Q so that the column reads of the last 32-column step
    // stay inside (padding is never used unmasked): cumulative decay in log2 units, dt,
    // and exp(a_r - a_j) dt_j with a_r the last column of j's 32-column step
    __shared__ float acs[256 + 32], dts[256 + 32], ecs[256 + 32];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
    const int li = lane & 15, lg = lane >> 4;
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;  // first token of the chunk
    const int nblk = (Q + JB - 1) / JB;
    const int nt = Q >> 4;
    // this wavefront's row tile: the k-th wavefront on SIMD s (wave = 4k + s) takes
    // tile 8(k/2) + s for even k and 8(k/2) + 7 - s for odd k
    int t;
    if (nt == NW && NW >= 8) {
        const int s = wave & 3, k = wave >> 2;
        t = 8 * (k >> 1) + ((k & 1) ? 7 - s : s);
    } else {
        t = wave < nt ? wave : -1;
    }
    const int ibase = 16 * t;

    // Buffer resources over this chunk's valid rows of X and B: loads of rows past
    // the chunk or the sequence return zeros.
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(x + ((size_t)b * L + tc) * H * P + (size_t)h * P, (uint32_t)(((vrows - 1) * H * P + P) * sizeof(TIn)));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(Bm + ((size_t)b * L + tc) * G * N + (size_t)g * N, (uint32_t)(((vrows - 1) * G * N + N) * sizeof(TIn)));

    Raw8<TIn> bpre[BPT];
    Raw8<TIn> xpre[XPT][XR];
    auto prefetch = [&](int jbk) {
        const int j0 = jbk * JB;
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * NT;
            if (u < BU) {
                const int jr = u / (N / 8), cg = u % (N / 8);
                bpre[k].load(rb, (uint32_t)((j0 + jr) * G * N + 8 * cg));
            }
        }
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * NT;
            if (u < XU) {
                const int jr = u / (P / 8), cg = u % (P / 8), j = j0 + XR * jr;
#pragma unroll
                for (int e = 0; e < XR; ++e) xpre[k][e].load(rx, (uint32_t)((j + e) * H * P + 8 * cg));
            }
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * NT;
            if (u < BU) {
                const int jr = u / (N / 8), cg = u % (N / 8);
                bpre[k].store(&bs[buf][jr * LDB + 8 * cg]);
            }
        }
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * NT;
            if (u < XU) {
                const int jr = u / (P / 8), cg = u % (P / 8);
                if constexpr (F32) {
                    float v0[8], v1[8];
                    xpre[k][0].to_f32(v0);
                    xpre[k][XR - 1].to_f32(v1);
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) store_pair(&xs[buf][(8 * cg + kk) * LDX + 2 * jr], v0[kk], v1[kk]);
                } else {
                    *reinterpret_cast<uint4 *>(&xs[buf][jr * LDX + 8 * cg]) = raw8_to_f16x8(xpre[k][0]);
                }
            }
        }
    };

    // ---- prologue: C fragments, block 0, decay tables, entering state.  The C loads
    // go first: the wait for block 0 then covers them on every path, so no wait for
    // them is left inside the main loop (which would also drain the next prefetch).
    // C rows of this wavefront's tile: GEMM1^T B operand and off-diagonal A operand
    bf16x8 cb[F32 ? 1 : KS];
    float cf[F32 ? KS : 1];
    {
        // buffer resource over this chunk's valid rows of C: rows past the sequence (and
        // the negative offsets of a wavefront without a tile) read as zeros, no branches
        const int vr = (int)((L - tc) < Q ? (L - tc) : Q);
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(Cm + ((size_t)b * L + tc) * G * N + (size_t)g * N, (uint32_t)(((vr - 1) * G * N + N) * sizeof(TIn)));
        const uint32_t row = (uint32_t)((ibase + li) * G * N);
        if constexpr (F32) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                cf[ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(4u * (row + ks * 4 + lg)), 0, 0));
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
        }
    }
    prefetch(0);
    for (int i = tid; i < 256 + 32; i += NT) {
        float a = 0.f, d = 0.f, e = 0.f;
        if (i < Q) {
            const int ir = min(32 * (i >> 5) + 31, Q - 1);
            a = acum[bhc * Q + i] * kLog2e;
            d = dtc[bhc * Q + i];
            e = __builtin_amdgcn_exp2f(acum[bhc * Q + ir] * kLog2e - a) * d;
        }
        acs[i] = a;
        dts[i] = d;
        ecs[i] = e;
    }
    const float *hp = hen + bhc * P * N;
    if constexpr (!F32) {
        float4 hv[HPT][2];
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int u = tid + k * NT;
            if (u < HU) {
                const int row = u / (N / 8), cg = u % (N / 8);
                hv[k][0] = *reinterpret_cast<const float4 *>(hp + row * N + 8 * cg);
                hv[k][1] = *reinterpret_cast<const float4 *>(hp + row * N + 8 * cg + 4);
            }
        }
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int u = tid + k * NT;
            if (u < HU) {
                const int row = u / (N / 8), cg = u % (N / 8);
                uint4 w;
                w.x = pack_f16x2(hv[k][0].x, hv[k][0].y);
                w.y = pack_f16x2(hv[k][0].z, hv[k][0].w);
                w.z = pack_f16x2(hv[k][1].x, hv[k][1].y);
                w.w = pack_f16x2(hv[k][1].z, hv[k][1].w);
                *reinterpret_cast<uint4 *>(&hs[row * LDH + 8 * cg]) = w;
            }
        }
    }
    const float Dh = D ? D[h] : 0.f;
    commit(0);
    __syncthreads();
    if (nblk > 1) prefetch(1);

    f32x4 acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();

    // ---- Step-4: exp(a_i) * (C_i . H_enter[p, :]) for this wavefront's rows
    if (t >= 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 ch;
            if constexpr (!F32) ch = bf16x8_to_f16x8(cb[ks]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                if constexpr (F32) {
                    acc[pt] = mfma16x16x4_f32(cf[ks], hp[(pt * 16 + li) * N + ks * 4 + lg], acc[pt]);
                } else {
                    const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                    acc[pt] = mfma16x16x32_f16(ch, hf, acc[pt]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(acs[ibase + 4 * lg + r]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= e;
        }
    }

    // ---- Step-1: stream the causal column blocks
    const int irow = ibase + li;
    const float ai = t >= 0 ? acs[irow] : 0.f;
    for (int jbk = 0; jbk < nblk; ++jbk) {
        const int buf = jbk & 1;
        if (t >= 0 && jbk * JB <= ibase + 15) {
#pragma unroll
            for (int js = 0; js < JB; js += 32) {
                const int jb = jbk * JB + js;
                if (jb > ibase + 15) break;                 // whole step above the diagonal
                const bool has1 = jb + 16 <= ibase + 15;    // second 16-column tile not all masked
                // GEMM1^T: d0 = G^T[jb .. jb+15][rows], d1 = G^T[jb+16 .. jb+31][rows]
                // (has1 is wave-uniform; testing it outside the k loop keeps each variant
                // straight-line, so the LDS reads are issued together ahead of the MFMAs)
                f32x4 d0 = zero4(), d1 = zero4();
                if constexpr (F32) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) d0 = mfma16x16x4_f32(bs[buf][(js + li) * LDB + ks * 4 + lg], cf[ks], d0);
                    if (has1) {
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks)
                            d1 = mfma16x16x4_f32(bs[buf][(js + 16 + li) * LDB + ks * 4 + lg], cf[ks], d1);
                    }
                } else {
                    const raw_t *b0 = &bs[buf][(js + li) * LDB + 8 * lg];
                    if (has1) {
                        bf16x8 a0[KS], a1[KS];
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            a0[ks] = *reinterpret_cast<const bf16x8 *>(b0 + ks * 32);
                            a1[ks] = *reinterpret_cast<const bf16x8 *>(b0 + 16 * LDB + ks * 32);
                        }
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            d0 = mfma16x16x32_bf16(a0[ks], cb[ks], d0);
                            d1 = mfma16x16x32_bf16(a1[ks], cb[ks], d1);
                        }
                    } else {
                        bf16x8 a0[KS];
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) a0[ks] = *reinterpret_cast<const bf16x8 *>(b0 + ks * 32);
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) d0 = mfma16x16x32_bf16(a0[ks], cb[ks], d0);
                    }
                }
                // Hadamard: decay exp(a_i - a_j), dt_j and the causal mask, in registers.
                // Lane holds G[irow][jb + 4 lg + r] (d0) and G[irow][jb + 16 + 4 lg + r] (d1).
                float r0[4], r1[4];
                if (jb + 31 <= ibase) {
                    // Step strictly below the diagonal: factor the decay through the step's
                    // last column a_r, exp(a_i - a_j) = exp(a_i - a_r) exp(a_r - a_j).  Both
                    // factors are <= 1 (a is non-increasing for A <= 0) and any underflow
                    // drops a term smaller still; exp(a_r - a_j) dt_j is the chunk table.
                    const float er = __builtin_amdgcn_exp2f(ai - acs[jb + 31]);
                    const float4 e0 = *reinterpret_cast<const float4 *>(&ecs[jb + 4 * lg]);
                    const float4 e1 = *reinterpret_cast<const float4 *>(&ecs[jb + 16 + 4 * lg]);
                    const float ej0[4] = {e0.x, e0.y, e0.z, e0.w}, ej1[4] = {e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        r0[r] = d0[r] * (er * ej0[r]);
                        r1[r] = d1[r] * (er * ej1[r]);
                    }
                } else {
                    // diagonal step: direct exponentials under the causal mask
                    const float4 a0v = *reinterpret_cast<const float4 *>(&acs[jb + 4 * lg]);
                    const float4 t0v = *reinterpret_cast<const float4 *>(&dts[jb + 4 * lg]);
                    const float4 a1v = *reinterpret_cast<const float4 *>(&acs[jb + 16 + 4 * lg]);
                    const float4 t1v = *reinterpret_cast<const float4 *>(&dts[jb + 16 + 4 * lg]);
                    const float aj0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, tj0[4] = {t0v.x, t0v.y, t0v.z, t0v.w};
                    const float aj1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, tj1[4] = {t1v.x, t1v.y, t1v.z, t1v.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        r0[r] = (jb + 4 * lg + r <= irow) ? d0[r] * __builtin_amdgcn_exp2f(ai - aj0[r]) * tj0[r] : 0.f;
                        r1[r] = (has1 && jb + 16 + 4 * lg + r <= irow) ? d1[r] * __builtin_amdgcn_exp2f(ai - aj1[r]) * tj1[r]
                                                                       : 0.f;
                    }
                }
                // GEMM2: k slots of lane group lg are columns {jb+4lg+r, jb+16+4lg+r}
                if constexpr (F32) {
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        const op_t *xr = &xs[buf][(pt * 16 + li) * LDX + js + 4 * lg];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(r0[r], xr[r], acc[pt]);
                        if (has1) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(r1[r], xr[16 + r], acc[pt]);
                        }
                    }
                } else {
                    f16x8 a;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a[r] = static_cast<f16>(r0[r]);
                        a[4 + r] = static_cast<f16>(r1[r]);
                    }
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        // lane li receives X[jb + 4 lg + r][16 pt + li] and X[jb + 16 + 4 lg + r][16 pt + li]
                        const int ox = tr16_offset(lane, js, pt * 16, LDX);
                        const f16x4 lo = lds_read_tr16(&xs[buf][ox]);
                        const f16x4 hi = lds_read_tr16(&xs[buf][ox + 16 * LDX]);
                        const f16x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc[pt] = mfma16x16x32_f16(a, bx, acc[pt]);
                    }
                }
            }
            if (ibase / JB == jbk) {
                // This block holds the tile's own rows, so the tile is complete: add the skip
                // term and store it now, while the other wavefronts still compute.
                if constexpr (!F32) {
                    // the transposing read hands lane li the values X[ibase + 4 lg + r][16 pt + li],
                    // exactly the accumulator positions (exact for bf16 inputs in fp16 range)
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        const f16x4 xv = lds_read_tr16(&xs[buf][tr16_offset(lane, ibase - jbk * JB, pt * 16, LDX)]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * static_cast<float>(xv[r]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const long tt = tc + ibase + 4 * lg + r;
                    if (tt < L) {
#pragma unroll
                        for (int pt = 0; pt < TP; ++pt) {
                            const size_t idx = (((size_t)b * L + tt) * H + h) * P + pt * 16 + li;
                            if constexpr (F32)
                                y[idx] = acc[pt][r] + Dh * load_in(x + idx);
                            else
                                y[idx] = acc[pt][r];
                        }
                    }
                }
            }
        }
        if (jbk + 1 < nblk) {
            commit(buf ^ 1);  // the other buffer was last read before the previous barrier
            __syncthreads();
            if (jbk + 2 < nblk) prefetch(jbk + 2);
        }
    }

}

template <typename TIn, int P>
static hipError_t launch_scan_n(const void *x, const void *Bm, const void *Cm, const float *acum,
                                const float *dtc, const float *hen, const float *D, float *y,
                                const Dims &d, hipStream_t s)
{
    const dim3 grid(d.nc, d.H, d.B);
    const TIn *xx = static_cast<const TIn *>(x), *bb = static_cast<const TIn *>(Bm),
              *cc = static_cast<const TIn *>(Cm);
#define SSD_SCAN_LAUNCH(NN, NWV)                                                                      \
    chunk_scan_kernel<TIn, P, NN, NWV><<<grid, 64 * NWV, 0, s>>>(xx, bb, cc, acum, dtc, hen, D, y, d.L, \
                                                                 d.H, d.G, d.Q, d.nc)
#define SSD_SCAN_BY_Q(NN)                                  \
    if (d.Q == 256)                                        \
        SSD_SCAN_LAUNCH(NN, 16);                           \
    else if (d.Q == 128)                                   \
        SSD_SCAN_LAUNCH(NN, 8);                            \
    else                                                   \
        SSD_SCAN_LAUNCH(NN, 4)
    // one wavefront per 16-row tile (4 for chunks of 64 tokens or fewer)
    switch (d.N) {
    case 32: SSD_SCAN_BY_Q(32); break;
    case 64: SSD_SCAN_BY_Q(64); break;
    case 128: SSD_SCAN_BY_Q(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_SCAN_BY_Q
#undef SSD_SCAN_LAUNCH
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
