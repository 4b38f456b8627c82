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
// entering state and X are read from memory once.  Rows come in 16-row
// tiles; a wavefront owns one tile, or two (t and nt-1-t, which balances the
// causal triangle) when the chunk has twice as many tiles as wavefronts.
// Per 32-column step a wavefront computes two 16x16 tiles of G^T = B C^T on
// the matrix cores (bf16 inputs are exact operands), which leaves every lane
// holding one row i and four columns j of G per tile -- a row-slice of the
// GEMM2 A operand once the X operand uses the same column order.  The
// mask/decay/dt scaling is applied in registers and the result is rounded to
// fp16 for GEMM2 (bf16 would round the computed scores to 2^-9, too coarse
// for the error budget).  B and X are streamed through LDS in blocks of JB
// tokens, both row-major as they arrive from memory; the GEMM2 operand, whose
// reduction index is the token, is read with the transposing LDS read (fp32
// inputs store X transposed instead).  The blocks are double-buffered: the global loads of block k+1 are
// issued into registers before block k is computed and written to the other
// LDS buffer afterwards, so one barrier per block suffices and memory latency
// overlaps the matrix work.  Columns above the diagonal are skipped.
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <typename TIn, int P, int N, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu((NW == 8 && !Traits<TIn>::kF32) ? 4 : 2))) void chunk_scan_kernel(
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
    // X block: bf16 inputs keep it row-major [JB][P + 16] (fp16) and read the GEMM2
    // operand with the transposing LDS read; fp32 inputs store it transposed [P][JB + 4].
    constexpr int LDX = F32 ? JB + PADR : P + 16;
    constexpr int XSZ = F32 ? P * LDX : JB * LDX;
    constexpr int LDH = N + PADR;            // H_enter rows [P][N] (fp16), bf16 inputs only
    constexpr int TP = P / 16;
    constexpr int KS = F32 ? N / 4 : N / 32; // k steps over the state dim
    constexpr int MT = 2;                    // row tiles per wavefront (at most)
    constexpr int NT = 64 * NW;              // threads per workgroup
    constexpr int BU = JB * (N / 8), BPT = (BU + NT - 1) / NT;            // B block: 8-element units
    constexpr int XU = (JB / 2) * (P / 8), XPT = (XU + NT - 1) / NT;      // X block: two rows x 8 channels
    constexpr int HU = F32 ? 1 : P * N / 8, HPT = (HU + NT - 1) / NT;     // entering state
    __shared__ raw_t bs[2][JB * LDB];
    __shared__ op_t xs[2][XSZ];
    __shared__ op_t hs[F32 ? 1 : P * LDH];
    // chunk tables: cumulative decay in log2 units and dt, padded past Q so that the
    // column reads of the last 32-column step stay inside (padding is never used unmasked)
    __shared__ float acs[256 + 32], dts[256 + 32];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;  // first token of the chunk
    const int nblk = (Q + JB - 1) / JB;
    const int nt = Q >> 4;
    const int tile[MT] = {wave < nt ? wave : -1, nt > NW ? nt - 1 - wave : -1};

    Raw8<TIn> bpre[BPT];
    Raw8<TIn> xpre[XPT][2];

    // Buffer resources over this chunk's valid rows of X and B: loads of rows past
    // the chunk or the sequence return zeros.
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(x + ((size_t)b * L + tc) * H * P + (size_t)h * P, (uint32_t)(((vrows - 1) * H * P + P) * sizeof(TIn)));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(Bm + ((size_t)b * L + tc) * G * N + (size_t)g * N, (uint32_t)(((vrows - 1) * G * N + N) * sizeof(TIn)));

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
                const int jp = u / (P / 8), pg = u % (P / 8), j = j0 + 2 * jp;
#pragma unroll
                for (int e = 0; e < 2; ++e) xpre[k][e].load(rx, (uint32_t)((j + e) * H * P + 8 * pg));
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
                const int jp = u / (P / 8), pg = u % (P / 8);
                if constexpr (F32) {
                    float v0[8], v1[8];
                    xpre[k][0].to_f32(v0);
                    xpre[k][1].to_f32(v1);
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) store_pair(&xs[buf][(8 * pg + kk) * LDX + 2 * jp], v0[kk], v1[kk]);
                } else {
                    *reinterpret_cast<uint4 *>(&xs[buf][(2 * jp) * LDX + 8 * pg]) = raw8_to_f16x8(xpre[k][0]);
                    *reinterpret_cast<uint4 *>(&xs[buf][(2 * jp + 1) * LDX + 8 * pg]) = raw8_to_f16x8(xpre[k][1]);
                }
            }
        }
    };

    // ---- prologue: block 0, decay tables, entering state, C fragments
    prefetch(0);
    for (int i = tid; i < 256 + 32; i += NT) {
        acs[i] = i < Q ? acum[bhc * Q + i] * kLog2e : 0.f;
        dts[i] = i < Q ? dtc[bhc * Q + i] : 0.f;
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
    // C rows of this wavefront's tiles: GEMM1^T B operand and off-diagonal A operand
    bf16x8 cb[MT][F32 ? 1 : KS];
    float cf[MT][F32 ? KS : 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = tile[mt];
        const long ti = tc + 16 * t + li;
        const bool ok = t >= 0 && ti < L;
        const TIn *crow = Cm + (((size_t)b * L + (ok ? ti : 0)) * G + g) * N;
        if constexpr (F32) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cf[mt][ks] = ok ? crow[ks * 4 + lg] : 0.f;
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 u = make_uint4(0, 0, 0, 0);
                if (ok) u = *reinterpret_cast<const uint4 *>(crow + ks * 32 + 8 * lg);
                cb[mt][ks] = __builtin_bit_cast(bf16x8, u);
            }
        }
    }
    commit(0);
    __syncthreads();
    if (nblk > 1) prefetch(1);

    f32x4 acc[MT][TP];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[mt][pt] = zero4();

    // ---- Step-4: exp(a_i) * (C_i . H_enter[p, :]) for this wavefront's rows
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = tile[mt];
        if (t < 0) continue;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 ch;
            if constexpr (!F32) ch = bf16x8_to_f16x8(cb[mt][ks]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                if constexpr (F32) {
                    acc[mt][pt] = mfma16x16x4_f32(cf[mt][ks], hp[(pt * 16 + li) * N + ks * 4 + lg], acc[mt][pt]);
                } else {
                    const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                    acc[mt][pt] = mfma16x16x32_f16(ch, hf, acc[mt][pt]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(acs[16 * t + 4 * lg + r]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[mt][pt][r] *= e;
        }
    }

    const float Dh = D ? D[h] : 0.f;

    // ---- Step-1: stream the causal column blocks
    for (int jbk = 0; jbk < nblk; ++jbk) {
        const int buf = jbk & 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int t = tile[mt];
            if (t < 0) continue;
            const int ibase = 16 * t;
            if (jbk * JB > ibase + 15) continue;  // block entirely above this tile's diagonal
            const int irow = ibase + li;
            const float ai = acs[irow];
#pragma unroll
            for (int js = 0; js < JB; js += 32) {
                const int jb = jbk * JB + js;
                if (jb > ibase + 15) break;
                const bool has1 = jb + 16 <= ibase + 15;  // second 16-column tile not all masked
                // GEMM1^T: d0 = G^T[jb .. jb+15][rows], d1 = G^T[jb+16 .. jb+31][rows]
                f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if constexpr (F32) {
                        d0 = mfma16x16x4_f32(bs[buf][(js + li) * LDB + ks * 4 + lg], cf[mt][ks], d0);
                        if (has1) d1 = mfma16x16x4_f32(bs[buf][(js + 16 + li) * LDB + ks * 4 + lg], cf[mt][ks], d1);
                    } else {
                        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&bs[buf][(js + li) * LDB + ks * 32 + 8 * lg]);
                        d0 = mfma16x16x32_bf16(a0, cb[mt][ks], d0);
                        if (has1) {
                            const bf16x8 a1 =
                                *reinterpret_cast<const bf16x8 *>(&bs[buf][(js + 16 + li) * LDB + ks * 32 + 8 * lg]);
                            d1 = mfma16x16x32_bf16(a1, cb[mt][ks], d1);
                        }
                    }
                }
                // Hadamard: decay exp(a_i - a_j), dt_j and the causal mask, in registers.
                // Lane holds G[irow][jb + 4 lg + r] (d0) and G[irow][jb + 16 + 4 lg + r] (d1).
                const float4 a0v = *reinterpret_cast<const float4 *>(&acs[jb + 4 * lg]);
                const float4 t0v = *reinterpret_cast<const float4 *>(&dts[jb + 4 * lg]);
                const float4 a1v = *reinterpret_cast<const float4 *>(&acs[jb + 16 + 4 * lg]);
                const float4 t1v = *reinterpret_cast<const float4 *>(&dts[jb + 16 + 4 * lg]);
                const float aj0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, tj0[4] = {t0v.x, t0v.y, t0v.z, t0v.w};
                const float aj1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, tj1[4] = {t1v.x, t1v.y, t1v.z, t1v.w};
                float r0[4], r1[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    r0[r] = d0[r] * __builtin_amdgcn_exp2f(ai - aj0[r]) * tj0[r];
                    r1[r] = has1 ? d1[r] * __builtin_amdgcn_exp2f(ai - aj1[r]) * tj1[r] : 0.f;
                }
                if (jb + 31 > ibase) {  // the step reaches the diagonal: mask columns j > i
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (jb + 4 * lg + r > irow) r0[r] = 0.f;
                        if (jb + 16 + 4 * lg + r > irow) r1[r] = 0.f;
                    }
                }
                // GEMM2: k slots of lane group lg are columns {jb+4lg+r, jb+16+4lg+r}
                if constexpr (F32) {
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        const op_t *xr = &xs[buf][(pt * 16 + li) * LDX + js + 4 * lg];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][pt] = mfma16x16x4_f32(r0[r], xr[r], acc[mt][pt]);
                        if (has1) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[mt][pt] = mfma16x16x4_f32(r1[r], xr[16 + r], acc[mt][pt]);
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
                        acc[mt][pt] = mfma16x16x32_f16(a, bx, acc[mt][pt]);
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

    // ---- epilogue: skip term and store; lane holds rows 16t + 4 lg + r, column 16 pt + li
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = tile[mt];
        if (t < 0) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long tt = tc + 16 * t + 4 * lg + r;
            if (tt < L) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const size_t idx = (((size_t)b * L + tt) * H + h) * P + pt * 16 + li;
                    y[idx] = acc[mt][pt][r] + Dh * load_in(x + idx);
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
    // 8 wavefronts (two 16-row tiles each) for 256-token chunks, else 4.
    const dim3 grid(d.nc, d.H, d.B);
    const TIn *xx = static_cast<const TIn *>(x), *bb = static_cast<const TIn *>(Bm),
              *cc = static_cast<const TIn *>(Cm);
#define SSD_SCAN_LAUNCH(NN, NWV)                                                                     \
    chunk_scan_kernel<TIn, P, NN, NWV><<<grid, 64 * NWV, 0, s>>>(xx, bb, cc, acum, dtc, hen, D, y, d.L, \
                                                                 d.H, d.G, d.Q, d.nc)
    const bool wide = d.Q == 256;  // 8 wavefronts (two 16-row tiles each) for 256-token chunks, else 4
    switch (d.N) {
    case 32: if (wide) SSD_SCAN_LAUNCH(32, 8); else SSD_SCAN_LAUNCH(32, 4); break;
    case 64: if (wide) SSD_SCAN_LAUNCH(64, 8); else SSD_SCAN_LAUNCH(64, 4); break;
    case 128: if (wide) SSD_SCAN_LAUNCH(128, 8); else SSD_SCAN_LAUNCH(128, 4); break;
    default: return hipErrorInvalidValue;
    }
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
