// ssd_chunk_state_pair.hip -- Step-0 and Step-2 for two heads per workgroup, with the
// Step-1 GEMM1 workgroups in the same grid: the prefill's first launch for bf16 and fp8
// problems with 256-token chunks, P = 64 and an even number of heads per group.
//
// Same arithmetic, in the same order, as ssd_chunk_state.hip with the fused cumulative
// decay ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A:
// the chunk state S_c = (X_c * w)^T B_c with w_j = exp(dA_cum[Q-1] - dA_cum[j]) dt_j),
// so the results are the same bit for bit.  What differs is the work split: every head
// of a group reads the same B rows of a chunk, so a workgroup of 8 wavefronts takes two
// heads of one group (wavefronts 0-3 and 4-7, each half as the single-head kernel's
// workgroup does) and stages the chunk's B rows once for both.  That removes a quarter
// of the launch's reads through the compute units' load path (the B rows were read once
// per head), which is what bounds this launch when its whole grid is resident.
//
// The whole chunk is requested at once (four 64-token blocks in registers), then
// contracted block by block through double-buffered LDS with one barrier per block.  fp8
// inputs are requested 16 values per load (one token's 16 channels or state columns), half
// the loads of the bf16 layout for the same elements.
// Workgroups share nothing, so the grid may take any number of rounds; on grids much
// larger than the GPU the whole-chunk requests keep 128 KB of X per compute unit in
// flight (two workgroups of two heads), which is what HBM needs to stream near its rate.
#include "ssd_common.h"
#include "ssd_gemm1_body.h"
#include "ssd_launch.h"

namespace ssd {

// TX: storage of x, B and C (bf16 or fp8 e4m3); dt is bf16 either way.  XCP: cache policy of
// the X loads (kStream when X cannot stay in the Infinity Cache until the chunk scan reads it).
template <typename TX, int N, int XCP>
__global__ __launch_bounds__(512) void chunk_state_pair_kernel(
    const TX *__restrict__ x, const TX *__restrict__ Bm, const bf16_t *__restrict__ dt,
    const float *__restrict__ A, float *__restrict__ acum, float *__restrict__ dtc, f16 *__restrict__ states,
    const TX *__restrict__ Cm, void *__restrict__ cb, SsdOpts opt, int L, int H, int G, int sx, int sbc, int sdt,
    int nc)
{
    constexpr int P = 64, Q = 256, JB = 64, NBLK = Q / JB;
    constexpr int LDXR = P + 16, LDBR = N + 16;  // (width + 16) halves: the transposing reads hit distinct banks
    constexpr int XSZ = JB * LDXR, BSZ = JB * LDBR;
    constexpr int TP = P / 16, TN = N / 16, NT = TP * TN;
    constexpr int TPW = (NT + 3) / 4;  // output tiles per wavefront of a head
    constexpr int XU = (JB / 2) * (P / 8);                      // units of two tokens x 8 channels, per head
    constexpr int BU = (JB / 2) * (N / 8), BPT = (BU + 511) / 512;  // of B, over the whole workgroup
    // fp8: one 16-byte load carries 16 values, so a unit is one token x 16 channels (state
    // columns): half the loads of the two-token bf16 units for the same elements
    constexpr bool F8 = std::is_same<TX, fp8_t>::value;
    constexpr int BU8 = JB * (N / 16), BPT8 = (BU8 + 511) / 512;
    static_assert(XU == 256, "one X unit per thread of a head");
    typedef Gemm1Chunk<TX, N, 4, 256> G1;
    constexpr int kStateBytes = 2 * (2 * XSZ + BSZ) * 2 + 2 * Q * 4;
    constexpr int kBytes = G1::kLdsBytes > kStateBytes ? G1::kLdsBytes : kStateBytes;
    __shared__ __align__(16) unsigned char smem[kBytes];

    const int tid = threadIdx.x;
    if ((int)blockIdx.y < 4 * G) {
        // GEMM1 workgroups: four wavefronts each (the others have nothing to do)
        if (tid >= 256) return;
        G1::run(Bm, Cm, cb, L, G, sbc, Q, nc, blockIdx.x, blockIdx.y >> 2, blockIdx.z, smem, blockIdx.y & 3);
        return;
    }
    // xs[buf][hw]: the head's weighted X block (fp16); bs[buf]: the shared B block (fp16);
    // ws[hw]: the head's decay weights
    f16 *xsb = reinterpret_cast<f16 *>(smem);
    f16 *bsb = reinterpret_cast<f16 *>(smem + 2 * 2 * XSZ * 2);
    float *wsb = reinterpret_cast<float *>(smem + 2 * (2 * XSZ + BSZ) * 2);
    auto xs = [&](int buf, int hw) { return xsb + (buf * 2 + hw) * XSZ; };
    auto bs = [&](int buf) { return bsb + buf * BSZ; };

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave >> 2, lw = wave & 3, ht = tid & 255;  // head of the pair, its wavefront and thread
    const int li = lane & 15, lg = lane >> 4;
    const int c = blockIdx.x, b = blockIdx.z;
    const int h = 2 * ((int)blockIdx.y - 4 * G) + hw;
    const int g = h / (H / G);
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;
    float *ws = wsb + hw * Q;
    // the head's completion counter of a chunk scan that runs Step-3 itself starts at zero
    if (opt.sync && c == 0 && ht == 0) opt.sync[((size_t)b * H + h) * kSyncStride] = 0u;
    // ... and the prefill's give-up word is clear
    if (opt.ctl && c == 0 && h == 0 && b == 0 && tid == 0) opt.ctl[1] = 0u;

    // ---- prologue: the step sizes first (wavefront 0 of each head), then every block of
    // the chunk: X for this thread's head, B shared by the pair
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + ((size_t)b * L + tc) * sx + (size_t)h * P,
                                                (uint32_t)(((vrows - 1) * sx + P) * sizeof(TX)));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bm + ((size_t)b * L + tc) * sbc + (size_t)g * N,
                                                (uint32_t)(((vrows - 1) * sbc + N) * sizeof(TX)));
    unsigned short dtraw[4];
    const float dbias = opt.dt_bias ? opt.dt_bias[h] : 0.f;  // read before the block loads
    if (lw == 0) {
        const __amdgpu_buffer_rsrc_t rd =
            make_rsrc(dt + ((size_t)b * L + tc) * sdt + h, (uint32_t)(((vrows - 1) * sdt + 1) * 2));
#pragma unroll
        for (int k = 0; k < 4; ++k) dtraw[k] = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)((lane * 4 + k) * sdt * 2), 0, 0);
    }
    Raw8<TX> px[F8 ? 1 : NBLK][2], pb[F8 ? 1 : NBLK][BPT][2];
    uint4 px8[F8 ? NBLK : 1], pb8[F8 ? NBLK : 1][BPT8];
#pragma unroll
    for (int m = 0; m < NBLK; ++m) {
        if constexpr (F8) {
            const int j = JB * m + ht / (P / 16), pg = ht % (P / 16);
            px8[m] = buf_load16<XCP>(rx, (uint32_t)(j * sx + 16 * pg));
#pragma unroll
            for (int k = 0; k < BPT8; ++k) {
                const int u = tid + k * 512;
                if (BU8 % 512 == 0 || u < BU8) {
                    const int jb = JB * m + u / (N / 16), ng = u % (N / 16);
                    pb8[m][k] = buf_load16(rb, (uint32_t)(jb * sbc + 16 * ng));
                }
            }
        } else {
            {
                const int jp = ht / (P / 8), pg = ht % (P / 8), j = JB * m + 2 * jp;
#pragma unroll
                for (int e = 0; e < 2; ++e) px[m][e].template load<XCP>(rx, (uint32_t)((j + e) * sx + 8 * pg));
            }
#pragma unroll
            for (int k = 0; k < BPT; ++k) {
                const int u = tid + k * 512;
                if (BU % 512 == 0 || u < BU) {
                    const int jp = u / (N / 8), ng = u % (N / 8), j = JB * m + 2 * jp;
#pragma unroll
                    for (int e = 0; e < 2; ++e) pb[m][k][e].load(rb, (uint32_t)((j + e) * sbc + 8 * ng));
                }
            }
        }
    }
    // Step-0 (wavefront 0 of each head): inclusive scan of dt_t A_h over the chunk, four
    // tokens per lane serially, then across the lanes; dA_cum and dt_c for the later
    // stages, and the weights w_j
    if (lw == 0) {
        const float Ah = A[h];
        float part[4], dv[4], run = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = lane * 4 + k;
            // (the empty asm keeps this first use of the step size after the block loads)
            unsigned short raw = dtraw[k];
            asm volatile("" : "+v"(raw));
            float d = 0.f;
            if (tc + i < L) d = dt_effective_b(__uint_as_float((uint32_t)raw << 16), dbias, opt.dt_softplus);
            dv[k] = d;
            run += d * Ah;
            part[k] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.f;
        const float aend = __shfl(incl, 63, 64);  // total over the chunk (padding adds 0)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = lane * 4 + k;
            const float ac = excl + part[k];
            acum[bhc * Q + i] = ac;
            dtc[bhc * Q + i] = dv[k];
            ws[i] = exp_fast(aend - ac) * dv[k];
        }
    }
    __syncthreads();

    // block m into LDS buffer buf: the head's X weighted by w_j (fp16), the shared B (fp16)
    auto commit = [&](int m, int buf) {
        if constexpr (F8) {
            const int j = ht / (P / 16), pg = ht % (P / 16);
            const float w = ws[JB * m + j];
            Raw8<fp8_t> lo, hi;
            lo.v = make_uint2(px8[m].x, px8[m].y);
            hi.v = make_uint2(px8[m].z, px8[m].w);
            *reinterpret_cast<uint4 *>(&xs(buf, hw)[j * LDXR + 16 * pg]) = raw8_to_f16x8(lo, w);
            *reinterpret_cast<uint4 *>(&xs(buf, hw)[j * LDXR + 16 * pg + 8]) = raw8_to_f16x8(hi, w);
#pragma unroll
            for (int k = 0; k < BPT8; ++k) {
                const int u = tid + k * 512;
                if (BU8 % 512 == 0 || u < BU8) {
                    const int jb = u / (N / 16), ng = u % (N / 16);
                    *reinterpret_cast<uint4 *>(&bs(buf)[jb * LDBR + 16 * ng]) =
                        f8x8_to_f16x8(make_uint2(pb8[m][k].x, pb8[m][k].y));
                    *reinterpret_cast<uint4 *>(&bs(buf)[jb * LDBR + 16 * ng + 8]) =
                        f8x8_to_f16x8(make_uint2(pb8[m][k].z, pb8[m][k].w));
                }
            }
        } else {
            {
                const int jp = ht / (P / 8), pg = ht % (P / 8), j = 2 * jp;
                const float w0 = ws[JB * m + j], w1 = ws[JB * m + j + 1];
                *reinterpret_cast<uint4 *>(&xs(buf, hw)[j * LDXR + 8 * pg]) = raw8_to_f16x8(px[m][0], w0);
                *reinterpret_cast<uint4 *>(&xs(buf, hw)[(j + 1) * LDXR + 8 * pg]) = raw8_to_f16x8(px[m][1], w1);
            }
#pragma unroll
            for (int k = 0; k < BPT; ++k) {
                const int u = tid + k * 512;
                if (BU % 512 == 0 || u < BU) {
                    const int jp = u / (N / 8), ng = u % (N / 8);
                    *reinterpret_cast<uint4 *>(&bs(buf)[(2 * jp) * LDBR + 8 * ng]) = raw8_to_f16x8(pb[m][k][0]);
                    *reinterpret_cast<uint4 *>(&bs(buf)[(2 * jp + 1) * LDBR + 8 * ng]) = raw8_to_f16x8(pb[m][k][1]);
                }
            }
        }
    };
    f32x4 acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = zero4();
    // The head's wavefront lw takes the state-column tiles lw + 4 j (j < TN / 4) crossed with
    // every channel tile (TN >= 4), or one state-column tile with TPW channel tiles (TN = 2);
    // each distinct operand is read once per 32-token step.  Reduction slots of lane group lg:
    // tokens ks + 4 lg + r and ks + 16 + 4 lg + r.
    auto contract = [&](int buf) {
        constexpr int NB = TN >= 4 ? TN / 4 : 1, NX = TN >= 4 ? TP : TPW;
#pragma unroll
        for (int ks = 0; ks < JB; ks += 32) {
            f16x8 bo[NB], xo[NX];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int nt = TN >= 4 ? lw + 4 * j : lw % TN;
                const int ob = tr16_offset(lane, ks, nt * 16, LDBR);
                const f16x4 b0 = lds_read_tr16(&bs(buf)[ob]);
                const f16x4 b1 = lds_read_tr16(&bs(buf)[ob + 16 * LDBR]);
                bo[j] = f16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            }
#pragma unroll
            for (int q = 0; q < NX; ++q) {
                const int pt = TN >= 4 ? q : lw / TN + (4 / TN) * q;
                const int ox = tr16_offset(lane, ks, pt * 16, LDXR);
                const f16x4 a0 = lds_read_tr16(&xs(buf, hw)[ox]);
                const f16x4 a1 = lds_read_tr16(&xs(buf, hw)[ox + 16 * LDXR]);
                xo[q] = f16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int j = TN >= 4 ? tt % NB : 0, q = TN >= 4 ? tt / NB : tt;
                acc[tt] = mfma16x16x32_f16(bo[j], xo[q], acc[tt]);
            }
        }
    };
    commit(0, 0);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NBLK; ++m) {
        contract(m & 1);
        if (m + 1 < NBLK) {
            commit(m + 1, (m + 1) & 1);
            __syncthreads();
        }
    }

    // ---- S_c [P][N] (fp16): lane holds columns n = 16 nt + 4 lg + r of row p = 16 pt + li.
    // The tiles go through LDS (the blocks' buffers are free once every wavefront is past the
    // last contraction), so that the state -- one contiguous P x N block per head -- leaves as
    // whole rows, 16 bytes per lane and 1 KB per store instruction, instead of 32-byte pieces
    // of 16 rows.
    constexpr int LDS_ = N + 8;  // padded row of the staged state (fp16)
    static_assert(2 * P * LDS_ * 2 <= kBytes, "staged chunk states fit the block buffers");
    f16 *sst = reinterpret_cast<f16 *>(smem) + hw * P * LDS_;
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        int pt, nt;
        if constexpr (TN >= 4) {
            constexpr int NB = TN / 4;
            pt = tt / NB;
            nt = lw + 4 * (tt % NB);
        } else {
            pt = lw / TN + (4 / TN) * tt;
            nt = lw % TN;
        }
        uint2 v;
        v.x = pack_f16x2(acc[tt][0], acc[tt][1]);
        v.y = pack_f16x2(acc[tt][2], acc[tt][3]);
        *reinterpret_cast<uint2 *>(&sst[(pt * 16 + li) * LDS_ + nt * 16 + 4 * lg]) = v;
    }
    __syncthreads();
    constexpr int RU = N / 8;  // 16-byte pieces of a state row
    static_assert((P * RU) % 256 == 0, "whole pieces per thread of a head");
#pragma unroll
    for (int k = 0; k < P * RU / 256; ++k) {
        const int u = ht + 256 * k, row = u / RU, piece = u % RU;
        *reinterpret_cast<uint4 *>(states + bhc * P * N + (size_t)row * N + 8 * piece) =
            *reinterpret_cast<const uint4 *>(&sst[row * LDS_ + 8 * piece]);
    }
}

bool chunk_state_pair_fits(const Dims &d)
{
    return d.half() && d.Q == 256 && d.P == 64 && d.N <= 128 && d.G > 0 && (d.H / d.G) % 2 == 0;
}

hipError_t launch_chunk_state_pair(const void *x, const void *Bm, const void *dt, const float *A, float *acum,
                                   float *dtc, void *states, const void *Cm, void *cb, const SsdOpts &o,
                                   const Dims &d, hipStream_t s)
{
    if (!chunk_state_pair_fits(d)) return hipErrorInvalidValue;
    const dim3 grid(d.nc, d.H / 2 + 4 * d.G, d.B);
    const bf16_t *dd = static_cast<const bf16_t *>(dt);
    f16 *st = static_cast<f16 *>(states);
#define SSD_CSP_LAUNCH2(NN, CP)                                                                                     \
    do {                                                                                                            \
        if (d.in == kInFp8)                                                                                         \
            launch_kernel("chunk_state_pair_kernel", chunk_state_pair_kernel<fp8_t, NN, CP>, grid, 512, s,        \
                          static_cast<const fp8_t *>(x), static_cast<const fp8_t *>(Bm), dd, A, acum, dtc, st,    \
                          static_cast<const fp8_t *>(Cm), cb, o, d.L, d.H, d.G, d.sx, d.sbc, d.sdt, d.nc);        \
        else                                                                                                        \
            launch_kernel("chunk_state_pair_kernel", chunk_state_pair_kernel<bf16_t, NN, CP>, grid, 512, s,       \
                          static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(Bm), dd, A, acum, dtc, st,  \
                          static_cast<const bf16_t *>(Cm), cb, o, d.L, d.H, d.G, d.sx, d.sbc, d.sdt, d.nc);       \
    } while (0)
#define SSD_CSP_LAUNCH(NN)                   \
    do {                                     \
        if (o.stream_x)                      \
            SSD_CSP_LAUNCH2(NN, kStream);    \
        else                                 \
            SSD_CSP_LAUNCH2(NN, 0);          \
    } while (0)
    switch (d.N) {
    case 32: SSD_CSP_LAUNCH(32); break;
    case 64: SSD_CSP_LAUNCH(64); break;
    case 128: SSD_CSP_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_CSP_LAUNCH
#undef SSD_CSP_LAUNCH2
    return hipGetLastError();
}

}  // namespace ssd
