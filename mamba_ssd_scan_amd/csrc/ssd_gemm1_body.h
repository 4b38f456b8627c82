// ssd_gemm1_body.h -- one (batch, group, chunk) of Step-1 GEMM1, C.B^T, for a workgroup of
// NWAVES wavefronts; used by the stand-alone GEMM1 kernel and, as extra workgroups, by
// the prefill's chunk-state launch.  Output layout: see ssd_chunk_gemm1.hip.
#pragma once

#include <type_traits>

#include "ssd_common.h"

namespace ssd {

// ROWS: chunk rows the LDS holds (>= Q).  NWAVES: 16 (one row tile each, SIMD-balanced
// order), 8 or 4.  With 4 wavefronts a wavefront takes up to four row tiles in turn:
// {w, 7-w, 8+w, 15-w} for 16 tiles (18 32-column steps each), {w, 7-w} for 8.
template <typename TIn, int N, int NWAVES, int ROWS> struct Gemm1Chunk {
    typedef Traits<TIn> Tr;
    typedef typename Tr::raw_t raw_t;
    static constexpr bool F32 = Tr::kF32;
    // e4m3 inputs: B rows are widened to fp16 when staged and C rows when loaded (exact), and
    // the products run on fp16 matrix cores; bf16 inputs run on bf16 ones
    static constexpr bool F8 = std::is_same<TIn, fp8_t>::value;
    typedef typename std::conditional<F8, f16x8, bf16x8>::type mop_t;
    static constexpr int LDB = N + (F32 ? 4 : 8);  // row pitch: 16 rows read together hit distinct banks
    static constexpr int KS = F32 ? N / 4 : N / 32;
    static constexpr int NT = 64 * NWAVES;
    // B rows are held in LDS 128 at a time: a 32-column step reads rows 32s .. 32s+31, so
    // every step lies in one pass and each output slice is still formed once.
    static constexpr int PASS_ROWS = ROWS < 128 ? ROWS : 128;
    static constexpr int kLdsBytes = PASS_ROWS * LDB * (int)sizeof(raw_t);
    static constexpr int TPW = NWAVES == 4 ? 4 : 1;  // row tiles per wavefront

    // row tile of slot k of wavefront w (-1: none), for nt 16-row tiles
    static __device__ __forceinline__ int tile_of(int w, int k, int nt)
    {
        if constexpr (NWAVES == 4) {
            if (nt == 16) return k == 0 ? w : k == 1 ? 7 - w : k == 2 ? 8 + w : 15 - w;
            if (nt == 8) return k == 0 ? w : k == 1 ? 7 - w : -1;
            return (k == 0 && w < nt) ? w : -1;
        } else {
            if (nt == NWAVES && NWAVES >= 8) {
                const int s = w & 3, q = w >> 2;
                return 8 * (q >> 1) + ((q & 1) ? 7 - s : s);
            }
            return w < nt ? w : -1;
        }
    }

    // part < 0: this workgroup forms every row tile of the chunk.  part = 0..3 (four
    // wavefronts only): one of four workgroups sharing the chunk; wavefront w forms row
    // tile tile_of(part, w) alone, so the four workgroups take the balanced tile sets
    // {p, 7-p, 8+p, 15-p} and no wavefront walks more than one tile.
    static __device__ __forceinline__ void run(const TIn *__restrict__ Bm, const TIn *__restrict__ Cm,
                                               void *__restrict__ cb, int L, int G, int sbc, int Q, int nc, int c,
                                               int g, int b, unsigned char *smem, int part = -1)
    {
        raw_t *bs = reinterpret_cast<raw_t *>(smem);
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int li = lane & 15, lg = lane >> 4;
        const long tc = (long)c * Q;
        const int nt = Q >> 4;

        const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
        // the group's N values of the chunk's first token; tokens sbc elements apart
        const size_t row0 = ((size_t)b * L + tc) * sbc + (size_t)g * N;
        const uint32_t bytes = (uint32_t)(((vrows - 1) * sbc + N) * sizeof(TIn));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bm + row0, bytes);
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + row0, bytes);

        // C rows of a row tile (the GEMM1^T B operand), held in registers
        mop_t cbf[F32 ? 1 : KS];
        float cf[F32 ? KS : 1];
        auto load_c = [&](int t) {
            const uint32_t row = (uint32_t)((16 * t + li) * sbc);
            if constexpr (F32) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    cf[ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(4u * (row + ks * 4 + lg)), 0, 0));
            } else if constexpr (F8) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) cbf[ks] = __builtin_bit_cast(f16x8, f8x8_to_f16x8(buf_load8(rc, row + ks * 32 + 8 * lg)));
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) cbf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
            }
        };
        auto tile = [&](int k) { return part < 0 ? tile_of(wave, k, nt) : (k == 0 ? tile_of(part, wave, nt) : -1); };
        const int t0 = tile(0);
        if (t0 >= 0) load_c(t0);

        const int spc = (nt & 1) ? ((nt >> 1) + 1) * ((nt >> 1) + 1) : (nt >> 1) * ((nt >> 1) + 1);
        const size_t chunk0 = (((size_t)b * G + g) * nc + c) * (size_t)spc;  // the chunk's first slice
        const int npass = (16 * nt + PASS_ROWS - 1) / PASS_ROWS;  // 1 or 2
        // B rows of both passes are requested at once (rows past the chunk or the sequence
        // read as zeros; a fixed trip count keeps every load in flight): the second pass's
        // rows wait in registers while the first pass computes.
        constexpr int BU = PASS_ROWS * (N / 8), BPT = (BU + NT - 1) / NT;
        constexpr int NPASS_MAX = ROWS > 128 ? 2 : 1;
        Raw8<TIn> bv[NPASS_MAX][BPT];
#pragma unroll
        for (int q = 0; q < NPASS_MAX; ++q)
#pragma unroll
            for (int k = 0; k < BPT; ++k) {
                const int u = tid + k * NT;
                if (u < BU) {
                    if (q < npass)
                        bv[q][k].load(rb, (uint32_t)((q * PASS_ROWS + u / (N / 8)) * sbc + 8 * (u % (N / 8))));
                    else
                        bv[q][k].zero();
                }
            }
#pragma unroll
        for (int pass = 0; pass < NPASS_MAX; ++pass) {
        if (pass >= npass) break;
        const int r0 = pass * PASS_ROWS;  // first B row held in LDS during this pass
        if (pass > 0) __syncthreads();    // the previous pass's readers are done with the rows
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * NT;
            if (u < BU) bv[pass][k].store(&bs[(u / (N / 8)) * LDB + 8 * (u % (N / 8))]);
        }
        __syncthreads();

#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = tile(k);
            if (t < 0) continue;
            if (k > 0 || pass > 0) load_c(t);
            const int ibase = 16 * t;
            const int Tt = (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);
            const int ns = (ibase + 15) / 32 + 1;
            // this pass's steps of the tile: columns 32 s in [r0, r0 + PASS_ROWS)
            const int s_lo = r0 / 32, s_hi = min(ns, (r0 + PASS_ROWS) / 32);
            for (int s = s_lo; s < s_hi; ++s) {
                const int jb = 32 * s - r0;  // LDS row of the step's first column
                const bool has1 = 32 * s + 16 <= ibase + 15;  // second 16-column half not entirely above the diagonal
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
                    auto mma = [](mop_t a, mop_t b, f32x4 c) {
                        if constexpr (F8)
                            return mfma16x16x32_f16(a, b, c);
                        else
                            return mfma16x16x32_bf16(a, b, c);
                    };
                    if (has1) {
                        mop_t a0[KS], a1[KS];
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            a0[ks] = *reinterpret_cast<const mop_t *>(b0 + ks * 32);
                            a1[ks] = *reinterpret_cast<const mop_t *>(b0 + 16 * LDB + ks * 32);
                        }
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            d0 = mma(a0[ks], cbf[ks], d0);
                            d1 = mma(a1[ks], cbf[ks], d1);
                        }
                    } else {
                        mop_t a0[KS];
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) a0[ks] = *reinterpret_cast<const mop_t *>(b0 + ks * 32);
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) d0 = mma(a0[ks], cbf[ks], d0);
                    }
                }
                const size_t slice = chunk0 + Tt + s;
                if constexpr (F32) {
                    float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(cb) + (slice * 64 + lane) * 8);
                    o[0] = make_float4(d0[0], d0[1], d0[2], d0[3]);
                    o[1] = make_float4(d1[0], d1[1], d1[2], d1[3]);
                } else {
                    uint4 w;
                    w.x = pack_f16x2(d0[0], d0[1]);
                    w.y = pack_f16x2(d0[2], d0[3]);
                    w.z = pack_f16x2(d1[0], d1[1]);
                    w.w = pack_f16x2(d1[2], d1[3]);
                    *reinterpret_cast<uint4 *>(static_cast<f16 *>(cb) + (slice * 64 + lane) * 8) = w;
                }
            }
        }
        }  // pass
    }
};

}  // namespace ssd
