// ssd_chunk_state.hip -- Step-2: the state each chunk leaves from a zero start.
//
//   S_c[p, n] = sum_j w_j x_j[p] B_j[n],   w_j = exp(dA_cum[Q-1] - dA_cum[j]) dt_j
//
// i.e. S_c = (X_c * w)^T B_c, a [P, Q] x [Q, N] contraction over the chunk's
// time axis.  The chunked method needs it to hand state from chunk to chunk
// ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec.
// III-A: the recurrent state links the chunks; Step-3 consumes these states).
//
// One 256-thread workgroup (4 wavefronts) per (b, h, c); each wavefront owns
// every fourth 16x16 output tile.  The chunk is streamed through LDS in
// blocks of JB tokens.  With bf16 inputs both tiles are kept row-major
// ([token][channel], fp16) exactly as they arrive from memory -- every thread
// converts and stores 16 contiguous bytes -- and the matrix-core operands,
// whose reduction index is the token, are read with the transposing LDS
// read.  The decay weight is folded into X on the way in; the weighted X is a
// computed operand, so both operands go to the matrix cores as fp16 (B
// converts exactly), accumulating in fp32.  (fp32 inputs keep transposed fp32
// tiles for the 16x16x4 fp32 path.)  Two blocks of global loads are kept in
// flight in registers ahead of the block being contracted; LDS is
// double-buffered with one barrier per block.
//
// With bf16 inputs S_c is stored in fp16 (fp32 accumulation, one rounding at
// the end): the chunk states and the entering states made from them travel
// between the kernels at half the bytes, and the chunk-scan kernel feeds the
// entering state to the matrix cores in fp16 anyway.
#include "ssd_common.h"
#include "ssd_gemm1_body.h"
#include "ssd_launch.h"

namespace ssd {

// Step-0 fused in (FUSE_CUMSUM): one wavefront scans this chunk's dt*A (as the
// stand-alone cumulative-decay kernel does) and writes dA_cum / dt_c for the
// later stages, instead of reading them; the other wavefronts start loading.
// Step-1 GEMM1 fused in (GR > 0, chunks of up to GR tokens): the first 4G rows of
// the grid (blockIdx.y < 4G) are GEMM1 workgroups, four per (b, group, chunk), each
// forming a balanced quarter of the chunk's row tiles of C.B^T into `cb`, while the
// chunk-state workgroups (blockIdx.y = 4G + h) run; they come first in the grid so
// that they are dispatched first.
// JBT: tokens per staged block.  32 keeps LDS small enough for four workgroups per
// CU (grids with many workgroups); 64 halves the barriers when the whole grid is
// resident at once anyway (two workgroups per CU).
template <typename TIn, int P, int N, bool FUSE_CUMSUM, int GR, int JBT>
__global__ __launch_bounds__(256) void chunk_state_kernel(const TIn *__restrict__ x,
                                                          const TIn *__restrict__ Bm,
                                                          const typename Traits<TIn>::dt_t *__restrict__ dt,
                                                          const float *__restrict__ A,
                                                          float *__restrict__ acum,
                                                          float *__restrict__ dtc,
                                                          void *__restrict__ states,
                                                          const TIn *__restrict__ Cm, void *__restrict__ cb,
                                                          SsdOpts opt, int L, int H, int G, int sx, int sbc, int sdt, int Q, int nc)
{
    typedef Traits<TIn> Tr;
    typedef typename Tr::op_t op_t;
    constexpr bool F32 = Tr::kF32;
    constexpr int JB = Traits<TIn>::kF32 ? 32 : JBT;   // tokens per staged block
    // one-round grids (64-token blocks): every block of the chunk prefetched at once
    constexpr bool ALLPF = !Traits<TIn>::kF32 && JBT == 64;
    constexpr int NBMAX = 256 / JB;                    // blocks of the longest chunk
    // bf16 inputs: row-major fp16 tiles; a pitch of (width + 16) halves puts the 16
    // rows one transposing read touches on distinct bank groups.
    constexpr int LDXR = P + 16, LDBR = N + 16;
    constexpr int LDT = JB + 4;                         // fp32 inputs: transposed tiles
    constexpr int XSZ = F32 ? P * LDT : JB * LDXR;
    constexpr int BSZ = F32 ? N * LDT : JB * LDBR;
    constexpr int TP = P / 16, TN = N / 16, NT = TP * TN;
    constexpr int TPW = (NT + 3) / 4;                   // output tiles per wavefront
    constexpr int XU = (JB / 2) * (P / 8), XPT = (XU + 255) / 256;  // two tokens x 8 channels
    constexpr int BU = (JB / 2) * (N / 8), BPT = (BU + 255) / 256;
    typedef Gemm1Chunk<TIn, N, 4, (GR > 0 ? GR : 64)> G1;
    constexpr int kStateBytes = 2 * (XSZ + BSZ) * (int)sizeof(op_t) + 256 * 4;
    constexpr int kBytes = (GR > 0 && G1::kLdsBytes > kStateBytes) ? G1::kLdsBytes : kStateBytes;
    __shared__ __align__(16) unsigned char smem[kBytes];
    if constexpr (GR > 0) {
        if ((int)blockIdx.y < 4 * G) {
            G1::run(Bm, Cm, cb, L, G, sbc, Q, nc, blockIdx.x, blockIdx.y >> 2, blockIdx.z, smem, blockIdx.y & 3);
            return;
        }
    }
    op_t(*xs)[XSZ] = reinterpret_cast<op_t(*)[XSZ]>(smem);
    op_t(*bs)[BSZ] = reinterpret_cast<op_t(*)[BSZ]>(smem + 2 * XSZ * sizeof(op_t));
    float *ws = reinterpret_cast<float *>(smem + 2 * (XSZ + BSZ) * sizeof(op_t));  // decay weights w_j of the chunk

    const int c = blockIdx.x, h = blockIdx.y - (GR > 0 ? 4 * G : 0), b = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
    const int li = lane & 15, lg = lane >> 4;
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;
    const int nblk = (Q + JB - 1) / JB;
    // the head's completion counter of a chunk scan that runs Step-3 itself starts at zero
    if (FUSE_CUMSUM && opt.sync && c == 0 && tid == 0) opt.sync[((size_t)b * H + h) * kSyncStride] = 0u;
    // ... and the prefill's give-up word is clear
    if (FUSE_CUMSUM && opt.ctl && c == 0 && h == 0 && b == 0 && tid == 0) opt.ctl[1] = 0u;

    struct Stage {
        Raw8<TIn> x[XPT][2], b[BPT][2];
    };
    // Buffer resources over this chunk's valid rows of X and B: loads of rows past
    // the chunk or the sequence return zeros.
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(x + ((size_t)b * L + tc) * sx + (size_t)h * P, (uint32_t)(((vrows - 1) * sx + P) * sizeof(TIn)));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(Bm + ((size_t)b * L + tc) * sbc + (size_t)g * N, (uint32_t)(((vrows - 1) * sbc + N) * sizeof(TIn)));

    // (live == false: a block past the chunk; its loads read an empty range)
    auto prefetch = [&](Stage &st, int jbk, bool live = true) {
        const int j0 = live ? jbk * JB : 0;
        const __amdgpu_buffer_rsrc_t bx = live ? rx : make_rsrc(x, 0u);
        const __amdgpu_buffer_rsrc_t bb = live ? rb : make_rsrc(Bm, 0u);
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * 256;
            if (XU % 256 == 0 || u < XU) {  // (true at compile time when every thread has a unit)
                const int jp = u / (P / 8), pg = u % (P / 8), j = j0 + 2 * jp;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    // (a uniform branch: X streamed past the Infinity Cache, see SsdOpts::stream_x)
                    if (opt.stream_x)
                        st.x[k][e].template load<kStream>(bx, (uint32_t)((j + e) * sx + 8 * pg));
                    else
                        st.x[k][e].load(bx, (uint32_t)((j + e) * sx + 8 * pg));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * 256;
            if (BU % 256 == 0 || u < BU) {
                const int jp = u / (N / 8), ng = u % (N / 8), j = j0 + 2 * jp;
#pragma unroll
                for (int e = 0; e < 2; ++e) st.b[k][e].load(bb, (uint32_t)((j + e) * sbc + 8 * ng));
            }
        }
    };
    auto commit = [&](const Stage &st, int buf, int jbk) {
        const int j0 = jbk * JB;
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * 256;
            if (XU % 256 == 0 || u < XU) {  // (true at compile time when every thread has a unit)
                const int jp = u / (P / 8), pg = u % (P / 8), j = j0 + 2 * jp;
                const float w0 = j < Q ? ws[j] : 0.f, w1 = j + 1 < Q ? ws[j + 1] : 0.f;
                if constexpr (F32) {
                    float v0[8], v1[8];
                    st.x[k][0].to_f32(v0);
                    st.x[k][1].to_f32(v1);
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) store_pair(&xs[buf][(8 * pg + kk) * LDT + 2 * jp], v0[kk] * w0, v1[kk] * w1);
                } else {
                    *reinterpret_cast<uint4 *>(&xs[buf][(2 * jp) * LDXR + 8 * pg]) = raw8_to_f16x8(st.x[k][0], w0);
                    *reinterpret_cast<uint4 *>(&xs[buf][(2 * jp + 1) * LDXR + 8 * pg]) = raw8_to_f16x8(st.x[k][1], w1);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * 256;
            if (BU % 256 == 0 || u < BU) {
                const int jp = u / (N / 8), ng = u % (N / 8);
                if constexpr (F32) {
                    float v0[8], v1[8];
                    st.b[k][0].to_f32(v0);
                    st.b[k][1].to_f32(v1);
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) store_pair(&bs[buf][(8 * ng + kk) * LDT + 2 * jp], v0[kk], v1[kk]);
                } else {
                    *reinterpret_cast<uint4 *>(&bs[buf][(2 * jp) * LDBR + 8 * ng]) = raw8_to_f16x8(st.b[k][0]);
                    *reinterpret_cast<uint4 *>(&bs[buf][(2 * jp + 1) * LDBR + 8 * ng]) = raw8_to_f16x8(st.b[k][1]);
                }
            }
        }
    };

    f32x4 acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = zero4();

    auto contract = [&](int buf, int jbk) {
        for (int ks = 0; ks < JB && jbk * JB + ks < Q; ks += 32) {
            if constexpr (!F32) {
                // The wavefront's tiles t = wave + 4 tt share operands: with TN >= 4 they are
                // the state-column tiles wave + 4 j (j < TN / 4) crossed with every channel
                // tile; with TN = 2, one state-column tile crossed with TPW channel tiles.
                // Each distinct operand is read from LDS once per 32-token step.
                // Reduction slots of lane group lg: tokens ks + 4 lg + r and ks + 16 + 4 lg + r.
                constexpr int NB = TN >= 4 ? TN / 4 : 1, NX = TN >= 4 ? TP : TPW;
                f16x8 bo[NB], xo[NX];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int nt = TN >= 4 ? wave + 4 * j : wave % TN;
                    const int ob = tr16_offset(lane, ks, nt * 16, LDBR);
                    const f16x4 b0 = lds_read_tr16(&bs[buf][ob]);
                    const f16x4 b1 = lds_read_tr16(&bs[buf][ob + 16 * LDBR]);
                    bo[j] = f16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                }
#pragma unroll
                for (int q = 0; q < NX; ++q) {
                    const int pt = TN >= 4 ? q : wave / TN + (4 / TN) * q;
                    const int ox = tr16_offset(lane, ks, pt * 16, LDXR);
                    const f16x4 a0 = lds_read_tr16(&xs[buf][ox]);
                    const f16x4 a1 = lds_read_tr16(&xs[buf][ox + 16 * LDXR]);
                    xo[q] = f16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                }
                // S^T tiles: the B rows are the A operand, so a lane's accumulator holds
                // four consecutive state columns n of one row p (contiguous stores)
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    const int j = TN >= 4 ? tt % NB : 0, q = TN >= 4 ? tt / NB : tt;
                    acc[tt] = mfma16x16x32_f16(bo[j], xo[q], acc[tt]);
                }
                continue;
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int t = wave + 4 * tt;
                if (t < NT) {
                    const int pt = t / TN, nt = t % TN;
                    // S^T tiles: the B rows are the A operand, so a lane's accumulator holds
                    // four consecutive state columns n of one row p (contiguous stores)
                    if constexpr (F32) {
                        const op_t *xa = &xs[buf][(pt * 16 + li) * LDT + ks];
                        const op_t *ba = &bs[buf][(nt * 16 + li) * LDT + ks];
#pragma unroll
                        for (int s = 0; s < 8; ++s) acc[tt] = mfma16x16x4_f32(ba[4 * s + lg], xa[4 * s + lg], acc[tt]);
                    } else {
                        // reduction slots of lane group lg: tokens ks + 4 lg + r and ks + 16 + 4 lg + r
                        const int ox = tr16_offset(lane, ks, pt * 16, LDXR);
                        const int ob = tr16_offset(lane, ks, nt * 16, LDBR);
                        const f16x4 a0 = lds_read_tr16(&xs[buf][ox]);
                        const f16x4 a1 = lds_read_tr16(&xs[buf][ox + 16 * LDXR]);
                        const f16x4 b0 = lds_read_tr16(&bs[buf][ob]);
                        const f16x4 b1 = lds_read_tr16(&bs[buf][ob + 16 * LDBR]);
                        const f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                        const f16x8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                        acc[tt] = mfma16x16x32_f16(bb, a, acc[tt]);
                    }
                }
            }
        }
    };

    // ---- prologue.  The step sizes (or the tables) are requested first, so that waiting
    // for them never waits for the block loads issued after them.
    const int per = Q > 64 ? Q / 64 : 1;
    unsigned short dtraw[4];  // FUSE_CUMSUM, wavefront 0: raw bf16 step sizes, Q/64 per lane
    float dtf[4];             // (fp32 inputs)
    float tac = 0.f, tdt = 0.f, tend = 0.f;  // !FUSE_CUMSUM: this thread's table entries
    const float dbias = (FUSE_CUMSUM && opt.dt_bias) ? opt.dt_bias[h] : 0.f;  // read before the block loads
    if constexpr (FUSE_CUMSUM) {
        if (wave == 0) {
            const long vq = (L - tc) < Q ? (L - tc) : Q;
            const __amdgpu_buffer_rsrc_t rd =
                make_rsrc(dt + ((size_t)b * L + tc) * sdt + h, (uint32_t)(((vq - 1) * sdt + 1) * sizeof(typename Tr::dt_t)));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // (for k >= per this reads a neighbour's token, or zero past the range: unused,
                // but a select here would become a branch, and a branch hides the load count)
                const uint32_t off = (uint32_t)((lane * per + k) * sdt * sizeof(typename Tr::dt_t));
                if constexpr (F32)
                    dtf[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (int)off, 0, 0));
                else
                    dtraw[k] = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)off, 0, 0);
            }
        }
    } else {
        tend = acum[bhc * Q + Q - 1];
        if (tid < Q) {
            tac = acum[bhc * Q + tid];
            tdt = dtc[bhc * Q + tid];
        }
    }
    // An empty asm statement that reads and rewrites a value: it keeps in program order
    // (after the block loads) the first instruction that consumes a loaded value, so the
    // wait for that load is placed here and not right after the load itself.
    auto pin = [](uint32_t v) {
        asm volatile("" : "+v"(v));
        return v;
    };
    auto pin16 = [](unsigned short v) {  // (before the widening, which is itself an instruction)
        asm volatile("" : "+v"(v));
        return v;
    };
    // Step-0 (fused) or the decay weights from the tables, into ws
    auto form_weights = [&]() {
        if constexpr (FUSE_CUMSUM) {
            if (wave == 0) {
                // inclusive scan of a_t = dt_t * A_h over the chunk: Q/64 tokens per lane
                // serially, then a wavefront scan of the lane totals
                const float Ah = A[h];
                float part[4], dts[4], run = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = lane * per + k;
                    float d = 0.f;
                    const float raw = F32 ? __uint_as_float(pin(__float_as_uint(dtf[k])))
                                          : __uint_as_float((uint32_t)pin16(dtraw[k]) << 16);
                    if (k < per && i < Q && tc + i < L) d = dt_effective_b(raw, dbias, opt.dt_softplus);
                    dts[k] = d;
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
                    const int i = lane * per + k;
                    if (k < per && i < Q) {
                        const float ac = excl + part[k];
                        acum[bhc * Q + i] = ac;
                        dtc[bhc * Q + i] = dts[k];
                        ws[i] = exp_fast(aend - ac) * dts[k];
                    }
                }
            }
        } else {
            if (tid < Q)
                ws[tid] = exp_fast(__uint_as_float(pin(__float_as_uint(tend))) - __uint_as_float(pin(__float_as_uint(tac)))) *
                          __uint_as_float(pin(__float_as_uint(tdt)));
        }
    };

    if constexpr (ALLPF) {
        // The whole chunk is requested at once (all blocks in registers), then contracted
        // block by block with no further waits for memory: for grids that fit the GPU in
        // one round, where each workgroup does exactly one chunk.
        Stage sa[NBMAX];
#pragma unroll
        for (int k = 0; k < NBMAX; ++k) prefetch(sa[k], k, k < nblk);
        form_weights();
        __syncthreads();
        commit(sa[0], 0, 0);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NBMAX; ++k) {
            if (k < nblk) {
                contract(k & 1, k);
                if (k + 1 < NBMAX && k + 1 < nblk) {
                    commit(sa[k + 1], (k + 1) & 1, k + 1);
                    __syncthreads();
                }
            }
        }
    } else {
        // blocks 0 and 1 in flight while the decay weights are formed
        Stage s0, s1;
        prefetch(s0, 0);
        if (nblk > 1) prefetch(s1, 1);
        form_weights();
        __syncthreads();
        commit(s0, 0, 0);
        __syncthreads();

        // main loop, unrolled by two so that each register stage has a fixed name:
        // block k is in LDS buffer k&1; the stage that held block k is refilled with block k+2.
        for (int jbk = 0; jbk < nblk; jbk += 2) {
            if (jbk + 2 < nblk) prefetch(s0, jbk + 2);
            contract(0, jbk);
            if (jbk + 1 < nblk) {
                commit(s1, 1, jbk + 1);
                __syncthreads();
                if (jbk + 3 < nblk) prefetch(s1, jbk + 3);
                contract(1, jbk + 1);
                if (jbk + 2 < nblk) {
                    commit(s0, 0, jbk + 2);
                    __syncthreads();
                }
            }
        }
    }

    // ---- write S_c [P][N] (fp32, or fp16 for bf16 inputs): lane holds columns
    // n = 16 nt + 4 lg + r of row p = 16 pt + li.  fp16 states go through LDS (the block
    // buffers, free after the last contraction) when they fit there, so that the state -- one
    // contiguous P x N block -- is stored as whole rows, 16 bytes per lane, instead of 32-byte
    // pieces of 16 rows.
    constexpr int LDS_ = N + 8;
    constexpr bool STAGE = !F32 && P * LDS_ * 2 <= 2 * (XSZ + BSZ) * (int)sizeof(op_t);
    f16 *sst = reinterpret_cast<f16 *>(smem);
    if constexpr (STAGE) __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int t = wave + 4 * tt;
        if (t < NT) {
            const int pt = t / TN, nt = t % TN;
            const size_t e = bhc * P * N + (size_t)(pt * 16 + li) * N + nt * 16 + 4 * lg;
            if constexpr (F32) {
                *reinterpret_cast<float4 *>(static_cast<float *>(states) + e) =
                    make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
            } else {
                uint2 v;
                v.x = pack_f16x2(acc[tt][0], acc[tt][1]);
                v.y = pack_f16x2(acc[tt][2], acc[tt][3]);
                if constexpr (STAGE)
                    *reinterpret_cast<uint2 *>(&sst[(pt * 16 + li) * LDS_ + nt * 16 + 4 * lg]) = v;
                else
                    *reinterpret_cast<uint2 *>(static_cast<f16 *>(states) + e) = v;
            }
        }
    }
    if constexpr (STAGE) {
        __syncthreads();
        constexpr int RU = N / 8, NU = P * RU;  // 16-byte pieces of a state row, of the state
#pragma unroll
        for (int k = 0; k < (NU + 255) / 256; ++k) {
            const int u = tid + 256 * k, row = u / RU, piece = u % RU;
            if (NU % 256 == 0 || u < NU)
                *reinterpret_cast<uint4 *>(static_cast<f16 *>(states) + bhc * P * N + (size_t)row * N + 8 * piece) =
                    *reinterpret_cast<const uint4 *>(&sst[row * LDS_ + 8 * piece]);
        }
    }
}

template <typename TIn, int P, bool FUSE, int GR>
static hipError_t launch_cs_n(const void *x, const void *Bm, const void *dt, const float *A, float *acum,
                              float *dtc, void *states, const void *Cm, void *cb, const SsdOpts &o, const Dims &d,
                              bool big, hipStream_t s)
{
    const dim3 grid(d.nc, d.H + (GR > 0 ? 4 * d.G : 0), d.B);
    const TIn *xx = static_cast<const TIn *>(x), *bb = static_cast<const TIn *>(Bm), *cc = static_cast<const TIn *>(Cm);
    const typename Traits<TIn>::dt_t *dd = static_cast<const typename Traits<TIn>::dt_t *>(dt);
#define SSD_CS_LAUNCH(NN, JJ)                                                                                      \
    launch_kernel("chunk_state_kernel", chunk_state_kernel<TIn, P, NN, FUSE, GR, JJ>, grid, 256, s, xx, bb, \
                  dd, A, acum, dtc, states, cc, cb, o, d.L, d.H, d.G, d.sx, d.sbc, d.sdt, d.Q, d.nc)
#define SSD_CS_BY_JB(NN)          \
    if (big || sizeof(TIn) == 4)  \
        SSD_CS_LAUNCH(NN, 32);    \
    else                          \
        SSD_CS_LAUNCH(NN, 64)
    switch (d.N) {
    case 32: SSD_CS_BY_JB(32); break;
    case 64: SSD_CS_BY_JB(64); break;
    case 128: SSD_CS_BY_JB(128); break;
    case 256: SSD_CS_BY_JB(256); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_CS_BY_JB
#undef SSD_CS_LAUNCH
    return hipGetLastError();
}

template <typename TIn, bool FUSE, int GR>
static hipError_t launch_cs_t(const void *x, const void *Bm, const void *dt, const float *A, float *acum,
                              float *dtc, void *states, const void *Cm, void *cb, const SsdOpts &o, const Dims &d,
                              hipStream_t s)
{
    // the kernels size their buffer ranges by the element type: never run one on the other's inputs
    if (d.in != InOf<TIn>::v) return hipErrorInvalidValue;
    // More workgroups than two per compute unit: the smaller staged blocks (more resident
    // workgroups) pay off; otherwise the larger ones (fewer barriers).
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long nwg = (long)d.nc * (d.H + (GR > 0 ? 4 * d.G : 0)) * d.B;
    const bool big = nwg > 2L * (ncu > 0 ? ncu : 1);
    switch (d.P) {
    case 32: return launch_cs_n<TIn, 32, FUSE, GR>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, big, s);
    case 64: return launch_cs_n<TIn, 64, FUSE, GR>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, big, s);
    case 128: return launch_cs_n<TIn, 128, FUSE, GR>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, big, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_state(const void *x, const void *Bm, const float *acum, const float *dtc,
                              void *states, const Dims &d, hipStream_t s)
{
    float *ac = const_cast<float *>(acum), *dc = const_cast<float *>(dtc);  // read-only in this mode
    const SsdOpts o = {nullptr, 0, nullptr, 0};
    if (d.in == kInFp8)
        return launch_cs_t<fp8_t, false, 0>(x, Bm, nullptr, nullptr, ac, dc, states, nullptr, nullptr, o, d, s);
    return d.in == kInBf16 ? launch_cs_t<bf16_t, false, 0>(x, Bm, nullptr, nullptr, ac, dc, states, nullptr, nullptr, o, d, s)
                           : launch_cs_t<float, false, 0>(x, Bm, nullptr, nullptr, ac, dc, states, nullptr, nullptr, o, d, s);
}

template <typename TIn>
static hipError_t launch_fused_t(const void *x, const void *Bm, const void *dt, const float *A, float *acum,
                                 float *dtc, void *states, const void *Cm, void *cb, const SsdOpts &o, const Dims &d,
                                 hipStream_t s)
{
    // GEMM1 workgroups hold up to 128 rows of the chunk's B in LDS: size them by the chunk length
    if (d.Q > 128) return launch_cs_t<TIn, true, 256>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
    if (d.Q > 64) return launch_cs_t<TIn, true, 128>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
    return launch_cs_t<TIn, true, 64>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
}

hipError_t launch_cumsum_chunk_state_gemm1(const void *x, const void *Bm, const void *dt, const float *A,
                                           float *acum, float *dtc, void *states, const void *Cm, void *cb,
                                           const SsdOpts &o, const Dims &d, hipStream_t s, bool pair)
{
    if (!d.half()) return launch_fused_t<float>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
    if (pair && chunk_state_pair_fits(d))
        return launch_chunk_state_pair(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
    if (d.in == kInFp8) return launch_fused_t<fp8_t>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
    return launch_fused_t<bf16_t>(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s);
}

}  // namespace ssd
