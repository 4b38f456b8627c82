// ssd_chunk_scan.hip -- Step-1 (Hadamard mask + GEMM2) + Step-4 (off-diagonal) + skip.
//
// For token i of chunk c (chunk-local index), with the chunk's cumulative
// decay a = dA_cum, the state H_enter entering the chunk and the chunk's
// C.B^T products G (formed once per group by the GEMM1 kernel):
//
//   y_i = sum_{j<=i} G[i, j] exp(a_i - a_j) dt_j x_j     Step-1: Hadamard mask, GEMM2 over j
//       + exp(a_i) H_enter C_i                           Step-4: off-diagonal
//       + D_h x_i                                        skip
//
// Sources: "Mamba-Family State-Space Model Kernels on a Programmable CGLA",
// Sec. III-A and IV-B (Step-1 = GEMM1, element-wise mask of R, GEMM2; a
// fused mask+GEMM2 removes a round trip per chunk) and "Mambalaya: Einsum-
// Based Fusion Optimizations on State-Space Models", Fig. 2-5 (fusing
// consecutive Einsums removes the inter-Einsum traffic).  Here the mask,
// GEMM2, the off-diagonal product and the skip term are fused in one kernel:
// the masked score tile never leaves registers.
//
// Work split: a persistent grid (one workgroup of one wavefront per 16-row tile, 16
// wavefronts for Q = 256, as many workgroups as the compute units hold) in which each
// workgroup loops over a contiguous run of (b, c, h) items, the heads of a chunk in a row.
// The four wavefronts that share a SIMD take tiles {s, 7-s, 8+s, 15-s}, which balances the
// causal triangle across the SIMDs.  Per item the chunk's X (fp16, row-major as it arrives),
// the entering state (fp16) and the decay tables are staged in LDS, with two barriers; after
// them every wavefront runs on its own.  A wavefront holds the fp16 slices of G for its row
// tile (one coalesced 1 KB read per 32-column step) and its C rows in registers, and keeps
// them for the next head of the same chunk; every lane holds one row i and eight columns j
// of a slice -- a row-slice of the GEMM2 A operand.  The mask/decay/dt scaling is applied in
// registers and the result is rounded to fp16 for GEMM2 (bf16 would round the computed
// scores to 2^-9, too coarse for the error budget); the X operand, whose reduction index is
// the token, is read with the transposing LDS read.  fp32 inputs store X transposed and run
// the fp32 matrix path.  Columns above the diagonal are skipped.
#include <atomic>
#include <type_traits>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

// LDS plan of one workgroup.  bf16 inputs whose footprint allows it also get a raw
// staging area that the next item's X, entering state and chunk tables stream into
// (direct-to-LDS loads: no registers held while the current item is computed).
template <typename TIn, int P, int N, int NW> struct ScanLds {
    typedef Traits<TIn> Tr;
    typedef typename Tr::op_t op_t;
    static constexpr bool F32 = Tr::kF32;
    static constexpr int ROWS = 16 * NW;               // chunk rows held (>= Q)
    // X: bf16 inputs keep it row-major [ROWS][P + 16] (fp16), read for GEMM2 with the
    // transposing LDS read; fp32 inputs store it transposed [P][ROWS + 4].
    static constexpr int LDX = F32 ? ROWS + 4 : P + 16;
    static constexpr int XSZ = F32 ? P * LDX : ROWS * LDX;
    static constexpr int LDH = N + 8;                  // H_enter rows [P][N] (fp16), bf16 only
    static constexpr int HSZ = F32 ? 1 : P * LDH;
    static constexpr int TAB = ROWS + 32;              // tables padded past the last step
    // tables: dA_cum and dt in fp32, the off-diagonal column factors in fp32 (fp32 inputs) or
    // fp16 (bf16 inputs, which scale their fp16 scores in packed fp16)
    static constexpr int base = XSZ * (int)sizeof(op_t) + HSZ * 2 + 2 * TAB * 4 + TAB * (F32 ? 4 : 2);
    // raw staging: X rows, fp16 entering state, dA_cum and dt, and 1 KB that absorbs the
    // surplus loads of streaming wavefronts with less to stream (each issues the same count)
    static constexpr int SX = ROWS * P * 2, SH = P * N * 2, ST = 2 * ROWS * 4, SD = 1024;
    static constexpr int SALL = SX + SH + ST + SD;
    // (fp8 inputs: no staging; their rows are loaded into registers and widened)
    static constexpr bool STAGE = !F32 && std::is_same<TIn, bf16_t>::value && base + SALL <= 160 * 1024;
    static constexpr int bytes = base + (STAGE ? SALL : 0);
};

// OPT: the options of the model-adjacent entry point (z gate, bf16 y) are compiled in;
// without them the kernel is exactly the plain chunk scan.
template <typename TIn, int P, int N, int NW, bool OPT>
__global__ __launch_bounds__(64 * NW) void chunk_scan_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ Cm, const void *__restrict__ cbg,
    const float *__restrict__ acum, const float *__restrict__ dtc, const void *__restrict__ henv,
    const float *__restrict__ D, void *__restrict__ y, SsdOpts opt, int L, int H, int G, int sx, int sbc, int sz, int Q, int nc,
    int nitems)
{
    typedef ScanLds<TIn, P, N, NW> S;
    typedef typename S::op_t op_t;
    constexpr bool F32 = S::F32, STAGE = S::STAGE;
    constexpr int ROWS = S::ROWS, LDX = S::LDX, LDH = S::LDH;
    constexpr int TP = P / 16;
    constexpr int KS = F32 ? N / 4 : N / 32;  // k steps over the state dim
    constexpr int NT = 64 * NW;               // threads per workgroup (>= S::TAB)
    constexpr int NSMAX = NW >= 8 ? NW / 2 : 2;  // most 32-column steps of one row tile
    __shared__ op_t xs[S::XSZ];
    __shared__ op_t hs[S::HSZ];
    // chunk tables: cumulative decay in log2 units, dt, and exp(a_r - a_j) dt_j with a_r the
    // last column of j's 32-column step (zero past the chunk; padding is never used unmasked)
    __shared__ float acs[S::TAB], dts[S::TAB];
    __shared__ __align__(16) float ecs[F32 ? S::TAB : 1];
    __shared__ __align__(16) f16 ech[F32 ? 1 : S::TAB];
    __shared__ __align__(16) unsigned char stg[STAGE ? S::SALL : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
    const int li = lane & 15, lg = lane >> 4;
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
    const int ns = t >= 0 ? (ibase + 15) / 32 + 1 : 0;  // 32-column steps up to the diagonal
    const int spc = (nt & 1) ? ((nt >> 1) + 1) * ((nt >> 1) + 1) : (nt >> 1) * ((nt >> 1) + 1);
    const int Tt = t < 0 ? 0 : (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);

    // Per-lane addresses of the staging, conversion and store code do not change from
    // item to item; left alone, the compiler computes them all once and keeps them live
    // across the item loop, which spills registers.  Adding an opaque zero, produced
    // afresh in every iteration, makes it recompute them where they are used instead.
    auto opaque_zero = [] {
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        return z;
    };

    // Item k is head h of chunk c of batch entry b, k = (b nc + c) H + h: consecutive items
    // share the chunk's C rows and C.B^T slices (one group per H / G heads).
    struct Item {
        int c, h, b, g, vrows;
        size_t bhc;
        long tc;
    };
    auto decode = [&](int item) {
        Item it;
        it.h = item % H;
        it.c = (item / H) % nc;
        it.b = item / (nc * H);
        it.g = it.h / (H / G);
        it.bhc = ((size_t)it.b * H + it.h) * nc + it.c;
        it.tc = (long)it.c * Q;
        it.vrows = (int)((L - it.tc) < Q ? (L - it.tc) : Q);
        return it;
    };
    // buffer resource over the item's valid rows of X: rows past the chunk or the
    // sequence read as zeros (the masked columns of the last step multiply finite values)
    auto x_rsrc = [&](const Item &it) {
        return make_rsrc(x + ((size_t)it.b * L + it.tc) * sx + (size_t)it.h * P,
                         (uint32_t)(((it.vrows - 1) * sx + P) * sizeof(TIn)));
    };

    // ---- staging (bf16 inputs): direct-to-LDS loads of the raw X rows, the fp16 entering
    // state and the item's dA_cum / dt, each wavefront instruction filling 1 KB (or 256 B for
    // the tables) of the staging area.  Every streaming wavefront issues the same number of
    // loads; a surplus one reads an empty range into the spare 1 KB.  (With live == false
    // every load reads an empty range: the count stays the same.)
    auto stage_issue = [&](const Item &it, bool live) {
        if constexpr (STAGE) {
            // Only the wavefronts with the light row tiles (the first NL, whose tiles have at
            // most half of the steps) stream the next item: the heavy tiles' wavefronts go
            // straight from the barrier to their steps instead of queueing behind the store
            // traffic at the vector-memory path.
            constexpr int NL = NW >= 8 ? NW / 2 : NW;
            if (wave >= NL) return;
            const int lane = (tid & 63) + opaque_zero();
            constexpr int XI = S::SX / 1024, HI = S::SH / 1024, TI = ROWS / 64;
            unsigned char *spare = stg + S::SX + S::SH + S::ST;
            const __amdgpu_buffer_rsrc_t rx = live ? x_rsrc(it) : make_rsrc(x, 0u);
#pragma unroll
            for (int k = 0; k < (XI + NL - 1) / NL; ++k) {
                const int wi = k * NL + wave;
                const int byte = 1024 * wi + 16 * lane, row = byte / (2 * P), col = byte % (2 * P);
                // (a uniform branch: X streamed past the Infinity Cache, see SsdOpts::stream_x)
                if (opt.stream_x)
                    buf_load_lds16<kStream>(wi < XI ? rx : make_rsrc(x, 0u), wi < XI ? stg + 1024 * wi : spare,
                                            (uint32_t)(row * sx * 2 + col));
                else
                    buf_load_lds16(wi < XI ? rx : make_rsrc(x, 0u), wi < XI ? stg + 1024 * wi : spare,
                                   (uint32_t)(row * sx * 2 + col));
            }
            const f16 *hen = static_cast<const f16 *>(henv);
            const __amdgpu_buffer_rsrc_t rh = make_rsrc(hen + it.bhc * P * N, live ? (uint32_t)S::SH : 0u);
#pragma unroll
            for (int k = 0; k < (HI + NL - 1) / NL; ++k) {
                const int wi = k * NL + wave;
                if (opt.stream_x)
                    buf_load_lds16<kStream>(wi < HI ? rh : make_rsrc(hen, 0u), wi < HI ? stg + S::SX + 1024 * wi : spare,
                                            (uint32_t)(1024 * wi + 16 * lane));
                else
                    buf_load_lds16(wi < HI ? rh : make_rsrc(hen, 0u), wi < HI ? stg + S::SX + 1024 * wi : spare,
                                   (uint32_t)(1024 * wi + 16 * lane));
            }
            // tables: slots 0 .. TI-1 stream dA_cum, TI .. 2TI-1 stream dt (zeros past Q)
#pragma unroll
            for (int k = 0; k < (2 * TI + NL - 1) / NL; ++k) {
                const int slot = k * NL + wave;
                const bool has = live && slot < 2 * TI;
                const int tab = has ? slot / TI : 0, wi = has ? slot % TI : 0;
                const float *src = (tab == 0 ? acum : dtc) + it.bhc * Q;
                const __amdgpu_buffer_rsrc_t rt = make_rsrc(src, has ? (uint32_t)(Q * 4) : 0u);
                buf_load_lds4(rt, has ? stg + S::SX + S::SH + tab * ROWS * 4 + 256 * wi : spare,
                                (uint32_t)(4 * (64 * wi + lane)));
            }
        }
    };
    // staged (or, without staging, freshly loaded) item -> the compute layout in LDS
    auto stage_commit = [&](const Item &it) {
        const int tid = threadIdx.x + opaque_zero();
        constexpr int XR = F32 ? 2 : 1;  // X rows per unit
        constexpr int XU = (ROWS / XR) * (P / 8), XPT = (XU + NT - 1) / NT;
        constexpr int HU = F32 ? 1 : P * N / 8, HPT = (HU + NT - 1) / NT;
        float ta = 0.f, tr = 0.f, td = 0.f;
        const int ir = min(32 * (tid >> 5) + 31, Q - 1);
        if constexpr (STAGE) {
            const bf16_t *sx = reinterpret_cast<const bf16_t *>(stg);
            const f16 *sh = reinterpret_cast<const f16 *>(stg + S::SX);
            const float *st = reinterpret_cast<const float *>(stg + S::SX + S::SH);
#pragma unroll
            for (int k = 0; k < XPT; ++k) {
                const int u = tid + k * NT;
                if (u < XU) {
                    Raw8<bf16_t> r;
                    r.v = *reinterpret_cast<const uint4 *>(sx + 8 * u);
                    *reinterpret_cast<uint4 *>(&xs[(u / (P / 8)) * LDX + 8 * (u % (P / 8))]) = raw8_to_f16x8(r);
                }
            }
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int u = tid + k * NT;
                if (u < HU)
                    *reinterpret_cast<uint4 *>(&hs[(u / (N / 8)) * LDH + 8 * (u % (N / 8))]) =
                        *reinterpret_cast<const uint4 *>(sh + 8 * u);
            }
            if (tid < Q) {
                ta = st[tid];
                tr = st[ir];
                td = st[ROWS + tid];
            }
        } else {
            const __amdgpu_buffer_rsrc_t rx = x_rsrc(it);
            Raw8<TIn> px[XPT][XR];
            uint4 ph[HPT];
#pragma unroll
            for (int k = 0; k < XPT; ++k) {
                const int u = tid + k * NT;
                if (u < XU) {
                    const int jr = u / (P / 8), cg = u % (P / 8);
#pragma unroll
                    for (int e = 0; e < XR; ++e) px[k][e].load(rx, (uint32_t)((XR * jr + e) * sx + 8 * cg));
                }
            }
            if constexpr (!F32) {
                const f16 *hp = static_cast<const f16 *>(henv) + it.bhc * P * N;
#pragma unroll
                for (int k = 0; k < HPT; ++k) {
                    const int u = tid + k * NT;
                    if (u < HU) ph[k] = *reinterpret_cast<const uint4 *>(hp + 8 * u);
                }
            }
            if (tid < Q) {
                ta = acum[it.bhc * Q + tid];
                tr = acum[it.bhc * Q + ir];
                td = dtc[it.bhc * Q + tid];
            }
#pragma unroll
            for (int k = 0; k < XPT; ++k) {
                const int u = tid + k * NT;
                if (u < XU) {
                    const int jr = u / (P / 8), cg = u % (P / 8);
                    if constexpr (F32) {
                        float v0[8], v1[8];
                        px[k][0].to_f32(v0);
                        px[k][XR - 1].to_f32(v1);
#pragma unroll
                        for (int kk = 0; kk < 8; ++kk) store_pair(&xs[(8 * cg + kk) * LDX + 2 * jr], v0[kk], v1[kk]);
                    } else {
                        *reinterpret_cast<uint4 *>(&xs[jr * LDX + 8 * cg]) = raw8_to_f16x8(px[k][0]);
                    }
                }
            }
            if constexpr (!F32) {
#pragma unroll
                for (int k = 0; k < HPT; ++k) {
                    const int u = tid + k * NT;
                    if (u < HU) *reinterpret_cast<uint4 *>(&hs[(u / (N / 8)) * LDH + 8 * (u % (N / 8))]) = ph[k];
                }
            }
        }
        if (tid < S::TAB) {
            float a = 0.f, d = 0.f, e = 0.f;
            if (tid < Q) {
                a = ta * kLog2e;
                d = td;
                e = __builtin_amdgcn_exp2f(tr * kLog2e - a) * d;
            }
            acs[tid] = a;
            dts[tid] = d;
            if constexpr (F32)
                ecs[tid] = e;
            else
                ech[tid] = static_cast<f16>(e);
        }
    };

    // ---- per-wavefront operands of an item, held in registers: the C rows of the tile
    // (off-diagonal A operand) and, for bf16 inputs, all of the tile's fp16 slices of G
    bf16x8 cb[F32 ? 1 : KS];  // bf16 as loaded; fp16 bit patterns once converted (cfresh false)
    float cf[F32 ? KS : 1];
    f16x8 gs[F32 ? 1 : NSMAX - 1];  // the steps below the diagonal
    f16x8 gdg;                      // the diagonal step
    bool cfresh = false;  // cb holds newly loaded raw rows (wavefront-uniform)
    // Issued when an item's chunk or group differs from the previous item's, at the end of
    // the previous item.  A wavefront without a tile reads slice 0 and C rows past the buffer
    // range, which return zeros.
    auto load_tile_operands = [&](const Item &it) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + ((size_t)it.b * L + it.tc) * sbc + (size_t)it.g * N,
                                                    (uint32_t)(((it.vrows - 1) * sbc + N) * sizeof(TIn)));
        const uint32_t row = (uint32_t)((ibase + li) * sbc);
        if constexpr (F32) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                cf[ks] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(4u * (row + ks * 4 + lg)), 0, 0));
        } else {
            const size_t slice0 = (((size_t)it.b * G + it.g) * nc + it.c) * (size_t)spc + Tt;
            const f16 *gq = static_cast<const f16 *>(cbg) + (slice0 * 64 + lane) * 8;
            const int slast = ns > 0 ? ns - 1 : 0;
#pragma unroll
            for (int s = 0; s < NSMAX - 1; ++s) gs[s] = *reinterpret_cast<const f16x8 *>(gq + (size_t)min(s, slast) * 512);
            gdg = *reinterpret_cast<const f16x8 *>(gq + (size_t)slast * 512);
            if constexpr (std::is_same<TIn, fp8_t>::value) {
                // e4m3 rows (8 bytes per 8 elements) in the low half, widened with the bf16 rows
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint2 v = buf_load8(rc, row + ks * 32 + 8 * lg);
                    cb[ks] = __builtin_bit_cast(bf16x8, make_uint4(v.x, v.y, 0u, 0u));
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
            }
            cfresh = true;
        }
    };

    // The output tile is formed transposed: every product takes X (or the entering state) as
    // the A operand and the scores (or the C rows) as the B operand, so that lane (li, lg)
    // holds y[ibase + li][16 pt + 4 lg + r], r = 0..3 -- four consecutive channels of one row,
    // written with one 16-byte store per channel tile.  y of an item is written when the
    // wavefront's tile is done, as its youngest memory operations (buffer stores over the
    // item's valid rows, which drop rows past the sequence and every store of a wavefront
    // without a tile: every wavefront issues TP of them).
    f32x4 acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
    // s_waitcnt with vmcnt(TP) (expcnt and lgkmcnt left at their maxima): the gfx9 encoding
    // splits vmcnt over bits 3:0 and 15:14
    constexpr int kWaitStores = (TP & 15) | (7 << 4) | (15 << 8) | ((TP >> 4) << 14);
    auto store_y = [&](const Item &it, bool live) {
        const int lane = (tid & 63) + opaque_zero(), li = lane & 15, lg = lane >> 4;
        const size_t base = (((size_t)it.b * L + it.tc) * H + it.h) * P;
        const bool y16 = OPT && opt.y_bf16;
        const uint32_t es = y16 ? 2u : 4u;  // y element size
        const __amdgpu_buffer_rsrc_t ry =
            make_rsrc(y16 ? (void *)(static_cast<uint16_t *>(y) + base) : (void *)(static_cast<float *>(y) + base),
                      live && t >= 0 ? (uint32_t)(((it.vrows - 1) * H * P + P) * es) : 0u);
        // the lane's four consecutive channels 16 pt + 4 lg .. +3 of row ibase + li: one 16-byte
        // store (8 bytes for bf16) per channel tile; rows past the sequence fall outside the range
        const uint32_t e = (uint32_t)((ibase + li) * H * P + 4 * lg);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
            if (y16) {
                const uint2 d = {pack_bf16x2(acc[pt][0], acc[pt][1]), pack_bf16x2(acc[pt][2], acc[pt][3])};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, d), ry,
                                                      (int)(2u * (e + 16 * pt)), 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, acc[pt]), ry,
                                                       (int)(4u * (e + 16 * pt)), 0, 0);
            }
        }
    };

    // Every load and store below is issued unconditionally (empty ranges stand in for
    // the ones with nothing to do), so that each wait counts exactly the younger
    // operations it may leave in flight.
    // Each workgroup takes a contiguous run of items: the heads of a chunk follow one another,
    // so a wavefront keeps its tile operands (the C rows and the C.B^T slices of its row tile)
    // in registers from one head to the next and loads them again only when the chunk or the
    // group changes.  Workgroups are dispatched to the XCDs in turn; the runs are laid out so
    // that the workgroups of one XCD take adjacent runs and share the chunks in its L2.
    const int nwg = gridDim.x;
    const int vw = (nwg & 7) == 0 ? (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int per = nitems / nwg, extra = nitems % nwg;
    int item = vw * per + min(vw, extra);
    const int last = item + per + (vw < extra ? 1 : 0);
    Item cur = decode(item);
    stage_issue(cur, true);
    load_tile_operands(cur);
    store_y(cur, false);  // empty range: the same youngest operations as every later item sees
    for (;;) {
        const float Dh = D ? D[cur.h] : 0.f;
        // Every memory operation but this wavefront's y stores of the previous item (its TP
        // youngest) has completed: the item's staged loads have landed, and so have the tile
        // operand loads issued before those stores.  The stores drain during this item.
        __builtin_amdgcn_s_waitcnt(kWaitStores);
        __syncthreads();  // ... and every wavefront's staged loads have landed; the previous item's readers are done
        stage_commit(cur);
        __syncthreads();
        const int next = item + 1;
        const bool more = next < last;
        const Item nx = more ? decode(next) : cur;
        stage_issue(nx, more);

        if (t >= 0) {
            const int irow = ibase + li;
            const float ai = acs[irow];
            // ---- Step-4 first: exp(a_i) * (C_i . H_enter[p, :]) for this wavefront's rows,
            // scaled in the accumulator that Step-1 then adds to
            {
                const float *hp = static_cast<const float *>(henv) + cur.bhc * P * N;  // fp32 inputs only
                if constexpr (!F32) {
                    // the C rows of a new chunk: to fp16 once, kept for the chunk's other heads
                    // (exact for bf16 inputs in fp16 range)
                    if (cfresh) {
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, held_to_f16x8<TIn>(cb[ks]));
                        cfresh = false;
                    }
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        if constexpr (F32) {
                            acc[pt] = mfma16x16x4_f32(hp[(pt * 16 + li) * N + ks * 4 + lg], cf[ks], acc[pt]);
                        } else {
                            const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                            acc[pt] = mfma16x16x32_f16(hf, __builtin_bit_cast(f16x8, cb[ks]), acc[pt]);
                        }
                    }
                }
                const float e = __builtin_amdgcn_exp2f(ai);  // the lane's row: exp(a_i)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[pt][r] *= e;
            }
            // ---- Step-1: the causal 32-column steps of this row tile.  All but the last lie
            // strictly below the diagonal; the last one holds it (tile t: steps 0 .. t/2).
            const size_t slice0 = (((size_t)cur.b * G + cur.g) * nc + cur.c) * (size_t)spc + Tt;
            const float *gf = static_cast<const float *>(cbg) + (slice0 * 64 + lane) * 8;
            // Lane holds G[irow][jb + 4 lg + r] (d0) and G[irow][jb + 16 + 4 lg + r] (d1): the B
            // operand of the transposed product, column irow of the score tile.
            auto slice = [&](int s, float d0[4], float d1[4]) {
                if constexpr (F32) {
                    const float4 g0 = reinterpret_cast<const float4 *>(gf + (size_t)s * 512)[0];
                    const float4 g1 = reinterpret_cast<const float4 *>(gf + (size_t)s * 512)[1];
                    d0[0] = g0.x; d0[1] = g0.y; d0[2] = g0.z; d0[3] = g0.w;
                    d1[0] = g1.x; d1[1] = g1.y; d1[2] = g1.z; d1[3] = g1.w;
                }
            };
            // GEMM2 of one step (bf16 inputs): the fp16 score fragment a times X, k slots of lane
            // group lg being columns {jb+4lg+r, jb+16+4lg+r}
            auto gemm2h = [&](int jb, const f16x8 &a) {
                if constexpr (!F32) {
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        // lane li receives X[jb + 4 lg + r][16 pt + li] and X[jb + 16 + 4 lg + r][16 pt + li]
                        const int ox = tr16_offset(lane, jb, pt * 16, LDX);
                        const f16x4 lo = lds_read_tr16(&xs[ox]);
                        const f16x4 hi = lds_read_tr16(&xs[ox + 16 * LDX]);
                        const f16x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc[pt] = mfma16x16x32_f16(bx, a, acc[pt]);
                    }
                }
            };
            auto gemm2 = [&](int jb, bool has1, const float r0[4], const float r1[4]) {
                if constexpr (F32) {
#pragma unroll
                    for (int pt = 0; pt < TP; ++pt) {
                        const op_t *xr = &xs[(pt * 16 + li) * LDX + jb + 4 * lg];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(xr[r], r0[r], acc[pt]);
                        if (has1) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[pt] = mfma16x16x4_f32(xr[16 + r], r1[r], acc[pt]);
                        }
                    }
                } else {
                    f16x8 a;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a[r] = static_cast<f16>(r0[r]);
                        a[4 + r] = static_cast<f16>(r1[r]);
                    }
                    gemm2h(jb, a);
                }
            };
#pragma unroll
            for (int s = 0; s + 1 < NSMAX; ++s) {
                if (s + 1 < ns) {
                    // Strictly below the diagonal: factor the decay through the step's last
                    // column a_r, exp(a_i - a_j) = exp(a_i - a_r) exp(a_r - a_j).  Both factors
                    // are <= 1 (a is non-increasing for A <= 0) and any underflow drops a term
                    // smaller still; exp(a_r - a_j) dt_j is the chunk table.
                    const int jb = 32 * s;
                    const float er = __builtin_amdgcn_exp2f(ai - acs[jb + 31]);
                    if constexpr (F32) {
                        float d0[4], d1[4];
                        slice(s, d0, d1);
                        const float4 e0 = *reinterpret_cast<const float4 *>(&ecs[jb + 4 * lg]);
                        const float4 e1 = *reinterpret_cast<const float4 *>(&ecs[jb + 16 + 4 * lg]);
                        const float ej0[4] = {e0.x, e0.y, e0.z, e0.w}, ej1[4] = {e1.x, e1.y, e1.z, e1.w};
                        float r0[4], r1[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            r0[r] = d0[r] * (er * ej0[r]);
                            r1[r] = d1[r] * (er * ej1[r]);
                        }
                        gemm2(jb, true, r0, r1);
                    } else {
                        // in packed fp16: G (fp16) * (exp(a_i - a_r) * table), both factors in
                        // (0, 1] times dt; a factor below the fp16 range drops a negligible term
                        const f16x4 e0 = *reinterpret_cast<const f16x4 *>(&ech[jb + 4 * lg]);
                        const f16x4 e1 = *reinterpret_cast<const f16x4 *>(&ech[jb + 16 + 4 * lg]);
                        const f16x8 ej = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
                        gemm2h(jb, gs[s] * (ej * static_cast<f16>(er)));
                    }
                }
            }
            {
                // the diagonal step: direct exponentials under the causal mask
                const int sd = ns - 1, jb = 32 * sd;
                const bool has1 = jb + 16 <= ibase + 15;  // second 16-column half not all masked
                float d0[4], d1[4];
                if constexpr (F32) {
                    slice(sd, d0, d1);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        d0[r] = static_cast<float>(gdg[r]);
                        d1[r] = static_cast<float>(gdg[4 + r]);
                    }
                }
                const float4 a0v = *reinterpret_cast<const float4 *>(&acs[jb + 4 * lg]);
                const float4 t0v = *reinterpret_cast<const float4 *>(&dts[jb + 4 * lg]);
                const float4 a1v = *reinterpret_cast<const float4 *>(&acs[jb + 16 + 4 * lg]);
                const float4 t1v = *reinterpret_cast<const float4 *>(&dts[jb + 16 + 4 * lg]);
                const float aj0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, tj0[4] = {t0v.x, t0v.y, t0v.z, t0v.w};
                const float aj1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, tj1[4] = {t1v.x, t1v.y, t1v.z, t1v.w};
                float r0[4], r1[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    r0[r] = (jb + 4 * lg + r <= irow) ? d0[r] * __builtin_amdgcn_exp2f(ai - aj0[r]) * tj0[r] : 0.f;
                    r1[r] = (has1 && jb + 16 + 4 * lg + r <= irow) ? d1[r] * __builtin_amdgcn_exp2f(ai - aj1[r]) * tj1[r]
                                                                   : 0.f;
                }
                gemm2(jb, has1, r0, r1);
            }
            // ---- skip term
            if constexpr (F32) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * xs[(pt * 16 + 4 * lg + r) * LDX + irow];
            } else {
                // the lane's four channels of its row, one 8-byte read (exact for bf16 inputs in
                // fp16 range)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const f16x4 xv = *reinterpret_cast<const f16x4 *>(&xs[irow * LDX + pt * 16 + 4 * lg]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * static_cast<float>(xv[r]);
                }
            }
        }
        // ---- optional output gate: y <- y * z * sigmoid(z), z laid out as x
        if (OPT && opt.z && t >= 0) {
            typedef typename Traits<TIn>::dt_t zt;  // bf16 beside fp8 inputs
            const zt *zp = static_cast<const zt *>(opt.z) + ((size_t)cur.b * L + cur.tc) * sz + (size_t)cur.h * P;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(zp, (uint32_t)(((cur.vrows - 1) * sz + P) * sizeof(zt)));
            // all of the lane's z values are requested before the first is used
            uint32_t zr[TP][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const uint32_t e = (uint32_t)((ibase + li) * sz + pt * 16 + 4 * lg + r);
                    if constexpr (F32)
                        zr[pt][r] = __builtin_amdgcn_raw_buffer_load_b32(rz, (int)(4u * e), 0, 0);
                    else
                        zr[pt][r] = __builtin_amdgcn_raw_buffer_load_b16(rz, (int)(2u * e), 0, 0);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const float zf = F32 ? __uint_as_float(zr[pt][r]) : __uint_as_float(zr[pt][r] << 16);
                    acc[pt][r] *= silu(zf);
                }
        }
        // the next item's tile operands when its chunk or group differs, in flight while its
        // staging completes
        if (more && (nx.c != cur.c || nx.b != cur.b || nx.g != cur.g)) load_tile_operands(nx);
        // y last: a wavefront's stores go out when its own tile is done (the light tiles'
        // first), after every load that the next item's wait must see completed
        store_y(cur, true);
        if (!more) break;
        item = next;
        cur = nx;
    }
}

// ---- The pipelined chunk scan (bf16 or fp8 inputs, P = 64, N = 128, 256-token chunks): the same
// arithmetic in the same order as chunk_scan_kernel (the compiler may contract the decay
// table's multiply-add differently, a last-bit difference in a few table entries), with one
// barrier per item instead of two.  The compute layout is double-buffered: while every
// wavefront forms item k from one buffer set, the wavefronts with the light row tiles (the
// first eight, whose tiles have at most four 32-column steps) stream item k+1 with
// direct-to-LDS loads -- X rows raw into a staging area, the fp16 entering state straight
// into the other set's padded rows (one 256-byte row per load), the decay tables raw -- and,
// once their own tile is done, convert the X rows and tables they loaded themselves into the
// other set.  The heavy tiles' wavefronts only compute and store.  Each buffer set is its own
// LDS array and the set an item uses is fixed at compile time (the item loop is unrolled by
// two), so the compiler can tell the loads in flight from the reads of the current set.
// Row pitches: X rows (P + 16) halves, so that the 16 rows of one transposing read fall on
// distinct bank groups; entering-state rows (N + 16) halves, which took the 2.7B chunk scan
// 122 -> 119.5 us against (N + 8) (fewer LDS bank conflicts in the Step-4 reads).
template <int P, int N, int NW> struct PipeLds {
    static constexpr int ROWS = 16 * NW, LDX = P + 16, LDH = N + 16, TAB = ROWS + 32;
    static constexpr int XS = ROWS * LDX, HS = P * LDH;           // halves per set
    static constexpr int SX = ROWS * P * 2, ST = 2 * ROWS * 4;    // raw X rows, raw tables
    static constexpr int bytes = 2 * (XS * 2 + HS * 2 + TAB * (4 + 4 + 2)) + SX + ST;
    static constexpr bool fits = bytes <= 160 * 1024;
};

// TX: storage of x and C (bf16, or fp8 e4m3: half the raw X bytes to stream; both widen to
// fp16 exactly).  GATE: the z gate is applied; Y16: y is stored as bf16.  Each combination is
// its own instantiation, so the plain and the bf16-y kernels carry no registers for the gate.
// SCP: cache policy of the X and entering-state streams (kStream when X is too large to stay
// in the Infinity Cache between launches: neither is read again, and streamed they leave the
// cache to what the next launches read back).
template <typename TX, int P, int N, int NW, bool GATE, bool Y16, int SCP>
__global__ __launch_bounds__(64 * NW) void chunk_scan_pipe_kernel(
    const TX *__restrict__ x, const TX *__restrict__ Cm, const void *__restrict__ cbg,
    const float *__restrict__ acum, const float *__restrict__ dtc, const void *__restrict__ henv,
    const float *__restrict__ D, void *__restrict__ y, SsdOpts opt, int L, int H, int G, int sx, int sbc, int sz,
    int Q, int nc, int nitems)
{
    typedef PipeLds<P, N, NW> S;
    constexpr int ROWS = S::ROWS, LDX = S::LDX, LDH = S::LDH, TAB = S::TAB;
    constexpr int TP = P / 16, KS = N / 32, NSMAX = NW / 2;
    constexpr int NL = NW / 2;            // streaming wavefronts: the light row tiles
    constexpr bool F8 = std::is_same<TX, fp8_t>::value;
    constexpr int RB = P * (int)sizeof(TX);                  // bytes of one raw X row
    constexpr int XI = ROWS * RB / 1024;  // 1 KB X slots; wavefront q owns slots q, q + NL, ...
    constexpr int TI = ROWS / 64;         // 64-row table blocks; wavefront q < TI owns block q
    static_assert(NW == 16 && 2 * N == 256 && XI % NL == 0 && P % NL == 0 && TI <= NL, "pipelined scan shape");
    __shared__ __align__(16) f16 xs0[S::XS];
    __shared__ __align__(16) f16 xs1[S::XS];
    __shared__ __align__(16) f16 hs0[S::HS];
    __shared__ __align__(16) f16 hs1[S::HS];
    __shared__ __align__(16) float acs0[TAB];
    __shared__ __align__(16) float acs1[TAB];
    __shared__ __align__(16) float dts0[TAB];
    __shared__ __align__(16) float dts1[TAB];
    __shared__ __align__(16) f16 ech0[TAB];
    __shared__ __align__(16) f16 ech1[TAB];
    __shared__ __align__(16) unsigned char stg[S::SX + S::ST];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    // row tile: the k-th wavefront on SIMD s (wave = 4k + s) takes tile 8(k/2) + s for even k
    // and 8(k/2) + 7 - s for odd k (tiles 0..7 for the first eight wavefronts)
    const int t = [&] {
        const int s = wave & 3, k = wave >> 2;
        return 8 * (k >> 1) + ((k & 1) ? 7 - s : s);
    }();
    const int ibase = 16 * t;
    const int ns = (ibase + 15) / 32 + 1;  // 32-column steps up to the diagonal
    const int nt = Q >> 4;
    const int spc = (nt >> 1) * ((nt >> 1) + 1);
    const int Tt = (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);
    const bool light = wave < NL;

    auto opaque_zero = [] {
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        return z;
    };
    struct Item {
        int c, h, b, g, vrows;
        size_t bhc;
        long tc;
    };
    auto decode = [&](int item) __attribute__((always_inline)) {
        Item it;
        it.h = item % H;
        it.c = (item / H) % nc;
        it.b = item / (nc * H);
        it.g = it.h / (H / G);
        it.bhc = ((size_t)it.b * H + it.h) * nc + it.c;
        it.tc = (long)it.c * Q;
        it.vrows = (int)((L - it.tc) < Q ? (L - it.tc) : Q);
        return it;
    };

    // the table rows past the chunk (read, always masked or zero-weighted, by the last steps)
    if (tid < TAB - ROWS) {
        acs0[ROWS + tid] = 0.f;
        acs1[ROWS + tid] = 0.f;
        dts0[ROWS + tid] = 0.f;
        dts1[ROWS + tid] = 0.f;
        ech0[ROWS + tid] = static_cast<f16>(0.f);
        ech1[ROWS + tid] = static_cast<f16>(0.f);
    }

    // ---- streaming (light wavefronts): X rows raw into the staging slots this wavefront
    // owns, the entering state's rows straight into the next set, and (the first TI) the raw
    // dA_cum / dt block they own.  live == false: empty ranges (nothing is read).
    auto stream = [&](const Item &it, bool live, f16 *hsn) __attribute__((always_inline)) {
        const int ln = lane + opaque_zero();
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(x + ((size_t)it.b * L + it.tc) * sx + (size_t)it.h * P,
                      live ? (uint32_t)(((it.vrows - 1) * sx + P) * sizeof(TX)) : 0u);
#pragma unroll
        for (int k = 0; k < XI / NL; ++k) {
            const int wi = k * NL + wave;
            const int byte = 1024 * wi + 16 * ln, row = byte / RB, col = byte % RB;
            buf_load_lds16<SCP>(rx, stg + 1024 * wi, (uint32_t)(row * sx * (int)sizeof(TX) + col));
        }
        const __amdgpu_buffer_rsrc_t rh =
            make_rsrc(static_cast<const f16 *>(henv) + it.bhc * P * N, live ? (uint32_t)(P * N * 2) : 0u);
#pragma unroll
        for (int k = 0; k < P / NL; ++k) {
            const int p = k * NL + wave;
            buf_load_lds4<SCP>(rh, hsn + p * LDH, (uint32_t)(p * N * 2 + 4 * ln));
        }
        if (wave < TI) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(acum + it.bhc * Q, live ? (uint32_t)(Q * 4) : 0u);
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(dtc + it.bhc * Q, live ? (uint32_t)(Q * 4) : 0u);
            buf_load_lds4(ra, stg + S::SX + 256 * wave, (uint32_t)(4 * (64 * wave + ln)));
            buf_load_lds4(rd, stg + S::SX + ROWS * 4 + 256 * wave, (uint32_t)(4 * (64 * wave + ln)));
        }
    };
    // ---- conversion (light wavefronts, after their own loads have landed): the X rows of the
    // slots they own to fp16, and the tables of the block they own
    auto convert = [&](f16 *xsn, float *acsn, float *dtsn, f16 *echn) __attribute__((always_inline)) {
        const int ln = lane + opaque_zero();
#pragma unroll
        for (int k = 0; k < XI / NL; ++k) {
            const int u = 64 * (k * NL + wave) + ln;  // 16-byte unit of the staged rows
            const uint4 r = *reinterpret_cast<const uint4 *>(stg + 16 * u);
            if constexpr (F8) {
                // 16 channels: row u / (P / 16), channels 16 (u % (P / 16)) onwards
                f16 *dst = &xsn[(u / (P / 16)) * LDX + 16 * (u % (P / 16))];
                *reinterpret_cast<uint4 *>(dst) = f8x8_to_f16x8(make_uint2(r.x, r.y));
                *reinterpret_cast<uint4 *>(dst + 8) = f8x8_to_f16x8(make_uint2(r.z, r.w));
            } else {
                // 8 channels: row u / (P / 8), channels 8 (u % (P / 8)) onwards
                Raw8<bf16_t> rr;
                rr.v = r;
                *reinterpret_cast<uint4 *>(&xsn[(u / (P / 8)) * LDX + 8 * (u % (P / 8))]) = raw8_to_f16x8(rr);
            }
        }
        if (wave < TI) {
            const float *sta = reinterpret_cast<const float *>(stg + S::SX);
            const float *std_ = reinterpret_cast<const float *>(stg + S::SX + ROWS * 4);
            const int j = 64 * wave + ln;
            float a = 0.f, d = 0.f, e = 0.f;
            if (j < Q) {
                const int ir = min(32 * (j >> 5) + 31, Q - 1);
                a = sta[j] * kLog2e;
                d = std_[j];
                e = __builtin_amdgcn_exp2f(sta[ir] * kLog2e - a) * d;
            }
            acsn[j] = a;
            dtsn[j] = d;
            echn[j] = static_cast<f16>(e);
        }
    };

    // ---- tile operands in registers, kept while the chunk and group stay the same
    bf16x8 cb[KS];  // bf16 as loaded; fp16 bit patterns once converted (cfresh false)
    f16x8 gs[NSMAX - 1];
    f16x8 gdg;
    bool cfresh = false;
    auto load_tile_operands = [&](const Item &it) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + ((size_t)it.b * L + it.tc) * sbc + (size_t)it.g * N,
                                                    (uint32_t)(((it.vrows - 1) * sbc + N) * sizeof(TX)));
        const uint32_t row = (uint32_t)((ibase + li) * sbc);
        const size_t slice0 = (((size_t)it.b * G + it.g) * nc + it.c) * (size_t)spc + Tt;
        const f16 *gq = static_cast<const f16 *>(cbg) + (slice0 * 64 + lane) * 8;
        const int slast = ns - 1;
#pragma unroll
        for (int s = 0; s < NSMAX - 1; ++s) gs[s] = *reinterpret_cast<const f16x8 *>(gq + (size_t)min(s, slast) * 512);
        gdg = *reinterpret_cast<const f16x8 *>(gq + (size_t)slast * 512);
        if constexpr (F8) {
            // e4m3 rows (8 bytes per 8 elements) in the low half, widened with the bf16 rows
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint2 v = buf_load8(rc, row + ks * 32 + 8 * lg);
                cb[ks] = __builtin_bit_cast(bf16x8, make_uint4(v.x, v.y, 0u, 0u));
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
        }
        cfresh = true;
    };

    // ---- the output tile, transposed (lane (li, lg) holds y[ibase + li][16 pt + 4 lg + r]),
    // stored when the wavefront's tile is done, as its TP youngest memory operations
    f32x4 acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
    constexpr int kWaitStores = (TP & 15) | (7 << 4) | (15 << 8) | ((TP >> 4) << 14);  // vmcnt(TP)
    auto store_y = [&](const Item &it, bool live) __attribute__((always_inline)) {
        const int ln = lane + opaque_zero(), lli = ln & 15, llg = ln >> 4;
        const size_t base = (((size_t)it.b * L + it.tc) * H + it.h) * P;
        constexpr bool y16 = Y16;
        constexpr uint32_t es = y16 ? 2u : 4u;
        const __amdgpu_buffer_rsrc_t ry =
            make_rsrc(y16 ? (void *)(static_cast<uint16_t *>(y) + base) : (void *)(static_cast<float *>(y) + base),
                      live ? (uint32_t)(((it.vrows - 1) * H * P + P) * es) : 0u);
        const uint32_t e = (uint32_t)((ibase + lli) * H * P + 4 * llg);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
            if constexpr (y16) {
                const uint2 d = {pack_bf16x2(acc[pt][0], acc[pt][1]), pack_bf16x2(acc[pt][2], acc[pt][3])};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, d), ry,
                                                      (int)(2u * (e + 16 * pt)), 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, acc[pt]),
                                                       ry, (int)(4u * (e + 16 * pt)), 0, 0);
            }
        }
    };

    // ---- one item from one buffer set: Step-4, Step-1 (off-diagonal steps, diagonal step),
    // skip term, optional gate -- chunk_scan_kernel's bf16 arithmetic
    auto compute = [&](const Item &cur, const f16 *xs, const f16 *hs, const float *acs, const float *dts,
                       const f16 *ech) __attribute__((always_inline)) {
        const float Dh = D ? D[cur.h] : 0.f;
        const int irow = ibase + li;
        const float ai = acs[irow];
        if (cfresh) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, held_to_f16x8<TX>(cb[ks]));
            cfresh = false;
        }
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                acc[pt] = mfma16x16x32_f16(hf, __builtin_bit_cast(f16x8, cb[ks]), acc[pt]);
            }
        }
        {
            const float e = __builtin_amdgcn_exp2f(ai);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pt][r] *= e;
        }
        auto gemm2h = [&](int jb, const f16x8 &a) __attribute__((always_inline)) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                const int ox = tr16_offset(lane, jb, pt * 16, LDX);
                const f16x4 lo = lds_read_tr16(&xs[ox]);
                const f16x4 hi = lds_read_tr16(&xs[ox + 16 * LDX]);
                const f16x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[pt] = mfma16x16x32_f16(bx, a, acc[pt]);
            }
        };
#pragma unroll
        for (int s = 0; s + 1 < NSMAX; ++s) {
            if (s + 1 < ns) {
                const int jb = 32 * s;
                const float er = __builtin_amdgcn_exp2f(ai - acs[jb + 31]);
                const f16x4 e0 = *reinterpret_cast<const f16x4 *>(&ech[jb + 4 * lg]);
                const f16x4 e1 = *reinterpret_cast<const f16x4 *>(&ech[jb + 16 + 4 * lg]);
                const f16x8 ej = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
                gemm2h(jb, gs[s] * (ej * static_cast<f16>(er)));
            }
        }
        {
            const int jb = 32 * (ns - 1);
            const bool has1 = jb + 16 <= ibase + 15;
            float d0[4], d1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                d0[r] = static_cast<float>(gdg[r]);
                d1[r] = static_cast<float>(gdg[4 + r]);
            }
            const float4 a0v = *reinterpret_cast<const float4 *>(&acs[jb + 4 * lg]);
            const float4 t0v = *reinterpret_cast<const float4 *>(&dts[jb + 4 * lg]);
            const float4 a1v = *reinterpret_cast<const float4 *>(&acs[jb + 16 + 4 * lg]);
            const float4 t1v = *reinterpret_cast<const float4 *>(&dts[jb + 16 + 4 * lg]);
            const float aj0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, tj0[4] = {t0v.x, t0v.y, t0v.z, t0v.w};
            const float aj1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, tj1[4] = {t1v.x, t1v.y, t1v.z, t1v.w};
            f16x8 a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float r0 = (jb + 4 * lg + r <= irow) ? d0[r] * __builtin_amdgcn_exp2f(ai - aj0[r]) * tj0[r] : 0.f;
                const float r1 =
                    (has1 && jb + 16 + 4 * lg + r <= irow) ? d1[r] * __builtin_amdgcn_exp2f(ai - aj1[r]) * tj1[r] : 0.f;
                a[r] = static_cast<f16>(r0);
                a[4 + r] = static_cast<f16>(r1);
            }
            gemm2h(jb, a);
        }
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
            const f16x4 xv = *reinterpret_cast<const f16x4 *>(&xs[irow * LDX + pt * 16 + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * static_cast<float>(xv[r]);
        }
        if constexpr (GATE) {
            const bf16_t *zp = static_cast<const bf16_t *>(opt.z) + ((size_t)cur.b * L + cur.tc) * sz + (size_t)cur.h * P;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(zp, (uint32_t)(((cur.vrows - 1) * sz + P) * 2));
            uint32_t zr[TP][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    zr[pt][r] = __builtin_amdgcn_raw_buffer_load_b16(
                        rz, (int)(2u * (uint32_t)((ibase + li) * sz + pt * 16 + 4 * lg + r)), 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= silu(__uint_as_float(zr[pt][r] << 16));
        }
    };

    // ---- the run of items (contiguous, heads of a chunk in a row, XCD-adjacent runs)
    const int nwg = gridDim.x;
    const int vw = (nwg & 7) == 0 ? (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int per = nitems / nwg, extra = nitems % nwg;
    int item = vw * per + min(vw, extra);
    const int last = item + per + (vw < extra ? 1 : 0);
    Item cur = decode(item);
    if (light) {
        stream(cur, true, hs0);
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wavefront's loads have landed
        convert(xs0, acs0, dts0, ech0);
    }
    load_tile_operands(cur);
    store_y(cur, false);  // empty range: the same youngest operations as every later item leaves
    __builtin_amdgcn_s_waitcnt(kWaitStores);
    __syncthreads();
    auto body = [&](auto parity) __attribute__((always_inline)) {
        constexpr bool ODD = decltype(parity)::value;
        const bool more = item + 1 < last;
        const Item nx = more ? decode(item + 1) : cur;
        if (light) stream(nx, more, ODD ? hs0 : hs1);
        compute(cur, ODD ? xs1 : xs0, ODD ? hs1 : hs0, ODD ? acs1 : acs0, ODD ? dts1 : dts0, ODD ? ech1 : ech0);
        if (light) {
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wavefront's loads of the next item have landed
            convert(ODD ? xs0 : xs1, ODD ? acs0 : acs1, ODD ? dts0 : dts1, ODD ? ech0 : ech1);
        }
        if (more && (nx.c != cur.c || nx.b != cur.b || nx.g != cur.g)) load_tile_operands(nx);
        store_y(cur, true);
        // everything but the y stores has completed: the next set is converted and the tile
        // operands are in; the barrier hands the set over and retires this one
        __builtin_amdgcn_s_waitcnt(kWaitStores);
        __syncthreads();
        if (more) {
            ++item;
            cur = nx;
        }
        return more;
    };
    for (;;) {
        if (!body(std::integral_constant<bool, false>{})) break;
        if (!body(std::integral_constant<bool, true>{})) break;
    }
}

template <typename TIn, int P>
static hipError_t launch_scan_n(const void *x, const void *Cm, const void *cbg, const float *acum,
                                const float *dtc, const void *hen, const float *D, void *y,
                                const SsdOpts &o, const Dims &d, int ncu, hipStream_t s)
{
    // persistent: enough workgroups for 16 wavefronts per compute unit, each looping over
    // its run of (b, c, h) items
    const int nitems = d.nc * d.H * d.B;
    const TIn *xx = static_cast<const TIn *>(x), *cc = static_cast<const TIn *>(Cm);
    // bf16, P = 64, N = 128, 256-token chunks: the pipelined kernel, one workgroup per CU
    if constexpr ((std::is_same<TIn, bf16_t>::value || std::is_same<TIn, fp8_t>::value) && P == 64) {
        if (d.N == 128 && d.Q == 256) {
            static_assert(PipeLds<64, 128, 16>::fits, "pipelined chunk scan LDS");
            const int nwg = nitems < ncu ? nitems : ncu;
#define SSD_PIPE_LAUNCH2(GT, YB, CP)                                                                         \
    launch_kernel("chunk_scan_pipe_kernel", chunk_scan_pipe_kernel<TIn, 64, 128, 16, GT, YB, CP>, nwg, 1024, s, xx, \
                  cc, cbg, acum, dtc, hen, D, y, o, d.L, d.H, d.G, d.sx, d.sbc, d.sz, d.Q, d.nc, nitems)
#define SSD_PIPE_LAUNCH(GT, YB)                  \
    do {                                         \
        if (o.stream_x)                          \
            SSD_PIPE_LAUNCH2(GT, YB, kStream);   \
        else                                     \
            SSD_PIPE_LAUNCH2(GT, YB, 0);         \
    } while (0)
            if (o.z && o.y_bf16)
                SSD_PIPE_LAUNCH(true, true);
            else if (o.z)
                SSD_PIPE_LAUNCH(true, false);
            else if (o.y_bf16)
                SSD_PIPE_LAUNCH(false, true);
            else
                SSD_PIPE_LAUNCH(false, false);
#undef SSD_PIPE_LAUNCH
#undef SSD_PIPE_LAUNCH2
            return hipGetLastError();
        }
    }
    // up to 16 wavefronts per compute unit, as many workgroups as the LDS holds
#define SSD_SCAN_LAUNCH(NN, NWV)                                                                          \
    do {                                                                                                  \
        const int fit = (160 * 1024) / ScanLds<TIn, P, NN, NWV>::bytes, per_cu = fit < 16 / NWV ? fit : 16 / NWV; \
        const int nwg = nitems < ncu * per_cu ? nitems : ncu * per_cu;                                   \
        if (o.z || o.y_bf16)                                                                              \
            launch_kernel("chunk_scan_kernel", chunk_scan_kernel<TIn, P, NN, NWV, true>, nwg, 64 * NWV, s, xx, \
                          cc, cbg, acum, dtc, hen, D, y, o, d.L, d.H, d.G, d.sx, d.sbc, d.sz, d.Q, d.nc,       \
                          nitems);                                                                             \
        else                                                                                              \
            launch_kernel("chunk_scan_kernel", chunk_scan_kernel<TIn, P, NN, NWV, false>, nwg, 64 * NWV, s,  \
                          xx, cc, cbg, acum, dtc, hen, D, y, o, d.L, d.H, d.G, d.sx, d.sbc, d.sz, d.Q, d.nc, \
                          nitems);                                                                           \
    } while (0)
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
    case 256: SSD_SCAN_BY_Q(256); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_SCAN_BY_Q
#undef SSD_SCAN_LAUNCH
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_scan_t(const void *x, const void *Cm, const void *cbg, const float *acum,
                                const float *dtc, const void *hen, const float *D, void *y,
                                const SsdOpts &o, const Dims &d, int ncu, hipStream_t s)
{
    switch (d.P) {
    case 32: return launch_scan_n<TIn, 32>(x, Cm, cbg, acum, dtc, hen, D, y, o, d, ncu, s);
    case 64: return launch_scan_n<TIn, 64>(x, Cm, cbg, acum, dtc, hen, D, y, o, d, ncu, s);
    case 128: return launch_scan_n<TIn, 128>(x, Cm, cbg, acum, dtc, hen, D, y, o, d, ncu, s);
    default: return hipErrorInvalidValue;
    }
}

// Compute units per device, looked up once per device (an immutable property; two threads
// that look it up at once store the same value).
static std::atomic<int> g_ncu[64];
hipError_t device_cu_count(int *ncu)
{
    int dev = 0;
    *ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) *ncu = g_ncu[dev].load(std::memory_order_relaxed);
    if (*ncu <= 0) {
        e = hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (*ncu <= 0) *ncu = 1;
        if (e == hipSuccess && dev >= 0 && dev < 64) g_ncu[dev].store(*ncu, std::memory_order_relaxed);
    }
    return e;
}

hipError_t launch_chunk_scan(const void *x, const void *Cm, const void *cb, const float *acum,
                             const float *dtc, const void *h_enter, const float *D, void *y,
                             const SsdOpts &o, const Dims &d, hipStream_t s)
{
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    if (chunk_scan_small_fits(d, ncu)) {
        SsdOpts po = o;
        po.sync = nullptr;  // entering states given
        return launch_chunk_scan_small(x, Cm, cb, acum, dtc, const_cast<void *>(h_enter), nullptr, nullptr, D, y, po,
                                       d, ncu, s);
    }
    if (d.in == kInFp8) return launch_scan_t<fp8_t>(x, Cm, cb, acum, dtc, h_enter, D, y, o, d, ncu, s);
    return d.in == kInBf16 ? launch_scan_t<bf16_t>(x, Cm, cb, acum, dtc, h_enter, D, y, o, d, ncu, s)
                           : launch_scan_t<float>(x, Cm, cb, acum, dtc, h_enter, D, y, o, d, ncu, s);
}

}  // namespace ssd
