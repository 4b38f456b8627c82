// ssd_chunk_scan_small.hip -- the chunk scan (Step-1 mask + GEMM2, Step-4 off-diagonal,
// skip term) for problems whose (b, h, chunk) items all fit the GPU at once.
//
// Same arithmetic as ssd_chunk_scan.hip ("Mamba-Family State-Space Model Kernels on a
// Programmable CGLA", Sec. III-A and IV-B: intra-chunk C.B^T masked by the segment decay
// times X, plus the off-diagonal C . H_enter and the skip term), organised for a different
// regime.  The persistent kernel keeps one 16-wavefront workgroup per compute unit and
// streams items through it; when there are fewer items than two per compute unit (a
// 4096-token 130M-shaped layer has 384), that leaves half the compute units with a second
// item after the first round.  Here each workgroup takes exactly one item with 8
// wavefronts, each forming two 16-row tiles in turn, so two workgroups fit per compute
// unit (LDS 60 KB, at most 128 VGPRs) and every item runs in the first round.
//
// Chunks of 256 tokens, bf16 inputs (fp16 matrix-core operands, fp32 accumulation),
// fp16 entering states.  Wavefront w forms tiles w and 15 - w: the two wavefronts of a
// SIMD (w and w + 4) then hold tiles {s, 15-s, s+4, 11-s}, 18 32-column steps per SIMD.
//
// With every item resident at once, the launch can also run Step-3 (same paper, Sec. IV-C:
// the entering state of chunk c+1 is that of chunk c decayed by the chunk's total decay
// plus the chunk's own state): the workgroups of one (b, h) split the P*N state elements
// between them, each walks the chunk recurrence for its share over all chunks, and each
// reads back its own chunk's entering state once all of them have counted themselves done.
// That replaces the separate state-passing launch (its read and write of every state, and
// a launch) with one extra read of the chunk's state per workgroup, taken after the first
// tile's steps, by which time the head's other workgroups are done.
#include <algorithm>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

// Cache-policy bit of buffer loads and stores: coherent across the whole device (the
// per-XCD L2 caches are not coherent with each other; such accesses go through to memory).
constexpr int kDeviceCoherent = 16;

// PNC = 0: hen holds the entering states [B, H, nc, P, N] (fp16).
// PNC > 0 (nc <= PNC): hen holds the chunk states; Step-3 runs inside this launch.  The
// workgroup of chunk c walks the chunk recurrence for its 1/nc share of the P*N state elements
// of its (b, h), writing every chunk's entering state over its chunk state (and the final
// state to fin), then counts itself done in sync[b, h] (zeroed by the chunk-state launch) and
// waits until all nc workgroups of the head are; all items are resident at once, so the wait
// ends.
// TX: storage of x and C (bf16, or fp8 e4m3; both widen to fp16 exactly).
template <typename TX, int P, int N, bool OPT, int PNC>
__global__ __launch_bounds__(512, 4) void chunk_scan_small_kernel(  // 4 waves per SIMD: <= 128 VGPRs
    const TX *__restrict__ x, const TX *__restrict__ Cm, const void *__restrict__ cbg,
    const float *__restrict__ acum, const float *__restrict__ dtc, f16 *hen, const float *init, float *fin,
    unsigned *sync, const float *__restrict__ D, void *__restrict__ y, SsdOpts opt, int L, int H, int G, int sx, int sbc,
    int sz, int nc,
    int nwhole)
{
    constexpr int Q = 256, ROWS = 256, NT = 512, NSMAX = 8;
    constexpr int TP = P / 16, KS = N / 32;
    constexpr int LDX = P + 16, LDH = N + 8, TAB = ROWS + 32;
    constexpr int SPC = 72;  // 32-column steps of a 256-token chunk (T(16))
    __shared__ f16 xs[ROWS * LDX];
    __shared__ f16 hs[P * LDH];
    __shared__ float acs[TAB], dts[TAB], ecs[TAB];
    // bf16 y (OPT only): each wavefront's 16-row output tile, regrouped so that the stores
    // write whole rows
    constexpr int YLD = P + 8;
    __shared__ __align__(16) uint16_t ybuf[OPT ? 8 * 16 * YLD : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    // Workgroups below nwhole take a whole item; the others take half an item each (half 0
    // and half 1), one 16-row tile per wavefront.  The first nwhole workgroups land one per
    // compute unit and the halves fill the second slots, so every compute unit gets the
    // same work when items are between one and two per compute unit.  The two halves of an
    // item are 8 workgroups apart: workgroups go to the XCDs in turn, so both land on the
    // same XCD and the second one's X and state reads hit that XCD's L2.
    const int wg = blockIdx.x, j = wg - nwhole;
    const int half = wg < nwhole ? -1 : (j >> 3) & 1;
    const int item = wg < nwhole ? wg : nwhole + ((j >> 4) << 3) + (j & 7);
    const int c = item % nc, h = (item / nc) % H, b = item / (nc * H), g = h / (H / G);
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const float Dh = D ? D[h] : 0.f;

    // ---- the first tile's GEMM1 slices (fp16, accumulator order), requested first: the
    // item's SPC slices (1 KB each) start at slice T(t) for tile t; slots past the tile's
    // steps read past the range (zeros), so every slot is loaded and the waits stay exact
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc(static_cast<const f16 *>(cbg) + (((size_t)b * G + g) * nc + c) * SPC * 512, SPC * 1024u);
    f16x8 gs[NSMAX];
    auto load_g = [&](int t) {
        const int ns = (16 * t + 15) / 32 + 1;
        const int Tt = (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);
#pragma unroll
        for (int s = 0; s < NSMAX; ++s) {
            const uint32_t off = (s < ns ? (uint32_t)(Tt + s) : (uint32_t)SPC) * 1024u + 16u * lane;
            gs[s] = __builtin_bit_cast(f16x8, buf_load16(rg, off));
        }
    };
    // whole item: tiles w and 15 - w; half 0: tiles {0, 3, 5, 6, 15, 12, 10, 9}, half 1:
    // {1, 2, 4, 7, 14, 13, 11, 8} by wavefront (36 steps per half, 9 per SIMD)
    auto tile_of = [&](int k) {
        return half < 0 ? (k == 0 ? wave : 15 - wave) : (int)(((half ? 0x8BDE7421u : 0x9ACF6530u) >> (4 * wave)) & 15u);
    };
    load_g(tile_of(0));

    // ---- Step-3 operands first (PNC > 0): word q = w0 + tid (two state elements) of each
    // chunk's state, the chunks' total decays and the initial state.  Every load is issued
    // unconditionally (slots past nc or past the share read past a buffer range: zeros), so
    // that the waits for them and for the loads issued after them stay exact.
    constexpr bool PASS = PNC > 0;
    constexpr int PN2 = P * N / 2;  // 32-bit words (two fp16 elements) of one state
    constexpr int PS = PASS ? PNC : 1;
    const size_t bh = (size_t)b * H + h;
    const int share = (PN2 + nc - 1) / nc, w0 = c * share;
    const int nw = half == 1 ? 0 : min(share, PN2 - w0);  // (half 1 of an item leaves Step-3 to half 0)
    __amdgpu_buffer_rsrc_t rp = make_rsrc(hen, 0u), ri = rp, rf = rp;
    uint32_t pv[PS], pi0 = 0u, pi1 = 0u;
    float pdec[PS];
    auto pass_load = [&](int q) {  // chunk states and initial state of word w0 + q
        const bool act = q < nw;
#pragma unroll
        for (int k = 0; k < PS; ++k) {
            const uint32_t off = (k < nc && act) ? 4u * (uint32_t)(k * PN2 + w0 + q) : 0x80000000u;
            pv[k] = __builtin_amdgcn_raw_buffer_load_b32(rp, (int)off, 0, 0);
        }
        const uint32_t oi = act ? 8u * (uint32_t)(w0 + q) : 0x80000000u;
        pi0 = __builtin_amdgcn_raw_buffer_load_b32(ri, (int)oi, 0, 0);
        pi1 = __builtin_amdgcn_raw_buffer_load_b32(ri, (int)(oi + 4u), 0, 0);
    };
    // The recurrence over the chunk slots (a slot past nc is the identity step), storing each
    // chunk's entering state (device-coherent) and the final state; q past the share stores
    // nothing (past the ranges).
    auto pass_run = [&](int q) {
        const bool act = q < nw;
        float r0 = __uint_as_float(pi0), r1 = __uint_as_float(pi1);
#pragma unroll
        for (int k = 0; k < PS; ++k) {
            const uint32_t off = (k < nc && act) ? 4u * (uint32_t)(k * PN2 + w0 + q) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b32(pack_f16x2(r0, r1), rp, (int)off, 0, kDeviceCoherent);
            const float r = k < nc ? exp_fast(pdec[k]) : 1.f;
            const f16x2 sv = __builtin_bit_cast(f16x2, pv[k]);
            r0 = fmaf(r, r0, static_cast<float>(sv[0]));
            r1 = fmaf(r, r1, static_cast<float>(sv[1]));
            // fp32 carry, converted by the next store (the standalone Step-3 kernel's
            // rounding): no multiply-add that rounds straight to fp16
            asm volatile("" : "+v"(r0), "+v"(r1));
        }
        const uint32_t of = act ? 8u * (uint32_t)(w0 + q) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r0), rf, (int)of, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r1), rf, (int)(of + 4u), 0, 0);
    };
    if constexpr (PASS) {
        rp = make_rsrc(hen + bh * nc * P * N, (uint32_t)(nc * PN2 * 4));
        ri = make_rsrc(init ? init + bh * P * N : nullptr, init ? (uint32_t)(PN2 * 8) : 0u);
        rf = make_rsrc(fin ? fin + bh * P * N : nullptr, fin ? (uint32_t)(PN2 * 8) : 0u);
        const float *ac = acum + bh * nc * Q + (Q - 1);
#pragma unroll
        for (int k = 0; k < PS; ++k) pdec[k] = ac[(size_t)min(k, nc - 1) * Q];
        pass_load(tid);
    }

    // ---- the item's X rows (fp16), entering state and decay tables into LDS
    {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + ((size_t)b * L + tc) * sx + (size_t)h * P,
                                                    (uint32_t)(((vrows - 1) * sx + P) * sizeof(TX)));
        constexpr int XU = ROWS * (P / 8), XPT = XU / NT;
        constexpr int HU = P * N / 8, HPT = (HU + NT - 1) / NT;
        Raw8<TX> px[XPT];
        uint4 ph[HPT];
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * NT;
            px[k].load(rx, (uint32_t)((u / (P / 8)) * sx + 8 * (u % (P / 8))));
        }
        const f16 *hp = hen + bhc * P * N;
        if constexpr (!PASS) {
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int u = tid + k * NT;
                if (HU % NT == 0 || u < HU) ph[k] = *reinterpret_cast<const uint4 *>(hp + 8 * u);
            }
        }
        // tables: dA_cum in log2 units, dt, and exp(a_r - a_j) dt_j with a_r the last column
        // of the 32-column step holding j
        float ta = 0.f, tr = 0.f, td = 0.f;
        const int ir = min(32 * (tid >> 5) + 31, Q - 1);
        if (tid < Q) {
            ta = acum[bhc * Q + tid];
            tr = acum[bhc * Q + ir];
            td = dtc[bhc * Q + tid];
        }
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * NT;
            *reinterpret_cast<uint4 *>(&xs[(u / (P / 8)) * LDX + 8 * (u % (P / 8))]) = raw8_to_f16x8(px[k]);
        }
        if constexpr (PASS) {
            // Step-3 for this workgroup's share: the first word per thread (loaded above),
            // then, when the share is longer than the workgroup, the rest in turn
            pass_run(tid);
            for (int q = tid + NT; q < share; q += NT) {
                pass_load(q);
                pass_run(q);
            }
        } else {
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int u = tid + k * NT;
                if (HU % NT == 0 || u < HU)
                    *reinterpret_cast<uint4 *>(&hs[(u / (N / 8)) * LDH + 8 * (u % (N / 8))]) = ph[k];
            }
        }
        if (tid < TAB) {
            float a = 0.f, d = 0.f, e = 0.f;
            if (tid < Q) {
                a = ta * kLog2e;
                d = td;
                e = __builtin_amdgcn_exp2f(tr * kLog2e - a) * d;
            }
            acs[tid] = a;
            dts[tid] = d;
            ecs[tid] = e;
        }
    }
    constexpr int HU = P * N / 8, HPT = (HU + NT - 1) / NT;  // uint4 words of the entering state
    uint4 hv[HPT];
    if constexpr (PASS) {
        // The entering-state stores are device-coherent (they write through the XCD's L2);
        // once every wavefront's stores have completed the workgroup counts itself done, and
        // the entering state is read back with device-coherent loads issued only after the
        // count reached nc.  (No L2 write-back or invalidation is needed: nothing else this
        // kernel exchanges between workgroups.)
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wavefront's stores are done
        __syncthreads();
        if (tid == 0 && half != 1)
            __hip_atomic_fetch_add(sync + ((size_t)b * H + h) * kSyncStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    } else {
        __syncthreads();
    }

    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + ((size_t)b * L + tc) * sbc + (size_t)g * N,
                                                (uint32_t)(((vrows - 1) * sbc + N) * sizeof(TX)));
    const size_t base_y = (((size_t)b * L + tc) * H + h) * P;
    const bool y16 = OPT && opt.y_bf16;
    const uint32_t es = y16 ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(
        y16 ? (void *)(static_cast<uint16_t *>(y) + base_y) : (void *)(static_cast<float *>(y) + base_y),
        (uint32_t)(((vrows - 1) * H * P + P) * es));

#pragma unroll 1
    for (int k = 0; k < (half < 0 ? 2 : 1); ++k) {
        const int t = tile_of(k);
        const int ibase = 16 * t;
        const int ns = (ibase + 15) / 32 + 1;  // 32-column steps up to the diagonal
        if (k > 0) load_g(t);

        f32x4 acc[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
        const int irow = ibase + li;
        const float ai = acs[irow];
        // GEMM2 of one step: k slots of lane group lg are columns {jb+4lg+r, jb+16+4lg+r}
        auto gemm2 = [&](int jb, const float r0[4], const float r1[4]) {
            f16x8 a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] = static_cast<f16>(r0[r]);
                a[4 + r] = static_cast<f16>(r1[r]);
            }
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                const int ox = tr16_offset(lane, jb, pt * 16, LDX);
                const f16x4 lo = lds_read_tr16(&xs[ox]);
                const f16x4 hi = lds_read_tr16(&xs[ox + 16 * LDX]);
                const f16x8 bx = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[pt] = mfma16x16x32_f16(a, bx, acc[pt]);
            }
        };
        // steps strictly below the diagonal: decay factored through the step's last column
#pragma unroll
        for (int s = 0; s + 1 < NSMAX; ++s) {
            if (s + 1 < ns) {
                const int jb = 32 * s;
                const float er = __builtin_amdgcn_exp2f(ai - acs[jb + 31]);
                const float4 e0 = *reinterpret_cast<const float4 *>(&ecs[jb + 4 * lg]);
                const float4 e1 = *reinterpret_cast<const float4 *>(&ecs[jb + 16 + 4 * lg]);
                const float ej0[4] = {e0.x, e0.y, e0.z, e0.w}, ej1[4] = {e1.x, e1.y, e1.z, e1.w};
                float r0[4], r1[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    r0[r] = static_cast<float>(gs[s][r]) * (er * ej0[r]);
                    r1[r] = static_cast<float>(gs[s][4 + r]) * (er * ej1[r]);
                }
                gemm2(jb, r0, r1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        {
            // the diagonal step: direct exponentials under the causal mask
            const int sd = ns - 1, jb = 32 * sd;
            const bool has1 = jb + 16 <= ibase + 15;
            f16x8 gd = gs[0];
#pragma unroll
            for (int s = 1; s < NSMAX; ++s)
                if (s == sd) gd = gs[s];
            const float4 a0v = *reinterpret_cast<const float4 *>(&acs[jb + 4 * lg]);
            const float4 t0v = *reinterpret_cast<const float4 *>(&dts[jb + 4 * lg]);
            const float4 a1v = *reinterpret_cast<const float4 *>(&acs[jb + 16 + 4 * lg]);
            const float4 t1v = *reinterpret_cast<const float4 *>(&dts[jb + 16 + 4 * lg]);
            const float aj0[4] = {a0v.x, a0v.y, a0v.z, a0v.w}, tj0[4] = {t0v.x, t0v.y, t0v.z, t0v.w};
            const float aj1[4] = {a1v.x, a1v.y, a1v.z, a1v.w}, tj1[4] = {t1v.x, t1v.y, t1v.z, t1v.w};
            float r0[4], r1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                r0[r] = (jb + 4 * lg + r <= irow) ? static_cast<float>(gd[r]) * __builtin_amdgcn_exp2f(ai - aj0[r]) * tj0[r]
                                                  : 0.f;
                r1[r] = (has1 && jb + 16 + 4 * lg + r <= irow)
                            ? static_cast<float>(gd[4 + r]) * __builtin_amdgcn_exp2f(ai - aj1[r]) * tj1[r]
                            : 0.f;
            }
            gemm2(jb, r0, r1);
        }
        if (PASS && k == 0) {
            // The entering state, once, before the first off-diagonal (the first tile's steps
            // gave the head's other workgroups time to count in): wait for all nc counts, read
            // it through to memory (written by other workgroups; words past the state read past
            // the range: zeros, not stored), and put it into LDS (rows p, padded).
            if (tid == 0) {
                // Bounded: past the bound the workgroup gives up, sets bit 31 of the head's
                // counter (which also releases the head's other waiters) and the prefill's
                // give-up word, and goes on; the output is then not valid.
                unsigned *cnt = sync + ((size_t)b * H + h) * kSyncStride;
                const unsigned polls = spin_polls(opt.spin);
                bool done = false;
                for (unsigned it = 0; it < polls; ++it) {
                    if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)nc) {
                        done = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(8);
                }
                if (!done) {
                    __hip_atomic_fetch_or(cnt, 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (opt.ctl) __hip_atomic_fetch_or(&opt.ctl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();
            const __amdgpu_buffer_rsrc_t rh = make_rsrc(hen + bhc * P * N, (uint32_t)(P * N * 2));
#pragma unroll
            for (int kk = 0; kk < HPT; ++kk)
                hv[kk] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)(16u * (tid + kk * NT)), 0, kDeviceCoherent));
#pragma unroll
            for (int kk = 0; kk < HPT; ++kk) {
                const int u = tid + kk * NT;  // uint4 index: elements 8u .. 8u + 7
                if (HU % NT == 0 || u < HU) *reinterpret_cast<uint4 *>(&hs[(u / (N / 8)) * LDH + 8 * (u % (N / 8))]) = hv[kk];
            }
            __syncthreads();
        }
        // ---- Step-4: exp(a_i) * (C_i . H_enter[p, :]), then the skip term (the C rows are
        // loaded only now, so that they do not hold registers through the steps)
        {
            bf16x8 cb[KS];
            const uint32_t row = (uint32_t)((ibase + li) * sbc);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (std::is_same<TX, fp8_t>::value) {  // e4m3: 8 bytes, in the low half
                    const uint2 v = buf_load8(rc, row + ks * 32 + 8 * lg);
                    cb[ks] = __builtin_bit_cast(bf16x8, make_uint4(v.x, v.y, 0u, 0u));
                } else {
                    cb[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
                }
            }
            f32x4 off[TP];
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) off[pt] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 ch = held_to_f16x8<TX>(cb[ks]);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                    off[pt] = mfma16x16x32_f16(ch, hf, off[pt]);
                }
                // keeps the scheduler from hoisting every LDS read of the loop (registers)
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(acs[ibase + 4 * lg + r]);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) acc[pt][r] += e * off[pt][r];
            }
        }
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
            // lane li receives X[ibase + 4 lg + r][16 pt + li], the accumulator positions
            const f16x4 xv = lds_read_tr16(&xs[tr16_offset(lane, ibase, pt * 16, LDX)]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * static_cast<float>(xv[r]);
        }
        // ---- optional output gate: y <- y * z * sigmoid(z), z laid out as x
        if (OPT && opt.z) {
            const bf16_t *zp = static_cast<const bf16_t *>(opt.z) + ((size_t)b * L + tc) * sz + (size_t)h * P;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(zp, (uint32_t)(((vrows - 1) * sz + P) * 2));
            uint32_t zr[TP][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    zr[pt][r] = __builtin_amdgcn_raw_buffer_load_b16(
                        rz, (int)(2u * (uint32_t)((ibase + 4 * lg + r) * sz + pt * 16 + li)), 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= silu(__uint_as_float(zr[pt][r] << 16));
        }
        // ---- y: buffer stores over the item's valid rows (rows past the sequence dropped);
        // bf16: whole rows through LDS (below).  The stores write
        // through the L2 (device scope): left dirty there, the whole y (25 MB at the 130M
        // shape, most of the L2s) is written back when the kernel ends, after the last
        // workgroup, where nothing overlaps it; streamed out as produced, the step is
        // ~1.4 us shorter.  (The persistent kernel streams many rounds of y through the L2,
        // whose write combining it needs: write-through there costs 10%.)
        if (OPT && y16) {
            // bf16: the tile goes through this wavefront's own LDS rows (LDS operations of one
            // wavefront complete in order, so no barrier), then every lane stores 16 bytes of
            // one row: eight lanes write a whole 128-byte row, a wavefront eight rows at once
            uint16_t *yb = ybuf + wave * (16 * YLD);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) yb[(4 * lg + r) * YLD + pt * 16 + li] = f32_to_bf16_rne(acc[pt][r]);
            // the 2-byte writes are read back as 16-byte words by other lanes: wait for them and
            // keep the compiler from moving the reads above them (they differ in type)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            constexpr int CH = P / 8;  // 16-byte pieces of a row
#pragma unroll
            for (int k = 0; k < 16 * CH / 64; ++k) {
                const int u = lane + 64 * k, row = u / CH, piece = u % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(&yb[row * YLD + 8 * piece]);
                const uint32_t e = (uint32_t)((ibase + row) * H * P + 8 * piece);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                                       ry, (int)(2u * e), 0, kDeviceCoherent);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const uint32_t e = (uint32_t)((ibase + 4 * lg + r) * H * P + pt * 16 + li);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[pt][r]), ry, (int)(es * e), 0, kDeviceCoherent);
                }
            }
        }
    }
}

// Whether the one-round kernel takes this problem: bf16 inputs, chunks of 256 tokens,
// supported P, and no more items than two per compute unit.
bool chunk_scan_small_shape(const Dims &d) { return d.half() && d.Q == 256 && d.P == 64 && d.N <= 128; }
bool chunk_scan_small_fits(const Dims &d, int ncu)
{
    return chunk_scan_small_shape(d) && (long)d.nc * d.H * d.B <= 2L * ncu;
}

// Whether the one-round kernel can also run Step-3 itself: at most 16 chunks per sequence
// (a thread keeps one state word of every chunk in registers).
bool chunk_scan_small_pass_shape(const Dims &d) { return chunk_scan_small_shape(d) && d.nc <= 16; }
bool chunk_scan_small_pass_fits(const Dims &d, int ncu) { return chunk_scan_small_pass_shape(d) && chunk_scan_small_fits(d, ncu); }

// Whether the one-round launch's workgroups can all be resident at once on this device: the
// occupancy the compiled instantiation allows (registers and LDS) times the compute units
// must cover the grid, since the workgroups of a head wait for each other.
hipError_t chunk_scan_small_resident(const Dims &d, const SsdOpts &o, int ncu, bool *ok)
{
    *ok = false;
    const long items = (long)d.nc * d.H * d.B;
    const long nsplit = (items > ncu && items <= 2L * ncu) ? std::min(items - ncu, 2L * ncu - items) / 8 * 8 : 0;
    const long wgs = items + nsplit;
    int per_cu = 0;
    hipError_t e = hipSuccess;
    const bool opt = o.z || o.y_bf16;
#define SSD_SMALL_OCC(NN, OO, PP) \
    e = d.in == kInFp8                                                                                    \
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk_scan_small_kernel<fp8_t, 64, NN, OO, PP>, \
                                                           512, 0)                                                 \
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk_scan_small_kernel<bf16_t, 64, NN, OO, PP>, \
                                                           512, 0)
#define SSD_SMALL_OCC2(NN, PP)              \
    do {                                    \
        if (opt) SSD_SMALL_OCC(NN, true, PP); \
        else SSD_SMALL_OCC(NN, false, PP);  \
    } while (0)
#define SSD_SMALL_OCC3(NN)                      \
    do {                                        \
        if (!o.sync) SSD_SMALL_OCC2(NN, 0);     \
        else if (d.nc <= 8) SSD_SMALL_OCC2(NN, 8); \
        else SSD_SMALL_OCC2(NN, 16);            \
    } while (0)
    switch (d.N) {
    case 32: SSD_SMALL_OCC3(32); break;
    case 64: SSD_SMALL_OCC3(64); break;
    case 128: SSD_SMALL_OCC3(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_SMALL_OCC3
#undef SSD_SMALL_OCC2
#undef SSD_SMALL_OCC
    if (e != hipSuccess) return e;
    *ok = (long)per_cu * ncu >= wgs;
    return hipSuccess;
}

hipError_t launch_chunk_scan_small(const void *x, const void *Cm, const void *cb, const float *acum,
                                   const float *dtc, void *h, const float *init, float *fin, const float *D,
                                   void *y, const SsdOpts &o, const Dims &d, int ncu, hipStream_t s)
{
    if (o.sync && d.nc > 16) return hipErrorInvalidValue;
    const int items = d.nc * d.H * d.B;
    // Between one and two items per compute unit: split items past the first ncu in two (in
    // groups of 8, see the kernel), as many as keep the grid within two per compute unit
    // (the Step-3 wait needs every workgroup resident).
    const int nsplit = (items > ncu && items <= 2 * ncu) ? min(items - ncu, 2 * ncu - items) / 8 * 8 : 0;
    const int nwhole = items - nsplit;
    const unsigned nitems = (unsigned)(nwhole + 2 * nsplit);  // workgroups
    f16 *hh = static_cast<f16 *>(h);
#define SSD_SMALL_LAUNCH3(NN, OO, PP)                                                                            \
    do {                                                                                                         \
        if (d.in == kInFp8)                                                                                      \
            launch_kernel("chunk_scan_small_kernel", chunk_scan_small_kernel<fp8_t, 64, NN, OO, PP>, nitems, 512, \
                          s, static_cast<const fp8_t *>(x), static_cast<const fp8_t *>(Cm), cb, acum, dtc, hh,   \
                          init, fin, o.sync, D, y, o, d.L, d.H, d.G, d.sx, d.sbc, d.sz, d.nc, nwhole);           \
        else                                                                                                     \
            launch_kernel("chunk_scan_small_kernel", chunk_scan_small_kernel<bf16_t, 64, NN, OO, PP>, nitems,     \
                          512, s, static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(Cm), cb, acum, dtc, \
                          hh, init, fin, o.sync, D, y, o, d.L, d.H, d.G, d.sx, d.sbc, d.sz, d.nc, nwhole);       \
    } while (0)
#define SSD_SMALL_LAUNCH2(NN, PP)                                                                            \
    do {                                                                                                     \
        if (o.z || o.y_bf16) SSD_SMALL_LAUNCH3(NN, true, PP);                                                \
        else SSD_SMALL_LAUNCH3(NN, false, PP);                                                               \
    } while (0)
#define SSD_SMALL_LAUNCH(NN)                                                                                 \
    do {                                                                                                     \
        if (!o.sync) SSD_SMALL_LAUNCH2(NN, 0);                                                               \
        else if (d.nc <= 8) SSD_SMALL_LAUNCH2(NN, 8);                                                        \
        else SSD_SMALL_LAUNCH2(NN, 16);                                                                      \
    } while (0)
    switch (d.N) {
    case 32: SSD_SMALL_LAUNCH(32); break;
    case 64: SSD_SMALL_LAUNCH(64); break;
    case 128: SSD_SMALL_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_SMALL_LAUNCH
#undef SSD_SMALL_LAUNCH2
#undef SSD_SMALL_LAUNCH3
    return hipGetLastError();
}

}  // namespace ssd
