// ssd_prefill_fused.hip -- single-pass chunked prefill for grids of many rounds: every
// (b, h, chunk) item forms its chunk state, receives the state entering its chunk from the
// items before it, and writes its chunk's output, so that neither the chunk states nor the
// entering states make a round trip through HBM and x is read once.
//
// Method ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A,
// IV-B, IV-C; "Mambalaya: Einsum-Based Fusion Optimizations on State-Space Models", Fig. 2
// and the abstract: fusing the cascade removes the inter-Einsum traffic).  For chunk c of
// head h, with a = the chunk's inclusive cumulative sum of dt*A, w_j = exp(a_end - a_j) dt_j
// and d_c = exp(a_end):
//   Step-0   a, w, d_c                                   (wavefront prefix scan)
//   Step-2   S_c = sum_j w_j x_j B_j^T                    (fp16 matrix cores, fp32 accumulation)
//   Step-3   H_enter[c+1] = d_c H_enter[c] + S_c,  H_enter[0] = the initial state
//   Step-1   y_i  = sum_{j<=i} (C_i . B_j) exp(a_i - a_j) dt_j x_j   (mask + GEMM2)
//   Step-4        + H_enter[c] (exp(a_i) C_i) + D_h x_i
//
// Step-3 is a chain through the chunks of each (b, h).  A plain chain hands every entering
// state from one workgroup to the next (~2 us per hand-off through device-coherent memory on
// MI355X, 64 hand-offs for a 16384-token sequence of 256-token chunks), so the chain is
// shortened by a fixed look-back of DEPTH chunks: as soon as item c has formed S_c it
// publishes it (its "aggregate", with d_c); once it can, it forms
//   H_enter[c] = fold of I_{c-DEPTH} (the entering state of chunk c-DEPTH+1, published by
//                item c-DEPTH) through the aggregates of chunks c-DEPTH+1 .. c-1,
// publishes I_c = H_enter[c+1] = d_c H_enter[c] + S_c, and goes on to its output.  I_c then
// depends on I_{c-DEPTH} only: DEPTH interleaved chains of nc/DEPTH hand-offs each.
//
// Items are handed out by an atomic ticket in chunk-major order (all heads of chunk 0, then
// chunk 1, ...), and an item waits only for items of earlier chunks, i.e. smaller tickets:
// those workgroups are already running, so the waits end however the grid is scheduled (no
// co-residency is assumed).  Every wait is bounded; a wait that gives up sets a sticky word
// in the workspace (ssd_prefill_check reports it) and the item goes on, so the launch always
// drains.
//
// Exchange memory: per (b, h), 2*DEPTH ring slots of aggregates and 2*DEPTH ring slots of
// inclusive states (fp32, in the accumulator lane layout), and one status word per slot
// holding the chunk index + 1 of its content.  Aggregate slot k % R is rewritten by item
// k + R only after the items that read it (k .. k + DEPTH - 1) have published their own
// inclusive states; inclusive slot k % R is read only by item k + DEPTH, and item k + R
// publishes only after I_{k + R - DEPTH}, which (R a multiple of DEPTH) follows I_{k+DEPTH}.
// All exchange loads and stores are device-coherent (the eight XCD L2 caches are not
// coherent with each other): a store with the device-scope cache policy writes through to
// memory, the producer waits for its stores to complete (s_waitcnt vmcnt(0)) and meets its
// workgroup at a barrier before one thread stores the status word with the same policy; a
// consumer polls the status word and then loads the slot with device-scope loads, which do
// not hit stale lines in its own L2.
//
// Shape: bf16 inputs, Q = 256, P = 64, N in {64, 128}; one item per 8-wavefront
// workgroup (<= 80 KB of LDS, <= 128 VGPRs: two workgroups per compute unit).
#include "ssd_common.h"
#include "ssd_gemm1_body.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kDev = 16;  // cache policy of the exchange: coherent across the whole device

// Status word reads and writes (device scope).
__device__ __forceinline__ unsigned flag_load(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(unsigned *p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wavefront waits for several status words at once: each lane with `act` polls its own
// word until it reads >= want, all of them at most `polls` times (polls = 0: give up at
// once).  Returns (wave-uniform) whether any lane gave up.
__device__ __forceinline__ bool wave_wait(bool act, const unsigned *p, unsigned want, unsigned polls)
{
    bool done = !act;
    for (unsigned it = 0; it < polls; ++it) {
        if (!done) done = flag_load(p) >= want;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        __builtin_amdgcn_s_sleep(2);
    }
    return __builtin_amdgcn_ballot_w64(!done) != 0;
}

}  // namespace

// Workspace of the fused prefill (byte offsets from its base, each 256-byte aligned).
//   ctl    64 uint32: [0] the ticket counter, [1] the give-up word
//   flags  [B*H][64] uint32 per (b, h): aggregate status [0, R), inclusive status [16, 16+R),
//          the aggregates' chunk decays d_k (fp32) [32, 32+R)
//   ring   [B*H][2R][P*N] fp32: aggregate slots, then inclusive slots
//   cb     the GEMM1 products (fp16), as the chunk-state launch writes them
struct FusedWs {
    size_t ctl, flags, ring, cb, total;
};
static FusedWs fused_ws(const Dims &d)
{
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t bh = (size_t)d.B * d.H;
    FusedWs w;
    w.ctl = 0;
    w.flags = 256;
    w.ring = up(w.flags + bh * 64 * 4);
    w.cb = up(w.ring + bh * (size_t)(2 * kFusedRing) * d.P * d.N * 4);
    w.total = up(w.cb + (size_t)d.B * d.G * d.nc * gemm1_steps_per_chunk(d.Q) * 512 * 2);
    return w;
}
size_t fused_prefill_ws_bytes(const Dims &d) { return fused_ws(d).total; }
bool fused_prefill_shape(const Dims &d)
{
    return d.in == kInBf16 && d.Q == 256 && d.P == 64 && (d.N == 64 || d.N == 128) && d.nc >= 1 &&
           (long long)d.B * d.H * d.nc < 0x7fffffffLL;  // one workgroup (and ticket) per item
}

// First launch of the fused prefill: the GEMM1 products (four workgroups per chunk, as in the
// chunk-state launch), and workgroup (0, 0, 0) clears the ticket, the give-up word and every
// status word.
template <int N>
__global__ __launch_bounds__(256) void fused_prep_kernel(const bf16_t *__restrict__ Bm, const bf16_t *__restrict__ Cm,
                                                         void *__restrict__ cb, unsigned *ctl, unsigned *flags,
                                                         int nflags, int L, int G, int sbc, int nc)
{
    typedef Gemm1Chunk<bf16_t, N, 4, 256> G1;
    __shared__ __align__(16) unsigned char smem[G1::kLdsBytes];
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
        if (threadIdx.x < 64) ctl[threadIdx.x] = 0u;
        for (int i = threadIdx.x; i < nflags; i += 256) flags[i] = 0u;
    }
    G1::run(Bm, Cm, cb, L, G, sbc, 256, nc, blockIdx.x, blockIdx.y >> 2, blockIdx.z, smem, blockIdx.y & 3);
}

template <int N, bool OPT, int DEPTH>
__global__ __launch_bounds__(512, 4) void chunk_fused_kernel(  // 4 waves per SIMD: <= 128 VGPRs
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Bm, const bf16_t *__restrict__ Cm,
    const bf16_t *__restrict__ dt, const float *__restrict__ A, const float *__restrict__ D,
    const float *__restrict__ init, float *__restrict__ fin, const void *__restrict__ cbg, void *__restrict__ y,
    unsigned *ctl, unsigned *flags, float *ring, SsdOpts opt, int L, int H, int G, int BH, int sx, int sbc, int sdt,
    int sz, int nc)
{
    const unsigned spin_limit = spin_polls(opt.spin);
    constexpr int P = 64, Q = 256, JB = 64, NBLK = Q / JB, NSMAX = 8, SPC = 72;
    constexpr int R = kFusedRing;                    // ring slots per (b, h), each kind
    static_assert(R % DEPTH == 0 && R >= 2 * DEPTH && R <= 16, "ring");
    constexpr int TP = P / 16, KS = N / 32, NTN = N / 16;
    constexpr int TPW = NTN / 2;                     // chunk-state tiles per wavefront (of 4 * NTN)
    constexpr int LDX = P + 16, LDB = N + 16, LDH = N + 8;
    constexpr int BSZ = JB * LDB;                    // one B block, fp16
    constexpr int USZ = 2 * BSZ > P * LDH ? 2 * BSZ : P * LDH;
    constexpr int BU = JB * (N / 8), BPT = BU / 512;  // 16-byte units of a B block per thread
    constexpr int XPT = Q * (P / 8) / 512;           // 16-byte units of X per thread (4)
    constexpr int PN = P * N;
    static_assert(BU % 512 == 0 && TPW >= 1, "shape");
    __shared__ f16 xs[Q * LDX];          // the chunk's X rows (fp16)
    __shared__ f16 un[USZ];              // B blocks during Step-2, then the entering state (fp16)
    __shared__ float acs[Q], dts[Q], ecs[Q];  // a (log2 units), dt, and w_j then exp(a_r - a_j) dt_j
    __shared__ unsigned bc[4 + DEPTH];   // ticket; the aggregates' decays of the fold

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;

    // ---- the item: ticket t, chunk-major
    if (tid == 0) bc[0] = __hip_atomic_fetch_add(ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const unsigned t = bc[0];
    const int c = (int)(t / (unsigned)BH), bh = (int)(t % (unsigned)BH);
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const long tc = (long)c * Q;
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    unsigned *fl = flags + (size_t)bh * 64;
    float *ra = ring + (size_t)bh * (2 * R) * PN;  // aggregate slots; inclusive slots at + R * PN
    bool gave_up = false;

    // ---- prologue loads: dt (wavefront 0), every X and B row of the chunk
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + ((size_t)b * L + tc) * sx + (size_t)h * P,
                                                (uint32_t)(((vrows - 1) * sx + P) * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bm + ((size_t)b * L + tc) * sbc + (size_t)g * N,
                                                (uint32_t)(((vrows - 1) * sbc + N) * 2));
    const float dbias = opt.dt_bias ? opt.dt_bias[h] : 0.f;
    unsigned short dtraw[4];
    if (wave == 0) {
        const __amdgpu_buffer_rsrc_t rd =
            make_rsrc(dt + ((size_t)b * L + tc) * sdt + h, (uint32_t)(((vrows - 1) * sdt + 1) * 2));
#pragma unroll
        for (int k = 0; k < 4; ++k)
            dtraw[k] = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)((lane * 4 + k) * sdt * 2), 0, 0);
    }
    Raw8<bf16_t> px[XPT], pb[NBLK][BPT];
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
        const int u = tid + 512 * k;
        px[k].load(rx, (uint32_t)((u / (P / 8)) * sx + 8 * (u % (P / 8))));
    }
#pragma unroll
    for (int m = 0; m < NBLK; ++m)
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + 512 * k;
            pb[m][k].load(rb, (uint32_t)((JB * m + u / (N / 8)) * sbc + 8 * (u % (N / 8))));
        }

    // ---- Step-0 (wavefront 0): inclusive scan of dt*A over the chunk, four tokens per lane
    // serially, then across the lanes
    float dchunk = 0.f;  // d_c, valid in wavefront 0 (broadcast below)
    if (wave == 0) {
        const float Ah = A[h];
        float part[4], dv[4], run = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = lane * 4 + k;
            unsigned short raw = dtraw[k];
            asm volatile("" : "+v"(raw));  // first use after the block loads are issued
            float dd = 0.f;
            if (tc + i < L) dd = dt_effective_b(__uint_as_float((uint32_t)raw << 16), dbias, opt.dt_softplus);
            dv[k] = dd;
            run += dd * Ah;
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
        const float aend = __shfl(incl, 63, 64);
        dchunk = exp_fast(aend);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = lane * 4 + k;
            const float ac = excl + part[k];
            acs[i] = ac * kLog2e;
            dts[i] = dv[k];
            ecs[i] = exp_fast(aend - ac) * dv[k];  // w_i, the chunk-state weight
        }
        if (lane == 0) bc[1] = __float_as_uint(dchunk);
    }
    // X rows to LDS (fp16, exact for bf16 values in the fp16 range)
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
        const int u = tid + 512 * k;
        *reinterpret_cast<uint4 *>(&xs[(u / (P / 8)) * LDX + 8 * (u % (P / 8))]) = raw8_to_f16x8(px[k]);
    }
    __syncthreads();
    dchunk = __uint_as_float(bc[1]);

    // ---- Step-2: S_c^T = (w . B)^T X through LDS blocks of 64 tokens.  Wavefront w takes the
    // state-column tile w % NTN crossed with TPW channel tiles; lane (li, lg) of tile (nt, pt)
    // holds S[p = 16 pt + li][n = 16 nt + 4 lg + r], r = 0..3.
    f16 *bs0 = un, *bs1 = un + BSZ;
    auto commit = [&](int m, f16 *bsb) {
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + 512 * k, j = u / (N / 8), ng = u % (N / 8);
            *reinterpret_cast<uint4 *>(&bsb[j * LDB + 8 * ng]) = raw8_to_f16x8(pb[m][k], ecs[JB * m + j]);
        }
    };
    const int snt = wave % NTN, spt0 = (wave / NTN) * TPW;
    f32x4 sacc[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) sacc[q] = zero4();
    auto contract = [&](int m, const f16 *bsb) {
#pragma unroll
        for (int ks = 0; ks < JB; ks += 32) {
            const int ob = tr16_offset(lane, ks, snt * 16, LDB);
            const f16x4 b0 = lds_read_tr16(&bsb[ob]);
            const f16x4 b1 = lds_read_tr16(&bsb[ob + 16 * LDB]);
            const f16x8 bo = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int q = 0; q < TPW; ++q) {
                const int ox = tr16_offset(lane, JB * m + ks, (spt0 + q) * 16, LDX);
                const f16x4 a0 = lds_read_tr16(&xs[ox]);
                const f16x4 a1 = lds_read_tr16(&xs[ox + 16 * LDX]);
                const f16x8 xo = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                sacc[q] = mfma16x16x32_f16(bo, xo, sacc[q]);
            }
        }
    };
    commit(0, bs0);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NBLK; ++m) {
        contract(m, (m & 1) ? bs1 : bs0);
        if (m + 1 < NBLK) {
            commit(m + 1, ((m + 1) & 1) ? bs1 : bs0);
            __syncthreads();
        }
    }

    // ---- the first tile's GEMM1 slices (fp16, accumulator order), requested now: slots past
    // the tile's steps read past the range (zeros), so every slot is loaded
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc(static_cast<const f16 *>(cbg) + (((size_t)b * G + g) * nc + c) * SPC * 512, SPC * 1024u);
    f16x8 gs[NSMAX];
    auto load_g = [&](int tt) {
        const int ns = (16 * tt + 15) / 32 + 1;
        const int Tt = (tt & 1) ? ((tt >> 1) + 1) * ((tt >> 1) + 1) : (tt >> 1) * ((tt >> 1) + 1);
#pragma unroll
        for (int s = 0; s < NSMAX; ++s) {
            const uint32_t off = (s < ns ? (uint32_t)(Tt + s) : (uint32_t)SPC) * 1024u + 16u * lane;
            gs[s] = __builtin_bit_cast(f16x8, buf_load16(rg, off));
        }
    };
    load_g(wave);

    // ---- publish the aggregate (S_c, d_c) unless this is the last chunk; its slot is free
    // once the items that read the previous content (chunks c-R .. c-R+DEPTH-1) have
    // published their inclusive states (long before, with R >= 2 DEPTH).  The stores are
    // issued now and complete while tile 0's GEMM2 runs; the status word follows after it.
    const bool publish_agg = c + 1 < nc;
    if (wave == 0) {
        const int k = c - R + lane;
        const bool act = publish_agg && lane < DEPTH && k >= 0;
        if (wave_wait(act, &fl[16 + (act ? k % R : 0)], (unsigned)k + 1u, spin_limit)) gave_up = true;
    }
    __syncthreads();  // (also: every Step-2 read of the B blocks and the weights is done)
    if (publish_agg) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(ra + (size_t)(c % R) * PN, (uint32_t)(PN * 4));
#pragma unroll
        for (int q = 0; q < TPW; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, sacc[q]),
                                                   rs, (int)(16u * (uint32_t)((wave * TPW + q) * 64 + lane)), 0, kDev);
        if (tid == 0) __hip_atomic_store(&fl[32 + c % R], __float_as_uint(dchunk), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the GEMM2 decay table, exp(a_r - a_j) dt_j with a_r the last column of j's 32-column step
    if (tid < Q) {
        const int ir = 32 * (tid >> 5) + 31;
        ecs[tid] = __builtin_amdgcn_exp2f(acs[ir] - acs[tid]) * dts[tid];
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + ((size_t)b * L + tc) * sbc + (size_t)g * N,
                                                (uint32_t)(((vrows - 1) * sbc + N) * 2));
    const size_t base_y = (((size_t)b * L + tc) * H + h) * P;
    const bool y16 = OPT && opt.y_bf16;
    const uint32_t es = y16 ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(
        y16 ? (void *)(static_cast<uint16_t *>(y) + base_y) : (void *)(static_cast<float *>(y) + base_y),
        (uint32_t)(((vrows - 1) * H * P + P) * es));
    const float Dh = D ? D[h] : 0.f;
    f16 *hs = un;

#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int tt = k == 0 ? wave : 15 - wave;
        const int ibase = 16 * tt;
        const int ns = (ibase + 15) / 32 + 1;

        f32x4 acc[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt] = zero4();
        const int irow = ibase + li;
        const float ai = acs[irow];
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
        // ---- Step-1 steps strictly below the diagonal: decay factored through the step's
        // last column
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

        if (k == 0) {
            // ---- Step-3: the state entering this chunk, and the one leaving it.  First the
            // aggregate's status word (its stores, issued before the GEMM2, are done by now).
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wavefront's aggregate stores are done
            __syncthreads();
            if (tid == 0 && publish_agg) flag_store(&fl[c % R], (unsigned)c + 1u);
            const int k0 = c - DEPTH;  // the inclusive state the fold starts from (< 0: the initial state)
            if (wave == 0) {
                // lane 0: I_{k0}; lanes 1 .. DEPTH-1: the aggregates of chunks k0+1 .. c-1
                const int kk = k0 + lane;
                const bool act = lane < DEPTH && kk >= 0;
                const unsigned *w = act ? &fl[(lane == 0 ? 16 : 0) + kk % R] : fl;
                if (wave_wait(act, w, (unsigned)kk + 1u, spin_limit)) gave_up = true;
                if (lane > 0 && act) bc[4 + lane - 1] = flag_load(&fl[32 + kk % R]);
            }
            __syncthreads();
            // every load of the fold is issued before the first is used: the start, I_{k0}
            // (device-coherent) or the initial state (or zeros), then the aggregates of chunks
            // k0+1 .. c-1 (slots of chunks before 0 read an empty range)
            f32x4 hv[TPW], av[DEPTH > 1 ? DEPTH - 1 : 1][TPW];
            {
                const int lo = (wave * TPW) * 64 + lane;  // float4 index of this lane's first tile
                if (k0 >= 0) {
                    const __amdgpu_buffer_rsrc_t ri = make_rsrc(ra + (size_t)(R + k0 % R) * PN, (uint32_t)(PN * 4));
#pragma unroll
                    for (int q = 0; q < TPW; ++q)
                        hv[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (int)(16u * (uint32_t)(lo + 64 * q)), 0, kDev));
                } else {
                    const __amdgpu_buffer_rsrc_t ri =
                        make_rsrc(init ? init + (size_t)bh * PN : nullptr, init ? (uint32_t)(PN * 4) : 0u);
#pragma unroll
                    for (int q = 0; q < TPW; ++q) {
                        const int p = 16 * (spt0 + q) + li, n = 16 * snt + 4 * lg;
                        hv[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (int)(4u * (uint32_t)(p * N + n)), 0, 0));
                    }
                }
#pragma unroll
                for (int i = 0; i + 1 < DEPTH; ++i) {
                    const int kk = k0 + 1 + i;
                    const __amdgpu_buffer_rsrc_t rs =
                        make_rsrc(ra + (size_t)((kk >= 0 ? kk : 0) % R) * PN, kk >= 0 ? (uint32_t)(PN * 4) : 0u);
#pragma unroll
                    for (int q = 0; q < TPW; ++q)
                        av[i][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(16u * (uint32_t)(lo + 64 * q)), 0, kDev));
                }
                // H <- d_k H + S_k over the aggregates, in chunk order
#pragma unroll
                for (int i = 0; i + 1 < DEPTH; ++i) {
                    if (k0 + 1 + i < 0) continue;
                    const float dk = __uint_as_float(bc[4 + i]);
#pragma unroll
                    for (int q = 0; q < TPW; ++q)
#pragma unroll
                        for (int r = 0; r < 4; ++r) hv[q][r] = fmaf(dk, hv[q][r], av[i][q][r]);
                }
            }
            // the entering state as the off-diagonal operand (fp16, rows p, padded)
#pragma unroll
            for (int q = 0; q < TPW; ++q) {
                const int p = 16 * (spt0 + q) + li, n = 16 * snt + 4 * lg;
                uint2 w;
                w.x = pack_f16x2(hv[q][0], hv[q][1]);
                w.y = pack_f16x2(hv[q][2], hv[q][3]);
                *reinterpret_cast<uint2 *>(&hs[p * LDH + n]) = w;
            }
            // I_c = d_c H_enter[c] + S_c: to the ring, or (last chunk) to the final state
            if (c + 1 < nc) {
                const __amdgpu_buffer_rsrc_t ri = make_rsrc(ra + (size_t)(R + c % R) * PN, (uint32_t)(PN * 4));
#pragma unroll
                for (int q = 0; q < TPW; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = fmaf(dchunk, hv[q][r], sacc[q][r]);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                                           ri, (int)(16u * (uint32_t)((wave * TPW + q) * 64 + lane)), 0, kDev);
                }
            } else {
                const __amdgpu_buffer_rsrc_t rf = make_rsrc(fin ? fin + (size_t)bh * PN : nullptr, fin ? (uint32_t)(PN * 4) : 0u);
#pragma unroll
                for (int q = 0; q < TPW; ++q) {
                    const int p = 16 * (spt0 + q) + li, n = 16 * snt + 4 * lg;
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = fmaf(dchunk, hv[q][r], sacc[q][r]);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                                           rf, (int)(4u * (uint32_t)(p * N + n)), 0, 0);
                }
            }
            // tile 1's GEMM1 slices, requested now (the fold's registers are free): they arrive
            // while the inclusive state is published and tile 0's off-diagonal runs.  The wait
            // leaves exactly those 8 younger loads in flight and retires the state's stores.
            load_g(15 - wave);
            __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): the inclusive-state stores are done
            __syncthreads();                     // (also: the entering state is in LDS)
            if (tid == 0) {
                if (c + 1 < nc) flag_store(&fl[16 + c % R], (unsigned)c + 1u);
                if (gave_up) __hip_atomic_fetch_or(&ctl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }

        // ---- Step-4: (exp(a_i) C_i) . H_enter[p, :] accumulated into the output: the row
        // scale is applied to the C operand (rows i = ibase + li of the A operand scale rows i
        // of the product) before its one rounding to fp16, then the skip term
        {
            bf16x8 cv[KS];
            const uint32_t row = (uint32_t)((ibase + li) * sbc);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cv[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
            const float ei = __builtin_amdgcn_exp2f(acs[ibase + li]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 u = __builtin_bit_cast(uint4, cv[ks]);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
                f16x8 ch;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    ch[2 * q] = static_cast<f16>(__uint_as_float(w[q] << 16) * ei);
                    ch[2 * q + 1] = static_cast<f16>(__uint_as_float(w[q] & 0xFFFF0000u) * ei);
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const f16x8 hf = *reinterpret_cast<const f16x8 *>(&hs[(pt * 16 + li) * LDH + ks * 32 + 8 * lg]);
                    acc[pt] = mfma16x16x32_f16(ch, hf, acc[pt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
            const f16x4 xv = lds_read_tr16(&xs[tr16_offset(lane, ibase, pt * 16, LDX)]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] += Dh * static_cast<float>(xv[r]);
        }
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
        // ---- y over the item's valid rows (rows past the sequence dropped by the range);
        // bf16: the even lane of each pair of columns stores both values
        const bool drop = y16 && (li & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                const float v = acc[pt][r];
                uint32_t data = __float_as_uint(v);
                if constexpr (OPT) data = y16 ? pack_bf16x2(v, swap_adjacent_lanes(v)) : data;
                const uint32_t e = (uint32_t)((ibase + 4 * lg + r) * H * P + pt * 16 + li);
                __builtin_amdgcn_raw_buffer_store_b32(data, ry, (int)(drop ? 0x7ffffff0u : es * e), 0, 0);
            }
        }
    }
}

hipError_t launch_prefill_fused(const void *x, const void *Bm, const void *Cm, const void *dt, const float *A,
                                const float *D, const float *init, float *fin, void *y, void *ws, const SsdOpts &o,
                                const Dims &d, hipStream_t s)
{
    if (!fused_prefill_shape(d)) return hipErrorInvalidValue;
    const FusedWs w = fused_ws(d);
    char *base = static_cast<char *>(ws);
    unsigned *ctl = reinterpret_cast<unsigned *>(base + w.ctl);
    unsigned *flags = reinterpret_cast<unsigned *>(base + w.flags);
    float *ring = reinterpret_cast<float *>(base + w.ring);
    void *cb = base + w.cb;
    const bf16_t *xx = static_cast<const bf16_t *>(x), *bb = static_cast<const bf16_t *>(Bm),
                 *cc = static_cast<const bf16_t *>(Cm), *dd = static_cast<const bf16_t *>(dt);
    const int BH = d.B * d.H;
    const dim3 pgrid(d.nc, 4 * d.G, d.B);
    const unsigned items = (unsigned)BH * (unsigned)d.nc;
#define SSD_FUSED_LAUNCH(NN, OO)                                                                                   \
    do {                                                                                                           \
        launch_kernel("fused_prep_kernel", fused_prep_kernel<NN>, pgrid, 256, s, bb, cc, cb, ctl, flags, \
                      BH * 64, d.L, d.G, d.sbc, d.nc);                                                   \
        launch_kernel("chunk_fused_kernel", chunk_fused_kernel<NN, OO, kFusedDepth>, items, 512, s, xx, bb, \
                      cc, dd, A, D, init, fin, cb, y, ctl, flags, ring, o, d.L, d.H, d.G, BH, d.sx, d.sbc,  \
                      d.sdt, d.sz, d.nc);                                                                   \
    } while (0)
#define SSD_FUSED_LAUNCH2(NN)                                      \
    do {                                                           \
        if (o.z || o.y_bf16) SSD_FUSED_LAUNCH(NN, true);           \
        else SSD_FUSED_LAUNCH(NN, false);                          \
    } while (0)
    switch (d.N) {
    case 64: SSD_FUSED_LAUNCH2(64); break;
    case 128: SSD_FUSED_LAUNCH2(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_FUSED_LAUNCH2
#undef SSD_FUSED_LAUNCH
    return hipGetLastError();
}

}  // namespace ssd
