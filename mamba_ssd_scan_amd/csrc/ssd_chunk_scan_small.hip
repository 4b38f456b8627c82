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
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

template <int P, int N, bool OPT>
__global__ __launch_bounds__(512, 4) void chunk_scan_small_kernel(  // 4 waves per SIMD: <= 128 VGPRs
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ Cm, const void *__restrict__ cbg,
    const float *__restrict__ acum, const float *__restrict__ dtc, const f16 *__restrict__ hen,
    const float *__restrict__ D, void *__restrict__ y, SsdOpts opt, int L, int H, int G, int nc)
{
    constexpr int Q = 256, ROWS = 256, NT = 512, NSMAX = 8;
    constexpr int TP = P / 16, KS = N / 32;
    constexpr int LDX = P + 16, LDH = N + 8, TAB = ROWS + 32;
    constexpr int SPC = 72;  // 32-column steps of a 256-token chunk (T(16))
    __shared__ f16 xs[ROWS * LDX];
    __shared__ f16 hs[P * LDH];
    __shared__ float acs[TAB], dts[TAB], ecs[TAB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int item = blockIdx.x;
    const int c = item % nc, h = (item / nc) % H, b = item / (nc * H), g = h / (H / G);
    const size_t bhc = ((size_t)b * H + h) * nc + c;
    const long tc = (long)c * Q;
    const int vrows = (int)((L - tc) < Q ? (L - tc) : Q);
    const float Dh = D ? D[h] : 0.f;

    // ---- the item's X rows (fp16), entering state and decay tables into LDS
    {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + ((size_t)b * L + tc) * H * P + (size_t)h * P,
                                                    (uint32_t)(((vrows - 1) * H * P + P) * 2));
        constexpr int XU = ROWS * (P / 8), XPT = XU / NT;
        constexpr int HU = P * N / 8, HPT = (HU + NT - 1) / NT;
        Raw8<bf16_t> px[XPT];
        uint4 ph[HPT];
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int u = tid + k * NT;
            px[k].load(rx, (uint32_t)((u / (P / 8)) * H * P + 8 * (u % (P / 8))));
        }
        const f16 *hp = hen + bhc * P * N;
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int u = tid + k * NT;
            if (HU % NT == 0 || u < HU) ph[k] = *reinterpret_cast<const uint4 *>(hp + 8 * u);
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
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int u = tid + k * NT;
            if (HU % NT == 0 || u < HU) *reinterpret_cast<uint4 *>(&hs[(u / (N / 8)) * LDH + 8 * (u % (N / 8))]) = ph[k];
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
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cm + ((size_t)b * L + tc) * G * N + (size_t)g * N,
                                                (uint32_t)(((vrows - 1) * G * N + N) * 2));
    const size_t base_y = (((size_t)b * L + tc) * H + h) * P;
    const bool y16 = OPT && opt.y_bf16;
    const uint32_t es = y16 ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(
        y16 ? (void *)(static_cast<uint16_t *>(y) + base_y) : (void *)(static_cast<float *>(y) + base_y),
        (uint32_t)(((vrows - 1) * H * P + P) * es));

#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int t = k == 0 ? wave : 15 - wave;
        const int ibase = 16 * t;
        const int ns = (ibase + 15) / 32 + 1;  // 32-column steps up to the diagonal
        const int Tt = (t & 1) ? ((t >> 1) + 1) * ((t >> 1) + 1) : (t >> 1) * ((t >> 1) + 1);
        // the tile's GEMM1 slices (fp16, accumulator order) and C rows
        const size_t slice0 = (((size_t)b * G + g) * nc + c) * SPC + Tt;
        const f16 *gq = static_cast<const f16 *>(cbg) + (slice0 * 64 + lane) * 8;
        f16x8 gs[NSMAX];
#pragma unroll
        for (int s = 0; s < NSMAX; ++s)
            if (s < ns) gs[s] = *reinterpret_cast<const f16x8 *>(gq + (size_t)s * 512);

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
        // ---- Step-4: exp(a_i) * (C_i . H_enter[p, :]), then the skip term (the C rows are
        // loaded only now, so that they do not hold registers through the steps)
        {
            bf16x8 cb[KS];
            const uint32_t row = (uint32_t)((ibase + li) * G * N);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cb[ks] = __builtin_bit_cast(bf16x8, buf_load16(rc, 2u * (row + ks * 32 + 8 * lg)));
            f32x4 off[TP];
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) off[pt] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 ch = bf16x8_to_f16x8(cb[ks]);
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
            const bf16_t *zp = static_cast<const bf16_t *>(opt.z) + ((size_t)b * L + tc) * H * P + (size_t)h * P;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(zp, (uint32_t)(((vrows - 1) * H * P + P) * 2));
            uint32_t zr[TP][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    zr[pt][r] = __builtin_amdgcn_raw_buffer_load_b16(
                        rz, (int)(2u * (uint32_t)((ibase + 4 * lg + r) * H * P + pt * 16 + li)), 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= silu(__uint_as_float(zr[pt][r] << 16));
        }
        // ---- y: buffer stores over the item's valid rows (rows past the sequence dropped);
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

// Whether the one-round kernel takes this problem: bf16 inputs, chunks of 256 tokens,
// supported P, and no more items than two per compute unit.
bool chunk_scan_small_fits(const Dims &d, int ncu)
{
    return d.bf16 && d.Q == 256 && d.P == 64 && (long)d.nc * d.H * d.B <= 2L * ncu;
}

hipError_t launch_chunk_scan_small(const void *x, const void *Cm, const void *cb, const float *acum,
                                   const float *dtc, const void *h_enter, const float *D, void *y,
                                   const SsdOpts &o, const Dims &d, hipStream_t s)
{
    const unsigned nitems = (unsigned)(d.nc * d.H * d.B);
    const bf16_t *xx = static_cast<const bf16_t *>(x), *cc = static_cast<const bf16_t *>(Cm);
    const f16 *hh = static_cast<const f16 *>(h_enter);
#define SSD_SMALL_LAUNCH(NN)                                                                                   \
    do {                                                                                                       \
        if (o.z || o.y_bf16)                                                                                   \
            chunk_scan_small_kernel<64, NN, true><<<nitems, 512, 0, s>>>(xx, cc, cb, acum, dtc, hh, D, y, o, d.L, \
                                                                         d.H, d.G, d.nc);                      \
        else                                                                                                   \
            chunk_scan_small_kernel<64, NN, false><<<nitems, 512, 0, s>>>(xx, cc, cb, acum, dtc, hh, D, y, o,     \
                                                                          d.L, d.H, d.G, d.nc);                \
    } while (0)
    switch (d.N) {
    case 32: SSD_SMALL_LAUNCH(32); break;
    case 64: SSD_SMALL_LAUNCH(64); break;
    case 128: SSD_SMALL_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_SMALL_LAUNCH
    return hipGetLastError();
}

}  // namespace ssd
