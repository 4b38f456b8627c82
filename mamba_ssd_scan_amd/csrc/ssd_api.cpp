// ssd_api.cpp -- the C ABI declared in include/ssd.h.
//
// Validates every argument before touching HIP, carves the caller's
// workspace, and enqueues the kernels on the caller's stream.  No device
// memory is allocated or freed here and no global state is kept.
#include "ssd.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <new>

#include "ssd_launch.h"

namespace ssd {
LaunchTiming *&launch_timing()
{
    static thread_local LaunchTiming *t = nullptr;
    return t;
}
}  // namespace ssd

namespace {


constexpr size_t kWsAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes the kernels are built for (the stage entry points take only these); the prefill
// and the decode step take any multiple of 16 up to 256 (the prefill pads to a built size).
bool native_p(int v) { return v == 32 || v == 64 || v == 128; }
bool native_n(int v) { return v == 32 || v == 64 || v == 128 || v == 256; }
bool any16(int v) { return v >= 16 && v <= 256 && v % 16 == 0; }
bool supported_chunk(int q) { return q == 16 || q == 32 || q == 64 || q == 128 || q == 256; }

// Common shape checks.  seqlen < 0 => not a sequence call (decode).  native: only the
// built sizes of P and N (stage entry points).
int check_shape(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk,
                bool need_chunk, bool native = false)
{
    if (batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0) return SSD_ERR_INVALID_ARG;
    if (need_chunk && (seqlen < 0 || chunk <= 0)) return SSD_ERR_INVALID_ARG;
    if (nheads % ngroups != 0) return SSD_ERR_INVALID_ARG;
    if (native ? !(native_p(headdim) && native_n(dstate)) : !(any16(headdim) && any16(dstate)))
        return SSD_ERR_UNSUPPORTED;
    if (need_chunk && !supported_chunk(chunk)) return SSD_ERR_UNSUPPORTED;
    if (batch > 65535 || nheads > 65535) return SSD_ERR_UNSUPPORTED;  // grid y/z limits
    // chunk counts and token offsets are formed in 32-bit ints
    if (need_chunk && (long long)seqlen + chunk > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    const long long hx = headdim > 128 ? 2LL * nheads : nheads;  // heads as the kernels see them (see PadPlan)
    if (need_chunk && hx + 4LL * ngroups > 65535) return SSD_ERR_UNSUPPORTED;  // chunk-state grid y
    if ((long long)batch * hx > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    // One chunk of x or B/C is addressed with 32-bit byte offsets inside the kernels.
    if (need_chunk && (long long)chunk * 4 * ((long long)nheads * headdim > (long long)ngroups * dstate
                                                  ? (long long)nheads * headdim
                                                  : (long long)ngroups * dstate) >= 0x7fffffffLL)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// input storage (x, B, C): fp32, bf16 or fp8 e4m3; y: fp32 or bf16
int check_dtype(ssd_dtype_t t)
{
    return (t == SSD_F32 || t == SSD_BF16 || t == SSD_FP8_E4M3) ? SSD_OK : SSD_ERR_INVALID_ARG;
}
int check_ydtype(ssd_dtype_t t) { return (t == SSD_F32 || t == SSD_BF16) ? SSD_OK : SSD_ERR_INVALID_ARG; }

// bytes of one x, B or C element; of one dt or z element (bf16 beside fp8 inputs)
size_t in_size(ssd_dtype_t t) { return t == SSD_BF16 ? 2 : t == SSD_FP8_E4M3 ? 1 : 4; }
size_t dt_size(ssd_dtype_t t) { return t == SSD_F32 ? 4 : 2; }

struct WsLayout {
    size_t ctl, acum, dtc, states, cb, sync, total;  // byte offsets of each region, then total bytes
};

// fp32 elements of the GEMM1 output: 512 per 32-column step of every chunk of every group
size_t gemm1_elems(int batch, int ngroups, int nchunks, int chunk)
{
    return (size_t)batch * ngroups * nchunks * ssd::gemm1_steps_per_chunk(chunk) * 512;
}

ssd::Dims make_dims(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk,
                    ssd_dtype_t t);

// The workspace of every prefill path.  The first 256 bytes are the control block that all
// paths share (word 1: the give-up word that ssd_prefill_check reads); the staged and
// one-round paths carve their regions after it, the single-pass path carves its own layout
// from offset 0 (its control block is the same 256 bytes), and the size covers both.
WsLayout ws_layout(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk)
{
    const size_t nc = ((size_t)seqlen + chunk - 1) / chunk;
    const size_t bhq = (size_t)batch * nheads * nc * chunk;
    WsLayout w;
    w.ctl = 0;
    w.acum = kWsAlign;
    w.dtc = align_up(w.acum + 4 * bhq, kWsAlign);
    w.states = align_up(w.dtc + 4 * bhq, kWsAlign);
    w.cb = align_up(w.states + 4 * (size_t)batch * nheads * nc * headdim * dstate, kWsAlign);
    w.sync = align_up(w.cb + 4 * gemm1_elems(batch, ngroups, (int)nc, chunk), kWsAlign);
    w.total = align_up(w.sync + 4 * (size_t)batch * nheads * ssd::kSyncStride, kWsAlign);  // a counter per (b, h)
    const ssd::Dims d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, SSD_BF16);
    if (ssd::fused_prefill_shape(d)) w.total = std::max(w.total, ssd::fused_prefill_ws_bytes(d));
    return w;
}

// Whether X cannot stay in the Infinity Cache (256 MiB on MI355X) from the prefill's first
// launch to its chunk scan: in between, the chunk states are written, read and written back
// as entering states, and the scan writes y as it goes.  Then the launches that stream X (and
// the scan's entering states, read once) read them non-temporally, which leaves the cache to
// the states and to y on its way out.  The bound is half the cache, as measured: in-process
// A/B, the 2.7B 16384-token step 235 -> 226-229 us, the 370M 8 x 2048-token step 119.5 -> 117
// us (fp32 y) and 117 -> 112.5 us (bf16 y, 268 MB in all); at the 130M 4096-token shape (50 MB)
// the chunk scan still finds X in the cache, and streaming made the step ~5% longer.
bool stream_x(const ssd::Dims &d, bool y_bf16)
{
    const double tok = (double)d.B * d.L * d.H * d.P;
    const double xb = tok * (d.in == ssd::kInFp8 ? 1 : d.in == ssd::kInBf16 ? 2 : 4);
    const double sb = (double)d.B * d.H * d.nc * d.P * d.N * (d.half() ? 2 : 4);
    const double yb = tok * (y_bf16 ? 2 : 4);
    return xb + 2.0 * sb + yb > 128.0 * 1024 * 1024;
}

// How the prefill runs a shape whose P or N the kernels are not built for: P and N padded to
// the next built size (zero channels of x and z, zero state columns of B, C and the states),
// and a head of more than 128 channels run as two heads of half as many (its channels evolve
// independently and share dt, A, D and the head's group of B and C).
struct PadPlan {
    int H, P, N;  // the problem as the kernels see it
    int split;    // 1, or 2 kernel heads per head
};
PadPlan pad_plan(int nheads, int headdim, int dstate)
{
    PadPlan q;
    const int P = headdim <= 32 ? 32 : headdim <= 64 ? 64 : headdim <= 128 ? 128 : 256;
    q.N = dstate <= 32 ? 32 : dstate <= 64 ? 64 : dstate <= 128 ? 128 : 256;
    q.split = P == 256 ? 2 : 1;
    q.P = P / q.split;
    q.H = nheads * q.split;
    return q;
}
// The padded route's workspace: the padded problem's own workspace first (its control block
// at offset 0, so ssd_prefill_check reads the same word), then the padded copies.
struct PadWs {
    size_t inner, x, z, b, c, dt, A, D, bias, h0, y, fin, total;
};
PadWs pad_ws(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk)
{
    const PadPlan q = pad_plan(nheads, headdim, dstate);
    const size_t tok = (size_t)batch * seqlen, xel = tok * q.H * q.P, bel = tok * ngroups * q.N;
    const size_t sel = (size_t)batch * q.H * q.P * q.N;
    PadWs w;
    w.inner = ws_layout(batch, seqlen, q.H, q.P, q.N, ngroups, chunk).total;
    w.x = align_up(w.inner, kWsAlign);
    w.z = align_up(w.x + 4 * xel, kWsAlign);
    w.b = align_up(w.z + 4 * xel, kWsAlign);
    w.c = align_up(w.b + 4 * bel, kWsAlign);
    w.dt = align_up(w.c + 4 * bel, kWsAlign);
    w.A = align_up(w.dt + 4 * tok * q.H, kWsAlign);
    w.D = align_up(w.A + 4 * (size_t)q.H, kWsAlign);
    w.bias = align_up(w.D + 4 * (size_t)q.H, kWsAlign);
    w.h0 = align_up(w.bias + 4 * (size_t)q.H, kWsAlign);
    w.y = align_up(w.h0 + 4 * sel, kWsAlign);
    w.fin = align_up(w.y + 4 * xel, kWsAlign);
    w.total = align_up(w.fin + 4 * sel, kWsAlign);
    return w;
}
bool native_shape(int headdim, int dstate) { return native_p(headdim) && native_n(dstate); }
size_t prefill_ws_bytes(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk)
{
    return native_shape(headdim, dstate) ? ws_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk).total
                                         : pad_ws(batch, seqlen, nheads, headdim, dstate, ngroups, chunk).total;
}

ssd::Dims make_dims(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk,
                    ssd_dtype_t t)
{
    ssd::Dims d;
    d.B = batch; d.L = seqlen; d.H = nheads; d.P = headdim; d.N = dstate; d.G = ngroups; d.Q = chunk;
    d.nc = chunk > 0 ? (int)(((long long)seqlen + chunk - 1) / chunk) : 0;
    d.in = t == SSD_FP8_E4M3 ? ssd::kInFp8 : t == SSD_BF16 ? ssd::kInBf16 : ssd::kInF32;
    d.sx = nheads * headdim; d.sbc = ngroups * dstate; d.sdt = nheads; d.sz = nheads * headdim;
    return d;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// Argument checks of one decode token (ssd_step_ex and every token of a decode graph).
int check_step_args(const float *state, const void *x, const void *dt, const float *A, const void *Bm,
                    const void *Cm, const float *D, const float *dt_bias, const void *z, const void *y,
                    ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int dstate,
                    int ngroups)
{
    if (check_dtype(in_dtype) != SSD_OK || check_ydtype(y_dtype) != SSD_OK) return SSD_ERR_INVALID_ARG;
    const int st = check_shape(batch, -1, nheads, headdim, dstate, ngroups, 0, false);
    if (st != SSD_OK) return st;
    if (!state || !x || !dt || !A || !Bm || !Cm || !y) return SSD_ERR_INVALID_ARG;
    const size_t es = in_size(in_dtype), ds = dt_size(in_dtype);
    if (!aligned(state, 16) || !aligned(x, es) || !aligned(dt, ds) || !aligned(Bm, es) || !aligned(Cm, es) ||
        !aligned(A, 4) || !aligned(D, 4) || !aligned(y, in_size(y_dtype)) || !aligned(dt_bias, 4) || !aligned(z, ds))
        return SSD_ERR_INVALID_ARG;
    return SSD_OK;
}

#define SSD_TRY(expr)                      \
    do {                                   \
        const int _s = (expr);             \
        if (_s != SSD_OK) return _s;       \
    } while (0)

int check_seq_inputs(const void *x, const void *dt, const void *Bm, ssd_dtype_t t)
{
    if (!x || !dt || !Bm) return SSD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(Bm, 16) || !aligned(dt, dt_size(t))) return SSD_ERR_INVALID_ARG;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_status_string(int status)
{
    switch (status) {
    case SSD_OK: return "SSD_OK: success";
    case SSD_ERR_INVALID_ARG: return "SSD_ERR_INVALID_ARG: null/misaligned pointer, bad size or dtype, or nheads % ngroups != 0";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: headdim/dstate not a multiple of 16 in 16..256 (stage entry points: 32/64/128, and 256 for dstate), chunk not 16..256 (power of two), size limits, or a forced path that does not apply";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing, smaller than ssd_prefill_workspace_size() or not 256-byte aligned";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP kernel launch failed";
    case SSD_ERR_SYNC: return "SSD_ERR_SYNC: a bounded wait between workgroups of the last prefill gave up; its output is not valid";
    default: return "unknown ssd status";
    }
}

int ssd_version(void) { return (4 << 16) | 4; }

size_t ssd_prefill_workspace_size(int batch, int seqlen, int nheads, int headdim, int dstate,
                                  int ngroups, int chunk)
{
    if (check_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, true) != SSD_OK) return 0;
    return prefill_ws_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk);
}

int ssd_chunk_cumsum(const void *dt, const float *A, float *dA_cum, float *dt_c, ssd_dtype_t in_dtype,
                     int batch, int seqlen, int nheads, int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    // headdim/dstate do not enter this stage; pass a supported placeholder.
    SSD_TRY(check_shape(batch, seqlen, nheads, 64, 64, 1, chunk, true));
    if (seqlen == 0) return SSD_OK;
    if (!dt || !A || !dA_cum || !dt_c) return SSD_ERR_INVALID_ARG;
    if (!aligned(dt, dt_size(in_dtype)) || !aligned(A, 4) || !aligned(dA_cum, 16) || !aligned(dt_c, 16))
        return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, seqlen, nheads, 64, 64, 1, chunk, in_dtype);
    return hip_status(ssd::launch_chunk_cumsum(dt, A, dA_cum, dt_c, d, (hipStream_t)hip_stream));
}

int ssd_chunk_state(const void *x, const void *Bm, const float *dA_cum, const float *dt_c, void *states,
                    ssd_dtype_t in_dtype, int batch, int seqlen, int nheads, int headdim, int dstate,
                    int ngroups, int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    SSD_TRY(check_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, true, true));
    if (seqlen == 0) return SSD_OK;
    SSD_TRY(check_seq_inputs(x, dt_c, Bm, SSD_F32));
    if (!dA_cum || !states || !aligned(dA_cum, 16) || !aligned(states, 16)) return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, in_dtype);
    return hip_status(ssd::launch_chunk_state(x, Bm, dA_cum, dt_c, states, d, (hipStream_t)hip_stream));
}

int ssd_state_passing(void *states, const float *dA_cum, const float *initial_state, float *final_state,
                      ssd_dtype_t in_dtype, int batch, int nheads, int headdim, int dstate, int nchunks,
                      int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    if (nchunks < 0) return SSD_ERR_INVALID_ARG;
    if ((long long)nchunks * chunk > 0x7fffffffLL - 256) return SSD_ERR_UNSUPPORTED;  // nchunks * chunk is an int below
    SSD_TRY(check_shape(batch, nchunks, nheads, headdim, dstate, 1, chunk, true, true));
    if (!aligned(initial_state, 16) || !aligned(final_state, 16)) return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, nchunks * chunk, nheads, headdim, dstate, 1, chunk, in_dtype);
    hipStream_t s = (hipStream_t)hip_stream;
    if (nchunks == 0) {
        if (final_state)
            return hip_status(ssd::launch_fill_state(final_state, initial_state,
                                                     (size_t)batch * nheads * headdim * dstate, s));
        return SSD_OK;
    }
    if (!states || !dA_cum || !aligned(states, 16) || !aligned(dA_cum, 16)) return SSD_ERR_INVALID_ARG;
    return hip_status(ssd::launch_state_passing(states, dA_cum, initial_state, final_state, d, s));
}

size_t ssd_chunk_gemm1_size(int batch, int seqlen, int ngroups, int chunk)
{
    // headdim/dstate/nheads do not enter the size; pass supported placeholders.
    if (check_shape(batch, seqlen, ngroups, 64, 64, ngroups, chunk, true, true) != SSD_OK) return 0;
    return 4 * gemm1_elems(batch, ngroups, (seqlen + chunk - 1) / chunk, chunk);
}

int ssd_chunk_gemm1(const void *Bm, const void *Cm, float *cb, ssd_dtype_t in_dtype, int batch, int seqlen,
                    int dstate, int ngroups, int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    SSD_TRY(check_shape(batch, seqlen, ngroups, 64, dstate, ngroups, chunk, true, true));
    if (seqlen == 0) return SSD_OK;
    if (!Bm || !Cm || !cb || !aligned(Bm, 16) || !aligned(Cm, 16) || !aligned(cb, 16)) return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, seqlen, ngroups, 64, dstate, ngroups, chunk, in_dtype);
    return hip_status(ssd::launch_chunk_gemm1(Bm, Cm, cb, d, (hipStream_t)hip_stream));
}

int ssd_chunk_scan(const void *x, const void *Cm, const float *cb, const float *dA_cum, const float *dt_c,
                   const void *h_enter, const float *D, float *y, ssd_dtype_t in_dtype, int batch,
                   int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    SSD_TRY(check_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, true, true));
    if (seqlen == 0) return SSD_OK;
    SSD_TRY(check_seq_inputs(x, dt_c, Cm, SSD_F32));
    if (!cb || !dA_cum || !h_enter || !y) return SSD_ERR_INVALID_ARG;
    if (!aligned(cb, 16) || !aligned(dA_cum, 16) || !aligned(h_enter, 16) || !aligned(y, 16) || !aligned(D, 4))
        return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, in_dtype);
    const ssd::SsdOpts o = {nullptr, 0, nullptr, 0};
    return hip_status(
        ssd::launch_chunk_scan(x, Cm, cb, dA_cum, dt_c, h_enter, D, y, o, d, (hipStream_t)hip_stream));
}

int ssd_chunk_scan_passing(const void *x, const void *Cm, const float *cb, const float *dA_cum, const float *dt_c,
                           void *states, const float *initial_state, float *final_state, const float *D, float *y,
                           unsigned *sync, ssd_dtype_t in_dtype, int batch, int seqlen, int nheads, int headdim,
                           int dstate, int ngroups, int chunk, void *hip_stream)
{
    SSD_TRY(check_dtype(in_dtype));
    SSD_TRY(check_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, true, true));
    if (seqlen == 0) return SSD_OK;
    SSD_TRY(check_seq_inputs(x, dt_c, Cm, SSD_F32));
    if (!cb || !dA_cum || !states || !y || !sync) return SSD_ERR_INVALID_ARG;
    if (!aligned(cb, 16) || !aligned(dA_cum, 16) || !aligned(states, 16) || !aligned(y, 16) || !aligned(D, 4) ||
        !aligned(sync, 16) || !aligned(initial_state, 16) || !aligned(final_state, 16))
        return SSD_ERR_INVALID_ARG;
    const ssd::Dims d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, in_dtype);
    if (!ssd::chunk_scan_small_pass_shape(d)) return SSD_ERR_UNSUPPORTED;
    int ncu = 0;
    SSD_TRY(hip_status(ssd::device_cu_count(&ncu)));
    if (!ssd::chunk_scan_small_pass_fits(d, ncu)) return SSD_ERR_UNSUPPORTED;
    ssd::SsdOpts o = {nullptr, 0, nullptr, 0};
    o.sync = sync;
    bool resident = false;
    SSD_TRY(hip_status(ssd::chunk_scan_small_resident(d, o, ncu, &resident)));
    if (!resident) return SSD_ERR_UNSUPPORTED;
    return hip_status(ssd::launch_chunk_scan_small(x, Cm, cb, dA_cum, dt_c, states, initial_state, final_state, D, y,
                                                   o, d, ncu, (hipStream_t)hip_stream));
}

}  // extern "C"

namespace {

int prefill_impl(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                 const float *dt_bias, int dt_softplus, const void *z, const float *initial_state, float *final_state,
                 void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen, int nheads, int headdim,
                 int dstate, int ngroups, int chunk, long long x_stride, long long bc_stride, long long dt_stride,
                 long long z_stride, void *workspace, size_t workspace_bytes, void *hip_stream, int path,
                 long long spin_limit);

// The prefill of a shape the kernels are not built for (see PadPlan): the inputs are copied
// into the workspace padded, the built prefill runs on the copies, and y and the final state
// are copied back without the padding.  Strides are the resolved (nonzero) ones.
int prefill_padded(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                   const float *dt_bias, int dt_softplus, const void *z, const float *initial_state,
                   float *final_state, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                   int nheads, int headdim, int dstate, int ngroups, int chunk, long long sx, long long sbc,
                   long long sdt, long long sz, void *workspace, size_t workspace_bytes, hipStream_t s, int path,
                   long long spin_limit)
{
    const PadPlan q = pad_plan(nheads, headdim, dstate);
    const PadWs w = pad_ws(batch, seqlen, nheads, headdim, dstate, ngroups, chunk);
    if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < w.total) return SSD_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const int es = (int)in_size(in_dtype), ds = (int)dt_size(in_dtype), ys = (int)in_size(y_dtype);
    const long long tok = (long long)batch * seqlen;
    const int Pp = q.P * q.split;  // padded channels of one head
    auto pad = [&](const void *src, size_t off, int e, long long nout, int nin_s, int nin_d, int slen, int dlen,
                   long long so, long long si, long long sk) {
        return hip_status(ssd::launch_pad_copy(src, ws + off, e, nout, nin_s, nin_d, slen, dlen, so, si, sk, s));
    };
    SSD_TRY(pad(x, w.x, es, tok, nheads, nheads, headdim, Pp, sx, headdim, 1));
    if (z) SSD_TRY(pad(z, w.z, ds, tok, nheads, nheads, headdim, Pp, sz, headdim, 1));
    SSD_TRY(pad(Bm, w.b, es, tok, ngroups, ngroups, dstate, q.N, sbc, dstate, 1));
    SSD_TRY(pad(Cm, w.c, es, tok, ngroups, ngroups, dstate, q.N, sbc, dstate, 1));
    // per-head parameters of split heads: each value twice, in place for both halves
    const void *dt2 = dt;
    const float *A2 = A, *D2 = D, *bias2 = dt_bias;
    long long dt_stride2 = sdt;
    if (q.split == 2) {
        SSD_TRY(pad(dt, w.dt, ds, tok, nheads, nheads, 2, 2, sdt, 1, 0));
        SSD_TRY(pad(A, w.A, 4, 1, nheads, nheads, 2, 2, 0, 1, 0));
        if (D) SSD_TRY(pad(D, w.D, 4, 1, nheads, nheads, 2, 2, 0, 1, 0));
        if (dt_bias) SSD_TRY(pad(dt_bias, w.bias, 4, 1, nheads, nheads, 2, 2, 0, 1, 0));
        dt2 = ws + w.dt;
        A2 = reinterpret_cast<const float *>(ws + w.A);
        D2 = D ? reinterpret_cast<const float *>(ws + w.D) : nullptr;
        bias2 = dt_bias ? reinterpret_cast<const float *>(ws + w.bias) : nullptr;
        dt_stride2 = 0;
    }
    const long long hs = (long long)headdim * dstate;
    if (initial_state)
        SSD_TRY(pad(initial_state, w.h0, 4, (long long)batch * nheads, headdim, Pp, dstate, q.N, hs, dstate, 1));
    SSD_TRY(prefill_impl(ws + w.x, dt2, A2, ws + w.b, ws + w.c, D2, bias2, dt_softplus, z ? ws + w.z : nullptr,
                         initial_state ? reinterpret_cast<const float *>(ws + w.h0) : nullptr,
                         final_state ? reinterpret_cast<float *>(ws + w.fin) : nullptr, ws + w.y, in_dtype, y_dtype,
                         batch, seqlen, q.H, q.P, q.N, ngroups, chunk, 0, 0, dt_stride2, 0, workspace, w.inner, s,
                         path, spin_limit));
    // y [B, L, H, Pp] -> [B, L, H, P]; final [B, H, Pp, N'] -> [B, H, P, N]
    SSD_TRY(hip_status(ssd::launch_pad_copy(ws + w.y, y, ys, tok, nheads, nheads, headdim, headdim,
                                            (long long)nheads * Pp, Pp, 1, s)));
    if (final_state)
        SSD_TRY(hip_status(ssd::launch_pad_copy(ws + w.fin, final_state, 4, (long long)batch * nheads, headdim,
                                                headdim, dstate, dstate, (long long)Pp * q.N, q.N, 1, s)));
    return SSD_OK;
}

// The prefill with an explicit path (0: the library's choice) and wait bound (< 0: default).
int prefill_impl(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                 const float *dt_bias, int dt_softplus, const void *z, const float *initial_state, float *final_state,
                 void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen, int nheads, int headdim,
                 int dstate, int ngroups, int chunk, long long x_stride, long long bc_stride, long long dt_stride,
                 long long z_stride, void *workspace, size_t workspace_bytes, void *hip_stream, int path,
                 long long spin_limit)
{
    SSD_TRY(check_dtype(in_dtype));
    SSD_TRY(check_ydtype(y_dtype));
    if (path < SSD_PATH_AUTO || path > SSD_PATH_STAGED_ONE_HEAD) return SSD_ERR_INVALID_ARG;
    if (!aligned(dt_bias, 4) || !aligned(z, dt_size(in_dtype))) return SSD_ERR_INVALID_ARG;
    SSD_TRY(check_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, true));
    // token strides: 0 = dense; x, B and C rows are read with 16-byte loads
    const long long esz = (long long)in_size(in_dtype), hp = (long long)nheads * headdim,
                    gn = (long long)ngroups * dstate;
    const long long sx = x_stride ? x_stride : hp, sbc = bc_stride ? bc_stride : gn,
                    sdt = dt_stride ? dt_stride : nheads, sz = z_stride ? z_stride : hp;
    if (sx < hp || sbc < gn || sdt < nheads || sz < hp) return SSD_ERR_INVALID_ARG;
    if ((sx * esz) % 16 != 0 || (sbc * esz) % 16 != 0) return SSD_ERR_INVALID_ARG;
    const long long dsz = (long long)dt_size(in_dtype);
    const long long smax = std::max(std::max(sx * esz, sbc * esz), std::max(sdt * dsz, sz * dsz));  // bytes
    if ((long long)chunk * smax >= 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;  // 32-bit offsets per chunk
    if (!aligned(initial_state, 16) || !aligned(final_state, 16)) return SSD_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)hip_stream;
    if (seqlen == 0) {
        if (final_state)
            return hip_status(ssd::launch_fill_state(final_state, initial_state,
                                                     (size_t)batch * nheads * headdim * dstate, s));
        return SSD_OK;
    }
    SSD_TRY(check_seq_inputs(x, dt, Bm, in_dtype));
    if (!A || !Cm || !y || !aligned(A, 4) || !aligned(Cm, 16) || !aligned(y, 16) || !aligned(D, 4))
        return SSD_ERR_INVALID_ARG;
    if (!native_shape(headdim, dstate))
        return prefill_padded(x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, initial_state, final_state, y, in_dtype,
                              y_dtype, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, sx, sbc, sdt, sz,
                              workspace, workspace_bytes, s, path, spin_limit);
    const WsLayout w = ws_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk);
    if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < w.total) return SSD_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    float *acum = reinterpret_cast<float *>(ws + w.acum);
    float *dtc = reinterpret_cast<float *>(ws + w.dtc);
    void *states = ws + w.states;
    float *cb = reinterpret_cast<float *>(ws + w.cb);
    ssd::Dims d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, in_dtype);
    d.sx = (int)sx; d.sbc = (int)sbc; d.sdt = (int)sdt; d.sz = (int)sz;

    ssd::SsdOpts o = {dt_bias, dt_softplus ? 1 : 0, z, y_dtype == SSD_BF16 ? 1 : 0};
    o.ctl = reinterpret_cast<unsigned *>(ws + w.ctl);
    o.spin = spin_limit < 0 ? 0u : (unsigned)std::min(spin_limit, 0x7fffffffLL) + 1u;
    o.stream_x = stream_x(d, y_dtype == SSD_BF16) ? 1 : 0;
    int ncu = 0;
    SSD_TRY(hip_status(ssd::device_cu_count(&ncu)));
    // The one-round path needs every workgroup of the chunk scan resident at once (its
    // workgroups of a head wait for each other): the grid must fit and the compiled kernel's
    // occupancy must allow it.
    bool one_round = false;
    if (ssd::chunk_scan_small_pass_fits(d, ncu)) {
        ssd::SsdOpts po = o;
        po.sync = reinterpret_cast<unsigned *>(ws + w.sync);
        SSD_TRY(hip_status(ssd::chunk_scan_small_resident(d, po, ncu, &one_round)));
    }
    const bool single_pass = ssd::fused_prefill_shape(d);
    // The single pass is taken only when asked for: measured on MI355X it is slower than the
    // three launches on every many-round shape tried (0.58-0.99x), its items being bound by
    // the latency of their device-coherent exchange rather than by HBM.
    if (path == SSD_PATH_AUTO) path = one_round ? SSD_PATH_ONE_ROUND : SSD_PATH_STAGED;
    if ((path == SSD_PATH_ONE_ROUND && !one_round) || (path == SSD_PATH_SINGLE_PASS && !single_pass))
        return SSD_ERR_UNSUPPORTED;

    if (path == SSD_PATH_ONE_ROUND) {
        // every (b, h, chunk) item is resident at once: Step-3 runs inside the chunk scan
        o.sync = reinterpret_cast<unsigned *>(ws + w.sync);
        SSD_TRY(hip_status(ssd::launch_cumsum_chunk_state_gemm1(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s)));
        return hip_status(ssd::launch_chunk_scan_small(x, Cm, cb, acum, dtc, states, initial_state, final_state, D, y,
                                                       o, d, ncu, s));
    }
    if (path == SSD_PATH_SINGLE_PASS)
        return hip_status(ssd::launch_prefill_fused(x, Bm, Cm, dt, A, D, initial_state, final_state, y, workspace, o,
                                                    d, s));
    // Three launches (SSD_PATH_STAGED_ONE_HEAD: one head per chunk-state workgroup, so that a
    // comparison with the other paths covers the two-heads-per-workgroup kernel too).
    SSD_TRY(hip_status(ssd::launch_cumsum_chunk_state_gemm1(x, Bm, dt, A, acum, dtc, states, Cm, cb, o, d, s,
                                                            path != SSD_PATH_STAGED_ONE_HEAD)));
    SSD_TRY(hip_status(ssd::launch_state_passing(states, acum, initial_state, final_state, d, s)));
    return hip_status(ssd::launch_chunk_scan(x, Cm, cb, acum, dtc, states, D, y, o, d, s));
}

}  // namespace

extern "C" {

int ssd_prefill_strided(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                        const float *dt_bias, int dt_softplus, const void *z, const float *initial_state,
                        float *final_state, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch,
                        int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk, long long x_stride,
                        long long bc_stride, long long dt_stride, long long z_stride, void *workspace,
                        size_t workspace_bytes, void *hip_stream)
{
    return prefill_impl(x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, initial_state, final_state, y, in_dtype, y_dtype,
                        batch, seqlen, nheads, headdim, dstate, ngroups, chunk, x_stride, bc_stride, dt_stride,
                        z_stride, workspace, workspace_bytes, hip_stream, SSD_PATH_AUTO, -1);
}

int ssd_prefill_forced(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                       const float *dt_bias, int dt_softplus, const void *z, const float *initial_state,
                       float *final_state, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                       int nheads, int headdim, int dstate, int ngroups, int chunk, long long x_stride,
                       long long bc_stride, long long dt_stride, long long z_stride, void *workspace,
                       size_t workspace_bytes, void *hip_stream, int path, long long spin_limit)
{
    return prefill_impl(x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, initial_state, final_state, y, in_dtype, y_dtype,
                        batch, seqlen, nheads, headdim, dstate, ngroups, chunk, x_stride, bc_stride, dt_stride,
                        z_stride, workspace, workspace_bytes, hip_stream, path, spin_limit);
}

int ssd_prefill_timed(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                      const float *dt_bias, int dt_softplus, const void *z, const float *initial_state,
                      float *final_state, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                      int nheads, int headdim, int dstate, int ngroups, int chunk, long long x_stride,
                      long long bc_stride, long long dt_stride, long long z_stride, void *workspace,
                      size_t workspace_bytes, void *hip_stream, int path, long long spin_limit,
                      void *const *start_events, void *const *stop_events, const char **kernel_names,
                      int capacity, int *n_launches)
{
    if (capacity < 0 || (capacity > 0 && (!start_events || !stop_events))) return SSD_ERR_INVALID_ARG;
    for (int i = 0; i < capacity; i++)
        if (!start_events[i] || !stop_events[i]) return SSD_ERR_INVALID_ARG;
    ssd::LaunchTiming t = {start_events, stop_events, kernel_names, capacity, 0};
    ssd::LaunchTiming *&cur = ssd::launch_timing();
    ssd::LaunchTiming *const prev = cur;
    cur = &t;
    const int r = prefill_impl(x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, initial_state, final_state, y, in_dtype,
                               y_dtype, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, x_stride, bc_stride,
                               dt_stride, z_stride, workspace, workspace_bytes, hip_stream, path, spin_limit);
    cur = prev;
    if (n_launches) *n_launches = t.n;
    return r;
}

int ssd_prefill_check(const void *workspace, size_t workspace_bytes, void *hip_stream)
{
    if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < kWsAlign) return SSD_ERR_WORKSPACE;
    SSD_TRY(hip_status(hipStreamSynchronize((hipStream_t)hip_stream)));
    unsigned v = 0;
    SSD_TRY(hip_status(hipMemcpy(&v, static_cast<const char *>(workspace) + 4, 4, hipMemcpyDeviceToHost)));
    return v ? SSD_ERR_SYNC : SSD_OK;
}

int ssd_prefill_ex(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                   const float *dt_bias, int dt_softplus, const void *z, const float *initial_state,
                   float *final_state, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                   int nheads, int headdim, int dstate, int ngroups, int chunk, void *workspace,
                   size_t workspace_bytes, void *hip_stream)
{
    return ssd_prefill_strided(x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, initial_state, final_state, y, in_dtype,
                               y_dtype, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, 0, 0, 0, 0, workspace,
                               workspace_bytes, hip_stream);
}

int ssd_prefill(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                const float *initial_state, float *final_state, float *y, ssd_dtype_t in_dtype, int batch,
                int seqlen, int nheads, int headdim, int dstate, int ngroups, int chunk, void *workspace,
                size_t workspace_bytes, void *hip_stream)
{
    return ssd_prefill_ex(x, dt, A, Bm, Cm, D, nullptr, 0, nullptr, initial_state, final_state, y, in_dtype, SSD_F32,
                          batch, seqlen, nheads, headdim, dstate, ngroups, chunk, workspace, workspace_bytes,
                          hip_stream);
}

int ssd_step_strided(float *state, const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
                     const float *D, const float *dt_bias, int dt_softplus, const void *z, void *y,
                     ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int dstate,
                     int ngroups, long long x_stride, long long bc_stride, long long dt_stride, long long z_stride,
                     void *hip_stream)
{
    SSD_TRY(check_step_args(state, x, dt, A, Bm, Cm, D, dt_bias, z, y, in_dtype, y_dtype, batch, nheads, headdim,
                            dstate, ngroups));
    // batch strides: 0 = dense; each at least its dense row (element loads: no other alignment)
    const long long hp = (long long)nheads * headdim, gn = (long long)ngroups * dstate;
    const long long sx = x_stride ? x_stride : hp, sbc = bc_stride ? bc_stride : gn,
                    sdt = dt_stride ? dt_stride : nheads, sz = z_stride ? z_stride : hp;
    if (sx < hp || sbc < gn || sdt < nheads || sz < hp) return SSD_ERR_INVALID_ARG;
    if (std::max(std::max(sx, sbc), std::max(sdt, sz)) > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    ssd::Dims d = make_dims(batch, 1, nheads, headdim, dstate, ngroups, 1, in_dtype);
    d.sx = (int)sx; d.sbc = (int)sbc; d.sdt = (int)sdt; d.sz = (int)sz;
    const ssd::SsdOpts o = {dt_bias, dt_softplus ? 1 : 0, z, y_dtype == SSD_BF16 ? 1 : 0};
    return hip_status(ssd::launch_step(state, x, dt, A, Bm, Cm, D, y, o, d, (hipStream_t)hip_stream));
}

int ssd_step_ex(float *state, const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
                const float *D, const float *dt_bias, int dt_softplus, const void *z, void *y, ssd_dtype_t in_dtype,
                ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int dstate, int ngroups, void *hip_stream)
{
    return ssd_step_strided(state, x, dt, A, Bm, Cm, D, dt_bias, dt_softplus, z, y, in_dtype, y_dtype, batch, nheads,
                            headdim, dstate, ngroups, 0, 0, 0, 0, hip_stream);
}

int ssd_step(float *state, const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
             const float *D, float *y, ssd_dtype_t in_dtype, int batch, int nheads, int headdim, int dstate,
             int ngroups, void *hip_stream)
{
    return ssd_step_ex(state, x, dt, A, Bm, Cm, D, nullptr, 0, nullptr, y, in_dtype, SSD_F32, batch, nheads, headdim,
                       dstate, ngroups, hip_stream);
}

// ---- decode loop as one HIP graph

struct ssd_decode_graph {
    hipGraphExec_t exec;
    int device;
    int nsteps;
};

int ssd_decode_graph_create(ssd_decode_graph **out, int nsteps, float *state, const void *x, const void *dt,
                            const float *A, const void *Bm, const void *Cm, const float *D, const float *dt_bias,
                            int dt_softplus, const void *z, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype,
                            int batch, int nheads, int headdim, int dstate, int ngroups)
{
    if (!out) return SSD_ERR_INVALID_ARG;
    *out = nullptr;
    if (nsteps < 1 || nsteps > SSD_DECODE_GRAPH_MAX_STEPS) return SSD_ERR_INVALID_ARG;
    SSD_TRY(check_step_args(state, x, dt, A, Bm, Cm, D, dt_bias, z, y, in_dtype, y_dtype, batch, nheads, headdim,
                            dstate, ngroups));
    // Byte strides of one token's slot in the step-major buffers.
    const size_t es = in_size(in_dtype), ds = dt_size(in_dtype);
    const size_t sx = (size_t)batch * nheads * headdim * es, sdt = (size_t)batch * nheads * ds;
    const size_t sz = (size_t)batch * nheads * headdim * ds;
    const size_t sbc = (size_t)batch * ngroups * dstate * es;
    const size_t sy = (size_t)batch * nheads * headdim * in_size(y_dtype);
    const ssd::Dims d = make_dims(batch, 1, nheads, headdim, dstate, ngroups, 1, in_dtype);

    int dev = 0;
    SSD_TRY(hip_status(hipGetDevice(&dev)));
    hipStream_t s = nullptr;
    SSD_TRY(hip_status(hipStreamCreateWithFlags(&s, hipStreamNonBlocking)));
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        hipError_t le = hipSuccess;
        for (int t = 0; t < nsteps && le == hipSuccess; ++t) {
            const char *zt = z ? static_cast<const char *>(z) + t * sz : nullptr;
            const ssd::SsdOpts o = {dt_bias, dt_softplus ? 1 : 0, zt, y_dtype == SSD_BF16 ? 1 : 0};
            le = ssd::launch_step(state, static_cast<const char *>(x) + t * sx, static_cast<const char *>(dt) + t * sdt,
                                  A, static_cast<const char *>(Bm) + t * sbc, static_cast<const char *>(Cm) + t * sbc,
                                  D, static_cast<char *>(y) + t * sy, o, d, s);
        }
        e = hipStreamEndCapture(s, &graph);  // always ends the capture, also after a failed launch
        if (le != hipSuccess) e = le;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(s);
    if (e != hipSuccess) {
        if (exec) (void)hipGraphExecDestroy(exec);
        return SSD_ERR_HIP;
    }
    ssd_decode_graph *g = new (std::nothrow) ssd_decode_graph{exec, dev, nsteps};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        return SSD_ERR_HIP;
    }
    *out = g;
    return SSD_OK;
}

int ssd_decode_graph_launch(ssd_decode_graph *g, void *hip_stream)
{
    if (!g) return SSD_ERR_INVALID_ARG;
    int dev = -1;
    SSD_TRY(hip_status(hipGetDevice(&dev)));
    if (dev != g->device) return SSD_ERR_INVALID_ARG;
    return hip_status(hipGraphLaunch(g->exec, (hipStream_t)hip_stream));
}

int ssd_decode_graph_steps(const ssd_decode_graph *g) { return g ? g->nsteps : 0; }

int ssd_decode_graph_destroy(ssd_decode_graph *g)
{
    if (!g) return SSD_OK;
    const hipError_t e = hipGraphExecDestroy(g->exec);
    delete g;
    return hip_status(e);
}

}  // extern "C"
