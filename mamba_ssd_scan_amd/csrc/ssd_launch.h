// ssd_launch.h -- host-side launchers of the gfx950 SSD kernels.
// Shapes are validated by the C ABI layer before any of these is called;
// each launcher only picks the template instance and the grid.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "ssd_common.h"

namespace ssd {

// Per-launch timing of a prefill (ssd_prefill_timed).  While such a call runs on a thread,
// every kernel launch of that thread binds the next caller event pair to the kernel itself
// (HIP's launch-with-events extension: the events take the kernel's own start and end, with
// no marker packets between launches) and records the kernel's name.
struct LaunchTiming {
    void *const *start;  // hipEvent_t[cap]
    void *const *stop;   // hipEvent_t[cap]
    const char **names;  // [cap] or nullptr
    int cap;             // event pairs available
    int n;               // launches made so far (may pass cap: those are not timed)
};
// The calling thread's current timing, nullptr outside a timed call.
LaunchTiming *&launch_timing();

// Launch of `k` on `s`, timed when the calling thread has a timing in place.  Launch errors
// are left for the caller's hipGetLastError(), as with the <<< >>> form.
template <typename... P, typename... A>
inline void launch_kernel(const char *name, void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A... a)
{
    LaunchTiming *t = launch_timing();
    if (t == nullptr) {
        k<<<grid, block, 0, s>>>(a...);
        return;
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (t->n < t->cap) {
        e0 = static_cast<hipEvent_t>(t->start[t->n]);
        e1 = static_cast<hipEvent_t>(t->stop[t->n]);
        if (t->names) t->names[t->n] = name;
    }
    t->n++;
    hipExtLaunchKernelGGL(k, grid, block, 0, s, e0, e1, 0u, a...);
}

// Storage type of x, B and C (the ABI's ssd_dtype_t values): fp32, bf16 or fp8 e4m3 (whose
// dt and z are bf16).  bf16 and fp8 inputs take the same paths, with fp16 chunk and
// entering states.
enum InType { kInF32 = 0, kInBf16 = 1, kInFp8 = 2 };

// The InType of a kernel instantiation's input element.
template <typename T> struct InOf;
template <> struct InOf<float> { static constexpr int v = kInF32; };
template <> struct InOf<bf16_t> { static constexpr int v = kInBf16; };
template <> struct InOf<fp8_t> { static constexpr int v = kInFp8; };

struct Dims {
    int B, L, H, P, N, G, Q, nc;  // batch, seqlen, heads, headdim, dstate, groups, chunk, chunks
    int in;                       // InType
    bool half() const { return in != kInF32; }  // fp16 states, fp16 matrix-core operands
    // elements between consecutive tokens of x, of B and C, of dt and of z (dense: H*P, G*N,
    // H, H*P); the prefill's kernels read their inputs with these, y is always dense
    int sx, sbc, sdt, sz;
};

hipError_t launch_chunk_cumsum(const void *dt, const float *A, float *acum, float *dtc,
                               const Dims &d, hipStream_t s);
// states: [B, H, nc, P, N], fp16 for bf16 and fp8 inputs (d.half()), fp32 otherwise; likewise below.
hipError_t launch_chunk_state(const void *x, const void *Bm, const float *acum, const float *dtc,
                              void *states, const Dims &d, hipStream_t s);
// Step-0 and Step-1 GEMM1 fused into the Step-2 launch: writes acum/dtc (same values as
// launch_chunk_cumsum), states, and the GEMM1 products cb (same as launch_chunk_gemm1).
// pair: whether two heads per workgroup may be used where they fit (same results)
hipError_t launch_cumsum_chunk_state_gemm1(const void *x, const void *Bm, const void *dt, const float *A,
                                           float *acum, float *dtc, void *states, const void *Cm, void *cb,
                                           const SsdOpts &o, const Dims &d, hipStream_t s, bool pair = true);
// The same launch with two heads of a group per workgroup (bf16, Q = 256, P = 64, an even
// number of heads per group): identical results.
bool chunk_state_pair_fits(const Dims &d);
hipError_t launch_chunk_state_pair(const void *x, const void *Bm, const void *dt, const float *A, float *acum,
                                   float *dtc, void *states, const void *Cm, void *cb, const SsdOpts &o,
                                   const Dims &d, hipStream_t s);
hipError_t launch_state_passing(void *states, const float *acum, const float *init, float *fin,
                                const Dims &d, hipStream_t s);
// Step-1 GEMM1 once per (batch, group, chunk): cb holds B * G * nc * gemm1_steps_per_chunk(Q)
// slices of 512 values, fp16 for bf16 inputs and fp32 for fp32 inputs (fragment order, see
// ssd_chunk_gemm1.hip).
int gemm1_steps_per_chunk(int q);
hipError_t launch_chunk_gemm1(const void *Bm, const void *Cm, void *cb, const Dims &d, hipStream_t s);
// h_enter: entering states [B, H, nc, P, N], fp16 for bf16 inputs (the off-diagonal
// operand precision), fp32 for fp32 inputs.
hipError_t launch_chunk_scan(const void *x, const void *Cm, const void *cb, const float *acum,
                             const float *dtc, const void *h_enter, const float *D, void *y,
                             const SsdOpts &o, const Dims &d, hipStream_t s);
// The chunk scan for problems whose items all fit at once (one item per workgroup, two
// workgroups per compute unit): bf16 inputs, Q = 256, P = 64, items <= 2 * ncu.
// o.sync == nullptr: h holds the entering states (fp16).  o.sync != nullptr: h holds the
// chunk states (fp16) and Step-3 runs inside the launch (entering states written over h,
// final state to fin, initial state from init); o.sync holds B*H counters that the
// chunk-state launch zeroed (launch_cumsum_chunk_state_gemm1 with the same o.sync).
bool chunk_scan_small_fits(const Dims &d, int ncu);
bool chunk_scan_small_pass_fits(const Dims &d, int ncu);  // ... and o.sync may be set (nc <= 16)
bool chunk_scan_small_pass_shape(const Dims &d);          // the part of it that needs no device query
hipError_t device_cu_count(int *ncu);  // compute units of the current device
// Whether the one-round launch (with o.sync as given) can have every workgroup resident at
// once on the current device (its occupancy, queried for the instantiation it would launch).
hipError_t chunk_scan_small_resident(const Dims &d, const SsdOpts &o, int ncu, bool *ok);
hipError_t launch_chunk_scan_small(const void *x, const void *Cm, const void *cb, const float *acum,
                                   const float *dtc, void *h, const float *init, float *fin, const float *D,
                                   void *y, const SsdOpts &o, const Dims &d, int ncu, hipStream_t s);
// The single-pass prefill for grids of many rounds (bf16, Q = 256, P = 64, N in {64, 128}):
// a GEMM1 launch, then one launch in which every (b, h, chunk) item forms its chunk state,
// receives its entering state through a look-back of kFusedDepth chunks and writes its
// output.  ws: fused_prefill_ws_bytes(d) bytes, 256-byte aligned; its first word after the
// ticket (byte 4) is the give-up word (nonzero: a bounded wait gave up, the output is not
// valid); o.spin bounds the waits.
constexpr int kFusedDepth = 2;
constexpr int kFusedRing = 8;  // ring slots per (b, h) of each kind (aggregates, inclusive states)
bool fused_prefill_shape(const Dims &d);
size_t fused_prefill_ws_bytes(const Dims &d);
hipError_t launch_prefill_fused(const void *x, const void *Bm, const void *Cm, const void *dt, const float *A,
                                const float *D, const float *init, float *fin, void *y, void *ws, const SsdOpts &o,
                                const Dims &d, hipStream_t s);
// Zero-padding copy: dst[(o * nin_dst + i) * dlen + k] = (i < nin_src && k < slen) ?
// src[o * so + i * si + k * sk] : 0 for o < nout, i < nin_dst, k < dlen; elements of 1, 2 or 4 bytes.
hipError_t launch_pad_copy(const void *src, void *dst, int elem_bytes, long long nout, int nin_src, int nin_dst,
                           int slen, int dlen, long long so, long long si, long long sk, hipStream_t s);
// dst[i] = src ? src[i] : 0 for i < n (n a multiple of 4, 16-byte aligned pointers).
hipError_t launch_fill_state(float *dst, const float *src, size_t n, hipStream_t s);
hipError_t launch_step(float *state, const void *x, const void *dt, const float *A, const void *Bm,
                       const void *Cm, const float *D, void *y, const SsdOpts &o, const Dims &d, hipStream_t s);

}  // namespace ssd
