/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD layer core.
 *
 * The layer core is the per-head state-space recurrence with a scalar
 * ("input-dependent diagonal") decay:
 *
 *   H_t = exp(dt_t * A_h) * H_{t-1} + dt_t * x_t * B_t^T      (state [P, N])
 *   y_t = H_t * C_t + D_h * x_t                               (output [P])
 *
 * for every batch entry b and head h, head h reading group g = h / (H/G) of
 * B and C.  Sources: "Mamba-Family State-Space Model Kernels on a
 * Programmable CGLA", Sec. III-A (in-projection output [z, x, B, C, dt];
 * chunks of Q tokens; Step-1 intra-chunk GEMM1 / Hadamard mask / GEMM2;
 * Step-3 sequential inter-chunk update of the recurrent state with a
 * diagonal A_c), Sec. IV-B and IV-C; "Compiler-First State Space Duality and
 * Portable O(1) Autoregressive Caching for Inference", abstract (diagonal
 * per-head dynamics, fixed-size chunking, a cached state for O(1) decode).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers, dense, row-major in the
 *   layouts written next to each argument; base addresses 16-byte aligned.
 * - The caller owns all memory.  The library never allocates or frees device
 *   memory; scratch comes from the caller's workspace, except for
 *   ssd_prefill_noalloc, whose scratch is a device array of the library's own (one per
 *   GPU, see there).  Apart from that array, its per-device address and the per-thread
 *   pointer through which ssd_prefill_timed reaches its own launches (set for the length
 *   of that call only), no global state: calls are reentrant and thread-safe.
 *   The one object the library creates is a decode graph, owned by the
 *   caller through its handle (ssd_decode_graph_create / _destroy).
 * - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *   stream) and return after enqueueing; nothing synchronises inside.
 * - Errors are negative return codes, never exceptions.  Every argument is
 *   validated before any HIP call, so a rejected call launches nothing.
 *   SSD_ERR_HIP means a launch failed; faults inside a kernel surface at the
 *   caller's next synchronisation.
 * - `in_dtype` selects the storage type of x, dt, B, C (and z): SSD_BF16 (uint16 bit
 *   patterns of bfloat16) or SSD_F32; or SSD_FP8_E4M3, where x, B and C are OCP fp8 e4m3
 *   codes (one byte: sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities, the
 *   codes 0x7f and 0xff are NaN) and dt and z stay bf16.  fp8 inputs take the bf16 paths
 *   (they widen exactly to fp16) and halve the bytes of x, B and C; the single-pass prefill
 *   path does not take them.  A and D are always fp32; the initial and final states and y are
 *   fp32 (y may be bf16 through the _ex calls, never fp8).  Accumulation is fp32.
 * - Precision inside a prefill (bf16 and fp8 inputs): the matrix-core operands are fp16 (the inputs
 *   convert exactly; computed operands -- the masked scores, the weighted B or X, the
 *   entering state of the off-diagonal product -- are rounded once).  Between kernels the
 *   staged and one-round paths keep the chunk and entering states in fp16; the single-pass
 *   path keeps them in fp32.  Range contract for bf16 inputs: |x|, |B|, |C|, every |C_i.B_j|
 *   and, on the staged and one-round paths, every state (initial, entering and chunk states)
 *   must stay below 65504, the fp16 limit; past it the values turn to inf in y (no error is
 *   raised).  fp32 inputs keep every product and state in fp32.
 * - Non-finite values are propagated, not trapped.
 *
 * Supported shapes: batch >= 1; seqlen >= 0; nheads % ngroups == 0;
 * chunk (Q) in {16, 32, 64, 128, 256}; headdim (P) and dstate (N) any multiple of 16
 * from 16 to 256 for the prefill and decode calls.  The kernels are built for
 * P in {32, 64, 128} and N in {32, 64, 128, 256}: the prefill runs other sizes padded
 * to the next built size inside its workspace (zero channels and zero state columns,
 * which add exact zeros), and a P above 128 as two heads of P/2 channels (a head's
 * channels evolve independently); the decode step takes every such size directly.
 * The stage entry points take only the built sizes.  Anything else returns
 * SSD_ERR_UNSUPPORTED (or SSD_ERR_INVALID_ARG for non-positive sizes).
 */
#ifndef MAMBA_SSD_SCAN_AMD_SSD_H
#define MAMBA_SSD_SCAN_AMD_SSD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_FP8_E4M3 = 2 } ssd_dtype_t;

enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer, H % G != 0 */
    SSD_ERR_UNSUPPORTED = -2, /* valid but unsupported P, N, Q or dtype */
    SSD_ERR_WORKSPACE = -3,   /* workspace missing, too small or not 256-byte aligned */
    SSD_ERR_HIP = -4,         /* a HIP launch failed */
    SSD_ERR_SYNC = -5         /* ssd_prefill_check: a bounded wait of the last prefill gave up */
};

/* Static description of a status code (never NULL). */
const char *ssd_status_string(int status);

/* Library ABI version, (major << 16) | minor. */
int ssd_version(void);

/*
 * Bytes of caller-provided workspace that ssd_prefill needs, or 0 for
 * invalid/unsupported shapes.  The first 256 bytes are a control block (word 1: the
 * give-up word that ssd_prefill_check reads); the rest is carved by whichever path the
 * prefill takes (below), and the size covers every path.  Staged and one-round paths,
 * each region 256-byte aligned:
 *   dA_cum  [B, H, nc, Q] fp32   per-chunk inclusive cumsum of dt*A
 *   dt_c    [B, H, nc, Q] fp32   dt regrouped per chunk (0 past seqlen)
 *   states  [B, H, nc, P, N] x 4 bytes: the chunk states, then the entering
 *           states (fp16 for bf16 inputs -- half the region -- fp32 for fp32 inputs)
 *   cb      ssd_chunk_gemm1_size(B, L, G, Q) bytes: the C.B^T products
 *   sync    [B, H] uint32 counters, one per 256 bytes, of the one-round path
 * Single-pass path: per (b, h) status words and 16 ring slots of P*N fp32 states, and the
 * C.B^T products.  nc = ceil(seqlen / Q).  For a P or N the kernels are not built for, the
 * workspace of the padded problem comes first, then padded copies of x, z, B, C, dt, A, D,
 * the dt bias, the initial state, y and the final state (4 bytes per element).
 * ssd_prefill_workspace_size returns the size of the layout the shape takes.
 */
size_t ssd_prefill_workspace_size(int batch, int seqlen, int nheads, int headdim,
                                  int dstate, int ngroups, int chunk);

/*
 * Chunked prefill over a whole sequence ("Mamba-Family State-Space Model Kernels on a
 * Programmable CGLA", Sec. III-A: chunks of Q tokens, Step-1 intra-chunk GEMM1 / mask /
 * GEMM2, Step-3 inter-chunk recurrence of the state with a diagonal A_c, Sec. IV-C;
 * "Compiler-First State Space Duality and Portable O(1) Autoregressive Caching for
 * Inference", abstract: fixed-size chunking, the final state as the decode cache).
 * Paths, all computing the same result up to rounding:
 *  - one-round (two launches), taken when every (b, h, chunk) item is resident at once
 *    (bf16, Q = 256, P = 64, nc <= 16, items <= 2 x compute units, and the compiled
 *    kernel's occupancy confirmed on the device): chunk states, then a chunk scan that
 *    walks Step-3 itself, its workgroups of a head waiting for each other;
 *  - staged (three launches), taken otherwise: the stage entry points below in order;
 *  - single pass (a GEMM1 launch, then one launch; bf16, Q = 256, P = 64, N in {64, 128}),
 *    only through ssd_prefill_forced: each item forms its chunk state, takes the state
 *    entering its chunk from the items of earlier chunks (they hold smaller tickets, so no
 *    co-residency is assumed) and writes its output.  It keeps the states in fp32 and moves
 *    about half the HBM bytes of the staged path, but on MI355X its device-coherent
 *    hand-offs make it slower, so the library does not pick it.
 * The waits between workgroups are bounded.  A wait that gives up (which needs a device
 * that stops running some of the launch's workgroups for about a second) sets the give-up
 * word; the kernels still finish, but y and final_state are then not valid:
 * ssd_prefill_check reports it.
 *
 *   x   [B, L, H, P] in_dtype       dt [B, L, H] in_dtype (used as given:
 *   A   [H] fp32                          positive step sizes, no softplus)
 *   Bm  [B, L, G, N] in_dtype       Cm [B, L, G, N] in_dtype
 *   D   [H] fp32, or NULL for no skip term
 *   initial_state [B, H, P, N] fp32, or NULL for zeros
 *   final_state   [B, H, P, N] fp32, or NULL; may alias initial_state
 *   y   [B, L, H, P] fp32 (written)
 *   workspace: >= ssd_prefill_workspace_size(...) bytes, 256-byte aligned,
 *              contents on entry ignored, clobbered on exit.
 * The result does not depend on `chunk` beyond rounding.  seqlen == 0 only
 * copies the initial state (or zeros) into final_state.
 */
int ssd_prefill(const void *x, const void *dt, const float *A, const void *Bm,
                const void *Cm, const float *D, const float *initial_state,
                float *final_state, float *y, ssd_dtype_t in_dtype, int batch,
                int seqlen, int nheads, int headdim, int dstate, int ngroups,
                int chunk, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * ssd_prefill with the work adjacent to the SSD core in a Mamba-2 block fused in
 * ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A:
 * the in-projection emits the gate z and the raw step-size channel next to x, B, C):
 *   dt_bias [H] fp32 or NULL   added to dt before the softplus (0 if NULL)
 *   dt_softplus                nonzero: the recurrence uses softplus(dt + dt_bias)
 *                              = log(1 + exp(dt + dt_bias)) as its step size;
 *                              zero: dt + dt_bias as given (must then be > 0)
 *   z [B, L, H, P] in_dtype or NULL   output gate: y <- y * z * sigmoid(z), applied
 *                              to the whole output (skip term included)
 *   y [B, L, H, P] y_dtype     SSD_F32, or SSD_BF16 (fp32 result rounded to nearest even)
 * Everything else as ssd_prefill; ssd_prefill is ssd_prefill_ex with NULL, 0, NULL, SSD_F32.
 */
int ssd_prefill_ex(const void *x, const void *dt, const float *A, const void *Bm,
                   const void *Cm, const float *D, const float *dt_bias, int dt_softplus,
                   const void *z, const float *initial_state, float *final_state, void *y,
                   ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                   int nheads, int headdim, int dstate, int ngroups, int chunk,
                   void *workspace, size_t workspace_bytes, void *hip_stream);
/*
 * ssd_prefill_ex with the sequence inputs read in place from wider token rows, so
 * that a Mamba-2 layer needs no copies between its projections and the SSD core
 * ("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A: the
 * input projection yields z, x, B, C and the step sizes side by side for each token).
 * x, B and C can then point into the convolved [x | B | C] rows and dt and z into the
 * input-projection rows; each is read as [B, L, ...] with consecutive tokens the given
 * number of elements apart, and batches L tokens apart (token (b, t) of x starts at
 * x + (b * L + t) * x_stride).
 *
 *   x_stride    >= H * P     (0: H * P, dense)
 *   bc_stride   >= G * N     B and C share it (0: G * N)
 *   dt_stride   >= H         (0: H)
 *   z_stride    >= H * P     (0: H * P; unused without z)
 * x, B and C are read with 16-byte loads: their pointers must be 16-byte aligned and
 * x_stride and bc_stride whole multiples of 16 bytes (8 bf16 or 4 fp32 elements).
 * y, the states and the workspace are as in ssd_prefill_ex (y dense [B, L, H, P]).
 * Errors: SSD_ERR_INVALID_ARG for a stride below its dense row or misaligned;
 * SSD_ERR_UNSUPPORTED when chunk * stride * element size reaches 2^31 bytes (one
 * chunk is addressed with 32-bit offsets).  ssd_prefill_ex is this call with all
 * four strides 0.
 */
int ssd_prefill_strided(const void *x, const void *dt, const float *A, const void *Bm,
                        const void *Cm, const float *D, const float *dt_bias, int dt_softplus,
                        const void *z, const float *initial_state, float *final_state, void *y,
                        ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                        int nheads, int headdim, int dstate, int ngroups, int chunk,
                        long long x_stride, long long bc_stride, long long dt_stride,
                        long long z_stride, void *workspace, size_t workspace_bytes,
                        void *hip_stream);
/*
 * Test and diagnostic entry point: ssd_prefill_strided on a path of the caller's choice,
 * with the bound of the waits between workgroups set by the caller.
 *   path        SSD_PATH_AUTO (the library's choice, as ssd_prefill_strided),
 *               SSD_PATH_STAGED (three launches), SSD_PATH_ONE_ROUND, SSD_PATH_SINGLE_PASS,
 *               or SSD_PATH_STAGED_ONE_HEAD (three launches with one head per chunk-state
 *               workgroup: the same result as SSD_PATH_STAGED and SSD_PATH_ONE_ROUND bit for
 *               bit, from other kernels); a path whose conditions (see ssd_prefill) do not
 *               hold returns SSD_ERR_UNSUPPORTED.
 *   spin_limit  < 0: the default bound; >= 0: polls per wait before it gives up (0: every
 *               wait gives up at once -- the output is then not valid and
 *               ssd_prefill_check returns SSD_ERR_SYNC; for tests of that report).
 */
enum {
    SSD_PATH_AUTO = 0,
    SSD_PATH_STAGED = 1,
    SSD_PATH_ONE_ROUND = 2,
    SSD_PATH_SINGLE_PASS = 3,
    SSD_PATH_STAGED_ONE_HEAD = 4
};
int ssd_prefill_forced(const void *x, const void *dt, const float *A, const void *Bm,
                       const void *Cm, const float *D, const float *dt_bias, int dt_softplus,
                       const void *z, const float *initial_state, float *final_state, void *y,
                       ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                       int nheads, int headdim, int dstate, int ngroups, int chunk,
                       long long x_stride, long long bc_stride, long long dt_stride,
                       long long z_stride, void *workspace, size_t workspace_bytes,
                       void *hip_stream, int path, long long spin_limit);
/*
 * Measurement entry point: ssd_prefill_forced with each kernel launch of the call timed
 * on the device.  Launch i (in the order the call enqueues them) is made with
 * start_events[i] and stop_events[i] bound to the kernel itself (HIP's launch-with-events
 * extension), so hipEventElapsedTime(start_events[i], stop_events[i]) is that kernel's own
 * execution time, and the stop event of one launch and the start event of the next bound
 * the gap between them; no marker is enqueued between launches.  The results are those
 * of ssd_prefill_forced with the same arguments.
 *   start_events, stop_events  hipEvent_t[capacity], created by the caller with timing
 *                              enabled (owned by the caller; each call rebinds them)
 *   kernel_names               const char *[capacity] or NULL: receives the name of each
 *                              timed launch's kernel (static strings of the library)
 *   capacity                   >= 0; launches past it run untimed
 *   n_launches                 NULL, or receives the number of kernel launches the call made
 * Errors: those of ssd_prefill_forced; SSD_ERR_INVALID_ARG for capacity < 0 or a NULL
 * array or event within capacity.  The timing is per calling thread and lasts for the
 * call only.
 */
int ssd_prefill_timed(const void *x, const void *dt, const float *A, const void *Bm,
                      const void *Cm, const float *D, const float *dt_bias, int dt_softplus,
                      const void *z, const float *initial_state, float *final_state, void *y,
                      ssd_dtype_t in_dtype, ssd_dtype_t y_dtype, int batch, int seqlen,
                      int nheads, int headdim, int dstate, int ngroups, int chunk,
                      long long x_stride, long long bc_stride, long long dt_stride,
                      long long z_stride, void *workspace, size_t workspace_bytes,
                      void *hip_stream, int path, long long spin_limit,
                      void *const *start_events, void *const *stop_events,
                      const char **kernel_names, int capacity, int *n_launches);
/*
 * Whether the last prefill that used `workspace` completed its waits between workgroups
 * (a prefill with seqlen == 0 does not touch the workspace and is not that prefill).
 * Synchronises `hip_stream` (so call it after the prefill was enqueued there), then reads
 * the workspace's give-up word: SSD_OK, or SSD_ERR_SYNC when a bounded wait gave up and
 * that prefill's y and final_state are not valid.  SSD_ERR_WORKSPACE for a NULL,
 * misaligned or too small (< 256 bytes) workspace; SSD_ERR_HIP if the synchronisation or
 * the read failed (e.g. a kernel fault).
 */
int ssd_prefill_check(const void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * ssd_prefill for callers that cannot allocate device memory -- code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: the same arguments without the
 * workspace.  The scratch comes from a device array inside the library of
 * SSD_PREFILL_NOALLOC_MAX_BYTES on each GPU it runs on (held until the process ends; its
 * address is looked up once per device on the first call there).  The call allocates
 * nothing.  It runs the three-launch path (no waits between workgroups), whose y and
 * final_state equal ssd_prefill's bit for bit.
 * Errors: as ssd_prefill, plus SSD_ERR_WORKSPACE when ssd_prefill_workspace_size(...) for
 * the shape exceeds SSD_PREFILL_NOALLOC_MAX_BYTES.  Every call on one GPU uses that GPU's
 * one array: calls that may overlap in time on one GPU (streams with no ordering between
 * them) race and give undefined results.
 */
#define SSD_PREFILL_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int ssd_prefill_noalloc(const void *x, const void *dt, const float *A, const void *Bm,
                        const void *Cm, const float *D, const float *initial_state,
                        float *final_state, float *y, ssd_dtype_t in_dtype, int batch,
                        int seqlen, int nheads, int headdim, int dstate, int ngroups,
                        int chunk, void *hip_stream);

/*
 * One decode token for every (b, h), fused ("Compiler-First State Space Duality and
 * Portable O(1) Autoregressive Caching for Inference", abstract: cached O(1) decode carries
 * the recurrent state from token to token; "Mamba-Family State-Space Model Kernels on a
 * Programmable CGLA", Sec. III-A: the per-token recurrence with a diagonal decay): the state is read once,
 * decayed, updated with the token's input and written back in place, and
 * the output is read off the updated state.
 *
 *   state [B, H, P, N] fp32 (in/out)   x [B, H, P] in_dtype   dt [B, H] in_dtype
 *   A [H] fp32   Bm, Cm [B, G, N] in_dtype   D [H] fp32 or NULL   y [B, H, P] fp32
 */
int ssd_step(float *state, const void *x, const void *dt, const float *A,
             const void *Bm, const void *Cm, const float *D, float *y,
             ssd_dtype_t in_dtype, int batch, int nheads, int headdim, int dstate,
             int ngroups, void *hip_stream);
/*
 * ssd_step with the options of ssd_prefill_ex: dt_bias [H] fp32 or NULL,
 * dt_softplus, z [B, H, P] in_dtype or NULL, y [B, H, P] in y_dtype.
 */
int ssd_step_ex(float *state, const void *x, const void *dt, const float *A,
                const void *Bm, const void *Cm, const float *D, const float *dt_bias,
                int dt_softplus, const void *z, void *y, ssd_dtype_t in_dtype,
                ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int dstate,
                int ngroups, void *hip_stream);
/*
 * ssd_step_ex with a decode token's inputs read in place from wider rows, as
 * ssd_prefill_strided does for a sequence: x, B and C from the convolution step's
 * [x | B | C] row of each batch entry, dt and z from its input-projection row.  The
 * strides are the elements between consecutive batch entries (0: dense):
 *   x_stride >= H * P, bc_stride >= G * N (B and C share it), dt_stride >= H,
 *   z_stride >= H * P.
 * The step reads its inputs element by element: pointers need only their element's
 * alignment.  y is dense [B, H, P].  Errors: SSD_ERR_INVALID_ARG for a stride below
 * its dense row; SSD_ERR_UNSUPPORTED for a stride of 2^31 elements or more.
 * ssd_step_ex is this call with all four strides 0.
 */
int ssd_step_strided(float *state, const void *x, const void *dt, const float *A,
                     const void *Bm, const void *Cm, const float *D, const float *dt_bias,
                     int dt_softplus, const void *z, void *y, ssd_dtype_t in_dtype,
                     ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int dstate,
                     int ngroups, long long x_stride, long long bc_stride,
                     long long dt_stride, long long z_stride, void *hip_stream);

/*
 * A decode loop of `nsteps` tokens captured once as a HIP graph and replayed
 * with one launch ("Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference", abstract: the autoregressive loop is
 * compiled to run on the device, carrying the cached state from token to
 * token).  Token t is ssd_step_ex on slot t of step-major buffers
 *
 *   x, z [nsteps, B, H, P] in_dtype   dt [nsteps, B, H] in_dtype
 *   Bm, Cm [nsteps, B, G, N] in_dtype   y [nsteps, B, H, P] y_dtype (written)
 *
 * with state [B, H, P, N] fp32 updated in place token after token, and A, D,
 * dt_bias, dt_softplus as in ssd_step_ex.  The graph holds the pointers, not the
 * values: the caller may rewrite the inputs and the state between launches, and
 * keeps every buffer allocated until ssd_decode_graph_destroy.
 *
 * ssd_decode_graph_create validates like ssd_step_ex (plus 1 <= nsteps <=
 * SSD_DECODE_GRAPH_MAX_STEPS), captures the tokens on a private stream of the
 * current device and stores the handle in *out (NULL on any error).  It
 * allocates the graph objects (host memory, and the HIP runtime's own kernel
 * argument storage); nothing is launched.  SSD_ERR_HIP: capture or
 * instantiation failed.
 * ssd_decode_graph_launch enqueues the nsteps tokens on hip_stream, after the
 * work already queued there.  The current device must be the one the handle
 * was created on (else SSD_ERR_INVALID_ARG).  Launches of one handle write the
 * same state and y: launches that may overlap in time (different streams with
 * no ordering between them) race.
 * ssd_decode_graph_steps returns nsteps (0 for NULL).
 * ssd_decode_graph_destroy frees the handle (NULL: no-op); call it once no
 * launch of the handle is pending.
 */
#define SSD_DECODE_GRAPH_MAX_STEPS 65536
typedef struct ssd_decode_graph ssd_decode_graph;
int ssd_decode_graph_create(ssd_decode_graph **out, int nsteps, float *state, const void *x,
                            const void *dt, const float *A, const void *Bm, const void *Cm,
                            const float *D, const float *dt_bias, int dt_softplus,
                            const void *z, void *y, ssd_dtype_t in_dtype, ssd_dtype_t y_dtype,
                            int batch, int nheads, int headdim, int dstate, int ngroups);
int ssd_decode_graph_launch(ssd_decode_graph *g, void *hip_stream);
int ssd_decode_graph_steps(const ssd_decode_graph *g);
int ssd_decode_graph_destroy(ssd_decode_graph *g);

/* ---- Stage entry points (the kernels ssd_prefill runs, in this order: chunk_cumsum +
 *      chunk_state + chunk_gemm1 in one launch, state_passing, chunk_scan).  The chunk
 *      and entering states between them are fp16 for bf16 inputs and fp32 for fp32 inputs. ---- */

/*
 * Step-0: per-chunk inclusive cumulative sum of dt*A (wavefront prefix scan).
 *   dt [B, L, H] in_dtype; A [H] fp32
 *   dA_cum [B, H, nc, Q] fp32 (written): sum_{k<=i} dt[cQ+k]*A[h], held
 *          constant past seqlen; dt_c [B, H, nc, Q] fp32 (written): dt, 0 past seqlen.
 */
int ssd_chunk_cumsum(const void *dt, const float *A, float *dA_cum, float *dt_c,
                     ssd_dtype_t in_dtype, int batch, int seqlen, int nheads,
                     int chunk, void *hip_stream);

/*
 * Step-2: chunk states, the state each chunk alone leaves from a zero start:
 *   states[b,h,c] = sum_j exp(dA_cum[c][Q-1] - dA_cum[c][j]) * dt_c[c][j] * x_j B_j^T
 *   x [B, L, H, P], Bm [B, L, G, N] in_dtype; dA_cum, dt_c as written by
 *   ssd_chunk_cumsum; states [B, H, nc, P, N] (written): fp32 accumulation, stored
 *   fp32 for fp32 inputs and rounded once to fp16 for bf16 inputs.
 */
int ssd_chunk_state(const void *x, const void *Bm, const float *dA_cum, const float *dt_c,
                    void *states, ssd_dtype_t in_dtype, int batch, int seqlen,
                    int nheads, int headdim, int dstate, int ngroups, int chunk,
                    void *hip_stream);

/*
 * Step-3: inter-chunk state passing, sequential over chunks, in place:
 *   run = initial_state (or 0); for c: tmp = states[c]; states[c] = run;
 *   run = exp(dA_cum[c][Q-1]) * run + tmp.   final_state = run (if non-NULL;
 *   may alias initial_state).  On return states[c] holds the state entering chunk c.
 *   states [B, H, nc, P, N]: fp16 when in_dtype is SSD_BF16, fp32 when SSD_F32 (the
 *   type ssd_chunk_state writes for that input type); the carry `run` is fp32 and
 *   each entering state is rounded once when stored.
 */
int ssd_state_passing(void *states, const float *dA_cum, const float *initial_state,
                      float *final_state, ssd_dtype_t in_dtype, int batch, int nheads,
                      int headdim, int dstate, int nchunks, int chunk, void *hip_stream);

/*
 * Step-1 GEMM1 ("Mamba-Family State-Space Model Kernels on a Programmable
 * CGLA", Sec. III-A): the products G_c[i, j] = C_i . B_j of chunk-local
 * tokens j <= i, once per (batch, group, chunk) -- every head of a group
 * shares them.
 *   Bm, Cm [B, L, G, N] in_dtype; cb (written): ssd_chunk_gemm1_size(...)
 *   bytes, 16-byte aligned, an opaque fp32 layout read by ssd_chunk_scan
 *   (tile order of the matrix-core accumulators; entries above the diagonal
 *   are unused).
 */
size_t ssd_chunk_gemm1_size(int batch, int seqlen, int ngroups, int chunk);
int ssd_chunk_gemm1(const void *Bm, const void *Cm, float *cb, ssd_dtype_t in_dtype,
                    int batch, int seqlen, int dstate, int ngroups, int chunk,
                    void *hip_stream);
/*
 * Step-1 mask + GEMM2, Step-4 and skip: the output of every chunk,
 *   y_i = sum_{j<=i} G_c[i, j] exp(dA_cum[i] - dA_cum[j]) dt_c[j] x_j        (intra-chunk)
 *       + exp(dA_cum[i]) * H_enter C_i  + D_h x_i                           (off-diagonal, skip)
 *   cb: ssd_chunk_gemm1 output for the same B/C; h_enter [B, H, nc, P, N]: the
 *   entering states (ssd_state_passing output), fp16 for bf16 inputs and fp32 for
 *   fp32 inputs; y [B, L, H, P] fp32 (written).
 */
int ssd_chunk_scan(const void *x, const void *Cm, const float *cb, const float *dA_cum,
                   const float *dt_c, const void *h_enter, const float *D, float *y,
                   ssd_dtype_t in_dtype, int batch, int seqlen, int nheads, int headdim,
                   int dstate, int ngroups, int chunk, void *hip_stream);

/*
 * Step-3 and the chunk scan in one launch, for problems whose (b, h, chunk)
 * items all fit the device at once (the two-launch ssd_prefill path):
 * bf16 inputs, Q = 256, P = 64, nc <= 16 and B*H*nc <= 2 x compute units;
 * any other shape returns SSD_ERR_UNSUPPORTED.  The result equals
 * ssd_state_passing followed by ssd_chunk_scan bit for bit.
 *   states [B, H, nc, P, N] fp16: the chunk states (ssd_chunk_state output) on
 *          entry, the entering states on exit
 *   initial_state / final_state: as in ssd_state_passing (NULL allowed)
 *   sync   B*H*64 uint32 (256 bytes per (b, h)), ZERO on entry; each (b, h)
 *          counter holds nc on exit.  The launch's workgroups of one (b, h) wait
 *          for each other through it, which needs them resident together (the call
 *          checks the kernel's occupancy on the device: SSD_ERR_UNSUPPORTED if it cannot
 *          hold the grid).  The wait is bounded: a workgroup that gives up sets bit 31 of
 *          its head's counter, and y and the states of that head are then not valid.
 *   Other arguments as ssd_chunk_scan; y [B, L, H, P] fp32 (written).
 */
int ssd_chunk_scan_passing(const void *x, const void *Cm, const float *cb, const float *dA_cum,
                           const float *dt_c, void *states, const float *initial_state,
                           float *final_state, const float *D, float *y, unsigned *sync,
                           ssd_dtype_t in_dtype, int batch, int seqlen, int nheads, int headdim,
                           int dstate, int ngroups, int chunk, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_SCAN_AMD_SSD_H */
