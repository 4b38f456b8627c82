"""Python binding of the C ABI in ``include/ssd.h`` (``libssd.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The
library must have been built (``python -m mamba_ssd_scan_amd.build`` or
``__graft_entry__.build()``); importing a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_F32, SSD_BF16, SSD_FP8_E4M3 = 0, 1, 2
SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, SSD_ERR_SYNC = 0, -1, -2, -3, -4, -5

# Every symbol include/ssd.h declares.
EXPORTS = ("ssd_status_string", "ssd_version", "ssd_prefill_workspace_size", "ssd_prefill", "ssd_step",
           "ssd_prefill_ex", "ssd_prefill_strided", "ssd_prefill_forced", "ssd_prefill_timed", "ssd_prefill_check",
           "ssd_prefill_noalloc",
           "ssd_step_ex", "ssd_step_strided",
           "ssd_decode_graph_create", "ssd_decode_graph_launch", "ssd_decode_graph_steps", "ssd_decode_graph_destroy",
           "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_gemm1_size",
           "ssd_chunk_gemm1", "ssd_chunk_scan", "ssd_chunk_scan_passing")


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -m mamba_ssd_scan_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.ssd_status_string.argtypes = [i]
    L.ssd_status_string.restype = ctypes.c_char_p
    L.ssd_version.argtypes = []
    L.ssd_version.restype = i
    L.ssd_prefill_workspace_size.argtypes = [i] * 7
    L.ssd_prefill_workspace_size.restype = sz
    L.ssd_prefill.argtypes = [vp] * 9 + [i] * 8 + [vp, sz, vp]
    L.ssd_prefill.restype = i
    L.ssd_step.argtypes = [vp] * 8 + [i] * 6 + [vp]
    L.ssd_step.restype = i
    L.ssd_prefill_ex.argtypes = [vp] * 7 + [i] + [vp] * 4 + [i] * 9 + [vp, sz, vp]
    L.ssd_prefill_ex.restype = i
    ll = ctypes.c_longlong
    L.ssd_prefill_strided.argtypes = [vp] * 7 + [i] + [vp] * 4 + [i] * 9 + [ll] * 4 + [vp, sz, vp]
    L.ssd_prefill_strided.restype = i
    L.ssd_prefill_forced.argtypes = [vp] * 7 + [i] + [vp] * 4 + [i] * 9 + [ll] * 4 + [vp, sz, vp, i, ll]
    L.ssd_prefill_forced.restype = i
    L.ssd_prefill_timed.argtypes = ([vp] * 7 + [i] + [vp] * 4 + [i] * 9 + [ll] * 4 + [vp, sz, vp, i, ll]
                                    + [vp, vp, vp, i, ctypes.POINTER(i)])
    L.ssd_prefill_timed.restype = i
    L.ssd_prefill_check.argtypes = [vp, sz, vp]
    L.ssd_prefill_check.restype = i
    L.ssd_prefill_noalloc.argtypes = [vp] * 9 + [i] * 8 + [vp]
    L.ssd_prefill_noalloc.restype = i
    L.ssd_step_ex.argtypes = [vp] * 8 + [i] + [vp] * 2 + [i] * 7 + [vp]
    L.ssd_step_ex.restype = i
    L.ssd_step_strided.argtypes = [vp] * 8 + [i] + [vp] * 2 + [i] * 7 + [ctypes.c_longlong] * 4 + [vp]
    L.ssd_step_strided.restype = i
    L.ssd_decode_graph_create.argtypes = [ctypes.POINTER(vp), i] + [vp] * 8 + [i] + [vp] * 2 + [i] * 7
    L.ssd_decode_graph_create.restype = i
    L.ssd_decode_graph_launch.argtypes = [vp, vp]
    L.ssd_decode_graph_launch.restype = i
    L.ssd_decode_graph_steps.argtypes = [vp]
    L.ssd_decode_graph_steps.restype = i
    L.ssd_decode_graph_destroy.argtypes = [vp]
    L.ssd_decode_graph_destroy.restype = i
    L.ssd_chunk_cumsum.argtypes = [vp] * 4 + [i] * 5 + [vp]
    L.ssd_chunk_cumsum.restype = i
    L.ssd_chunk_state.argtypes = [vp] * 5 + [i] * 8 + [vp]
    L.ssd_chunk_state.restype = i
    L.ssd_state_passing.argtypes = [vp] * 4 + [i] * 7 + [vp]
    L.ssd_state_passing.restype = i
    L.ssd_chunk_gemm1_size.argtypes = [i] * 4
    L.ssd_chunk_gemm1_size.restype = sz
    L.ssd_chunk_gemm1.argtypes = [vp] * 3 + [i] * 6 + [vp]
    L.ssd_chunk_gemm1.restype = i
    L.ssd_chunk_scan.argtypes = [vp] * 8 + [i] * 8 + [vp]
    L.ssd_chunk_scan.restype = i
    L.ssd_chunk_scan_passing.argtypes = [vp] * 11 + [i] * 8 + [vp]
    L.ssd_chunk_scan_passing.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().ssd_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SSD_OK:
        raise SsdError(status, where)


# ---------------------------------------------------------------------------
# torch-facing wrappers


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.float8_e4m3fn:
        return SSD_FP8_E4M3
    raise TypeError(f"inputs must be bfloat16, float32 or float8_e4m3fn, got {t.dtype}")


def _check_types(x, dt, B, C, z=None) -> int:
    """The input dtype code: B and C share x's dtype; dt and z too, except beside float8_e4m3fn
    x, B and C, where they are bfloat16."""
    torch = _torch()
    code = _dtype_code(x)
    for t in (B, C):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, B and C must share one dtype")
    want = torch.bfloat16 if code == SSD_FP8_E4M3 else x.dtype
    for t in (dt, z):
        if t is not None and t.dtype != want:
            raise TypeError("dt and z must share x's dtype (bfloat16 beside float8_e4m3fn x, B and C)")
    return code


def _y_code(y_dtype) -> int:
    torch = _torch()
    if y_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"y must be float32 or bfloat16, got {y_dtype}")
    return _dtype_code(torch.empty(0, dtype=y_dtype))


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def _token_stride(t, name: str) -> int:
    """Elements between consecutive tokens of a [B, L, ...] sequence input.

    Each token's values must be contiguous; the tokens may sit in wider rows (a view
    into a buffer holding other channels too), with batches L tokens apart.
    """
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    shape, st = t.shape, t.stride()
    if t.numel() == 0:  # nothing is read: treat as dense
        tail = 1
        for v in shape[2:]:
            tail *= v
        return tail
    tail = 1
    for k in range(t.dim() - 1, 1, -1):
        if shape[k] != 1 and st[k] != tail:
            raise ValueError(f"{name}: the values of one token must be contiguous (strides {st})")
        tail *= shape[k]
    b, l = shape[0], shape[1]
    ts = st[1] if l > 1 else (st[0] if b > 1 else tail)
    if b > 1 and st[0] != l * ts:
        raise ValueError(f"{name}: batches must be seqlen tokens apart (strides {st})")
    return ts


def _seq_strides(x, dt, B, C, z):
    """Token strides (x, B and C, dt, z) and whether all are dense."""
    sx, sb, sc = _token_stride(x, "x"), _token_stride(B, "B"), _token_stride(C, "C")
    sd, sz = _token_stride(dt, "dt"), _token_stride(z, "z")
    if sb != sc:
        raise ValueError("B and C must have the same token stride")
    hp, gn = x.shape[2] * x.shape[3], B.shape[2] * B.shape[3]
    dense = sx == hp and sb == gn and sd == x.shape[2] and (z is None or sz == hp)
    return (sx, sb, sd, sz), dense


def _batch_stride(t, name: str) -> int:
    """Elements between consecutive batch entries of a [B, ...] decode input whose per-entry
    values are contiguous (a view into wider rows is fine)."""
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    shape, st = t.shape, t.stride()
    tail = 1
    for k in range(t.dim() - 1, 0, -1):
        if shape[k] != 1 and st[k] != tail:
            raise ValueError(f"{name}: the values of one batch entry must be contiguous (strides {st})")
        tail *= shape[k]
    return st[0] if shape[0] > 1 and t.numel() > 0 else tail


def _step_strides(x, dt, B, C, z):
    """Batch strides (x, B and C, dt, z) and whether all are dense."""
    sx, sb, sc = _batch_stride(x, "x"), _batch_stride(B, "B"), _batch_stride(C, "C")
    sd, sz = _batch_stride(dt, "dt"), _batch_stride(z, "z")
    if sb != sc:
        raise ValueError("B and C must have the same batch stride")
    hp, gn = x.shape[1] * x.shape[2], B.shape[1] * B.shape[2]
    dense = sx == hp and sb == gn and sd == x.shape[1] and (z is None or sz == hp)
    return (sx, sb, sd, sz), dense


def _f32(*ts):
    torch = _torch()
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise TypeError("A, D, states, workspace views and outputs must be float32")


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def nchunks(seqlen: int, chunk: int) -> int:
    return -(-seqlen // chunk)


def workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk) -> int:
    n = lib().ssd_prefill_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
    if n == 0 and seqlen > 0:
        raise SsdError(SSD_ERR_UNSUPPORTED, "ssd_prefill_workspace_size")
    return n


def alloc_workspace(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, device="cuda"):
    torch = _torch()
    n = workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


PATH_AUTO, PATH_STAGED, PATH_ONE_ROUND, PATH_SINGLE_PASS, PATH_STAGED_ONE_HEAD = 0, 1, 2, 3, 4


def _on_stream(stream):
    """Context in which the wrappers allocate: the caller's stream when one is given, so that
    the caching allocator does not hand the memory (the workspace above all) to other work
    while the kernels on that stream still use it."""
    import contextlib
    torch = _torch()
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _prefill(x, dt, A, B, C, D, initial_state, dt_bias, dt_softplus, z, y_dtype, chunk, y, final_state, workspace,
             stream, path, spin_limit, plain, timing=None):
    torch = _torch()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    code = _check_types(x, dt, B, C, z)
    y_dtype = torch.float32 if y_dtype is None else y_dtype
    ycode = _y_code(y_dtype)
    strides, dense = _seq_strides(x, dt, B, C, z)  # views into wider token rows are read in place
    _dev(A, D, initial_state, y, workspace, dt_bias)
    _f32(A, D, initial_state, dt_bias)
    with _on_stream(stream):
        if y is None:
            y = torch.empty((batch, seqlen, nheads, headdim), dtype=y_dtype, device=x.device)
        elif y.dtype != y_dtype:
            raise TypeError("y does not have y_dtype")
        if isinstance(final_state, str):
            final_state = torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = alloc_workspace(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, x.device)
    _dev(final_state)
    _f32(final_state)
    wbytes = workspace.numel() * workspace.element_size()
    shape = (batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
    opts = (_ptr(dt_bias), int(bool(dt_softplus)), _ptr(z))
    ins = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D))
    if timing is not None:
        starts, stops, names, n = timing
        _check(lib().ssd_prefill_timed(*ins, *opts, _ptr(initial_state), _ptr(final_state), _ptr(y), code, ycode,
                                       *shape, *strides, _ptr(workspace), wbytes, _stream(stream), int(path),
                                       -1 if spin_limit is None else int(spin_limit), starts, stops, names,
                                       len(starts), ctypes.byref(n)), "ssd_prefill_timed")
    elif path != PATH_AUTO or spin_limit is not None:
        _check(lib().ssd_prefill_forced(*ins, *opts, _ptr(initial_state), _ptr(final_state), _ptr(y), code, ycode,
                                        *shape, *strides, _ptr(workspace), wbytes, _stream(stream), int(path),
                                        -1 if spin_limit is None else int(spin_limit)), "ssd_prefill_forced")
    elif not dense:
        _check(lib().ssd_prefill_strided(*ins, *opts, _ptr(initial_state), _ptr(final_state), _ptr(y), code, ycode,
                                         *shape, *strides, _ptr(workspace), wbytes, _stream(stream)),
               "ssd_prefill_strided")
    elif plain:
        _check(lib().ssd_prefill(*ins, _ptr(initial_state), _ptr(final_state), _ptr(y), code, *shape,
                                 _ptr(workspace), wbytes, _stream(stream)), "ssd_prefill")
    else:
        _check(lib().ssd_prefill_ex(*ins, *opts, _ptr(initial_state), _ptr(final_state), _ptr(y), code, ycode,
                                    *shape, _ptr(workspace), wbytes, _stream(stream)), "ssd_prefill_ex")
    return y, final_state


def prefill(x, dt, A, B, C, D=None, initial_state=None, *, chunk: int = 256, y=None, final_state="new",
            workspace=None, stream=None, path=PATH_AUTO, spin_limit=None) -> Tuple[object, Optional[object]]:
    """Chunked SSD prefill.  Returns (y [B,L,H,P] fp32, final_state [B,H,P,N] fp32 or None).

    x, dt, B and C may be views into wider token rows (e.g. slices of a layer's
    projection output): they are then read in place through ssd_prefill_strided.

    ``final_state``: "new" allocates it, None skips it, or pass a tensor
    (which may be ``initial_state`` itself for an in-place update).
    ``path`` / ``spin_limit`` (tests and diagnostics): run through ssd_prefill_forced on the
    given path (PATH_*) with the given bound of the waits between workgroups.
    """
    if y is not None:
        _f32(y)
    return _prefill(x, dt, A, B, C, D, initial_state, None, False, None, None, chunk, y, final_state, workspace,
                    stream, path, spin_limit, plain=True)


def prefill_ex(x, dt, A, B, C, D=None, initial_state=None, *, dt_bias=None, dt_softplus=False, z=None,
               y_dtype=None, chunk: int = 256, y=None, final_state="new", workspace=None, stream=None,
               path=PATH_AUTO, spin_limit=None):
    """ssd_prefill_ex: prefill with dt = softplus(dt + dt_bias) (or dt + dt_bias), the z gate
    y * z * sigmoid(z), and y stored as float32 or bfloat16 (``y_dtype``, default float32).
    Returns (y, final_state or None)."""
    return _prefill(x, dt, A, B, C, D, initial_state, dt_bias, dt_softplus, z, y_dtype, chunk, y, final_state,
                    workspace, stream, path, spin_limit, plain=False)


class LaunchEvents:
    """Event pairs for prefill_timed: ``pairs`` (start, stop) HIP timing events, created through
    the HIP runtime that libssd.so links with the flag hipEventDisableSystemFence.  An event
    bound to a launch otherwise gives that kernel a system-scope release (a write-back and
    invalidation of the L2s at its end), which plain back-to-back launches on a stream do not
    pay: with the flag a timed kernel runs as it does untimed.  Read the times after a
    synchronisation of the device (the events themselves do not synchronise-with the work)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, pairs: int):
        rt = lib()  # its dependency, the HIP runtime, resolves the hipEvent* symbols
        self._rt = rt
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventCreateWithFlags.restype = ctypes.c_int
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventElapsedTime.restype = ctypes.c_int
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        rt.hipEventDestroy.restype = ctypes.c_int
        arr = ctypes.c_void_p * pairs
        self._starts, self._stops = arr(), arr()
        for a in (self._starts, self._stops):
            for i in range(pairs):
                e = ctypes.c_void_p()
                r = rt.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
                if r != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({r})")
                a[i] = e.value
        self._names = (ctypes.c_char_p * pairs)()
        self._n = ctypes.c_int(0)
        self.pairs = pairs
        self.names = []

    def __del__(self):
        rt = getattr(self, "_rt", None)
        if rt is None:
            return
        for a in (self._starts, self._stops):
            for e in a:
                if e:
                    rt.hipEventDestroy(e)

    def _args(self):
        return self._starts, self._stops, self._names, self._n

    def _done(self):
        k = min(self._n.value, self.pairs)
        self.names = [self._names[i].decode() for i in range(k)]
        return self._n.value

    def _ms(self, a, b):
        t = ctypes.c_float()
        r = self._rt.hipEventElapsedTime(ctypes.byref(t), a, b)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return t.value

    def durations_ms(self):
        """Per timed launch of the last call: its kernel's execution time in ms."""
        return [self._ms(self._starts[i], self._stops[i]) for i in range(len(self.names))]

    def gaps_ms(self):
        """Between consecutive timed launches of the last call: end of one to start of the next."""
        return [self._ms(self._stops[i], self._starts[i + 1]) for i in range(len(self.names) - 1)]

    def span_ms(self):
        """First timed launch's start to the last one's end."""
        return self._ms(self._starts[0], self._stops[len(self.names) - 1])

    def since_ms(self, other: "LaunchEvents"):
        """End of ``other``'s last timed launch to the start of this call's first."""
        return self._ms(other._stops[len(other.names) - 1], self._starts[0])


def prefill_timed(x, dt, A, B, C, D=None, initial_state=None, *, events: LaunchEvents, dt_bias=None,
                  dt_softplus=False, z=None, y_dtype=None, chunk: int = 256, y=None, final_state="new",
                  workspace=None, stream=None, path=PATH_AUTO, spin_limit=None):
    """ssd_prefill_timed: prefill_ex (on the path ``path``) with each kernel launch bound to the
    next event pair of ``events``.  Returns (y, final_state or None, launches made); after a
    synchronisation, ``events.names`` and ``events.durations_ms()`` hold each timed launch's
    kernel and its execution time."""
    if y is not None and y_dtype is None:
        _f32(y)
    r = _prefill(x, dt, A, B, C, D, initial_state, dt_bias, dt_softplus, z, y_dtype, chunk, y, final_state,
                 workspace, stream, path, spin_limit, plain=False, timing=events._args())
    return r[0], r[1], events._done()


NOALLOC_MAX_BYTES = 64 << 20  # SSD_PREFILL_NOALLOC_MAX_BYTES


def prefill_noalloc(x, dt, A, B, C, D=None, initial_state=None, *, chunk: int = 256, y, final_state=None,
                    stream=None):
    """ssd_prefill_noalloc: the prefill with the library's own scratch (no workspace, nothing
    allocated by the library).  y [B,L,H,P] fp32 and final_state (or None) are the caller's;
    x, dt, B and C must be dense.  Returns (y, final_state)."""
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    code = _check_types(x, dt, B, C)
    for t in (x, dt, B, C):
        if not t.is_contiguous():
            raise TypeError("x, dt, B and C must be dense")
    _dev(A, D, initial_state, y, final_state)
    _f32(A, D, initial_state, y, final_state)
    _check(lib().ssd_prefill_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state),
                                     _ptr(final_state), _ptr(y), code, batch, seqlen, nheads, headdim, dstate,
                                     ngroups, chunk, _stream(stream)), "ssd_prefill_noalloc")
    return y, final_state


def prefill_check(workspace, stream=None) -> int:
    """ssd_prefill_check: synchronise ``stream`` and return SSD_OK, or SSD_ERR_SYNC when a bounded
    wait of the last prefill on ``workspace`` gave up (its output is then not valid)."""
    return int(lib().ssd_prefill_check(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def step_ex(state, x, dt, A, B, C, D=None, *, dt_bias=None, dt_softplus=False, z=None, y_dtype=None, y=None,
            stream=None):
    """ssd_step_ex: one decode token with the options of prefill_ex; ``state`` is updated in place."""
    torch = _torch()
    batch, nheads, headdim, dstate = state.shape
    ngroups = B.shape[1]
    code = _check_types(x, dt, B, C, z)
    y_dtype = torch.float32 if y_dtype is None else y_dtype
    ycode = _y_code(y_dtype)
    strides, dense = _step_strides(x, dt, B, C, z)  # views into wider rows are read in place
    _dev(state, A, D, y, dt_bias)
    _f32(state, A, D, dt_bias)
    if y is None:
        y = torch.empty((batch, nheads, headdim), dtype=y_dtype, device=x.device)
    if not dense:
        _check(lib().ssd_step_strided(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(dt_bias), int(bool(dt_softplus)), _ptr(z), _ptr(y), code, ycode, batch,
                                      nheads, headdim, dstate, ngroups, *strides, _stream(stream)), "ssd_step_strided")
        return y
    _check(lib().ssd_step_ex(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
                             int(bool(dt_softplus)), _ptr(z), _ptr(y), code, ycode, batch, nheads, headdim, dstate,
                             ngroups, _stream(stream)), "ssd_step_ex")
    return y


def step(state, x, dt, A, B, C, D=None, *, y=None, stream=None):
    """One fused decode token; ``state`` [B,H,P,N] fp32 is updated in place.  Returns y [B,H,P] fp32.

    x, dt, B and C may be views into wider per-entry rows (a layer's projection outputs):
    they are then read in place through ssd_step_strided."""
    torch = _torch()
    batch, nheads, headdim, dstate = state.shape
    ngroups = B.shape[1]
    code = _check_types(x, dt, B, C)
    strides, dense = _step_strides(x, dt, B, C, None)  # views into wider rows are read in place
    _dev(state, A, D, y)
    _f32(state, A, D, y)
    if y is None:
        y = torch.empty((batch, nheads, headdim), dtype=torch.float32, device=x.device)
    if not dense:
        _check(lib().ssd_step_strided(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), None, 0,
                                      None, _ptr(y), code, SSD_F32, batch, nheads, headdim, dstate, ngroups, *strides,
                                      _stream(stream)), "ssd_step_strided")
        return y
    _check(lib().ssd_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y), code,
                          batch, nheads, headdim, dstate, ngroups, _stream(stream)), "ssd_step")
    return y


class DecodeGraph:
    """ssd_decode_graph_*: ``nsteps`` decode tokens captured once as a HIP graph.

    Token t runs ssd_step_ex on slot t of the step-major inputs x [T,B,H,P], dt [T,B,H],
    B/C [T,B,G,N], z [T,B,H,P] and writes y [T,B,H,P]; ``state`` [B,H,P,N] is updated in
    place token after token.  The graph keeps the buffers' addresses: rewrite their
    contents between launches, never reallocate them.  The tensors are referenced here
    so they outlive the graph.
    """

    def __init__(self, state, x, dt, A, B, C, D=None, *, dt_bias=None, dt_softplus=False, z=None, y_dtype=None,
                 y=None):
        torch = _torch()
        self._handle = None
        nsteps, batch, nheads, headdim = x.shape
        dstate = state.shape[3]
        ngroups = B.shape[2]
        if tuple(state.shape) != (batch, nheads, headdim, dstate):
            raise ValueError("state must be [B,H,P,N] matching x [T,B,H,P]")
        if tuple(dt.shape) != (nsteps, batch, nheads) or tuple(B.shape) != (nsteps, batch, ngroups, dstate) \
                or tuple(C.shape) != tuple(B.shape) or (z is not None and tuple(z.shape) != tuple(x.shape)):
            raise ValueError("step-major inputs must be x [T,B,H,P], dt [T,B,H], B/C [T,B,G,N], z like x")
        code = _check_types(x, dt, B, C, z)
        y_dtype = torch.float32 if y_dtype is None else y_dtype
        ycode = _y_code(y_dtype)
        _dev(state, x, dt, A, B, C, D, y, dt_bias, z)
        _f32(state, A, D, dt_bias)
        if y is None:
            y = torch.empty(tuple(x.shape), dtype=y_dtype, device=x.device)
        elif tuple(y.shape) != tuple(x.shape) or y.dtype != y_dtype:
            raise ValueError("y must be [T,B,H,P] of y_dtype")
        self.y = y
        self._keep = (state, x, dt, A, B, C, D, dt_bias, z, y)
        self.device = x.device
        h = ctypes.c_void_p()
        with torch.cuda.device(x.device):
            _check(lib().ssd_decode_graph_create(ctypes.byref(h), nsteps, _ptr(state), _ptr(x), _ptr(dt), _ptr(A),
                                                 _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), int(bool(dt_softplus)),
                                                 _ptr(z), _ptr(y), code, ycode, batch, nheads, headdim, dstate,
                                                 ngroups), "ssd_decode_graph_create")
        self._handle = h
        self.nsteps = lib().ssd_decode_graph_steps(h)

    def launch(self, stream=None):
        """Enqueue the nsteps tokens on ``stream`` (default: the current stream); returns y."""
        if self._handle is None:
            raise RuntimeError("decode graph is closed")
        torch = _torch()
        with torch.cuda.device(self.device):
            _check(lib().ssd_decode_graph_launch(self._handle, _stream(stream)), "ssd_decode_graph_launch")
        return self.y

    def close(self):
        """Destroy the graph once no launch is pending (synchronises the device first)."""
        if self._handle is not None:
            torch = _torch()
            with torch.cuda.device(self.device):
                torch.cuda.synchronize()
                _check(lib().ssd_decode_graph_destroy(self._handle), "ssd_decode_graph_destroy")
            self._handle = None
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- stage entry points (for unit tests and per-kernel timing)


def chunk_cumsum(dt, A, *, chunk: int, acum=None, dtc=None, stream=None):
    torch = _torch()
    batch, seqlen, nheads = dt.shape
    nc = nchunks(seqlen, chunk)
    _dev(dt, A, acum, dtc)
    if acum is None:
        acum = torch.empty((batch, nheads, nc, chunk), dtype=torch.float32, device=dt.device)
    if dtc is None:
        dtc = torch.empty((batch, nheads, nc, chunk), dtype=torch.float32, device=dt.device)
    _check(lib().ssd_chunk_cumsum(_ptr(dt), _ptr(A), _ptr(acum), _ptr(dtc), _dtype_code(dt), batch, seqlen, nheads,
                                  chunk, _stream(stream)), "ssd_chunk_cumsum")
    return acum, dtc


def _state_dtype(x):
    """Element type of the chunk / entering states for inputs like ``x``."""
    torch = _torch()
    return torch.float32 if x.dtype == torch.float32 else torch.float16  # fp16 beside bf16 and fp8 inputs


def chunk_state(x, B, acum, dtc, *, chunk: int, states=None, stream=None):
    """Chunk states [B,H,nc,P,N]: float16 for bfloat16 inputs, float32 for float32 inputs."""
    torch = _torch()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    nc = nchunks(seqlen, chunk)
    _dev(x, B, acum, dtc, states)
    if states is None:
        states = torch.empty((batch, nheads, nc, headdim, dstate), dtype=_state_dtype(x), device=x.device)
    elif states.dtype != _state_dtype(x):
        raise TypeError(f"states must be {_state_dtype(x)} for {x.dtype} inputs")
    _check(lib().ssd_chunk_state(_ptr(x), _ptr(B), _ptr(acum), _ptr(dtc), _ptr(states), _dtype_code(x), batch, seqlen,
                                 nheads, headdim, dstate, ngroups, chunk, _stream(stream)), "ssd_chunk_state")
    return states


def state_passing(states, acum, initial_state=None, *, chunk: int, final_state="new", stream=None):
    """In place: ``states`` [B,H,nc,P,N] (float16 or float32) becomes the entering states.  Returns final_state."""
    torch = _torch()
    batch, nheads, nc, headdim, dstate = states.shape
    _dev(states, acum, initial_state)
    if states.dtype == torch.float16:
        code = SSD_BF16
    elif states.dtype == torch.float32:
        code = SSD_F32
    else:
        raise TypeError("states must be float16 (bfloat16 or float8_e4m3fn inputs) or float32 (float32 inputs)")
    if isinstance(final_state, str):
        final_state = torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=states.device)
    _check(lib().ssd_state_passing(_ptr(states), _ptr(acum), _ptr(initial_state), _ptr(final_state), code, batch,
                                   nheads, headdim, dstate, nc, chunk, _stream(stream)), "ssd_state_passing")
    return final_state


def chunk_gemm1_size(batch, seqlen, ngroups, chunk) -> int:
    n = lib().ssd_chunk_gemm1_size(batch, seqlen, ngroups, chunk)
    if n == 0 and seqlen > 0:
        raise SsdError(SSD_ERR_UNSUPPORTED, "ssd_chunk_gemm1_size")
    return n


def chunk_gemm1(B, C, *, chunk: int, cb=None, stream=None):
    """C.B^T products of every chunk, once per group (opaque fp32 buffer for chunk_scan)."""
    torch = _torch()
    batch, seqlen, ngroups, dstate = B.shape
    _dev(B, C, cb)
    if C.dtype != B.dtype:
        raise TypeError("B and C must share one dtype")
    if cb is None:
        cb = torch.empty(max(chunk_gemm1_size(batch, seqlen, ngroups, chunk) // 4, 4), dtype=torch.float32,
                         device=B.device)
    _check(lib().ssd_chunk_gemm1(_ptr(B), _ptr(C), _ptr(cb), _dtype_code(B), batch, seqlen, dstate, ngroups, chunk,
                                 _stream(stream)), "ssd_chunk_gemm1")
    return cb


def chunk_scan(x, C, cb, acum, dtc, h_enter, D=None, *, chunk: int, y=None, stream=None):
    """``h_enter`` [B,H,nc,P,N]: float16 for bfloat16 inputs, float32 for float32 inputs."""
    torch = _torch()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = C.shape[2], C.shape[3]
    _dev(x, C, cb, acum, dtc, h_enter, D, y)
    want = torch.float32 if x.dtype == torch.float32 else torch.float16
    if h_enter.dtype != want:
        raise TypeError(f"h_enter must be {want} for {x.dtype} inputs")
    if y is None:
        y = torch.empty((batch, seqlen, nheads, headdim), dtype=torch.float32, device=x.device)
    _check(lib().ssd_chunk_scan(_ptr(x), _ptr(C), _ptr(cb), _ptr(acum), _ptr(dtc), _ptr(h_enter), _ptr(D), _ptr(y),
                                _dtype_code(x), batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                _stream(stream)), "ssd_chunk_scan")
    return y


SYNC_WORDS_PER_HEAD = 64  # ssd_chunk_scan_passing: one uint32 counter per 256 bytes


def alloc_sync(batch, nheads, device="cuda"):
    """Zeroed counters for ssd_chunk_scan_passing (zero them again before every call)."""
    torch = _torch()
    return torch.zeros(batch * nheads * SYNC_WORDS_PER_HEAD, dtype=torch.int32, device=device)


def chunk_scan_passing(x, C, cb, acum, dtc, states, sync, D=None, initial_state=None, *, chunk: int, y=None,
                       final_state="new", stream=None):
    """ssd_chunk_scan_passing: Step-3 and the chunk scan in one launch (one-round bf16 problems).

    ``states`` float16 [B,H,nc,P,N]: chunk states in, entering states out.  ``sync``: zeroed
    counters (alloc_sync).  Returns (y fp32, final_state or None); raises SsdError with
    SSD_ERR_UNSUPPORTED for shapes that do not take this path.
    """
    torch = _torch()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = C.shape[2], C.shape[3]
    _dev(x, C, cb, acum, dtc, states, sync, D, initial_state, y)
    _f32(D, initial_state, y)
    if states.dtype != torch.float16:
        raise TypeError("states must be float16 (bfloat16 or float8_e4m3fn inputs)")
    if sync.numel() * sync.element_size() < batch * nheads * SYNC_WORDS_PER_HEAD * 4:
        raise ValueError("sync is smaller than batch * nheads * 256 bytes")
    if y is None:
        y = torch.empty((batch, seqlen, nheads, headdim), dtype=torch.float32, device=x.device)
    if isinstance(final_state, str):
        final_state = torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=x.device)
    _dev(final_state)
    _f32(final_state)
    _check(lib().ssd_chunk_scan_passing(_ptr(x), _ptr(C), _ptr(cb), _ptr(acum), _ptr(dtc), _ptr(states),
                                        _ptr(initial_state), _ptr(final_state), _ptr(D), _ptr(y), _ptr(sync),
                                        _dtype_code(x), batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                        _stream(stream)), "ssd_chunk_scan_passing")
    return y, final_state
