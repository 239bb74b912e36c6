"""Thin ctypes binding of the C ABI in include/la.h.

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current stream.  There is
no CPU path: if the library or a GPU is missing, calls raise.

The ``la_*`` functions mirror the C entry points one to one (tensors in
place of pointers, sizes inferred from the tensors).  The functions without
the prefix allocate outputs and workspace and return them.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

LA_F32, LA_BF16 = 0, 1
LA_OP_FWD_CAUSAL, LA_OP_FWD_NONCAUSAL, LA_OP_BWD_CAUSAL, LA_OP_DECODE, LA_OP_BWD_NONCAUSAL = 0, 1, 2, 3, 4
LA_OP_FWD_DECAY, LA_OP_BWD_DECAY = 5, 6
LA_FEATURE_ELU1, LA_FEATURE_IDENTITY = 0, 1
LA_FORM_AUTO, LA_FORM_TWO_LAUNCH, LA_FORM_ONE_LAUNCH = 0, 1, 2
LA_ERR_WAIT = 10
ENTRY_POINTS = ("la_version", "la_workspace_size", "la_checkpoint_size", "la_segment_length", "la_forward_causal",
                "la_forward_noncausal", "la_backward_causal", "la_backward_noncausal", "la_decode_step",
                "la_status_string", "la_last_error", "la_kernel_names", "la_forward_wait_status",
                "la_forward_causal_noalloc",
                "la_feature_random", "la_feature_random_vjp", "la_feature_poly2",
                "la_feature_poly2_vjp")

_lib = None


class Options(ctypes.Structure):
    """la_options of include/la.h: per-call options (all zero = the defaults)."""

    _fields_ = [("segment_chunks", ctypes.c_int), ("forward_form", ctypes.c_int), ("wait_polls", ctypes.c_int),
                ("event_pairs", ctypes.c_int), ("status", ctypes.c_void_p), ("timed_kernel", ctypes.c_char_p),
                ("events", ctypes.c_void_p), ("events_used", ctypes.POINTER(ctypes.c_int))]


def options(segment_chunks: int = 0, forward_form: int = LA_FORM_AUTO, wait_polls: int = 0, status=None,
            timer=None) -> Options:
    """Per-call options: segment length in 64-token chunks (0 automatic), form of the causal forward, the
    one-launch forward's wait limit (0 default, < 0 none), an optional int32 device tensor of one element that the
    one-launch forward ORs 1 into when a wait gave up, and an optional KernelTimer."""
    if segment_chunks < 0:
        raise ValueError("segment_chunks must be >= 0")
    if forward_form not in (LA_FORM_AUTO, LA_FORM_TWO_LAUNCH, LA_FORM_ONE_LAUNCH):
        raise ValueError("forward_form must be LA_FORM_AUTO, LA_FORM_TWO_LAUNCH or LA_FORM_ONE_LAUNCH")
    o = Options(int(segment_chunks), int(forward_form), int(wait_polls), 0, None, None, None, None)
    if status is not None:
        if status.dtype != torch.int32 or status.numel() < 1 or not status.is_cuda:
            raise ValueError("status must be an int32 device tensor")
        o.status = status.data_ptr()
        o._status = status  # keep it alive with the options
    if timer is not None:
        timer.attach(o)
    return o


def _opt(o):
    return ctypes.byref(o) if o is not None else None


class LAError(RuntimeError):
    def __init__(self, status: int, func: str):
        lib = load()
        name = lib.la_status_string(status).decode()
        detail = lib.la_last_error().decode()
        super().__init__(f"{func} failed: {name} ({status}): {detail}")
        self.status = status


def load(path: str | None = None):
    """Load the in-tree library (building it first only if it does not exist)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or _build.ensure_built()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} not found")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    op = ctypes.POINTER(Options)
    lib.la_version.restype = i
    lib.la_workspace_size.restype = sz
    lib.la_workspace_size.argtypes = [i] * 7 + [op]
    lib.la_checkpoint_size.restype = sz
    lib.la_checkpoint_size.argtypes = [i] * 5 + [op]
    lib.la_segment_length.restype = i
    lib.la_segment_length.argtypes = [i] * 5 + [op]
    lib.la_forward_wait_status.restype = i
    lib.la_forward_wait_status.argtypes = [vp, sz] + [i] * 6 + [vp, op]
    lib.la_forward_causal.restype = i
    lib.la_forward_causal.argtypes = [vp] * 11 + [i] * 7 + [vp, sz, vp, op]
    lib.la_forward_causal_noalloc.restype = i
    lib.la_forward_causal_noalloc.argtypes = [vp] * 11 + [i] * 7 + [vp, op]
    lib.la_forward_noncausal.restype = i
    lib.la_forward_noncausal.argtypes = [vp] * 6 + [i] * 7 + [vp, sz, vp, op]
    lib.la_backward_causal.restype = i
    lib.la_backward_causal.argtypes = [vp] * 18 + [i] * 7 + [vp, sz, vp, op]
    lib.la_backward_noncausal.restype = i
    lib.la_backward_noncausal.argtypes = [vp] * 9 + [i] * 7 + [vp, sz, vp, op]
    lib.la_decode_step.restype = i
    lib.la_decode_step.argtypes = [vp] * 7 + [i] * 6 + [vp, op]
    for name, nptr in (("la_feature_random", 3), ("la_feature_random_vjp", 4), ("la_feature_poly2", 2),
                       ("la_feature_poly2_vjp", 3)):
        getattr(lib, name).restype = i
        getattr(lib, name).argtypes = [vp] * nptr + [i] * 6 + [vp]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_status_string.argtypes = [i]
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_kernel_names.restype = ctypes.c_char_p
    if path is None or _lib is None:
        _lib = lib
    return lib


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return LA_F32
    if dt == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {dt}: use torch.float32 or torch.bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, func: str):
    if status != 0:
        raise LAError(status, func)


# ---------------------------------------------------------------- validation
# The C library receives raw pointers, so every tensor's shape and dtype is checked here against the sizes the
# call passes: a mismatch would make a kernel read or write past the end of a buffer.
def _expect(name, t, shape, dtype):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def feature_shape(B, H, N, C):
    """Shape of C-wide feature vectors: [B,H,N,C] up to 64 features, else feature-sliced [B,H,C/64,N,64] (slice s
    holds features 64s..64s+63 of every token), the layout the library's wide kernels read and write."""
    return (B, H, N, C) if C <= 64 else (B, H, C // 64, N, 64)


def to_sliced(x):
    """[B,H,N,C] -> feature-sliced [B,H,C/64,N,64] (a copy; C a multiple of 64)."""
    B, H, N, C = x.shape
    if C % 64:
        raise ValueError("the feature-sliced layout needs C to be a multiple of 64")
    return x.reshape(B, H, N, C // 64, 64).permute(0, 1, 3, 2, 4).contiguous()


def from_sliced(x):
    """Feature-sliced [B,H,ns,N,64] -> [B,H,N,ns*64] (a copy)."""
    B, H, ns, N, c = x.shape
    return x.permute(0, 1, 3, 2, 4).reshape(B, H, N, ns * c).contiguous()


def _sizes(q, k, v):
    """(B, H, N, D, M) from Q [B,H,N,D] (or feature-sliced [B,H,D/64,N,64] for D > 64), K like Q, V [B,H,N,M] of
    Q's dtype."""
    if not all(isinstance(t, torch.Tensor) for t in (q, k, v)):
        raise TypeError("Q, K and V must be torch tensors")
    if q.dim() == 5 and v.dim() == 4:
        B, H, ns, N, c = q.shape
        if c != 64 or ns < 2:
            raise ValueError("feature-sliced Q/K must be [B,H,D/64,N,64] with D/64 >= 2")
        D = ns * 64
    elif q.dim() == 4 and v.dim() == 4:
        B, H, N, D = q.shape
        if D > 64:
            raise ValueError("Q/K wider than 64 features must be feature-sliced: [B,H,D/64,N,64] (see to_sliced)")
    else:
        raise ValueError("expected Q/K [B,H,N,D] (or [B,H,D/64,N,64]) and V [B,H,N,M]")
    M = v.shape[-1]
    dtype_code(q.dtype)
    _expect("K", k, q.shape, q.dtype)
    _expect("V", v, (B, H, N, M), q.dtype)
    return B, H, N, D, M


def _expect_state(names, s, z, B, H, D, M):
    _expect(names[0], s, (B, H, D, M), torch.float32)
    _expect(names[1], z, (B, H, D), torch.float32)


def _expect_ckpt(ck, B, H, N, D, M, opts):
    if ck is None:
        return
    if ck.dtype != torch.float32 or ck.numel() * 4 != checkpoint_size(B, H, N, D, M, opts):
        raise ValueError(f"ckpt must be float32 with {checkpoint_size(B, H, N, D, M, opts)} bytes for these sizes and "
                         f"options (got {ck.numel() * ck.element_size()} bytes of {ck.dtype})")


def _expect_ws(ws):
    if ws is not None and (not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1):
        raise ValueError("ws must be a 1-D uint8 tensor")


def workspace_size(op: int, B, H, N, D, M, dtype: int, opts: Options | None = None) -> int:
    return int(load().la_workspace_size(op, B, H, N, D, M, dtype, _opt(opts)))


def checkpoint_size(B, H, N, D, M, opts: Options | None = None) -> int:
    return int(load().la_checkpoint_size(B, H, N, D, M, _opt(opts)))


def segment_length(B, H, N, D, M, opts: Options | None = None) -> int:
    return int(load().la_segment_length(B, H, N, D, M, _opt(opts)))


def forward_wait_status(ws, B, H, N, D, M, dtype: int, opts: Options | None = None, stream=None) -> int:
    """Status word of the last one-launch forward on `ws` (synchronises the stream): 0, or LA_ERR_WAIT."""
    st = load().la_forward_wait_status(_ptr(ws), ws.numel() if ws is not None else 0, B, H, N, D, M, dtype,
                                       _stream(stream), _opt(opts))
    if st not in (0, LA_ERR_WAIT):
        _check(st, "la_forward_wait_status")
    return st


def alloc_workspace(op: int, B, H, N, D, M, dtype: int, device, opts: Options | None = None) -> torch.Tensor:
    n = workspace_size(op, B, H, N, D, M, dtype, opts)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------ measurement
class KernelTimer:
    """Caller-owned HIP events for la_options' timed_kernel: the library records a pair around every launch of
    the named kernel on its launch stream.  Events are created without the system-scope fence (timing only)."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, kernel: str, pairs: int = 4096):
        if KernelTimer._hip is None:
            KernelTimer._hip = ctypes.CDLL("libamdhip64.so")
        hip = KernelTimer._hip
        # kept on the instance: module globals (ctypes included) may be gone when it is collected at exit
        self._lib, self._vp = hip, ctypes.c_void_p
        self.kernel = kernel.encode()
        self.pairs = int(pairs)
        self.events = (ctypes.c_void_p * (2 * self.pairs))()
        for e in range(2 * self.pairs):
            ev = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(self.FLAGS)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events[e] = ev.value
        self.used = ctypes.c_int(0)

    def attach(self, o: Options):
        o.timed_kernel = self.kernel
        o.events = ctypes.cast(self.events, ctypes.c_void_p)
        o.event_pairs = self.pairs
        o.events_used = ctypes.pointer(self.used)
        o._timer = self

    def reset(self):
        self.used.value = 0

    @property
    def launches(self) -> int:
        return self.used.value

    def collect(self):
        """(summed ms, launches) of the recorded pairs (synchronises on the last event); resets the count."""
        hip = KernelTimer._hip
        total = 0.0
        n = self.used.value
        if n:
            if hip.hipEventSynchronize(ctypes.c_void_p(self.events[2 * n - 1])) != 0:
                raise RuntimeError("hipEventSynchronize failed")
        for i in range(n):
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.events[2 * i]),
                                       ctypes.c_void_p(self.events[2 * i + 1])) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            total += ms.value
        self.used.value = 0
        return total, n

    def __del__(self):
        hip, vp = getattr(self, "_lib", None), getattr(self, "_vp", None)
        if hip is None or vp is None:
            return
        for e in range(2 * self.pairs):
            if self.events[e]:
                hip.hipEventDestroy(vp(self.events[e]))


# --------------------------------------------------------- one-to-one calls
def la_forward_causal(Q, K, V, O, den=None, S0=None, Z0=None, S_out=None, Z_out=None, ckpt=None, ws=None,
                      stream=None, logA=None, feature=0, opts=None):
    B, H, N, D, M = _sizes(Q, K, V)
    _expect("O", O, (B, H, N, M), Q.dtype)
    _expect("den", den, (B, H, N), torch.float32)
    _expect("logA", logA, (B, H, N), torch.float32)
    _expect_state(("S0", "Z0"), S0, Z0, B, H, D, M)
    _expect_state(("S_out", "Z_out"), S_out, Z_out, B, H, D, M)
    _expect_ckpt(ckpt, B, H, N, D, M, opts)
    _expect_ws(ws)
    dt = dtype_code(Q.dtype)
    nb = ws.numel() if ws is not None else 0
    st = load().la_forward_causal(_ptr(Q), _ptr(K), _ptr(V), _ptr(logA), _ptr(O), _ptr(den), _ptr(S0), _ptr(Z0),
                                  _ptr(S_out), _ptr(Z_out), _ptr(ckpt), B, H, N, D, M, dt, feature, _ptr(ws), nb,
                                  _stream(stream), _opt(opts))
    _check(st, "la_forward_causal")


def la_forward_causal_noalloc(Q, K, V, O, den=None, S0=None, Z0=None, S_out=None, Z_out=None, ckpt=None,
                              stream=None, logA=None, feature=0, opts=None):
    """la_forward_causal with the library's static per-GPU scratch in place of a workspace (allocates nothing;
    calls that overlap on one GPU race)."""
    B, H, N, D, M = _sizes(Q, K, V)
    _expect("O", O, (B, H, N, M), Q.dtype)
    _expect("den", den, (B, H, N), torch.float32)
    _expect("logA", logA, (B, H, N), torch.float32)
    _expect_state(("S0", "Z0"), S0, Z0, B, H, D, M)
    _expect_state(("S_out", "Z_out"), S_out, Z_out, B, H, D, M)
    _expect_ckpt(ckpt, B, H, N, D, M, opts)
    st = load().la_forward_causal_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(logA), _ptr(O), _ptr(den), _ptr(S0),
                                          _ptr(Z0), _ptr(S_out), _ptr(Z_out), _ptr(ckpt), B, H, N, D, M,
                                          dtype_code(Q.dtype), feature, _stream(stream), _opt(opts))
    _check(st, "la_forward_causal_noalloc")


def la_forward_noncausal(Q, K, V, O, ws=None, stream=None, feature=0, S_out=None, Z_out=None, opts=None):
    B, H, N, D, M = _sizes(Q, K, V)
    _expect("O", O, (B, H, N, M), Q.dtype)
    _expect_state(("S_out", "Z_out"), S_out, Z_out, B, H, D, M)
    _expect_ws(ws)
    nb = ws.numel() if ws is not None else 0
    st = load().la_forward_noncausal(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(S_out), _ptr(Z_out), B, H, N, D, M,
                                     dtype_code(Q.dtype), feature, _ptr(ws), nb, _stream(stream), _opt(opts))
    _check(st, "la_forward_noncausal")


def la_backward_causal(Q, K, V, O, den, dO, dQ, dK, dV, S0=None, Z0=None, ckpt=None, dS_N=None, dZ_N=None,
                       dS0=None, dZ0=None, ws=None, stream=None, logA=None, dlogA=None, feature=0, opts=None):
    B, H, N, D, M = _sizes(Q, K, V)
    for name, t, shape in (("O", O, (B, H, N, M)), ("dO", dO, (B, H, N, M)), ("dQ", dQ, feature_shape(B, H, N, D)),
                           ("dK", dK, feature_shape(B, H, N, D)), ("dV", dV, (B, H, N, M))):
        _expect(name, t, shape, Q.dtype)
    _expect("den", den, (B, H, N), torch.float32)
    _expect("logA", logA, (B, H, N), torch.float32)
    _expect("dlogA", dlogA, (B, H, N), torch.float32)
    _expect_state(("S0", "Z0"), S0, Z0, B, H, D, M)
    _expect_state(("dS_N", "dZ_N"), dS_N, dZ_N, B, H, D, M)
    _expect_state(("dS0", "dZ0"), dS0, dZ0, B, H, D, M)
    _expect_ckpt(ckpt, B, H, N, D, M, opts)
    _expect_ws(ws)
    nb = ws.numel() if ws is not None else 0
    st = load().la_backward_causal(_ptr(Q), _ptr(K), _ptr(V), _ptr(logA), _ptr(O), _ptr(den), _ptr(dO), _ptr(S0),
                                   _ptr(Z0), _ptr(ckpt), _ptr(dS_N), _ptr(dZ_N), _ptr(dQ), _ptr(dK), _ptr(dV),
                                   _ptr(dlogA), _ptr(dS0), _ptr(dZ0), B, H, N, D, M, dtype_code(Q.dtype), feature,
                                   _ptr(ws), nb, _stream(stream), _opt(opts))
    _check(st, "la_backward_causal")


def la_backward_noncausal(Q, K, V, dO, dQ, dK, dV, ws=None, stream=None, feature=0, S_tot=None, Z_tot=None,
                          opts=None):
    B, H, N, D, M = _sizes(Q, K, V)
    for name, t, shape in (("dO", dO, (B, H, N, M)), ("dQ", dQ, feature_shape(B, H, N, D)),
                           ("dK", dK, feature_shape(B, H, N, D)), ("dV", dV, (B, H, N, M))):
        _expect(name, t, shape, Q.dtype)
    _expect_state(("S_tot", "Z_tot"), S_tot, Z_tot, B, H, D, M)
    _expect_ws(ws)
    nb = ws.numel() if ws is not None else 0
    st = load().la_backward_noncausal(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(S_tot), _ptr(Z_tot), _ptr(dQ),
                                      _ptr(dK), _ptr(dV), B, H, N, D, M, dtype_code(Q.dtype), feature, _ptr(ws), nb,
                                      _stream(stream), _opt(opts))
    _check(st, "la_backward_noncausal")


def la_decode_step(q, k, v, S, Z, y, stream=None, logA=None, feature=0, opts=None):
    if not all(isinstance(t, torch.Tensor) for t in (q, k, v, S, Z, y)):
        raise TypeError("q, k, v, S, Z and y must be torch tensors")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("decode expects q, k [B,H,D], v [B,H,M]")
    B, H, D = q.shape
    M = v.shape[-1]
    dtype_code(q.dtype)
    _expect("k", k, (B, H, D), q.dtype)
    _expect("v", v, (B, H, M), q.dtype)
    _expect("y", y, (B, H, M), q.dtype)
    _expect_state(("S", "Z"), S, Z, B, H, D, M)
    _expect("logA", logA, (B, H), torch.float32)
    st = load().la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(logA), _ptr(S), _ptr(Z), _ptr(y), B, H, D, M,
                               dtype_code(q.dtype), feature, _stream(stream), _opt(opts))
    _check(st, "la_decode_step")


# ------------------------------------------------------ allocating helpers
def forward_causal(q, k, v, *, s0=None, z0=None, return_state=False, checkpoint=True, log_a=None, feature=0,
                   opts=None):
    """Causal forward (decayed by exp(log_a) [B,H,N] float32 when given).  Returns dict(o, den, ckpt, ws[, s, z]);
    the checkpoint is laid out by opts.segment_chunks, so a backward from it takes the same options."""
    B, H, N, D, M = _sizes(q, k, v)
    dev = q.device
    o = torch.empty((B, H, N, M), dtype=q.dtype, device=dev)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ck = torch.empty(checkpoint_size(B, H, N, D, M, opts) // 4, dtype=torch.float32, device=dev) if checkpoint else None
    s = z = None
    if return_state:
        s = torch.empty((B, H, D, M), dtype=torch.float32, device=dev)
        z = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    ws = alloc_workspace(LA_OP_FWD_DECAY if log_a is not None else LA_OP_FWD_CAUSAL, B, H, N, D, M,
                         dtype_code(q.dtype), dev, opts)
    la_forward_causal(q, k, v, o, den, s0, z0, s, z, ck, ws, logA=log_a, feature=feature, opts=opts)
    out = {"o": o, "den": den, "ckpt": ck, "ws": ws}
    if return_state:
        out["s"], out["z"] = s, z
    return out


def forward_noncausal(q, k, v, feature=0, return_state=False, opts=None):
    """Non-causal forward.  Returns O, or (O, S, Z) with the totals when return_state."""
    B, H, N, D, M = _sizes(q, k, v)
    o = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    s = z = None
    if return_state:
        s = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(LA_OP_FWD_NONCAUSAL, B, H, N, D, M, dtype_code(q.dtype), q.device, opts)
    la_forward_noncausal(q, k, v, o, ws, feature=feature, S_out=s, Z_out=z, opts=opts)
    return (o, s, z) if return_state else o


def backward_causal(q, k, v, o, den, do, *, s0=None, z0=None, ckpt=None, ds_n=None, dz_n=None, state_grad=False,
                    log_a=None, feature=0, opts=None):
    """Causal backward.  Returns (dq, dk, dv), then dlog_a when log_a is given, then (ds0, dz0) with
    state_grad: the gradient with respect to the initial state; ds_n, dz_n are the upstream gradients of the
    final state (None: not in the loss).  A checkpoint must come from a forward with the same options."""
    B, H, N, D, M = _sizes(q, k, v)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ds0 = dz0 = dla = None
    if state_grad:
        ds0 = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
        dz0 = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    if log_a is not None:
        dla = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(LA_OP_BWD_DECAY if log_a is not None else LA_OP_BWD_CAUSAL, B, H, N, D, M,
                         dtype_code(q.dtype), q.device, opts)
    la_backward_causal(q, k, v, o, den, do, dq, dk, dv, s0, z0, ckpt, ds_n, dz_n, ds0, dz0, ws, logA=log_a, dlogA=dla,
                       feature=feature, opts=opts)
    out = (dq, dk, dv) + ((dla,) if log_a is not None else ())
    return out + ((ds0, dz0) if state_grad else ())


def backward_noncausal(q, k, v, do, feature=0, s=None, z=None, opts=None):
    """Non-causal backward; s, z: the forward's totals (None: formed again)."""
    B, H, N, D, M = _sizes(q, k, v)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = alloc_workspace(LA_OP_BWD_NONCAUSAL, B, H, N, D, M, dtype_code(q.dtype), q.device, opts)
    la_backward_noncausal(q, k, v, do, dq, dk, dv, ws, feature=feature, S_tot=s, Z_tot=z, opts=opts)
    return dq, dk, dv


def decode_step(q, k, v, s, z, y=None, log_a=None, feature=0, opts=None):
    """One RNN step (decayed by exp(log_a) [B,H] when given): updates s, z in place and returns y."""
    if y is None:
        y = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    la_decode_step(q, k, v, s, z, y, logA=log_a, feature=feature, opts=opts)
    return y


class CausalLinearAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in the HIP library.  With an initial state (s0, z0,
    float32) the gradient reaches it; with return_state the final state (s, z) is returned as well and its
    gradient flows back through the same backward."""

    @staticmethod
    def forward(ctx, q, k, v, s0, z0, return_state, log_a, feature, opts):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        if (s0 is None) != (z0 is None):
            raise ValueError("s0 and z0 go together")
        if s0 is not None:
            s0, z0 = s0.contiguous(), z0.contiguous()
        if log_a is not None:
            log_a = log_a.contiguous()
        out = forward_causal(q, k, v, s0=s0, z0=z0, return_state=return_state, log_a=log_a, feature=feature,
                             opts=opts)
        ctx.feature = feature
        ctx.opts = opts  # the checkpoint's layout depends on the segment option: the backward takes the same
        ctx.has_state = s0 is not None
        ctx.has_decay = log_a is not None
        ctx.save_for_backward(q, k, v, out["o"], out["den"], out["ckpt"], s0, z0, log_a)
        if return_state:
            return out["o"], out["s"], out["z"]
        return out["o"]

    @staticmethod
    def backward(ctx, do, ds_n=None, dz_n=None):
        q, k, v, o, den, ck, s0, z0, log_a = ctx.saved_tensors
        want_state = ctx.has_state and (ctx.needs_input_grad[3] or ctx.needs_input_grad[4])
        if ds_n is not None:
            ds_n, dz_n = ds_n.contiguous(), dz_n.contiguous()
        g = list(backward_causal(q, k, v, o, den, do.contiguous(), s0=s0, z0=z0, ckpt=ck, ds_n=ds_n, dz_n=dz_n,
                                 state_grad=want_state, log_a=log_a, feature=ctx.feature, opts=ctx.opts))
        dla = g.pop(3) if ctx.has_decay else None
        ds0, dz0 = (g[3], g[4]) if want_state else (None, None)
        return g[0], g[1], g[2], ds0, dz0, None, dla, None, None


def causal_linear_attention(q, k, v, s0=None, z0=None, return_state=False, log_a=None, feature=0, opts=None):
    """Causal linear attention through the HIP library, differentiable in q, k, v, the initial state (s0, z0)
    and the log-decay log_a [B,H,N] (float32, <= 0) when given.  feature=LA_FEATURE_IDENTITY takes q, k as
    feature vectors already (see feature_map)."""
    return CausalLinearAttention.apply(q, k, v, s0, z0, return_state, log_a, feature, opts)


class NonCausalLinearAttention(torch.autograd.Function):
    """Autograd wrapper of the non-causal form: forward and backward both run in the HIP library."""

    @staticmethod
    def forward(ctx, q, k, v, feature):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, s, z = forward_noncausal(q, k, v, feature=feature, return_state=True)
        ctx.save_for_backward(q, k, v, s, z)
        ctx.feature = feature
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, s, z = ctx.saved_tensors
        return backward_noncausal(q, k, v, do.contiguous(), feature=ctx.feature, s=s, z=z) + (None,)


def noncausal_linear_attention(q, k, v, feature=0):
    return NonCausalLinearAttention.apply(q, k, v, feature)


# ------------------------------------------------------------ feature maps
def _check_x(x):
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("expected X [B,H,N,Din]")
    dtype_code(x.dtype)
    return x.shape


def feature_random(x, w):
    """Positive random features exp(W x - |x|^2 / 2) / sqrt(C) (w [H,C,Din] float32) in x's dtype."""
    B, H, N, Din = _check_x(x)
    C = w.shape[1] if w.dim() == 3 else -1
    _expect("W", w, (H, C, Din), torch.float32)
    phi = torch.empty(feature_shape(B, H, N, C), dtype=x.dtype, device=x.device)
    _check(load().la_feature_random(_ptr(x), _ptr(w), _ptr(phi), B, H, N, Din, C, dtype_code(x.dtype),
                                    _stream(None)), "la_feature_random")
    return phi


def feature_random_vjp(x, w, dphi):
    B, H, N, Din = _check_x(x)
    C = w.shape[1] if w.dim() == 3 else -1
    _expect("W", w, (H, C, Din), torch.float32)
    _expect("dPhi", dphi, feature_shape(B, H, N, C), x.dtype)
    dx = torch.empty_like(x)
    _check(load().la_feature_random_vjp(_ptr(x), _ptr(w), _ptr(dphi), _ptr(dx), B, H, N, Din, C,
                                        dtype_code(x.dtype), _stream(None)), "la_feature_random_vjp")
    return dx


def feature_poly2(x, C):
    """Degree-2 polynomial features (1, x, x_a x_b, zeros) of size C in x's dtype."""
    B, H, N, Din = _check_x(x)
    phi = torch.empty(feature_shape(B, H, N, C), dtype=x.dtype, device=x.device)
    _check(load().la_feature_poly2(_ptr(x), _ptr(phi), B, H, N, Din, C, dtype_code(x.dtype), _stream(None)),
           "la_feature_poly2")
    return phi


def feature_poly2_vjp(x, dphi):
    B, H, N, Din = _check_x(x)
    if dphi.dim() == 5:
        C = dphi.shape[2] * dphi.shape[4]
    elif dphi.dim() == 4:
        C = dphi.shape[-1]
    else:
        raise ValueError("expected dPhi [B,H,N,C] (or [B,H,C/64,N,64])")
    _expect("dPhi", dphi, feature_shape(B, H, N, C), x.dtype)
    dx = torch.empty_like(x)
    _check(load().la_feature_poly2_vjp(_ptr(x), _ptr(dphi), _ptr(dx), B, H, N, Din, C,
                                       dtype_code(x.dtype), _stream(None)), "la_feature_poly2_vjp")
    return dx


class RandomFeatures(torch.autograd.Function):
    """Positive random features through the HIP library (the projection w is not differentiated)."""

    @staticmethod
    def forward(ctx, x, w):
        x, w = x.contiguous(), w.contiguous()
        ctx.save_for_backward(x, w)
        return feature_random(x, w)

    @staticmethod
    def backward(ctx, dphi):
        x, w = ctx.saved_tensors
        return feature_random_vjp(x, w, dphi.contiguous()), None


class Poly2Features(torch.autograd.Function):
    """Degree-2 polynomial features through the HIP library."""

    @staticmethod
    def forward(ctx, x, C):
        x = x.contiguous()
        ctx.save_for_backward(x)
        return feature_poly2(x, C)

    @staticmethod
    def backward(ctx, dphi):
        (x,) = ctx.saved_tensors
        return feature_poly2_vjp(x, dphi.contiguous()), None


def random_features(x, w):
    return RandomFeatures.apply(x, w)


def poly2_features(x, C):
    return Poly2Features.apply(x, C)


# -------------------------------------------------------------------- misc
def kernel_names():
    return load().la_kernel_names().decode().split(",")
