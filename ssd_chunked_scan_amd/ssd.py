"""Python binding of ``libssd.so`` (the C ABI in ``include/ssd.h``).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``libssd.so``.  PyTorch provides device memory (``torch.empty``) and
the current HIP stream.  Tensors must already be contiguous, on the GPU and of
the documented dtypes; nothing is copied or converted silently.  If the library
is missing the first call raises, there is no fallback.

Names follow the C ABI: ``fwd`` (= ``ssd_fwd``), the per-step entry points
``chunk_cumsum``, ``chunk_cb``, ``chunk_state``, ``state_passing``,
``seq_final_states``, ``chunk_scan``, the decode step ``step`` (= ``ssd_step``)
and the backward ``bwd`` (= ``ssd_bwd``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssd.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}

EXPORTED = ["ssd_abi_version", "ssd_status_string", "ssd_fwd_workspace_size", "ssd_fwd",
            "ssd_chunk_cumsum", "ssd_chunk_cb", "ssd_chunk_state", "ssd_state_passing",
            "ssd_seq_final_states", "ssd_chunk_scan", "ssd_step", "ssd_bwd_workspace_size", "ssd_bwd",
            "ssd_fwd_gated", "ssd_conv1d_silu", "ssd_fwd_noalloc", "ssd_bwd_stage_times", "ssd_check_seq_idx"]

# SSD_BWD_MAX_STAGES in include/ssd.h
BWD_MAX_STAGES = 24

# The static scratch of ssd_fwd_noalloc (SSD_NOALLOC_SCRATCH_BYTES in include/ssd.h).
NOALLOC_SCRATCH_BYTES = 128 << 20


class FwdArgs(ctypes.Structure):
    """Mirror of ``ssd_fwd_args``."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("initial_states", ctypes.c_void_p), ("seq_idx", ctypes.c_void_p), ("nseq", ctypes.c_int64),
        ("y", ctypes.c_void_p), ("final_states", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class StepArgs(ctypes.Structure):
    """Mirror of ``ssd_step_args``."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("state", ctypes.c_void_p), ("y", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ``ssd_bwd_args``."""
    _fields_ = [
        ("dy", ctypes.c_void_p), ("dfinal_states", ctypes.c_void_p), ("dx", ctypes.c_void_p),
        ("ddt", ctypes.c_void_p), ("dA", ctypes.c_void_p), ("dB", ctypes.c_void_p), ("dC", ctypes.c_void_p),
        ("dD", ctypes.c_void_p), ("dinitial_states", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("fwd_workspace", ctypes.c_void_p), ("fwd_workspace_bytes", ctypes.c_size_t),
    ]


class ConvArgs(ctypes.Structure):
    """Mirror of ``ssd_conv_args``."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("width", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("xbc", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("seq_idx", ctypes.c_void_p), ("x", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
    ]


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load ``libssd.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc for gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(FwdArgs)
    vp = ctypes.c_void_p
    lib.ssd_abi_version.restype = ctypes.c_int
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int32]
    lib.ssd_fwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_fwd.argtypes = [P, vp]
    lib.ssd_chunk_cumsum.argtypes = [P, vp, vp, vp]
    lib.ssd_chunk_cb.argtypes = [P, vp, vp]
    lib.ssd_chunk_state.argtypes = [P, vp, vp, vp, vp, vp]
    lib.ssd_state_passing.argtypes = [P, vp, vp, vp]
    lib.ssd_seq_final_states.argtypes = [P, vp, vp, vp, vp, vp]
    lib.ssd_chunk_scan.argtypes = [P, vp, vp, vp, vp, vp]
    lib.ssd_step.argtypes = [ctypes.POINTER(StepArgs), vp]
    lib.ssd_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_bwd.argtypes = [P, ctypes.POINTER(BwdArgs), vp]
    lib.ssd_fwd_gated.argtypes = [P, vp, vp]
    lib.ssd_conv1d_silu.argtypes = [ctypes.POINTER(ConvArgs), vp]
    lib.ssd_fwd_noalloc.argtypes = [P, vp]
    for name in EXPORTED[2:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (no silent copies)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Problem:
    """Validated tensors and the matching ``FwdArgs`` for one call."""

    def __init__(self, x, dt, A, B, C, chunk, D=None, initial_states=None, seq_idx=None,
                 nseq=None, dt_softplus=True):
        if x.dim() != 4:
            raise ValueError("x must be [batch, seqlen, nheads, headdim]")
        b, T, H, P = x.shape
        if B.dim() != 4:
            raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
        G, N = B.shape[2], B.shape[3]
        if x.dtype not in _DTYPES:
            raise TypeError("x must be float32 or bfloat16")
        dev = x.device
        _check(x, "x", device=dev)
        _check(dt, "dt", x.dtype, (b, T, H), dev)
        _check(A, "A", torch.float32, (H,), dev)
        _check(B, "B", x.dtype, (b, T, G, N), dev)
        _check(C, "C", x.dtype, (b, T, G, N), dev)
        _check(D, "D", torch.float32, (H,), dev)
        _check(initial_states, "initial_states", torch.float32, (b, H, P, N), dev)
        if seq_idx is not None:
            _check(seq_idx, "seq_idx", torch.int32, None, dev)
            if seq_idx.numel() != T:
                raise ValueError("seq_idx must hold seqlen int32 ids")
            if nseq is None:
                raise ValueError("nseq is required with seq_idx (no device->host read)")
        self.x, self.dt, self.A, self.B, self.C = x, dt, A, B, C
        self.D, self.initial_states, self.seq_idx = D, initial_states, seq_idx
        self.b, self.T, self.H, self.P, self.N, self.G, self.Q = b, T, H, P, N, G, int(chunk)
        self.nc = (T + self.Q - 1) // self.Q
        self.NT = 64 if N <= 64 else 128 if N <= 128 else 256   # state width the kernels use
        self.nseq = int(nseq) if seq_idx is not None else 0
        self.dtype = x.dtype
        self.device = dev
        self.args = FwdArgs(b, T, H, P, N, G, self.Q, _DTYPES[x.dtype], int(bool(dt_softplus)),
                            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                            _ptr(initial_states), _ptr(seq_idx), self.nseq,
                            None, None, None, 0)

    # shapes of the outputs and intermediates
    def final_shape(self):
        return (self.nseq if self.seq_idx is not None else self.b, self.H, self.P, self.N)

    def cb_shape(self):
        # per (b, c, g): CB (Q x Q), C (Q x NT) and B^T (NT x Q), fragment-major
        return (self.b, self.nc, self.G, self.Q * (self.Q + 2 * self.NT))

    def empty(self, shape, dtype=None):
        return torch.empty(shape, dtype=dtype or self.dtype, device=self.device)

    def call(self, name, *ptrs, stream=None):
        lib = load_library()
        st = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        rc = getattr(lib, name)(ctypes.byref(self.args), *ptrs, ctypes.c_void_p(st))
        if rc != 0:
            raise SSDError(rc, name)


def check_seq_idx(seq_idx: torch.Tensor, nseq: int, stream=None) -> int:
    """``ssd_check_seq_idx``: the first position whose segment id breaks the
    packed-stream precondition (ids non-decreasing, in [0, nseq)), or -1.
    Waits for the stream to read the result."""
    if seq_idx.dtype != torch.int32 or seq_idx.device.type != "cuda" or not seq_idx.is_contiguous():
        raise ValueError("seq_idx must be a contiguous int32 device tensor")
    out = torch.empty((), dtype=torch.int32, device=seq_idx.device)
    st = stream if stream is not None else torch.cuda.current_stream(seq_idx.device).cuda_stream
    rc = load_library().ssd_check_seq_idx(ctypes.c_void_p(seq_idx.data_ptr()), ctypes.c_int64(seq_idx.numel()),
                                          ctypes.c_int64(nseq), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st))
    if rc != 0:
        raise SSDError(rc, "ssd_check_seq_idx")
    torch.cuda.synchronize(seq_idx.device)
    return int(out.item())


def workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().ssd_fwd_workspace_size(ctypes.byref(p.args), ctypes.byref(n))
    if rc != 0:
        raise SSDError(rc, "ssd_fwd_workspace_size")
    return int(n.value)


def fwd(x, dt, A, B, C, chunk, D=None, initial_states=None, seq_idx=None, nseq=None,
        dt_softplus=True, y=None, final_states=None, workspace=None, stream=None,
        want_final=True):
    """y, final_states = SSD forward (see ``include/ssd.h``).

    ``y``, ``final_states`` and ``workspace`` may be passed pre-allocated (e.g.
    for timing loops); otherwise they are allocated with ``torch.empty``.
    """
    return _fwd(None, x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus, y,
                final_states, workspace, stream, want_final)


def fwd_gated(x, dt, A, B, C, chunk, z, D=None, initial_states=None, seq_idx=None, nseq=None,
              dt_softplus=True, y=None, final_states=None, workspace=None, stream=None,
              want_final=True):
    """y * SiLU(z), final_states (``ssd_fwd_gated``): the forward with the block's
    gate fused into its last kernel; z is [b,T,H,P] like x."""
    return _fwd(z, x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus, y,
                final_states, workspace, stream, want_final)


def fwd_noalloc(x, dt, A, B, C, chunk, D=None, initial_states=None, seq_idx=None, nseq=None,
                dt_softplus=True, y=None, final_states=None, stream=None, want_final=True):
    """y, final_states = SSD forward through ``ssd_fwd_noalloc``: the library's
    static device scratch replaces the workspace (the problem's workspace must fit
    ``NOALLOC_SCRATCH_BYTES``).  Pass ``y`` and ``final_states`` pre-allocated for
    a call that allocates nothing at all."""
    p = Problem(x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus)
    if y is None:
        y = p.empty(x.shape)
    _check(y, "y", x.dtype, x.shape, p.device)
    if want_final and final_states is None:
        final_states = p.empty(p.final_shape(), torch.float32)
    _check(final_states, "final_states", torch.float32, p.final_shape(), p.device)
    p.args.y = _ptr(y)
    p.args.final_states = _ptr(final_states)
    p.call("ssd_fwd_noalloc", stream=stream)
    return y, final_states


def _fwd(z, x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus, y, final_states,
         workspace, stream, want_final):
    p = Problem(x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus)
    if z is not None:
        _check(z, "z", x.dtype, x.shape, p.device)
    if y is None:
        y = p.empty(x.shape)
    _check(y, "y", x.dtype, x.shape, p.device)
    if want_final and final_states is None:
        final_states = p.empty(p.final_shape(), torch.float32)
    _check(final_states, "final_states", torch.float32, p.final_shape(), p.device)
    need = workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=p.device)
    _check(workspace, "workspace", torch.uint8, None, p.device)
    p.args.y = _ptr(y)
    p.args.final_states = _ptr(final_states)
    p.args.workspace = _ptr(workspace)
    p.args.workspace_bytes = workspace.numel()
    if z is None:
        p.call("ssd_fwd", stream=stream)
    else:
        p.call("ssd_fwd_gated", _ptr(z), stream=stream)
    return y, final_states


# ---------------------------------------------------------------------------
# the block's convolution prologue
# ---------------------------------------------------------------------------

def conv1d_silu(xbc, weight, nheads, headdim, ngroups, dstate, bias=None, seq_idx=None, x=None, B=None, C=None,
                stream=None):
    """x, B, C = split(SiLU(causal depthwise conv1d(xbc) + bias)) (``ssd_conv1d_silu``):
    xbc [b,T,H*P + 2*G*N] fp32/bf16, weight [H*P + 2*G*N, width] fp32, bias fp32 or
    None, seq_idx [T] int32 or None (batch 1); x [b,T,H,P], B and C [b,T,G,N]."""
    if xbc.dim() != 3:
        raise ValueError("xbc must be [batch, seqlen, channels]")
    if xbc.dtype not in _DTYPES:
        raise TypeError("xbc must be float32 or bfloat16")
    b, T, CC = xbc.shape
    dev = xbc.device
    if CC != nheads * headdim + 2 * ngroups * dstate:
        raise ValueError("xbc must have nheads*headdim + 2*ngroups*dstate channels")
    _check(xbc, "xbc", device=dev)
    if weight.dim() != 2:
        raise ValueError("weight must be [channels, width]")
    _check(weight, "weight", torch.float32, (CC, weight.shape[1]), dev)
    _check(bias, "bias", torch.float32, (CC,), dev)
    if seq_idx is not None:
        _check(seq_idx, "seq_idx", torch.int32, (T,), dev)
    x = torch.empty((b, T, nheads, headdim), dtype=xbc.dtype, device=dev) if x is None else x
    B = torch.empty((b, T, ngroups, dstate), dtype=xbc.dtype, device=dev) if B is None else B
    C = torch.empty((b, T, ngroups, dstate), dtype=xbc.dtype, device=dev) if C is None else C
    _check(x, "x", xbc.dtype, (b, T, nheads, headdim), dev)
    _check(B, "B", xbc.dtype, (b, T, ngroups, dstate), dev)
    _check(C, "C", xbc.dtype, (b, T, ngroups, dstate), dev)
    a = ConvArgs(batch=b, seqlen=T, nheads=nheads, headdim=headdim, ngroups=ngroups, dstate=dstate,
                 width=weight.shape[1], dtype=_DTYPES[xbc.dtype], reserved=0, xbc=_ptr(xbc), weight=_ptr(weight),
                 bias=_ptr(bias), seq_idx=_ptr(seq_idx), x=_ptr(x), B=_ptr(B), C=_ptr(C))
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    rc = load_library().ssd_conv1d_silu(ctypes.byref(a), ctypes.c_void_p(st))
    if rc != 0:
        raise SSDError(rc, "ssd_conv1d_silu")
    return x, B, C


# ---------------------------------------------------------------------------
# per-step entry points (explicit intermediates; used for per-kernel checks and
# per-kernel timing)
# ---------------------------------------------------------------------------

def chunk_cumsum(p: Problem, delta=None, cs=None, stream=None):
    shape = (p.b, p.H, p.nc, p.Q)
    delta = p.empty(shape, torch.float32) if delta is None else delta
    cs = p.empty(shape, torch.float32) if cs is None else cs
    _check(delta, "delta", torch.float32, shape, p.device)
    _check(cs, "cs", torch.float32, shape, p.device)
    p.call("ssd_chunk_cumsum", _ptr(delta), _ptr(cs), stream=stream)
    return delta, cs


def chunk_cb(p: Problem, cb=None, stream=None):
    shape = p.cb_shape()
    cb = p.empty(shape) if cb is None else cb
    _check(cb, "cb", p.dtype, shape, p.device)
    p.call("ssd_chunk_cb", _ptr(cb), stream=stream)
    return cb


def chunk_state(p: Problem, delta, cs, cb, states=None, stream=None):
    """Chunk end states; also (re)writes ``delta`` and ``cs`` (the cumsum step)."""
    shape = (p.b, p.nc, p.H, p.P, p.N)
    cshape = (p.b, p.H, p.nc, p.Q)
    _check(delta, "delta", torch.float32, cshape, p.device)
    _check(cs, "cs", torch.float32, cshape, p.device)
    states = p.empty(shape) if states is None else states
    _check(cb, "cb", p.dtype, p.cb_shape(), p.device)
    _check(states, "states", p.dtype, shape, p.device)
    p.call("ssd_chunk_state", _ptr(delta), _ptr(cs), _ptr(cb), _ptr(states), stream=stream)
    return states


def state_passing(p: Problem, cs, states, final_states=None, stream=None):
    """In place: ``states`` (chunk-local end states) becomes the entering states."""
    _check(states, "states", p.dtype, (p.b, p.nc, p.H, p.P, p.N), p.device)
    if final_states is not None:
        _check(final_states, "final_states", torch.float32, p.final_shape(), p.device)
    p.args.final_states = _ptr(final_states)
    try:
        p.call("ssd_state_passing", _ptr(cs), _ptr(states), stream=stream)
    finally:
        p.args.final_states = None
    return states, final_states


def seq_final_states(p: Problem, delta, cs, states, final_states=None, seg_end=None, stream=None):
    final_states = p.empty(p.final_shape(), torch.float32) if final_states is None else final_states
    _check(final_states, "final_states", torch.float32, p.final_shape(), p.device)
    seg_end = p.empty((max(p.nseq, 1),), torch.int32) if seg_end is None else seg_end
    p.args.final_states = _ptr(final_states)
    try:
        p.call("ssd_seq_final_states", _ptr(delta), _ptr(cs), _ptr(states), _ptr(seg_end),
               stream=stream)
    finally:
        p.args.final_states = None
    return final_states


def chunk_scan(p: Problem, delta, cs, cb, states, y=None, stream=None):
    y = p.empty(p.x.shape) if y is None else y
    _check(y, "y", p.dtype, p.x.shape, p.device)
    _check(cb, "cb", p.dtype, p.cb_shape(), p.device)
    p.args.y = _ptr(y)
    try:
        p.call("ssd_chunk_scan", _ptr(delta), _ptr(cs), _ptr(cb), _ptr(states), stream=stream)
    finally:
        p.args.y = None
    return y


# ---------------------------------------------------------------------------
# decode: one recurrence step per batch row, state updated in place
# ---------------------------------------------------------------------------

def step_args(x, dt, A, B, C, state, D=None, dt_softplus=True, y=None):
    """Validated ``StepArgs`` (and y) for ``ssd_step``: x [b,H,P], dt [b,H], A [H],
    B and C [b,G,N], state [b,H,P,N] fp32 (updated in place), D [H] or None."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, nheads, headdim]")
    b, H, P = x.shape
    if B.dim() != 3:
        raise ValueError("B must be [batch, ngroups, dstate]")
    G, N = B.shape[1], B.shape[2]
    if x.dtype not in _DTYPES:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    _check(x, "x", device=dev)
    _check(dt, "dt", x.dtype, (b, H), dev)
    _check(A, "A", torch.float32, (H,), dev)
    _check(B, "B", x.dtype, (b, G, N), dev)
    _check(C, "C", x.dtype, (b, G, N), dev)
    _check(D, "D", torch.float32, (H,), dev)
    _check(state, "state", torch.float32, (b, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", x.dtype, (b, H, P), dev)
    a = StepArgs(batch=b, nheads=H, headdim=P, dstate=N, ngroups=G, dtype=_DTYPES[x.dtype],
                 dt_softplus=1 if dt_softplus else 0, x=_ptr(x), dt=_ptr(dt), A=_ptr(A), B=_ptr(B),
                 C=_ptr(C), D=_ptr(D), state=_ptr(state), y=_ptr(y))
    return a, y


def step(x, dt, A, B, C, state, D=None, dt_softplus=True, y=None, stream=None):
    """y = one decode step (``ssd_step``); ``state`` is updated in place."""
    a, y = step_args(x, dt, A, B, C, state, D, dt_softplus, y)
    lib = load_library()
    st = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    rc = lib.ssd_step(ctypes.byref(a), ctypes.c_void_p(st))
    if rc != 0:
        raise SSDError(rc, "ssd_step")
    return y


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def bwd_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().ssd_bwd_workspace_size(ctypes.byref(p.args), ctypes.byref(n))
    if rc != 0:
        raise SSDError(rc, "ssd_bwd_workspace_size")
    return int(n.value)


def bwd(x, dt, A, B, C, chunk, y, dy, D=None, initial_states=None, dfinal_states=None, dt_softplus=True,
        grads=None, workspace=None, stream=None, want_dinit=True, fwd_workspace=None, seq_idx=None, nseq=None,
        stage_times=None):
    """Gradients of sum(y * dy) + sum(final_states * dfinal_states) (see ``ssd_bwd``
    in ``include/ssd.h``).  ``y`` is the forward output.  Returns a dict with dx,
    ddt, dA, dB, dC, dD (None without D) and dinitial_states (None unless
    ``want_dinit``); ``grads`` may pass those tensors pre-allocated.
    ``fwd_workspace``: the workspace of the ``fwd`` call that produced ``y`` (on
    these same inputs, untouched since), whose chunk intermediates are then read
    instead of recomputed (not for packed streams).  With ``seq_idx`` (packed
    streams, batch 1) ``dfinal_states`` is [nseq, H, P, N], one per segment.
    ``stage_times``: a list that receives (stage name, ms) pairs; the call then
    goes through ``ssd_bwd_stage_times`` and waits for the stream."""
    p = Problem(x, dt, A, B, C, chunk, D, initial_states, seq_idx, nseq, dt_softplus)
    _check(y, "y", x.dtype, x.shape, p.device)
    _check(dy, "dy", x.dtype, x.shape, p.device)
    _check(dfinal_states, "dfinal_states", torch.float32, p.final_shape(), p.device)
    g = dict(grads or {})
    g.setdefault("dx", p.empty(x.shape))
    g.setdefault("ddt", p.empty(dt.shape))
    g.setdefault("dA", p.empty((p.H,), torch.float32))
    g.setdefault("dB", p.empty(B.shape))
    g.setdefault("dC", p.empty(C.shape))
    g.setdefault("dD", p.empty((p.H,), torch.float32) if D is not None else None)
    g.setdefault("dinitial_states", p.empty((p.b, p.H, p.P, p.N), torch.float32) if want_dinit else None)
    _check(g["dx"], "dx", x.dtype, x.shape, p.device)
    _check(g["ddt"], "ddt", x.dtype, dt.shape, p.device)
    _check(g["dA"], "dA", torch.float32, (p.H,), p.device)
    _check(g["dB"], "dB", x.dtype, B.shape, p.device)
    _check(g["dC"], "dC", x.dtype, C.shape, p.device)
    _check(g["dD"], "dD", torch.float32, (p.H,), p.device)
    _check(g["dinitial_states"], "dinitial_states", torch.float32, (p.b, p.H, p.P, p.N), p.device)
    need = bwd_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=p.device)
    _check(workspace, "workspace", torch.uint8, None, p.device)
    _check(fwd_workspace, "fwd_workspace", torch.uint8, None, p.device)
    p.args.y = _ptr(y)
    ga = BwdArgs(dy=_ptr(dy), dfinal_states=_ptr(dfinal_states), dx=_ptr(g["dx"]), ddt=_ptr(g["ddt"]),
                 dA=_ptr(g["dA"]), dB=_ptr(g["dB"]), dC=_ptr(g["dC"]), dD=_ptr(g["dD"]),
                 dinitial_states=_ptr(g["dinitial_states"]), workspace=_ptr(workspace),
                 workspace_bytes=workspace.numel(), fwd_workspace=_ptr(fwd_workspace),
                 fwd_workspace_bytes=0 if fwd_workspace is None else fwd_workspace.numel())
    st = stream if stream is not None else torch.cuda.current_stream(p.device).cuda_stream
    if stage_times is None:
        rc = load_library().ssd_bwd(ctypes.byref(p.args), ctypes.byref(ga), ctypes.c_void_p(st))
        if rc != 0:
            raise SSDError(rc, "ssd_bwd")
        return g
    ms = (ctypes.c_float * BWD_MAX_STAGES)()
    names = (ctypes.c_char_p * BWD_MAX_STAGES)()
    n = ctypes.c_int(0)
    rc = load_library().ssd_bwd_stage_times(ctypes.byref(p.args), ctypes.byref(ga), ctypes.c_void_p(st),
                                            BWD_MAX_STAGES, ms, names, ctypes.byref(n))
    if rc != 0:
        raise SSDError(rc, "ssd_bwd_stage_times")
    stage_times.extend((names[i].decode(), float(ms[i])) for i in range(n.value))
    return g
