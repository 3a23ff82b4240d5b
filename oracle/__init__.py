"""fp64 CPU oracle for the scalar-decay multi-head SSM forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The GPU product path
never calls it and shares no code with it.

The heavy lifting is the C recurrence in ``ssd_oracle.c`` (loaded with ctypes);
this module only converts arrays to contiguous fp64 and back.  Inputs given in
bf16 or fp32 are upcast exactly, so the oracle sees the very values the GPU
sees.

``backward`` is the reverse-mode derivative of that recurrence (the chain rule
applied step by step in reverse; the pages give no backward equations),
``step`` is the recurrence over one token (the decode step), and
``conv1d_silu`` / ``gated`` are the block's steps on either side of the SSD
(causal depthwise convolution + SiLU before it, the SiLU gate after it), in
plain fp64 numpy.

``forward`` follows the literal recurrence of the "Mamba 2 -- Transformers are
SSMs" paper story (ai.tomabc.com), section 3.1: ``h_t = a_t h_{t-1} +
Delta_t B_t x_t^T``, ``y_t = C_t^T h_t`` (+ ``D x_t``), with ``a_t =
exp(Delta_t A)``; ``chunk_cumsum`` gives Delta and the within-chunk cumulative
log-decay.  See ``ssd_oracle.c`` for every reading taken where the pages are
silent.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .build import LIB, build_oracle

_lib = None


class _Args(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("dt_softplus", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p), ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("initial_states", ctypes.c_void_p), ("seq_idx", ctypes.c_void_p),
        ("nseq", ctypes.c_int64), ("unit_mask", ctypes.c_void_p),
        ("chunk", ctypes.c_int64), ("chunk_local", ctypes.c_int32),
        ("y", ctypes.c_void_p), ("final_states", ctypes.c_void_p),
        ("chunk_end_states", ctypes.c_void_p),
    ]


def load():
    """Load ``libssd_oracle.so``, compiling it first only if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        lib.ssd_oracle_forward.argtypes = [ctypes.POINTER(_Args)]
        lib.ssd_oracle_forward.restype = ctypes.c_int
        lib.ssd_oracle_chunk_cumsum.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int32] + [ctypes.c_void_p] * 5
        lib.ssd_oracle_chunk_cumsum.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        lib.ssd_oracle_backward.argtypes = [ctypes.POINTER(_BwdArgs)]
        lib.ssd_oracle_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(load().ssd_oracle_max_threads())


def _f64(a) -> np.ndarray:
    """Exact upcast of a numpy array or CPU torch tensor (any float dtype) to fp64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (bf16 has no numpy dtype: go through fp32, exact)
        import torch
        a = a.detach().to("cpu")
        if a.dtype == torch.bfloat16 or a.dtype == torch.float16:
            a = a.to(torch.float32)
        a = a.numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


@dataclass
class OracleResult:
    y: np.ndarray                      # [b,T,H,P]
    final_states: Optional[np.ndarray]  # [b,H,P,N] or [nseq,H,P,N]
    chunk_end_states: Optional[np.ndarray]  # [b,nc,H,P,N]


def forward(x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, nseq=None,
            dt_softplus=True, chunk=0, chunk_local=False, want_chunk_states=False,
            unit_mask=None) -> OracleResult:
    """Run the recurrence.  Shapes: x[b,T,H,P], dt[b,T,H], A[H], B,C[b,T,G,N].

    ``unit_mask`` ([b,H] bool, optional) restricts the work to sampled (b, h)
    pairs; outputs of the others are left at zero.
    """
    x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
    D = _f64(D)
    init = _f64(initial_states)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, T, H) and A.shape == (H,)
    assert B.shape == (b, T, G, N) and C.shape == (b, T, G, N)
    sidx = None
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        sidx = np.ascontiguousarray(np.asarray(seq_idx).reshape(-1), dtype=np.int32)
        assert sidx.shape == (T,) and b == 1
        if nseq is None:
            nseq = int(sidx.max()) + 1
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(b * H))
    y = np.zeros((b, T, H, P), np.float64)
    fs = np.zeros(((nseq if sidx is not None else b), H, P, N), np.float64)
    nc = (T + chunk - 1) // chunk if chunk > 0 else 0
    ces = np.zeros((b, nc, H, P, N), np.float64) if want_chunk_states else None
    args = _Args(b, T, H, P, N, G, int(bool(dt_softplus)),
                 _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(sidx),
                 int(nseq or 0), _ptr(mask), int(chunk), int(bool(chunk_local)),
                 _ptr(y), _ptr(fs), _ptr(ces))
    rc = load().ssd_oracle_forward(ctypes.byref(args))
    if rc != 0:
        raise ValueError(f"ssd_oracle_forward failed with status {rc}")
    return OracleResult(y, fs, ces)


class _BwdArgs(ctypes.Structure):
    _fields_ = [("f", _Args), ("dy", ctypes.c_void_p), ("dfinal", ctypes.c_void_p), ("dx", ctypes.c_void_p),
                ("ddt", ctypes.c_void_p), ("dA", ctypes.c_void_p), ("dB", ctypes.c_void_p),
                ("dC", ctypes.c_void_p), ("dD", ctypes.c_void_p), ("dinit", ctypes.c_void_p)]


@dataclass
class OracleGrads:
    dx: np.ndarray       # [b,T,H,P]
    ddt: np.ndarray      # [b,T,H]
    dA: np.ndarray       # [H]
    dB: np.ndarray       # [b,T,G,N]
    dC: np.ndarray       # [b,T,G,N]
    dD: Optional[np.ndarray]      # [H] (None when D is None)
    dinit: np.ndarray    # [b,H,P,N]


def backward(x, dt, A, B, C, dy, D=None, initial_states=None, dfinal=None, seq_idx=None, nseq=None,
             dt_softplus=True) -> OracleGrads:
    """Gradients of L = sum(y * dy) + sum(final_states * dfinal) with respect to
    every input of ``forward``: the chain rule applied to the recurrence, one
    step at a time in reverse (see ``ssd_oracle_backward`` in ``ssd_oracle.c``)."""
    x, dt, A, B, C, dy = map(_f64, (x, dt, A, B, C, dy))
    D, init, dfin = _f64(D), _f64(initial_states), _f64(dfinal)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape
    sidx = None
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        sidx = np.ascontiguousarray(np.asarray(seq_idx).reshape(-1), dtype=np.int32)
        if nseq is None:
            nseq = int(sidx.max()) + 1
    out = OracleGrads(np.zeros_like(x), np.zeros((b, T, H)), np.zeros(H), np.zeros((b, T, G, N)),
                      np.zeros((b, T, G, N)), None if D is None else np.zeros(H), np.zeros((b, H, P, N)))
    f = _Args(b, T, H, P, N, G, int(bool(dt_softplus)),
              _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(sidx),
              int(nseq or 0), None, 0, 0, None, None, None)
    args = _BwdArgs(f, _ptr(dy), _ptr(dfin), _ptr(out.dx), _ptr(out.ddt), _ptr(out.dA), _ptr(out.dB),
                    _ptr(out.dC), _ptr(out.dD), _ptr(out.dinit))
    rc = load().ssd_oracle_backward(ctypes.byref(args))
    if rc != 0:
        raise ValueError(f"ssd_oracle_backward failed with status {rc}")
    return out


def step(x, dt, A, B, C, state, D=None, dt_softplus=True):
    """One step of the recurrence for one new token per batch row (the
    recurrent, constant-memory mode of section 3.1 of "Mamba 2 -- Transformers
    are SSMs"): the literal recurrence above run over a sequence of length 1
    that starts from ``state``.  Shapes: x[b,H,P], dt[b,H], A[H], B,C[b,G,N],
    state[b,H,P,N].  Returns (y[b,H,P], new state[b,H,P,N]) in fp64; ``state`` is
    not modified."""
    x, dt, B, C = _f64(x), _f64(dt), _f64(B), _f64(C)
    r = forward(x[:, None], dt[:, None], A, B[:, None], C[:, None], D, state, dt_softplus=dt_softplus)
    return r.y[:, 0], r.final_states


def chunk_cumsum(dt, A, chunk, dt_softplus=True, seq_idx=None):
    """Delta and the within-chunk (and within-segment) inclusive cumsum of
    Delta*A, both [b,H,nc,Q] fp64."""
    dt, A = _f64(dt), _f64(A)
    sidx = None
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        sidx = np.ascontiguousarray(np.asarray(seq_idx).reshape(-1), dtype=np.int32)
    b, T, H = dt.shape
    nc = (T + chunk - 1) // chunk
    delta = np.zeros((b, H, nc, chunk), np.float64)
    cs = np.zeros((b, H, nc, chunk), np.float64)
    rc = load().ssd_oracle_chunk_cumsum(b, T, H, chunk, int(bool(dt_softplus)),
                                        _ptr(dt), _ptr(A), _ptr(sidx), _ptr(delta), _ptr(cs))
    if rc != 0:
        raise ValueError(f"ssd_oracle_chunk_cumsum failed with status {rc}")
    return delta, cs


def chunk_cb(B, C, chunk):
    """cb[b,c,g,t,s] = sum_n C[cQ+t,g,n] B[cQ+s,g,n] in fp64 (rows past T are zero):
    the Q K^T of the dual form ("Mamba 2 -- Transformers are SSMs" paper story,
    section 3.2, formula 1) restricted to one chunk, written as a plain matmul."""
    B, C = _f64(B), _f64(C)
    b, T, G, N = B.shape
    nc = (T + chunk - 1) // chunk
    pad = nc * chunk - T
    Bp = np.pad(B, ((0, 0), (0, pad), (0, 0), (0, 0))).reshape(b, nc, chunk, G, N)
    Cp = np.pad(C, ((0, 0), (0, pad), (0, 0), (0, 0))).reshape(b, nc, chunk, G, N)
    return np.einsum("bctgn,bcsgn->bcgts", Cp, Bp)


# ---------------------------------------------------------------------------
# the Mamba-2 block around the SSD ("SSM 家族全景图（下）：Mamba-2 与 Jamba",
# section five, the block's data flow): a causal one-dimensional convolution and
# a SiLU on the main path before the SSD, a SiLU on the gate path, and the
# elementwise product of the two paths.  Plain fp64 numpy, no C.
# ---------------------------------------------------------------------------

def silu(v):
    """SiLU(v) = v / (1 + e^-v), elementwise, fp64."""
    v = _f64(v)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def causal_conv1d(xbc, weight, bias=None, seq_idx=None):
    """Depthwise causal convolution over time, before the activation:
    ``v[b,t,c] = bias[c] + sum_k weight[c,k] * xbc[b, t-(K-1)+k, c]`` over taps k
    in [0, K), an input position counting only when it is >= 0 and, with
    ``seq_idx`` (batch 1), in the same segment as t (the convolution restarts
    with every packed sequence).  xbc [b,T,C], weight [C,K] -> v [b,T,C] fp64."""
    xbc, weight = _f64(xbc), _f64(weight)
    b, T, Cc = xbc.shape
    K = weight.shape[1]
    seg = None
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        seg = np.asarray(seq_idx).reshape(-1)
    v = np.zeros((b, T, Cc), np.float64)
    if bias is not None:
        v += _f64(bias)[None, None, :]
    for t in range(T):
        for k in range(K):
            s = t - (K - 1) + k
            if s < 0 or (seg is not None and seg[s] != seg[t]):
                continue
            v[:, t, :] += weight[None, :, k] * xbc[:, s, :]
    return v


def conv1d_silu(xbc, weight, nheads, headdim, ngroups, dstate, bias=None, seq_idx=None):
    """SiLU(causal_conv1d(...)) split along channels into x [b,T,H,P] (the first
    H*P channels), B and C [b,T,G,N] (the next G*N each), fp64."""
    a = silu(causal_conv1d(xbc, weight, bias, seq_idx))
    b, T, _ = a.shape
    hp, gn = nheads * headdim, ngroups * dstate
    x = a[:, :, :hp].reshape(b, T, nheads, headdim)
    Bm = a[:, :, hp:hp + gn].reshape(b, T, ngroups, dstate)
    Cm = a[:, :, hp + gn:hp + 2 * gn].reshape(b, T, ngroups, dstate)
    return x, Bm, Cm


def gated(y, z):
    """The gate of the block: y * SiLU(z), elementwise, fp64."""
    return _f64(y) * silu(z)
