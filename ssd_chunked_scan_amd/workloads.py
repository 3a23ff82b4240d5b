"""Seeded synthetic inputs for the SSD forward pass.

This module only draws random numbers: it holds none of the method's
arithmetic (no softplus, no decay, no recurrence), so the GPU path and the CPU
oracle can both be fed from it without sharing any computation.

Every tensor is drawn in fp64 from ``numpy.random.Generator(PCG64(seed))``,
cast to fp32, and for bf16 workloads rounded to bf16 (round-to-nearest-even,
torch's CPU cast).  A, D and the initial states stay fp32.  Draw order:
(packed workloads: the sequence lengths) -> A -> D -> dt -> x -> B -> C ->
(optional) initial states.

Distributions (shapes follow the workloads the pages discuss: 2K sequences at
batch 8, a 2.7B-scale model, 16K sequences, state sizes 64-256, chunk 64-256,
packed variable-length sequences):

    x ~ N(0, 1)            B, C ~ N(0, 1) / sqrt(N)       D ~ N(0, 1)
    A_h = -exp(U[0, log 16])  (or a caller-chosen log-range; A = 0 allowed)
    dt  ~ N(mu, 0.5) passed raw with softplus on, so Delta = softplus(dt)
    initial states ~ N(0, std) when requested

Packed workloads concatenate sequences of lengths U[lo, hi] into one stream
(batch 1), pad it to a multiple of the chunk length, and label the padding as a
segment of its own with x = B = C = 0.

``device_inputs`` draws the same recipe on the GPU with torch's generator, for
the maximum-size cases whose host draw would be too large (billions of
elements).

The block around the SSD (``block_inputs``, its own seed) draws the
pre-convolution channels xBC ~ N(0, 1), depthwise taps and bias ~ U[-1/sqrt(w),
1/sqrt(w)] for w taps, and the gate input z ~ N(0, 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# The five workload shapes.  Index = workload id; ``seed = 1000 + id``.
WORKLOADS = {
    0: dict(name="tiny_fp32_T256", batch=1, seqlen=256, nheads=2, headdim=16, dstate=16,
            ngroups=1, chunk=64, dtype="fp32", dt_mean=-2.0, init_std=None),
    1: dict(name="small_bf16_b2_T2048_H24_N64", batch=2, seqlen=2048, nheads=24, headdim=64,
            dstate=64, ngroups=1, chunk=64, dtype="bf16", dt_mean=-2.0, init_std=0.1),
    2: dict(name="2.7B_bf16_b8_T2048_H80_N128", batch=8, seqlen=2048, nheads=80, headdim=64,
            dstate=128, ngroups=1, chunk=128, dtype="bf16", dt_mean=-2.0, init_std=None),
    3: dict(name="long_bf16_b1_T16384_H32_N256", batch=1, seqlen=16384, nheads=32, headdim=64,
            dstate=256, ngroups=1, chunk=256, dtype="bf16", dt_mean=-3.0, init_std=None),
    4: dict(name="packed16_bf16_H64_N128_G8", batch=1, seqlen=None, nheads=64, headdim=64,
            dstate=128, ngroups=8, chunk=128, dtype="bf16", dt_mean=-2.0, init_std=None,
            packed=dict(nseqs=16, lo=128, hi=2048)),
}


# Decode (one token per sequence, the state carried): the 2.7B-scale heads at a
# serving batch of 64 sequences; the carried state ~ N(0, 0.5).  Seed 2000.
DECODE = dict(name="decode_2.7B_bf16_b64_H80_N128", batch=64, nheads=80, headdim=64, dstate=128,
              ngroups=1, dtype="bf16", dt_mean=-2.0, init_std=0.5)


@dataclass
class StepInputs:
    x: torch.Tensor                 # [b,H,P]  dtype
    dt: torch.Tensor                # [b,H]    dtype (raw, softplus applied downstream)
    A: torch.Tensor                 # [H] fp32
    B: torch.Tensor                 # [b,G,N]  dtype
    C: torch.Tensor                 # [b,G,N]  dtype
    D: Optional[torch.Tensor]       # [H] fp32
    state: torch.Tensor             # [b,H,P,N] fp32, the carried state
    dt_softplus: bool = True
    name: str = ""

    def to(self, device) -> "StepInputs":
        mv = lambda t: None if t is None else t.to(device).contiguous()
        return StepInputs(mv(self.x), mv(self.dt), mv(self.A), mv(self.B), mv(self.C), mv(self.D),
                          mv(self.state), self.dt_softplus, self.name)


@dataclass
class Inputs:
    x: torch.Tensor                 # [b,T,H,P]  workload dtype
    dt: torch.Tensor                # [b,T,H]    workload dtype (raw, softplus applied downstream)
    A: torch.Tensor                 # [H] fp32
    B: torch.Tensor                 # [b,T,G,N]  workload dtype
    C: torch.Tensor                 # [b,T,G,N]  workload dtype
    D: Optional[torch.Tensor]       # [H] fp32
    initial_states: Optional[torch.Tensor]  # [b,H,P,N] fp32
    seq_idx: Optional[torch.Tensor]  # [T] int32 (batch 1 only)
    nseq: int                        # number of segment ids (0 when not packed)
    chunk: int
    dt_softplus: bool = True
    lengths: list = field(default_factory=list)   # real sequence lengths (packed)
    real_tokens: int = 0                           # tokens that carry data (excludes padding)
    name: str = ""

    @property
    def shape(self):
        b, T, H, P = self.x.shape
        return dict(batch=b, seqlen=T, nheads=H, headdim=P, dstate=self.B.shape[3],
                    ngroups=self.B.shape[2], chunk=self.chunk)

    def to(self, device) -> "Inputs":
        mv = lambda t: None if t is None else t.to(device).contiguous()
        return Inputs(mv(self.x), mv(self.dt), mv(self.A), mv(self.B), mv(self.C), mv(self.D),
                      mv(self.initial_states), mv(self.seq_idx), self.nseq, self.chunk,
                      self.dt_softplus, list(self.lengths), self.real_tokens, self.name)


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a.astype(np.float32)))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype}")
    return t.contiguous()


def make_inputs(batch: int, seqlen: Optional[int], nheads: int, headdim: int, dstate: int,
                ngroups: int, chunk: int, dtype: str, seed: int, dt_mean: float = -2.0,
                dt_std: float = 0.5, a_log_range=(0.0, math.log(16.0)), a_zero: bool = False,
                init_std: Optional[float] = None, with_d: bool = True,
                packed: Optional[dict] = None, name: str = "") -> Inputs:
    """Draw one seeded input set (see the module docstring for the recipe)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = []
    seq_idx = None
    nseq = 0
    if packed is not None:
        lengths = [int(v) for v in rng.integers(packed["lo"], packed["hi"], size=packed["nseqs"],
                                                endpoint=True)]
        real = sum(lengths)
        seqlen = ((real + chunk - 1) // chunk) * chunk
        ids = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(lengths)])
        nseq = len(lengths)
        if seqlen > real:  # the padding is a segment of its own
            ids = np.concatenate([ids, np.full(seqlen - real, nseq, np.int32)])
            nseq += 1
        seq_idx = torch.from_numpy(ids)
        real_tokens = real
    else:
        real_tokens = batch * seqlen
    T, H, P, N, G = seqlen, nheads, headdim, dstate, ngroups

    lo, hi = a_log_range
    A = -np.exp(rng.uniform(lo, hi, size=H))
    if a_zero:
        A = np.zeros(H)
    D = rng.standard_normal(H)
    dt = rng.normal(dt_mean, dt_std, size=(batch, T, H))
    x = rng.standard_normal((batch, T, H, P))
    Bm = rng.standard_normal((batch, T, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal((batch, T, G, N)) / math.sqrt(N)
    init = rng.normal(0.0, init_std, size=(batch, H, P, N)) if init_std is not None else None
    if packed is not None and seqlen > sum(lengths):
        real = sum(lengths)
        x[:, real:] = 0.0
        Bm[:, real:] = 0.0
        Cm[:, real:] = 0.0

    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a.astype(np.float32)))
    return Inputs(
        x=_cast(x, dtype), dt=_cast(dt, dtype), A=f32(A), B=_cast(Bm, dtype), C=_cast(Cm, dtype),
        D=f32(D) if with_d else None, initial_states=None if init is None else f32(init),
        seq_idx=seq_idx, nseq=nseq, chunk=chunk, dt_softplus=True, lengths=lengths,
        real_tokens=real_tokens, name=name)


def workload(idx: int, **overrides) -> Inputs:
    """The seeded inputs of workload ``idx`` (seed 1000 + idx); ``overrides`` may
    change shape fields for reduced-size variants of the same recipe."""
    cfg = dict(WORKLOADS[idx])
    cfg.update(overrides)
    name = cfg.pop("name")
    seed = cfg.pop("seed", 1000 + idx)
    return make_inputs(seed=seed, name=name, **cfg)


def token(inp: "Inputs", t: int, state: Optional[torch.Tensor] = None) -> StepInputs:
    """Token t of every batch row of ``inp`` as decode-step inputs, carrying
    ``state`` (default: ``inp``'s initial states, or zeros)."""
    b, T, H, P = inp.x.shape
    N = inp.B.shape[3]
    if state is None:
        state = inp.initial_states if inp.initial_states is not None else torch.zeros(b, H, P, N)
    c = lambda a: a[:, t].contiguous()
    return StepInputs(c(inp.x), c(inp.dt), inp.A, c(inp.B), c(inp.C), inp.D, state.contiguous(),
                      inp.dt_softplus, inp.name)


def decode_inputs(seed: int = 2000, **overrides) -> StepInputs:
    """The seeded decode-step inputs (``DECODE``, optionally with shape
    overrides): one token per batch row drawn by the same recipe as the
    forward workloads, and a carried state ~ N(0, init_std)."""
    cfg = dict(DECODE)
    cfg.update(overrides)
    inp = make_inputs(cfg["batch"], 1, cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"], 64,
                      cfg["dtype"], seed, dt_mean=cfg["dt_mean"], init_std=cfg["init_std"], name=cfg["name"])
    return token(inp, 0)


def device_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int, chunk: int,
                  dtype: str, seed: int, device, dt_mean: float = -3.0, dt_std: float = 0.5,
                  init_std: Optional[float] = 0.1, name: str = "") -> Inputs:
    """The same recipe and draw order as ``make_inputs``, drawn on ``device`` by
    torch's generator (seeded with ``seed``) for sizes whose fp64 host draw would
    not fit in host memory or time: billions of elements.  x, dt, B and C are
    drawn in fp32 and rounded to bf16 on the device for bf16 inputs; A, D and
    the initial states stay fp32.  The values differ from ``make_inputs``'s for
    the same seed (a different generator); the distributions are the same."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    T, H, P, N, G = seqlen, nheads, headdim, dstate, ngroups
    el = torch.bfloat16 if dtype == "bf16" else torch.float32
    kw = dict(device=device, generator=gen)
    A = -torch.exp(torch.rand(H, **kw) * math.log(16.0))
    D = torch.randn(H, **kw)
    dt = (torch.randn(batch, T, H, **kw) * dt_std + dt_mean).to(el)
    x = torch.empty(batch, T, H, P, dtype=el, device=device)
    for t0 in range(0, T, 1 << 16):   # in slabs, so no fp32 copy of all of x is held at once
        t1 = min(T, t0 + (1 << 16))
        x[:, t0:t1] = torch.randn(batch, t1 - t0, H, P, **kw).to(el)
    Bm = (torch.randn(batch, T, G, N, **kw) / math.sqrt(N)).to(el)
    Cm = (torch.randn(batch, T, G, N, **kw) / math.sqrt(N)).to(el)
    init = torch.randn(batch, H, P, N, **kw) * init_std if init_std is not None else None
    return Inputs(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, initial_states=init, seq_idx=None, nseq=0, chunk=chunk,
                  dt_softplus=True, lengths=[], real_tokens=batch * T, name=name)


@dataclass
class BlockInputs:
    """The Mamba-2 block's tensors on either side of the SSD for one ``Inputs``:
    the pre-convolution main path xBC = [x | B | C], its depthwise taps and bias,
    and the gate path z.  dt, A, D, initial states and the packing come from the
    ``Inputs`` (its x, B and C are not used: the convolution produces them)."""
    xbc: torch.Tensor               # [b,T,H*P + 2*G*N] workload dtype
    weight: torch.Tensor            # [H*P + 2*G*N, width] fp32
    bias: Optional[torch.Tensor]    # [H*P + 2*G*N] fp32
    z: torch.Tensor                 # [b,T,H,P] workload dtype
    width: int = 4


def block_inputs(inp: Inputs, seed: int, width: int = 4, with_bias: bool = True) -> BlockInputs:
    """Seeded block tensors drawn in fp64 from ``PCG64(seed)`` in the order
    xbc -> weight -> bias -> z: xbc, z ~ N(0, 1); weight and bias ~ U[-1/sqrt(width),
    1/sqrt(width)] (the usual fan-in scale of a depthwise convolution).  In packed
    inputs the padding tokens' xbc is zero, like the forward's padding."""
    rng = np.random.Generator(np.random.PCG64(seed))
    b, T, H, P = inp.x.shape
    G, N = inp.B.shape[2], inp.B.shape[3]
    CC = H * P + 2 * G * N
    dtype = "bf16" if inp.x.dtype == torch.bfloat16 else "fp32"
    xbc = rng.standard_normal((b, T, CC))
    bound = 1.0 / math.sqrt(width)
    w = rng.uniform(-bound, bound, size=(CC, width))
    bias = rng.uniform(-bound, bound, size=CC)
    z = rng.standard_normal((b, T, H, P))
    if inp.seq_idx is not None and inp.real_tokens < T:
        xbc[:, inp.real_tokens:] = 0.0
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a.astype(np.float32)))
    return BlockInputs(xbc=_cast(xbc, dtype), weight=f32(w), bias=f32(bias) if with_bias else None,
                       z=_cast(z, dtype), width=width)
