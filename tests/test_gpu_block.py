"""GPU parity of the Mamba-2 block's steps around the SSD, through the C ABI,
against the fp64 oracle on the same seeded inputs:

  ssd_conv1d_silu -- causal depthwise convolution + SiLU, split into x, B, C.
      Per element: |got - ref| <= 2^-8 |ref| + 1e-5 for bf16 outputs (one
      round-to-nearest-even of an fp32 result, 2^-9 relative, plus fp32 sums of
      at most 4 taps), 1e-5 |ref| + 1e-6 for fp32 outputs.
  ssd_fwd_gated -- the forward with y * SiLU(z) in its last kernel: max relative
      L2 error per (batch, head) slice over (T, P) <= 1e-4 (fp32) and <= 2e-2
      (bf16), the forward's bars; final states bit-identical to ssd_fwd's.
  the two chained (the block from xBC and z to the gated output), with the same
      bars as the gated forward.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from ssd_chunked_scan_amd import ssd
from ssd_chunked_scan_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()
    torch.cuda.set_device(0)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else float(np.linalg.norm(a))


def worst_bh(got, ref):
    """max over (batch, head) of the relative L2 error over (T, P)"""
    b, _, H, _ = ref.shape
    return max(rel(got[i, :, h], ref[i, :, h]) for i in range(b) for h in range(H))


def check_elementwise(got, ref, dtype, what):
    g = f64(got)
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    else:
        bound = 1e-5 * np.abs(ref) + 1e-6
    err = np.abs(g - ref)
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float(err.max()), np.argwhere(bad)[:4].tolist())
    assert np.isfinite(g).all(), what


def run_conv(inp, blk, dtype, seq_idx=None):
    H, P = inp.x.shape[2], inp.x.shape[3]
    G, N = inp.B.shape[2], inp.B.shape[3]
    dev = "cuda:0"
    x, B, C = ssd.conv1d_silu(blk.xbc.to(dev), blk.weight.to(dev), H, P, G, N,
                              bias=None if blk.bias is None else blk.bias.to(dev),
                              seq_idx=None if seq_idx is None else seq_idx.to(dev))
    torch.cuda.synchronize()
    return x, B, C


def check_conv(inp, blk, dtype, label="", seq_idx=None):
    H, P = inp.x.shape[2], inp.x.shape[3]
    G, N = inp.B.shape[2], inp.B.shape[3]
    _log(f"[conv] {label} xbc={tuple(blk.xbc.shape)} H={H} P={P} G={G} N={N} width={blk.width} {dtype}")
    x, B, C = run_conv(inp, blk, dtype, seq_idx)
    rx, rB, rC = oracle.conv1d_silu(blk.xbc, blk.weight, H, P, G, N, blk.bias, seq_idx)
    check_elementwise(x, rx, dtype, "x")
    check_elementwise(B, rB, dtype, "B")
    check_elementwise(C, rC, dtype, "C")
    return x, B, C


# (b, T, H, P, G, N): T not a multiple of the 16-token blocks, T = 1, several
# channel splits (x, B and C of different widths), heads sharing groups
CONV_SHAPES = [(2, 37, 2, 16, 1, 16), (1, 1, 4, 32, 2, 16), (3, 100, 3, 48, 1, 64), (1, 257, 8, 64, 2, 128),
               (2, 16, 2, 80, 1, 32)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("width", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "b%d_T%d_H%d_P%d_G%d_N%d" % s)
def test_conv_matches_oracle(dtype, width, shape):
    b, T, H, P, G, N = shape
    inp = wl.make_inputs(b, T, H, P, N, G, 64, dtype, sum(shape) + width)
    blk = wl.block_inputs(inp, seed=T + width, width=width, with_bias=width != 2)
    check_conv(inp, blk, dtype, label=str(shape))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_conv_restarts_in_packed_sequences(dtype):
    inp = wl.make_inputs(1, None, 4, 32, 32, 1, 64, dtype, 77, packed=dict(nseqs=9, lo=1, hi=40))
    blk = wl.block_inputs(inp, seed=78)
    check_conv(inp, blk, dtype, label=f"packed {inp.lengths}", seq_idx=inp.seq_idx)


def _nan_tail(t, extra=4096):
    t = t.to("cuda:0")
    buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device=t.device)
    buf[:t.numel()] = t.reshape(-1)
    return buf[:t.numel()].view(t.shape)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_conv_reads_nothing_past_the_end(dtype):
    inp = wl.make_inputs(1, 21, 2, 16, 16, 1, 64, dtype, 9)
    blk = wl.block_inputs(inp, seed=10)
    x, B, C = ssd.conv1d_silu(_nan_tail(blk.xbc), _nan_tail(blk.weight), 2, 16, 1, 16, bias=_nan_tail(blk.bias))
    torch.cuda.synchronize()
    rx, rB, rC = oracle.conv1d_silu(blk.xbc, blk.weight, 2, 16, 1, 16, blk.bias)
    for got, ref, k in ((x, rx, "x"), (B, rB, "B"), (C, rC, "C")):
        check_elementwise(got, ref, dtype, k)


def gated_ref(inp, x, B, C, z, seq_idx=None, nseq=None):
    r = oracle.forward(x, inp.dt, inp.A, B, C, inp.D, inp.initial_states, seq_idx, nseq, inp.dt_softplus)
    return oracle.gated(r.y, z), r.final_states


def check_gated(inp, z, dtype, label=""):
    g = inp.to("cuda:0")
    _log(f"[gated] {label} x={tuple(inp.x.shape)} N={inp.B.shape[3]} Q={inp.chunk} {dtype}")
    kw = dict(D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx, nseq=inp.nseq or None,
              dt_softplus=inp.dt_softplus)
    y, fin = ssd.fwd_gated(g.x, g.dt, g.A, g.B, g.C, inp.chunk, z.to("cuda:0"), **kw)
    _, fin_plain = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, **kw)
    torch.cuda.synchronize()
    ref_y, _ = gated_ref(inp, inp.x, inp.B, inp.C, z, inp.seq_idx, inp.nseq or None)
    e = worst_bh(f64(y), ref_y)
    _log(f"    max rel-L2 gated y={e:.3e} (tol {TOL[dtype]:.0e})")
    assert e <= TOL[dtype]
    assert torch.isfinite(y).all()
    assert torch.equal(fin, fin_plain)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_fwd_gated_matches_oracle(dtype, Q):
    inp = wl.make_inputs(2, 2 * Q + 37, 4, 64, 64, 2, Q, dtype, Q + 3, init_std=0.3)
    z = wl.block_inputs(inp, seed=Q).z
    check_gated(inp, z, dtype, label=f"Q{Q}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [dict(P=32, N=128, H=2, G=1, T=150), dict(P=48, N=256, H=2, G=1, T=300),
                                   dict(P=16, N=16, H=2, G=2, T=1), dict(P=80, N=48, H=3, G=3, T=70)],
                         ids=lambda d: "P{P}_N{N}_H{H}_G{G}_T{T}".format(**d))
def test_fwd_gated_shapes(dtype, shape):
    inp = wl.make_inputs(1, shape["T"], shape["H"], shape["P"], shape["N"], shape["G"], 64, dtype,
                         shape["T"] + shape["P"], init_std=0.3)
    check_gated(inp, wl.block_inputs(inp, seed=shape["T"]).z, dtype, label=str(shape))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_gated_packed(dtype):
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, 64, dtype, 31, packed=dict(nseqs=6, lo=5, hi=150))
    check_gated(inp, wl.block_inputs(inp, seed=32).z, dtype, label=f"packed {inp.lengths}")


def check_block(inp, blk, dtype, label=""):
    """xBC and z -> conv + SiLU -> SSD -> y * SiLU(z), both sides end to end."""
    H, P = inp.x.shape[2], inp.x.shape[3]
    G, N = inp.B.shape[2], inp.B.shape[3]
    _log(f"[block] {label} T={inp.x.shape[1]} H={H} P={P} N={N} Q={inp.chunk} {dtype}")
    x, B, C = run_conv(inp, blk, dtype, inp.seq_idx)
    g = inp.to("cuda:0")
    y, _ = ssd.fwd_gated(x, g.dt, g.A, B, C, inp.chunk, blk.z.to("cuda:0"), D=g.D,
                         initial_states=g.initial_states, seq_idx=g.seq_idx, nseq=inp.nseq or None)
    torch.cuda.synchronize()
    # the oracle's chain starts from its own fp64 convolution, rounded to the
    # dtype the SSD takes (the GPU's x, B and C are rounded once, the same way)
    rx, rB, rC = oracle.conv1d_silu(blk.xbc, blk.weight, H, P, G, N, blk.bias, inp.seq_idx)
    cast = (lambda a: torch.from_numpy(a).to(torch.bfloat16)) if dtype == "bf16" else \
        (lambda a: torch.from_numpy(a).float())
    ref_y, _ = gated_ref(inp, cast(rx), cast(rB), cast(rC), blk.z, inp.seq_idx, inp.nseq or None)
    e = worst_bh(f64(y), ref_y)
    _log(f"    max rel-L2 block y={e:.3e} (tol {TOL[dtype]:.0e})")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_block_chain_matches_oracle(dtype):
    inp = wl.make_inputs(2, 300, 4, 64, 64, 1, 64, dtype, 51, init_std=0.3)
    check_block(inp, wl.block_inputs(inp, seed=52), dtype, label="small")


def test_block_chain_packed():
    inp = wl.make_inputs(1, None, 4, 64, 128, 2, 128, "bf16", 53, packed=dict(nseqs=5, lo=20, hi=300))
    check_block(inp, wl.block_inputs(inp, seed=54), "bf16", label=f"packed {inp.lengths}")


def test_block_small_workload_full_size():
    """The small workload's shape (2 x 2048 tokens, 24 heads of 64, N = 64, chunk 64,
    bf16) through the whole block."""
    inp = wl.workload(1)
    check_block(inp, wl.block_inputs(inp, seed=1101), "bf16", label=inp.name)


def test_block_long_workload_full_size():
    """The block measured by the benchmark: the long workload's shape (16384 tokens,
    32 heads of 64, N = 256, chunk 256, bf16; xBC of 2560 channels, 4 taps), the
    convolution checked on every element, the gated forward on every (batch,
    head) slice."""
    inp = wl.workload(3)
    blk = wl.block_inputs(inp, seed=4000)
    x, B, C = check_conv(inp, blk, "bf16", label=inp.name)
    g = inp.to("cuda:0")
    y, _ = ssd.fwd_gated(x, g.dt, g.A, B, C, inp.chunk, blk.z.to("cuda:0"), D=g.D, initial_states=g.initial_states)
    torch.cuda.synchronize()
    b, T, H, P = inp.x.shape
    # the oracle's chain starts from its own convolution, rounded to bf16 once
    H_, P_, G_, N_ = H, P, inp.B.shape[2], inp.B.shape[3]
    rx, rB, rC = (torch.from_numpy(a).to(torch.bfloat16)
                  for a in oracle.conv1d_silu(blk.xbc, blk.weight, H_, P_, G_, N_, blk.bias))
    r = oracle.forward(rx, inp.dt, inp.A, rB, rC, inp.D, inp.initial_states)
    ref = oracle.gated(r.y, blk.z)
    got = f64(y)
    e = max(rel(got[i, :, h], ref[i, :, h]) for i in range(b) for h in range(H))
    _log(f"    all {b * H} (batch, head) slices: max rel-L2 gated y={e:.3e}")
    assert e <= TOL["bf16"]
