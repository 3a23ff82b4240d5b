"""GPU parity of the backward pass (ssd_bwd, through the C ABI) against the fp64
oracle's reverse-mode derivative of the recurrence, on the same seeded inputs.

The forward output y that ssd_bwd takes is the GPU forward's own output.  Each
gradient is compared per slice with the forward's bars (max relative L2 error
<= 1e-4 for fp32 inputs, <= 2e-2 for bf16 inputs):
  dx per (batch, head) over (T, P);  ddt per (batch, head) over T;
  dB, dC per (batch, group) over (T, N);  dinit per (batch, head) over (P, N);
  dA, dD over the heads.
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
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else float(np.linalg.norm(a))


def worst(got, ref, axes):
    """max rel-L2 over the slices that remain after moving `axes` (the slice
    index axes) to the front"""
    g = np.moveaxis(got, axes, list(range(len(axes))))
    r = np.moveaxis(ref, axes, list(range(len(axes))))
    lead = g.shape[:len(axes)]
    return max(rel(g[idx], r[idx]) for idx in np.ndindex(*lead))


def run_bwd(inp, dtype, seed=0, with_dfinal=True):
    g = inp.to("cuda:0")
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states,
                   dt_softplus=inp.dt_softplus)
    rng = np.random.default_rng(100 + seed)
    b, T, H, P = inp.x.shape
    N = inp.B.shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32))
    dy = dy.to(torch.bfloat16) if dtype == "bf16" else dy
    dfin = torch.from_numpy(rng.standard_normal((b, H, P, N)).astype(np.float32)) if with_dfinal else None
    gr = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy.to("cuda:0"), D=g.D,
                 initial_states=g.initial_states,
                 dfinal_states=None if dfin is None else dfin.to("cuda:0"), dt_softplus=inp.dt_softplus)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.initial_states, dfin,
                          dt_softplus=inp.dt_softplus)
    return gr, ref


def check_bwd(inp, dtype, label="", **kw):
    _log(f"[bwd] {label} x={tuple(inp.x.shape)} N={inp.B.shape[3]} G={inp.B.shape[2]} Q={inp.chunk} {dtype}")
    gr, ref = run_bwd(inp, dtype, **kw)
    errs = {
        "dx": worst(f64(gr["dx"]), ref.dx, [0, 2]),
        "ddt": worst(f64(gr["ddt"]), ref.ddt, [0, 2]),
        "dB": worst(f64(gr["dB"]), ref.dB, [0, 2]),
        "dC": worst(f64(gr["dC"]), ref.dC, [0, 2]),
        "dinit": worst(f64(gr["dinitial_states"]), ref.dinit, [0, 1]),
        "dA": rel(f64(gr["dA"]), ref.dA),
    }
    if ref.dD is not None:
        errs["dD"] = rel(f64(gr["dD"]), ref.dD)
    _log("    " + "  ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f"  (tol {TOL[dtype]:.0e})")
    for k, v in errs.items():
        assert v <= TOL[dtype], (k, v)
    for k, t in gr.items():
        if t is not None:
            assert torch.isfinite(t).all(), k


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_largest_tiles(dtype):
    """The largest tile configuration: N = 256, Q = 256 and P = 128 (two p tiles),
    two groups, an initial state and a ragged last chunk."""
    inp = wl.make_inputs(1, 2 * 256 + 37, 4, 128, 256, 2, 256, dtype, 257, init_std=0.3)
    check_bwd(inp, dtype, label="largest tiles")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_bwd_matches_oracle(dtype, Q):
    # several chunks and a ragged tail; heads sharing groups; initial state
    inp = wl.make_inputs(2, 2 * Q + 37, 4, 64, 64, 2, Q, dtype, Q + 5, init_std=0.3)
    check_bwd(inp, dtype, label=f"Q{Q}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [dict(P=32, N=128, H=2, G=1, T=150), dict(P=128, N=32, H=3, G=3, T=100),
                                   dict(P=48, N=256, H=2, G=1, T=300), dict(P=64, N=48, H=4, G=1, T=65),
                                   dict(P=16, N=16, H=2, G=2, T=1)],
                         ids=lambda d: "P{P}_N{N}_H{H}_G{G}_T{T}".format(**d))
def test_bwd_shapes(dtype, shape):
    inp = wl.make_inputs(1, shape["T"], shape["H"], shape["P"], shape["N"], shape["G"], 64, dtype,
                         shape["T"] + shape["P"], init_std=0.3)
    check_bwd(inp, dtype, label=str(shape))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["no_D_no_init", "raw_dt", "slow_decay", "no_dfinal"])
def test_bwd_variants(dtype, variant):
    import math
    kw = dict(init_std=0.3)
    if variant == "no_D_no_init":
        kw = dict(with_d=False)
    if variant == "slow_decay":
        kw["a_log_range"] = (math.log(0.01), math.log(0.1))
    inp = wl.make_inputs(2, 200, 3, 32, 64, 1, 64, dtype, 41, **kw)
    if variant == "raw_dt":
        inp.dt_softplus = False
        inp.dt = inp.dt.float().abs().to(inp.x.dtype)
    check_bwd(inp, dtype, label=variant, with_dfinal=variant != "no_dfinal")


def test_bwd_deterministic():
    inp = wl.make_inputs(1, 300, 4, 64, 64, 1, 64, "bf16", 3, init_std=0.3)
    a, _ = run_bwd(inp, "bf16")
    b, _ = run_bwd(inp, "bf16")
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_bwd_small_workload_full_size():
    """The small workload (2 x 2048 tokens, 24 heads, N = 64, bf16) at full size."""
    inp = wl.workload(1)
    check_bwd(inp, "bf16", label=inp.name)


def _nan_tail(t, extra=4096):
    t = t.to("cuda:0")
    buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device=t.device)
    buf[:t.numel()] = t.reshape(-1)
    return buf[:t.numel()].view(t.shape)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 70])
def test_bwd_reads_nothing_past_the_last_row(dtype, T):
    """Narrow rows (H*P = 32, G*N = 32, N = 16) with a ragged last chunk, every
    input followed by NaNs in memory and a NaN-filled workspace: no gradient
    may pick any of it up."""
    inp = wl.make_inputs(1, T, 2, 16, 16, 2, 64, dtype, 7 + T, init_std=0.3)
    x, dt, B, C = (_nan_tail(t) for t in (inp.x, inp.dt, inp.B, inp.C))
    A, D, init = inp.A.cuda(), inp.D.cuda(), inp.initial_states.cuda()
    y, _ = ssd.fwd(x, dt, A, B, C, 64, D=D, initial_states=init)
    y = _nan_tail(y)
    rng = np.random.default_rng(5)
    dy_c = torch.from_numpy(rng.standard_normal(tuple(inp.x.shape)).astype(np.float32)).to(inp.x.dtype)
    dy = _nan_tail(dy_c)
    p = ssd.Problem(x, dt, A, B, C, 64, D, init)
    ws = torch.full((ssd.bwd_workspace_bytes(p) // 4 + 1,), float("nan"), dtype=torch.float32,
                    device="cuda:0").view(torch.uint8)
    gr = ssd.bwd(x, dt, A, B, C, 64, y, dy, D=D, initial_states=init, workspace=ws)
    torch.cuda.synchronize()
    for k, t in gr.items():
        if t is not None:
            assert torch.isfinite(t).all(), k
    ref = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy_c, inp.D, inp.initial_states)
    tol = TOL[dtype]
    assert worst(f64(gr["dx"]), ref.dx, [0, 2]) <= tol
    assert worst(f64(gr["ddt"]), ref.ddt, [0, 2]) <= tol
    assert worst(f64(gr["dB"]), ref.dB, [0, 2]) <= tol
    assert worst(f64(gr["dC"]), ref.dC, [0, 2]) <= tol
    assert worst(f64(gr["dinitial_states"]), ref.dinit, [0, 1]) <= tol


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_bwd_with_the_forwards_workspace(Q):
    """Reading the forward's chunk intermediates from its workspace gives the very
    gradients of recomputing them (bit for bit), and leaves that workspace as it
    was."""
    inp = wl.make_inputs(2, 2 * Q + 37, 4, 64, 64, 2, Q, "bf16", 200 + Q, init_std=0.3)
    g = inp.to("cuda:0")
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, Q, g.D, g.initial_states)
    fws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, Q, D=g.D, initial_states=g.initial_states, workspace=fws)
    torch.cuda.synchronize()
    keep = fws.clone()
    dy = torch.randn(tuple(inp.x.shape), generator=torch.Generator().manual_seed(Q)).to(torch.bfloat16).cuda()
    dfin = torch.randn((2, 4, 64, 64), generator=torch.Generator().manual_seed(Q + 1)).cuda()
    kw = dict(D=g.D, initial_states=g.initial_states, dfinal_states=dfin)
    a = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, Q, y, dy, **kw)
    b = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, Q, y, dy, fwd_workspace=fws, **kw)
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    assert torch.equal(fws, keep)


def test_bwd_long_workload_full_size():
    """The benchmark's backward configuration: the long workload (16384 tokens,
    32 heads of 64, N = 256, chunk 256, bf16) at full size, the forward's
    intermediates read from its workspace as the benchmark times it, every
    gradient against the oracle."""
    inp = wl.workload(3)
    _log(f"[bwd] {inp.name} full size")
    g = inp.to("cuda:0")
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, inp.chunk, g.D, g.initial_states)
    fws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states, workspace=fws)
    rng = np.random.default_rng(7)
    b, T, H, P = inp.x.shape
    N = inp.B.shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32)).to(torch.bfloat16)
    dfin = torch.from_numpy(rng.standard_normal((b, H, P, N)).astype(np.float32))
    gr = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy.to("cuda:0"), D=g.D, initial_states=g.initial_states,
                 dfinal_states=dfin.to("cuda:0"), fwd_workspace=fws)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.initial_states, dfin)
    errs = {"dx": worst(f64(gr["dx"]), ref.dx, [0, 2]), "ddt": worst(f64(gr["ddt"]), ref.ddt, [0, 2]),
            "dB": worst(f64(gr["dB"]), ref.dB, [0, 2]), "dC": worst(f64(gr["dC"]), ref.dC, [0, 2]),
            "dinit": worst(f64(gr["dinitial_states"]), ref.dinit, [0, 1]), "dA": rel(f64(gr["dA"]), ref.dA),
            "dD": rel(f64(gr["dD"]), ref.dD)}
    _log("    " + "  ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f"  (tol {TOL['bf16']:.0e})")
    for k, v in errs.items():
        assert v <= TOL["bf16"], (k, v)


# ---------------------------------------------------------------------------
# packed streams
# ---------------------------------------------------------------------------

def check_bwd_packed(inp, dtype, label="", seed=0, ddt_min_len=0):
    """The backward of a packed stream against the oracle's, per (segment, head)
    slice of dx and ddt, per (segment, group) slice of dB and dC, per head of
    dinit, and over the heads for dA and dD; dfinal holds one gradient per
    segment id.

    ddt has one value per token, so the ddt slice of a sequence of a few tokens
    holds a few numbers, each one dot product whose true value can lie
    arbitrarily close to zero, where no rounded computation keeps a relative
    error bound.  With ddt_min_len = L, the ddt of the sequences shorter than L
    tokens is compared per head as one slice pooled over all of them (every
    value is still compared); longer sequences keep their own slices."""
    _log(f"[bwd packed] {label} T={inp.x.shape[1]} nseq={len(inp.lengths)} Q={inp.chunk} {dtype}")
    g = inp.to("cuda:0")
    nseq = inp.nseq
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states,
                   seq_idx=g.seq_idx, nseq=nseq, dt_softplus=inp.dt_softplus)
    rng = np.random.default_rng(300 + seed)
    b, T, H, P = inp.x.shape
    N = inp.B.shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32))
    dy = dy.to(torch.bfloat16) if dtype == "bf16" else dy
    dfin = torch.from_numpy(rng.standard_normal((nseq, H, P, N)).astype(np.float32))
    gr = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y, dy.to("cuda:0"), D=g.D,
                 initial_states=g.initial_states, dfinal_states=dfin.to("cuda:0"),
                 dt_softplus=inp.dt_softplus, seq_idx=g.seq_idx, nseq=nseq)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.initial_states, dfin,
                          seq_idx=inp.seq_idx, nseq=nseq, dt_softplus=inp.dt_softplus)
    ids = inp.seq_idx.numpy()
    segs = [np.flatnonzero(ids == s) for s in np.unique(ids)]

    def seg_worst(got, want, slices=segs):
        # got / want [1, T, K, ...]: slices (segment, k) over (tokens of the segment, ...)
        return max(rel(got[0, sl, k], want[0, sl, k]) for sl in slices for k in range(got.shape[2]))

    ddt_slices = segs
    if ddt_min_len:
        short = [sl for sl in segs if len(sl) < ddt_min_len]
        ddt_slices = [sl for sl in segs if len(sl) >= ddt_min_len] + ([np.concatenate(short)] if short else [])

    errs = {
        "dx": seg_worst(f64(gr["dx"]), ref.dx),
        "ddt": seg_worst(f64(gr["ddt"])[..., None], ref.ddt[..., None], ddt_slices),
        "dB": seg_worst(f64(gr["dB"]), ref.dB),
        "dC": seg_worst(f64(gr["dC"]), ref.dC),
        "dA": rel(f64(gr["dA"]), ref.dA),
    }
    if inp.initial_states is not None:
        errs["dinit"] = worst(f64(gr["dinitial_states"]), ref.dinit, [0, 1])
    if ref.dD is not None:
        errs["dD"] = rel(f64(gr["dD"]), ref.dD)
    _log("    " + "  ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f"  (tol {TOL[dtype]:.0e})")
    for k, v in errs.items():
        assert v <= TOL[dtype], (k, v)
    for k, t in gr.items():
        if t is not None:
            assert torch.isfinite(t).all(), k
    return gr


def test_bwd_past_32bit_offsets():
    """The maximum-size case of the backward: 16 sequences of 66,770 tokens (261
    chunks of 256, the last ragged) x 32 heads x 64 in bf16, N = 64, so x, dy and
    dx hold 2.19e9 elements (4.1 GiB each) and the last sequence lies wholly
    past 2^31 elements.  Inputs and dy are drawn on the GPU.  The oracle runs on
    four heads of the last sequence (heads are independent given the shared B
    and C): dx and ddt over that sequence's tokens, and dinit.  dB and dC (sums
    over all heads) and dA and dD (sums over all sequences) need every unit; they
    are held to the oracle at full size on the long workload instead."""
    b, T, H, P, N, Q = 16, 65536 + 1234, 32, 64, 64, 256
    dev = "cuda:0"
    inp = wl.device_inputs(b, T, H, P, N, 1, Q, "bf16", seed=7001, device=dev, name="b16_T66770_bf16")
    _log(f"[bwd max] b={b} T={T} H={H} P={P} N={N}: x {inp.x.numel() * 2 / 2**30:.2f} GiB")
    y, _ = ssd.fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, Q, D=inp.D, initial_states=inp.initial_states)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7002)
    dy = torch.empty_like(inp.x)
    for t0 in range(0, T, 1 << 14):
        t1 = min(T, t0 + (1 << 14))
        dy[:, t0:t1] = torch.randn(b, t1 - t0, H, P, device=dev, generator=gen).to(torch.bfloat16)
    dfin = torch.randn(b, H, P, N, device=dev, generator=gen)
    gr = ssd.bwd(inp.x, inp.dt, inp.A, inp.B, inp.C, Q, y, dy, D=inp.D, initial_states=inp.initial_states,
                 dfinal_states=dfin)
    torch.cuda.synchronize()
    for k in ("dx", "ddt", "dB", "dC", "dA", "dD", "dinitial_states"):
        assert torch.isfinite(gr[k]).all(), k
    bb, heads = b - 1, [0, 17, 30, 31]
    hs = lambda t: t[bb:bb + 1][:, :, heads].contiguous().cpu()   # [1, T, 4, ...] of the last sequence
    ref = oracle.backward(hs(inp.x), hs(inp.dt), inp.A[heads].cpu(), inp.B[bb:bb + 1].cpu(),
                          inp.C[bb:bb + 1].cpu(), hs(dy), inp.D[heads].cpu(),
                          inp.initial_states[bb:bb + 1, heads].cpu(), dfin[bb:bb + 1, heads].cpu())
    errs = {"dx": worst(f64(hs(gr["dx"])), ref.dx, [0, 2]), "ddt": worst(f64(hs(gr["ddt"])), ref.ddt, [0, 2]),
            "dinit": worst(f64(gr["dinitial_states"][bb:bb + 1, heads]), ref.dinit, [0, 1])}
    _log("    sequence %d, heads %s: " % (bb, heads) + "  ".join(f"{k}={v:.2e}" for k, v in errs.items())
         + f"  (tol {TOL['bf16']:.0e})")
    for k, v in errs.items():
        assert v <= TOL["bf16"], (k, v)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_bwd_packed(dtype, Q):
    """Packed sequences with boundaries inside chunks, an initial state (the first
    sequence's), several sequences sharing a chunk, groups."""
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, Q, dtype, 400 + Q, init_std=0.3,
                         packed=dict(nseqs=7, lo=20, hi=300))
    check_bwd_packed(inp, dtype, label="mid-chunk boundaries")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_packed_many_short_sequences(dtype):
    """The largest segment count for the backward: 1500 packed sequences of 1 to
    80 tokens (each padded to its own chunks in the backward's layout: about
    1500 chunks for about 60K tokens), every slice against the oracle.  fp32
    holds even the one-token sequences' ddt to 1e-4 on their own.  In bf16 the
    gradient states and the C.B products are rounded to bf16, and the ddt of a
    one-token sequence is a single dot product (x . y') that can nearly cancel
    (measured: 0.0119 against the oracle's 0.0106 for one such token, 12 %,
    where the whole tensor's error is 0.25 %).  There the ddt of the sequences shorter than 64 tokens (the row
    count of every other slice) is compared per head as one pooled slice."""
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, 64, dtype, 78, init_std=0.3,
                         packed=dict(nseqs=1500, lo=1, hi=80))
    assert min(inp.lengths) == 1
    check_bwd_packed(inp, dtype, label="1500 short sequences", ddt_min_len=64 if dtype == "bf16" else 0)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_packed_slow_decay_sparse_ids(dtype):
    """Slow decay (the carried state and dfinal matter far back), segment ids with
    gaps that start above 0, and sequences that end exactly on a chunk boundary
    (64, 128) as well as inside one."""
    import math
    Q = 64
    lengths, sids, nseq = [64, 70, 128, 5, 93], [1, 2, 4, 5, 7], 9
    T = sum(lengths)
    ids = np.concatenate([np.full(L, s) for s, L in zip(sids, lengths)]).astype(np.int32)
    base = wl.make_inputs(1, T, 3, 32, 48, 1, Q, dtype, 77, init_std=0.4,
                          a_log_range=(math.log(0.01), math.log(0.1)))
    inp = wl.Inputs(base.x, base.dt, base.A, base.B, base.C, base.D, base.initial_states,
                    torch.from_numpy(ids), nseq, Q, lengths=lengths)
    check_bwd_packed(inp, dtype, label="slow decay, sparse ids")


def test_bwd_packed_raw_dt_no_D():
    inp = wl.make_inputs(1, None, 2, 32, 64, 1, 128, "fp32", 91, with_d=False,
                         packed=dict(nseqs=4, lo=50, hi=400))
    inp.dt_softplus = False
    inp.dt = inp.dt.float().abs() * 0.3
    check_bwd_packed(inp, "fp32", label="raw dt, no D")


def test_bwd_packed_deterministic():
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, 128, "bf16", 92, packed=dict(nseqs=5, lo=30, hi=500))
    a = check_bwd_packed(inp, "bf16", label="determinism 1")
    b = check_bwd_packed(inp, "bf16", label="determinism 2")
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_bwd_packed_nan_workspace():
    """A packed stream whose padded layout ends in chunks of padding only (6
    sequences of 20-200 tokens, Q = 64), with a NaN-filled workspace: the
    per-chunk kernels skip those chunks, so their workspace slots keep the NaNs,
    and no gradient may pick any of them up.  The gradients equal those of a
    zero-filled workspace bit for bit."""
    Q = 64
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, Q, "bf16", 93, init_std=0.3, packed=dict(nseqs=6, lo=20, hi=200))
    T, nseq = inp.x.shape[1], inp.nseq
    counts = np.bincount(inp.seq_idx.numpy(), minlength=nseq)   # every segment, the padding one too
    padded = int(sum((L + Q - 1) // Q * Q for L in counts))
    bound = (T + nseq * (Q - 1) + Q - 1) // Q * Q   # the padded length the library lays out
    assert bound - padded >= Q, "the case must have a chunk of padding only"
    g = inp.to("cuda:0")
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, Q, D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx,
                   nseq=nseq)
    rng = np.random.default_rng(9)
    b, _, H, P = inp.x.shape
    N = inp.B.shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32)).to(torch.bfloat16).to("cuda:0")
    dfin = torch.from_numpy(rng.standard_normal((nseq, H, P, N)).astype(np.float32)).to("cuda:0")
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, Q, g.D, g.initial_states, g.seq_idx, nseq)
    nbytes = ssd.bwd_workspace_bytes(p)
    runs = []
    for fill in (0.0, float("nan")):
        ws = torch.full((nbytes // 4 + 1,), fill, dtype=torch.float32, device="cuda:0").view(torch.uint8)
        runs.append(ssd.bwd(g.x, g.dt, g.A, g.B, g.C, Q, y, dy, D=g.D, initial_states=g.initial_states,
                            dfinal_states=dfin, seq_idx=g.seq_idx, nseq=nseq, workspace=ws))
    torch.cuda.synchronize()
    for k, t in runs[1].items():
        if t is not None:
            assert torch.isfinite(t).all(), k
            assert torch.equal(t, runs[0][k]), k


def test_bwd_packed_workload_full_size():
    """The packed workload (16 sequences of 128-2048 tokens plus the padding
    segment, 64 heads, N = 128, 8 groups, chunk 128, bf16) at full size, every
    (segment, head) slice against the oracle."""
    inp = wl.workload(4)
    check_bwd_packed(inp, "bf16", label=inp.name)


@pytest.mark.parametrize("mode", ["recompute", "fwd_workspace", "packed"])
def test_bwd_stage_times(mode):
    """The stage-timed backward computes the very gradients of ssd_bwd (bit for
    bit) and reports every stage of its path once, with a positive duration."""
    Q = 128
    if mode == "packed":
        inp = wl.make_inputs(1, None, 8, 64, 64, 2, Q, "bf16", 77, init_std=0.3,
                             packed=dict(nseqs=5, lo=20, hi=300))
    else:
        inp = wl.make_inputs(2, 3 * Q + 21, 8, 64, 64, 2, Q, "bf16", 78, init_std=0.3)
    _log(f"[bwd stage times] {mode} T={inp.x.shape[1]}")
    g = inp.to("cuda:0")
    nseq = inp.nseq if inp.seq_idx is not None else None
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, Q, g.D, g.initial_states, g.seq_idx, nseq)
    fws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    y, _ = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, Q, D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx,
                   nseq=nseq, workspace=fws)
    gen = torch.Generator().manual_seed(5)
    dy = torch.randn(tuple(inp.x.shape), generator=gen).to(torch.bfloat16).cuda()
    dfin = torch.randn(p.final_shape(), generator=gen).cuda()
    kw = dict(D=g.D, initial_states=g.initial_states, dfinal_states=dfin, seq_idx=g.seq_idx, nseq=nseq,
              fwd_workspace=fws if mode == "fwd_workspace" else None)
    a = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, Q, y, dy, **kw)
    stages = []
    b = ssd.bwd(g.x, g.dt, g.A, g.B, g.C, Q, y, dy, stage_times=stages, **kw)
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    names = [n for n, _ in stages]
    core = ["chunk_cb_rev", "chunk_state_grad", "state_passing_rev", "chunk_scan_dx",
            "chunk_scan_dy_hin", "m_rows_cols", "dl_ddt_dA_dD", "dC", "dB"]
    want = {"recompute": ["chunk_cb", "chunk_state", "state_passing"] + core,
            "fwd_workspace": core,
            "packed": ["chunk_map", "chunk_cb", "chunk_state", "state_passing"] + core[:2] + ["inject_dfinal"]
                      + core[2:]}[mode]
    assert names == want
    assert all(ms > 0 for _, ms in stages), stages
    _log("    " + " ".join(f"{n}={ms * 1e3:.0f}us" for n, ms in stages))
