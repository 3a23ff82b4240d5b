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
