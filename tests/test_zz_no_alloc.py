"""ssd_fwd_noalloc (the forward with the library's static scratch instead of a
caller workspace) against ssd_fwd, through the C ABI: two calls in a row, the
second on a smaller problem, so the second runs on scratch the first left
behind.  Outputs must equal ssd_fwd's bit for bit (the same kernels on the same
inputs), and both are held to the oracle's bar (max relative L2 per slice)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from ssd_chunked_scan_amd import ssd
from ssd_chunked_scan_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()
    torch.cuda.set_device(0)


def _rel_max(got, ref, slices):
    worst = 0.0
    for sl in slices:
        r = ref[sl]
        nr = np.linalg.norm(r)
        if nr < 1e-30:
            continue
        worst = max(worst, np.linalg.norm(got[sl] - r) / nr)
    return worst


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _both(inp):
    g = inp.to("cuda:0")
    nseq = inp.nseq if inp.seq_idx is not None else None
    kw = dict(D=g.D, initial_states=g.initial_states, seq_idx=g.seq_idx, nseq=nseq,
              dt_softplus=inp.dt_softplus)
    # poison the outputs so that anything left unwritten shows
    y_n = torch.full_like(g.x, float("nan"))
    p = ssd.Problem(g.x, g.dt, g.A, g.B, g.C, inp.chunk, g.D, g.initial_states, g.seq_idx, nseq)
    f_n = torch.full(p.final_shape(), float("nan"), dtype=torch.float32, device="cuda:0")
    y_n, f_n = ssd.fwd_noalloc(g.x, g.dt, g.A, g.B, g.C, inp.chunk, y=y_n, final_states=f_n, **kw)
    y_w, f_w = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, **kw)
    torch.cuda.synchronize()
    return y_n, f_n, y_w, f_w


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_fwd_twice_second_smaller(dtype, packed):
    if packed:
        big = wl.make_inputs(1, None, 4, 64, 64, 2, 128, dtype, 61, init_std=0.3,
                             packed=dict(nseqs=6, lo=100, hi=600))
        small = wl.make_inputs(1, None, 2, 32, 32, 1, 64, dtype, 62, init_std=0.3,
                               packed=dict(nseqs=3, lo=20, hi=150))
    else:
        big = wl.make_inputs(2, 1500, 6, 64, 128, 2, 128, dtype, 63, init_std=0.3)
        small = wl.make_inputs(1, 333, 3, 32, 64, 1, 64, dtype, 64, init_std=0.3)
    for label, inp in (("first (larger)", big), ("second (smaller)", small)):
        print(f"[noalloc] {label} dtype={dtype} packed={packed} x={tuple(inp.x.shape)}", flush=True)
        y_n, f_n, y_w, f_w = _both(inp)
        assert torch.equal(y_n, y_w), label
        assert torch.equal(f_n, f_w), label
        ref = oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states, inp.seq_idx,
                             inp.nseq or None, inp.dt_softplus)
        b, T, H, _ = inp.x.shape
        if inp.seq_idx is None:
            ys = [(bi, slice(None), h) for bi in range(b) for h in range(H)]
            fsl = [(bi, h) for bi in range(b) for h in range(H)]
        else:
            st = np.cumsum([0] + inp.lengths)
            ys = [(0, slice(st[k], st[k] + L), h) for k, L in enumerate(inp.lengths) for h in range(H)]
            fsl = [(k, h) for k in range(len(inp.lengths)) for h in range(H)]
        assert _rel_max(_f64(y_n), ref.y, ys) <= TOL[dtype]
        assert _rel_max(_f64(f_n), ref.final_states, fsl) <= TOL[dtype]


def test_noalloc_long_workload_fits_and_matches():
    """The long 16K-token workload (about 92 MiB of workspace) runs in the static
    scratch and gives ssd_fwd's outputs bit for bit; a tiny problem after it too."""
    inp = wl.workload(3)
    print(f"[noalloc] workload 3 x={tuple(inp.x.shape)}", flush=True)
    y_n, f_n, y_w, f_w = _both(inp)
    assert torch.equal(y_n, y_w) and torch.equal(f_n, f_w)
    tiny = wl.workload(0)
    print(f"[noalloc] workload 0 x={tuple(tiny.x.shape)}", flush=True)
    y_n, f_n, y_w, f_w = _both(tiny)
    assert torch.equal(y_n, y_w) and torch.equal(f_n, f_w)


def test_noalloc_refuses_too_large():
    inp = wl.make_inputs(8, 2048, 80, 64, 128, 1, 128, "bf16", 65)
    g = inp.to("cuda:0")
    with pytest.raises(ssd.SSDError, match="scratch"):
        ssd.fwd_noalloc(g.x, g.dt, g.A, g.B, g.C, 128, D=g.D)
