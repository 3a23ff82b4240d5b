"""GPU parity of the decode step (ssd_step, through the C ABI) against the fp64
oracle's step on the same seeded inputs, and against the chunked forward: T
steps from the initial state give the forward's y and final state.

Bar: max relative L2 error per (batch, head) slice, y over P and the state over
(P, N), <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs (the same bars as
the forward).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from ssd_chunked_scan_amd import ssd
from ssd_chunked_scan_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


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


def worst(got, ref):
    """max over (batch, head) of the relative L2 error of the trailing axes"""
    b, H = ref.shape[:2]
    return max(rel(got[i, h], ref[i, h]) for i in range(b) for h in range(H))


def gpu_step(s: wl.StepInputs):
    g = s.to("cuda:0")
    state = g.state.clone()
    y = ssd.step(g.x, g.dt, g.A, g.B, g.C, state, D=g.D, dt_softplus=s.dt_softplus)
    torch.cuda.synchronize()
    return y, state


def check_step(s: wl.StepInputs, dtype, label=""):
    _log(f"[step] {label} x={tuple(s.x.shape)} N={s.B.shape[2]} G={s.B.shape[1]} dtype={dtype}")
    y, state = gpu_step(s)
    y_ref, st_ref = oracle.step(s.x, s.dt, s.A, s.B, s.C, s.state, s.D, s.dt_softplus)
    ey, es = worst(f64(y), y_ref), worst(f64(state), st_ref)
    _log(f"    max rel-L2 y={ey:.3e} state={es:.3e} (tol {TOL[dtype]:.0e})")
    assert ey <= TOL[dtype] and es <= TOL[dtype], (ey, es)
    assert torch.isfinite(y).all() and torch.isfinite(state).all()


# (b, H, P, N, G): every lane width of the kernel (N/4 = 4, 12 -> 16, 16, 32, 64),
# several row blocks (P up to 128), heads sharing groups
SHAPES = [(3, 4, 64, 128, 2), (2, 2, 16, 16, 1), (1, 3, 48, 48, 1), (2, 2, 128, 256, 1),
          (5, 8, 32, 64, 4), (2, 4, 80, 112, 2)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_H%d_P%d_N%d_G%d" % s)
def test_step_matches_oracle(dtype, shape):
    b, H, P, N, G = shape
    s = wl.decode_inputs(seed=sum(shape), batch=b, nheads=H, headdim=P, dstate=N, ngroups=G, dtype=dtype)
    check_step(s, DT[dtype], label=str(shape))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["no_D", "raw_dt", "zero_state", "no_decay"])
def test_step_variants(dtype, variant):
    kw = dict(batch=2, nheads=4, headdim=64, dstate=64, ngroups=1, dtype=dtype)
    s = wl.decode_inputs(seed=11, **kw)
    if variant == "no_D":
        s.D = None
    if variant == "raw_dt":
        s.dt_softplus = False
        s.dt = s.dt.abs()
    if variant == "zero_state":
        s.state = torch.zeros_like(s.state)
    if variant == "no_decay":
        s.A = torch.zeros_like(s.A)
    check_step(s, DT[dtype], label=variant)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_steps_replay_the_forward(dtype):
    """T decode steps from the initial state = the chunked forward over the same
    T tokens: every y_t and the final state, and both against the oracle."""
    T = 150
    inp = wl.make_inputs(2, T, 4, 64, 64, 1, 64, dtype, 21, init_std=0.3,
                         a_log_range=(np.log(0.05), np.log(0.5)))
    g = inp.to("cuda:0")
    _log(f"[step] replay T={T} dtype={dtype}")
    y_f, fin_f = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states)
    state = g.initial_states.clone()
    ys = []
    for t in range(T):
        s = wl.token(g, t, state)
        ys.append(ssd.step(s.x, s.dt, s.A, s.B, s.C, state, D=s.D))
    torch.cuda.synchronize()
    y_s = torch.stack(ys, dim=1)
    ref = oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states)
    tol = TOL[DT[dtype]]
    # y per (batch, head) over (T, P)
    ysw = worst(f64(y_s).transpose(0, 2, 1, 3), ref.y.transpose(0, 2, 1, 3))
    yfw = worst(f64(y_f).transpose(0, 2, 1, 3), f64(y_s).transpose(0, 2, 1, 3))
    sw = worst(f64(state), ref.final_states)
    sf = worst(f64(state), f64(fin_f))
    _log(f"    steps vs oracle: y={ysw:.3e} state={sw:.3e}; steps vs forward: y={yfw:.3e} state={sf:.3e}")
    assert max(ysw, sw, yfw, sf) <= tol


def test_step_full_decode_workload():
    """The benchmark's decode configuration (64 sequences, 80 heads of 64, N = 128,
    bf16), launched exactly as the benchmark launches it, against the oracle on
    every (sequence, head)."""
    s = wl.decode_inputs()
    check_step(s, torch.bfloat16, label=s.name)


def test_step_updates_only_the_state_and_y():
    s = wl.decode_inputs(seed=5, batch=2, nheads=4, headdim=32, dstate=64, dtype="bf16")
    g = s.to("cuda:0")
    keep = [t.clone() for t in (g.x, g.dt, g.A, g.B, g.C, g.D)]
    state = g.state.clone()
    ssd.step(g.x, g.dt, g.A, g.B, g.C, state, D=g.D)
    torch.cuda.synchronize()
    for a, k in zip((g.x, g.dt, g.A, g.B, g.C, g.D), keep):
        assert torch.equal(a, k)
    assert not torch.equal(state, g.state)
