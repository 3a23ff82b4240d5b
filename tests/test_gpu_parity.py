"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.

Bar (per slice: y per (batch, head) over (T, P), or per (segment, head) for a
packed stream with padding excluded; final states per (batch|segment, head)
over (P, N)): max relative L2 error <= 1e-4 for fp32 inputs and <= 2e-2 for
bf16 inputs, for y and for the final states alike.  Per-step intermediates are
held to the same bars.  The five workloads are also checked at full size on
every slice, through the entry point and launch configuration the benchmark
times.
"""
import math
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
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy().astype(np.float64)


def run_gpu(inp, chunk=None, **kw):
    g = inp.to("cuda:0")
    y, fs = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, chunk or inp.chunk, D=g.D,
                    initial_states=g.initial_states, seq_idx=g.seq_idx,
                    nseq=inp.nseq if inp.seq_idx is not None else None,
                    dt_softplus=inp.dt_softplus, **kw)
    torch.cuda.synchronize()
    return y, fs


def run_oracle(inp, **kw):
    return oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states,
                          inp.seq_idx, inp.nseq or None, inp.dt_softplus, **kw)


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else (0.0 if np.linalg.norm(a) == 0 else np.inf)


def y_slices(inp, mask=None):
    """(batch, head, time-slice) triples over which y is compared."""
    b, T, H, _ = inp.x.shape
    out = []
    if inp.seq_idx is None:
        for bi in range(b):
            for h in range(H):
                if mask is None or mask[bi, h]:
                    out.append((bi, h, slice(0, T)))
    else:
        starts = np.cumsum([0] + inp.lengths)
        for k, L in enumerate(inp.lengths):  # padding excluded
            for h in range(H):
                if mask is None or mask[0, h]:
                    out.append((0, h, slice(starts[k], starts[k] + L)))
    return out


def max_rel_y(y_gpu, y_ref, inp, mask=None):
    yg = f64(y_gpu)
    worst = 0.0
    for bi, h, sl in y_slices(inp, mask):
        ref = y_ref[bi, sl, h]
        if np.linalg.norm(ref) < 1e-30:  # below fp32 range: must be ~0 too
            assert np.linalg.norm(yg[bi, sl, h]) <= 1e-30
            continue
        worst = max(worst, rel(yg[bi, sl, h], ref))
    return worst


def max_rel_states(fs_gpu, fs_ref, rows=None, mask=None):
    fg = f64(fs_gpu)
    worst = 0.0
    for r in (range(fs_ref.shape[0]) if rows is None else rows):
        for h in range(fs_ref.shape[1]):
            if mask is not None and not mask[min(r, mask.shape[0] - 1), h]:
                continue
            if np.linalg.norm(fs_ref[r, h]) < 1e-30:  # below fp32 range: must be ~0 too
                assert np.linalg.norm(fg[r, h]) <= 1e-30
                continue
            worst = max(worst, rel(fg[r, h], fs_ref[r, h]))
    return worst


def check(inp, dtype, chunk=None, label=""):
    _log(f"[parity] {label} x={tuple(inp.x.shape)} N={inp.B.shape[3]} G={inp.B.shape[2]} "
         f"Q={chunk or inp.chunk} dtype={dtype} packed={inp.seq_idx is not None}")
    y, fs = run_gpu(inp, chunk)
    ref = run_oracle(inp)
    ey = max_rel_y(y, ref.y, inp)
    rows = None
    if inp.seq_idx is not None:
        rows = range(len(inp.lengths))   # padding segment excluded
    es = max_rel_states(fs, ref.final_states, rows)
    _log(f"    max rel-L2 y={ey:.3e} states={es:.3e} (tol {TOL[dtype]:.0e})")
    assert ey <= TOL[dtype], ey
    assert es <= TOL[dtype], es
    assert torch.isfinite(y).all()
    return y, fs, ref


def small(dtype, T, H=4, P=64, N=64, G=1, chunk=64, b=2, seed=1, **kw):
    return wl.make_inputs(b, T, H, P, N, G, chunk, dtype, seed, **kw)


# ---------------------------------------------------------------------------
# end to end at oracle-friendly sizes: several tiles, ragged tails
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("N,G,init", [(64, 1, False), (128, 2, True), (32, 1, True)])
def test_fwd_matches_oracle(dtype, Q, N, G, init):
    T = 2 * Q + 37
    inp = small(dtype, T, H=4, P=64, N=N, G=G, chunk=Q, seed=Q + N + G,
                init_std=0.3 if init else None)
    check(inp, DT[dtype], label=f"Q{Q}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", ["slow_decay", "no_decay", "init_only", "no_D", "raw_dt"])
def test_fwd_variants(dtype, variant):
    """Variants where the inter-chunk terms dominate (slow or no decay, initial
    state only), so a state-passing error cannot hide under fast decay."""
    kw = dict(init_std=0.5)
    if variant in ("slow_decay", "init_only"):
        kw["a_log_range"] = (math.log(0.01), math.log(0.1))
    if variant == "no_decay":
        kw["a_zero"] = True
    if variant == "no_D":
        kw["with_d"] = False
    inp = small(dtype, 333, H=3, P=32, N=64, G=1, chunk=64, seed=77, **kw)
    if variant == "init_only":
        inp.x = torch.zeros_like(inp.x)
    if variant == "raw_dt":
        inp.dt = (inp.dt.float().abs() * 0.3).to(inp.dt.dtype)
        inp.dt_softplus = False
    check(inp, DT[dtype], label=variant)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_fwd_packed(dtype, Q):
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, Q, dtype, 5 + Q, init_std=0.4,
                         packed=dict(nseqs=7, lo=20, hi=300))
    check(inp, DT[dtype], label="packed")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_packed_many_short_sequences(dtype):
    """The largest segment count: 1500 packed sequences of 1 to 80 tokens (many
    boundaries in every chunk, sequences of a single token, about 60K tokens),
    every (sequence, head) slice against the oracle."""
    inp = wl.make_inputs(1, None, 4, 64, 64, 2, 64, dtype, 77, init_std=0.3,
                         packed=dict(nseqs=1500, lo=1, hi=80))
    assert min(inp.lengths) == 1
    check(inp, DT[dtype], label="1500 short sequences")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_packed_slow_decay(dtype):
    inp = wl.make_inputs(1, None, 3, 32, 64, 1, 64, dtype, 8, init_std=0.4,
                         a_log_range=(math.log(0.01), math.log(0.1)),
                         packed=dict(nseqs=6, lo=30, hi=200))
    check(inp, DT[dtype], label="packed slow decay")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_packed_sparse_ids(dtype):
    """Segment ids with a gap, starting above 0 and ending below nseq - 1: every id
    that never occurs gets a zero final state, both in the forward (where
    chunk_state records the segment ends) and through the per-step entry point
    (which records them with its own kernel); the two agree bit for bit."""
    Q = 64
    lengths, sids, nseq = [70, 150, 90], [2, 3, 6], 9
    T = sum(lengths)
    ids = np.concatenate([np.full(L, s) for s, L in zip(sids, lengths)]).astype(np.int32)
    base = small(dtype, T, H=3, P=32, N=32, b=1, seed=31, init_std=0.3)
    inp = wl.Inputs(base.x, base.dt, base.A, base.B, base.C, base.D, base.initial_states,
                    torch.from_numpy(ids), nseq, Q, lengths=lengths)
    _log(f"[parity] sparse segment ids {sids} of nseq={nseq} dtype={dtype}")
    y, fs = run_gpu(inp)
    ref = run_oracle(inp)
    assert max_rel_y(y, ref.y, inp) <= TOL[DT[dtype]]
    assert max_rel_states(fs, ref.final_states, rows=sids) <= TOL[DT[dtype]]
    absent = [i for i in range(nseq) if i not in sids]
    assert torch.count_nonzero(fs[absent]) == 0
    # the per-step path
    g = inp.to("cuda:0")
    p = _problem(g, inp)
    delta, cs = ssd.chunk_cumsum(p)
    cb = ssd.chunk_cb(p)
    states = ssd.chunk_state(p, delta, cs, cb)
    ssd.state_passing(p, cs, states)
    fs_step = ssd.seq_final_states(p, delta, cs, states)
    assert torch.equal(fs_step, fs)


@pytest.mark.parametrize("shape", [
    dict(T=1), dict(T=37), dict(T=64), dict(T=65), dict(P=16, N=16, H=2, T=256),
    dict(P=128, N=64, T=150), dict(P=48, N=48, T=200), dict(N=256, T=300, H=2), dict(H=6, G=3, T=129),
])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_shapes(shape, dtype):
    kw = dict(H=4, P=64, N=64, G=1, T=100)
    kw.update(shape)
    inp = small(dtype, kw["T"], H=kw["H"], P=kw["P"], N=kw["N"], G=kw["G"], chunk=64, seed=kw["T"],
                init_std=0.2)
    check(inp, DT[dtype], label=str(shape))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_largest_tiles(dtype):
    """The largest tile configuration the kernels are built for: N = 256 (the
    widest state), Q = 256, and P = 128 (two 64-wide p tiles per head), with two
    groups, an initial state and a ragged last chunk."""
    inp = small(dtype, 2 * 256 + 37, H=4, P=128, N=256, G=2, chunk=256, b=1, seed=256, init_std=0.3)
    check(inp, DT[dtype], label="largest tiles")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_empty_sequence(dtype):
    inp = small(dtype, 0, H=2, P=16, N=16, init_std=0.5)
    y, fs = run_gpu(inp)
    assert y.numel() == 0
    assert torch.equal(fs.cpu(), inp.initial_states)


def test_chunk_length_invariance():
    inp = small("fp32", 700, H=3, P=64, N=64, seed=3, init_std=0.3,
                a_log_range=(math.log(0.05), math.log(0.5)))
    outs = [run_gpu(inp, Q) for Q in (64, 128, 256)]
    for y, fs in outs[1:]:
        assert rel(f64(y), f64(outs[0][0])) < 1e-5
        assert rel(f64(fs), f64(outs[0][1])) < 1e-5


def test_split_resume():
    inp = small("fp32", 500, H=2, P=32, N=64, seed=4, init_std=0.3)
    y, fs = run_gpu(inp)
    T1 = 211
    cut = lambda t, a, b_: None if t is None else t[:, a:b_].contiguous()
    first = wl.Inputs(cut(inp.x, 0, T1), cut(inp.dt, 0, T1), inp.A, cut(inp.B, 0, T1),
                      cut(inp.C, 0, T1), inp.D, inp.initial_states, None, 0, 64)
    y1, fs1 = run_gpu(first)
    second = wl.Inputs(cut(inp.x, T1, 500), cut(inp.dt, T1, 500), inp.A, cut(inp.B, T1, 500),
                       cut(inp.C, T1, 500), inp.D, fs1.cpu(), None, 0, 64)
    y2, fs2 = run_gpu(second)
    assert rel(f64(torch.cat([y1, y2], 1)), f64(y)) < 1e-5
    assert rel(f64(fs2), f64(fs)) < 1e-5


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_deterministic(dtype):
    inp = wl.workload(1, batch=1, seqlen=1000, nheads=8) if dtype == "bf16" else \
        small("fp32", 900, H=4, seed=9, init_std=0.1)
    y1, f1 = run_gpu(inp)
    y2, f2 = run_gpu(inp)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_nan_isolation_across_chunk_aligned_sequences():
    """A NaN/Inf input inside one packed sequence that owns whole chunks stays in
    that sequence: the state reset at the boundary is a select."""
    Q = 64
    lengths = [128, 192, 64, 100]
    T = sum(lengths)
    H, P, N = 2, 32, 32
    ids = np.concatenate([np.full(L, i) for i, L in enumerate(lengths)]).astype(np.int32)
    base = small("fp32", T, H=H, P=P, N=N, b=1, seed=12)
    inp = wl.Inputs(base.x, base.dt, base.A, base.B, base.C, base.D, None, torch.from_numpy(ids),
                    len(lengths), Q, lengths=lengths)
    y0, f0 = run_gpu(inp)
    x = inp.x.clone()
    x[0, 128 + 5, 0, 3] = float("nan")
    x[0, 128 + 70, 1, 0] = float("inf")
    dt = inp.dt.clone()
    dt[0, 128 + 9, 1] = float("nan")
    bad = wl.Inputs(x, dt, inp.A, inp.B, inp.C, inp.D, None, inp.seq_idx, inp.nseq, Q, lengths=lengths)
    y1, f1 = run_gpu(bad)
    keep = torch.from_numpy(ids != 1).cuda()
    assert torch.equal(y1[0, keep], y0[0, keep])
    for k in (0, 2, 3):
        assert torch.equal(f1[k], f0[k])
    assert not torch.isfinite(y1[0, ~keep]).all()


def _poisoned_run(dtype, Q, what, lengths, seq, pos, seed=14):
    """A packed stream whose boundaries mostly fall inside chunks, run clean and
    with one non-finite input (x, B or dt) at token `pos` of sequence `seq`."""
    T = sum(lengths)
    H, P, N, G = 4, 32, 32, 2
    ids = np.concatenate([np.full(L, i) for i, L in enumerate(lengths)]).astype(np.int32)
    base = small(dtype, T, H=H, P=P, N=N, G=G, b=1, seed=seed, init_std=0.3)
    inp = wl.Inputs(base.x, base.dt, base.A, base.B, base.C, base.D, base.initial_states,
                    torch.from_numpy(ids), len(lengths), Q, lengths=lengths)
    y0, f0 = run_gpu(inp)
    t = int(np.cumsum([0] + lengths)[seq]) + pos
    x, B, dt = inp.x.clone(), inp.B.clone(), inp.dt.clone()
    if what == "x":
        x[0, t, 1, 3] = float("nan")
    elif what == "x_inf":
        x[0, t, 2, 0] = float("inf")
    elif what == "B":
        B[0, t, 1, 5] = float("nan")
    else:
        dt[0, t, 0] = float("nan")
    bad = wl.Inputs(x, dt, inp.A, B, inp.C, inp.D, inp.initial_states, inp.seq_idx, inp.nseq, Q,
                    lengths=lengths)
    y1, f1 = run_gpu(bad)
    return ids, t, y0, f0, y1, f1


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("what", ["x", "x_inf", "B", "dt"])
def test_nan_isolation_mid_chunk_boundaries(dtype, Q, what):
    """A NaN or Inf in x, B or dt inside one packed sequence, with sequence
    boundaries inside chunks (several sequences share a chunk, some shorter than a
    K step): every other sequence's outputs and final state are bit-identical to
    the clean run, and the poisoned sequence's final state is not finite.  (The
    state reset at a boundary is a select, and the GPU path drops the tokens of
    other sequences by selects wherever it would otherwise multiply them by a zero
    weight.)"""
    lengths = [37, 90, 5, 61, 140, 23, 9, 200]
    for seq, pos in ((3, 10), (4, 0), (3, 60), (2, 2), (7, 150)):
        _log(f"[nan mid-chunk] dtype={dtype} Q={Q} {what} in sequence {seq} at +{pos}")
        ids, t, y0, f0, y1, f1 = _poisoned_run(dtype, Q, what, lengths, seq, pos)
        keep = torch.from_numpy(ids != seq).cuda()
        assert torch.equal(y1[0, keep], y0[0, keep]), (seq, pos)
        for k in range(len(lengths)):
            if k != seq:
                assert torch.equal(f1[k], f0[k]), (seq, pos, k)
        assert not torch.isfinite(f1[seq]).all()
        # the poisoned sequence before the poisoned token's 32-token block (chunks
        # start at multiples of 32) is untouched too
        start = int(np.cumsum([0] + lengths)[seq])
        clean_to = max(start, (t // 32) * 32)
        assert torch.equal(y1[0, start:clean_to], y0[0, start:clean_to])


# ---------------------------------------------------------------------------
# per-step pins against oracle intermediates
# ---------------------------------------------------------------------------

def unpack_cb(buf, Q, NT):
    """Dense CB [.., Q, Q], C copy [.., Q, NT] and B^T copy [.., NT, Q] from the
    chunk_cb buffer [.., Q*(Q+2*NT)]: each part is 16 x 32 blocks (row block, K
    block), each block 64 lanes x 8, lane = row % 16 + 16 * (column % 32 // 8)."""
    def dense(m, nrow, ncol):
        lead = m.shape[:-1]
        m = m.reshape(*lead, nrow // 16, ncol // 32, 4, 16, 8)    # rb, kb, lg, li, e
        n = len(lead)
        m = m.transpose(*range(n), n, n + 3, n + 1, n + 2, n + 4)  # rb, li, kb, lg, e
        return m.reshape(*lead, nrow, ncol)
    qq, qn = Q * Q, Q * NT
    return (dense(buf[..., :qq], Q, Q), dense(buf[..., qq:qq + qn], Q, NT),
            dense(buf[..., qq + qn:], NT, Q))


def _problem(g, inp):
    return ssd.Problem(g.x, g.dt, g.A, g.B, g.C, inp.chunk, g.D, g.initial_states, g.seq_idx,
                       inp.nseq if inp.seq_idx is not None else None, inp.dt_softplus)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("packed", [False, True])
def test_per_step_pins(dtype, Q, packed):
    if packed:
        inp = wl.make_inputs(1, None, 4, 64, 64, 2, Q, dtype, 21 + Q, init_std=0.3,
                             packed=dict(nseqs=6, lo=40, hi=400))
    else:
        inp = small(dtype, 3 * Q - 19, H=4, P=64, N=64, G=2, chunk=Q, seed=Q, init_std=0.3)
    tol = TOL[DT[dtype]]
    _log(f"[per-step] dtype={dtype} Q={Q} packed={packed} T={inp.x.shape[1]}")
    g = inp.to("cuda:0")
    p = _problem(g, inp)
    b, T, H, P = inp.x.shape
    nc = p.nc

    # chunk_cumsum
    delta, cs = ssd.chunk_cumsum(p)
    d_ref, cs_ref = oracle.chunk_cumsum(inp.dt, inp.A, Q, inp.dt_softplus, inp.seq_idx)
    torch.cuda.synchronize()
    assert rel(f64(delta), d_ref) < 1e-6
    assert rel(f64(cs), cs_ref) < 1e-6

    # chunk_cb: CB (lower block triangle of 64x64 tiles) and the C copy, both
    # fragment-major inside the buffer (layout documented in include/ssd.h)
    cb = ssd.chunk_cb(p, torch.zeros(p.cb_shape(), dtype=p.dtype, device=p.device))   # upper tiles stay unwritten
    cb_ref = oracle.chunk_cb(inp.B, inp.C, Q)
    torch.cuda.synchronize()
    cbm, cm, btm = unpack_cb(f64(cb), Q, p.NT)
    ti = np.arange(Q)[:, None] // 64
    si = np.arange(Q)[None, :] // 64
    lower = np.broadcast_to(si <= ti, cb_ref.shape)
    assert rel(cbm[lower], cb_ref[lower]) < (1e-5 if dtype == "fp32" else 1e-2)
    N = inp.B.shape[3]
    c_pad = np.zeros((b, nc * Q, inp.C.shape[2], p.NT))
    c_pad[:, :T, :, :N] = f64(inp.C)
    want_c = c_pad.reshape(b, nc, Q, -1, p.NT).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(cm, want_c)   # a copy: exact, zero past seqlen and N
    b_pad = np.zeros_like(c_pad)
    b_pad[:, :T, :, :N] = f64(inp.B)
    want_bt = b_pad.reshape(b, nc, Q, -1, p.NT).transpose(0, 1, 3, 4, 2)
    assert np.array_equal(btm, want_bt)

    # chunk_state: each chunk's end state from its own inputs (oracle chunk-local mode)
    delta_c, cs_c = delta.clone(), cs.clone()
    states = ssd.chunk_state(p, delta, cs, cb)   # runs the cumsum step again, in place
    torch.cuda.synchronize()
    assert torch.equal(delta, delta_c) and torch.equal(cs, cs_c)
    loc = run_oracle(inp, chunk=Q, chunk_local=True, want_chunk_states=True)
    torch.cuda.synchronize()
    sg = f64(states)
    for bi in range(b):
        for h in range(H):
            assert rel(sg[bi, :, h], loc.chunk_end_states[bi, :, h]) < tol

    # state_passing: entering state of chunk c = oracle state after chunk c-1
    fin = None if packed else torch.empty(b, H, P, inp.B.shape[3], device="cuda:0")
    ssd.state_passing(p, cs, states, fin)
    full = run_oracle(inp, chunk=Q, want_chunk_states=True)
    torch.cuda.synchronize()
    hin = f64(states)
    init = np.zeros_like(hin[:, 0]) if inp.initial_states is None else f64(inp.initial_states)
    want = np.concatenate([init[:, None], full.chunk_end_states[:, :nc - 1]], axis=1)
    for bi in range(b):
        for h in range(H):
            for c in range(nc):
                if np.linalg.norm(want[bi, c, h]) > 0:
                    assert rel(hin[bi, c, h], want[bi, c, h]) < tol, (bi, h, c)
    if not packed:
        assert max_rel_states(fin, full.final_states) < tol
    else:
        fs = ssd.seq_final_states(p, delta, cs, states)
        torch.cuda.synchronize()
        assert max_rel_states(fs, full.final_states, rows=range(len(inp.lengths))) < tol

    # chunk_scan: y from the GPU intermediates
    y = ssd.chunk_scan(p, delta, cs, cb, states)
    torch.cuda.synchronize()
    assert max_rel_y(y, full.y, inp) < tol
    # the per-step pipeline and ssd_fwd run the same kernels: bitwise equal
    y2, _ = run_gpu(inp)
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# the five workloads at full size, every slice
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_full_workloads(idx):
    """Each workload at its full size, through the entry point and launch
    configuration the benchmark times, against the oracle on every (batch, head)
    slice of y and of the final states (every (sequence, head) in the packed
    workload, padding excluded)."""
    inp = wl.workload(idx)
    dtype = DT[wl.WORKLOADS[idx]["dtype"]]
    _log(f"[full] workload {idx} {inp.name} x={tuple(inp.x.shape)} dtype={dtype}")
    g = inp.to("cuda:0")
    p = _problem(g, inp)
    ws = torch.empty(ssd.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    y, fs = ssd.fwd(g.x, g.dt, g.A, g.B, g.C, inp.chunk, D=g.D, initial_states=g.initial_states,
                    seq_idx=g.seq_idx, nseq=inp.nseq if inp.seq_idx is not None else None,
                    workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(fs).all()
    ref = run_oracle(inp)
    ey = max_rel_y(y, ref.y, inp)
    rows = range(len(inp.lengths)) if inp.seq_idx is not None else None
    es = max_rel_states(fs, ref.final_states, rows)
    nsl = len(y_slices(inp))
    _log(f"    all {nsl} slices: max rel-L2 y={ey:.3e} states={es:.3e} (tol {TOL[dtype]:.0e})")
    assert ey <= TOL[dtype] and es <= TOL[dtype]


def test_long_sequence_past_32bit_offsets():
    """The maximum-size case along the sequence: 1,052,897 tokens (4113 chunks of
    256, the last one ragged) x 32 heads x 64 in bf16, so x and y hold 2.16e9
    elements (4.3 GB) and every token past about 2^19 (bytes) or 2^20 (elements)
    lies beyond 32-bit offsets; the chunk states take another 1 GB.  Inputs are
    drawn on the GPU (``workloads.device_inputs``).  The oracle runs on one head's
    slice at a time (heads are independent given the shared B and C): the first
    and the last head, y over (T, P) and the final state over (P, N)."""
    T, H, P, N, Q = (1 << 20) + 4321, 32, 64, 64, 256
    dev = "cuda:0"
    inp = wl.device_inputs(1, T, H, P, N, 1, Q, "bf16", seed=7000, device=dev, name="long1M_bf16")
    _log(f"[max] T={T} H={H} P={P} N={N} Q={Q}: x {inp.x.numel() * 2 / 2**30:.2f} GiB")
    y, fs = ssd.fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, Q, D=inp.D, initial_states=inp.initial_states)
    torch.cuda.synchronize()
    assert torch.isfinite(fs).all()
    Bh, Ch = inp.B.cpu(), inp.C.cpu()
    for h in (0, H - 1):
        sl = slice(h, h + 1)
        ref = oracle.forward(inp.x[:, :, sl].contiguous().cpu(), inp.dt[:, :, sl].contiguous().cpu(),
                             inp.A[sl].cpu(), Bh, Ch, inp.D[sl].cpu(), inp.initial_states[:, sl].contiguous().cpu())
        yh = y[:, :, sl].contiguous()
        assert torch.isfinite(yh).all()
        ey = rel(f64(yh), ref.y)
        es = rel(f64(fs[:, sl]), ref.final_states)
        _log(f"    head {h}: rel-L2 y={ey:.3e} final state={es:.3e} (tol {TOL[torch.bfloat16]:.0e})")
        assert ey <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def _nan_tail(t, extra=4096):
    """A copy of t on the GPU whose storage is followed by NaNs: the head of a
    larger NaN-filled buffer (still contiguous), so any read past the tensor's
    end shows up in the outputs."""
    t = t.to("cuda:0")
    buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device=t.device)
    buf[:t.numel()] = t.reshape(-1)
    return buf[:t.numel()].view(t.shape)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fwd_reads_nothing_past_the_last_row(dtype):
    """Row pitches below one 64-column tile (H*P = 32, G*N = 16, N = 16) with a
    ragged last chunk: the rows past the sequence end must read as zeros, not
    as whatever follows the tensors in memory, and the workspace may hold
    anything."""
    inp = small(dtype, 70, H=2, P=16, N=16, G=1, chunk=64, b=1, seed=70, init_std=0.3)
    x, dt, B, C = (_nan_tail(t) for t in (inp.x, inp.dt, inp.B, inp.C))
    p = ssd.Problem(x, dt, inp.A.cuda(), B, C, 64, inp.D.cuda(), inp.initial_states.cuda())
    ws = torch.full((ssd.workspace_bytes(p) // 4 + 1,), float("nan"), dtype=torch.float32,
                    device="cuda:0").view(torch.uint8)
    y, fs = ssd.fwd(x, dt, inp.A.cuda(), B, C, 64, D=inp.D.cuda(), initial_states=inp.initial_states.cuda(),
                    workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(fs).all()
    ref = run_oracle(inp)
    assert max_rel_y(y, ref.y, inp) <= TOL[DT[dtype]]
    assert max_rel_states(fs, ref.final_states) <= TOL[DT[dtype]]


def test_check_seq_idx_finds_the_first_violation():
    """The device-side precondition check: -1 for valid packed ids (including
    ids that never occur and an empty stream), else the first position whose id
    is out of range or smaller than its predecessor's."""
    dev = torch.device("cuda:0")
    lengths = [37, 90, 5, 61, 140, 23, 9, 200, 1, 4000]
    ids = np.concatenate([np.full(L, 2 * i, np.int32) for i, L in enumerate(lengths)])   # odd ids never occur
    nseq = 2 * len(lengths)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    assert ssd.check_seq_idx(t(ids), nseq) == -1
    assert ssd.check_seq_idx(t(ids[:0]), nseq) == -1
    bad = ids.copy(); bad[777] = bad[776] - 1          # decreasing
    assert ssd.check_seq_idx(t(bad), nseq) == 777
    bad = ids.copy(); bad[3000] = nseq                 # out of range (and later ids smaller)
    assert ssd.check_seq_idx(t(bad), nseq) == 3000
    bad = ids.copy(); bad[0] = -1                      # negative
    assert ssd.check_seq_idx(t(bad), nseq) == 0
    bad = ids.copy(); bad[4000] = 0; bad[100] = -5     # two violations: the first one counts
    assert ssd.check_seq_idx(t(bad), nseq) == 100
    big = np.repeat(np.arange(1000, dtype=np.int32), 1024)   # a million positions
    assert ssd.check_seq_idx(t(big), 1000) == -1
    big[len(big) - 1] = 998
    assert ssd.check_seq_idx(t(big), 1000) == len(big) - 1
