"""Pins for the fp64 CPU oracle (``oracle/``), each against something other than
the oracle itself: the pages' dual (quadratic) form, closed forms, a library
routine for a special case, structural invariants and brute force.

Page references are by title and section:
  [tomabc]  "Mamba 2 -- Transformers are SSMs" paper story (ai.tomabc.com)
  [jsqmd]   "Transformers与SSMs的隐藏联系" (jsqmd.com)
  [scwac]   "SSM 家族全景图（下）：Mamba-2 与 Jamba" (scwacadex)
  [freetools] "从Transformer的二次复杂度困境到Mamba的线性突围" (answer.freetools.me)
"""
import math

import numpy as np
import pytest

import oracle
from ssd_chunked_scan_amd import workloads as wl


def _np(t):
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def _softplus_ref(z):
    # library form, independent of the oracle's max/log1p evaluation
    return np.logaddexp(0.0, z)


def _small(seed=7, b=1, T=37, H=3, P=4, N=5, G=1, chunk=16, init_std=None, dtype="fp32", **kw):
    return wl.make_inputs(b, T, H, P, N, G, chunk, dtype, seed, init_std=init_std, **kw)


def _run(inp, **kw):
    return oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states,
                          inp.seq_idx, inp.nseq or None, inp.dt_softplus, **kw)


def dual_form(inp):
    """y = M x + D x + (init term), with M materialised as the T x T matrix of the
    dual form Y = (L o Q K^T) V, Q = C, K = B, V = Delta x, L_{t,s} = a_t ... a_{s+1}
    ([tomabc] section 3.2, formula 1; [tomabc] section 2.1 for the expansion
    y_t = sum_s C_t^T (A_t...A_{s+1}) B_s x_s).  The decay products are formed by
    explicit multiplication, never by a cumulative sum of logs."""
    x, dt, A, B, C = map(_np, (inp.x, inp.dt, inp.A, inp.B, inp.C))
    D = _np(inp.D)
    init = _np(inp.initial_states)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    delta = _softplus_ref(dt) if inp.dt_softplus else dt
    seq = None if inp.seq_idx is None else inp.seq_idx.numpy()
    y = np.zeros_like(x)
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(delta[bi, :, h] * A[h])
            if seq is not None:  # a boundary sets a_t to 0 ([jsqmd] section 4.2)
                a = a.copy()
                a[1:][seq[1:] != seq[:-1]] = 0.0
            L = np.zeros((T, T))
            for t in range(T):
                prod = 1.0
                L[t, t] = 1.0
                for s in range(t - 1, -1, -1):
                    prod *= a[s + 1]
                    L[t, s] = prod
            CB = C[bi, :, g, :] @ B[bi, :, g, :].T
            M = L * CB * delta[bi, :, h][None, :]
            y[bi, :, h, :] = M @ x[bi, :, h, :]
            if D is not None:
                y[bi, :, h, :] += D[h] * x[bi, :, h, :]
            if init is not None:
                carry = np.cumprod(a)  # prod_{k<=t} a_k: decay of h_{-1} up to t
                y[bi, :, h, :] += carry[:, None] * (C[bi, :, g, :] @ init[bi, h].T)
    return y


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# dual (quadratic) form == recurrence
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,H", [(1, 3), (3, 3), (2, 4)])
@pytest.mark.parametrize("with_init", [False, True])
def test_dual_form_matches_recurrence(G, H, with_init):
    inp = _small(seed=11 + G + H, b=2, H=H, G=G, init_std=0.3 if with_init else None)
    y = _run(inp).y
    assert rel(y, dual_form(inp)) < 1e-12


def test_dual_form_packed_sequences():
    inp = wl.make_inputs(1, None, 2, 3, 4, 1, 8, "fp32", 5, init_std=0.5,
                         packed=dict(nseqs=4, lo=3, hi=11))
    assert inp.seq_idx is not None and inp.nseq >= 4
    y = _run(inp).y
    assert rel(y, dual_form(inp)) < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _const_inputs(T, H, P, N, delta, A, xbar, Bbar, Cbar, D, h0):
    import torch
    f = lambda a: torch.tensor(np.asarray(a, np.float32))
    x = np.broadcast_to(xbar[None, None, :, :], (1, T, H, P))
    dt = np.full((1, T, H), delta)
    Bm = np.broadcast_to(Bbar[None, None, None, :], (1, T, 1, N))
    Cm = np.broadcast_to(Cbar[None, None, None, :], (1, T, 1, N))
    return wl.Inputs(x=f(x), dt=f(dt), A=f(A), B=f(Bm), C=f(Cm), D=f(D),
                     initial_states=f(h0[None]), seq_idx=None, nseq=0, chunk=T,
                     dt_softplus=False)


@pytest.mark.parametrize("A_vals", [(-0.7, -2.3), (0.0, -0.05)])
def test_closed_form_constant_inputs(A_vals):
    """x, B, C, Delta constant: the recurrence is a geometric series
    h_t = a^{t+1} h_{-1} + delta x B^T (1 - a^{t+1}) / (1 - a),
    y_t = C^T h_t + D x, with (1-a^k)/(1-a) -> k at a = 1."""
    rng = np.random.default_rng(3)
    T, H, P, N = 29, 2, 3, 4
    delta = 0.375
    xbar = rng.standard_normal((H, P)).astype(np.float32).astype(np.float64)
    Bbar = rng.standard_normal(N).astype(np.float32).astype(np.float64)
    Cbar = rng.standard_normal(N).astype(np.float32).astype(np.float64)
    D = rng.standard_normal(H).astype(np.float32).astype(np.float64)
    h0 = rng.standard_normal((H, P, N)).astype(np.float32).astype(np.float64)
    A = np.array(A_vals, np.float32).astype(np.float64)
    inp = _const_inputs(T, H, P, N, delta, A, xbar, Bbar, Cbar, D, h0)
    out = _run(inp)
    for h in range(H):
        a = math.exp(delta * A[h])
        geo = lambda k: k if a == 1.0 else (1.0 - a ** k) / (1.0 - a)
        for t in range(T):
            ht = a ** (t + 1) * h0[h] + delta * np.outer(xbar[h], Bbar) * geo(t + 1)
            want = ht @ Cbar + D[h] * xbar[h]
            assert np.allclose(out.y[0, t, h], want, rtol=1e-12, atol=1e-12)
        hT = a ** T * h0[h] + delta * np.outer(xbar[h], Bbar) * geo(T)
        assert np.allclose(out.final_states[0, h], hT, rtol=1e-12, atol=1e-12)


def test_closed_form_constant_decay_powers():
    """Constant Delta = delta (softplus off): L_{t,s} = a^{t-s} computed with pow,
    a Toeplitz mask independent of any cumulative sum ([tomabc] section 3.2)."""
    inp = _small(seed=21, T=31, H=2, P=3, N=4)
    import torch
    delta = 0.2
    inp.dt = torch.full_like(inp.dt, delta)
    inp.dt_softplus = False
    x, A, B, C, D = map(_np, (inp.x, inp.A, inp.B, inp.C, inp.D))
    y = _run(inp).y
    T = x.shape[1]
    d32 = float(np.float32(delta))
    for h in range(2):
        a = math.exp(d32 * A[h])
        t_idx, s_idx = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
        L = np.where(t_idx >= s_idx, np.power(a, np.maximum(t_idx - s_idx, 0)), 0.0)
        want = (L * (C[0, :, 0] @ B[0, :, 0].T) * d32) @ x[0, :, h] + D[h] * x[0, :, h]
        assert rel(y[0, :, h], want) < 1e-12


def test_linear_attention_special_case():
    """A = 0 makes every a_t = 1: L is the causal mask and the state is a prefix
    sum of Delta_s B_s x_s^T, i.e. causal linear attention ([freetools], Mamba-2 and
    state-space duality: with all a_t = 1 the mask is the standard causal mask)."""
    inp = _small(seed=31, T=40, H=2, P=3, N=5, a_zero=True)
    x, dt, B, C, D = map(_np, (inp.x, inp.dt, inp.B, inp.C, inp.D))
    delta = _softplus_ref(dt)
    out = _run(inp)
    for h in range(2):
        outer = delta[0, :, h, None, None] * x[0, :, h, :, None] * B[0, :, 0, None, :]  # [T,P,N]
        hs = np.cumsum(outer, axis=0)
        want = np.einsum("tpn,tn->tp", hs, C[0, :, 0]) + D[h] * x[0, :, h]
        assert rel(out.y[0, :, h], want) < 1e-12
        assert rel(out.final_states[0, h], hs[-1]) < 1e-12


# ---------------------------------------------------------------------------
# structure of M: N-semiseparable ([tomabc] section 2.2)
# ---------------------------------------------------------------------------

def test_semiseparable_rank():
    import torch
    T, N = 24, 3
    inp = _small(seed=41, T=T, H=1, P=1, N=N, with_d=False)
    M = np.zeros((T, T))
    for i in range(T):  # column i of M is the response to an impulse at i
        imp = torch.zeros_like(inp.x)
        imp[0, i, 0, 0] = 1.0
        inp_i = wl.Inputs(imp, inp.dt, inp.A, inp.B, inp.C, None, None, None, 0, inp.chunk)
        M[:, i] = _run(inp_i).y[0, :, 0, 0]
    assert np.allclose(np.triu(M, 1), 0.0)
    ranks = []
    for j0 in range(T):
        blk = M[j0:, : j0 + 1]
        sv = np.linalg.svd(blk, compute_uv=False)
        ranks.append(int((sv > 1e-10 * sv[0]).sum()) if sv[0] > 0 else 0)
    assert max(ranks) <= N
    assert max(ranks) == N  # generic inputs reach the bound
    assert rel(M @ _np(inp.x)[0, :, 0, 0], _run(inp).y[0, :, 0, 0]) < 1e-12


# ---------------------------------------------------------------------------
# packed sequences and resets ([jsqmd] section 4.2)
# ---------------------------------------------------------------------------

def _packed(seed=51, H=2, P=3, N=4, G=1, chunk=8, init_std=0.4):
    return wl.make_inputs(1, None, H, P, N, G, chunk, "fp32", seed, init_std=init_std,
                          packed=dict(nseqs=5, lo=4, hi=13))


def test_packed_equals_separate_runs():
    inp = _packed()
    out = _run(inp)
    starts = np.cumsum([0] + inp.lengths)
    for k, L in enumerate(inp.lengths):
        sl = slice(starts[k], starts[k] + L)
        init = inp.initial_states if k == 0 else None  # h_{-1} flows into segment 0 only
        sub = wl.Inputs(inp.x[:, sl], inp.dt[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl], inp.D,
                        init, None, 0, inp.chunk)
        ref = _run(sub)
        assert rel(out.y[:, sl], ref.y) < 1e-14
        assert rel(out.final_states[k], ref.final_states[0]) < 1e-14


def test_nan_does_not_cross_boundaries():
    import torch
    inp = _packed(seed=52)
    clean = _run(inp)
    k = 2
    starts = np.cumsum([0] + inp.lengths)
    x = inp.x.clone()
    x[0, starts[k] + 1, 0, 0] = float("nan")
    x[0, starts[k] + 2, 1, 2] = float("inf")
    bad = _run(wl.Inputs(x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states,
                         inp.seq_idx, inp.nseq, inp.chunk))
    for j, L in enumerate(inp.lengths):
        sl = slice(starts[j], starts[j] + L)
        if j == k:
            assert not np.isfinite(bad.y[:, sl]).all()
            continue
        assert np.array_equal(bad.y[:, sl], clean.y[:, sl])
        assert np.array_equal(bad.final_states[j], clean.final_states[j])


# ---------------------------------------------------------------------------
# linearity, split/resume, batch and group broadcast
# ---------------------------------------------------------------------------

def test_linearity_in_x_and_initial_state():
    inp = _small(seed=61, init_std=0.5)
    inp.x = inp.x.double()  # form the combination exactly in fp64
    x2 = _small(seed=62).x.double()
    base = lambda x, init, d=inp.D: _run(wl.Inputs(x, inp.dt, inp.A, inp.B, inp.C, d, init,
                                                    None, 0, inp.chunk))
    al, be = 0.75, -1.25
    lhs = base(al * inp.x + be * x2, None).y
    rhs = al * base(inp.x, None).y + be * base(x2, None).y
    assert rel(lhs, rhs) < 1e-12
    full = base(inp.x, inp.initial_states)
    parts = base(inp.x, None).y + base(inp.x * 0, inp.initial_states).y
    assert rel(full.y, parts) < 1e-12
    nod = base(inp.x, inp.initial_states, None).y
    want = _np(inp.D)[None, None, :, None] * _np(inp.x)
    assert np.allclose(full.y - nod, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T1", [1, 16, 23])
def test_split_resume(T1):
    inp = _small(seed=71, T=40, init_std=0.2)
    full = _run(inp)
    a = _run(wl.Inputs(inp.x[:, :T1], inp.dt[:, :T1], inp.A, inp.B[:, :T1], inp.C[:, :T1], inp.D,
                       inp.initial_states, None, 0, inp.chunk))
    import torch
    h1 = torch.tensor(a.final_states)
    b = _run(wl.Inputs(inp.x[:, T1:], inp.dt[:, T1:], inp.A, inp.B[:, T1:], inp.C[:, T1:], inp.D,
                       h1, None, 0, inp.chunk))
    assert rel(np.concatenate([a.y, b.y], axis=1), full.y) < 1e-13
    assert rel(b.final_states, full.final_states) < 1e-13


def test_batch_rows_independent():
    inp = _small(seed=81, b=3, init_std=0.3)
    full = _run(inp)
    for bi in range(3):
        sl = slice(bi, bi + 1)
        one = _run(wl.Inputs(inp.x[sl], inp.dt[sl], inp.A, inp.B[sl], inp.C[sl], inp.D,
                             inp.initial_states[sl], None, 0, inp.chunk))
        assert np.array_equal(one.y, full.y[sl])
        assert np.array_equal(one.final_states, full.final_states[sl])


def test_group_broadcast_contiguous_heads():
    """G groups over H heads: head h reads group floor(h*G/H).  Equivalent to
    G = H with B, C replicated per head."""
    inp = _small(seed=91, H=6, G=2)
    out = _run(inp)
    rep = lambda t: t[:, :, [h * 2 // 6 for h in range(6)], :].contiguous()
    wide = _run(wl.Inputs(inp.x, inp.dt, inp.A, rep(inp.B), rep(inp.C), inp.D, None, None, 0,
                          inp.chunk))
    assert np.array_equal(out.y, wide.y)


def test_unit_mask_samples_heads():
    inp = _small(seed=95, b=2, H=4, init_std=0.1)
    full = _run(inp)
    mask = np.zeros((2, 4), bool)
    mask[0, 1] = mask[1, 3] = True
    part = _run(inp, unit_mask=mask)
    assert np.array_equal(part.y[0, :, 1], full.y[0, :, 1])
    assert np.array_equal(part.y[1, :, 3], full.y[1, :, 3])
    assert np.array_equal(part.final_states[1, 3], full.final_states[1, 3])
    assert not part.y[0, :, 0].any()


# ---------------------------------------------------------------------------
# softplus, chunk cumsum, chunk snapshots
# ---------------------------------------------------------------------------

def test_softplus_reading():
    """dt passed raw with softplus on == softplus(dt) passed with softplus off."""
    inp = _small(seed=101)
    import torch
    z = _np(inp.dt)
    on = _run(inp).y
    off = _run(wl.Inputs(inp.x, torch.tensor(_softplus_ref(z)), inp.A, inp.B, inp.C, inp.D,
                         None, None, 0, inp.chunk, dt_softplus=False)).y
    assert rel(on, off) < 1e-12
    # softplus at special points: ln 2 at 0, ~z for large z, ~e^z for very negative z
    vals = np.array([[[0.0], [40.0], [-40.0]]])
    delta, _ = oracle.chunk_cumsum(vals, np.array([-1.0]), 3)
    assert delta[0, 0, 0, 0] == pytest.approx(math.log(2.0), rel=1e-15)
    assert delta[0, 0, 0, 1] == pytest.approx(40.0, rel=1e-15)
    assert delta[0, 0, 0, 2] == pytest.approx(math.exp(-40.0), rel=1e-12)


@pytest.mark.parametrize("T,Q", [(64, 16), (50, 16), (7, 8)])
def test_chunk_cumsum(T, Q):
    """exp(cs_t - cs_s) must equal the explicit product a_{s+1}...a_t inside a chunk,
    with tail positions past T carrying Delta = 0 and an unchanged cs."""
    rng = np.random.default_rng(T + Q)
    H = 3
    dt = rng.normal(-1.0, 1.0, size=(2, T, H))
    A = -np.exp(rng.uniform(0, 2, size=H))
    delta, cs = oracle.chunk_cumsum(dt, A, Q)
    nc = (T + Q - 1) // Q
    sp = _softplus_ref(dt)
    for b in range(2):
        for h in range(H):
            for c in range(nc):
                n_real = min(Q, T - c * Q)
                assert np.allclose(delta[b, h, c, :n_real], sp[b, c * Q:c * Q + n_real, h], rtol=1e-14)
                assert (delta[b, h, c, n_real:] == 0).all()
                assert (cs[b, h, c, n_real:] == cs[b, h, c, n_real - 1]).all()
                a = np.exp(sp[b, c * Q:c * Q + n_real, h] * A[h])
                for t in range(n_real):
                    assert math.exp(cs[b, h, c, t]) == pytest.approx(np.prod(a[: t + 1]), rel=1e-12)
                    s = t // 2
                    assert math.exp(cs[b, h, c, t] - cs[b, h, c, s]) == pytest.approx(
                        np.prod(a[s + 1: t + 1]), rel=1e-12)


def test_chunk_cumsum_restarts_at_segments():
    """Packed: exp(cs_t) is the decay product from the later of the chunk start and
    t's segment start, so exp(cs_t - cs_s) = a_{s+1}...a_t for s, t in one segment."""
    inp = _packed(seed=57, chunk=8)
    dt, A = _np(inp.dt), _np(inp.A)
    sid = inp.seq_idx.numpy()
    T, Q = dt.shape[1], 8
    delta, cs = oracle.chunk_cumsum(dt, A, Q, seq_idx=sid)
    sp = _softplus_ref(dt)
    for h in range(dt.shape[2]):
        a = np.exp(sp[0, :, h] * A[h])
        for t in range(T):
            c, i = divmod(t, Q)
            start = t
            while start > c * Q and sid[start - 1] == sid[t]:
                start -= 1
            assert math.exp(cs[0, h, c, i]) == pytest.approx(np.prod(a[start: t + 1]), rel=1e-12)


@pytest.mark.parametrize("packed", [False, True])
def test_chunk_end_states(packed):
    """Normal mode: the state after chunk c equals the final state of a run over the
    prefix [0, (c+1)Q).  Chunk-local mode: the state at each chunk end computed from
    that chunk's inputs alone with a zero start ([scwac], the four-step chunked
    algorithm: step 2 uses only the chunk's own inputs)."""
    Q = 8
    if packed:
        inp = _packed(seed=111, chunk=Q)
    else:
        inp = _small(seed=112, T=45, chunk=Q, init_std=0.3)
    T = inp.x.shape[1]
    nc = (T + Q - 1) // Q
    full = _run(inp, chunk=Q, want_chunk_states=True)
    loc = _run(inp, chunk=Q, chunk_local=True, want_chunk_states=True)
    for c in range(nc):
        e = min((c + 1) * Q, T)
        sid = None if inp.seq_idx is None else inp.seq_idx[:e]
        pre = _run(wl.Inputs(inp.x[:, :e], inp.dt[:, :e], inp.A, inp.B[:, :e], inp.C[:, :e], inp.D,
                             inp.initial_states, sid, inp.nseq, Q))
        if inp.seq_idx is None:
            want = pre.final_states
        else:
            want = pre.final_states[int(inp.seq_idx[e - 1])][None]
        assert rel(full.chunk_end_states[:, c], want) < 1e-13
        s0 = c * Q
        sid = None if inp.seq_idx is None else inp.seq_idx[s0:e]
        one = _run(wl.Inputs(inp.x[:, s0:e], inp.dt[:, s0:e], inp.A, inp.B[:, s0:e], inp.C[:, s0:e],
                             inp.D, None, sid, inp.nseq, Q))
        want = one.final_states if sid is None else one.final_states[int(sid[-1])][None]
        assert rel(loc.chunk_end_states[:, c], want) < 1e-13


def test_brute_force_three_steps():
    """T = 3, one head, P = N = 1, written out step by step from the recurrence."""
    import torch
    x = [0.5, -1.25, 2.0]
    dt = [0.1, 0.3, 0.2]
    Bv, Cv = [1.5, -0.5, 0.25], [0.75, 2.0, -1.0]
    A, D, h0 = -1.5, 0.5, 0.8
    f = lambda v, shape: torch.tensor(v, dtype=torch.float64).reshape(shape)
    inp = wl.Inputs(f(x, (1, 3, 1, 1)), f(dt, (1, 3, 1)), f([A], (1,)), f(Bv, (1, 3, 1, 1)),
                    f(Cv, (1, 3, 1, 1)), f([D], (1,)), f([h0], (1, 1, 1, 1)), None, 0, 3,
                    dt_softplus=False)
    out = _run(inp)
    h = h0
    for t in range(3):
        h = math.exp(dt[t] * A) * h + dt[t] * Bv[t] * x[t]
        assert out.y[0, t, 0, 0] == pytest.approx(Cv[t] * h + D * x[t], rel=1e-14)
    assert out.final_states[0, 0, 0, 0] == pytest.approx(h, rel=1e-14)


def test_golden_regression_fixture():
    """The oracle still reproduces the fixture ``tests/golden/make_golden.py`` wrote."""
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    lines = [l for l in open(make_golden.OUT) if not l.startswith("#")]
    y_ref = np.array(lines[0].split(), float)
    fs_ref = np.array(lines[1].split(), float)
    inp = make_golden.tiny_inputs()
    out = _run(inp)
    assert np.allclose(out.y.reshape(-1), y_ref, rtol=1e-14, atol=1e-15)
    assert np.allclose(out.final_states.reshape(-1), fs_ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("G,H", [(1, 2), (2, 4)])
def test_chunk_cb_rebuilds_chunk_outputs(G, H):
    """Within one chunk and with a zero incoming state, the dual form gives
    y_t = sum_{s<=t} exp(cs_t - cs_s) CB[t][s] Delta_s x_s + D x_t ([tomabc] section
    3.2, formula 1, with Q = C and K = B).  Rebuilt from the oracle's chunk_cb and
    chunk_cumsum, it must equal the recurrence's y of a zero-start run over each chunk
    alone.  CB is not symmetric, so a transposed or mis-indexed product fails here."""
    Q, T, P, N = 8, 21, 3, 5
    inp = _small(seed=131, T=T, H=H, P=P, N=N, G=G, chunk=Q)
    x, dt, A, D = _np(inp.x), _np(inp.dt), _np(inp.A), _np(inp.D)
    cb = oracle.chunk_cb(_np(inp.B), _np(inp.C), Q)
    delta, cs = oracle.chunk_cumsum(dt, A, Q)
    nc = (T + Q - 1) // Q
    assert cb.shape == (1, nc, G, Q, Q)
    for c in range(nc):
        s0, e = c * Q, min((c + 1) * Q, T)
        one = _run(wl.Inputs(inp.x[:, s0:e], inp.dt[:, s0:e], inp.A, inp.B[:, s0:e], inp.C[:, s0:e],
                             inp.D, None, None, 0, Q))
        for h in range(H):
            g = h // (H // G)
            n = e - s0
            W = np.zeros((n, n))
            for t in range(n):
                for s in range(t + 1):
                    W[t, s] = math.exp(cs[0, h, c, t] - cs[0, h, c, s]) * cb[0, c, g, t, s] * delta[0, h, c, s]
            y = W @ x[0, s0:e, h, :] + D[h] * x[0, s0:e, h, :]
            assert rel(y, one.y[0, :, h, :]) < 1e-13


def test_step_replays_the_recurrence():
    """oracle.step applied token after token, carrying its state, reproduces the
    forward over the whole sequence: y of every token and the final state.  A
    swapped axis or a mis-shaped operand in the step's marshalling fails here."""
    inp = wl.make_inputs(2, 9, 4, 16, 16, 2, 64, "fp32", 5, init_std=0.5)
    ref = _run(inp)
    state = inp.initial_states.double().numpy()
    for t in range(9):
        s = wl.token(inp, t)
        y, state = oracle.step(s.x, s.dt, s.A, s.B, s.C, state, s.D, s.dt_softplus)
        assert np.allclose(y, ref.y[:, t], rtol=1e-12, atol=1e-14)
    assert np.allclose(state, ref.final_states, rtol=1e-12, atol=1e-14)


def test_step_closed_forms():
    """Two cases with a closed form ("Mamba 2 -- Transformers are SSMs", section
    3.1, one step of the recurrence):
    - zero state, x one-hot at row p: only row p of the new state is nonzero and it
      equals Delta * B_g (head h uses group h*G/H), so y_p = Delta * C_g.B_g + D x_p;
    - A = 0 with the raw step size: nothing decays, state' = state + dt x B^T."""
    b, H, P, N, G = 1, 4, 3, 5, 2
    rng = np.random.default_rng(3)
    Bv = rng.standard_normal((b, G, N))
    Cv = rng.standard_normal((b, G, N))
    dt = np.array([[0.3, -0.2, 1.1, 0.05]])
    A = np.array([-1.0, -2.0, -0.5, -4.0])
    D = np.array([0.5, -1.0, 2.0, 0.0])
    x = np.zeros((b, H, P))
    x[0, :, 1] = 1.0
    y, st = oracle.step(x, dt, A, Bv, Cv, np.zeros((b, H, P, N)), D, dt_softplus=True)
    for h in range(H):
        g = h * G // H
        delta = math.log1p(math.exp(dt[0, h]))
        want = np.zeros((P, N))
        want[1] = delta * Bv[0, g]
        assert np.allclose(st[0, h], want, rtol=1e-14, atol=1e-15)
        assert y[0, h, 1] == pytest.approx(delta * float(Cv[0, g] @ Bv[0, g]) + D[h], rel=1e-13)
        assert y[0, h, 0] == 0.0 and y[0, h, 2] == 0.0
    x = rng.standard_normal((b, H, P))
    s0 = rng.standard_normal((b, H, P, N))
    _, st = oracle.step(x, dt, np.zeros(H), Bv, Cv, s0, None, dt_softplus=False)
    for h in range(H):
        g = h * G // H
        assert np.allclose(st[0, h], s0[0, h] + dt[0, h] * np.outer(x[0, h], Bv[0, g]), rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# the backward (reverse-mode derivative of the recurrence)
# ---------------------------------------------------------------------------

def _torch_loss(inp, dy, dfin, seq_idx=None, nseq=None):
    """An independent torch fp64 implementation of the recurrence (vectorised
    over batch, heads and p; resets at segment starts), returning the leaves and
    L = sum(y dy) + sum(final dfinal) so that autograd gives reference gradients."""
    import torch
    leaf = lambda a: torch.tensor(np.asarray(a.double()), dtype=torch.float64, requires_grad=True)
    x, dt, A, B, C, D, h0 = [leaf(v) for v in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states)]
    b, T, H, P = x.shape
    G = B.shape[2]
    delta = torch.nn.functional.softplus(dt) if inp.dt_softplus else dt
    h = h0
    ys, finals = [], {}
    for t in range(T):
        a = torch.exp(delta[:, t] * A)
        if seq_idx is not None and t > 0 and seq_idx[t] != seq_idx[t - 1]:
            a = torch.zeros_like(a)
        Bh = B[:, t].repeat_interleave(H // G, dim=1)
        Ch = C[:, t].repeat_interleave(H // G, dim=1)
        h = a[..., None, None] * h + (delta[:, t, :, None] * x[:, t])[..., None] * Bh[:, :, None, :]
        ys.append((h * Ch[:, :, None, :]).sum(-1) + D[:, None] * x[:, t])
        if seq_idx is not None and (t == T - 1 or seq_idx[t + 1] != seq_idx[t]):
            finals[int(seq_idx[t])] = h[0]
    y = torch.stack(ys, 1)
    L = (y * torch.tensor(dy)).sum()
    if seq_idx is None:
        L = L + (h * torch.tensor(dfin)).sum()
    else:
        for s, hf in finals.items():
            L = L + (hf * torch.tensor(dfin[s])).sum()
    L.backward()
    return dict(dx=x.grad, ddt=dt.grad, dA=A.grad, dB=B.grad, dC=C.grad, dD=D.grad, dinit=h0.grad)


@pytest.mark.parametrize("softplus", [True, False])
def test_backward_matches_autograd(softplus):
    """Every gradient of the oracle's reverse sweep against torch autograd through
    an independently written recurrence (groups shared by two heads, an initial
    state, a final-state gradient, D)."""
    inp = wl.make_inputs(2, 13, 4, 5, 6, 2, 64, "fp32", 3, init_std=0.5)
    if not softplus:
        inp.dt_softplus = False
        inp.dt = inp.dt.abs()
    rng = np.random.default_rng(1)
    dy = rng.standard_normal(tuple(inp.x.shape))
    dfin = rng.standard_normal(tuple(inp.initial_states.shape))
    gr = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.initial_states, dfin,
                         dt_softplus=inp.dt_softplus)
    ref = _torch_loss(inp, dy, dfin)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit"):
        r = ref[k].numpy()
        assert np.allclose(getattr(gr, k), r, rtol=1e-11, atol=1e-12 * max(1.0, np.abs(r).max())), k


def test_backward_packed_matches_autograd():
    """Packed segments: the carry is cut at each segment start, so the gradient
    must not flow across a boundary; each segment's final state has its own
    gradient."""
    lengths, nseq = [5, 7, 4], 3
    ids = np.concatenate([np.full(L, s) for s, L in enumerate(lengths)]).astype(np.int32)
    base = wl.make_inputs(1, sum(lengths), 2, 3, 4, 1, 64, "fp32", 9, init_std=0.4)
    rng = np.random.default_rng(4)
    dy = rng.standard_normal(tuple(base.x.shape))
    dfin = rng.standard_normal((nseq, 2, 3, 4))
    gr = oracle.backward(base.x, base.dt, base.A, base.B, base.C, dy, base.D, base.initial_states, dfin,
                         seq_idx=ids, nseq=nseq)
    ref = _torch_loss(base, dy, dfin, seq_idx=ids, nseq=nseq)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit"):
        r = ref[k].numpy()
        assert np.allclose(getattr(gr, k), r, rtol=1e-11, atol=1e-12 * max(1.0, np.abs(r).max())), k


def test_backward_finite_differences():
    """Central differences of L = sum(y dy) + sum(final dfinal), computed from the
    oracle's forward alone, against the backward on a tiny problem, for a few
    elements of every input (no torch involved)."""
    inp = wl.make_inputs(1, 6, 2, 3, 4, 1, 64, "fp32", 12, init_std=0.5)
    rng = np.random.default_rng(7)
    dy = rng.standard_normal(tuple(inp.x.shape))
    dfin = rng.standard_normal(tuple(inp.initial_states.shape))
    arrs = {k: getattr(inp, k).double().numpy().copy() for k in ("x", "dt", "A", "B", "C", "D", "initial_states")}

    def loss(a):
        r = oracle.forward(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["initial_states"])
        return float((r.y * dy).sum() + (r.final_states * dfin).sum())

    gr = oracle.backward(arrs["x"], arrs["dt"], arrs["A"], arrs["B"], arrs["C"], dy, arrs["D"],
                         arrs["initial_states"], dfin)
    names = dict(x="dx", dt="ddt", A="dA", B="dB", C="dC", D="dD", initial_states="dinit")
    eps = 1e-6
    for k, gname in names.items():
        flat = arrs[k].reshape(-1)
        for i in rng.choice(flat.size, size=min(4, flat.size), replace=False):
            keep = flat[i]
            flat[i] = keep + eps
            lp = loss(arrs)
            flat[i] = keep - eps
            lm = loss(arrs)
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            got = getattr(gr, gname).reshape(-1)[i]
            assert got == pytest.approx(fd, rel=1e-6, abs=1e-8), (k, i)


# ---------------------------------------------------------------------------
# the block's convolution prologue and gate epilogue ([scwac], section five, the
# Mamba-2 block's data flow)
# ---------------------------------------------------------------------------

def _conv_case(seed, b=2, T=29, Cc=12, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, T, Cc)), rng.uniform(-0.5, 0.5, (Cc, K)), rng.uniform(-0.5, 0.5, Cc))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_is_numpy_convolve_per_channel(K):
    """Without segments every channel is a full linear convolution with the taps
    reversed, cut to the first T outputs (numpy's routine)."""
    xbc, w, bias = _conv_case(10 + K, K=K)
    v = oracle.causal_conv1d(xbc, w, bias)
    b, T, Cc = xbc.shape
    for i in range(b):
        for c in range(Cc):
            ref = np.convolve(xbc[i, :, c], w[c, ::-1])[:T] + bias[c]
            np.testing.assert_allclose(v[i, :, c], ref, rtol=1e-13, atol=1e-13)


def test_conv_is_torch_depthwise_conv1d():
    """The same convolution as torch's grouped conv1d (one group per channel,
    K-1 zeros of padding, first T outputs), and SiLU as torch's, in fp64."""
    import torch
    import torch.nn.functional as F
    xbc, w, bias = _conv_case(3, b=3, T=41, Cc=20, K=4)
    xt = torch.from_numpy(xbc).transpose(1, 2)          # [b, C, T]
    ref = F.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias), padding=3, groups=20)
    ref = F.silu(ref[..., :41]).transpose(1, 2).numpy()
    got = oracle.silu(oracle.causal_conv1d(xbc, w, bias))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_silu_closed_forms():
    # SiLU(0) = 0; sigma(ln 3) = 3/4; SiLU(v) - SiLU(-v) = v; the tails
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([math.log(3.0)]))[0] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    v = np.linspace(-7, 7, 57)
    np.testing.assert_allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-14)
    assert oracle.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-20)
    assert abs(oracle.silu(np.array([-60.0]))[0]) < 1e-24
    assert oracle.silu(np.array([-800.0]))[0] == 0.0      # e^800 overflows to inf: -800/inf = -0


def test_conv_is_causal_and_local():
    """A change of the input at t* moves exactly the outputs t* .. t*+K-1."""
    K, ts = 4, 11
    xbc, w, bias = _conv_case(5, K=K)
    v0 = oracle.causal_conv1d(xbc, w, bias)
    x2 = xbc.copy()
    x2[:, ts, :] += 1.0
    v1 = oracle.causal_conv1d(x2, w, bias)
    T = xbc.shape[1]
    np.testing.assert_array_equal(v0[:, :ts], v1[:, :ts])
    np.testing.assert_array_equal(v0[:, ts + K:], v1[:, ts + K:])
    # the difference is the taps themselves: d v[t*+j] = w[:, K-1-j]
    for j in range(K):
        np.testing.assert_allclose(v1[:, ts + j] - v0[:, ts + j], np.broadcast_to(w[:, K - 1 - j], (2, 12)),
                                   rtol=1e-12, atol=1e-12)
    assert T > ts + K


def test_conv_restarts_in_every_packed_sequence():
    """Packed: the output equals each sequence convolved on its own."""
    xbc, w, bias = _conv_case(6, b=1, T=30, K=4)
    lens = [7, 2, 1, 14, 6]
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(lens)])
    got = oracle.causal_conv1d(xbc, w, bias, seq_idx=seq)
    o = 0
    for L in lens:
        np.testing.assert_array_equal(got[:, o:o + L], oracle.causal_conv1d(xbc[:, o:o + L], w, bias))
        o += L


def test_conv1d_silu_splits_x_then_B_then_C():
    """One tap of weight 1 and no bias turns the convolution into SiLU of the input
    itself; channel k of xbc holds the value k/100, so every output names the
    channel it came from: x takes 0 .. H*P-1 (head-major), B the next G*N (group-
    major), C the last G*N."""
    b, T, H, P, G, N = 1, 3, 2, 3, 2, 2
    Cc = H * P + 2 * G * N
    xbc = np.broadcast_to(np.arange(Cc) / 100.0, (b, T, Cc)).copy()
    x, Bm, Cm = oracle.conv1d_silu(xbc, np.ones((Cc, 1)), H, P, G, N)
    s = lambda k: (k / 100.0) / (1.0 + math.exp(-k / 100.0))
    assert x[0, 2, 1, 2] == pytest.approx(s(1 * P + 2), rel=1e-15)
    assert Bm[0, 0, 1, 0] == pytest.approx(s(H * P + 1 * N + 0), rel=1e-15)
    assert Cm[0, 1, 0, 1] == pytest.approx(s(H * P + G * N + 1), rel=1e-15)


def test_gate_is_y_times_torch_silu():
    import torch
    rng = np.random.default_rng(8)
    y, z = rng.standard_normal((2, 5, 3, 4)), rng.standard_normal((2, 5, 3, 4)) * 4
    ref = y * torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(oracle.gated(y, z), ref, rtol=1e-13, atol=1e-15)
    assert np.all(oracle.gated(y, np.zeros_like(z)) == 0.0)
