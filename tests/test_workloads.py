"""The seeded input recipe: determinism, shapes, dtypes and the packed layout."""
import math

import numpy as np
import torch

from ssd_chunked_scan_amd import workloads as wl


def test_deterministic_and_seeded():
    a = wl.workload(0)
    b = wl.workload(0)
    c = wl.workload(0, seed=5)
    assert torch.equal(a.x, b.x) and torch.equal(a.dt, b.dt) and torch.equal(a.A, b.A)
    assert not torch.equal(a.x, c.x)


def test_tiny_fp32_shapes_and_laws():
    w = wl.workload(0)
    assert w.x.shape == (1, 256, 2, 16) and w.x.dtype == torch.float32
    assert w.B.shape == (1, 256, 1, 16) and w.C.shape == (1, 256, 1, 16)
    assert w.dt.shape == (1, 256, 2) and w.A.shape == (2,) and w.D.shape == (2,)
    assert w.initial_states is None and w.seq_idx is None and w.chunk == 64
    assert ((w.A <= -1.0) & (w.A >= -16.0)).all()


def test_bf16_workload_is_rounded_from_fp32():
    w = wl.workload(1, batch=1, seqlen=128, nheads=2)  # same recipe, reduced shape
    assert w.x.dtype == torch.bfloat16 and w.dt.dtype == torch.bfloat16
    assert w.A.dtype == torch.float32 and w.initial_states.dtype == torch.float32
    assert w.initial_states.shape == (1, 2, 64, 64)
    assert abs(float(w.initial_states.std()) - 0.1) < 0.01
    assert abs(float(w.B.float().std()) * math.sqrt(64) - 1.0) < 0.05


def test_packed_layout():
    # the lengths are the first draw, so a reduced-width variant has the same packing
    w = wl.workload(4, nheads=2, headdim=4, dstate=8, ngroups=1)
    assert len(w.lengths) == 16 and all(128 <= L <= 2048 for L in w.lengths)
    T = w.x.shape[1]
    assert T % 128 == 0 and T - sum(w.lengths) < 128
    sid = w.seq_idx.numpy()
    assert sid.shape == (T,) and (np.diff(sid) >= 0).all() and sid[0] == 0
    real = sum(w.lengths)
    if T > real:
        assert w.nseq == 17 and (sid[real:] == 16).all()
        assert not w.x[:, real:].any() and not w.B[:, real:].any() and not w.C[:, real:].any()
    else:
        assert w.nseq == 16
    assert w.real_tokens == real


def test_device_inputs_recipe():
    """The device-side draw (used for the maximum-size case) on the CPU: seeded,
    the recipe's shapes, dtypes and laws."""
    a = wl.device_inputs(1, 3000, 4, 64, 32, 1, 256, "bf16", seed=3, device="cpu")
    b = wl.device_inputs(1, 3000, 4, 64, 32, 1, 256, "bf16", seed=3, device="cpu")
    c = wl.device_inputs(1, 3000, 4, 64, 32, 1, 256, "bf16", seed=4, device="cpu")
    assert torch.equal(a.x, b.x) and torch.equal(a.B, b.B) and torch.equal(a.A, b.A)
    assert not torch.equal(a.x, c.x)
    assert a.x.shape == (1, 3000, 4, 64) and a.x.dtype == torch.bfloat16
    assert a.B.shape == (1, 3000, 1, 32) and a.C.shape == (1, 3000, 1, 32) and a.dt.shape == (1, 3000, 4)
    assert a.A.dtype == torch.float32 and a.initial_states.shape == (1, 4, 64, 32)
    assert ((a.A <= -1.0) & (a.A >= -16.0)).all()
    assert abs(float(a.x.float().std()) - 1.0) < 0.02
    assert abs(float(a.B.float().std()) * math.sqrt(32) - 1.0) < 0.05
    assert abs(float(a.dt.float().mean()) + 3.0) < 0.02 and abs(float(a.dt.float().std()) - 0.5) < 0.02
    assert abs(float(a.initial_states.std()) - 0.1) < 0.01
