"""Host-only checks of the C ABI (no GPU work): the library loads, exports every
entry point that include/ssd.h declares, and rejects invalid arguments with the
documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from ssd_chunked_scan_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULLP, SHAPE, DTYPE, CHUNK, GROUPS, SEQ, WS, MISAL, ALIAS, HIP, SCRATCH = range(12)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssd_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd.so not built")
    return ssd.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ssd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ssd_abi_version() == 2


def test_status_strings(lib):
    for code in range(12):
        s = ssd.status_string(code)
        assert s and s != "unknown status"
    assert ssd.status_string(99) == "unknown status"


def _args(**kw):
    base = dict(batch=1, seqlen=256, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64,
                dtype=1, dt_softplus=1)
    base.update({k: v for k, v in kw.items() if k in base})
    a = ssd.FwdArgs(base["batch"], base["seqlen"], base["nheads"], base["headdim"], base["dstate"],
                    base["ngroups"], base["chunk"], base["dtype"], base["dt_softplus"])
    # fake, 16-byte aligned, non-overlapping host addresses: validation never dereferences them
    addr = 0x10000000
    for name in ("x", "dt", "A", "B", "C", "D", "y", "final_states", "workspace"):
        setattr(a, name, kw.get(name, addr))
        addr += 0x10000000
    a.workspace_bytes = kw.get("workspace_bytes", 1 << 40)
    if "seq_idx" in kw:
        a.seq_idx = kw["seq_idx"]
        a.nseq = kw.get("nseq", 1)
    return a


def _fwd(lib, a):
    return lib.ssd_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), DTYPE),
    (dict(chunk=32), CHUNK), (dict(chunk=100), CHUNK), (dict(chunk=512), CHUNK),
    (dict(nheads=6, ngroups=4), GROUPS),
    (dict(headdim=24), SHAPE), (dict(dstate=40), SHAPE), (dict(dstate=512), SHAPE),
    (dict(batch=0), SHAPE), (dict(seqlen=-1), SHAPE), (dict(headdim=8), SHAPE),
    (dict(batch=2, seq_idx=0x90000000, nseq=3), SEQ),
    (dict(seq_idx=0x90000000, nseq=0), SEQ),
    (dict(x=0), NULLP), (dict(A=0), NULLP), (dict(y=0), NULLP), (dict(workspace=0), NULLP),
    (dict(x=0x10000008), MISAL), (dict(D=0x60000004), MISAL),
    (dict(workspace_bytes=16), WS),
    (dict(y=0x10000000), ALIAS),                 # y == x
    (dict(final_states=0x70000000 + 64), ALIAS),  # overlaps y
    (dict(workspace=0x10000000), ALIAS),
])
def test_fwd_rejects_invalid_arguments(lib, kw, code):
    assert _fwd(lib, _args(**kw)) == code


def test_workspace_size(lib):
    a = _args(batch=2, seqlen=2048, nheads=24, headdim=64, dstate=64, chunk=64)
    n = ctypes.c_size_t()
    assert lib.ssd_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == OK
    nc = 32
    al = lambda v: (v + 255) // 256 * 256
    # delta and cs; CB plus the C and B^T copies (Q x (Q + 2 * 64) per chunk and group); the chunk states
    want = al(2 * 24 * nc * 64 * 4) * 2 + al(2 * nc * 1 * 64 * (64 + 2 * 64) * 2) + al(2 * nc * 24 * 64 * 64 * 2)
    assert n.value == want
    bad = _args(chunk=48)
    assert lib.ssd_fwd_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == CHUNK


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """ssd_fwd_noalloc validates like ssd_fwd and refuses, before any HIP call, a
    problem whose workspace exceeds the static scratch (the 2.7B-shaped workload
    needs about 190 MiB; the long 16K-token one about 92 MiB fits)."""
    big = _args(batch=8, seqlen=2048, nheads=80, headdim=64, dstate=128, chunk=128, workspace=0)
    n = ctypes.c_size_t()
    assert lib.ssd_fwd_workspace_size(ctypes.byref(big), ctypes.byref(n)) == OK
    assert n.value > ssd.NOALLOC_SCRATCH_BYTES
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), None) == SCRATCH
    fits = _args(batch=1, seqlen=16384, nheads=32, headdim=64, dstate=256, chunk=256)
    assert lib.ssd_fwd_workspace_size(ctypes.byref(fits), ctypes.byref(n)) == OK
    assert n.value <= ssd.NOALLOC_SCRATCH_BYTES
    # the ordinary argument checks come first
    assert lib.ssd_fwd_noalloc(ctypes.byref(_args(chunk=32)), None) == CHUNK
    assert lib.ssd_fwd_noalloc(ctypes.byref(_args(x=0)), None) == NULLP
    assert lib.ssd_fwd_noalloc(ctypes.byref(_args(y=0x10000000)), None) == ALIAS
    assert lib.ssd_fwd_noalloc(None, None) == NULLP


def test_step_entry_points_validate(lib):
    a = _args()
    p = ctypes.c_void_p
    assert lib.ssd_chunk_cumsum(ctypes.byref(a), None, p(0x90000000), None) == NULLP
    assert lib.ssd_chunk_cumsum(ctypes.byref(a), p(0x90000004), p(0x90000000), None) == MISAL
    assert lib.ssd_chunk_cb(ctypes.byref(a), None, None) == NULLP
    assert lib.ssd_chunk_state(ctypes.byref(a), p(0x90000000), None, p(0xb0000000), p(0xa0000000), None) == NULLP
    assert lib.ssd_chunk_state(ctypes.byref(a), p(0x90000000), p(0x98000000), None, p(0xa0000000), None) == NULLP
    assert lib.ssd_state_passing(ctypes.byref(a), None, p(0xa0000000), None) == NULLP
    assert lib.ssd_chunk_scan(ctypes.byref(a), p(1 << 33), p(2 << 33), None, p(3 << 33), None) == NULLP
    # seq_final_states only makes sense for a packed stream
    assert lib.ssd_seq_final_states(ctypes.byref(a), p(1 << 33), p(2 << 33), p(3 << 33), p(4 << 33),
                                    None) == SEQ
    bad = _args(chunk=96)
    assert lib.ssd_chunk_cb(ctypes.byref(bad), p(1 << 33), None) == CHUNK


def test_binding_rejects_host_tensors_and_copies():
    x = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError, match="GPU"):
        ssd.Problem(x, x[..., 0], torch.zeros(2), x[:, :, :1], x[:, :, :1], 64)


def _step_args(**kw):
    base = dict(batch=8, nheads=4, headdim=64, dstate=128, ngroups=1, dtype=1, dt_softplus=1)
    base.update({k: v for k, v in kw.items() if k in base})
    a = ssd.StepArgs(**base)
    addr = 0x10000000
    for name in ("x", "dt", "A", "B", "C", "D", "state", "y"):
        setattr(a, name, kw.get(name, addr))
        addr += 0x10000000
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), DTYPE),
    (dict(nheads=6, ngroups=4), GROUPS),
    (dict(headdim=24), SHAPE), (dict(dstate=40), SHAPE), (dict(dstate=272), SHAPE),
    (dict(batch=0), SHAPE), (dict(headdim=0), SHAPE), (dict(batch=1 << 20, nheads=1 << 12), SHAPE),
    (dict(x=0), NULLP), (dict(dt=0), NULLP), (dict(A=0), NULLP), (dict(B=0), NULLP), (dict(C=0), NULLP),
    (dict(state=0), NULLP), (dict(y=0), NULLP),
    (dict(x=0x10000008), MISAL), (dict(state=0x70000004), MISAL), (dict(D=0x60000002), MISAL),
    (dict(y=0x10000000), ALIAS),                 # y == x
    (dict(state=0x40000000), ALIAS),             # state == B
    (dict(y=0x70000000 + 1024), ALIAS),          # y inside the state
])
def test_step_rejects_invalid_arguments(lib, kw, code):
    assert lib.ssd_step(ctypes.byref(_step_args(**kw)), None) == code
    assert lib.ssd_step(None, None) == NULLP


def test_step_binding_checks_shapes():
    x = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        ssd.step_args(x, torch.zeros(2, 4), torch.zeros(4), torch.zeros(2, 1, 64), torch.zeros(2, 1, 64),
                      torch.zeros(2, 4, 64, 64))
    with pytest.raises(ValueError, match="batch, nheads, headdim"):
        ssd.step_args(torch.zeros(2, 4, 1, 64), None, None, None, None, None)


def _bwd_args(**kw):
    addr = 0xa0000000
    g = ssd.BwdArgs()
    for name in ("dy", "dfinal_states", "dx", "ddt", "dA", "dB", "dC", "dD", "dinitial_states", "workspace"):
        setattr(g, name, kw.get(name, addr))
        addr += 0x10000000
    g.workspace_bytes = kw.get("workspace_bytes", 1 << 40)
    g.fwd_workspace = kw.get("fwd_workspace", 0)
    g.fwd_workspace_bytes = kw.get("fwd_workspace_bytes", 1 << 40)
    return g


@pytest.mark.parametrize("fkw,gkw,code", [
    (dict(seq_idx=0x90000000, nseq=1, batch=2), dict(), SEQ),   # packed streams need batch 1
    (dict(chunk=96), dict(), CHUNK),
    (dict(y=0), dict(), NULLP),                                 # the forward output is an input here
    (dict(), dict(dy=0), NULLP), (dict(), dict(dx=0), NULLP), (dict(), dict(dA=0), NULLP),
    (dict(), dict(dB=0), NULLP), (dict(), dict(workspace=0), NULLP),
    (dict(), dict(dx=0xa0000008), MISAL),
    (dict(), dict(workspace_bytes=64), WS),
    (dict(), dict(dx=0x10000000), ALIAS),                       # dx == x
    (dict(), dict(dC=0xa0000000 + 256), ALIAS),                 # dC inside dy
    (dict(), dict(dB=0xa0000000 + 0x20000000), ALIAS),          # dB == dx
    (dict(), dict(fwd_workspace=0x1a0000008), MISAL),
    (dict(), dict(fwd_workspace=0x1a0000000, fwd_workspace_bytes=256), WS),
    (dict(), dict(fwd_workspace=0xa0000000 + 0x20000000), ALIAS),   # the forward's workspace == dx
    (dict(), dict(fwd_workspace=0xa0000000 + 0x90000000), ALIAS),   # ... == the backward's workspace
])
def test_bwd_rejects_invalid_arguments(lib, fkw, gkw, code):
    a = _args(**fkw)
    if "y" in fkw:
        a.y = fkw["y"]
    assert lib.ssd_bwd(ctypes.byref(a), ctypes.byref(_bwd_args(**gkw)), None) == code
    # the stage-timed backward makes the same checks before it touches the GPU
    ms = (ctypes.c_float * ssd.BWD_MAX_STAGES)()
    names = (ctypes.c_char_p * ssd.BWD_MAX_STAGES)()
    n = ctypes.c_int(-1)
    assert lib.ssd_bwd_stage_times(ctypes.byref(a), ctypes.byref(_bwd_args(**gkw)), None, ssd.BWD_MAX_STAGES,
                                   ms, names, ctypes.byref(n)) == code
    assert n.value == 0


def test_bwd_stage_times_rejects_short_or_missing_outputs(lib):
    a, g = _args(), _bwd_args()
    ms = (ctypes.c_float * ssd.BWD_MAX_STAGES)()
    names = (ctypes.c_char_p * ssd.BWD_MAX_STAGES)()
    n = ctypes.c_int(0)
    f = lib.ssd_bwd_stage_times
    assert f(ctypes.byref(a), ctypes.byref(g), None, ssd.BWD_MAX_STAGES - 1, ms, names, ctypes.byref(n)) == SHAPE
    assert f(ctypes.byref(a), ctypes.byref(g), None, ssd.BWD_MAX_STAGES, None, names, ctypes.byref(n)) == NULLP
    assert f(ctypes.byref(a), ctypes.byref(g), None, ssd.BWD_MAX_STAGES, ms, None, ctypes.byref(n)) == NULLP
    assert f(ctypes.byref(a), ctypes.byref(g), None, ssd.BWD_MAX_STAGES, ms, names, None) == NULLP


def test_bwd_max_stages_matches_the_header():
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "ssd.h")).read()
    assert int(re.search(r"#define SSD_BWD_MAX_STAGES (\d+)", text).group(1)) == ssd.BWD_MAX_STAGES


def test_bwd_workspace_size(lib):
    a = _args(batch=2, seqlen=2048, nheads=24, headdim=64, dstate=64, chunk=64)
    n = ctypes.c_size_t()
    assert lib.ssd_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == OK
    m = ctypes.c_size_t()
    assert lib.ssd_fwd_workspace_size(ctypes.byref(a), ctypes.byref(m)) == OK
    assert n.value > m.value
    # a packed stream also holds its copy laid out with every segment starting at a
    # chunk start (each of the nseq segments padded by fewer than `chunk` tokens)
    plain = _args(seqlen=4096, nheads=8, chunk=128)
    packed = _args(seqlen=4096, nheads=8, chunk=128, seq_idx=0x90000000, nseq=5)
    assert lib.ssd_bwd_workspace_size(ctypes.byref(plain), ctypes.byref(n)) == OK
    assert lib.ssd_bwd_workspace_size(ctypes.byref(packed), ctypes.byref(m)) == OK
    assert m.value > n.value
    assert lib.ssd_bwd_workspace_size(ctypes.byref(_args(seq_idx=0x90000000, nseq=0)), ctypes.byref(n)) == SEQ


@pytest.mark.parametrize("z,code", [
    (0, NULLP), (0xb0000008, MISAL),
    (0x70000000, ALIAS),                 # z == y
    (0x80000000 + 128, ALIAS),           # z inside final_states
    (0x90000000, ALIAS),                 # z == workspace
])
def test_fwd_gated_rejects_invalid_gate(lib, z, code):
    a = _args()
    assert lib.ssd_fwd_gated(ctypes.byref(a), ctypes.c_void_p(z), None) == code


def test_fwd_gated_checks_the_forward_arguments_too(lib):
    assert lib.ssd_fwd_gated(ctypes.byref(_args(chunk=48)), ctypes.c_void_p(0xb0000000), None) == CHUNK
    assert lib.ssd_fwd_gated(ctypes.byref(_args(y=0x10000000)), ctypes.c_void_p(0xb0000000), None) == ALIAS


def _conv_args(**kw):
    base = dict(batch=1, seqlen=256, nheads=4, headdim=64, ngroups=1, dstate=64, width=4, dtype=1)
    base.update({k: v for k, v in kw.items() if k in base})
    a = ssd.ConvArgs(**base)
    addr = 0x10000000
    for name in ("xbc", "weight", "bias", "x", "B", "C"):
        setattr(a, name, kw.get(name, addr))
        addr += 0x10000000
    a.seq_idx = kw.get("seq_idx", 0)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), DTYPE),
    (dict(width=0), SHAPE), (dict(width=5), SHAPE), (dict(headdim=8), SHAPE), (dict(dstate=24), SHAPE),
    (dict(batch=0), SHAPE), (dict(seqlen=-1), SHAPE),
    (dict(nheads=1 << 40, headdim=1 << 40), SHAPE),          # no int64 overflow in the channel count
    (dict(batch=1 << 20, seqlen=1 << 20), SHAPE),            # beyond the supported element count
    (dict(nheads=6, ngroups=4), GROUPS),
    (dict(batch=2, seq_idx=0x90000000), SEQ),
    (dict(xbc=0), NULLP), (dict(weight=0), NULLP), (dict(C=0), NULLP),
    (dict(xbc=0x10000004), MISAL), (dict(bias=0x30000008), MISAL),
    (dict(x=0x10000000 + 512), ALIAS),     # x inside xbc
    (dict(B=0x60000000), ALIAS),           # B == C
    (dict(C=0x20000000), ALIAS),           # C == weight
    (dict(seqlen=0, xbc=0, x=0), OK),      # nothing to do, nothing read
])
def test_conv_rejects_invalid_arguments(lib, kw, code):
    assert lib.ssd_conv1d_silu(ctypes.byref(_conv_args(**kw)), None) == code


def test_conv_binding_checks_shapes():
    xbc = torch.zeros(1, 8, 4 * 16 + 2 * 16)
    with pytest.raises(ValueError, match="GPU"):
        ssd.conv1d_silu(xbc, torch.zeros(96, 4), 4, 16, 1, 16)
    with pytest.raises(ValueError, match="channels"):
        ssd.conv1d_silu(xbc, torch.zeros(96, 4), 4, 16, 1, 32)


def test_check_seq_idx_rejects_invalid_arguments(lib):
    p = ctypes.c_void_p
    f = lib.ssd_check_seq_idx
    i64 = ctypes.c_int64
    assert f(p(0x90000000), i64(100), i64(3), None, None) == NULLP
    assert f(None, i64(100), i64(3), p(0x90001000), None) == NULLP
    assert f(p(0x90000000), i64(-1), i64(3), p(0x90001000), None) == SHAPE
    assert f(p(0x90000000), i64(1 << 31), i64(3), p(0x90001000), None) == SHAPE
    assert f(p(0x90000000), i64(100), i64(0), p(0x90001000), None) == SEQ
    assert f(p(0x90000002), i64(100), i64(3), p(0x90001000), None) == MISAL
    assert f(p(0x90000000), i64(100), i64(3), p(0x90001002), None) == MISAL
