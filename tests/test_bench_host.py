"""Host-side pieces of bench.py: work counts, percentiles, counter records, the
one-GPU guard. No GPU needed."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_work_long_workload():
    # 16K tokens, 32 heads of 64, N = 256, one group, chunk 256, bf16
    shape = dict(batch=1, seqlen=16384, nheads=32, headdim=64, dstate=256, ngroups=1, chunk=256)
    w = bench.algorithmic_work(shape, 2, False)
    T, H, P, N, Q = 16384, 32, 64, 256, 256
    # chunk_state: one multiply-add per (t, h, p, n)
    assert w["chunk_state"]["flops"] == 2 * T * H * P * N
    # chunk_scan: the causal half (with diagonal) of the Q x Q block product, plus C h
    assert w["chunk_scan"]["flops"] == pytest.approx(2 * T * H * P * (Q + 1) / 2 + 2 * T * H * N * P)
    # state_passing reads and writes every bf16 state once, plus the fp32 chunk sums and
    # the fp32 initial and final states
    nc = T // Q
    assert w["state_passing"]["bytes"] == 2 * nc * H * P * N * 2 + H * nc * 4 + 2 * H * P * N * 4


def test_percentiles():
    p = bench.percentiles([float(i) for i in range(101)])
    assert (p["p10"], p["p50"], p["p90"]) == (10.0, 50.0, 90.0)
    assert bench.percentiles([3.0]) == {"p10": 3.0, "p50": 3.0, "p90": 3.0}


@pytest.mark.parametrize("pattern,prefix", [("*hbm_traffic*.md", "traffic-record: "),
                                            ("*mfma_util*.md", "mfma-record: ")])
def test_counter_records_parse(pattern, prefix):
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", pattern)))
    assert paths, f"no committed {pattern} records"
    src = bench.kernel_source_hash()
    for path in paths:
        recs = [json.loads(l[len(prefix):]) for l in open(path) if l.startswith(prefix)]
        assert recs, path
        for r in recs:
            assert {"kernel", "workload", "source_sha256"} <= set(r)
            if r["source_sha256"] != src:
                continue   # taken from older kernels: the bench ignores it
            if prefix.startswith("traffic"):
                assert bench.measured_traffic(r["kernel"], r["workload"]) == int(r["fetch_bytes"] + r["write_bytes"])
            else:
                assert bench.measured_mfma(r["kernel"], r["workload"]) == r["mfma_busy_pct"]
    assert bench.measured_traffic("chunk_scan", "no such workload") is None
    assert bench.measured_mfma("chunk_scan", "no such workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_point_picks_the_binding_roof():
    # bf16 ridge point: 2500 TFLOP/s over 8000 GB/s = 312.5 FLOP/B
    below = bench.roofline_point({"flops": 100e9, "bytes": 1e9}, 1e-3, 2)     # 100 FLOP/B
    assert below["bound"] == "hbm" and below["unit"] == "GB/s"
    assert below["achieved"] == pytest.approx(1000.0) and below["frac"] == pytest.approx(0.125)
    assert below["mfma_frac"] == pytest.approx(100 / 2500, abs=1e-4)
    above = bench.roofline_point({"flops": 1000e9, "bytes": 1e9}, 1e-3, 2)    # 1000 FLOP/B
    assert above["bound"] == "mfma" and above["unit"] == "TFLOP/s"
    assert above["frac"] == pytest.approx(0.4) and above["hbm_frac"] == pytest.approx(0.125)
    # fp32 has its own ridge: 157.3 TFLOP/s over 8000 GB/s ~ 19.7 FLOP/B
    assert bench.roofline_point({"flops": 100e9, "bytes": 1e9}, 1e-3, 4)["bound"] == "mfma"
    copy = bench.roofline_point({"bytes": 4e9}, 1e-3, 2)
    assert copy["bound"] == "hbm" and copy["frac"] == pytest.approx(0.5) and "mfma_frac" not in copy


def test_seq_final_work_counts_each_sequences_tail_rows():
    # chunk 4; ids 0 0 0 | 0 0 1 1 | 1 2 2 2 (nseq 4: id 3 never occurs)
    ids = [0, 0, 0, 0, 0, 1, 1, 1, 2, 2, 2]
    shape = dict(nheads=2, headdim=16, dstate=16, ngroups=1, chunk=4, nseq=4)
    w = bench.seq_final_work(shape, 2, ids)
    H, P, N, G = 2, 16, 16, 1
    # id 0 ends at t=4 (chunk 1, open since t=0): 1 row + the entering state
    # id 1 ends at t=7 (chunk 1, starts at t=5 inside it): 3 rows, no entering state
    # id 2 ends at t=10 (chunk 2, starts at t=8 = chunk start): 3 rows, no entering state
    rows = 1 + 3 + 3
    assert w["flops"] == 2.0 * rows * H * P * N
    want = 4 * H * P * N * 4 + len(ids) * 4 + rows * (H * P * 2 + G * N * 2 + 2 * H * 4) + H * P * N * 2
    assert w["bytes"] == want


def test_backward_stage_work_covers_every_stage():
    """Every stage name ssd_bwd_stage_times reports has an algorithmic work entry,
    and the products that dominate carry FLOPs."""
    import bench
    shape = dict(batch=1, seqlen=16384, nheads=32, headdim=64, dstate=256, ngroups=1, chunk=256)
    w = bench.backward_stage_work(shape, 2, nseq=0)
    names = ["chunk_cb", "chunk_state", "state_passing", "chunk_map", "chunk_cb_rev",
             "chunk_state_grad", "inject_dfinal", "state_passing_rev", "chunk_scan_dx", "chunk_scan_dy_hin",
             "m_rows_cols", "dl_ddt_dA_dD", "dC", "dB"]
    assert set(names) == set(w)
    for n in names:
        assert w[n]["bytes"] >= 0, n
    for n in ("chunk_state_grad", "chunk_scan_dx", "chunk_scan_dy_hin", "m_rows_cols", "dC", "dB"):
        assert w[n]["flops"] > 0, n
    # the reversed scan moves what the forward scan moves plus x, dx and its dot products
    f = bench.algorithmic_work(shape, 2, None)
    assert w["chunk_scan_dx"]["bytes"] > f["chunk_scan"]["bytes"]
