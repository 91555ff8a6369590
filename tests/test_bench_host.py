"""Host-side logic of bench.py (no GPU): the algorithmic bytes and flops
that the roofline divides by, the routing it mirrors, and the multi-GPU
refusal.  The reference figures are the per-token byte count and the
chunked method's flop formula applied by hand to the workload shapes."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mamba_ssd_chunked_chunk_amd.workloads import make_workload, with_bf16_states  # noqa: E402


def _flops_by_hand(lens, H, P, G, N, L=256):
    f = 0
    for n in lens:
        full, rem = divmod(n, L)
        for l in [L] * full + ([rem] if rem else []):
            f += 2 * l * N * P * H + 2 * l * N * P * H + l * (l + 1) * P * H + l * (l + 1) * N * G
    return f


def test_algorithmic_fixed_workload():
    """16 heads x 64, one group, dstate 256, 4 x 4096 tokens, zero initial
    states: 5184 bytes per token (x and y 2*16*64*2, B and C 2*256*2, dt
    16*4) plus each sequence's final state written (16*64*256*4)."""
    prob = make_workload("fixed_4x4096_h16_n256")
    a = bench.algorithmic(prob)
    T = 4 * 4096
    assert a["whole"]["bytes"] == T * 5184 + 4 * 16 * 64 * 256 * 4
    assert a["whole"]["flops"] == _flops_by_hand([4096] * 4, 16, 64, 1, 256)
    assert abs(a["whole"]["bytes"] / 1e6 - 89.1) < 0.1   # the figure quoted for this workload
    assert abs(a["whole"]["flops"] / 1e9 - 22.6) < 0.1
    # per kernel, the caller's buffers each kernel itself touches: chunk_scan
    # reads x and C and writes y; chunk_state reads x, B, C and dt; state
    # passing writes the pool
    assert a["ssd_chunk_scan"]["bytes"] == T * (2 * 16 * 64 * 2 + 256 * 2)
    assert a["ssd_chunk_state"]["bytes"] == T * (16 * 64 * 2 + 2 * 256 * 2 + 16 * 4)
    assert a["ssd_state_passing"]["bytes"] == 4 * 16 * 64 * 256 * 4
    assert "ssd_prep" not in a
    assert a["ssd_short"]["bytes"] == 0 and a["ssd_recur"]["bytes"] == 0


def test_algorithmic_short_routing_and_bf16_pool():
    """Short sequences count for the short-path kernels (1..4 tokens for the
    recurrence, 5..128 and zero-length ones for the MFMA kernel), the others
    for the chunked steps, and bf16 storage halves the pool bytes."""
    import numpy as np
    lens = [int(v) for v in np.random.default_rng(5).integers(0, 140, 512)]
    prob = dict(seqlens=lens, nheads=128, head_dim=64, ngroups=8, dstate=128,
                has_initial_state=np.ones(512, np.uint8), pool=np.zeros((1, 1), np.float32))
    a = bench.algorithmic(prob)
    slot = 128 * 64 * 128 * 4
    n_recur = sum(1 for n in lens if 1 <= n <= 4)
    n_short = sum(1 for n in lens if n == 0 or 5 <= n <= 128)
    tok = lambda seqs: sum(seqs) * (2 * 128 * 64 * 2 + 2 * 8 * 128 * 2 + 128 * 4)
    assert a["ssd_recur"]["bytes"] == tok([n for n in lens if 1 <= n <= 4]) + 2 * n_recur * slot
    # (a zero-length sequence with an initial state reads and writes its slot)
    assert a["ssd_short"]["bytes"] == tok([n for n in lens if 5 <= n <= 128]) + 2 * n_short * slot
    n_long = sum(1 for n in lens if n > 128)
    t_long = sum(n for n in lens if n > 128)
    assert a["ssd_chunk_state"]["bytes"] == t_long * (128 * 64 * 2 + 2 * 8 * 128 * 2 + 128 * 4)
    assert a["ssd_state_passing"]["bytes"] == 2 * n_long * slot
    off = bench.algorithmic(prob, short_max=0)  # every sequence through the chunked steps
    assert off["ssd_short"]["bytes"] == 0 and off["whole"]["bytes"] == a["whole"]["bytes"]
    b = bench.algorithmic(with_bf16_states(prob))
    assert a["whole"]["bytes"] - b["whole"]["bytes"] == 512 * 2 * slot // 2


def test_dstate_256_never_short():
    prob = make_workload("tiny_1x512_h4_n64")
    assert bench.is_short(96, 64, 128) and not bench.is_short(96, 256, 128)
    assert bench.is_short(0, 64, 128) and not bench.is_short(129, 64, 128)
    assert not bench.is_short(5, 64, 0)
    a = bench.algorithmic(prob)
    assert a["ssd_short"]["bytes"] == 0  # its one sequence is 512 tokens


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_counter_summary_ratios(tmp_path):
    """bench.py --summarize-counters: per-wavefront counts and the three
    ratios from two synthetic counter passes (two dispatches of one kernel,
    counters split over two instances; the median over dispatches)."""
    import csv
    vals = {"SQ_WAVES": 8, "SQ_WAVE_CYCLES": 1000, "SQ_BUSY_CYCLES": 1, "SQ_WAIT_INST_ANY": 1,
            "SQ_INSTS_VALU": 800, "SQ_INSTS_MFMA": 40, "SQ_INSTS_LDS": 80, "SQ_LDS_BANK_CONFLICT": 20,
            "SQ_VALU_MFMA_BUSY_CYCLES": 1280, "SQ_ACTIVE_INST_VALU": 1, "SQ_ACTIVE_INST_LDS": 1,
            "SQ_WAIT_ANY": 250, "SQ_INSTS_VMEM_RD": 16, "SQ_INSTS_VMEM_WR": 8, "SQ_INSTS_SALU": 24,
            "GRBM_GUI_ACTIVE": 1}
    for pas, names in bench.COUNTER_PASSES.items():
        d = tmp_path / pas
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for disp, scale in ((1, 1), (2, 3)):
                for c in names.split():
                    for inst in range(2):  # two instances of half the value each
                        w.writerow(dict(Dispatch_Id=disp, Kernel_Name="void ssd::ssd_chunk_scan_kernel<256, 4>(ssd::Params)",
                                        Counter_Name=c, Counter_Value=vals[c] * scale / 2))
    import contextlib, io
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench.summarize_counters(str(tmp_path))
    row = [r for r in out.getvalue().splitlines() if r.startswith("| ssd_chunk_scan")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    # median of dispatches (scale 1 and 3) = scale 2: 16 waves; per-wave counts unchanged
    assert cells == ["ssd_chunk_scan", "16", "100", "5", "10", "2", "1", "3", "0.25", "0.25", "32.00"]


def test_profile_summary_splits_read_and_write_flush_calls(tmp_path, monkeypatch):
    """bench.py --summarize-profile: the calls after the cache-evicting read
    (a reduce kernel) are the timed ones, those after a fill the comparison
    pass, and back-to-back calls count for neither; counters are calibrated
    by the copy kernel (synthetic rocprofv3 CSVs)."""
    import contextlib, csv, io
    root = tmp_path / "prof"
    names = {k: f"void ssd::{k}_kernel<256, 4>(ssd::Params)" for k in
             ("ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan")}
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int)"
    for which, per_kernel in (("fetch", 100.0), ("write", 50.0)):
        (root / which).mkdir(parents=True)
        with open(root / which / "run_counter_collection.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                               "Counter_Value"])
            w.writeheader()
            # the copy reads and writes 256 MiB: counters read half of that, so the factor is 2
            w.writerow(dict(Dispatch_Id=1, Kernel_Name=copy, Grid_Size=1, Counter_Name="X",
                            Counter_Value=bench.COPY_MIB * 1024 / 2))
            for i, n in enumerate(names.values()):
                w.writerow(dict(Dispatch_Id=2 + i, Kernel_Name=n, Grid_Size=1, Counter_Name="X",
                                Counter_Value=per_kernel))
    (root / "kt").mkdir()
    rows, t = [], 0

    def launch(name, us):
        nonlocal t
        rows.append(dict(Kernel_Name=name, Start_Timestamp=t, End_Timestamp=t + int(us * 1000)))
        t += int(us * 1000) + 500

    # a fill that sets up inputs, then a warm-up call: neither
    launch("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<unsigned char>>(int)", 70)
    for n in names.values():
        launch(n, 77)
    for call in range(2):  # timed: after the read
        launch("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<long>>(int)", 50)
        for k, n in names.items():
            launch(n, 10 + call)
    launch("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<unsigned char>>(int)", 70)
    for n in names.values():
        launch(n, 20)
    for n in names.values():  # back to back: neither
        launch(n, 99)
    with open(root / "kt" / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    with open(root / "kt" / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        for n in names.values():
            w.writerow(dict(Name=n, Calls=4, AverageNs=1000, MinNs=1000, MaxNs=1000))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "0123456789abcdef")
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench.summarize_profile(str(root), "fixed_4x4096_h16_n256")
    rows = {r.split("|")[1].strip(): [c.strip() for c in r.strip("|").split("|")]
            for r in out.getvalue().splitlines() if r.startswith("| ssd_")}
    assert rows["ssd_chunk_state"][5] == "10.50 (2)"   # after the read: 10 and 11 us
    assert rows["ssd_chunk_state"][6] == "20.00 (1)"   # after the fill
    d = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert d["sources_sha256_16"] == "0123456789abcdef"
    assert d["calibration"]["fetch"] == pytest.approx(2.0)
    # (100 + 50 KiB) x 2 per launch
    assert d["fixed_4x4096_h16_n256"]["ssd_chunk_scan"] == 300 * 1024


def test_short_path_launch_rule():
    """bench.py times the short path's kernels only where the library
    launches them: dstate <= 128, the path on, and not a single sequence
    longer than the limit."""
    def prob(lens, N):
        q = np.zeros(len(lens) + 1, np.int32)
        q[1:] = np.cumsum(lens)
        return dict(dstate=N, query_start_loc=q, total_len=int(q[-1]))
    f = bench.launches_short_path
    assert not f(prob([100, 50], 256), -1)
    assert not f(prob([100, 50], 128), 0)
    assert not f(prob([129], 64), -1) and f(prob([128], 64), -1)
    assert not f(prob([200], 128), 100) and f(prob([100], 128), 100)
    assert f(prob([300, 300], 128), -1) and f(prob([0], 64), -1)


def test_counted_traffic_sums_the_call(monkeypatch):
    """The whole call's counted traffic is the sum over its kernels, and
    nothing is reported where the counters do not apply (another routing,
    bf16 states, the separate-states entry) or a kernel has none."""
    import types
    table = {"w": {"ssd_chunk_state": 10, "ssd_state_passing": 20, "ssd_chunk_scan": 30}}
    monkeypatch.setattr(bench, "traffic_for", lambda k, w: table.get(w, {}).get(k))
    args = types.SimpleNamespace(short_max=bench.SHORT_MAX, state_dtype="f32", entry="inplace")
    ks = ["ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan"]
    t = bench.counted_traffic("w", ks, args)
    assert t["whole"] == 60 and t["ssd_chunk_scan"] == 30
    assert bench.counted_traffic("w", ks + ["ssd_short"], args)["whole"] is None
    assert bench.counted_traffic("other", ks, args)["whole"] is None
    for kw in (dict(short_max=0), dict(state_dtype="bf16"), dict(entry="separate")):
        a = types.SimpleNamespace(**dict(vars(args), **kw))
        t = bench.counted_traffic("w", ks, a)
        assert all(v is None for v in t.values()), kw
