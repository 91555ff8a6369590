#!/usr/bin/env python3
"""Benchmark of the libssd varlen SSD scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of ssd_chunk_scan_varlen_fwd_inplace (every kernel of the
scan) over one batch of synthetic input already resident in HBM.  Each timed
step first evicts the caches (a 512 MiB fill, outside the timed events), then
the call is bracketed by HIP events; ms_per_step is the mean over the K steps
and `value` = total tokens / that time.  Per-kernel durations come from the
events the library records between its launches on the same stream.

Prints ONE JSON line (the metric and workload of the 16-head x head_dim 64,
dstate 256 benchmark), with a roofline object for the dominant kernel and a
cpu_baseline object for the fp64 oracle timed on this host.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD scan µs/call + tokens/s (16h×64, dstate 256); % of HBM/MFMA roofline"
DEFAULT_WORKLOAD = "fixed_4x4096_h16_n256"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16/fp16 MFMA, TFLOP/s
CHUNK = 256
SHORT_MAX = 128              # the library's default short-path maximum
RECUR_MAX = 4                # of those, the longest the token-recurrence kernel takes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-workload lines (every workload of PER_CONFIG, timed after the headline)")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed calls per workload of the per-workload lines")
    ap.add_argument("--entry", choices=("inplace", "separate"), default="inplace",
                    help="entry point to time: the in-place pool operation (default) or the one with "
                         "separate initial_states / final_states (sequences without an initial state "
                         "start from zero rows; none at all passes NULL)")
    ap.add_argument("--short-max", type=int, default=SHORT_MAX,
                    help="ssd_problem.short_path_max of every call: longest sequence routed to the fused "
                         "short-sequence kernel (dstate <= 128; 0 sends every sequence through the chunked steps)")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default="f32",
                    help="storage type of the pool / states (bf16: rounded once per final state; the "
                         "arithmetic stays fp32)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU oracle time for the baseline sample")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="no GPU run: summarise the rocprofv3 output under DIR (kt/, fetch/, write/) "
                         "for --workload, print it as markdown and write profiles/traffic.json")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="no GPU run: print the shader-counter table of the two rocprofv3 --pmc passes "
                         "under DIR (p1/, p2/: the counters of COUNTER_PASSES)")
    return ap.parse_args()


# ------------------------------------------------------------------ HIP events

class Hip:
    """hipEvent_* through ctypes, so events can be recorded by the library on
    the very stream its kernels run on."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        t = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return t.value


# ------------------------------------------------------- algorithmic figures

def is_short(L, N, short_max):
    """Whether the library routes a sequence of L tokens to the short path
    (with the path on, zero-length sequences are finished there too)."""
    return N <= 128 and short_max > 0 and L <= short_max


def algorithmic(prob, short_max=SHORT_MAX):
    """Compulsory bytes and chunked-method MFMA flops of the whole call and of
    each kernel: bytes every call must move (x, y, B, C, dt, the pool slots
    read and written) and the MFMA flops of the chunked form.  Sequences the
    short path takes count for ssd_recur (up to RECUR_MAX tokens) or
    ssd_short, the others for the chunked steps."""
    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    lens = prob["seqlens"]
    hi = prob.get("has_initial_state")
    slot = H * P * N * (2 if prob.get("state_dtype", "f32") == "bf16" else 4)

    def part(seqs):
        T = sum(lens[b] for b in seqs)
        n_init = sum(int(hi[b]) for b in seqs) if hi is not None else 0
        bx, bbc, bdt = T * H * P * 2, T * G * N * 2, T * H * 4
        # flops per chunk of length l and head: state 2lNP, off-diagonal
        # 2lNP, causal diagonal l(l+1)P, causal C.B^T shared by the H/G heads
        f = dict(state=0, off=0, diag=0, cb=0)
        for b in seqs:
            full, rem = divmod(lens[b], CHUNK)
            for l in [CHUNK] * full + ([rem] if rem else []):
                f["state"] += 2 * l * N * P * H
                f["off"] += 2 * l * N * P * H
                f["diag"] += l * (l + 1) * P * H
                f["cb"] += l * (l + 1) * N * G
        return bx, bbc, bdt, (n_init + len(seqs)) * slot, f

    recur_max = min(short_max, RECUR_MAX)
    recur = [b for b in range(len(lens)) if is_short(lens[b], N, short_max) and 1 <= lens[b] <= recur_max]
    short = [b for b in range(len(lens)) if is_short(lens[b], N, short_max) and not 1 <= lens[b] <= recur_max]
    chunked = [b for b in range(len(lens)) if not is_short(lens[b], N, short_max)]
    bx, bbc, bdt, pool_rw, f = part(chunked)
    sx, sbc, sdt, spool, sf = part(short)
    rx, rbc, rdt, rpool, _ = part(recur)  # VALU recurrence: no MFMA flops
    fl = sum(f.values()) + sum(sf.values())
    # per kernel: the caller's buffers that kernel itself reads or writes (a
    # buffer that two kernels read counts for both, so the shares can sum to
    # more than the call; the whole call counts every buffer once)
    return dict(
        whole=dict(bytes=2 * (bx + sx + rx) + 2 * (bbc + sbc + rbc) + bdt + sdt + rdt + pool_rw + spool + rpool,
                   flops=fl),
        ssd_chunk_state=dict(bytes=bx + 2 * bbc + bdt, flops=f["state"] + f["cb"]),
        ssd_state_passing=dict(bytes=pool_rw, flops=0),
        ssd_chunk_scan=dict(bytes=2 * bx + bbc, flops=f["off"] + f["diag"]),
        ssd_short=dict(bytes=2 * sx + 2 * sbc + sdt + spool, flops=sum(sf.values())),
        ssd_recur=dict(bytes=2 * rx + 2 * rbc + rdt + rpool, flops=0),
    )


def roofline_entry(name, alg, t_us, traffic=None):
    a = alg[name]
    t_hbm = a["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = a["flops"] / (MFMA_BF16_PEAK_TFS * 1e12) * 1e6
    if t_mfma > t_hbm:
        achieved = a["flops"] / (t_us * 1e-6) / 1e12
        return dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_BF16_PEAK_TFS, 4), traffic=traffic, kernel=name)
    achieved = a["bytes"] / (t_us * 1e-6) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=name)


def kernel_sources_hash():
    """Hash of the kernel sources with comments and runs of white space
    removed: counters stay valid across edits that change no code."""
    import re
    csrc = os.path.join(ROOT, "mamba_ssd_chunked_chunk_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(csrc, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update((f + ":" + " ".join(text.split()) + "\n").encode())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("sources_sha256_16") != kernel_sources_hash():
        return None
    return d.get(workload, {}).get(kernel)


# ------------------------------------------------------- copy probe + counters

COPY_MIB = 256


def copy_probe(torch, dev, hip, stream, reps=5):
    """A plain streaming copy of COPY_MIB MiB (fp32 dst = src * 1) timed with
    HIP events: the achievable HBM rate beside the 8 TB/s peak, and the kernel
    of known size whose FETCH_SIZE / WRITE_SIZE readings calibrate the
    counters."""
    n = (COPY_MIB << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    e0, e1 = hip.event(), hip.event()
    hip.lib.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    hip.lib.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
    hip.lib.hipEventSynchronize(e1)
    ms = hip.elapsed_ms(e0, e1) / reps
    return round(2 * (COPY_MIB << 20) / (ms * 1e-3) / 1e9, 1)


def _per_dispatch(csv_path):
    """{dispatch id: (kernel name, grid size, summed counter value)} of one
    rocprofv3 counter-collection CSV (values summed over the instances)."""
    import csv
    out = {}
    for r in csv.DictReader(open(csv_path)):
        d = int(r["Dispatch_Id"])
        name, grid, v = out.get(d, (r["Kernel_Name"], int(r["Grid_Size"]), 0.0))
        out[d] = (name, grid, v + float(r["Counter_Value"]))
    return out


def _per_dispatch_counters(csv_path):
    """{dispatch id: (kernel name, {counter: value summed over instances})}."""
    import csv
    out = {}
    for r in csv.DictReader(open(csv_path)):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


COUNTER_PASSES = {
    "p1": "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
          "SQ_LDS_BANK_CONFLICT",
    "p2": "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_ANY SQ_INSTS_VMEM_RD "
          "SQ_INSTS_VMEM_WR SQ_INSTS_SALU GRBM_GUI_ACTIVE",
}


def summarize_counters(root):
    """Markdown table of the libssd kernels' shader counters from the two
    rocprofv3 --pmc passes under root/p1 and root/p2 (COUNTER_PASSES), the
    median over each kernel's dispatches."""
    vals = {}
    for pas in COUNTER_PASSES:
        for name, cs in _per_dispatch_counters(os.path.join(root, pas, "run_counter_collection.csv")).values():
            k = _short(name)
            if k.startswith("ssd_"):
                for c, v in cs.items():
                    vals.setdefault(k, {}).setdefault(c, []).append(v)
    lines = ["| kernel | waves | VALU / wave | MFMA / wave | LDS / wave | VMEM rd / wave | VMEM wr / wave "
             "| SALU / wave | SQ_WAIT_ANY / SQ_WAVE_CYCLES | SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS "
             "| SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals, key=lambda k: -statistics.median(vals[k]["SQ_WAVE_CYCLES"])):
        m = {c: statistics.median(v) for c, v in vals[k].items()}
        w = m["SQ_WAVES"]
        per = lambda c: f"{m[c] / w:.0f}"
        ratio = lambda a, b: "" if m[b] == 0 else f"{m[a] / m[b]:.2f}"
        lines.append(f"| {k} | {w:.0f} | {per('SQ_INSTS_VALU')} | {per('SQ_INSTS_MFMA')} | {per('SQ_INSTS_LDS')} "
                     f"| {per('SQ_INSTS_VMEM_RD')} | {per('SQ_INSTS_VMEM_WR')} | {per('SQ_INSTS_SALU')} "
                     f"| {ratio('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES')} | {ratio('SQ_LDS_BANK_CONFLICT', 'SQ_INSTS_LDS')} "
                     f"| {ratio('SQ_VALU_MFMA_BUSY_CYCLES', 'SQ_INSTS_MFMA')} |")
    print("\n".join(lines))


def _short(name):
    k = name.split("(")[0].replace("void ", "").split("<")[0].split("::")[-1]
    return k[:-len("_kernel")] if k.startswith("ssd_") and k.endswith("_kernel") else k


def summarize_profile(root, workload, short_max=SHORT_MAX):
    """Markdown summary of a kernel-trace run and two counter runs (FETCH_SIZE,
    WRITE_SIZE) of `bench.py --workload <workload> --no-cpu`, and the
    calibrated HBM bytes per launch of each libssd kernel -> traffic.json."""
    import csv
    from mamba_ssd_chunked_chunk_amd.workloads import make_workload
    prob = make_workload(workload)
    alg = algorithmic(prob, short_max)
    copy_kib = (COPY_MIB << 20) / 1024.0
    per = {}
    for which in ("fetch", "write"):
        disp = _per_dispatch(os.path.join(root, which, "run_counter_collection.csv"))
        copies = [v for (n, g, v) in disp.values() if "Mul" in n]
        cal = copy_kib / statistics.median(copies)
        per[which] = dict(cal=cal, raw={})
        for n, g, v in disp.values():
            k = _short(n)
            if k.startswith("ssd_"):
                per[which]["raw"].setdefault(k, []).append(v)
    stats = list(csv.DictReader(open(os.path.join(root, "kt", "run_kernel_stats.csv"))))
    # the calls bench.py times are the ones that follow its cache-evicting
    # read (a sum over the flush buffer); the comparison pass, later, follows
    # fills of it (fills before the first read set up inputs).  A call's
    # kernels run in order; a name seen again starts the next call.
    timed = {"read": {}, "write": {}}
    after, seen, any_read = None, set(), False
    trace = sorted(csv.DictReader(open(os.path.join(root, "kt", "run_kernel_trace.csv"))),
                   key=lambda r: int(r["Start_Timestamp"]))
    for r in trace:
        k = _short(r["Kernel_Name"])
        if "reduce_kernel" in r["Kernel_Name"]:
            after, seen, any_read = "read", set(), True
        elif "FillFunctor" in r["Kernel_Name"]:
            after, seen = ("write" if any_read else None), set()
        elif k.startswith("ssd_"):
            if k in seen:
                after = None
            seen.add(k)
            if after is not None:
                timed[after].setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        else:
            after = None

    def avg(which, k):
        v = timed[which].get(k)
        return "" if not v else f"{statistics.mean(v):.2f} ({len(v)})"
    lines = ["| kernel | calls | avg µs | min µs | max µs | avg µs, timed calls | avg µs, calls after a write "
             "flush | FETCH KiB/launch | WRITE KiB/launch | HBM MB/launch (calibrated) | algorithmic MB/launch |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    traffic = {}
    for r in stats:
        k = _short(r["Name"])
        f = w = None
        if k in per["fetch"]["raw"]:
            f = statistics.median(per["fetch"]["raw"][k])
            w = statistics.median(per["write"]["raw"][k])
            traffic[k] = round((f * per["fetch"]["cal"] + w * per["write"]["cal"]) * 1024)
        a = alg.get(k, {}).get("bytes")
        lines.append(f"| {k} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} "
                     f"| {float(r['MaxNs']) / 1e3:.2f} "
                     f"| {avg('read', k)} | {avg('write', k)} "
                     f"| {'' if f is None else f'{f:.0f}'} "
                     f"| {'' if w is None else f'{w:.0f}'} "
                     f"| {'' if k not in traffic else f'{traffic[k] / 1e6:.1f}'} "
                     f"| {'' if a is None else f'{a / 1e6:.1f}'} |")
    lines.append("")
    lines.append(f"Counter calibration on a {COPY_MIB} MiB fp32 copy kernel (dst = src * 1): "
                 f"FETCH_SIZE x {per['fetch']['cal']:.4f}, WRITE_SIZE x {per['write']['cal']:.4f}.")
    print("\n".join(lines))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(path)) if os.path.exists(path) else {}
    if d.get("sources_sha256_16") != kernel_sources_hash():
        d = {"sources_sha256_16": kernel_sources_hash()}
    d["calibration"] = {"copy_mib": COPY_MIB, "fetch": round(per["fetch"]["cal"], 5),
                        "write": round(per["write"]["cal"], 5)}
    d[workload] = traffic
    with open(path, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")


# ------------------------------------------------------------------ CPU leg

def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(prob, min_seconds, entry="inplace"):
    import oracle
    T = prob["total_len"]
    t0 = time.perf_counter()
    reps = 0
    while True:
        if entry == "inplace":
            oracle.recurrence(prob, want_pool=False, want_final=False)
        else:
            oracle.recurrence_separate(prob, None)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    # the oracle runs one OpenMP thread per (sequence, head) pair at a time
    pairs = prob["batch"] * prob["nheads"]
    return dict(value=round(reps * T / el, 1), unit="tokens/s", cores=min(oracle.num_threads(), pairs),
                kind="oracle", cpu=cpu_model(), host_cpus=len(os.sched_getaffinity(0)),
                sample=f"whole workload ({T} tokens, all heads), fp64 per-token recurrence, "
                       f"{reps} run(s) in {el:.1f} s")


# -------------------------------------------------------------------- main

# the five workloads the scan is measured on: the tiny case, the two
# 16-head / dstate-256 workloads, the ragged 128-head batch and the batch of
# short sequences; the headline is the 4 x 4096 one
PER_CONFIG = ["tiny_1x512_h4_n64", "fixed_4x4096_h16_n256", "long_8x16384_h16_n256",
              "ragged_32_h128_g8_n128", "short_512_h128_g8_n128"]


def launches_short_path(prob, short_max):
    """Whether the library launches the short path's kernels for this call:
    some sequence may take it (dstate <= 128, the path on, and not a single
    sequence longer than the limit)."""
    limit = SHORT_MAX if short_max < 0 else short_max
    if prob["dstate"] > 128 or limit == 0:
        return False
    return not (len(prob["query_start_loc"]) == 2 and prob["total_len"] > limit)


class CacheFlush:
    """A 512 MiB buffer, twice the memory-side cache, passed through before
    each timed call so that the call's inputs come from HBM.  read() sums it:
    every line the call touches is evicted and the caches hold only clean
    lines.  write(k) fills it, which also evicts the inputs but leaves up to
    the whole memory-side cache dirty with the buffer, and the timed call then
    pays for writing that back: the flush's cost, not the call's."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.buf.fill_(1)
        self.words = self.buf.view(torch.int64)
        self.out = torch.empty((), dtype=torch.int64, device=dev)
        self.torch = torch

    def read(self):
        self.torch.sum(self.words, dim=0, out=self.out)

    def write(self, k):
        self.buf.fill_(k & 0xFF)


class Runner:
    """One uploaded problem and the library calls that time it."""

    def __init__(self, torch, lib, hip, dev, prob, short_max, entry="inplace"):
        import numpy as np

        from mamba_ssd_chunked_chunk_amd import binding, torch_io
        self.torch, self.lib, self.hip, self.prob = torch, lib, hip, prob
        self.short_max = short_max
        d = torch_io.upload(prob, dev)
        self.d = d
        self.ps = torch_io.problem_struct(d, short_path_max=short_max)
        self.ws = torch.empty(binding.ssd_workspace_size(self.ps), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.nk = lib.ssd_kernel_count()
        knames = [lib.ssd_kernel_name(i).decode() for i in range(self.nk)]
        # the short path's kernels (the last two) are not launched where no
        # sequence can take it (dstate above 128, the path off, or one sequence
        # longer than its limit): their events are then only markers on the
        # stream, left out of the call time and the list
        assert knames[-2:] == ["ssd_short", "ssd_recur"]
        n_run = self.nk if launches_short_path(prob, short_max) else self.nk - 2
        self.n_run = n_run
        self.knames_run = knames[:n_run]

        def P(t):
            return None if t is None else ctypes.c_void_p(t.data_ptr())

        tail = [P(self.ws), ctypes.c_size_t(self.ws.numel()), ctypes.c_void_p(self.stream.cuda_stream)]
        if entry == "inplace":
            self.args = [P(d["y"]), P(d["x"]), P(d["dt"]), P(d["A"]), P(d["B"]), P(d["C"]), P(d["D"]),
                         P(d["dt_bias"]), P(d["pool"]), P(d["query_start_loc"]), P(d["has_initial_state"]),
                         P(d["cache_indices"])] + tail
            self.f_plain, self.f_prof = (lib.ssd_chunk_scan_varlen_fwd_inplace,
                                         lib.ssd_chunk_scan_varlen_fwd_inplace_profiled)
        else:
            # the same sequences' initial states as rows of their own tensor
            init_t = None
            hi = prob.get("has_initial_state")
            if hi is not None and np.any(hi):
                rows = d["pool"].index_select(0, d["cache_indices"].long())
                init_t = torch.where(d["has_initial_state"].bool()[:, None, None, None], rows,
                                     torch.zeros_like(rows)).contiguous()
            self.final_t = torch.empty((prob["batch"],) + tuple(d["pool"].shape[1:]), dtype=d["pool"].dtype,
                                       device=dev)
            self.init_t = init_t
            self.args = [P(d["y"]), P(d["x"]), P(d["dt"]), P(d["A"]), P(d["B"]), P(d["C"]), P(d["D"]),
                         P(d["dt_bias"]), P(init_t), P(self.final_t), P(d["query_start_loc"])] + tail
            self.f_plain, self.f_prof = lib.ssd_chunk_scan_varlen_fwd, lib.ssd_chunk_scan_varlen_fwd_profiled

    def call(self, events=None):
        if events is None:
            st = self.f_plain(ctypes.byref(self.ps), *self.args)
        else:
            arr = (ctypes.c_void_p * (self.nk + 1))(*[e.value for e in events])
            st = self.f_prof(ctypes.byref(self.ps), *self.args, arr, self.nk + 1)
        if st != 0:
            raise RuntimeError(self.lib.ssd_status_string(st).decode())

    def measure(self, steps, warmup, flush, warm=True, write_flush=False):
        """warmup untimed calls, then steps calls each preceded by a cache
        eviction (untimed) and bracketed by the kernels' own events.  The
        eviction reads a 512 MiB buffer; with write_flush it writes it (see
        CacheFlush)."""
        import numpy as np
        torch, hip = self.torch, self.hip
        ev_sets = [[hip.event() for _ in range(self.nk + 1)] for _ in range(steps)]
        for _ in range(warmup):
            self.call()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for k in range(steps):
            if write_flush:
                flush.write(k)
            else:
                flush.read()
            self.call(ev_sets[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per_call, per_kernel = [], {n: [] for n in self.knames_run}
        for evs in ev_sets:
            per_call.append(hip.elapsed_ms(evs[0], evs[self.n_run]))
            for i, n in enumerate(self.knames_run):
                per_kernel[n].append(hip.elapsed_ms(evs[i], evs[i + 1]))
        ms = statistics.fmean(per_call)
        out = dict(ms=ms, wall=wall, kern_us={n: statistics.fmean(v) * 1e3 for n, v in per_kernel.items()},
                   us_per_call={"mean": round(ms * 1e3, 2), "median": round(statistics.median(per_call) * 1e3, 2),
                                "p10": round(float(np.percentile(per_call, 10)) * 1e3, 2),
                                "p90": round(float(np.percentile(per_call, 90)) * 1e3, 2)})
        if warm:  # back-to-back, caches not evicted, for reference
            w0, w1 = hip.event(), hip.event()
            hip.lib.hipEventRecord(w0, ctypes.c_void_p(self.stream.cuda_stream))
            for _ in range(steps):
                self.call()
            hip.lib.hipEventRecord(w1, ctypes.c_void_p(self.stream.cuda_stream))
            hip.lib.hipEventSynchronize(w1)
            out["us_per_call"]["warm_back_to_back"] = round(hip.elapsed_ms(w0, w1) / steps * 1e3, 2)
        return out


def counted_traffic(workload, kernels, args):
    """HBM bytes per launch of each kernel from the committed counter runs,
    where they apply (they were taken with the default routing, fp32 states
    and the in-place entry point), and their sum for the whole call."""
    if args.short_max != SHORT_MAX or args.state_dtype != "f32" or args.entry != "inplace":
        per = {k: None for k in kernels}
    else:
        per = {k: traffic_for(k, workload) for k in kernels}
    vals = list(per.values())
    per["whole"] = sum(vals) if vals and all(v is not None for v in vals) else None
    return per


def config_line(prob, m, alg, traffic):
    """The per-workload summary: µs per call, tokens/s, the whole call and
    the longest kernel against their rooflines."""
    kern = m["kern_us"]
    dom = max(kern, key=kern.get)
    return {"tokens": prob["total_len"], "batch": prob["batch"], "us_per_call": m["us_per_call"],
            "tokens_per_s": round(prob["total_len"] / (m["ms"] * 1e-3), 1),
            "kernels_us": {n: round(v, 2) for n, v in kern.items()},
            "roofline_whole_call": roofline_entry("whole", alg, m["ms"] * 1e3, traffic["whole"]),
            "roofline_dominant_kernel": roofline_entry(dom, alg, kern[dom], traffic[dom])}


def main():
    args = parse()
    if args.short_max < 0:  # as in the library: a negative limit selects the default
        args.short_max = SHORT_MAX
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.short_max)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "libssd is a single-GPU library; this benchmark runs on exactly one "
                                   "GPU (--gpus 1); sharding over GPUs is not built."}))
        sys.exit(2)

    import torch

    from mamba_ssd_chunked_chunk_amd import binding
    from mamba_ssd_chunked_chunk_amd.workloads import make_workload, with_bf16_states

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = binding.load_library()
    hip = Hip()
    flush = CacheFlush(torch, dev)

    def load(name):
        p = make_workload(name)
        return with_bf16_states(p) if args.state_dtype == "bf16" else p

    prob = load(args.workload)
    T = prob["total_len"]
    run = Runner(torch, lib, hip, dev, prob, args.short_max, args.entry)
    m = run.measure(args.steps, args.warmup, flush)
    ms, kern_us = m["ms"], m["kern_us"]
    # the same calls after a flush that writes its buffer, for comparison
    mw = run.measure(args.steps, 2, flush, warm=False, write_flush=True)
    m["us_per_call"]["mean_after_write_flush"] = mw["us_per_call"]["mean"]

    copy_gbs = copy_probe(torch, dev, hip, run.stream)

    alg = algorithmic(prob, args.short_max)
    dom = max(kern_us, key=kern_us.get)
    traffic = counted_traffic(args.workload, run.knames_run, args)
    roof = roofline_entry(dom, alg, kern_us[dom], traffic[dom])
    whole = roofline_entry("whole", alg, ms * 1e3, traffic["whole"])
    per_kernel_roof = {n: roofline_entry(n, alg, kern_us[n]) for n in run.knames_run if alg[n]["bytes"] or alg[n]["flops"]}

    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": prob["batch"], "seq_len": prob["seqlens"][0]
                   if len(set(prob["seqlens"])) == 1 else None, "tokens": T, "nheads": prob["nheads"],
                   "head_dim": prob["head_dim"], "ngroups": prob["ngroups"], "dstate": prob["dstate"],
                   "chunk_size": CHUNK, "parallelism": "single-gpu",
                   **({} if args.entry == "inplace" else {"entry": "separate initial/final states"}),
                   **({} if args.short_max == SHORT_MAX else {"short_path_max": args.short_max}),
                   **({} if args.state_dtype == "f32" else {"state_dtype": "bf16 (storage)"})},
        "us_per_call": m["us_per_call"],
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "roofline": roof,
        "roofline_whole_call": whole,
        "roofline_per_kernel": per_kernel_roof,
        "achievable_copy_GBps": copy_gbs,
        "wall_s_timed_region": round(m["wall"], 3),
    }
    del run
    if not args.no_per_config:
        per = {}
        for name in PER_CONFIG:
            p = prob if name == args.workload else load(name)
            if name == args.workload:
                pm = m
            else:
                r = Runner(torch, lib, hip, dev, p, args.short_max, args.entry)
                pm = r.measure(args.config_steps, 2, flush, warm=False)
                del r
                torch.cuda.empty_cache()
            per[name] = config_line(p, pm, algorithmic(p, args.short_max),
                                    counted_traffic(name, list(pm["kern_us"]), args))
        out["per_config"] = per
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(prob, args.cpu_seconds, args.entry)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
