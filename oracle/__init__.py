"""CPU oracle of the Mamba-2 SSD varlen scan (fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
GPU library (``mamba_ssd_chunked_chunk_amd``) never imports it, and the two
share no code; both only consume the seeded inputs produced by
``mamba_ssd_chunked_chunk_amd.workloads`` (which holds no arithmetic of the
method).

Two independent formulations:
  * ``recurrence``: the per-token recurrence in C, fp64, OpenMP over
    (sequence, head) -- the plain definition ("mamba2_ssd_scan", section
    "Per-token recurrence"; in-place pool semantics from
    "Mamba2SSDChunkScanVarlenFwdInplace").  ``recurrence_separate`` is the
    same recurrence with separate initial and final states (the paragraph
    after "Per-token recurrence").
  * ``chunked_scan`` (``oracle.chunked``): the segment-sum / chunked
    reformulation in NumPy fp64 ("Mamba chunk scan with segsum",
    description), with per-chunk intermediates.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, special cases and a hand-worked example
(``tests/golden/``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .chunked import bf16_bits_to_f64, chunked_scan, softplus  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_recurrence.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            lib.ssd_oracle_recurrence.restype = ctypes.c_int
            lib.ssd_oracle_recurrence.argtypes = [
                ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P]
            lib.ssd_oracle_softplus.restype = ctypes.c_double
            lib.ssd_oracle_softplus.argtypes = [ctypes.c_double]
            lib.ssd_oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the OpenMP runtime of the C oracle will use."""
    return _load().ssd_oracle_num_threads()


def softplus_c(v: float) -> float:
    """The C oracle's softplus (exposed for its pin)."""
    return _load().ssd_oracle_softplus(float(v))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(prob: dict, *, seqs: tuple[int, int] | None = None,
               want_pool: bool = True, want_final: bool = True):
    """Run the fp64 per-token recurrence on a problem dict.

    Returns dict(y=[T,H,P] f64, final=[batch,H,P,N] f64 or None,
    pool=[S,H,P,N] f32 or None).  ``seqs=(lo, hi)`` restricts the work to
    sequences lo..hi-1 (rows of other sequences in ``y`` stay zero and the
    returned pool only has those sequences' slots written).
    """
    lib = _load()
    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    qsl = np.ascontiguousarray(prob["query_start_loc"], dtype=np.int32)
    batch = len(qsl) - 1
    T = int(qsl[-1]) if batch > 0 else 0
    x = np.ascontiguousarray(prob["x"], dtype=np.uint16)
    Bm = np.ascontiguousarray(prob["B"], dtype=np.uint16)
    Cm = np.ascontiguousarray(prob["C"], dtype=np.uint16)
    dt = np.ascontiguousarray(prob["dt"], dtype=np.float32)
    A = np.ascontiguousarray(prob["A"], dtype=np.float32)
    D = None if prob.get("D") is None else np.ascontiguousarray(prob["D"], dtype=np.float32)
    bias = None if prob.get("dt_bias") is None else np.ascontiguousarray(prob["dt_bias"], dtype=np.float32)
    pool = prob["pool"]
    if prob.get("state_dtype", "f32") == "bf16":  # bf16 bit patterns: their exact values
        pool = (np.ascontiguousarray(pool, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    pool = np.ascontiguousarray(pool, dtype=np.float32)
    max_slots = pool.shape[0]
    hi = prob.get("has_initial_state")
    hi = None if hi is None else np.ascontiguousarray(hi, dtype=np.uint8)
    ci = np.ascontiguousarray(prob["cache_indices"], dtype=np.uint32)
    assert x.size == T * H * P and Bm.size == T * G * N and Cm.size == T * G * N
    assert dt.size == T * H and pool.size == max_slots * H * P * N
    lo, hi_s = (0, batch) if seqs is None else seqs
    y = np.zeros((T, H, P), dtype=np.float64)
    final = np.zeros((batch, H, P, N), dtype=np.float64) if want_final else None
    pool_out = np.empty_like(pool) if want_pool else None
    rc = lib.ssd_oracle_recurrence(
        T, batch, H, P, G, N, max_slots, 1 if prob.get("dt_softplus", True) else 0,
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(bias), _ptr(pool),
        _ptr(qsl), _ptr(hi), _ptr(ci), lo, hi_s, _ptr(y), _ptr(final), _ptr(pool_out))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return dict(y=y, final=final, pool=pool_out)


def recurrence_separate(prob: dict, initial_states=None, *, seqs: tuple[int, int] | None = None):
    """The operation with separate initial and final states ("mamba2_ssd_scan",
    the paragraph after "Per-token recurrence": the state resets to zero, or
    to initial_states, at each query_start_loc boundary, and final_states
    (batch, nheads, head_dim, dstate) is written at each sequence end).

    Sequence b starts from ``initial_states[b]`` (fp32 [batch,H,P,N]) when it
    is given, else from zero; the problem's pool, has_initial_state and
    cache_indices are ignored.  It runs ``recurrence`` with the initial states
    as a pool of one slot per sequence, every sequence flagged.  Returns
    dict(y=[T,H,P] f64, final=[batch,H,P,N] f64).
    """
    H, P, N = prob["nheads"], prob["head_dim"], prob["dstate"]
    batch = len(prob["query_start_loc"]) - 1
    q = dict(prob)
    if initial_states is None:
        q["pool"] = np.zeros((1, H, P, N), np.float32)
        q["has_initial_state"] = None
        q["cache_indices"] = np.zeros(batch, np.uint32)
    else:
        q["pool"] = np.ascontiguousarray(initial_states, dtype=np.float32).reshape(batch, H, P, N)
        q["has_initial_state"] = np.ones(batch, np.uint8)
        q["cache_indices"] = np.arange(batch, dtype=np.uint32)
    r = recurrence(q, seqs=seqs, want_pool=False, want_final=True)
    return dict(y=r["y"], final=r["final"])
