"""Helpers shared by the tests: building problems from explicit values and
comparing results.  No arithmetic of the scan lives here."""

from __future__ import annotations

import copy

import numpy as np

from mamba_ssd_chunked_chunk_amd.workloads import (bf16_bits_to_f32, f32_to_bf16_bits,
                                                    make_problem)


def bf16(a) -> np.ndarray:
    """float values -> bf16 bit patterns (values must already be bf16-exact
    for exact tests; otherwise they are rounded to nearest even)."""
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def small_problem(seqlens, H=2, P=4, G=1, N=8, max_slots=None, seed=1, **kw):
    if max_slots is None:
        max_slots = max(1, len(seqlens)) + 2
    return make_problem(seqlens, nheads=H, head_dim=P, ngroups=G, dstate=N,
                        max_slots=max_slots, seed=seed, **kw)


def clone(prob: dict) -> dict:
    return copy.deepcopy(prob)


def sub_batch(prob: dict, seqs) -> dict:
    """The problem restricted to the listed sequences (in that order),
    sharing the pool and cache slots."""
    qsl = prob["query_start_loc"]
    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    T = int(qsl[-1])
    x = prob["x"].reshape(T, H, P)
    dt = prob["dt"].reshape(T, H)
    Bm = prob["B"].reshape(T, G, N)
    Cm = prob["C"].reshape(T, G, N)
    rows = np.concatenate([np.arange(qsl[b], qsl[b + 1]) for b in seqs]) if len(seqs) else np.zeros(0, int)
    lens = [int(qsl[b + 1] - qsl[b]) for b in seqs]
    out = clone(prob)
    out["x"] = np.ascontiguousarray(x[rows])
    out["dt"] = np.ascontiguousarray(dt[rows])
    out["B"] = np.ascontiguousarray(Bm[rows])
    out["C"] = np.ascontiguousarray(Cm[rows])
    out["seqlens"] = lens
    out["batch"] = len(seqs)
    q = np.zeros(len(seqs) + 1, dtype=np.int32)
    q[1:] = np.cumsum(lens)
    out["query_start_loc"] = q
    out["total_len"] = int(q[-1])
    if prob.get("has_initial_state") is not None:
        out["has_initial_state"] = np.ascontiguousarray(prob["has_initial_state"][list(seqs)])
    out["cache_indices"] = np.ascontiguousarray(prob["cache_indices"][list(seqs)])
    return out


def max_rel(a, b) -> float:
    """max |a-b| / max(|b|) (0 when both are zero)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.max(np.abs(b)) if b.size else 0.0
    diff = np.max(np.abs(a - b)) if a.size else 0.0
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def frob_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    nd = np.linalg.norm(a - b)
    return float(nd if nb == 0 else nd / nb)


def pad_by_hand(prob):
    """The same problem at the kernels' sizes, built on the host: head_dim
    rounded up to 64 m and split into m heads of 64 per head (dt, A, D,
    dt_bias repeated), dstate rounded up to 64 / 128 / 256; zeros in every
    added channel and column (x, B, C and the pool)."""
    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    T = int(prob["query_start_loc"][-1])
    m = (P + 63) // 64
    Np = 64 if N <= 64 else 128 if N <= 128 else 256
    q = dict(prob)
    x = np.zeros((T, H, 64 * m), np.uint16)
    x[:, :, :P] = prob["x"].reshape(T, H, P)
    q["x"] = x.reshape(T, H * m, 64)
    q["dt"] = np.repeat(prob["dt"].reshape(T, H), m, axis=1)
    for k in ("A", "D", "dt_bias"):
        if prob.get(k) is not None:
            q[k] = np.repeat(prob[k], m)
    for k in ("B", "C"):
        a = np.zeros((T, G, Np), np.uint16)
        a[:, :, :N] = prob[k].reshape(T, G, N)
        q[k] = a
    pool = prob["pool"]
    S = pool.shape[0]
    pp = np.zeros((S, H, 64 * m, Np), pool.dtype)
    pp[:, :, :P, :N] = pool
    q["pool"] = pp.reshape(S, H * m, 64, Np)
    q.update(nheads=H * m, head_dim=64, dstate=Np)
    return q
