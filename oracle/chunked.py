"""fp64 NumPy oracle of the chunked (segment-sum) formulation of the SSD scan.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.  Shares no code
with the GPU path.

Sources:
  * "Mamba chunk scan with segsum" (kernelindex.com, operation 043),
    description paragraph: the sequence is cut into chunks; inside a chunk a
    segment sum of the log-decays gives an attention-like causal block (the
    diagonal part); a state recurrence with exponential decay carries
    information from chunk to chunk (the off-diagonal part); the output is
    the sum of both.
  * "mamba2_ssd_scan" (Modular MAX kernels docs), summary paragraph: the
    chunked scan is a reformulation of the per-token linear recurrence and
    gives the same numbers up to rounding; section "Per-token recurrence"
    gives the recurrence itself.

Derivation used here (by unrolling the recurrence inside one chunk that
starts with state h_prev, with a_k = A * dts_k and cs_i = sum_{k<=i} a_k):

    h_i = exp(cs_i) h_prev + sum_{j<=i} exp(cs_i - cs_j) dts_j  x_j (outer) B_j
    y_i = C_i . h_i + D x_i
        = exp(cs_i) (C_i . h_prev)                      (off-diagonal part)
          + sum_{j<=i} (C_i . B_j) exp(cs_i - cs_j) dts_j x_j   (diagonal part)
          + D x_i
    state handed to the next chunk:
        h_next = exp(cs_last) h_prev + sum_j exp(cs_last - cs_j) dts_j x_j (outer) B_j

The function returns y, the final states and, per chunk, the intermediates
(dts, cs, the chunk's own state contribution S_c and the state entering the
chunk h_in) so a GPU pipeline that materialises them can be compared step by
step.  Chunks never straddle a sequence boundary: each sequence is cut on its
own, from its first token.

This implementation is meant for small inputs (it is pure NumPy with Python
loops over sequences, heads and chunks).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def softplus(v: np.ndarray) -> np.ndarray:
    """log(1 + e^v), evaluated without overflow."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def chunked_scan(prob: dict, chunk_size: int, *, keep_intermediates: bool = False):
    """Chunked SSD forward over a varlen batch, in float64.

    ``prob`` holds the problem in the boundary's dtypes (the keys of
    ``workloads.make_problem``): x, B, C as bf16 bit patterns, dt, A, D,
    dt_bias, pool as float32, query_start_loc int32, has_initial_state uint8
    (or None), cache_indices uint32, dt_softplus bool, and the sizes.

    Returns a dict with ``y`` [T,H,P], ``final`` [batch,H,P,N] (float64) and,
    when ``keep_intermediates``, ``chunks``: a list of per-chunk records
    (b, t0, length, h, dts, cs, S, h_in).
    """
    if chunk_size < 1:
        raise ValueError("chunk_size must be >= 1")
    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    qsl = np.asarray(prob["query_start_loc"], dtype=np.int64)
    batch = len(qsl) - 1
    T = int(qsl[-1]) if batch > 0 else 0
    x = bf16_bits_to_f64(prob["x"]).reshape(T, H, P)
    Bm = bf16_bits_to_f64(prob["B"]).reshape(T, G, N)
    Cm = bf16_bits_to_f64(prob["C"]).reshape(T, G, N)
    dt = np.asarray(prob["dt"], dtype=np.float64).reshape(T, H)
    A = np.asarray(prob["A"], dtype=np.float64)
    D = np.zeros(H) if prob.get("D") is None else np.asarray(prob["D"], np.float64)
    bias = np.zeros(H) if prob.get("dt_bias") is None else np.asarray(prob["dt_bias"], np.float64)
    pool = np.asarray(prob["pool"], dtype=np.float32)
    has_init = prob.get("has_initial_state")
    ci = np.asarray(prob["cache_indices"], dtype=np.int64)
    use_softplus = bool(prob.get("dt_softplus", True))
    hpg = H // G

    y = np.zeros((T, H, P))
    final = np.zeros((batch, H, P, N))
    chunks = []
    for b in range(batch):
        s, e = int(qsl[b]), int(qsl[b + 1])
        init = has_init is not None and bool(has_init[b])
        for h in range(H):
            g = h // hpg
            state = pool[ci[b], h].astype(np.float64) if init else np.zeros((P, N))
            for t0 in range(s, e, chunk_size):
                t1 = min(t0 + chunk_size, e)
                v = dt[t0:t1, h] + bias[h]
                dts = softplus(v) if use_softplus else v
                cs = np.cumsum(A[h] * dts)
                X = x[t0:t1, h, :]
                Bc = Bm[t0:t1, g, :]
                Cc = Cm[t0:t1, g, :]
                l = t1 - t0
                causal = np.tril(np.ones((l, l), dtype=bool))
                seg = np.where(causal, cs[:, None] - cs[None, :], -np.inf)
                decay = np.exp(seg)
                y_diag = ((Cc @ Bc.T) * decay * dts[None, :]) @ X
                y_off = np.exp(cs)[:, None] * (Cc @ state.T)
                y[t0:t1, h, :] = y_diag + y_off + D[h] * X
                S = (X * (np.exp(cs[-1] - cs) * dts)[:, None]).T @ Bc
                if keep_intermediates:
                    chunks.append(dict(b=b, t0=t0, length=l, h=h, dts=dts.copy(),
                                       cs=cs.copy(), S=S.copy(), h_in=state.copy()))
                state = np.exp(cs[-1]) * state + S
            final[b, h] = state
    out = dict(y=y, final=final)
    if keep_intermediates:
        out["chunks"] = chunks
    return out
