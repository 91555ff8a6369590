"""Seeded synthetic inputs for the SSD varlen scan.

This module only draws random inputs; it holds no arithmetic of the scan
itself, so both the GPU path and the CPU oracle can consume its output.

Every problem is a dict of NumPy arrays in the dtypes the C ABI takes:
x, B, C as bf16 bit patterns (uint16, rounded to nearest even from a float32
draw), dt, A, D, dt_bias and the state pool as float32,
query_start_loc int32, has_initial_state uint8 (or None), cache_indices
uint32, plus the sizes and the dt_softplus flag.

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per problem):
  1. sequence lengths (workload-specific recipe)
  2. A[h]       = -exp(U(0, ln 16))
  3. dt_bias[h] = u + log(-expm1(-u)),  u ~ U(1e-3, 1e-1)   (inverse softplus)
  4. D[h]       ~ N(0, 1)
  5. dt[t,h]    ~ N(0, 0.5)     (0.5 is the standard deviation)
  6. x[t,h,p]   ~ N(0, 1) -> bf16
  7. B[t,g,n]   ~ N(0, 1) -> bf16
  8. C[t,g,n]   ~ N(0, 1) -> bf16
  9. cache_indices = first `batch` entries of a permutation of the slots
 10. has_initial_state (workload-specific)
 11. pool: zeros, or N(0, pool_std) for every slot
The named workloads follow the shapes of the pages' benchmark (16 heads x
head_dim 64, one group, dstate 256, chunk 256) and of a ragged mixer-style
prefill; their seeds are 20260000 + index.
"""

from __future__ import annotations

import math

import numpy as np

CHUNK = 256


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_in.size, step):
        u = flat_in[i:i + step].astype(np.uint64)
        u += ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
        flat_out[i:i + step] = (u >> np.uint64(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng, shape, std=1.0):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def make_problem(seqlens, *, nheads, head_dim, ngroups, dstate, max_slots, seed,
                 init="none", pool_std=0.1, dt_softplus=True, with_D=True,
                 with_dt_bias=True, with_has_init=True, name="custom", state_dtype="f32"):
    """Draw a problem.

    ``seqlens``: list of ints, or a callable rng -> list (drawn first).
    ``init``: "none" (has_initial_state all 0, pool zeros), "all",
    "half" (exactly half the sequences, chosen by a permutation),
    "bernoulli" (p = 0.5 each), or an explicit 0/1 list.
    ``state_dtype``: "f32", or "bf16" for a pool stored as bf16 (the same
    draw, rounded to bf16 bit patterns; see ``with_bf16_states``).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = seqlens(rng) if callable(seqlens) else list(seqlens)
    lens = [int(v) for v in lens]
    batch = len(lens)
    H, P, G, N = nheads, head_dim, ngroups, dstate
    qsl = np.zeros(batch + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens, dtype=np.int64).astype(np.int32)
    T = int(qsl[-1])

    A = (-np.exp(rng.uniform(0.0, math.log(16.0), H))).astype(np.float32)
    u = rng.uniform(1e-3, 1e-1, H)
    dt_bias = (u + np.log(-np.expm1(-u))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    dt = (rng.standard_normal((T, H), dtype=np.float32) * np.float32(0.5))
    x = _normal_bf16(rng, (T, H, P))
    B = _normal_bf16(rng, (T, G, N))
    C = _normal_bf16(rng, (T, G, N))
    if batch > max_slots:
        raise ValueError("more sequences than pool slots")
    ci = rng.permutation(max_slots)[:batch].astype(np.uint32)

    if isinstance(init, str):
        if init == "none":
            hi = np.zeros(batch, dtype=np.uint8)
        elif init == "all":
            hi = np.ones(batch, dtype=np.uint8)
        elif init == "half":
            hi = np.zeros(batch, dtype=np.uint8)
            hi[rng.permutation(batch)[:batch // 2]] = 1
        elif init == "bernoulli":
            hi = (rng.uniform(size=batch) < 0.5).astype(np.uint8)
        else:
            raise ValueError(init)
    else:
        hi = np.asarray(init, dtype=np.uint8)
    if init == "none":
        pool = np.zeros((max_slots, H, P, N), dtype=np.float32)
    else:
        pool = np.empty((max_slots, H, P, N), dtype=np.float32)
        for s in range(max_slots):
            pool[s] = rng.standard_normal((H, P, N), dtype=np.float32) * np.float32(pool_std)

    out = dict(
        name=name, seqlens=lens, total_len=T, batch=batch,
        nheads=H, head_dim=P, ngroups=G, dstate=N, chunk_size=CHUNK,
        max_slots=max_slots, dt_softplus=bool(dt_softplus),
        query_start_loc=qsl, x=x, dt=dt, A=A, B=B, C=C,
        D=D if with_D else None, dt_bias=dt_bias if with_dt_bias else None,
        pool=pool, has_initial_state=hi if with_has_init else None,
        cache_indices=ci, seed=seed, state_dtype="f32")
    return with_bf16_states(out) if state_dtype == "bf16" else out


def with_bf16_states(prob: dict) -> dict:
    """The problem with its pool stored as bf16 (uint16 bit patterns,
    rounded to nearest even from the fp32 draw); everything else shared."""
    if prob.get("state_dtype", "f32") == "bf16":
        return prob
    q = dict(prob)
    q["pool"] = f32_to_bf16_bits(prob["pool"])
    q["state_dtype"] = "bf16"
    return q


def _loguniform_lengths(rng):
    return [int(round(math.exp(v))) for v in rng.uniform(math.log(17.0), math.log(8192.0), 32)]


def _uniform_short_lengths(rng):
    return [int(v) for v in rng.integers(1, 97, size=512)]


WORKLOADS = {
    # 1 x 512 tokens, 4 heads, dstate 64: the small case.
    "tiny_1x512_h4_n64": dict(
        seqlens=[512], nheads=4, head_dim=64, ngroups=1, dstate=64, max_slots=1,
        init="none", seed=20260000),
    # 4 x 4096 tokens, 16 heads x 64, one group, dstate 256, zero initial states.
    "fixed_4x4096_h16_n256": dict(
        seqlens=[4096] * 4, nheads=16, head_dim=64, ngroups=1, dstate=256, max_slots=8,
        init="none", seed=20260001),
    # 8 x 16384 tokens, same head shape, half the sequences resume from the pool.
    "long_8x16384_h16_n256": dict(
        seqlens=[16384] * 8, nheads=16, head_dim=64, ngroups=1, dstate=256, max_slots=16,
        init="half", pool_std=0.1, seed=20260002),
    # 32 ragged sequences (log-uniform in [17, 8192]), 128 heads in 8 groups, dstate 128.
    "ragged_32_h128_g8_n128": dict(
        seqlens=_loguniform_lengths, nheads=128, head_dim=64, ngroups=8, dstate=128,
        max_slots=64, init="bernoulli", pool_std=0.1, seed=20260003),
    # 512 short sequences (1..96 tokens), all resuming from a 1024-slot pool.
    "short_512_h128_g8_n128": dict(
        seqlens=_uniform_short_lengths, nheads=128, head_dim=64, ngroups=8, dstate=128,
        max_slots=1024, init="all", pool_std=0.1, seed=20260004),
    # one decode step: 512 sequences of one token each, same head shape, all
    # resuming from a 1024-slot pool.
    "decode_512_h128_g8_n128": dict(
        seqlens=[1] * 512, nheads=128, head_dim=64, ngroups=8, dstate=128,
        max_slots=1024, init="all", pool_std=0.1, seed=20260005),
}

WORKLOAD_ORDER = list(WORKLOADS)


def make_workload(name: str, **overrides) -> dict:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    seqlens = spec.pop("seqlens")
    return make_problem(seqlens, name=name, **spec)
