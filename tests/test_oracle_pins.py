"""Pins of the CPU oracle (both formulations) to facts fixed by the pages and
by the mathematics, independent of the oracle's own code.

The pages ("mamba2_ssd_scan", section "Per-token recurrence";
"Mamba2SSDChunkScanVarlenFwdInplace", description and tensor shapes;
"Mamba chunk scan with segsum", description) print no worked example and no
values, so the pins are closed forms, special cases that reduce to textbook
results, invariants the pages state (no cross-sequence bleed, the chunked
form equals the recurrence, the pool carries a sequence's state across
calls) and one example worked by hand (tests/golden/).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.chunked import chunked_scan, softplus
from ssd_testlib import bf16, bf16_to_f64, clone, frob_rel, max_rel, pad_by_hand, small_problem, sub_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- softplus

@pytest.mark.parametrize("sp", [softplus, oracle.softplus_c], ids=["numpy", "c"])
def test_softplus_identities(sp):
    f = (lambda v: float(sp(np.float64(v)))) if sp is softplus else sp
    assert f(0.0) == pytest.approx(math.log(2.0), rel=1e-15, abs=0)
    for v in [-30.0, -3.0, -0.1, 0.7, 5.0, 40.0]:
        # softplus(v) - softplus(-v) = v  and  softplus(ln(e^k - 1)) = k
        assert f(v) - f(-v) == pytest.approx(v, rel=1e-13, abs=1e-13)
    for k in [1e-3, 0.5, 2.0, 10.0]:
        assert f(math.log(math.expm1(k))) == pytest.approx(k, rel=1e-12)
    assert f(800.0) == 800.0            # no overflow for large arguments
    assert f(-800.0) == 0.0 or f(-800.0) < 1e-300
    assert f(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)


# ------------------------------------------------------- hand-worked example

def _golden_problem(spec):
    H, P, G, N = spec["nheads"], spec["head_dim"], spec["ngroups"], spec["dstate"]
    T = len(spec["dt"])
    pool = np.zeros((spec["max_slots"], H, P, N), np.float32)
    pool[1, 0, 0, :] = spec["pool_slot1"]
    pool[0] = np.float32(7.5)       # must stay untouched
    return dict(nheads=H, head_dim=P, ngroups=G, dstate=N, max_slots=spec["max_slots"],
                dt_softplus=spec["dt_softplus"],
                A=np.array(spec["A"], np.float32), dt_bias=np.array(spec["dt_bias"], np.float32),
                D=np.array(spec["D"], np.float32),
                dt=np.array(spec["dt"], np.float32).reshape(T, H),
                x=bf16(np.array(spec["x"]).reshape(T, H, P)),
                B=bf16(np.array(spec["B"]).reshape(T, G, N)),
                C=bf16(np.array(spec["C"]).reshape(T, G, N)),
                query_start_loc=np.array(spec["query_start_loc"], np.int32),
                has_initial_state=np.array(spec["has_initial_state"], np.uint8),
                cache_indices=np.array(spec["cache_indices"], np.uint32), pool=pool)


def test_golden_hand_example():
    with open(os.path.join(GOLDEN, "hand_3token_n2.json")) as f:
        fx = json.load(f)
    prob = _golden_problem(fx["problem"])
    exp_y = np.array(fx["expected"]["y"])
    exp_final = np.array(fx["expected"]["final"])
    out = oracle.recurrence(prob)
    np.testing.assert_allclose(out["y"].reshape(-1), exp_y, rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(out["final"].reshape(-1), exp_final, rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(out["pool"][1].reshape(-1), exp_final, rtol=1e-7)
    assert np.array_equal(out["pool"][0].view(np.uint32), prob["pool"][0].view(np.uint32))
    for L in (1, 2, 3):
        ch = chunked_scan(prob, L)
        np.testing.assert_allclose(ch["y"].reshape(-1), exp_y, rtol=1e-7, atol=1e-7)
        np.testing.assert_allclose(ch["final"].reshape(-1), exp_final, rtol=1e-7, atol=1e-7)


# ------------------------------------- chunked formulation == recurrence

MIXED_LENS = [300, 1, 0, 77, 520, 256]


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64, 256, 512])
@pytest.mark.parametrize("dt_softplus", [True, False])
def test_chunked_equals_recurrence(chunk, dt_softplus):
    prob = small_problem(MIXED_LENS, H=4, P=4, G=2, N=8, seed=11, init="bernoulli",
                         dt_softplus=dt_softplus)
    if not dt_softplus:
        # keep dts = dt + dt_bias positive so the decays stay below one
        prob["dt"] = np.abs(prob["dt"]) * np.float32(0.2)
        prob["dt_bias"] = np.full_like(prob["dt_bias"], 0.01)
    rec = oracle.recurrence(prob)
    ch = chunked_scan(prob, chunk)
    assert max_rel(ch["y"], rec["y"]) <= 1e-10
    assert max_rel(ch["final"], rec["final"]) <= 1e-10


@pytest.mark.parametrize("chunk", [1, 16, 256])
@pytest.mark.parametrize("case", ["positive_A", "negative_dts"])
def test_chunked_equals_recurrence_when_states_grow(chunk, case):
    """A * dts > 0 (a positive A, or negative dts without softplus): the state
    grows, and the chunked form still equals the recurrence (the segment-sum
    reformulation holds for any sign of the exponent)."""
    prob = small_problem(MIXED_LENS, H=4, P=4, G=2, N=8, seed=12, init="all")
    rng = np.random.default_rng(12)
    if case == "positive_A":
        prob["A"] = rng.uniform(0.01, 0.05, 4).astype(np.float32)
    else:
        prob["dt_softplus"] = False
        prob["dt"] = rng.uniform(-0.2, 0.05, prob["dt"].shape).astype(np.float32)
        prob["dt_bias"] = np.zeros(4, np.float32)
    rec = oracle.recurrence(prob)
    assert np.abs(rec["final"]).max() > 2.0 * np.abs(prob["pool"]).max()  # the states did grow
    ch = chunked_scan(prob, chunk)
    assert max_rel(ch["y"], rec["y"]) <= 1e-10
    assert max_rel(ch["final"], rec["final"]) <= 1e-10


@pytest.mark.parametrize("P,N", [(4, 5), (96, 100), (128, 8), (70, 3)])
def test_padding_changes_no_value(P, N):
    """What the size adapter relies on: zero columns of B and C, zero
    channels of x and zero state entries change no value of the others, and
    each 64-channel block of a head behaves as a head of its own with the
    head's dt, A, D and dt_bias.  The oracle on the hand-padded problem,
    cropped, equals the oracle on the problem itself, bit for bit."""
    prob = small_problem([50, 0, 7, 130], H=2, P=P, G=1, N=N, seed=13, init="bernoulli")
    q = pad_by_hand(prob)
    a = oracle.recurrence(prob)
    b = oracle.recurrence(q)
    T, H = prob["total_len"], prob["nheads"]
    m = q["nheads"] // H
    yb = b["y"].reshape(T, H, 64 * m)[:, :, :P]
    assert np.array_equal(a["y"].reshape(T, H, P), yb)
    fb = b["final"].reshape(-1, H, 64 * m, q["dstate"])[:, :, :P, :N]
    assert np.array_equal(a["final"].reshape(-1, H, P, N), fb)


# ------------------------------------------- A = 0: masked linear attention

def test_A_zero_is_masked_linear_attention():
    prob = small_problem([40, 13], H=2, P=3, G=1, N=5, seed=3, init="all", pool_std=0.3)
    prob["A"] = np.zeros_like(prob["A"])
    out = oracle.recurrence(prob)
    T = prob["total_len"]
    X = bf16_to_f64(prob["x"]).reshape(T, 2, 3)
    Bm = bf16_to_f64(prob["B"]).reshape(T, 5)
    Cm = bf16_to_f64(prob["C"]).reshape(T, 5)
    dts = softplus(prob["dt"].astype(np.float64) + prob["dt_bias"].astype(np.float64)[None, :])
    for b in range(2):
        s, e = prob["query_start_loc"][b], prob["query_start_loc"][b + 1]
        for h in range(2):
            h0 = prob["pool"][prob["cache_indices"][b], h].astype(np.float64)
            att = np.tril(Cm[s:e] @ Bm[s:e].T) * dts[s:e, h][None, :]
            y = att @ X[s:e, h] + (Cm[s:e] @ h0.T) + prob["D"][h] * X[s:e, h]
            np.testing.assert_allclose(out["y"][s:e, h], y, rtol=1e-11, atol=1e-11)
            fin = (X[s:e, h] * dts[s:e, h][:, None]).T @ Bm[s:e] + h0
            np.testing.assert_allclose(out["final"][b, h], fin, rtol=1e-11, atol=1e-11)


# ------------------------------- constant inputs: geometric series closed form

def test_constant_inputs_geometric_series():
    H, P, N = 2, 3, 4
    lens = [50, 7]
    prob = small_problem(lens, H=H, P=P, G=1, N=N, seed=5, init="all", pool_std=0.5)
    T = sum(lens)
    rng = np.random.default_rng(9)
    xv = bf16(rng.standard_normal((H, P)))
    bv = bf16(rng.standard_normal(N))
    cv = bf16(rng.standard_normal(N))
    prob["x"] = np.ascontiguousarray(np.broadcast_to(xv, (T, H, P)))
    prob["B"] = np.ascontiguousarray(np.broadcast_to(bv, (T, 1, N)))
    prob["C"] = np.ascontiguousarray(np.broadcast_to(cv, (T, 1, N)))
    prob["dt"] = np.ascontiguousarray(np.broadcast_to(np.float32([0.3, -0.2]), (T, H)))
    out = oracle.recurrence(prob)
    xf, bf, cf = bf16_to_f64(xv), bf16_to_f64(bv), bf16_to_f64(cv)
    for b in range(2):
        s = prob["query_start_loc"][b]
        for h in range(H):
            dts = softplus(np.float64(prob["dt"][0, h]) + np.float64(prob["dt_bias"][h]))
            r = math.exp(float(prob["A"][h]) * dts)
            q = dts * np.outer(xf[h], bf)
            h0 = prob["pool"][prob["cache_indices"][b], h].astype(np.float64)
            for m in range(1, lens[b] + 1):
                hm = r ** m * h0 + q * (1 - r ** m) / (1 - r)
                y = hm @ cf + prob["D"][h] * xf[h]
                np.testing.assert_allclose(out["y"][s + m - 1, h], y, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out["final"][b, h], hm, rtol=1e-11, atol=1e-12)


# --------------------------- scalar problem: first-order linear recurrence

def test_scalar_first_order_closed_form():
    lens = [64]
    prob = small_problem(lens, H=1, P=1, G=1, N=1, seed=21, init="all", pool_std=1.0)
    out = oracle.recurrence(prob)
    x = bf16_to_f64(prob["x"]).reshape(-1)
    Bv = bf16_to_f64(prob["B"]).reshape(-1)
    Cv = bf16_to_f64(prob["C"]).reshape(-1)
    dts = softplus(prob["dt"].reshape(-1).astype(np.float64) + float(prob["dt_bias"][0]))
    r = np.exp(float(prob["A"][0]) * dts)
    qv = dts * Bv * x
    h0 = float(prob["pool"][prob["cache_indices"][0]].reshape(-1)[0])
    for t in range(64):
        # h_t = (prod_{k<=t} r_k) h0 + sum_{j<=t} (prod_{j<k<=t} r_k) q_j
        ht = np.prod(r[:t + 1]) * h0 + sum(np.prod(r[j + 1:t + 1]) * qv[j] for j in range(t + 1))
        yt = Cv[t] * ht + float(prob["D"][0]) * x[t]
        assert out["y"].reshape(-1)[t] == pytest.approx(yt, rel=1e-11, abs=1e-13)
    assert out["final"].reshape(-1)[0] == pytest.approx(ht, rel=1e-11, abs=1e-13)


# -------------------------------------------- strong decay: no memory left

def test_strong_decay_forgets_everything():
    prob = small_problem([30, 5], H=2, P=3, G=1, N=6, seed=8, init="all", dt_softplus=False)
    prob["A"] = np.full(2, -1e4, np.float32)
    prob["dt"] = np.abs(prob["dt"]) + np.float32(0.2)
    prob["dt_bias"] = np.zeros(2, np.float32)
    out = oracle.recurrence(prob)
    T = prob["total_len"]
    X = bf16_to_f64(prob["x"]).reshape(T, 2, 3)
    Bm = bf16_to_f64(prob["B"]).reshape(T, 6)
    Cm = bf16_to_f64(prob["C"]).reshape(T, 6)
    dts = prob["dt"].astype(np.float64)
    for t in range(T):
        for h in range(2):
            y = dts[t, h] * (Cm[t] @ Bm[t]) * X[t, h] + prob["D"][h] * X[t, h]
            np.testing.assert_allclose(out["y"][t, h], y, rtol=1e-12, atol=1e-12)
    for b in range(2):
        last = prob["query_start_loc"][b + 1] - 1
        for h in range(2):
            np.testing.assert_allclose(out["final"][b, h], dts[last, h] * np.outer(X[last, h], Bm[last]),
                                       rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- B = 0 and C = 0

def test_B_zero_and_C_zero():
    prob = small_problem([33, 9], H=2, P=3, G=1, N=4, seed=4, init="all", pool_std=0.2)
    T = prob["total_len"]
    X = bf16_to_f64(prob["x"]).reshape(T, 2, 3)
    Dx = prob["D"].astype(np.float64)[None, :, None] * X
    pb = clone(prob)
    pb["B"] = np.zeros_like(pb["B"])
    ob = oracle.recurrence(pb)
    dts = softplus(prob["dt"].astype(np.float64) + prob["dt_bias"].astype(np.float64)[None, :])
    Cm = bf16_to_f64(prob["C"]).reshape(T, 4)
    for b in range(2):
        s, e = prob["query_start_loc"][b], prob["query_start_loc"][b + 1]
        for h in range(2):
            h0 = prob["pool"][prob["cache_indices"][b], h].astype(np.float64)
            cum = np.cumsum(prob["A"][h] * dts[s:e, h])
            # y_t = exp(A * sum_{k<=t} dts_k) C_t . h0 + D x_t ; final = exp(A sum dts) h0
            yexp = np.exp(cum)[:, None] * (Cm[s:e] @ h0.T) + Dx[s:e, h]
            np.testing.assert_allclose(ob["y"][s:e, h], yexp, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(ob["final"][b, h], math.exp(cum[-1]) * h0, rtol=1e-11, atol=1e-14)
    pc = clone(prob)
    pc["C"] = np.zeros_like(pc["C"])
    oc = oracle.recurrence(pc)
    assert np.array_equal(oc["y"], Dx)
    for L in (1, 7, 256):
        assert np.array_equal(chunked_scan(pc, L)["y"], Dx)


# -------------------------------------------------- length-1 sequence

def test_length_one_sequence_by_hand():
    prob = small_problem([1], H=1, P=3, G=1, N=4, seed=6, init="all", pool_std=0.5)
    out = oracle.recurrence(prob)
    x = bf16_to_f64(prob["x"]).reshape(3)
    Bv = bf16_to_f64(prob["B"]).reshape(4)
    Cv = bf16_to_f64(prob["C"]).reshape(4)
    dts = softplus(np.float64(prob["dt"][0, 0]) + np.float64(prob["dt_bias"][0]))
    r = math.exp(float(prob["A"][0]) * dts)
    h0 = prob["pool"][prob["cache_indices"][0], 0].astype(np.float64)
    h1 = r * h0 + dts * np.outer(x, Bv)
    np.testing.assert_allclose(out["y"].reshape(3), h1 @ Cv + prob["D"][0] * x, rtol=1e-13)
    np.testing.assert_allclose(out["final"][0, 0], h1, rtol=1e-13)


# ------------------------------------- separate initial and final states

def test_separate_states_by_hand():
    # sequence 0: one token from a given initial state; sequence 1: no tokens
    # (its final state is its initial state); sequence 2: one token from zero
    # when no initial states are given
    prob = small_problem([1, 0, 1], H=1, P=3, G=1, N=4, seed=61, init="none")
    rng = np.random.default_rng(62)
    s0 = rng.standard_normal((3, 1, 3, 4)).astype(np.float32)
    x = bf16_to_f64(prob["x"]).reshape(2, 3)
    Bv = bf16_to_f64(prob["B"]).reshape(2, 4)
    Cv = bf16_to_f64(prob["C"]).reshape(2, 4)
    dts = softplus(prob["dt"].reshape(2).astype(np.float64) + np.float64(prob["dt_bias"][0]))
    r = np.exp(float(prob["A"][0]) * dts)
    D = float(prob["D"][0])
    for init in (s0, None):
        out = oracle.recurrence_separate(prob, init)
        h0a = s0[0, 0].astype(np.float64) if init is not None else np.zeros((3, 4))
        h0c = s0[2, 0].astype(np.float64) if init is not None else np.zeros((3, 4))
        ha = r[0] * h0a + dts[0] * np.outer(x[0], Bv[0])
        hc = r[1] * h0c + dts[1] * np.outer(x[1], Bv[1])
        np.testing.assert_allclose(out["y"].reshape(2, 3)[0], ha @ Cv[0] + D * x[0], rtol=1e-13)
        np.testing.assert_allclose(out["y"].reshape(2, 3)[1], hc @ Cv[1] + D * x[1], rtol=1e-13)
        np.testing.assert_allclose(out["final"][0, 0], ha, rtol=1e-13)
        np.testing.assert_allclose(out["final"][2, 0], hc, rtol=1e-13)
        want1 = s0[1, 0].astype(np.float64) if init is not None else np.zeros((3, 4))
        assert np.array_equal(out["final"][1, 0], want1)


# ----------------------------------------------- varlen: no cross-sequence bleed

def test_varlen_isolation_concat_equals_separate():
    prob = small_problem([37, 0, 129, 5, 64], H=3, P=4, G=1, N=6, seed=12, init="bernoulli")
    whole = oracle.recurrence(prob)
    qsl = prob["query_start_loc"]
    for b in range(5):
        one = sub_batch(prob, [b])
        sep = oracle.recurrence(one)
        s, e = qsl[b], qsl[b + 1]
        assert np.array_equal(sep["y"], whole["y"][s:e])
        assert np.array_equal(sep["final"][0], whole["final"][b])
    for L in (4, 64):
        ch = chunked_scan(prob, L)
        for b in range(5):
            chs = chunked_scan(sub_batch(prob, [b]), L)
            assert np.array_equal(chs["y"], ch["y"][qsl[b]:qsl[b + 1]])


# ------------------------------------------ split-carry through the state pool

@pytest.mark.parametrize("split", [1, 100, 255, 256, 257, 399])
def test_split_carry_through_pool(split):
    prob = small_problem([400], H=2, P=4, G=1, N=8, seed=13, init="all", pool_std=0.3)
    full = oracle.recurrence(prob)
    first = sub_batch(prob, [0])
    T = 400
    H, P, N = 2, 4, 8
    def part(lo, hi, pool, init):
        p = clone(first)
        for k, shape in (("x", (T, H, P)), ("dt", (T, H)), ("B", (T, 1, N)), ("C", (T, 1, N))):
            p[k] = np.ascontiguousarray(first[k].reshape(shape)[lo:hi])
        p["query_start_loc"] = np.array([0, hi - lo], np.int32)
        p["pool"] = pool
        p["has_initial_state"] = np.array([init], np.uint8)
        return p
    a = oracle.recurrence(part(0, split, prob["pool"], 1))
    b = oracle.recurrence(part(split, T, a["pool"], 1))
    # the carried state went through fp32 once
    assert max_rel(np.concatenate([a["y"], b["y"]]), full["y"]) <= 1e-6
    assert frob_rel(b["final"], full["final"]) <= 1e-6


# -------------------------------------------------------- slot bookkeeping

def test_slot_bookkeeping_and_sentinel():
    prob = small_problem([20, 0, 9], H=2, P=3, G=1, N=4, max_slots=7, seed=14,
                         init=[0, 1, 0], pool_std=0.5)
    # slots of sequences without an initial state hold NaN: they must not be read
    ci = prob["cache_indices"]
    prob["pool"][ci[0]] = np.nan
    prob["pool"][ci[2]] = np.nan
    out = oracle.recurrence(prob)
    assert np.all(np.isfinite(out["y"]))
    written = set(int(c) for c in ci)
    for s in range(7):
        if s in written:
            b = list(ci).index(s)
            assert np.array_equal(out["pool"][s], out["final"][b].astype(np.float32))
        else:
            assert np.array_equal(out["pool"][s].view(np.uint32), prob["pool"][s].view(np.uint32))
    # the zero-length sequence (index 1, with an initial state) writes that state back
    assert np.array_equal(out["pool"][ci[1]], prob["pool"][ci[1]])
    # a zero-length sequence without an initial state writes zeros
    p2 = clone(prob)
    p2["has_initial_state"] = np.array([0, 0, 0], np.uint8)
    p2["pool"][ci[1]] = np.nan
    o2 = oracle.recurrence(p2)
    assert np.all(o2["pool"][ci[1]] == 0)


# -------------------------------------------------------- group mapping

def test_group_mapping_h_div_heads_per_group():
    H, G, P, N = 4, 2, 3, 5
    prob = small_problem([25, 18], H=H, P=P, G=G, N=N, seed=15, init="all")
    out = oracle.recurrence(prob)
    T = prob["total_len"]
    for h in range(H):
        g = h // (H // G)       # group id = h // (nheads // ngroups)
        one = clone(prob)
        one["nheads"], one["ngroups"] = 1, 1
        one["x"] = np.ascontiguousarray(prob["x"].reshape(T, H, P)[:, h:h + 1])
        one["dt"] = np.ascontiguousarray(prob["dt"].reshape(T, H)[:, h:h + 1])
        one["B"] = np.ascontiguousarray(prob["B"].reshape(T, G, N)[:, g:g + 1])
        one["C"] = np.ascontiguousarray(prob["C"].reshape(T, G, N)[:, g:g + 1])
        for k in ("A", "D", "dt_bias"):
            one[k] = prob[k][h:h + 1].copy()
        one["pool"] = np.ascontiguousarray(prob["pool"][:, h:h + 1])
        o1 = oracle.recurrence(one)
        assert np.array_equal(o1["y"][:, 0], out["y"][:, h])
        assert np.array_equal(o1["final"][:, 0], out["final"][:, h])


def test_one_group_equals_replicated_groups():
    H, P, N = 4, 3, 5
    prob = small_problem([31, 4], H=H, P=P, G=1, N=N, seed=16, init="bernoulli")
    rep = clone(prob)
    T = prob["total_len"]
    rep["ngroups"] = H
    rep["B"] = np.ascontiguousarray(np.repeat(prob["B"].reshape(T, 1, N), H, axis=1))
    rep["C"] = np.ascontiguousarray(np.repeat(prob["C"].reshape(T, 1, N), H, axis=1))
    a, b = oracle.recurrence(prob), oracle.recurrence(rep)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["final"], b["final"])


# -------------------------------------------------------- batch permutation

def test_batch_permutation():
    prob = small_problem([12, 40, 3, 27], H=2, P=3, G=1, N=4, max_slots=6, seed=17, init="bernoulli")
    perm = [2, 0, 3, 1]
    pp = sub_batch(prob, perm)
    a, b = oracle.recurrence(prob), oracle.recurrence(pp)
    qa, qb = prob["query_start_loc"], pp["query_start_loc"]
    for i, src in enumerate(perm):
        assert np.array_equal(b["y"][qb[i]:qb[i + 1]], a["y"][qa[src]:qa[src + 1]])
        assert np.array_equal(b["final"][i], a["final"][src])
    assert np.array_equal(a["pool"], b["pool"])


# ------------------------------------------------ intermediates of the chunked form

def test_chunked_intermediates_chain():
    """h_in of a sequence's first chunk is its initial state and each later
    h_in follows the exponential-decay recurrence over chunk states."""
    prob = small_problem([600], H=1, P=2, G=1, N=3, seed=18, init="all")
    ch = chunked_scan(prob, 256, keep_intermediates=True)["chunks"]
    assert [c["length"] for c in ch] == [256, 256, 88]
    h0 = prob["pool"][prob["cache_indices"][0], 0].astype(np.float64)
    assert np.array_equal(ch[0]["h_in"], h0)
    for k in range(1, 3):
        exp_h = math.exp(ch[k - 1]["cs"][-1]) * ch[k - 1]["h_in"] + ch[k - 1]["S"]
        np.testing.assert_allclose(ch[k]["h_in"], exp_h, rtol=1e-14)
    rec = oracle.recurrence(prob)
    np.testing.assert_allclose(math.exp(ch[2]["cs"][-1]) * ch[2]["h_in"] + ch[2]["S"],
                               rec["final"][0, 0], rtol=1e-10)


# ------------------------------------------------- bf16 state storage (widening)

def test_bf16_pool_widening_by_hand():
    """A pool stored as bf16 bit patterns is read as the exact values those
    patterns encode: 0x3FC0 is 1.5 and 0xBFC0 is -1.5 (sign, exponent 127,
    one fraction bit), 0x0001 is the smallest bf16 subnormal 2^-133.  With
    B = 0 and one token, the final state is exp(A dts) h0 and y = C.h1 + D x,
    worked out here from those values."""
    prob = small_problem([1], H=1, P=2, G=1, N=3, max_slots=2, seed=63, init="all", state_dtype="bf16")
    slot = int(prob["cache_indices"][0])
    pool = np.zeros((2, 1, 2, 3), np.uint16)
    pool[slot, 0] = [[0x3FC0, 0xBFC0, 0x0001], [0x0000, 0x4040, 0xC000]]   # 1.5 -1.5 2^-133 / 0 3 -2
    prob["pool"] = pool
    prob["B"] = bf16(np.zeros((1, 1, 3)))
    h0 = np.array([[1.5, -1.5, 2.0 ** -133], [0.0, 3.0, -2.0]])
    dts = softplus(np.float64(prob["dt"][0, 0]) + np.float64(prob["dt_bias"][0]))
    h1 = math.exp(float(prob["A"][0]) * dts) * h0
    x = bf16_to_f64(prob["x"]).reshape(2)
    Cv = bf16_to_f64(prob["C"]).reshape(3)
    out = oracle.recurrence(prob, want_pool=False)
    np.testing.assert_allclose(out["final"][0, 0], h1, rtol=1e-14, atol=0)
    np.testing.assert_allclose(out["y"].reshape(2), h1 @ Cv + float(prob["D"][0]) * x, rtol=1e-13)


def test_bf16_pool_equals_its_fp32_values():
    """The bf16-storage problem gives the same y and final states as the fp32
    problem whose pool holds exactly the bf16 values (widened here by
    placing the 16 bits above 16 zero bits of an fp32 word), bitwise."""
    prob = small_problem([40, 0, 300], H=2, P=4, G=1, N=8, max_slots=5, seed=64, init="bernoulli",
                         state_dtype="bf16")
    pf = clone(prob)
    pf["pool"] = (prob["pool"].astype(np.uint32) << np.uint32(16)).view(np.float32)
    pf["state_dtype"] = "f32"
    a = oracle.recurrence(prob, want_pool=False)
    b = oracle.recurrence(pf, want_pool=False)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["final"], b["final"])


# ----------------------------------------- random tiny shapes (property test)

try:
    from hypothesis import given, settings, strategies as st
    HAVE_HYPOTHESIS = True
except ImportError:  # pragma: no cover
    HAVE_HYPOTHESIS = False


if HAVE_HYPOTHESIS:
    @settings(max_examples=60, deadline=None, derandomize=True, database=None)
    @given(lens=st.lists(st.integers(0, 40), min_size=1, max_size=4),
           hg=st.sampled_from([(1, 1), (2, 1), (2, 2), (4, 2)]),
           P=st.integers(1, 3), N=st.integers(1, 5), chunk=st.integers(1, 50),
           init=st.sampled_from(["none", "all", "bernoulli"]), softplus_on=st.booleans(),
           seed=st.integers(0, 2 ** 31 - 1))
    def test_random_tiny_shapes_chunked_equals_recurrence(lens, hg, P, N, chunk, init, softplus_on, seed):
        """On random tiny shapes (ragged lengths with empty sequences, random
        chunk sizes, groups, initial states, both dt settings) the chunked
        formulation agrees with the per-token recurrence to fp64 rounding,
        and every pool slot outside cache_indices keeps its bits."""
        H, G = hg
        prob = small_problem(lens, H=H, P=P, G=G, N=N, seed=seed, init=init, dt_softplus=softplus_on)
        if not softplus_on:  # keep dts >= 0 so the decays stay decays
            prob["dt"] = np.abs(prob["dt"]) * np.float32(0.1)
            prob["dt_bias"] = np.full_like(prob["dt_bias"], 0.01)
        rec = oracle.recurrence(prob)
        ch = chunked_scan(prob, chunk)
        assert max_rel(ch["y"], rec["y"]) <= 1e-10
        assert max_rel(ch["final"], rec["final"]) <= 1e-10
        written = set(int(c) for c in prob["cache_indices"])
        for s in range(prob["pool"].shape[0]):
            if s not in written:
                assert np.array_equal(rec["pool"][s].view(np.uint32), prob["pool"][s].view(np.uint32))
