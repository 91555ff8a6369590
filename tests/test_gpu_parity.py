"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (elementwise on y, per written slot on the final states):
  |y_gpu - y_ref| <= 2e-2 * (1 + |y_ref|)          y_ref: fp64 recurrence
  ||pool_gpu[slot] - final_ref||_F <= 1e-3 * ||final_ref||_F   (exact zeros when 0)
  every slot outside cache_indices bit-identical to its value before the call.
Intermediates left in the workspace are compared step by step with the
chunked oracle (oracle.chunked) on small problems.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.chunked import chunked_scan
from ssd_testlib import bf16, bf16_to_f64, clone, frob_rel, small_problem, sub_batch

torch = pytest.importorskip("torch")
from mamba_ssd_chunked_chunk_amd import binding, torch_io  # noqa: E402
from mamba_ssd_chunked_chunk_amd.workloads import make_problem, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

Y_RTOL = 2e-2
FINAL_TOL = 1e-3
# bf16 state storage: the final state is rounded once to bf16 (8 significant
# bits, nearest even: each element moves by at most half a unit in the last
# place, 2^-8 of its magnitude), so the bound grows by 2^-8
FINAL_TOL_BF16 = FINAL_TOL + 2.0 ** -8


# ssd_problem.short_path_max: the library default (128), or every sequence chunked
DEFAULT = binding.SHORT_PATH_DEFAULT
CHUNKED = 0


def gpu_run(prob, short_max=DEFAULT, **kw):
    d = torch_io.upload(prob, "cuda")
    ws = torch_io.run(d, short_path_max=short_max, **kw)
    torch.cuda.synchronize()
    return d, ws


def y_host(d):
    return d["y"].float().cpu().numpy().astype(np.float64)


def assert_y(y_gpu, y_ref, what=""):
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite y"
    err = np.abs(y_gpu - y_ref)
    ratio = err / (Y_RTOL * (1.0 + np.abs(y_ref)))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: y error {worst:.3f} x the bound at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def assert_final(pool_slot, ref, what="", tol=FINAL_TOL):
    nref = np.linalg.norm(ref)
    if nref == 0:
        assert np.all(pool_slot == 0), f"{what}: expected zeros"
        return 0.0
    r = frob_rel(pool_slot, ref)
    assert r <= tol, f"{what}: final-state rel err {r:.2e}"
    return r


def assert_untouched(pool_after, pool_before, written):
    for s in range(pool_before.shape[0]):
        if s not in written:
            assert np.array_equal(pool_after[s].view(np.uint32), pool_before[s].view(np.uint32)), f"slot {s} modified"


def bits(t):
    """The tensor's bit patterns (for bitwise comparisons that NaNs survive)."""
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def full_check(prob, short_max=DEFAULT):
    """Run on GPU, compare every sequence with the oracle, check slot
    bookkeeping.  Returns (y worst ratio, final worst)."""
    tol = FINAL_TOL_BF16 if prob.get("state_dtype", "f32") == "bf16" else FINAL_TOL
    d = torch_io.upload(prob, "cuda")
    before = d["pool"].clone()
    torch_io.run(d, short_path_max=short_max)
    torch.cuda.synchronize()
    ci = prob["cache_indices"]
    ref = oracle.recurrence(prob, want_pool=False)
    wy = assert_y(y_host(d), ref["y"], prob.get("name", ""))
    wf = 0.0
    # the written slots, gathered on the device and copied back together
    fin = d["pool"].index_select(0, torch.from_numpy(ci.astype(np.int64)).cuda()).float().cpu().numpy()
    for b in range(len(ci)):
        wf = max(wf, assert_final(fin[b], ref["final"][b], f"seq {b}", tol))
    # slots outside cache_indices: bit-identical (compared on the device)
    written = torch.zeros(prob["pool"].shape[0], dtype=torch.bool, device="cuda")
    written[torch.from_numpy(ci.astype(np.int64)).cuda()] = True
    keep = (~written).nonzero().flatten()
    assert torch.equal(bits(d["pool"].index_select(0, keep)),
                       bits(before.index_select(0, keep))), "an untouched slot changed"
    assert bool(torch.isfinite(d["y"]).all()), "non-finite y"
    return wy, wf


# ------------------------------------------------------------- small cases

SMALL = {
    "edges_g2_n64": dict(seqlens=[0, 1, 255, 256, 257, 511], H=4, P=64, G=2, N=64, init="bernoulli"),
    "groups_eq_heads_n128": dict(seqlens=[300, 17, 600], H=4, P=64, G=4, N=128, init="all"),
    "n256_two_heads": dict(seqlens=[1000, 5], H=2, P=64, G=1, N=256, init="half"),
    "short_many_n128": dict(seqlens=list(np.random.default_rng(3).integers(1, 97, 48)), H=8, P=64, G=2,
                            N=128, init="all"),
    "single_token": dict(seqlens=[1], H=2, P=64, G=1, N=64, init="all"),
    "all_empty": dict(seqlens=[0, 0, 0], H=2, P=64, G=1, N=64, init=[1, 0, 1]),
}


@pytest.mark.parametrize("route", ["default", "chunked"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name, route):
    """Every case under the default routing (short sequences at dstate <= 128
    to the fused kernel) and with every sequence through the chunked steps."""
    spec = dict(SMALL[name])
    lens = spec.pop("seqlens")
    prob = small_problem(lens, seed=100 + len(name), **spec)
    full_check(prob, DEFAULT if route == "default" else CHUNKED)


@pytest.mark.parametrize("N,T,short_max", [(64, 129, DEFAULT), (128, 700, DEFAULT), (128, 128, DEFAULT),
                                           (64, 4, DEFAULT), (128, 200, 100), (64, 300, CHUNKED)])
def test_single_sequence_routing(N, T, short_max):
    """One sequence: the host knows its length, and launches the short path's
    kernels only when that length is within the limit; the result is the
    oracle's either way."""
    prob = small_problem([T], H=4, P=64, G=2, N=N, seed=90 + T, init="all")
    full_check(prob, short_max)


@pytest.mark.parametrize("nseq", [2, 4])
def test_head_blocks_dstate64(nseq):
    """dstate 64 with 16 heads in one group and 128 or 256 chunks: the
    chunked kernels pick 8 or 16 heads per workgroup (one workgroup per
    compute unit), a block size no other dstate-64 case reaches.  Every
    sequence is compared with the oracle."""
    prob = small_problem([16384] * nseq, H=16, P=64, G=1, N=64, max_slots=nseq + 2, seed=120 + nseq,
                         init="bernoulli")
    wy, wf = full_check(prob)
    print(f"dstate 64, {nseq} x 16384: worst y ratio {wy:.3f}, worst final {wf:.2e}")


# (heads, groups, dstate, sequence lengths) that make the chunked kernels split
# each (chunk, group) over nwg workgroups of HB heads, and so split the four
# row-block pairs of its C.B^T tiles differently (on a 256-CU device): nwg 16
# (workgroups 4..15 form no tile), 3 (pairs 0 and 3, 1, 2), 2 at dstate 256,
# and 8 at dstate 128 with the short path on
GRAM_SPLITS = {
    "nwg16_n256": (16, 1, 256, [300, 300]),
    "nwg3_n256": (12, 1, 256, [6800, 6800, 6800]),
    "nwg2_n256": (16, 1, 256, [8250] * 4),
    "nwg8_n128": (8, 1, 128, [700, 700]),
}


@pytest.mark.parametrize("name", list(GRAM_SPLITS))
def test_gram_tiles_split_over_head_blocks(name):
    """The workgroups of a chunk and group share its C.B^T tiles (each forms
    the tiles of its row-block pairs) and read them all back: every sequence
    is compared with the oracle."""
    H, G, N, lens = GRAM_SPLITS[name]
    prob = small_problem(lens, H=H, P=64, G=G, N=N, max_slots=len(lens) + 1, seed=140 + H + N,
                         init="bernoulli")
    wy, wf = full_check(prob)
    print(f"{name}: worst y ratio {wy:.3f}, worst final {wf:.2e}")


# lengths around the short-path limit and the fused kernel's 16-token K-steps
# and 32-token row blocks, with empty and chunked neighbours
MIXED_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 0, 64, 95, 96, 97, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("N,G,init", [(64, 2, "bernoulli"), (128, 4, "all"), (128, 1, "none")])
def test_short_path_mixed_lengths(N, G, init):
    prob = small_problem(MIXED_LENS, H=8, P=64, G=G, N=N, seed=90 + N + G, init=init)
    full_check(prob, binding.SHORT_PATH_LIMIT)


@pytest.mark.parametrize("limit", [1, 33, 96])
def test_short_path_limit_respected(limit):
    """A lower limit moves the longer short sequences back to the chunked
    steps: the chunk table holds exactly the sequences above the limit."""
    prob = small_problem(MIXED_LENS, H=4, P=64, G=2, N=128, seed=95, init="bernoulli")
    d, ws = gpu_run(prob, limit)
    ref = oracle.recurrence(prob, want_pool=False)
    assert_y(y_host(d), ref["y"], f"limit {limit}")
    for b, slot in enumerate(prob["cache_indices"]):
        assert_final(d["pool"][int(slot)].cpu().numpy(), ref["final"][b], f"seq {b}")
    L = binding.ssd_workspace_get_layout(torch_io.problem_struct(d))
    w = ws.cpu().numpy()
    nch = int(w[L["meta"]:L["meta"] + 4].view(np.int32)[0])
    assert nch == sum(-(-n // 256) for n in MIXED_LENS if n > limit)


def test_short_path_extremes():
    """Inputs that push the fused kernel's power-of-two scalings: large dt
    without softplus (decays near 0 and weights of ~10), an all-zero x head
    block, tiny B, and a huge initial state."""
    prob = small_problem([96, 1, 128, 40], H=4, P=64, G=2, N=128, seed=97, init="all", dt_softplus=False)
    T = prob["total_len"]
    rng = np.random.default_rng(197)
    prob["dt"] = rng.uniform(0.0, 10.0, prob["dt"].shape).astype(np.float32)
    prob["dt_bias"] = np.zeros_like(prob["dt_bias"])
    x = bf16_to_f64(prob["x"]).reshape(T, 4, 64)
    x[96:97 + 128] = 0.0
    prob["x"] = bf16(x)
    Bm = bf16_to_f64(prob["B"]).reshape(T, 2, 128)
    Bm[:, 1] *= 1e-6
    prob["B"] = bf16(Bm)
    prob["pool"] *= np.float32(1e4)
    full_check(prob)


def check_block_scaled(prob, short_max, rel=1e-2):
    """y against the oracle relative to its local magnitude: in every
    32-token block of a sequence (the kernels' row blocks) and head, the
    largest error is at most rel * the block's largest |y_ref|, and the
    block's error norm at most rel * its norm; final states and untouched
    slots as in full_check.  Returns the worst error / block max."""
    d = torch_io.upload(prob, "cuda")
    torch_io.run(d, short_path_max=short_max)
    torch.cuda.synchronize()
    ref = oracle.recurrence(prob, want_pool=False)
    y = y_host(d)
    assert np.all(np.isfinite(y))
    qsl = prob["query_start_loc"]
    worst = 0.0
    for b in range(len(qsl) - 1):
        for t0 in range(int(qsl[b]), int(qsl[b + 1]), 32):
            t1 = min(t0 + 32, int(qsl[b + 1]))
            for h in range(prob["nheads"]):
                r, g = ref["y"][t0:t1, h], y[t0:t1, h]
                s = np.abs(r).max()
                if s == 0:
                    assert np.all(g == 0)
                    continue
                e = np.abs(g - r).max() / s
                worst = max(worst, e)
                assert e <= rel, f"seq {b} tokens {t0}..{t1} head {h}: error {e:.2e} of the block's max |y|"
                assert np.linalg.norm(g - r) <= rel * np.linalg.norm(r)
    ci = prob["cache_indices"]
    fin = d["pool"].index_select(0, torch.from_numpy(ci.astype(np.int64)).cuda()).float().cpu().numpy()
    for b in range(len(ci)):
        assert_final(fin[b], ref["final"][b], f"seq {b}")
    return worst


@pytest.mark.parametrize("route", ["default", "chunked"])
@pytest.mark.parametrize("N,case", [(128, "positive_A"), (256, "positive_A"), (128, "negative_dts"),
                                    (64, "negative_dts")])
def test_growing_states(N, case, route):
    """A * dts > 0, where the state grows instead of decaying: a positive A
    (the recurrence of "mamba2_ssd_scan" takes A as given), or negative dts
    (dt + dt_bias < 0 without softplus).  |y| then grows by orders of
    magnitude along a sequence; the kernels' fp16 operands keep the error
    relative to the local magnitude (checked per 32-token block and head),
    while the elementwise bound's absolute floor of 2e-2 assumes |y| of
    order 10 (see test_scaled_inputs)."""
    prob = small_problem([700, 300, 40, 5, 0], H=4, P=64, G=2, N=N, seed=7 * len(case) + N, init="all")
    rng = np.random.default_rng(N + len(case))
    H, T = 4, prob["total_len"]
    if case == "positive_A":
        # the drawn dts are at most about 0.3: A * dts up to 0.015 per token, e^10.5 over 700
        prob["A"] = rng.uniform(0.01, 0.05, H).astype(np.float32)
    else:
        prob["dt_softplus"] = False
        prob["dt"] = rng.uniform(-0.2, 0.05, (T, H)).astype(np.float32).reshape(prob["dt"].shape)
        prob["dt_bias"] = np.zeros(H, np.float32)
        prob["A"] = -rng.uniform(0.05, 0.1, H).astype(np.float32)  # A * dts in (-0.005, 0.02)
    w = check_block_scaled(prob, DEFAULT if route == "default" else CHUNKED)
    print(f"{case} N={N} ({route}): worst error / block max |y| {w:.2e}", flush=True)


@pytest.mark.parametrize("scale", [100.0, 1000.0])
def test_scaled_inputs(scale):
    """y is linear in x and the initial states together: scaling both by k
    scales y by k, and the elementwise bound scales with it,
    |dy| <= 2e-2 (k + |y_ref|) (the bound of the problem divided by k)."""
    prob = small_problem([700, 300, 60], H=4, P=64, G=2, N=128, seed=95, init="all")
    prob["x"] = bf16(bf16_to_f64(prob["x"]) * scale)
    prob["pool"] = (prob["pool"] * np.float32(scale)).astype(np.float32)
    d, _ = gpu_run(prob)
    ref = oracle.recurrence(prob, want_pool=False)
    y = y_host(d)
    ratio = np.abs(y - ref["y"]) / (Y_RTOL * (scale + np.abs(ref["y"])))
    assert ratio.max() <= 1.0, f"error {ratio.max():.3f} x the scaled bound"
    ci = prob["cache_indices"]
    fin = d["pool"].cpu().numpy()[ci.astype(np.int64)]
    for b in range(len(ci)):
        assert_final(fin[b], ref["final"][b], f"seq {b}")
    print(f"x and states x{scale:.0f}: worst / scaled bound {ratio.max():.3f}", flush=True)


def test_short_nan_slot_not_read():
    """A short sequence without an initial state must not read its slot."""
    prob = small_problem([50, 7, 120], H=4, P=64, G=1, N=64, max_slots=5, seed=98, init=[0, 1, 0])
    ci = prob["cache_indices"]
    prob["pool"][ci[0]] = np.nan
    prob["pool"][ci[2]] = np.nan
    full_check(prob, binding.SHORT_PATH_LIMIT)


@pytest.mark.parametrize("opt", ["no_D", "no_dt_bias", "no_has_init", "no_softplus"])
def test_optional_inputs_and_flag(opt):
    kw = dict(init="all")
    if opt == "no_D":
        kw["with_D"] = False
    if opt == "no_dt_bias":
        kw["with_dt_bias"] = False
    if opt == "no_has_init":
        kw["with_has_init"] = False
    if opt == "no_softplus":
        kw["dt_softplus"] = False
    prob = small_problem([400, 130], H=4, P=64, G=1, N=128, seed=5, **kw)
    if opt == "no_softplus":
        prob["dt"] = (np.abs(prob["dt"]) * np.float32(0.1)).astype(np.float32)
        prob["dt_bias"] = np.full_like(prob["dt_bias"], 0.01)
    full_check(prob)


def test_tiny_workload_full():
    full_check(make_workload("tiny_1x512_h4_n64"))


# ---------------------------------------------------- per-step intermediates

def test_intermediates_match_chunked_oracle():
    prob = small_problem([600, 0, 255, 129], H=4, P=64, G=2, N=128, seed=31, init="bernoulli")
    d, ws = gpu_run(prob)
    prob_s = binding.make_problem(prob["total_len"], 4, 4, 64, 2, 128, prob["pool"].shape[0])
    L = binding.ssd_workspace_get_layout(prob_s)
    w = ws.cpu().numpy()
    ncm = L["nchunks_max"]
    H, P, N = 4, 64, 128
    nch = int(w[L["meta"]:L["meta"] + 4].view(np.int32)[0])
    assert nch == 3 + 0 + 1 + 1 <= ncm
    chunk_off = w[L["chunk_off"]:L["chunk_off"] + 5 * 4].view(np.int32)
    assert list(chunk_off) == [0, 3, 3, 4, 5]
    # only the call's nch rows of each table were written: rows past them are
    # left as the workspace held them and are not decoded
    desc = w[L["desc"]:L["desc"] + ncm * 16].view(np.int32).reshape(ncm, 4)[:nch]
    dts = w[L["dts"]:L["dts"] + ncm * H * 256 * 4].view(np.float32).reshape(ncm, H, 256)[:nch]
    cs2 = w[L["cs2"]:L["cs2"] + ncm * H * 256 * 4].view(np.float32).reshape(ncm, H, 256)[:nch]
    S16 = w[L["states"]:L["states"] + ncm * H * P * N * 2].view(np.float16).reshape(ncm, H, P, N)[:nch]
    sexp = w[L["sexp"]:L["sexp"] + ncm * H * 2 * (N // 32) * 4].view(np.int32).reshape(ncm, H, 2, N // 32)[:nch]
    # element (p, n) of a chunk's contribution is scaled by 2^sexp[p / 32][n / 32]
    S = S16.astype(np.float64) * np.exp2(-sexp.astype(np.float64)).repeat(32, axis=2).repeat(32, axis=3)
    hin16 = w[L["hin"]:L["hin"] + ncm * H * P * N * 2].view(np.float16).reshape(ncm, H, P, N)[:nch]
    hexp = w[L["hexp"]:L["hexp"] + ncm * H * P * 4].view(np.int32).reshape(ncm, H, P)[:nch]
    # row p of a chunk and head is scaled by 2^hexp[p]
    hin = hin16.astype(np.float64) * np.exp2(-hexp.astype(np.float64))[..., None]
    cbt16 = w[L["cbt"]:L["cbt"] + ncm * 2 * 36 * 1024 * 2].view(np.float16).reshape(ncm, 2, 36, 64, 16)[:nch]
    # one exponent per row-block pair (q, 7 - q) of each chunk and group
    gexp = w[L["gexp"]:L["gexp"] + ncm * 2 * 4 * 4].view(np.int32).reshape(ncm, 2, 4)[:nch]
    pair_of_tile = np.array([min(rb, 7 - rb) for rb in range(8) for _ in range(rb + 1)])
    cbt = cbt16.astype(np.float64) * np.exp2(-gexp[:, :, pair_of_tile].astype(np.float64))[..., None, None]
    xexp = w[L["xexp"]:L["xexp"] + ncm * H * 2 * 4].view(np.int32).reshape(ncm, H, 2)[:nch]
    ref = chunked_scan(prob, 256, keep_intermediates=True)["chunks"]
    qsl = prob["query_start_loc"]
    for rec in ref:
        b, h, t0, l = rec["b"], rec["h"], rec["t0"], rec["length"]
        c = chunk_off[b] + (t0 - qsl[b]) // 256
        assert tuple(desc[c][:3]) == (b, t0, l)
        np.testing.assert_allclose(dts[c, h, :l], rec["dts"], rtol=1e-5, atol=1e-7)
        assert np.all(dts[c, h, l:] == 0)
        cs2_ref = rec["cs"] * math.log2(math.e)
        tol = 3e-5 * (abs(cs2_ref[-1]) + 1.0)
        assert np.max(np.abs(cs2[c, h, :l] - cs2_ref)) <= tol
        assert frob_rel(S[c, h], rec["S"]) <= 1e-3
        assert frob_rel(hin[c, h], rec["h_in"]) <= 1e-3
        # each 32x32 tile of S is scaled so that its largest magnitude lies in
        # [2^14, 2^15) before the rounding to fp16, which can carry it to 2^15
        for ptile in range(2):
            for ntile in range(N // 32):
                tile = np.abs(S16[c, h, 32 * ptile:32 * ptile + 32, 32 * ntile:32 * ntile + 32].astype(np.float64))
                assert tile.max() == 0 or 2.0 ** 14 <= tile.max() <= 2.0 ** 15
        # each nonzero row of h_in likewise
        rows = np.abs(hin16[c, h].astype(np.float64)).max(axis=1)
        assert np.all((rows == 0) | ((rows >= 2.0 ** 14) & (rows <= 2.0 ** 15)))
        # C.B^T tiles (stored transposed, in MFMA accumulator order) against the plain product
        T = prob["total_len"]
        g = h // 2
        Bc = bf16_to_f64(prob["B"]).reshape(T, 2, N)[t0:t0 + l, g]
        Cc = bf16_to_f64(prob["C"]).reshape(T, 2, N)[t0:t0 + l, g]
        GT = np.zeros((256, 256))
        GT[:l, :l] = Bc @ Cc.T  # G^T[j][i] = B_j . C_i
        # what the kernel forms for every stored entry: B rows past the chunk
        # end are zero, C rows past it repeat its last row
        rows = np.minimum(np.arange(256), l - 1)
        Bz = np.zeros((256, N))
        Bz[:l] = Bc
        GTe = Bz @ Cc[rows].T
        # x exponent of the chunk, head and half of p: 2^xexp puts the
        # half's largest |x| in [2^14, 2^15) (1000 marks an all-zero half)
        for ph in range(2):
            xm = np.abs(bf16_to_f64(prob["x"]).reshape(T, H, P)[t0:t0 + l, h, 32 * ph:32 * ph + 32]).max()
            if xm > 0:
                assert 2.0 ** 14 <= xm * 2.0 ** xexp[c, h, ph] < 2.0 ** 15
            else:
                assert xexp[c, h, ph] == 1000
        lane = np.arange(64)[:, None]
        e = np.arange(16)[None, :]
        gm = np.zeros(4)
        for rb in range(8):
            for t in range(rb + 1):
                jj = 32 * t + 8 * (e // 4) + 4 * (lane // 32) + e % 4
                ii = 32 * rb + lane % 32
                inside = (jj < l) & (ii < l)  # entries past the chunk end are unspecified
                want = np.where(jj <= ii, GT[jj, ii], 0.0)  # the diagonal tile is zero above its diagonal
                np.testing.assert_allclose(cbt[c, g, rb * (rb + 1) // 2 + t][inside], want[inside],
                                           rtol=2.0 ** -11, atol=np.abs(GT).max() * 2.0 ** -24)
                # the stored tile's entries, rows past the chunk end included
                # (there B is zero and C repeats the chunk's last row)
                q = min(rb, 7 - rb)
                gm[q] = max(gm[q], np.abs(np.where(jj <= ii, GTe[jj, ii], 0.0)).max())
        # each pair's exponent puts its tiles' largest magnitude in [2^14,
        # 2^15), up to the rounding of the fp32 products (2^13 allows for it)
        for q in range(4):
            if gm[q] > 0:
                assert 2.0 ** 13 <= gm[q] * 2.0 ** gexp[c, g, q] < 2.0 ** 15


# --------------------------------------------------------------- invariants

def test_concat_equals_separate_bitwise():
    prob = small_problem([300, 45, 513], H=4, P=64, G=1, N=128, seed=41, init="all")
    d, _ = gpu_run(prob)
    yall = d["y"].cpu()
    qsl = prob["query_start_loc"]
    for b in range(3):
        one = sub_batch(prob, [b])
        d1, _ = gpu_run(one)
        assert torch.equal(d1["y"].cpu(), yall[qsl[b]:qsl[b + 1]])
        slot = int(prob["cache_indices"][b])
        assert torch.equal(d1["pool"][slot].cpu(), d["pool"][slot].cpu())


def test_deterministic_bitwise():
    prob = small_problem([700, 90], H=4, P=64, G=2, N=256, seed=42, init="half")
    d1, _ = gpu_run(prob)
    d2, _ = gpu_run(prob)
    assert torch.equal(d1["y"], d2["y"]) and torch.equal(d1["pool"], d2["pool"])


def test_concurrent_streams_bitwise():
    """The library keeps no state between calls: four problems of different
    sizes and routes (dstate 64, 128 and 256, short, chunked and decode
    sequences, a non-default short-path limit), each with its own workspace,
    launched alternately on two streams with nothing between the launches,
    give bitwise the results of the same calls made one at a time, and every
    sequence matches the oracle."""
    cases = [
        (small_problem([700, 3, 90, 257], H=4, P=64, G=2, N=128, seed=611, max_slots=7, init="bernoulli"), DEFAULT),
        (small_problem([1000, 40], H=2, P=64, G=1, N=256, seed=612, max_slots=4, init="all"), DEFAULT),
        (small_problem([5, 1, 128, 60, 0, 2], H=4, P=64, G=4, N=64, seed=613, max_slots=8, init="all"), DEFAULT),
        (small_problem([300, 33, 129], H=2, P=64, G=1, N=128, seed=614, max_slots=5, init="half"), 40),
    ]
    alone = [gpu_run(prob, sm)[0] for prob, sm in cases]
    ds = [torch_io.upload(prob, "cuda") for prob, _ in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    keep = []  # workspaces, alive until the streams are done
    for i, (d, (_, sm)) in enumerate(zip(ds, cases)):
        with torch.cuda.stream(streams[i % 2]):
            keep.append(torch_io.run(d, short_path_max=sm))
    torch.cuda.synchronize()
    for i, ((prob, _), a, d) in enumerate(zip(cases, alone, ds)):
        assert torch.equal(a["y"].view(torch.int16), d["y"].view(torch.int16)), f"problem {i}: y"
        assert torch.equal(a["pool"].view(torch.int32), d["pool"].view(torch.int32)), f"problem {i}: pool"
        ref = oracle.recurrence(prob)
        assert_y(y_host(d), ref["y"], f"problem {i}")
        fin = d["pool"].cpu().numpy()
        for b, slot in enumerate(prob["cache_indices"]):
            assert_final(fin[int(slot)], ref["final"][b], f"problem {i} seq {b}")


def test_nan_sentinel_slots_not_read():
    prob = small_problem([200, 0, 333], H=4, P=64, G=1, N=64, max_slots=6, seed=43, init=[0, 0, 1])
    ci = prob["cache_indices"]
    prob["pool"][ci[0]] = np.nan
    prob["pool"][ci[1]] = np.nan
    wy, wf = full_check(prob)
    # the zero-length sequence without an initial state writes zeros
    d, _ = gpu_run(prob)
    assert torch.all(d["pool"][int(ci[1])] == 0)


def test_split_carry_through_pool():
    prob = small_problem([900], H=2, P=64, G=1, N=128, seed=44, init="all")
    full = oracle.recurrence(prob, want_pool=False)
    T, H, P, N = 900, 2, 64, 128
    k = 333

    def part(lo, hi, pool):
        p = dict(prob)
        for key, shape in (("x", (T, H, P)), ("dt", (T, H)), ("B", (T, 1, N)), ("C", (T, 1, N))):
            p[key] = np.ascontiguousarray(prob[key].reshape(shape)[lo:hi])
        p["query_start_loc"] = np.array([0, hi - lo], np.int32)
        p["total_len"] = hi - lo
        p["pool"] = pool
        return p
    d1, _ = gpu_run(part(0, k, prob["pool"]))
    d2, _ = gpu_run(part(k, T, d1["pool"].cpu().numpy()))
    y = np.concatenate([y_host(d1), y_host(d2)])
    assert_y(y, full["y"], "split")
    slot = int(prob["cache_indices"][0])
    assert_final(d2["pool"][slot].cpu().numpy(), full["final"][0], "split final")


def test_short_limit_is_per_call():
    """The short-path limit travels in each call's problem: two calls back to
    back on one stream with different limits each route by their own limit
    (the chunk count in the workspace) and each matches the oracle."""
    prob = small_problem(MIXED_LENS, H=4, P=64, G=2, N=128, seed=96, init="bernoulli")
    ref = oracle.recurrence(prob, want_pool=False)
    d1 = torch_io.upload(prob, "cuda")
    d2 = torch_io.upload(prob, "cuda")
    ws1 = torch_io.run(d1, short_path_max=CHUNKED)
    ws2 = torch_io.run(d2, short_path_max=40)  # enqueued right behind the first, no sync between
    torch.cuda.synchronize()
    for d, ws, limit in ((d1, ws1, 0), (d2, ws2, 40)):
        assert_y(y_host(d), ref["y"], f"limit {limit}")
        for b, slot in enumerate(prob["cache_indices"]):
            assert_final(d["pool"][int(slot)].cpu().numpy(), ref["final"][b], f"limit {limit} seq {b}")
        L = binding.ssd_workspace_get_layout(torch_io.problem_struct(d))
        nch = int(ws.cpu().numpy()[L["meta"]:L["meta"] + 4].view(np.int32)[0])
        assert nch == sum(-(-n // 256) for n in MIXED_LENS if n > limit), limit


def test_canaries_around_outputs():
    """y and the pool placed inside larger buffers whose margins hold a
    canary pattern: no store of the call lands outside y's rows or the pool's
    slots (the margins are compared bitwise after the call)."""
    prob = small_problem([300, 0, 513, 17, 128], H=4, P=64, G=2, N=128, max_slots=7, seed=47, init="bernoulli")
    d = torch_io.upload(prob, "cuda")
    T, H, P = d["y"].shape
    pad = 16  # tokens / slots of margin on each side
    ybuf = torch.full((T + 2 * pad, H, P), -12345.0, dtype=torch.bfloat16, device="cuda")
    d["y"] = ybuf[pad:pad + T]
    S = d["pool"].shape[0]
    pbuf = torch.full((S + 2,) + tuple(d["pool"].shape[1:]), 777.0, dtype=torch.float32, device="cuda")
    pbuf[1:S + 1].copy_(d["pool"])
    d["pool"] = pbuf[1:S + 1]
    ycan, pcan = ybuf.clone(), pbuf.clone()
    pool0 = d["pool"].clone()
    ref = oracle.recurrence(prob, want_pool=False)
    for sm in (DEFAULT, CHUNKED):
        d["pool"].copy_(pool0)  # the call updates the pool in place: each run starts from the same states
        torch_io.run(d, short_path_max=sm)
        torch.cuda.synchronize()
        assert torch.equal(bits(ybuf[:pad]), bits(ycan[:pad])) and torch.equal(bits(ybuf[pad + T:]),
                                                                           bits(ycan[pad + T:])), sm
        assert torch.equal(bits(pbuf[0]), bits(pcan[0])) and torch.equal(bits(pbuf[S + 1]), bits(pcan[S + 1])), sm
        assert_y(y_host(d), ref["y"], f"canary run, short_path_max {sm}")


@pytest.mark.parametrize("short_max", [DEFAULT, CHUNKED])
def test_batch_permutation_bitwise(short_max):
    """Permuting the sequences together with their cache_indices and
    has_initial_state permutes the y rows and moves nothing else: each
    sequence's y rows and final state are bit-identical in both orders."""
    prob = small_problem([300, 45, 0, 513, 96, 1], H=4, P=64, G=2, N=128, max_slots=9, seed=48, init="bernoulli")
    perm = [3, 0, 5, 2, 4, 1]
    q = sub_batch(prob, perm)
    d1, _ = gpu_run(prob, short_max)
    d2, _ = gpu_run(q, short_max)
    qa, qb = prob["query_start_loc"], q["query_start_loc"]
    for i, b in enumerate(perm):
        assert torch.equal(bits(d1["y"][qa[b]:qa[b + 1]]), bits(d2["y"][qb[i]:qb[i + 1]])), b
    assert torch.equal(bits(d1["pool"]), bits(d2["pool"]))


def test_subnormal_initial_states():
    """Initial states whose rows are fp32 subnormals (1e-40), and a chunk of
    zero x after strong decay: the power-of-two scalings of the state rows
    must stay finite, and y and the final states match the oracle (the final
    states may carry the subnormal range's coarser rounding: a few units of
    2^-149 on top of the relative bar)."""
    for N, sm in ((128, DEFAULT), (128, CHUNKED), (256, DEFAULT)):
        prob = small_problem([700, 40, 300], H=2, P=64, G=1, N=N, max_slots=4, seed=49, init="all")
        ci = prob["cache_indices"]
        prob["pool"][ci[0]] = np.float32(1e-40)
        prob["pool"][ci[1]] = np.float32(-3e-41)
        # the third sequence: x zero on its second half, A strongly negative
        T = prob["total_len"]
        x = bf16_to_f64(prob["x"]).reshape(T, 2, 64)
        x[740 + 150:] = 0.0
        prob["x"] = bf16(x)
        prob["A"] = np.array([-16.0, -1.0], np.float32)
        d, _ = gpu_run(prob, sm)
        ref = oracle.recurrence(prob, want_pool=False)
        assert_y(y_host(d), ref["y"], f"N {N} short_max {sm}")
        for b, slot in enumerate(ci):
            got = d["pool"][int(slot)].cpu().numpy().astype(np.float64)
            want = ref["final"][b]
            err = np.linalg.norm(got - want)
            assert np.all(np.isfinite(got))
            assert err <= 1e-3 * np.linalg.norm(want) + 8 * 2.0 ** -149 * math.sqrt(got.size), (N, sm, b, err)


def test_validate_inputs_on_device():
    prob = small_problem([10, 20], H=2, P=64, G=1, N=64, max_slots=4, seed=45)
    d = torch_io.upload(prob, "cuda")
    ps = torch_io.problem_struct(d)
    assert binding.ssd_validate_inputs(ps, d["query_start_loc"], d["cache_indices"]) == 0
    bad = d["cache_indices"].clone()
    bad[1] = bad[0]
    assert binding.ssd_validate_inputs(ps, d["query_start_loc"], bad) == 5
    bad[1] = 4
    assert binding.ssd_validate_inputs(ps, d["query_start_loc"], bad) == 5
    q = d["query_start_loc"].clone()
    q[1] = 35  # beyond q[2] = 30: not non-decreasing
    assert binding.ssd_validate_inputs(ps, q, d["cache_indices"]) == 5


# ------------------------------------------------ workloads at full size

# ---------------------------------- separate initial and final states

def run_separate(prob, initial_states, *, aliased=False):
    """The entry point with separate states; final_states starts as NaN (or
    is the initial-states buffer itself when ``aliased``)."""
    d = torch_io.upload(prob, "cuda")
    batch = len(prob["query_start_loc"]) - 1
    H, P, N = prob["nheads"], prob["head_dim"], prob["dstate"]
    init_t = None if initial_states is None else torch.from_numpy(initial_states).cuda()
    if aliased:
        final_t = init_t
    else:
        final_t = torch.full((batch, H, P, N), float("nan"), dtype=torch.float32, device="cuda")
    torch_io.run_fwd(d, init_t, final_t)
    torch.cuda.synchronize()
    return d, final_t


def random_states(prob, seed, scale=0.5):
    batch = len(prob["query_start_loc"]) - 1
    shape = (batch, prob["nheads"], prob["head_dim"], prob["dstate"])
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("with_init", [True, False], ids=["initial", "zero"])
def test_separate_states_match_oracle(with_init):
    prob = small_problem([300, 0, 513, 17], H=4, P=64, G=2, N=128, seed=71, init="none")
    init = random_states(prob, 171) if with_init else None
    d, fin = run_separate(prob, init)
    ref = oracle.recurrence_separate(prob, init)
    assert_y(y_host(d), ref["y"], "separate states")
    fh = fin.cpu().numpy()
    for b in range(4):
        assert_final(fh[b], ref["final"][b], f"seq {b}")
    # the zero-length sequence hands its initial state (or zeros) straight through
    want = init[1] if with_init else np.zeros_like(fh[1])
    assert np.array_equal(fh[1].view(np.uint32), want.view(np.uint32))


def test_separate_equals_inplace_bitwise():
    prob = small_problem([700, 45, 0, 256], H=4, P=64, G=1, N=256, seed=72, init="none")
    init = random_states(prob, 172)
    # the same initial states placed in a pool at permuted slots
    q = clone(prob)
    slots = np.array([5, 0, 3, 1], np.uint32)
    pool = np.full((6,) + init.shape[1:], np.nan, np.float32)
    pool[slots] = init
    q["pool"], q["cache_indices"], q["has_initial_state"] = pool, slots, np.ones(4, np.uint8)
    d1, _ = gpu_run(q)
    d2, fin = run_separate(prob, init)
    assert torch.equal(d1["y"].view(torch.int16), d2["y"].view(torch.int16))
    for b in range(4):
        assert torch.equal(d1["pool"][int(slots[b])].view(torch.int32), fin[b].view(torch.int32)), b


def test_separate_states_aliased_buffer():
    prob = small_problem([400, 3, 0, 90], H=2, P=64, G=1, N=64, seed=73, init="none")
    init = random_states(prob, 173)
    d1, fin = run_separate(prob, init)
    d2, fin2 = run_separate(prob, init.copy(), aliased=True)
    assert torch.equal(d1["y"].view(torch.int16), d2["y"].view(torch.int16))
    assert torch.equal(fin.view(torch.int32), fin2.view(torch.int32))


@pytest.mark.parametrize("name,short_max", [
    ("fixed_4x4096_h16_n256", DEFAULT),
    ("long_8x16384_h16_n256", DEFAULT),
    ("ragged_32_h128_g8_n128", DEFAULT),
    # the same batch with every sequence through the chunked steps: the
    # state chain then walks the whole batch, short sequences included
    ("ragged_32_h128_g8_n128", CHUNKED),
    ("short_512_h128_g8_n128", DEFAULT),
    ("decode_512_h128_g8_n128", DEFAULT),
])
def test_workloads_full_size(name, short_max):
    """Every sequence of the full-size workloads against the fp64 oracle (y
    elementwise, every written slot, every other slot bitwise)."""
    prob = make_workload(name)
    print(f"\n{name} (short_path_max {short_max}): T={prob['total_len']} batch={prob['batch']}", flush=True)
    wy, wf = full_check(prob, short_max)
    print(f"{name}: every sequence: y worst/bound {wy:.3f}  final rel {wf:.2e}", flush=True)


# ------------------------------------------------- bf16 state storage

@pytest.mark.parametrize("name", ["n256_chunked", "n128_mixed_short", "n64_edges"])
def test_bf16_states_match_oracle(name):
    """bf16 pool: initial states read as their bf16 values, final states
    within FINAL_TOL_BF16 of the fp64 oracle, untouched slots bitwise."""
    spec = {
        "n256_chunked": dict(seqlens=[1000, 5, 0], H=2, G=1, N=256, init="half"),
        "n128_mixed_short": dict(seqlens=MIXED_LENS, H=8, G=4, N=128, init="all"),
        "n64_edges": dict(seqlens=[0, 1, 255, 256, 257, 511], H=4, G=2, N=64, init="bernoulli"),
    }[name]
    lens = spec.pop("seqlens")
    prob = small_problem(lens, P=64, seed=300 + len(name), state_dtype="bf16", **spec)
    full_check(prob, binding.SHORT_PATH_LIMIT)


@pytest.mark.parametrize("route", ["default", "chunked"])
def test_bf16_states_are_rounded_fp32_results(route):
    """With the same (bf16-representable) initial states, the bf16-storage
    run's final states are the fp32-storage run's, rounded to nearest even,
    bit for bit: the arithmetic is the same, only the store differs."""
    from mamba_ssd_chunked_chunk_amd.workloads import with_bf16_states
    prob = small_problem([300, 40, 0, 96, 700], H=4, P=64, G=2, N=128, seed=310, init="bernoulli")
    pb = with_bf16_states(prob)
    pf = clone(prob)
    pf["pool"] = bf16_to_f64(pb["pool"]).astype(np.float32)  # exactly the bf16 values
    sm = DEFAULT if route == "default" else CHUNKED
    df, _ = gpu_run(pf, sm)
    db, _ = gpu_run(pb, sm)
    assert torch.equal(bits(db["y"]), bits(df["y"]))
    assert torch.equal(bits(db["pool"]), bits(df["pool"].to(torch.bfloat16)))


def test_bf16_states_separate_entry():
    prob = small_problem([300, 0, 513, 17], H=4, P=64, G=2, N=128, seed=320, init="none")
    init = random_states(prob, 321)
    init_b = torch.from_numpy(init).to(torch.bfloat16)
    init_exact = init_b.float().numpy()
    d = torch_io.upload(prob, "cuda")
    fin = torch.full(init_b.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    torch_io.run_fwd(d, init_b.cuda(), fin, short_path_max=binding.SHORT_PATH_LIMIT)
    torch.cuda.synchronize()
    ref = oracle.recurrence_separate(prob, init_exact)
    assert_y(y_host(d), ref["y"], "bf16 separate")
    fh = fin.float().cpu().numpy()
    for b in range(4):
        assert_final(fh[b], ref["final"][b], f"seq {b}", FINAL_TOL_BF16)
    assert torch.equal(bits(fin[1].cpu()), bits(init_b[1]))  # zero-length: the initial state


@pytest.mark.parametrize("name", ["short_512_h128_g8_n128", "decode_512_h128_g8_n128"])
def test_bf16_states_workloads_full_size(name):
    from mamba_ssd_chunked_chunk_amd.workloads import with_bf16_states
    prob = with_bf16_states(make_workload(name))
    wy, wf = full_check(prob)
    print(f"{name}, bf16 states, every sequence: y worst/bound {wy:.3f}  final rel {wf:.2e}", flush=True)


# ------------------------------------------- token recurrence (decode steps)

@pytest.mark.parametrize("N,state_dtype", [(64, "f32"), (128, "f32"), (128, "bf16")])
def test_recur_path_lengths(N, state_dtype):
    """Sequences of 1..4 tokens take the token recurrence, 5 and more the
    MFMA short kernel: lengths on both sides of that boundary, with and
    without initial states, against the oracle."""
    lens = [1, 2, 3, 4, 5, 6, 9, 0, 1, 4]
    prob = small_problem(lens, H=4, P=64, G=2, N=N, seed=400 + N, init="bernoulli", state_dtype=state_dtype)
    full_check(prob, binding.SHORT_PATH_LIMIT)


def test_recur_limit_follows_short_limit():
    """With the short path limited to 2 tokens, the recurrence takes 1..2 and
    the chunked steps the rest (the chunk count checked)."""
    lens = [1, 2, 3, 8, 30]
    prob = small_problem(lens, H=4, P=64, G=1, N=128, seed=410, init="all")
    d, ws = gpu_run(prob, 2)
    ref = oracle.recurrence(prob, want_pool=False)
    assert_y(y_host(d), ref["y"], "limit 2")
    for b, slot in enumerate(prob["cache_indices"]):
        assert_final(d["pool"][int(slot)].cpu().numpy(), ref["final"][b], f"seq {b}")
    L = binding.ssd_workspace_get_layout(torch_io.problem_struct(d))
    assert int(ws.cpu().numpy()[L["meta"]:L["meta"] + 4].view(np.int32)[0]) == 3


# ------------------------------------------------------- HIP graph capture

@pytest.mark.parametrize("N,lens", [(128, MIXED_LENS), (256, [700, 300, 0, 45])])
def test_graph_capture_replays_match_eager(N, lens):
    """The call enqueues kernels only (no allocation, no memset, no host
    synchronisation), so it can be captured into a HIP graph.  Each replay
    (after the pool is restored by eager work) must equal the eager call,
    bit for bit, under the chunked and the short paths."""
    prob = small_problem(lens, H=4, P=64, G=2, N=N, seed=500 + N, init="bernoulli")
    d = torch_io.upload(prob, "cuda")
    pool0 = d["pool"].clone()
    ws = torch.empty(binding.ssd_workspace_size(torch_io.problem_struct(d)), dtype=torch.uint8, device="cuda")
    sm = binding.SHORT_PATH_LIMIT
    torch_io.run(d, ws, short_path_max=sm)
    torch.cuda.synchronize()
    y_ref, pool_ref = d["y"].clone(), d["pool"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        d["pool"].copy_(pool0)
        torch_io.run(d, ws, short_path_max=sm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    d["pool"].copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        torch_io.run(d, ws, short_path_max=sm)
    for rep in range(3):
        d["y"].zero_()
        d["pool"].copy_(pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(d["y"]), bits(y_ref)), f"replay {rep}: y differs"
        assert torch.equal(bits(d["pool"]), bits(pool_ref)), f"replay {rep}: pool differs"


# ------------------------------------- random tiny shapes (property test, GPU)

try:
    from hypothesis import given, settings, strategies as st
    HAVE_HYPOTHESIS = True
except ImportError:  # pragma: no cover
    HAVE_HYPOTHESIS = False

if HAVE_HYPOTHESIS:
    @settings(max_examples=24, deadline=None, derandomize=True, database=None)
    @given(lens=st.lists(st.one_of(st.integers(0, 8), st.integers(0, 700)), min_size=1, max_size=5),
           shape=st.sampled_from([(2, 1, 64), (4, 2, 64), (4, 4, 128), (8, 2, 128), (2, 1, 256), (4, 1, 256)]),
           init=st.sampled_from(["none", "all", "bernoulli"]),
           short_max=st.sampled_from([DEFAULT, CHUNKED, 1, 4, 33, 128]),
           state_dtype=st.sampled_from(["f32", "f32", "bf16"]),
           seed=st.integers(0, 2 ** 31 - 1))
    def test_random_tiny_shapes(lens, shape, init, short_max, state_dtype, seed):
        """A bounded number of random small problems (ragged lengths with
        empty and single-token sequences, every supported dstate, groups,
        initial states, short-path limits, state storage types) through the
        C ABI against the fp64 oracle."""
        H, G, N = shape
        prob = small_problem(lens, H=H, P=64, G=G, N=N, seed=seed, init=init, state_dtype=state_dtype)
        print(f"random case: lens={lens} H={H} G={G} N={N} init={init} short_max={short_max} "
              f"states={state_dtype} seed={seed}", flush=True)
        full_check(prob, short_max)
