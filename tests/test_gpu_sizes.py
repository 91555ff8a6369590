"""GPU parity for sizes the scan kernels do not take directly: any dstate up to
256 ("mamba2_ssd_scan", comptime MAX_DSTATE) and any head_dim up to 1024.
The call maps them onto head_dim 64 and dstate 64 / 128 / 256 through padded
copies; the oracle takes every size as it is.  Same bars as the other parity
tests, and bitwise agreement with the same problem padded by hand to the
kernels' sizes."""

import numpy as np
import pytest

import oracle
from ssd_testlib import pad_by_hand, small_problem
from test_gpu_parity import (CHUNKED, DEFAULT, assert_final, assert_y, full_check, random_states,
                             run_separate, y_host)

torch = pytest.importorskip("torch")
from mamba_ssd_chunked_chunk_amd import binding, torch_io  # noqa: E402

pytestmark = pytest.mark.gpu

SIZES = {
    # dstate padded (B, C and the states through copies)
    "n16_p64": dict(seqlens=[0, 1, 5, 100, 300, 700], H=4, P=64, G=2, N=16, init="bernoulli"),
    "n96_p64": dict(seqlens=[257, 33, 600, 2], H=4, P=64, G=2, N=96, init="all"),
    "n200_p64": dict(seqlens=[800, 40, 0], H=2, P=64, G=1, N=200, init="half"),
    # head_dim a multiple of 64: two heads of 64 per head, no copy of x, y or the states
    "n128_p128": dict(seqlens=[300, 17, 520], H=4, P=128, G=2, N=128, init="all"),
    "n256_p192": dict(seqlens=[600, 3], H=2, P=192, G=1, N=256, init="all"),
    # head_dim padded (x and y through copies), alone and with dstate
    "n128_p32": dict(seqlens=[513, 50], H=4, P=32, G=4, N=128, init="all"),
    "n64_p96": dict(seqlens=[90, 400, 1], H=2, P=96, G=1, N=64, init="bernoulli"),
    "n48_p200": dict(seqlens=[260, 70], H=2, P=200, G=1, N=48, init="all"),
    "n1_p1": dict(seqlens=[5, 300], H=2, P=1, G=1, N=1, init="all"),
    # the largest head_dim: sixteen heads of 64 per head
    "n32_p1024": dict(seqlens=[300, 9], H=1, P=1024, G=1, N=32, init="all"),
    # bf16 state storage through the padded area
    "n100_p64_bf16": dict(seqlens=[300, 20, 0, 64], H=4, P=64, G=2, N=100, init="all", state_dtype="bf16"),
}


@pytest.mark.parametrize("route", ["default", "chunked"])
@pytest.mark.parametrize("name", list(SIZES))
def test_sizes_match_oracle(name, route):
    """Every sequence against the oracle, every written slot, every other
    slot bit-identical; with the default routing and all sequences chunked."""
    spec = dict(SIZES[name])
    lens = spec.pop("seqlens")
    prob = small_problem(lens, seed=300 + len(name), max_slots=len(lens) + 3, **spec)
    wy, wf = full_check(prob, DEFAULT if route == "default" else CHUNKED)
    print(f"{name} ({route}): y worst/bound {wy:.3f}  final rel {wf:.2e}", flush=True)


@pytest.mark.parametrize("name", ["n96_p64", "n64_p96", "n48_p200", "n128_p128"])
def test_sizes_equal_padding_by_hand(name):
    """The mapped call gives the values of the hand-padded problem run at the
    kernels' sizes, exactly (every sequence has an initial state, so both
    runs take the same steps)."""
    spec = dict(SIZES[name], init="all")
    lens = spec.pop("seqlens")
    prob = small_problem(lens, seed=400 + len(name), max_slots=len(lens) + 2, **spec)
    q = pad_by_hand(prob)
    H, P, N = prob["nheads"], prob["head_dim"], prob["dstate"]
    T = int(prob["query_start_loc"][-1])
    m = q["nheads"] // H
    d1 = torch_io.upload(prob, "cuda")
    d2 = torch_io.upload(q, "cuda")
    torch_io.run(d1)
    torch_io.run(d2)
    torch.cuda.synchronize()
    y1 = d1["y"].float().cpu().numpy()
    y2 = d2["y"].float().cpu().numpy().reshape(T, H, 64 * m)[:, :, :P]
    assert np.array_equal(y1, y2)
    ci = prob["cache_indices"].astype(np.int64)
    f1 = d1["pool"].float().cpu().numpy()[ci]
    f2 = d2["pool"].float().cpu().numpy().reshape(-1, H, 64 * m, q["dstate"])[ci][:, :, :P, :N]
    assert np.array_equal(f1, f2)


@pytest.mark.parametrize("with_init", [True, False], ids=["initial", "zero"])
def test_sizes_separate_states(with_init):
    """The entry point with separate initial and final states at a padded
    head_dim and dstate."""
    prob = small_problem([300, 0, 513, 17], H=2, P=96, G=1, N=100, seed=471, init="none")
    init = random_states(prob, 172) if with_init else None
    d, fin = run_separate(prob, init)
    ref = oracle.recurrence_separate(prob, init)
    assert_y(y_host(d), ref["y"], "separate states")
    fh = fin.cpu().numpy()
    for b in range(4):
        assert_final(fh[b], ref["final"][b], f"seq {b}")
    want = init[1] if with_init else np.zeros_like(fh[1])
    assert np.array_equal(fh[1].view(np.uint32), want.view(np.uint32))


def test_sizes_noalloc_equals_workspace_entry():
    """The entry point without a workspace takes the same mapping (its
    scratch holds the copies too)."""
    spec = dict(SIZES["n64_p96"])
    lens = spec.pop("seqlens")
    prob = small_problem(lens, seed=481, max_slots=len(lens) + 2, **spec)
    d1 = torch_io.upload(prob, "cuda")
    d2 = torch_io.upload(prob, "cuda")
    torch_io.run(d1)
    binding.ssd_chunk_scan_varlen_fwd_inplace_noalloc(
        d2["y"], d2["x"], d2["dt"], d2["A"], d2["B"], d2["C"], d2["D"], d2["dt_bias"], d2["pool"],
        d2["query_start_loc"], d2["has_initial_state"], d2["cache_indices"], dt_softplus=d2["dt_softplus"])
    torch.cuda.synchronize()
    assert torch.equal(d1["y"].view(torch.int16), d2["y"].view(torch.int16))
    assert torch.equal(d1["pool"].view(torch.int32), d2["pool"].view(torch.int32))


def test_many_tiny_sequences():
    """3000 sequences of 0..8 tokens (the token recurrence, the short kernel
    and empty sequences) in one call, every one against the oracle."""
    lens = list(np.random.default_rng(9).integers(0, 9, 3000))
    prob = small_problem(lens, H=4, P=64, G=2, N=64, seed=491, max_slots=3100, init="bernoulli")
    wy, wf = full_check(prob)
    print(f"3000 tiny sequences: y worst/bound {wy:.3f}  final rel {wf:.2e}", flush=True)


def test_sizes_profiled_entry():
    """The entry point with per-kernel events (the one bench.py times) takes
    the same mapping: results bitwise those of the plain entry point, and the
    events span the call."""
    import bench
    spec = dict(SIZES["n64_p96"])
    lens = spec.pop("seqlens")
    prob = small_problem(lens, seed=493, max_slots=len(lens) + 2, **spec)
    hip = bench.Hip()
    run = bench.Runner(torch, binding.load_library(), hip, torch.device("cuda:0"), prob, bench.SHORT_MAX)
    events = [hip.event() for _ in range(run.nk + 1)]
    run.call(events)
    d = torch_io.upload(prob, "cuda")
    torch_io.run(d)
    torch.cuda.synchronize()
    assert torch.equal(run.d["y"].view(torch.int16), d["y"].view(torch.int16))
    assert torch.equal(run.d["pool"].view(torch.int32), d["pool"].view(torch.int32))
    assert hip.elapsed_ms(events[0], events[run.nk]) > 0.0
