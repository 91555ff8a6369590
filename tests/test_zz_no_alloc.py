"""The no-allocation entry point (ssd_chunk_scan_varlen_fwd_inplace_noalloc)
through the C ABI: the intermediates live in the library's own per-GPU
scratch array instead of a caller workspace.  Its outputs must equal those
of the workspace entry point on the same inputs, bit for bit (both run the
same kernels on the same values), on consecutive calls whose second problem
is smaller than the first (the scratch keeps the first call's contents), and
both must match the fp64 oracle."""

import numpy as np
import pytest

import oracle
from ssd_testlib import frob_rel, small_problem

torch = pytest.importorskip("torch")
from mamba_ssd_chunked_chunk_amd import binding, torch_io  # noqa: E402

pytestmark = pytest.mark.gpu


def _noalloc(d, short_max):
    binding.ssd_chunk_scan_varlen_fwd_inplace_noalloc(
        d["y"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dt_bias"], d["pool"],
        d["query_start_loc"], d["has_initial_state"], d["cache_indices"], dt_softplus=d["dt_softplus"],
        short_path_max=short_max)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("short_max", [binding.SHORT_PATH_DEFAULT, 0])
def test_noalloc_equals_workspace_entry_on_consecutive_calls(short_max):
    big = small_problem([700, 0, 300, 45, 257], H=4, P=64, G=2, N=128, max_slots=8, seed=801, init="bernoulli")
    small = small_problem([90, 300], H=2, P=64, G=1, N=256, max_slots=3, seed=802, init="all")
    for prob in (big, small):  # the second call is smaller than the first
        ps = binding.make_problem(prob["total_len"], prob["batch"], prob["nheads"], 64, prob["ngroups"],
                                  prob["dstate"], prob["pool"].shape[0])
        assert binding.ssd_workspace_size(ps) <= binding.NOALLOC_SCRATCH_BYTES
        d_ref = torch_io.upload(prob, "cuda")
        d = torch_io.upload(prob, "cuda")
        d["y"].fill_(float("nan"))
        torch_io.run(d_ref, short_path_max=short_max)
        _noalloc(d, short_max)
        torch.cuda.synchronize()
        assert torch.equal(_bits(d["y"]), _bits(d_ref["y"])), prob["seqlens"]
        assert torch.equal(_bits(d["pool"]), _bits(d_ref["pool"])), prob["seqlens"]
        ref = oracle.recurrence(prob, want_pool=False)
        y = d["y"].float().cpu().numpy().astype(np.float64)
        assert np.max(np.abs(y - ref["y"]) / (2e-2 * (1.0 + np.abs(ref["y"])))) <= 1.0
        for b, slot in enumerate(prob["cache_indices"]):
            assert frob_rel(d["pool"][int(slot)].cpu().numpy(), ref["final"][b]) <= 1e-3


def test_noalloc_rejects_problems_beyond_its_scratch():
    """A problem whose workspace exceeds the scratch array is refused before
    anything is launched: the outputs and the pool keep their bits."""
    prob = small_problem([4096] * 8, H=16, P=64, G=1, N=256, max_slots=9, seed=803, init="none")
    ps = binding.make_problem(prob["total_len"], 8, 16, 64, 1, 256, 9)
    assert binding.ssd_workspace_size(ps) > binding.NOALLOC_SCRATCH_BYTES
    d = torch_io.upload(prob, "cuda")
    d["y"].fill_(3.0)
    pool0 = d["pool"].clone()
    with pytest.raises(binding.SsdError) as e:
        _noalloc(d, binding.SHORT_PATH_DEFAULT)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((d["y"] == 3.0).all()) and torch.equal(_bits(d["pool"]), _bits(pool0))
