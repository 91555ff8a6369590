"""Move a host problem (NumPy arrays from ``workloads``) to device tensors and
call the library on it.  Plumbing only: no arithmetic of the scan."""

from __future__ import annotations

import numpy as np

from . import binding


def upload(prob: dict, device="cuda"):
    """Copy the problem's arrays to ``device``; returns a dict of tensors."""
    import torch

    def t(a, dtype=None):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    H, P, G, N = prob["nheads"], prob["head_dim"], prob["ngroups"], prob["dstate"]
    T = int(prob["query_start_loc"][-1])
    d = dict(
        x=t(prob["x"].reshape(T, H, P)).view(torch.bfloat16),
        dt=t(prob["dt"].reshape(T, H)),
        A=t(prob["A"]),
        B=t(prob["B"].reshape(T, G, N)).view(torch.bfloat16),
        C=t(prob["C"].reshape(T, G, N)).view(torch.bfloat16),
        D=t(prob.get("D")),
        dt_bias=t(prob.get("dt_bias")),
        pool=(t(prob["pool"]).view(torch.bfloat16) if prob.get("state_dtype", "f32") == "bf16"
              else t(prob["pool"])),
        query_start_loc=t(prob["query_start_loc"].astype(np.int32)),
        has_initial_state=t(prob.get("has_initial_state")),
        cache_indices=t(prob["cache_indices"].astype(np.int32)),
        dt_softplus=bool(prob.get("dt_softplus", True)),
    )
    d["y"] = torch.empty((T, H, P), dtype=torch.bfloat16, device=device)
    return d


def run(d: dict, workspace=None, stream=None, short_path_max=binding.SHORT_PATH_DEFAULT):
    """One call of the in-place scan on an uploaded problem (asynchronous)."""
    return binding.ssd_chunk_scan_varlen_fwd_inplace(
        d["y"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dt_bias"], d["pool"],
        d["query_start_loc"], d["has_initial_state"], d["cache_indices"],
        dt_softplus=d["dt_softplus"], short_path_max=short_path_max, workspace=workspace, stream=stream)


def run_fwd(d: dict, initial_states, final_states, workspace=None, stream=None,
            short_path_max=binding.SHORT_PATH_DEFAULT):
    """One call of the scan with separate initial/final states (asynchronous)."""
    return binding.ssd_chunk_scan_varlen_fwd(
        d["y"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dt_bias"], initial_states,
        final_states, d["query_start_loc"], dt_softplus=d["dt_softplus"], short_path_max=short_path_max,
        workspace=workspace, stream=stream)


def problem_struct(d: dict, short_path_max=binding.SHORT_PATH_DEFAULT):
    T, H, P = d["x"].shape
    G, N = d["B"].shape[1], d["B"].shape[2]
    import torch
    return binding.make_problem(T, d["query_start_loc"].numel() - 1, H, P, G, N,
                                d["pool"].shape[0], d["dt_softplus"],
                                state_dtype=(binding.STATE_BF16 if d["pool"].dtype == torch.bfloat16
                                             else binding.STATE_F32),
                                short_path_max=short_path_max)
