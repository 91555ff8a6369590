"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ssd.h declares, reports its version and status names,
sizes its workspace, and rejects malformed calls before launching anything
(only error paths that return before any HIP call are exercised here)."""

import ctypes
import os
import re

import pytest

from mamba_ssd_chunked_chunk_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert binding.ssd_abi_version() == binding.ABI_VERSION == 18
    for code, name in binding.STATUS_NAMES.items():
        assert lib.ssd_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.ssd_status_string(99)


def _prob(**kw):
    base = dict(total_len=1024, batch=4, nheads=16, head_dim=64, ngroups=1, dstate=256, max_slots=8)
    base.update(kw)
    return binding.make_problem(**base)


def test_workspace_layout_arithmetic(lib):
    """Offsets ascend, 256-byte aligned, each region holds its table; the
    tables have floor(T / 256) + (sequences the chunked steps can see) rows."""
    p = _prob()
    L = binding.ssd_workspace_get_layout(p)
    ncm = 1024 // 256 + 4  # dstate 256: no short path, all 4 sequences chunked
    assert L["nchunks_max"] == ncm
    assert L["total_bytes"] == binding.ssd_workspace_size(p)
    keys = ("meta", "chunk_off", "desc", "dts", "cs2", "cbt", "gexp", "states", "sexp", "hin",
            "hexp", "xexp", "seq_list", "recur_list")
    offs = [L[k] for k in keys]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    need = dict(meta=16, chunk_off=5 * 4, desc=ncm * 16, dts=ncm * 16 * 256 * 4, cs2=ncm * 16 * 256 * 4,
                cbt=ncm * 1 * 36 * 64 * 16 * 2, gexp=ncm * 1 * 4 * 4,
                states=ncm * 16 * 64 * 256 * 2, sexp=ncm * 16 * 2 * 8 * 4,
                hin=ncm * 16 * 64 * 256 * 2, hexp=ncm * 16 * 64 * 4,
                xexp=ncm * 16 * 2 * 4, seq_list=4 * 4, recur_list=4 * 4)
    ends = offs[1:] + [L["total_bytes"]]
    for k, o, e in zip(keys, offs, ends):
        assert e - o >= need[k], k
    # kernel sizes: no copies
    assert (L["core_nheads"], L["core_dstate"]) == (16, 256)
    for k in ("x_pad", "y_pad", "bc_pad", "head_wide", "state_pad"):
        assert L[k] == SIZE_MAX, k


SIZE_MAX = 2 ** (8 * ctypes.sizeof(ctypes.c_size_t)) - 1


def _up(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("P,N,state_dtype", [(96, 100, 0), (128, 256, 0), (64, 16, 1), (200, 64, 0), (32, 256, 1)])
def test_adapted_layout(lib, P, N, state_dtype):
    """Sizes the kernels do not take: the tables are the mapped problem's
    (ceil(P / 64) heads of 64 per head, dstate rounded up to 64 / 128 / 256),
    followed by the copies each size needs, 256-byte aligned and large
    enough, and the workspace ends with the last of them."""
    T, batch, H, G = 1000, 3, 8, 2
    kw = dict(total_len=T, batch=batch, nheads=H, head_dim=P, ngroups=G, dstate=N, max_slots=5,
              state_dtype=state_dtype)
    L = binding.ssd_workspace_get_layout(_prob(**kw))
    m = (P + 63) // 64
    Np = 64 if N <= 64 else 128 if N <= 128 else 256
    assert (L["core_nheads"], L["core_dstate"]) == (H * m, Np)
    # the tables: those of the mapped problem (one slot per sequence when states are padded)
    core = binding.ssd_workspace_get_layout(_prob(**dict(kw, nheads=H * m, head_dim=64, dstate=Np,
                                                         max_slots=batch if (P % 64 or N != Np) else 5)))
    for k in ("nchunks_max", "meta", "chunk_off", "desc", "dts", "cs2", "cbt", "gexp", "states", "sexp",
              "hin", "hexp", "xexp", "seq_list", "recur_list"):
        assert L[k] == core[k], k
    es = 2 if state_dtype == 1 else 4
    need = dict(x_pad=T * H * 64 * m * 2 if P % 64 else None,
                y_pad=T * H * 64 * m * 2 if P % 64 else None,
                bc_pad=2 * _up(T * G * Np * 2) if N != Np else None,
                head_wide=_up(T * H * m * 4) + 3 * _up(H * m * 4) if m > 1 else None,
                state_pad=batch * H * 64 * m * Np * es if (P % 64 or N != Np) else None)
    prev_end = core["total_bytes"]
    for k in ("x_pad", "y_pad", "bc_pad", "head_wide", "state_pad"):
        if need[k] is None:
            assert L[k] == SIZE_MAX, k
            continue
        assert L[k] % 256 == 0 and L[k] >= prev_end, k
        prev_end = L[k] + need[k]
    assert L["total_bytes"] == _up(prev_end) == binding.ssd_workspace_size(_prob(**kw))


def test_workspace_rows_follow_the_routing(lib):
    """With the short path on (dstate <= 128) only sequences longer than its
    limit reach the chunked steps, at most T / (limit + 1) of them: the
    tables get floor(T / 256) + that many rows."""
    kw = dict(total_len=512, batch=512, nheads=128, dstate=128, ngroups=8, max_slots=1024)
    assert binding.ssd_workspace_get_layout(_prob(**kw))["nchunks_max"] == 2 + 512 // 129
    assert binding.ssd_workspace_get_layout(_prob(short_path_max=4, **kw))["nchunks_max"] == 2 + 512 // 5
    assert binding.ssd_workspace_get_layout(_prob(short_path_max=0, **kw))["nchunks_max"] == 2 + 512
    # at dstate 256 the limit is ignored
    assert (binding.ssd_workspace_get_layout(_prob(short_path_max=0)) ==
            binding.ssd_workspace_get_layout(_prob(short_path_max=128)))


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(nheads=6, ngroups=4), 2), (dict(total_len=-1), 2),
    (dict(max_slots=0), 2), (dict(dstate=0), 2), (dict(head_dim=0), 2), (dict(dstate=257), 3),
    (dict(dstate=512), 3), (dict(head_dim=1025), 3), (dict(nheads=32768, head_dim=65), 3),
    (dict(chunk_size=128), 3), (dict(state_dtype=2), 3), (dict(state_dtype=-1), 3),
    (dict(short_path_max=129), 3), (dict(short_path_max=1 << 20), 3),
])
def test_bad_problems_rejected(lib, kw, status):
    n = ctypes.c_size_t(0)
    assert lib.ssd_workspace_size(ctypes.byref(_prob(**kw)), ctypes.byref(n)) == status


def test_null_and_workspace_errors_before_launch(lib):
    p = _prob()
    f = lib.ssd_chunk_scan_varlen_fwd_inplace
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    args = [fake] * 13
    need = binding.ssd_workspace_size(p)
    # NULL problem
    assert f(None, *args, need, None) == 1
    # each required pointer NULL in turn (y, x, dt, A, B, C, pool, qsl, cache_indices)
    for idx in (0, 1, 2, 3, 4, 5, 8, 9, 11):
        a = list(args)
        a[idx] = None
        assert f(ctypes.byref(p), *a, need, None) == 1, idx
    # workspace: NULL, too small, misaligned
    a = list(args)
    a[12] = None
    assert f(ctypes.byref(p), *a, need, None) == 4
    assert f(ctypes.byref(p), *args, need - 1, None) == 4
    a = list(args)
    a[12] = ctypes.c_void_p((1 << 20) + 16)
    assert f(ctypes.byref(p), *a, need, None) == 4
    # misaligned bf16 tensor
    a = list(args)
    a[1] = ctypes.c_void_p((1 << 20) + 2)
    assert f(ctypes.byref(p), *a, need, None) == 7
    # optional D / dt_bias / has_initial_state may be NULL: the call then only
    # fails on the (deliberately too small) workspace
    a = list(args)
    a[6] = a[7] = a[10] = None
    assert f(ctypes.byref(p), *a, need - 1, None) == 4


def test_separate_states_errors_before_launch(lib):
    p = _prob()
    f = lib.ssd_chunk_scan_varlen_fwd
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    args = [fake] * 12  # y x dt A B C D dt_bias initial final qsl workspace
    need = binding.ssd_workspace_size(p)
    assert f(None, *args, need, None) == 1
    # each required pointer NULL in turn (y, x, dt, A, B, C, final_states, qsl)
    for idx in (0, 1, 2, 3, 4, 5, 9, 10):
        a = list(args)
        a[idx] = None
        assert f(ctypes.byref(p), *a, need, None) == 1, idx
    # misaligned state tensors
    for idx in (8, 9):
        a = list(args)
        a[idx] = ctypes.c_void_p((1 << 20) + 8)
        assert f(ctypes.byref(p), *a, need, None) == 7, idx
    # workspace too small; optional D, dt_bias and initial_states may be NULL
    a = list(args)
    a[6] = a[7] = a[8] = None
    assert f(ctypes.byref(p), *a, need - 1, None) == 4
    # the profiled form checks its events first
    g = lib.ssd_chunk_scan_varlen_fwd_profiled
    assert g(ctypes.byref(p), *args, need, None, None, 5) == 1
    ev = (ctypes.c_void_p * 5)(*([fake] * 5))
    assert g(ctypes.byref(p), *args, need, None, ev, 4) == 2


def test_validate_inputs_host_errors(lib):
    assert lib.ssd_validate_inputs(None, None, None, None) == 1
    p = _prob()
    assert lib.ssd_validate_inputs(ctypes.byref(p), None, None, None) == 1
    assert lib.ssd_validate_inputs(ctypes.byref(_prob(batch=0)), None, None, None) == 2


def test_state_dtype_accepted_and_layout_unchanged(lib):
    """bf16 state storage is a valid problem and does not change the
    workspace (the intermediates are the same either way)."""
    a = binding.ssd_workspace_get_layout(_prob())
    b = binding.ssd_workspace_get_layout(_prob(state_dtype=binding.STATE_BF16))
    assert a == b


@pytest.mark.parametrize("idx,misalign", [
    # y, x, B, C, ssm_pool: 16 bytes (offsets 2 and 8 both break it)
    (0, 2), (1, 8), (4, 2), (5, 8), (8, 8), (8, 4),
    # dt, A, D, dt_bias, query_start_loc, cache_indices: 4 bytes
    (2, 2), (3, 1), (6, 2), (7, 2), (9, 2), (11, 1),
])
def test_alignment_status(lib, idx, misalign):
    """Each tensor pointer that breaks the documented alignment gives
    SSD_ERR_MISALIGNED before anything is launched; aligned pointers reach
    the (deliberately too small) workspace check instead."""
    p = _prob()
    f = lib.ssd_chunk_scan_varlen_fwd_inplace
    base = 1 << 20  # never dereferenced: every call below fails its host checks
    args = [ctypes.c_void_p(base)] * 13
    need = binding.ssd_workspace_size(p)
    a = list(args)
    a[idx] = ctypes.c_void_p(base + misalign)
    assert f(ctypes.byref(p), *a, need, None) == 7
    assert lib.ssd_status_string(7).decode().startswith("SSD_ERR_MISALIGNED")
    # has_initial_state is bytes: any address is aligned
    a = list(args)
    a[10] = ctypes.c_void_p(base + 1)
    assert f(ctypes.byref(p), *a, need - 1, None) == 4


def test_short_path_limit_is_a_problem_field(lib):
    """The short-path limit is part of each call's problem (no library
    state): negative selects the default, 0..SSD_SHORT_PATH_LIMIT are valid,
    larger values are rejected; the kernel list names the two short-path
    kernels last."""
    n128 = dict(dstate=128, nheads=16)
    for v in (-1, -100):
        assert (binding.ssd_workspace_get_layout(_prob(short_path_max=v, **n128)) ==
                binding.ssd_workspace_get_layout(_prob(short_path_max=binding.SHORT_PATH_LIMIT, **n128)))
    for v in (0, 1, 4, 64, binding.SHORT_PATH_LIMIT):
        assert binding.ssd_workspace_size(_prob(short_path_max=v, **n128)) > 0
    n = ctypes.c_size_t(0)
    assert lib.ssd_workspace_size(ctypes.byref(_prob(short_path_max=binding.SHORT_PATH_LIMIT + 1)),
                                  ctypes.byref(n)) == 3
    assert not hasattr(binding, "ssd_set_short_path_max")
    names = [lib.ssd_kernel_name(i).decode() for i in range(lib.ssd_kernel_count())]
    assert names == ["ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan", "ssd_short", "ssd_recur"]


def test_noalloc_entry_host_errors(lib):
    """The no-allocation entry point runs every host check before it looks up
    its scratch: a problem whose workspace exceeds SSD_NOALLOC_SCRATCH_BYTES
    gives SSD_ERR_SCRATCH, NULL and misaligned pointers their own statuses."""
    f = lib.ssd_chunk_scan_varlen_fwd_inplace_noalloc
    base = 1 << 20  # never dereferenced: every call below fails its host checks
    args = [ctypes.c_void_p(base)] * 12
    big = _prob(total_len=8 * 4096, batch=8)  # 8 x 4096 tokens, 16 heads, dstate 256
    assert binding.ssd_workspace_size(big) > binding.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), *args, None) == 8
    assert lib.ssd_status_string(8).decode().startswith("SSD_ERR_SCRATCH")
    assert f(None, *args, None) == 1
    a = list(args)
    a[8] = None  # ssm_pool
    assert f(ctypes.byref(_prob()), *a, None) == 1
    a = list(args)
    a[1] = ctypes.c_void_p(base + 2)  # x
    assert f(ctypes.byref(_prob()), *a, None) == 7
