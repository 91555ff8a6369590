"""Thin ctypes binding of libssd's C ABI (include/ssd.h).

Argument marshalling only: shapes, dtypes, devices and contiguity of torch
tensors are checked, then raw device pointers and the current HIP stream are
handed to the library.  Every step of the scan runs in the library's HIP
kernels; there is no fallback of any kind.  torch only provides device memory
(including the workspace) and the stream.
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_OK = 0
STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL_ARG", 2: "SSD_ERR_BAD_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
                4: "SSD_ERR_WORKSPACE", 5: "SSD_ERR_BAD_INPUT", 6: "SSD_ERR_HIP", 7: "SSD_ERR_MISALIGNED",
                8: "SSD_ERR_SCRATCH"}

# every symbol include/ssd.h declares
EXPORTED = ("ssd_abi_version", "ssd_status_string", "ssd_workspace_size",
            "ssd_workspace_get_layout", "ssd_chunk_scan_varlen_fwd_inplace",
            "ssd_kernel_count", "ssd_kernel_name", "ssd_chunk_scan_varlen_fwd_inplace_profiled",
            "ssd_chunk_scan_varlen_fwd", "ssd_chunk_scan_varlen_fwd_profiled", "ssd_validate_inputs",
            "ssd_chunk_scan_varlen_fwd_inplace_noalloc")


class SsdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class ssd_problem(ctypes.Structure):
    _fields_ = [("total_len", ctypes.c_int64), ("batch", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("max_slots", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("dt_softplus", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("short_path_max", ctypes.c_int32)]


class ssd_workspace_layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("nchunks_max", ctypes.c_int64),
                ("meta", ctypes.c_size_t), ("chunk_off", ctypes.c_size_t),
                ("desc", ctypes.c_size_t), ("dts", ctypes.c_size_t), ("cs2", ctypes.c_size_t),
                ("cbt", ctypes.c_size_t), ("gexp", ctypes.c_size_t),
                ("states", ctypes.c_size_t), ("sexp", ctypes.c_size_t),
                ("hin", ctypes.c_size_t), ("hexp", ctypes.c_size_t), ("xexp", ctypes.c_size_t),
                ("seq_list", ctypes.c_size_t), ("recur_list", ctypes.c_size_t),
                ("core_nheads", ctypes.c_int32), ("core_dstate", ctypes.c_int32),
                ("x_pad", ctypes.c_size_t), ("y_pad", ctypes.c_size_t), ("bc_pad", ctypes.c_size_t),
                ("head_wide", ctypes.c_size_t), ("state_pad", ctypes.c_size_t)]


_lock = threading.Lock()
_lib = None

# SSD_ABI_VERSION of include/ssd.h that the ctypes structures below mirror
ABI_VERSION = 18
NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES
STATE_F32, STATE_BF16 = 0, 1  # SSD_STATE_F32, SSD_STATE_BF16
SHORT_PATH_LIMIT = 128  # SSD_SHORT_PATH_LIMIT
MAX_DSTATE, MAX_HEAD_DIM = 256, 1024  # SSD_MAX_DSTATE, SSD_MAX_HEAD_DIM
SHORT_PATH_DEFAULT = -1  # ssd_problem.short_path_max: any negative value selects SHORT_PATH_LIMIT


def load_library():
    """Load libssd.so; raises if it has not been built (no fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it first "
                    "(python -m mamba_ssd_chunked_chunk_amd.build)")
            lib = ctypes.CDLL(LIB_PATH)
            V = ctypes.c_void_p
            PP = ctypes.POINTER(ssd_problem)
            lib.ssd_abi_version.restype = ctypes.c_int
            lib.ssd_abi_version.argtypes = []
            if lib.ssd_abi_version() != ABI_VERSION:
                raise RuntimeError(f"{LIB_PATH} has ABI version {lib.ssd_abi_version()}, the binding "
                                   f"expects {ABI_VERSION}: rebuild it")
            lib.ssd_status_string.restype = ctypes.c_char_p
            lib.ssd_status_string.argtypes = [ctypes.c_int]
            lib.ssd_workspace_size.restype = ctypes.c_int
            lib.ssd_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
            lib.ssd_workspace_get_layout.restype = ctypes.c_int
            lib.ssd_workspace_get_layout.argtypes = [PP, ctypes.POINTER(ssd_workspace_layout)]
            lib.ssd_chunk_scan_varlen_fwd_inplace.restype = ctypes.c_int
            lib.ssd_chunk_scan_varlen_fwd_inplace.argtypes = [PP] + [V] * 13 + [ctypes.c_size_t, V]
            lib.ssd_kernel_count.restype = ctypes.c_int
            lib.ssd_kernel_count.argtypes = []
            lib.ssd_kernel_name.restype = ctypes.c_char_p
            lib.ssd_kernel_name.argtypes = [ctypes.c_int]
            lib.ssd_chunk_scan_varlen_fwd_inplace_profiled.restype = ctypes.c_int
            lib.ssd_chunk_scan_varlen_fwd_inplace_profiled.argtypes = (
                [PP] + [V] * 13 + [ctypes.c_size_t, V, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int])
            lib.ssd_chunk_scan_varlen_fwd.restype = ctypes.c_int
            lib.ssd_chunk_scan_varlen_fwd.argtypes = [PP] + [V] * 12 + [ctypes.c_size_t, V]
            lib.ssd_chunk_scan_varlen_fwd_profiled.restype = ctypes.c_int
            lib.ssd_chunk_scan_varlen_fwd_profiled.argtypes = (
                [PP] + [V] * 12 + [ctypes.c_size_t, V, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int])
            lib.ssd_chunk_scan_varlen_fwd_inplace_noalloc.restype = ctypes.c_int
            lib.ssd_chunk_scan_varlen_fwd_inplace_noalloc.argtypes = [PP] + [V] * 12 + [V]
            lib.ssd_validate_inputs.restype = ctypes.c_int
            lib.ssd_validate_inputs.argtypes = [PP, V, V, V]
            _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != SSD_OK:
        lib = load_library()
        msg = lib.ssd_status_string(status).decode()
        raise SsdError(status, f"{what}: {msg}")


def make_problem(total_len, batch, nheads, head_dim, ngroups, dstate, max_slots,
                 dt_softplus=True, chunk_size=0, state_dtype=STATE_F32,
                 short_path_max=SHORT_PATH_DEFAULT) -> ssd_problem:
    return ssd_problem(int(total_len), int(batch), int(nheads), int(head_dim), int(ngroups),
                       int(dstate), int(max_slots), int(chunk_size), 1 if dt_softplus else 0,
                       int(state_dtype), int(short_path_max))


def _state_dtype(t, name):
    """SSD_STATE_* of a state tensor (fp32 or bf16)."""
    import torch
    if t.dtype == torch.float32:
        return STATE_F32
    if t.dtype == torch.bfloat16:
        return STATE_BF16
    raise TypeError(f"{name}: expected float32 or bfloat16 states, got {t.dtype}")


def ssd_abi_version() -> int:
    return load_library().ssd_abi_version()


def ssd_workspace_size(prob: ssd_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_workspace_size(ctypes.byref(prob), ctypes.byref(n)), "ssd_workspace_size")
    return n.value


def ssd_workspace_get_layout(prob: ssd_problem) -> dict:
    L = ssd_workspace_layout()
    _check(load_library().ssd_workspace_get_layout(ctypes.byref(prob), ctypes.byref(L)),
           "ssd_workspace_get_layout")
    return {name: getattr(L, name) for name, _ in ssd_workspace_layout._fields_}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return torch


def _opt(t, name, dtype, shape, device):
    if t is None or t.numel() == 0:
        return None
    _need(t, name, dtype, shape, device)
    return t


def problem_from_tensors(x, B, ssm_pool, query_start_loc, dt_softplus=True,
                         short_path_max=SHORT_PATH_DEFAULT) -> ssd_problem:
    T, H, P = x.shape
    _, G, N = B.shape
    return make_problem(T, query_start_loc.numel() - 1, H, P, G, N, ssm_pool.shape[0], dt_softplus,
                        state_dtype=_state_dtype(ssm_pool, "ssm_pool"), short_path_max=short_path_max)


def ssd_chunk_scan_varlen_fwd_inplace(y, x, dt, A, B, C, D, dt_bias, ssm_pool, query_start_loc,
                                      has_initial_state, cache_indices, *, dt_softplus=True,
                                      short_path_max=SHORT_PATH_DEFAULT, workspace=None, stream=None):
    """In-place varlen SSD forward (see include/ssd.h for the semantics).

    Tensors (torch, on one HIP device, contiguous): y, x bf16 [T,H,P];
    dt fp32 [T,H]; A fp32 [H]; B, C bf16 [T,G,N]; D, dt_bias fp32 [H] or
    None/empty; ssm_pool fp32 [S,H,P,N] (updated in place);
    query_start_loc int32 [batch+1]; has_initial_state uint8/bool [batch] or
    None/empty; cache_indices int32/uint32 [batch] (reinterpreted as uint32).
    ``workspace``: uint8 tensor of at least ssd_workspace_size() bytes, or
    None to allocate one.  Runs on ``stream`` (a torch.cuda.Stream) or the
    current stream; asynchronous.  Returns the workspace tensor.  A bf16
    ssm_pool selects bf16 state storage (arithmetic stays fp32).
    ``short_path_max``: longest sequence the short path takes (dstate <= 128;
    0: none, negative: the library default SHORT_PATH_LIMIT).
    """
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("libssd runs on a HIP device; got tensors on " + str(dev))
    T, H, P = x.shape
    if B.dim() != 3:
        raise ValueError("B must be [T, G, N]")
    G, N = B.shape[1], B.shape[2]
    batch = query_start_loc.numel() - 1
    S = ssm_pool.shape[0]
    _need(y, "y", torch.bfloat16, (T, H, P), dev)
    _need(x, "x", torch.bfloat16, (T, H, P), dev)
    _need(dt, "dt", torch.float32, (T, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", torch.bfloat16, (T, G, N), dev)
    _need(C, "C", torch.bfloat16, (T, G, N), dev)
    D = _opt(D, "D", torch.float32, (H,), dev)
    dt_bias = _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    sd = _state_dtype(ssm_pool, "ssm_pool")
    _need(ssm_pool, "ssm_pool", ssm_pool.dtype, (S, H, P, N), dev)
    _need(query_start_loc, "query_start_loc", torch.int32, (batch + 1,), dev)
    if has_initial_state is not None and has_initial_state.numel() > 0:
        if has_initial_state.dtype == torch.bool:
            has_initial_state = has_initial_state.view(torch.uint8)
        _need(has_initial_state, "has_initial_state", torch.uint8, (batch,), dev)
    else:
        has_initial_state = None
    if cache_indices.dtype not in (torch.int32, torch.uint32):
        raise TypeError("cache_indices must be int32 or uint32")
    if tuple(cache_indices.shape) != (batch,) or not cache_indices.is_contiguous() or cache_indices.device != dev:
        raise ValueError("cache_indices must be a contiguous [batch] tensor on the same device")
    prob = make_problem(T, batch, H, P, G, N, S, dt_softplus, state_dtype=sd, short_path_max=short_path_max)
    need = ssd_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.numel() < need or workspace.device != dev:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {dev}")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    status = load_library().ssd_chunk_scan_varlen_fwd_inplace(
        ctypes.byref(prob), _ptr(y), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(dt_bias), _ptr(ssm_pool), _ptr(query_start_loc), _ptr(has_initial_state),
        _ptr(cache_indices), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        ctypes.c_void_p(st.cuda_stream))
    _check(status, "ssd_chunk_scan_varlen_fwd_inplace")
    return workspace


def ssd_chunk_scan_varlen_fwd_inplace_noalloc(y, x, dt, A, B, C, D, dt_bias, ssm_pool, query_start_loc,
                                              has_initial_state, cache_indices, *, dt_softplus=True,
                                              short_path_max=SHORT_PATH_DEFAULT, stream=None):
    """The in-place operation without a workspace argument: the library's
    own scratch array (NOALLOC_SCRATCH_BYTES per GPU) holds the
    intermediates, and nothing is allocated.  Same tensors and checks as
    ssd_chunk_scan_varlen_fwd_inplace; calls that can overlap on one GPU race
    on the shared scratch (one stream orders them)."""
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("libssd runs on a HIP device; got tensors on " + str(dev))
    T, H, P = x.shape
    if B.dim() != 3:
        raise ValueError("B must be [T, G, N]")
    G, N = B.shape[1], B.shape[2]
    batch = query_start_loc.numel() - 1
    S = ssm_pool.shape[0]
    _need(y, "y", torch.bfloat16, (T, H, P), dev)
    _need(x, "x", torch.bfloat16, (T, H, P), dev)
    _need(dt, "dt", torch.float32, (T, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", torch.bfloat16, (T, G, N), dev)
    _need(C, "C", torch.bfloat16, (T, G, N), dev)
    D = _opt(D, "D", torch.float32, (H,), dev)
    dt_bias = _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    sd = _state_dtype(ssm_pool, "ssm_pool")
    _need(ssm_pool, "ssm_pool", ssm_pool.dtype, (S, H, P, N), dev)
    _need(query_start_loc, "query_start_loc", torch.int32, (batch + 1,), dev)
    if has_initial_state is not None and has_initial_state.numel() > 0:
        if has_initial_state.dtype == torch.bool:
            has_initial_state = has_initial_state.view(torch.uint8)
        _need(has_initial_state, "has_initial_state", torch.uint8, (batch,), dev)
    else:
        has_initial_state = None
    if cache_indices.dtype not in (torch.int32, torch.uint32):
        raise TypeError("cache_indices must be int32 or uint32")
    if tuple(cache_indices.shape) != (batch,) or not cache_indices.is_contiguous() or cache_indices.device != dev:
        raise ValueError("cache_indices must be a contiguous [batch] tensor on the same device")
    prob = make_problem(T, batch, H, P, G, N, S, dt_softplus, state_dtype=sd, short_path_max=short_path_max)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    status = load_library().ssd_chunk_scan_varlen_fwd_inplace_noalloc(
        ctypes.byref(prob), _ptr(y), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(dt_bias), _ptr(ssm_pool), _ptr(query_start_loc), _ptr(has_initial_state),
        _ptr(cache_indices), ctypes.c_void_p(st.cuda_stream))
    _check(status, "ssd_chunk_scan_varlen_fwd_inplace_noalloc")


def ssd_chunk_scan_varlen_fwd(y, x, dt, A, B, C, D, dt_bias, initial_states, final_states,
                              query_start_loc, *, dt_softplus=True, short_path_max=SHORT_PATH_DEFAULT,
                              workspace=None, stream=None):
    """Varlen SSD forward with separate initial and final states (see
    include/ssd.h): sequence b starts from ``initial_states[b]`` ([batch,H,P,N],
    or None/empty for zero) and its final state is written to
    ``final_states[b]`` ([batch,H,P,N]); both fp32, or both bf16 (bf16 state
    storage, arithmetic in fp32).  Other tensors as for
    ssd_chunk_scan_varlen_fwd_inplace.  Returns the workspace tensor.
    """
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("libssd runs on a HIP device; got tensors on " + str(dev))
    T, H, P = x.shape
    if B.dim() != 3:
        raise ValueError("B must be [T, G, N]")
    G, N = B.shape[1], B.shape[2]
    batch = query_start_loc.numel() - 1
    _need(y, "y", torch.bfloat16, (T, H, P), dev)
    _need(x, "x", torch.bfloat16, (T, H, P), dev)
    _need(dt, "dt", torch.float32, (T, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", torch.bfloat16, (T, G, N), dev)
    _need(C, "C", torch.bfloat16, (T, G, N), dev)
    D = _opt(D, "D", torch.float32, (H,), dev)
    dt_bias = _opt(dt_bias, "dt_bias", torch.float32, (H,), dev)
    if final_states is None:
        raise ValueError("final_states is required")
    sd = _state_dtype(final_states, "final_states")
    initial_states = _opt(initial_states, "initial_states", final_states.dtype, (batch, H, P, N), dev)
    _need(final_states, "final_states", final_states.dtype, (batch, H, P, N), dev)
    _need(query_start_loc, "query_start_loc", torch.int32, (batch + 1,), dev)
    prob = make_problem(T, batch, H, P, G, N, max(batch, 1), dt_softplus, state_dtype=sd,
                        short_path_max=short_path_max)
    need = ssd_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.numel() < need or workspace.device != dev:
        raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {dev}")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    status = load_library().ssd_chunk_scan_varlen_fwd(
        ctypes.byref(prob), _ptr(y), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(dt_bias), _ptr(initial_states), _ptr(final_states), _ptr(query_start_loc),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(st.cuda_stream))
    _check(status, "ssd_chunk_scan_varlen_fwd")
    return workspace


def ssd_validate_inputs(prob: ssd_problem, query_start_loc, cache_indices, stream=None) -> int:
    """Synchronous precondition check; returns the status code."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream(query_start_loc.device)
    return load_library().ssd_validate_inputs(ctypes.byref(prob), _ptr(query_start_loc),
                                              _ptr(cache_indices), ctypes.c_void_p(st.cuda_stream))
