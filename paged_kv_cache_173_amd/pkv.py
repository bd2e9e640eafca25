"""Python binding of libpkv.so: argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/pkv.h) and does nothing but turn tensors / arrays into pointers and
sizes, allocate outputs and workspaces with torch (device memory is
PyTorch's job here), and raise on a non-zero status. All computation happens
in the library's HIP kernels; there is no fallback: importing this module
fails if libpkv.so has not been built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY=libpkv_debug.so selects the debug build (LDS tiles NaN-filled
# before each prefill item); the default is the product library.
LIB_PATH = os.path.join(_HERE, os.environ.get("PKV_LIBRARY", "libpkv.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with paged_kv_cache_173_amd.build.build()")

_lib = ctypes.CDLL(LIB_PATH)

# status codes
PKV_OK = 0
PKV_ERR_INVALID_ARG = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_WORKSPACE_TOO_SMALL = 3
PKV_ERR_PLAN_MISMATCH = 4
PKV_ERR_HIP = 5
# dtypes
PKV_F16, PKV_BF16, PKV_F32 = 0, 1, 2
# plan kinds
PKV_KIND_DECODE, PKV_KIND_PREFILL, PKV_KIND_CASCADE, PKV_KIND_BLOCK_SPARSE, PKV_KIND_POD = 1, 2, 3, 4, 5

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_I32P = ctypes.POINTER(ctypes.c_int32)


class pkv_paged_kv(ctypes.Structure):
    _fields_ = [("k", _P), ("v", _P), ("page_stride", _I64), ("token_stride", _I64),
                ("head_stride", _I64), ("page_size", _I32), ("num_kv_heads", _I32),
                ("head_dim", _I32), ("dtype", _I32)]


class pkv_sched(ctypes.Structure):
    _fields_ = [("num_cus", _I32), ("wg_per_cu", _I32), ("min_chunk_tokens", _I32)]


class pkv_variant(ctypes.Structure):
    _fields_ = [("window_left", _I32), ("logits_soft_cap", _F32), ("sinks", _P)]


class pkv_plan_part(ctypes.Structure):
    _fields_ = [("num_items", _I32), ("num_groups", _I32), ("chunk_pages", _I32),
                ("rows_per_tile", _I32), ("num_slots", _I32), ("causal", _I32),
                ("window_left", _I32), ("reserved", _I32), ("items_off", _I64),
                ("groups_off", _I64), ("kv_len_off", _I64), ("part_o_off", _I64),
                ("part_ml_off", _I64)]


class pkv_plan_info(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("abi_version", _I32), ("kind", _I32),
                ("dtype", _I32), ("batch", _I32), ("num_qo_heads", _I32), ("num_kv_heads", _I32),
                ("head_dim", _I32), ("page_size", _I32), ("total_qo", _I32),
                ("sched", pkv_sched), ("int_ws", _P), ("float_ws", _P),
                ("int_ws_required", _I64), ("float_ws_required", _I64),
                ("order_off", _I64), ("num_blocks", _I32),
                ("batch2", _I32), ("part", pkv_plan_part * 2)]


def _sig(name, restype, argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = argtypes
    return fn


_lib_last_error = _sig("pkv_last_error", ctypes.c_char_p, [])
_lib_abi_version = _sig("pkv_abi_version", _I32, [])
_lib_plan_info_size = _sig("pkv_plan_info_size", _SZ, [])
_lib_default_sched = _sig("pkv_default_sched", _I32, [_I32, ctypes.POINTER(pkv_sched)])
_lib_default_sched_for = _sig("pkv_default_sched_for", _I32,
                              [_I32, _I32, ctypes.POINTER(pkv_sched)])
_VARP = ctypes.POINTER(pkv_variant)
_lib_plan_host = _sig("pkv_plan_host", _I32,
                      [_I32, _I32P, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32,
                       ctypes.POINTER(pkv_sched), _I32P, _I32, _I32P, _I32, _I32P])
_lib_workspace_size = _sig("pkv_workspace_size", _I32,
                           [_I32, _I32, _I32, _I32, _I32, _I64, ctypes.POINTER(_SZ),
                            ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)])
_lib_plan_export = _sig("pkv_plan_export", _I32,
                        [ctypes.POINTER(pkv_plan_info), _P, _I32, _I32P, _I32, _I32P, _I32])
_lib_decode_plan = _sig("pkv_decode_plan", _I32,
                        [_I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32, _VARP,
                         ctypes.POINTER(pkv_sched), _P, _SZ, _P, _SZ, _P, _SZ, _P,
                         ctypes.POINTER(pkv_plan_info)])
_lib_decode_run = _sig("pkv_decode_run", _I32,
                       [ctypes.POINTER(pkv_plan_info), _P, ctypes.POINTER(pkv_paged_kv), _P, _P,
                        _F32, _VARP, _P, _P, _P])
_lib_decode_run_timed = _sig("pkv_decode_run_timed", _I32,
                             [ctypes.POINTER(pkv_plan_info), _P, ctypes.POINTER(pkv_paged_kv), _P,
                              _P, _F32, _VARP, _P, _P, _P, _P, _P])
_lib_prefill_run_timed = _sig("pkv_prefill_run_timed", _I32,
                              [ctypes.POINTER(pkv_plan_info), _P, ctypes.POINTER(pkv_paged_kv), _P,
                               _P, _P, _F32, _VARP, _P, _P, _P, _P, _P])
_lib_prefill_plan = _sig("pkv_prefill_plan", _I32,
                         [_I32P, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VARP,
                          ctypes.POINTER(pkv_sched), _P, _SZ, _P, _SZ, _P, _SZ, _P,
                          ctypes.POINTER(pkv_plan_info)])
_lib_prefill_run = _sig("pkv_prefill_run", _I32,
                        [ctypes.POINTER(pkv_plan_info), _P, ctypes.POINTER(pkv_paged_kv), _P, _P,
                         _P, _F32, _VARP, _P, _P, _P])
_lib_single_decode = _sig("pkv_single_decode", _I32,
                          [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32,
                           ctypes.POINTER(pkv_sched), _P, _SZ, ctypes.POINTER(_I64), _P, _P, _P])
_lib_single_decode_noalloc = _sig("pkv_single_decode_noalloc", _I32,
                                  [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32,
                                   ctypes.POINTER(pkv_sched), _P, _P, _P])
_lib_merge_state = _sig("pkv_merge_state", _I32,
                        [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P])
_lib_merge_state_in_place = _sig("pkv_merge_state_in_place", _I32,
                                 [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P])
_lib_merge_states = _sig("pkv_merge_states", _I32,
                         [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P])
_lib_block_sparse_plan = _sig("pkv_block_sparse_plan", _I32,
                              [_I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                               ctypes.POINTER(pkv_sched), _P, _SZ, _P, _SZ, _P, _SZ, _P,
                               ctypes.POINTER(pkv_plan_info)])
_lib_block_sparse_run = _sig("pkv_block_sparse_run", _I32,
                             [ctypes.POINTER(pkv_plan_info), _P, _P, _P, _P, _P, _F32, _P, _P, _P])
_lib_append_paged_kv = _sig("pkv_append_paged_kv", _I32,
                            [_P, _P, _I32, _P, _P, _P, _P, ctypes.POINTER(pkv_paged_kv), _P, _P,
                             _P, _I32, _P])
_lib_append_positions = _sig("pkv_append_positions", _I32,
                             [_I32P, _I32P, _I32P, _I32, _I32, _I32P, _I32P])
_lib_cascade_plan = _sig("pkv_cascade_plan", _I32,
                         [_I32, _I32, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32,
                          ctypes.POINTER(pkv_sched), _P, _SZ, _P, _SZ, _P, _SZ, _P,
                          ctypes.POINTER(pkv_plan_info)])
_lib_cascade_run = _sig("pkv_cascade_run", _I32,
                        [ctypes.POINTER(pkv_plan_info), _P, ctypes.POINTER(pkv_paged_kv), _P, _P,
                         _P, _F32, _P, _P, _P])

_lib_pod_plan = _sig("pkv_pod_plan", _I32,
                     [_I32P, _I32P, _I32P, _I32, _I32, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32,
                      _I32, ctypes.POINTER(pkv_sched), _P, _SZ, _P, _SZ, _P, _SZ, _P,
                      ctypes.POINTER(pkv_plan_info)])
_lib_pod_run_timed = _sig("pkv_pod_run_timed", _I32,
                          [ctypes.POINTER(pkv_plan_info), ctypes.POINTER(pkv_paged_kv), _P, _P,
                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _F32, _P, _P, _P])
_lib_pod_run = _sig("pkv_pod_run", _I32,
                    [ctypes.POINTER(pkv_plan_info), ctypes.POINTER(pkv_paged_kv), _P, _P, _P, _P,
                     _P, _P, _P, _P, _P, _P, _P, _F32, _P])

if _lib_plan_info_size() != ctypes.sizeof(pkv_plan_info):
    raise ImportError("pkv_plan_info layout of the binding differs from the library's")


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {pkv_last_error()}")


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
_DTYPES = {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16, torch.float32: PKV_F32}


def dtype_code(t: torch.dtype) -> int:
    if t not in _DTYPES:
        raise TypeError(f"unsupported dtype {t}")
    return _DTYPES[t]


def _host_i32(a) -> np.ndarray:
    arr = a.cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)
    return np.ascontiguousarray(arr, dtype=np.int32)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _event(ev) -> int | None:
    """The hipEvent_t handle of a torch.cuda.Event (created on first use)."""
    if ev is None:
        return None
    if getattr(ev, "cuda_event", 0) == 0:
        ev.record()            # forces creation of the underlying event
        torch.cuda.synchronize()
    return ev.cuda_event


def _device_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def paged_kv(k_cache: torch.Tensor, v_cache: torch.Tensor) -> pkv_paged_kv:
    """Describe page pools k_cache / v_cache indexed [num_pages, P, Hkv, D] (any strides
    with a contiguous last dimension): an NHD pool as it is, an HND pool (stored
    [num_pages, Hkv, P, D]) as its view .permute(0, 2, 1, 3)."""
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    if k_cache.dim() != 4 or k_cache.stride(3) != 1:
        raise ValueError("KV pools must be [num_pages, page_size, num_kv_heads, head_dim] with "
                         "a contiguous head_dim")
    _device_tensor(k_cache, "k_cache")
    s = pkv_paged_kv()
    s.k, s.v = k_cache.data_ptr(), v_cache.data_ptr()
    s.page_stride, s.token_stride, s.head_stride = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    s.page_size, s.num_kv_heads, s.head_dim = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    s.dtype = dtype_code(k_cache.dtype)
    return s


class Workspace:
    """Device int / float workspaces plus a pinned host staging buffer for plans.

    A plan records the workspace addresses; keep this object alive (and do not
    grow it) for as long as the plan is used. A plan call queues the copy of its
    tables out of host_ws on its stream without waiting; the library makes the
    next plan call on this workspace wait for that copy before it writes host_ws.
    """

    def __init__(self, int_bytes: int = 8 << 20, float_bytes: int = 64 << 20, device=None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.int_ws = torch.empty(int_bytes, dtype=torch.uint8, device=self.device)
        self.float_ws = torch.empty(float_bytes, dtype=torch.uint8, device=self.device)
        self.host_ws = torch.empty(int_bytes, dtype=torch.uint8, pin_memory=True)

    def args(self):
        return (self.int_ws.data_ptr(), self.int_ws.numel(), self.float_ws.data_ptr(),
                self.float_ws.numel(), self.host_ws.data_ptr(), self.host_ws.numel())

    def grow(self, int_bytes: int, float_bytes: int) -> None:
        # earlier plans' copies may still read host_ws and write int_ws
        torch.cuda.synchronize(self.device)
        if int_bytes > self.int_ws.numel():
            self.int_ws = torch.empty(int_bytes, dtype=torch.uint8, device=self.device)
            self.host_ws = torch.empty(int_bytes, dtype=torch.uint8, pin_memory=True)
        if float_bytes > self.float_ws.numel():
            self.float_ws = torch.empty(float_bytes, dtype=torch.uint8, device=self.device)


def _sched_arg(sched):
    if sched is None:
        return None
    if isinstance(sched, pkv_sched):
        return ctypes.byref(sched)
    s = pkv_sched(*sched)
    return ctypes.byref(s)


def _plan_with_growth(call, workspace: Workspace, where: str) -> pkv_plan_info:
    info = pkv_plan_info()
    st = call(workspace, info)
    if st == PKV_ERR_WORKSPACE_TOO_SMALL:
        workspace.grow(info.int_ws_required, info.float_ws_required)
        info = pkv_plan_info()
        st = call(workspace, info)
    _check(st, where)
    return info


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def pkv_last_error() -> str:
    return _lib_last_error().decode()


def pkv_abi_version() -> int:
    return int(_lib_abi_version())


def pkv_plan_info_size() -> int:
    return int(_lib_plan_info_size())


def pkv_default_sched(device: int = 0) -> pkv_sched:
    s = pkv_sched()
    _check(_lib_default_sched(device, ctypes.byref(s)), "pkv_default_sched")
    return s


def pkv_default_sched_for(kind: int, device: int = 0) -> pkv_sched:
    s = pkv_sched()
    _check(_lib_default_sched_for(kind, device, ctypes.byref(s)), "pkv_default_sched_for")
    return s


def pkv_plan_host(kind, qo_indptr, kv_indptr, last_page_len, num_qo_heads, num_kv_heads,
                  page_size, causal, sched, window_left=-1):
    """Host-only plan: returns (items [n, 8], groups [m, 8], counts [4]) as int32 arrays."""
    kvp, lpl = _host_i32(kv_indptr), _host_i32(last_page_len)
    qop = None if qo_indptr is None else _host_i32(qo_indptr)
    batch = len(kvp) - 1
    counts = np.zeros(4, dtype=np.int32)
    s = sched if isinstance(sched, pkv_sched) else pkv_sched(*sched)
    args = lambda it, ic, gr, gc: _lib_plan_host(  # noqa: E731
        kind, None if qop is None else _i32p(qop), _i32p(kvp), _i32p(lpl), batch, num_qo_heads,
        num_kv_heads, page_size, causal, int(window_left), ctypes.byref(s), it, ic, gr, gc,
        _i32p(counts))
    st = args(None, 0, None, 0)
    if st not in (PKV_OK, PKV_ERR_WORKSPACE_TOO_SMALL):
        _check(st, "pkv_plan_host")
    items = np.zeros((max(1, counts[0]), 8), dtype=np.int32)
    groups = np.zeros((max(1, counts[1]), 8), dtype=np.int32)
    _check(args(_i32p(items), int(counts[0]), _i32p(groups), int(counts[1])), "pkv_plan_host")
    return items[:counts[0]], groups[:counts[1]], counts.copy()


def _variant(window_left=-1, logits_soft_cap=0.0, sinks=None):
    """A pkv_variant (by reference) for a call, or None when every variant is off.
    ``sinks`` is a float32 device tensor [num_qo_heads] or None."""
    if int(window_left) == -1 and float(logits_soft_cap) == 0.0 and sinks is None:
        return None
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 tensor [num_qo_heads]")
    return ctypes.byref(pkv_variant(int(window_left), float(logits_soft_cap),
                                    None if sinks is None else sinks.data_ptr()))


def pkv_decode_plan(kv_indptr, last_page_len, num_qo_heads, num_kv_heads, head_dim, page_size,
                    dtype, workspace: Workspace, sched=None, stream=None,
                    window_left=-1) -> pkv_plan_info:
    kvp, lpl = _host_i32(kv_indptr), _host_i32(last_page_len)
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    var = _variant(window_left)

    def call(ws, info):
        return _lib_decode_plan(_i32p(kvp), _i32p(lpl), len(kvp) - 1, num_qo_heads, num_kv_heads,
                                head_dim, page_size, code, var, _sched_arg(sched), *ws.args(),
                                _stream(stream), ctypes.byref(info))
    return _plan_with_growth(call, workspace, "pkv_decode_plan")


def pkv_decode_run(plan: pkv_plan_info, q, k_cache, v_cache, kv_indptr_d, kv_indices_d,
                   sm_scale: float, o=None, lse=None, stream=None, window_left=-1,
                   logits_soft_cap=0.0, sinks=None):
    """q [batch, Hq, D] -> (o like q, lse [batch, Hq] float32)."""
    kv = paged_kv(k_cache, v_cache)
    q = q.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_decode_run(ctypes.byref(plan), q.data_ptr(), ctypes.byref(kv),
                           kv_indptr_d.data_ptr(), kv_indices_d.data_ptr(), float(sm_scale),
                           _variant(window_left, logits_soft_cap, sinks), o.data_ptr(),
                           _ptr(lse), _stream(stream)), "pkv_decode_run")
    return o, lse


def pkv_decode_run_timed(plan: pkv_plan_info, q, k_cache, v_cache, kv_indptr_d, kv_indices_d,
                         sm_scale: float, attention_start, attention_done, o=None, lse=None,
                         stream=None, window_left=-1, logits_soft_cap=0.0, sinks=None):
    """pkv_decode_run with the torch.cuda.Events `attention_start` / `attention_done`
    (either may be None) taking the attention kernel's begin and end timestamps."""
    kv = paged_kv(k_cache, v_cache)
    q = q.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_decode_run_timed(ctypes.byref(plan), q.data_ptr(), ctypes.byref(kv),
                                 kv_indptr_d.data_ptr(), kv_indices_d.data_ptr(), float(sm_scale),
                                 _variant(window_left, logits_soft_cap, sinks), o.data_ptr(),
                                 _ptr(lse), _stream(stream), _event(attention_start),
                                 _event(attention_done)),
           "pkv_decode_run_timed")
    return o, lse


def pkv_prefill_plan(qo_indptr, kv_indptr, last_page_len, num_qo_heads, num_kv_heads, head_dim,
                     page_size, dtype, causal, workspace: Workspace, sched=None,
                     stream=None, window_left=-1) -> pkv_plan_info:
    qop, kvp, lpl = _host_i32(qo_indptr), _host_i32(kv_indptr), _host_i32(last_page_len)
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    var = _variant(window_left)

    def call(ws, info):
        return _lib_prefill_plan(_i32p(qop), _i32p(kvp), _i32p(lpl), len(kvp) - 1, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, code, int(causal), var,
                                 _sched_arg(sched), *ws.args(), _stream(stream),
                                 ctypes.byref(info))
    return _plan_with_growth(call, workspace, "pkv_prefill_plan")


def pkv_prefill_run(plan: pkv_plan_info, q, k_cache, v_cache, qo_indptr_d, kv_indptr_d,
                    kv_indices_d, sm_scale: float, o=None, lse=None, stream=None,
                    window_left=-1, logits_soft_cap=0.0, sinks=None):
    """q [total_qo, Hq, D] -> (o like q, lse [total_qo, Hq] float32)."""
    kv = paged_kv(k_cache, v_cache)
    q = q.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_prefill_run(ctypes.byref(plan), q.data_ptr(), ctypes.byref(kv),
                            qo_indptr_d.data_ptr(), kv_indptr_d.data_ptr(),
                            kv_indices_d.data_ptr(), float(sm_scale),
                            _variant(window_left, logits_soft_cap, sinks), o.data_ptr(),
                            _ptr(lse), _stream(stream)), "pkv_prefill_run")
    return o, lse


def pkv_prefill_run_timed(plan: pkv_plan_info, q, k_cache, v_cache, qo_indptr_d, kv_indptr_d,
                          kv_indices_d, sm_scale: float, attention_start, attention_done, o=None,
                          lse=None, stream=None, window_left=-1, logits_soft_cap=0.0, sinks=None):
    """pkv_prefill_run with `attention_start` / `attention_done` on the attention kernel
    (see pkv_decode_run_timed)."""
    kv = paged_kv(k_cache, v_cache)
    q = q.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_prefill_run_timed(ctypes.byref(plan), q.data_ptr(), ctypes.byref(kv),
                                  qo_indptr_d.data_ptr(), kv_indptr_d.data_ptr(),
                                  kv_indices_d.data_ptr(), float(sm_scale),
                                  _variant(window_left, logits_soft_cap, sinks), o.data_ptr(),
                                  _ptr(lse), _stream(stream), _event(attention_start),
                                  _event(attention_done)),
           "pkv_prefill_run_timed")
    return o, lse


def pkv_single_decode(q, k, v, sm_scale: float, float_ws=None, sched=None, o=None, lse=None,
                      stream=None):
    """q [Hq, D], contiguous k / v [kv_len, Hkv, D] -> (o [Hq, D], lse [Hq])."""
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [kv_len, num_kv_heads, head_dim]")
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:1], dtype=torch.float32, device=q.device) if lse is None else lse
    need = _I64(0)
    code = dtype_code(q.dtype)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), k.shape[0], q.shape[0], k.shape[1],
            k.shape[2], code, float(sm_scale), _sched_arg(sched))
    ws_ptr, ws_bytes = (0, 0) if float_ws is None else (float_ws.data_ptr(), float_ws.numel() *
                                                        float_ws.element_size())
    st = _lib_single_decode(*args, ws_ptr or None, ws_bytes, ctypes.byref(need), o.data_ptr(),
                            _ptr(lse), _stream(stream))
    if st == PKV_ERR_WORKSPACE_TOO_SMALL:
        float_ws = torch.empty(need.value, dtype=torch.uint8, device=q.device)
        st = _lib_single_decode(*args, float_ws.data_ptr(), need.value, ctypes.byref(need),
                                o.data_ptr(), _ptr(lse), _stream(stream))
    _check(st, "pkv_single_decode")
    return o, lse


def pkv_single_decode_noalloc(q, k, v, sm_scale: float, sched=None, o=None, lse=None,
                              stream=None):
    """As pkv_single_decode, with the partial states in the library's fixed device scratch
    (the call allocates no device memory; o / lse are allocated here only if not given)."""
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [kv_len, num_kv_heads, head_dim]")
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:1], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_single_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), k.shape[0],
                                      q.shape[0], k.shape[1], k.shape[2], dtype_code(q.dtype),
                                      float(sm_scale), _sched_arg(sched), o.data_ptr(),
                                      _ptr(lse), _stream(stream)), "pkv_single_decode_noalloc")
    return o, lse


def pkv_merge_state(va, sa, vb, sb, vo=None, so=None, stream=None):
    """va, vb [n, H, D]; sa, sb [n, H] float32 -> (vo, so)."""
    n, H, D = va.shape
    vo = torch.empty_like(va) if vo is None else vo
    so = torch.empty_like(sa) if so is None else so
    _check(_lib_merge_state(va.data_ptr(), sa.data_ptr(), vb.data_ptr(), sb.data_ptr(),
                            vo.data_ptr(), _ptr(so), n, H, D, dtype_code(va.dtype),
                            _stream(stream)), "pkv_merge_state")
    return vo, so


def pkv_merge_state_in_place(v, s, v_other, s_other, stream=None):
    n, H, D = v.shape
    _check(_lib_merge_state_in_place(v.data_ptr(), s.data_ptr(), v_other.data_ptr(),
                                     s_other.data_ptr(), n, H, D, dtype_code(v.dtype),
                                     _stream(stream)), "pkv_merge_state_in_place")
    return v, s


def pkv_merge_states(v, s, vo=None, so=None, stream=None):
    """v [n, K, H, D], s [n, K, H] -> (vo [n, H, D], so [n, H])."""
    n, K, H, D = v.shape
    vo = torch.empty((n, H, D), dtype=v.dtype, device=v.device) if vo is None else vo
    so = torch.empty((n, H), dtype=torch.float32, device=v.device) if so is None else so
    _check(_lib_merge_states(v.data_ptr(), s.data_ptr(), n, K, H, D, dtype_code(v.dtype),
                             vo.data_ptr(), _ptr(so), _stream(stream)), "pkv_merge_states")
    return vo, so


def pkv_cascade_plan(prefix_num_pages, prefix_last_page_len, suffix_indptr, suffix_last_page_len,
                     num_qo_heads, num_kv_heads, head_dim, page_size, dtype,
                     workspace: Workspace, sched=None, stream=None) -> pkv_plan_info:
    sip, slpl = _host_i32(suffix_indptr), _host_i32(suffix_last_page_len)
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)

    def call(ws, info):
        return _lib_cascade_plan(int(prefix_num_pages), int(prefix_last_page_len), _i32p(sip),
                                 _i32p(slpl), len(sip) - 1, num_qo_heads, num_kv_heads, head_dim,
                                 page_size, code, _sched_arg(sched), *ws.args(), _stream(stream),
                                 ctypes.byref(info))
    return _plan_with_growth(call, workspace, "pkv_cascade_plan")


def pkv_cascade_run(plan: pkv_plan_info, q, k_cache, v_cache, prefix_indices_d, suffix_indptr_d,
                    suffix_indices_d, sm_scale: float, o=None, lse=None, stream=None):
    kv = paged_kv(k_cache, v_cache)
    q = q.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_cascade_run(ctypes.byref(plan), q.data_ptr(), ctypes.byref(kv),
                            _ptr(prefix_indices_d), suffix_indptr_d.data_ptr(),
                            suffix_indices_d.data_ptr(), float(sm_scale), o.data_ptr(), _ptr(lse),
                            _stream(stream)), "pkv_cascade_run")
    return o, lse


def pkv_pod_plan(qo_indptr, kv_indptr_p, last_page_len_p, causal, kv_indptr_d, last_page_len_d,
                 num_qo_heads, num_kv_heads, head_dim, page_size, dtype, workspace: Workspace,
                 sched=None, stream=None) -> pkv_plan_info:
    """Plan a mixed batch: prefill requests (qo_indptr, kv_indptr_p, last_page_len_p) and
    decode requests (kv_indptr_d, last_page_len_d), host arrays, one launch."""
    qop, kvp, lpp = _host_i32(qo_indptr), _host_i32(kv_indptr_p), _host_i32(last_page_len_p)
    kvd, lpd = _host_i32(kv_indptr_d), _host_i32(last_page_len_d)
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)

    def call(ws, info):
        return _lib_pod_plan(_i32p(qop), _i32p(kvp), _i32p(lpp), len(kvp) - 1, int(causal),
                             _i32p(kvd), _i32p(lpd), len(kvd) - 1, num_qo_heads, num_kv_heads,
                             head_dim, page_size, code, _sched_arg(sched), *ws.args(),
                             _stream(stream), ctypes.byref(info))
    return _plan_with_growth(call, workspace, "pkv_pod_plan")


def pkv_pod_host_order(plan: pkv_plan_info, host_ws) -> np.ndarray:
    """The launch order a plan wrote into its host workspace (int32 [num_blocks])."""
    raw = np.frombuffer(host_ws, dtype=np.uint8)
    return raw[plan.order_off:plan.order_off + 4 * plan.num_blocks].view(np.int32).copy()


def pkv_pod_run(plan: pkv_plan_info, k_cache, v_cache, q_p, qo_indptr_d, kv_indptr_p_d,
                kv_indices_p_d, q_d, kv_indptr_d_d, kv_indices_d_d, sm_scale: float, o_p=None,
                lse_p=None, o_d=None, lse_d=None, stream=None, attention_start=None,
                attention_done=None):
    """One launch for both parts -> (o_p, lse_p, o_d, lse_d); the torch.cuda.Events
    `attention_start` / `attention_done` (if given) take the mixed kernel's begin and end
    timestamps (the merges are not included)."""
    kv = paged_kv(k_cache, v_cache)
    q_p, q_d = q_p.contiguous(), q_d.contiguous()
    o_p = torch.empty_like(q_p) if o_p is None else o_p
    o_d = torch.empty_like(q_d) if o_d is None else o_d
    f32 = dict(dtype=torch.float32, device=q_p.device)
    lse_p = torch.empty(q_p.shape[:2], **f32) if lse_p is None else lse_p
    lse_d = torch.empty(q_d.shape[:2], **f32) if lse_d is None else lse_d
    args = (ctypes.byref(plan), ctypes.byref(kv), q_p.data_ptr(), qo_indptr_d.data_ptr(),
            kv_indptr_p_d.data_ptr(), kv_indices_p_d.data_ptr(), o_p.data_ptr(), _ptr(lse_p),
            q_d.data_ptr(), kv_indptr_d_d.data_ptr(), kv_indices_d_d.data_ptr(), o_d.data_ptr(),
            _ptr(lse_d), float(sm_scale), _stream(stream))
    if attention_start is None and attention_done is None:
        _check(_lib_pod_run(*args), "pkv_pod_run")
    else:
        _check(_lib_pod_run_timed(*args, _event(attention_start), _event(attention_done)),
               "pkv_pod_run_timed")
    return o_p, lse_p, o_d, lse_d


def pkv_block_sparse_plan(bsr_indptr, bsr_indices, num_qo_tokens, num_kv_tokens, row_block,
                          col_block, num_qo_heads, num_kv_heads, head_dim, dtype,
                          workspace: Workspace, sched=None, stream=None) -> pkv_plan_info:
    """Plan block-sparse attention over query blocks of row_block tokens and key blocks of
    col_block tokens; (bsr_indptr, bsr_indices) are host arrays (BSR over the blocks)."""
    ip = _host_i32(bsr_indptr)
    ix = _host_i32(bsr_indices) if len(bsr_indices) else np.zeros(1, np.int32)
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)

    def call(ws, info):
        return _lib_block_sparse_plan(_i32p(ip), _i32p(ix), len(ip) - 1, int(num_qo_tokens),
                                      int(num_kv_tokens), int(row_block), int(col_block),
                                      num_qo_heads, num_kv_heads, head_dim, code, _sched_arg(sched),
                                      *ws.args(), _stream(stream), ctypes.byref(info))
    return _plan_with_growth(call, workspace, "pkv_block_sparse_plan")


def pkv_block_sparse_run(plan: pkv_plan_info, q, k, v, bsr_indptr_d, bsr_indices_d,
                         sm_scale: float, o=None, lse=None, stream=None):
    """q [N_q, Hq, D], k / v [N_kv, Hkv, D] -> (o like q, lse [N_q, Hq] float32)."""
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse is None else lse
    _check(_lib_block_sparse_run(ctypes.byref(plan), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 bsr_indptr_d.data_ptr(), bsr_indices_d.data_ptr(), float(sm_scale),
                                 o.data_ptr(), _ptr(lse), _stream(stream)), "pkv_block_sparse_run")
    return o, lse


def pkv_append_paged_kv(append_k, append_v, batch_indices_d, positions_d, k_cache, v_cache,
                        kv_indptr_d, kv_indices_d, last_page_len_d, stream=None):
    """Write appended rows append_k / append_v [nnz, Hkv, D] into the NHD pools k_cache /
    v_cache (in place) at the (request, position) each row names."""
    if append_k.shape != append_v.shape or append_k.dim() != 3:
        raise ValueError("append_k and append_v must both be [nnz, num_kv_heads, head_dim]")
    if append_k.dtype != k_cache.dtype or append_v.dtype != v_cache.dtype:
        raise ValueError("appended rows must have the cache's dtype")
    append_k, append_v = append_k.contiguous(), append_v.contiguous()
    layout = paged_kv(k_cache, v_cache)
    if append_k.shape[1] != layout.num_kv_heads or append_k.shape[2] != layout.head_dim:
        raise ValueError("appended rows must be [nnz, num_kv_heads, head_dim] of the cache")
    for name, t in (("batch_indices_d", batch_indices_d), ("positions_d", positions_d),
                    ("kv_indptr_d", kv_indptr_d), ("kv_indices_d", kv_indices_d),
                    ("last_page_len_d", last_page_len_d)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
        _device_tensor(t, name)
    nnz = append_k.shape[0]
    if batch_indices_d.numel() < nnz or positions_d.numel() < nnz:
        raise ValueError("batch_indices_d / positions_d need one entry per appended row")
    _check(_lib_append_paged_kv(append_k.data_ptr(), append_v.data_ptr(), nnz,
                                batch_indices_d.data_ptr(), positions_d.data_ptr(),
                                k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(layout),
                                kv_indptr_d.data_ptr(), kv_indices_d.data_ptr(),
                                last_page_len_d.data_ptr(), kv_indptr_d.numel() - 1,
                                _stream(stream)), "pkv_append_paged_kv")
    return k_cache, v_cache


def pkv_append_positions(append_indptr, kv_indptr, last_page_len, page_size):
    """(batch_indices, positions) int32 arrays for requests that append their new tokens at
    the end of their KV (host arrays; the page table describes the cache after the append)."""
    aip, kip, lpl = _host_i32(append_indptr), _host_i32(kv_indptr), _host_i32(last_page_len)
    nnz = int(aip[-1]) if aip.size else 0
    bi = np.zeros(max(nnz, 1), dtype=np.int32)
    pos = np.zeros(max(nnz, 1), dtype=np.int32)
    _check(_lib_append_positions(_i32p(aip), _i32p(kip), _i32p(lpl), len(kip) - 1, int(page_size),
                                 _i32p(bi), _i32p(pos)), "pkv_append_positions")
    return bi[:nnz], pos[:nnz]


def pkv_workspace_size(kind, batch, num_qo_heads, num_kv_heads, head_dim, max_items):
    """(int_ws_bytes, float_ws_bytes, host_ws_bytes) enough for any plan of `kind` with at
    most `max_items` work items."""
    i, f, h = _SZ(0), _SZ(0), _SZ(0)
    _check(_lib_workspace_size(int(kind), int(batch), int(num_qo_heads), int(num_kv_heads),
                               int(head_dim), int(max_items), ctypes.byref(i), ctypes.byref(f),
                               ctypes.byref(h)), "pkv_workspace_size")
    return int(i.value), int(f.value), int(h.value)


def pkv_plan_export(plan: pkv_plan_info, workspace: Workspace, part: int = 0):
    """A part's (items [n, 8], groups [m, 8]) from the host workspace the plan was made with."""
    p = plan.part[part] if 0 <= part < 2 else plan.part[0]
    items = np.zeros((max(1, p.num_items), 8), dtype=np.int32)
    groups = np.zeros((max(1, p.num_groups), 8), dtype=np.int32)
    _check(_lib_plan_export(ctypes.byref(plan), workspace.host_ws.data_ptr(), int(part),
                            _i32p(items), int(p.num_items), _i32p(groups), int(p.num_groups)),
           "pkv_plan_export")
    return items[:p.num_items].copy(), groups[:p.num_groups].copy()


def read_plan_tables(plan: pkv_plan_info, workspace: Workspace, part: int = 0):
    """Copy a plan's item and group tables back from the device int workspace."""
    if plan.int_ws != workspace.int_ws.data_ptr():
        raise ValueError("plan was not made with this workspace")
    p = plan.part[part]
    host = workspace.int_ws.cpu().numpy()
    items = host[p.items_off:p.items_off + p.num_items * 32].view(np.int32).reshape(-1, 8)
    groups = host[p.groups_off:p.groups_off + p.num_groups * 32].view(np.int32).reshape(-1, 8)
    return items.copy(), groups.copy()
