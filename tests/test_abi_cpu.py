"""The C ABI on a machine without a GPU: the library loads, exports every entry
point include/pkv.h declares, and rejects bad arguments before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} is declared in pkv.h but not exported"


def test_abi_version_and_struct_size(lib):
    assert lib.pkv_abi_version() == 4
    assert lib.pkv_plan_info_size() == ctypes.sizeof(lib.pkv_plan_info)


SCHED = (256, 4, 256)


def _decode_plan(lib, indptr, lpl, hq=32, hkv=8, head_dim=128, P=16, dtype=0, sched=SCHED,
                 variant=None):
    indptr = np.asarray(indptr, np.int32)
    lpl = np.asarray(lpl, np.int32)
    info = lib.pkv_plan_info()
    s = lib.pkv_sched(*sched)
    st = lib._lib_decode_plan(lib._i32p(indptr), lib._i32p(lpl), len(indptr) - 1, hq, hkv,
                              head_dim, P, dtype,
                              None if variant is None else ctypes.byref(variant),
                              ctypes.byref(s), None, 0, None, 0, None, 0, None,
                              ctypes.byref(info))
    return st, info


@pytest.mark.parametrize("indptr,lpl,code", [
    ([0, 3, 2], [5, 5], 1),          # non-monotone indptr
    ([0, 3, 5], [0, 5], 1),          # last_page_len 0 with pages
    ([0, 3, 5], [17, 5], 1),         # last_page_len > page_size
    ([0, 0, 5], [3, 5], 1),          # last_page_len != 0 without pages
    ([-1, 0], [0], 1),               # negative indptr
])
def test_decode_plan_rejects_bad_page_tables(lib, indptr, lpl, code):
    st, _ = _decode_plan(lib, indptr, lpl)
    assert st == code
    assert lib.pkv_last_error() != ""


def test_decode_plan_unsupported_and_invalid_geometry(lib):
    assert _decode_plan(lib, [0, 1], [1], head_dim=64)[0] == lib.PKV_ERR_UNSUPPORTED
    assert _decode_plan(lib, [0, 1], [1], dtype=2)[0] == lib.PKV_ERR_UNSUPPORTED
    assert _decode_plan(lib, [0, 1], [1], dtype=7)[0] == lib.PKV_ERR_INVALID_ARG
    assert _decode_plan(lib, [0, 1], [1], hq=30, hkv=8)[0] == lib.PKV_ERR_INVALID_ARG
    assert _decode_plan(lib, [0, 1], [1], hq=64, hkv=2)[0] == lib.PKV_ERR_UNSUPPORTED  # G = 32
    assert _decode_plan(lib, [0, 1], [1], sched=(0, 4, 256))[0] == lib.PKV_ERR_INVALID_ARG


def test_decode_plan_reports_workspace_sizes(lib):
    # 3 requests, one long enough to split at a small chunk size
    st, info = _decode_plan(lib, [0, 2, 2, 40], [7, 0, 16], sched=(64, 4, 16))
    assert st == lib.PKV_ERR_WORKSPACE_TOO_SMALL
    assert info.int_ws_required > 0 and info.float_ws_required > 0
    items, groups, counts = lib.pkv_plan_host(lib.PKV_KIND_DECODE, None, [0, 2, 2, 40],
                                              [7, 0, 16], 32, 8, 16, 0, (64, 4, 16))
    assert info.float_ws_required >= counts[3] * 4 * (128 + 1) * 4


def test_prefill_plan_rejects_bad_qo_indptr(lib):
    qo = np.array([0, 5, 3], np.int32)
    kv = np.array([0, 1, 2], np.int32)
    lpl = np.array([4, 4], np.int32)
    info = lib.pkv_plan_info()
    s = lib.pkv_sched(*SCHED)
    st = lib._lib_prefill_plan(lib._i32p(qo), lib._i32p(kv), lib._i32p(lpl), 2, 32, 8, 128, 16, 1,
                               1, None, ctypes.byref(s), None, 0, None, 0, None, 0, None,
                               ctypes.byref(info))
    assert st == lib.PKV_ERR_INVALID_ARG
    st = lib._lib_prefill_plan(lib._i32p(np.array([0, 1, 3], np.int32)), lib._i32p(kv),
                               lib._i32p(lpl), 2, 32, 8, 128, 16, 1, 2, None, ctypes.byref(s),
                               None, 0, None, 0, None, 0, None, ctypes.byref(info))
    assert st == lib.PKV_ERR_INVALID_ARG     # causal must be 0 or 1


def test_run_rejects_foreign_or_mismatched_plans(lib):
    bogus = lib.pkv_plan_info()
    kv = lib.pkv_paged_kv()
    st = lib._lib_decode_run(ctypes.byref(bogus), None, ctypes.byref(kv), None, None, 1.0, None,
                             None, None, None)
    assert st == lib.PKV_ERR_PLAN_MISMATCH
    # a well-formed plan header with a different page size than the KV description
    st, info = _decode_plan(lib, [0, 1], [1])
    assert st == lib.PKV_ERR_WORKSPACE_TOO_SMALL   # no workspaces given: header still filled
    info.magic = 0x31564B50
    info.abi_version = lib.pkv_abi_version()
    info.kind = lib.PKV_KIND_DECODE
    info.page_size, info.num_kv_heads, info.head_dim, info.dtype = 16, 8, 128, 0
    kv.k = kv.v = 1 << 20
    kv.page_size, kv.num_kv_heads, kv.head_dim, kv.dtype = 32, 8, 128, 0
    st = lib._lib_decode_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, 1.0, None,
                             None, None, None)
    assert st == lib.PKV_ERR_PLAN_MISMATCH
    kv.page_size = 16
    kv.token_stride = 12                          # not a multiple of 8 elements
    st = lib._lib_decode_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, 1.0, None,
                             None, None, None)
    assert st == lib.PKV_ERR_INVALID_ARG
    info.kind = lib.PKV_KIND_PREFILL
    st = lib._lib_decode_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, 1.0, None,
                             None, None, None)
    assert st == lib.PKV_ERR_PLAN_MISMATCH


def _fake_decode_plan(lib, window_left=-1):
    """A well-formed decode plan header (no workspaces) and a matching KV view."""
    st, info = _decode_plan(lib, [0, 1], [1], variant=lib.pkv_variant(window_left, 0.0, None))
    assert st == lib.PKV_ERR_WORKSPACE_TOO_SMALL
    info.magic = 0x31564B50
    info.abi_version = lib.pkv_abi_version()
    info.kind = lib.PKV_KIND_DECODE
    info.page_size, info.num_kv_heads, info.head_dim, info.dtype = 16, 8, 128, 0
    kv = lib.pkv_paged_kv()
    kv.k = kv.v = 1 << 20
    kv.page_size, kv.num_kv_heads, kv.head_dim, kv.dtype = 16, 8, 128, 0
    kv.page_stride, kv.token_stride, kv.head_stride = 16 * 8 * 128, 8 * 128, 128
    return info, kv


def _run(lib, info, kv, variant):
    return lib._lib_decode_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, 0.125,
                               None if variant is None else ctypes.byref(variant), None, None,
                               None)


def test_variant_validation(lib):
    """Plan: window_left < -1 is invalid; the plan records its window. Run: the window
    must equal the plan's; the soft cap must be finite and >= 0; sinks 4-byte aligned.
    Every check happens before any launch (q is NULL, so a valid variant then fails
    on the NULL q with INVALID_ARG, not with a GPU call)."""
    st, _ = _decode_plan(lib, [0, 1], [1], variant=lib.pkv_variant(-2, 0.0, None))
    assert st == lib.PKV_ERR_INVALID_ARG and "window_left" in lib.pkv_last_error()
    info, kv = _fake_decode_plan(lib, window_left=64)
    assert info.part[0].window_left == 64
    assert _run(lib, info, kv, None) == lib.PKV_ERR_PLAN_MISMATCH
    assert _run(lib, info, kv, lib.pkv_variant(63, 0.0, None)) == lib.PKV_ERR_PLAN_MISMATCH
    assert _run(lib, info, kv, lib.pkv_variant(64, -1.0, None)) == lib.PKV_ERR_INVALID_ARG
    assert _run(lib, info, kv, lib.pkv_variant(64, float("nan"), None)) == lib.PKV_ERR_INVALID_ARG
    assert _run(lib, info, kv, lib.pkv_variant(64, float("inf"), None)) == lib.PKV_ERR_INVALID_ARG
    assert _run(lib, info, kv, lib.pkv_variant(64, 1e-38, None)) == lib.PKV_ERR_INVALID_ARG
    assert _run(lib, info, kv, lib.pkv_variant(64, 30.0, (1 << 20) + 2)) == lib.PKV_ERR_INVALID_ARG
    assert "sinks" in lib.pkv_last_error()
    st = _run(lib, info, kv, lib.pkv_variant(64, 30.0, 1 << 20))
    assert st == lib.PKV_ERR_INVALID_ARG and "NULL" in lib.pkv_last_error()
    info, kv = _fake_decode_plan(lib)
    assert info.part[0].window_left == -1
    assert _run(lib, info, kv, lib.pkv_variant(5, 0.0, None)) == lib.PKV_ERR_PLAN_MISMATCH
    st = _run(lib, info, kv, None)
    assert st == lib.PKV_ERR_INVALID_ARG and "NULL" in lib.pkv_last_error()


def test_merge_rejects_bad_arguments(lib):
    assert lib._lib_merge_state(None, None, None, None, None, None, -1, 1, 1, 0, None) == 1
    assert lib._lib_merge_state(None, None, None, None, None, None, 1, 1, 1, 9, None) == 1
    assert lib._lib_merge_state(None, None, None, None, None, None, 1, 1, 128, 0, None) == 1
    assert lib._lib_merge_states(None, None, 2, -1, 1, 128, 0, None, None, None) == 1
    assert lib._lib_merge_state_in_place(None, None, None, None, 3, 0, 128, 0, None) == 1


def test_single_decode_reports_workspace_and_validates(lib):
    need = ctypes.c_int64(0)
    s = lib.pkv_sched(256, 2, 128)
    st = lib._lib_single_decode(None, None, None, 1024, 32, 32, 128, 0, 0.1, ctypes.byref(s),
                                None, 0, ctypes.byref(need), None, None, None)
    assert st == lib.PKV_ERR_WORKSPACE_TOO_SMALL
    # 8 chunks x 32 heads x 1 row: 128 floats of O + one LSE each
    assert need.value >= 32 * 8 * (128 + 1) * 4
    st = lib._lib_single_decode(None, None, None, -1, 32, 32, 128, 0, 0.1, ctypes.byref(s), None,
                                0, ctypes.byref(need), None, None, None)
    assert st == lib.PKV_ERR_INVALID_ARG
    # a non-empty cache needs k and v (checked before any launch; q and o are stand-ins)
    fake = ctypes.c_void_p(0x10000)
    st = lib._lib_single_decode(fake, None, None, 5, 32, 32, 128, 0, 0.1, ctypes.byref(s), None,
                                0, ctypes.byref(need), fake, None, None)
    assert st == lib.PKV_ERR_INVALID_ARG
    assert "k or v is NULL" in lib.pkv_last_error()


def test_cascade_plan_validation(lib):
    ind = np.array([0, 1, 1], np.int32)
    lpl = np.array([3, 0], np.int32)
    info = lib.pkv_plan_info()
    s = lib.pkv_sched(*SCHED)
    st = lib._lib_cascade_plan(4, 0, lib._i32p(ind), lib._i32p(lpl), 2, 32, 8, 128, 16, 0,
                               ctypes.byref(s), None, 0, None, 0, None, 0, None,
                               ctypes.byref(info))
    assert st == lib.PKV_ERR_INVALID_ARG      # prefix last_page_len 0 with 4 pages
    st = lib._lib_cascade_plan(4, 16, lib._i32p(ind), lib._i32p(lpl), 2, 32, 8, 128, 16, 0,
                               ctypes.byref(s), None, 0, None, 0, None, 0, None,
                               ctypes.byref(info))
    assert st == lib.PKV_ERR_WORKSPACE_TOO_SMALL
    assert info.float_ws_required >= 2 * 2 * 32 * 128 * 4


def test_runs_reject_bad_scales(lib):
    kv = lib.pkv_paged_kv()
    info = lib.pkv_plan_info()
    for scale in (0.0, -0.5, float("inf"), float("nan")):
        assert lib._lib_decode_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, scale,
                                   None, None, None, None) == lib.PKV_ERR_INVALID_ARG
        assert lib._lib_prefill_run(ctypes.byref(info), None, ctypes.byref(kv), None, None, None,
                                    scale, None, None, None, None) == lib.PKV_ERR_INVALID_ARG


def test_append_validates_before_any_launch(lib):
    def layout(P=16, H=8, D=128, dtype=0, ps=None, ts=None, hs=128):
        kv = lib.pkv_paged_kv()
        kv.page_size, kv.num_kv_heads, kv.head_dim, kv.dtype = P, H, D, dtype
        kv.token_stride = H * D if ts is None else ts
        kv.page_stride = P * kv.token_stride if ps is None else ps
        kv.head_stride = hs
        return kv

    def call(kv, nnz=4, ptr=16, batch=2):
        return lib._lib_append_paged_kv(ptr, ptr, nnz, ptr, ptr, ptr, ptr, ctypes.byref(kv),
                                        ptr, ptr, ptr, batch, None)

    assert lib._lib_append_paged_kv(None, None, 1, None, None, None, None, None, None, None,
                                    None, 1, None) == lib.PKV_ERR_INVALID_ARG   # NULL layout
    assert call(layout(), nnz=-1) == lib.PKV_ERR_INVALID_ARG
    assert call(layout(), batch=-1) == lib.PKV_ERR_INVALID_ARG
    assert call(layout(D=64)) == lib.PKV_ERR_UNSUPPORTED
    assert call(layout(H=33)) == lib.PKV_ERR_UNSUPPORTED
    assert call(layout(dtype=2)) == lib.PKV_ERR_UNSUPPORTED
    assert call(layout(P=0)) == lib.PKV_ERR_INVALID_ARG
    assert call(layout(hs=4)) == lib.PKV_ERR_INVALID_ARG                   # stride not a multiple of 8
    assert call(layout(ps=1 << 30)) == lib.PKV_ERR_INVALID_ARG             # page stride too large
    assert call(layout(), ptr=8) == lib.PKV_ERR_INVALID_ARG                # misaligned pointers
    kv = layout()
    assert lib._lib_append_paged_kv(None, None, 3, None, None, None, None, ctypes.byref(kv), None,
                                    None, None, 1, None) == lib.PKV_ERR_INVALID_ARG
    # nothing to append: no pointer is needed and nothing is launched
    assert lib._lib_append_paged_kv(None, None, 0, None, None, None, None, ctypes.byref(kv), None,
                                    None, None, 1, None) == lib.PKV_OK


def test_append_positions_host_helper(lib):
    bi, pos = lib.pkv_append_positions([0, 2, 2, 5], [0, 1, 1, 3], [3, 0, 2], 4)
    assert bi.tolist() == [0, 0, 2, 2, 2] and pos.tolist() == [1, 2, 3, 4, 5]
    for args in (([0, 5], [0, 1], [3], 4),         # more rows than the request holds
                 ([1, 2], [0, 1], [3], 4),         # append_indptr[0] != 0
                 ([0, 2, 1], [0, 1, 2], [3, 3], 4),  # not monotone
                 ([0, 1], [0, 1], [5], 4)):        # last_page_len > page_size
        with pytest.raises(lib.PkvError):
            lib.pkv_append_positions(*args)
