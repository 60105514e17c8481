"""C-ABI contract on the CPU: the library loads, exports every declared symbol, and its
host-side checks reject bad arguments before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import sparse_decode_attention_csa2_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.fail("libcsa2.so is not built (run __graft_entry__.build())")
    return csa2.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(csa2.EXPORTS) <= set(names)


def test_version_and_status_strings(lib):
    assert lib.csa2_version() == 2
    for code, text in ((0, b"ok"), (1, b"invalid argument"), (2, b"unsupported parameter"),
                       (3, b"workspace too small"), (4, b"HIP error")):
        assert lib.csa2_status_string(code) == text


def _rg(**kw):
    r = csa2._Ragged()
    r.num_requests, r.num_rows = kw.get("B", 1), kw.get("R", 1)
    fake = 0x10000  # never dereferenced: every call below fails its host checks first
    for f in ("entry_off", "block_off", "row_off", "row_req", "row_swa_start", "row_swa_len"):
        setattr(r, f, kw.get(f, fake))
    r.max_entries, r.total_entries = kw.get("max_entries", 100), kw.get("total_entries", 100)
    r.total_blocks, r.swa_tokens = kw.get("total_blocks", 2), kw.get("swa_tokens", 128)
    r.max_rows_per_request = kw.get("mrpr", 1)
    r.row_len = kw.get("row_len", None)
    r.page_table = kw.get("page_table", None)
    r.pages_ld, r.total_pages = kw.get("pages_ld", 0), kw.get("total_pages", 0)
    return r


def test_null_and_bad_descriptors_rejected(lib):
    assert lib.csa2_index_score(None, None, None, None, None, None, 0, None, 0, None) == csa2.ERR_INVALID_ARG
    assert b"NULL" in lib.csa2_last_error()
    rg = _rg(B=-1)
    assert lib.csa2_index_score(ctypes.byref(rg), None, None, None, None, None, 0, None, 0, None) == csa2.ERR_INVALID_ARG
    rg = _rg(entry_off=None)
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 16, 16, None, None, 0, 16, 100, None) == csa2.ERR_INVALID_ARG
    rg = _rg(max_entries=200, total_entries=100)
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 16, 16, None, None, 0, 16, 200, None) == csa2.ERR_INVALID_ARG
    rg = _rg(mrpr=17)
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 16, 16, None, None, 0, 16, 100, None) == csa2.ERR_UNSUPPORTED


def test_pointer_and_size_checks(lib):
    rg = _rg()
    # null inputs
    assert lib.csa2_index_score(ctypes.byref(rg), None, 16, 16, None, None, 0, 16, 100, None) == csa2.ERR_INVALID_ARG
    # misaligned q_idx
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 18, 16, None, None, 0, 16, 100, None) == csa2.ERR_INVALID_ARG
    assert b"aligned" in lib.csa2_last_error()
    # ld smaller than max_entries
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 16, 16, None, None, 0, 16, 99, None) == csa2.ERR_INVALID_ARG
    # kept_blocks without n_kept
    assert lib.csa2_index_score(ctypes.byref(rg), 16, 16, 16, 16, None, 65, 16, 100, None) == csa2.ERR_INVALID_ARG


def test_parameter_ranges(lib):
    rg = _rg()
    assert lib.csa2_block_filter(ctypes.byref(rg), 16, 16, 16, 0, 1, 16, 16, 16, 2, None) == csa2.ERR_UNSUPPORTED
    assert lib.csa2_block_filter(ctypes.byref(rg), 16, 16, 16, 129, 1, 16, 16, 16, 2, None) == csa2.ERR_UNSUPPORTED
    assert lib.csa2_block_filter(ctypes.byref(rg), 16, 16, 16, 64, 1, 16, 16, 16, 1, None) == csa2.ERR_INVALID_ARG
    assert lib.csa2_topk(ctypes.byref(rg), 16, 100, None, None, 0, 0, 16, 16, None, None) == csa2.ERR_UNSUPPORTED
    assert lib.csa2_topk(ctypes.byref(rg), 16, 100, None, None, 0, 2049, 16, 16, None, None) == csa2.ERR_UNSUPPORTED
    big = _rg(max_entries=9000, total_entries=9000)
    assert lib.csa2_topk(ctypes.byref(big), 16, 9000, None, None, 0, 512, 16, 16, None, None) == csa2.ERR_UNSUPPORTED


def test_attention_workspace_contract(lib):
    rg = _rg(R=1)
    need = lib.csa2_sparse_attn_workspace_size(ctypes.byref(rg), 512)
    assert need > 0   # one row splits its 640 keys over several workgroups
    st = lib.csa2_sparse_attn(ctypes.byref(rg), 16, 16, 16, 16, 512, 16, 16, ctypes.c_float(0.044), 16, 16, 256,
                              need - 1, None)
    assert st == csa2.ERR_WORKSPACE_TOO_SMALL
    st = lib.csa2_sparse_attn(ctypes.byref(rg), 16, 16, 16, 16, 512, 16, 16, ctypes.c_float(float("inf")), 16, 16,
                              256, need, None)
    assert st == csa2.ERR_INVALID_ARG


def test_decode_workspace_and_checks(lib):
    a = csa2._DecodeArgs()
    a.rg = _rg(R=4, B=4, max_entries=65536, total_entries=4 * 65536)
    a.k, a.n_keep, a.keep_newest, a.scan_mode = 512, 64, 1, 0
    need = lib.csa2_decode_workspace_size(ctypes.byref(a))
    # scores [4][65536] + block scores + kept + sel + attention partials
    assert need >= 4 * 65536 * 4
    for f in ("idx_k", "main_kv", "blk_sum", "swa", "swa_scale", "q", "q_idx", "w_idx", "out", "lse"):
        setattr(a, f, 0x10000)
    assert lib.csa2_decode(ctypes.byref(a), 0x10000, need - 1, None) == csa2.ERR_WORKSPACE_TOO_SMALL
    a.scan_mode = 2
    assert lib.csa2_decode(ctypes.byref(a), 0x10000, need, None) == csa2.ERR_UNSUPPORTED
    a.scan_mode = 0
    a.k = 4096
    assert lib.csa2_decode(ctypes.byref(a), 0x10000, need, None) == csa2.ERR_UNSUPPORTED
    a.k = 512
    a.sel_idx = 0x10000   # sel_idx without n_sel
    assert lib.csa2_decode(ctypes.byref(a), 0x10000, need, None) == csa2.ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(lib):
    rg = _rg(B=0, R=0, max_entries=0, total_entries=0)
    assert lib.csa2_index_score(ctypes.byref(rg), None, None, None, None, None, 0, None, 0, None) == csa2.OK
    assert lib.csa2_debug_dequant(0, None, None, 0, None, None) == csa2.OK
    assert lib.csa2_debug_dequant(7, None, None, 1, None, None) == csa2.ERR_INVALID_ARG


def test_stream_read_validates_before_launch(lib):
    assert lib.csa2_debug_stream_read(None, 0, None, None) == csa2.OK
    assert lib.csa2_debug_stream_read(None, 15, None, None) == csa2.ERR_INVALID_ARG
    assert lib.csa2_debug_stream_read(None, -16, None, None) == csa2.ERR_INVALID_ARG
    assert lib.csa2_debug_stream_read(None, 16, None, None) == csa2.ERR_INVALID_ARG      # null source
    assert lib.csa2_debug_stream_read(0x10008, 16, 0x20000, None) == csa2.ERR_INVALID_ARG  # misaligned


def test_clock_trace_validates_before_launch(lib):
    assert lib.csa2_debug_clock_trace(None, 0, 1, None) == csa2.OK
    assert lib.csa2_debug_clock_trace(None, -1, 1, None) == csa2.ERR_INVALID_ARG
    assert lib.csa2_debug_clock_trace(0x10000, 4, 0, None) == csa2.ERR_INVALID_ARG       # interval < 1
    assert lib.csa2_debug_clock_trace(0x10000, 65537, 1, None) == csa2.ERR_INVALID_ARG   # too many samples
    assert lib.csa2_debug_clock_trace(0x10000, 4000, 100000, None) == csa2.ERR_INVALID_ARG  # 4 s
    assert lib.csa2_debug_clock_trace(None, 4, 10, None) == csa2.ERR_INVALID_ARG         # null out
    assert lib.csa2_debug_clock_trace(0x10004, 4, 10, None) == csa2.ERR_INVALID_ARG      # misaligned


def test_paged_descriptor_checks(lib):
    fake = 0x10000
    args = (16, 16, 16, None, None, 0, 16, 100, None)
    # 100 entries need 2 pages per request; the pools hold 2 pages (128 rows, 2 summaries).
    ok = dict(page_table=fake, pages_ld=2, total_pages=2, total_entries=128, total_blocks=2)
    rg = _rg(**{**ok, "pages_ld": 1})
    assert lib.csa2_index_score(ctypes.byref(rg), *args) == csa2.ERR_INVALID_ARG
    assert b"pages_ld" in lib.csa2_last_error()
    rg = _rg(**{**ok, "total_pages": 0})
    assert lib.csa2_index_score(ctypes.byref(rg), *args) == csa2.ERR_INVALID_ARG
    rg = _rg(**{**ok, "total_pages": 3})                    # more pages than the pools hold
    assert lib.csa2_index_score(ctypes.byref(rg), *args) == csa2.ERR_INVALID_ARG
    rg = _rg(**{**ok, "total_entries": 127})
    assert lib.csa2_index_score(ctypes.byref(rg), *args) == csa2.ERR_INVALID_ARG
    # block_off may be NULL with a page table, not without one.
    rg = _rg(block_off=None)
    assert lib.csa2_index_score(ctypes.byref(rg), *args) == csa2.ERR_INVALID_ARG
    assert b"block_off" in lib.csa2_last_error()
    # The paged standalone attention also needs room for the translated rows.
    rg = _rg(R=1, **ok)
    plain = _rg(R=1)
    need = lib.csa2_sparse_attn_workspace_size(ctypes.byref(rg), 512)
    assert need >= lib.csa2_sparse_attn_workspace_size(ctypes.byref(plain), 512) + 512 * 4
    st = lib.csa2_sparse_attn(ctypes.byref(rg), 16, 16, 16, 16, 512, 16, 16, ctypes.c_float(0.044), 16, 16, 256,
                              need - 1, None)
    assert st == csa2.ERR_WORKSPACE_TOO_SMALL
