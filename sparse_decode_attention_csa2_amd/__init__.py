"""Python binding of libcsa2 (the gfx950 CSA2 sparse decode path).

Argument marshalling only: every step runs in the HIP kernels of ``libcsa2.so``.
PyTorch supplies device memory and the current stream.  The names follow the C ABI in
``include/csa2.h`` (``index_score``, ``block_filter``, ``topk``, ``sparse_attn``,
``decode``, ``debug_dequant``).  Importing succeeds without the library; the first call
raises ``Csa2Error`` if ``libcsa2.so`` has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

D, HEADS, IDX_D, IDX_HEADS, BLOCK, SWA_MAX = 512, 64, 128, 8, 64, 128
MAIN_BYTES, IDX_BYTES = 288, 68
K_MAX, KEEP_MAX, ROWS_PER_REQ_MAX, TOPK_ALL_MAX = 2048, 128, 16, 8192
DQ_MAIN, DQ_IDX, DQ_SWA = 0, 1, 2
QP_BF16, QP_MXFP8 = 0, 1
DECODE_EVENTS = 5

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = 0, 1, 2, 3, 4
STATIC_WS_BYTES = 64 << 20


class Csa2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"csa2 status {status}: {msg}")
        self.status = status


class _Ragged(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32), ("num_rows", ctypes.c_int32),
        ("entry_off", ctypes.c_void_p), ("block_off", ctypes.c_void_p), ("row_off", ctypes.c_void_p),
        ("row_req", ctypes.c_void_p), ("row_swa_start", ctypes.c_void_p), ("row_swa_len", ctypes.c_void_p),
        ("max_entries", ctypes.c_int64), ("total_entries", ctypes.c_int64), ("total_blocks", ctypes.c_int64),
        ("swa_tokens", ctypes.c_int64), ("max_rows_per_request", ctypes.c_int32),
        ("row_len", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("pages_ld", ctypes.c_int32),
        ("total_pages", ctypes.c_int64),
    ]


class _DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("rg", _Ragged),
        ("idx_k", ctypes.c_void_p), ("main_kv", ctypes.c_void_p), ("blk_sum", ctypes.c_void_p),
        ("swa", ctypes.c_void_p), ("swa_scale", ctypes.c_void_p), ("q", ctypes.c_void_p),
        ("q_idx", ctypes.c_void_p), ("w_idx", ctypes.c_void_p),
        ("k", ctypes.c_int32), ("n_keep", ctypes.c_int32), ("keep_newest", ctypes.c_int32),
        ("scan_mode", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("sel_idx", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
        ("kept_blocks", ctypes.c_void_p), ("n_kept", ctypes.c_void_p),
        ("scores", ctypes.c_void_p), ("scores_ld", ctypes.c_int64),
        ("events", ctypes.c_void_p), ("qp_route", ctypes.c_int32),
    ]


EXPORTS = ("csa2_index_score", "csa2_block_filter", "csa2_topk", "csa2_sparse_attn", "csa2_cache_write",
           "csa2_sparse_attn_workspace_size", "csa2_decode", "csa2_decode_workspace_size", "csa2_decode_static",
           "csa2_debug_dequant", "csa2_debug_mxfp8", "csa2_debug_stream_read", "csa2_debug_clock_trace",
           "csa2_status_string", "csa2_last_error",
           "csa2_version")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcsa2.so and declare its signatures (no GPU call is made)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Csa2Error(-1, f"{path} not found: build it with `python -m sparse_decode_attention_csa2_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    RG = ctypes.POINTER(_Ragged)
    DA = ctypes.POINTER(_DecodeArgs)
    sig = {
        "csa2_index_score": ([RG, P, P, P, P, P, I32, P, I64, P], ctypes.c_int),
        "csa2_block_filter": ([RG, P, P, P, I32, I32, P, P, P, I64, P], ctypes.c_int),
        "csa2_topk": ([RG, P, I64, P, P, I32, I32, P, P, P, P], ctypes.c_int),
        "csa2_sparse_attn": ([RG, P, P, P, P, I32, P, P, F32, P, P, P, SZ, P], ctypes.c_int),
        "csa2_sparse_attn_workspace_size": ([RG, I32], SZ),
        "csa2_decode": ([DA, P, SZ, P], ctypes.c_int),
        "csa2_decode_workspace_size": ([DA], SZ),
        "csa2_decode_static": ([DA, P], ctypes.c_int),
        "csa2_debug_dequant": ([I32, P, P, I64, P, P], ctypes.c_int),
        "csa2_debug_stream_read": ([P, I64, P, P], ctypes.c_int),
        "csa2_debug_clock_trace": ([P, I32, I32, P], ctypes.c_int),
        "csa2_debug_mxfp8": ([P, I64, P, P], ctypes.c_int),
        "csa2_cache_write": ([RG, P, P, P, P, P, P, P, F32, P, P, P, P], ctypes.c_int),
        "csa2_status_string": ([I32], ctypes.c_char_p),
        "csa2_last_error": ([], ctypes.c_char_p),
        "csa2_version": ([], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        raise Csa2Error(status, load_library().csa2_last_error().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtypes, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtypes and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


@dataclass
class Ragged:
    """Ragged batch descriptor: device offset tensors plus host maxima (see csa2.h).

    Optional: ``row_len`` (int64 [R], entries each row sees) and ``page_table`` (int32
    [B][pages_ld], paged pools of 64-entry pages, ``total_pages`` of them; then
    ``block_off`` may be None)."""
    entry_off: torch.Tensor       # int64 [B+1]
    block_off: torch.Tensor | None  # int64 [B+1]
    row_off: torch.Tensor         # int32 [B+1]
    row_req: torch.Tensor         # int32 [R]
    row_swa_start: torch.Tensor   # int64 [R]
    row_swa_len: torch.Tensor     # int32 [R]
    max_entries: int
    total_entries: int
    total_blocks: int
    swa_tokens: int
    max_rows_per_request: int
    row_len: torch.Tensor | None = None      # int64 [R]
    page_table: torch.Tensor | None = None   # int32 [B][pages_ld]
    total_pages: int = 0

    @property
    def num_requests(self) -> int:
        return self.entry_off.numel() - 1

    @property
    def num_rows(self) -> int:
        return self.row_req.numel()

    def c(self) -> _Ragged:
        for name, dt in (("entry_off", torch.int64), ("block_off", torch.int64), ("row_off", torch.int32),
                         ("row_req", torch.int32), ("row_swa_start", torch.int64), ("row_swa_len", torch.int32),
                         ("row_len", torch.int64), ("page_table", torch.int32)):
            if getattr(self, name) is not None:
                _dev(getattr(self, name), (dt,), name)
        pt = self.page_table
        if pt is not None and (pt.dim() != 2 or pt.shape[0] != self.num_requests):
            raise ValueError("page_table must be [num_requests][pages_ld]")
        return _Ragged(self.num_requests, self.num_rows, _ptr(self.entry_off), _ptr(self.block_off),
                       _ptr(self.row_off), _ptr(self.row_req), _ptr(self.row_swa_start), _ptr(self.row_swa_len),
                       int(self.max_entries), int(self.total_entries), int(self.total_blocks), int(self.swa_tokens),
                       int(self.max_rows_per_request), _ptr(self.row_len), _ptr(pt),
                       int(pt.shape[1]) if pt is not None else 0, int(self.total_pages))


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


def index_score(rg: Ragged, idx_k, q_idx, w_idx, scores=None, kept=None, n_kept=None) -> torch.Tensor:
    """Indexer scores [R][ld] (ld = max_entries unless ``scores`` is given)."""
    lib = load_library()
    _dev(idx_k, (torch.uint8,), "idx_k")
    _dev(q_idx, _BF16, "q_idx")
    _dev(w_idx, (torch.float32,), "w_idx")
    if scores is None:
        scores = torch.full((rg.num_rows, max(1, rg.max_entries)), float("nan"), dtype=torch.float32,
                            device=idx_k.device)
    _dev(scores, (torch.float32,), "scores")
    kept_ld = 0
    if kept is not None:
        _dev(kept, (torch.int32,), "kept")
        _dev(n_kept, (torch.int32,), "n_kept")
        kept_ld = kept.shape[-1]
    _check(lib.csa2_index_score(ctypes.byref(rg.c()), _ptr(idx_k), _ptr(q_idx), _ptr(w_idx), _ptr(kept),
                                _ptr(n_kept), kept_ld, _ptr(scores), scores.shape[-1], _stream()))
    return scores


def block_filter(rg: Ragged, blk_sum, q_idx, w_idx, n_keep: int = 64, keep_newest: bool = True):
    """(kept_blocks [R][n_keep+1], n_kept [R], block scores [R][ceil(max_entries/64)])."""
    lib = load_library()
    _dev(blk_sum, _BF16, "blk_sum")
    _dev(q_idx, _BF16, "q_idx")
    _dev(w_idx, (torch.float32,), "w_idx")
    R = rg.num_rows
    kept = _empty((R, n_keep + 1), torch.int32, q_idx)
    n_kept = _empty((R,), torch.int32, q_idx)
    blk_ld = max(1, -(-rg.max_entries // BLOCK))
    bscores = torch.full((R, blk_ld), float("nan"), dtype=torch.float32, device=q_idx.device)
    _check(lib.csa2_block_filter(ctypes.byref(rg.c()), _ptr(blk_sum), _ptr(q_idx), _ptr(w_idx), n_keep,
                                 1 if keep_newest else 0, _ptr(kept), _ptr(n_kept), _ptr(bscores), blk_ld,
                                 _stream()))
    return kept, n_kept, bscores


def topk(rg: Ragged, scores, kept=None, n_kept=None, k: int = 512, with_scores: bool = False):
    """(sel_idx [R][k] ascending with -1 padding, n_sel [R], sel_score or None)."""
    lib = load_library()
    _dev(scores, (torch.float32,), "scores")
    R = rg.num_rows
    sel = _empty((R, k), torch.int32, scores)
    n_sel = _empty((R,), torch.int32, scores)
    ss = _empty((R, k), torch.float32, scores) if with_scores else None
    kept_ld = 0
    if kept is not None:
        _dev(kept, (torch.int32,), "kept")
        _dev(n_kept, (torch.int32,), "n_kept")
        kept_ld = kept.shape[-1]
    _check(lib.csa2_topk(ctypes.byref(rg.c()), _ptr(scores), scores.shape[-1], _ptr(kept), _ptr(n_kept), kept_ld,
                         k, _ptr(sel), _ptr(n_sel), _ptr(ss), _stream()))
    return sel, n_sel, ss


def sparse_attn_workspace_size(rg: Ragged, sel_ld: int) -> int:
    return int(load_library().csa2_sparse_attn_workspace_size(ctypes.byref(rg.c()), sel_ld))


def sparse_attn(rg: Ragged, q, main_kv, sel_idx, n_sel, swa, swa_scale, sm_scale: float = 1.0 / math.sqrt(D),
                out=None, lse=None, ws=None):
    """(out fp32 [R][64][512], lse fp32 [R][64]); out/lse/ws may be caller-provided."""
    lib = load_library()
    _dev(q, _BF16, "q")
    _dev(main_kv, (torch.uint8,), "main_kv")
    _dev(sel_idx, (torch.int32,), "sel_idx")
    _dev(n_sel, (torch.int32,), "n_sel")
    _dev(swa, (torch.uint8,), "swa")
    _dev(swa_scale, (torch.float32,), "swa_scale")
    R = rg.num_rows
    out = _empty((R, HEADS, D), torch.float32, q) if out is None else _dev(out, (torch.float32,), "out")
    lse = _empty((R, HEADS), torch.float32, q) if lse is None else _dev(lse, (torch.float32,), "lse")
    c = rg.c()
    sel_ld = sel_idx.shape[-1]
    nws = lib.csa2_sparse_attn_workspace_size(ctypes.byref(c), sel_ld)
    if ws is None:
        ws = _empty((max(nws, 1),), torch.uint8, q)
    elif ws.numel() < nws:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nws} needed")
    _check(lib.csa2_sparse_attn(ctypes.byref(c), _ptr(q), _ptr(main_kv), _ptr(sel_idx), _ptr(n_sel), sel_ld,
                                _ptr(swa), _ptr(swa_scale), float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), nws,
                                _stream()))
    return out, lse


class Decoder:
    """csa2_decode with caller-owned outputs and workspace, reusable across calls.

    Builds the argument struct and allocates the workspace once, so ``run()`` only
    enqueues the kernels (suitable for timing loops and graph capture).
    """

    def __init__(self, rg: Ragged, idx_k, main_kv, blk_sum, swa, swa_scale, q, q_idx, w_idx, k: int = 512,
                 n_keep: int = 64, keep_newest: bool = True, sm_scale: float = 1.0 / math.sqrt(D),
                 scan_mode: int = 0, keep_intermediates: bool = True, qp_route: int = QP_BF16):
        lib = load_library()
        for t, dts, n in ((idx_k, (torch.uint8,), "idx_k"), (main_kv, (torch.uint8,), "main_kv"),
                          (blk_sum, _BF16, "blk_sum"), (swa, (torch.uint8,), "swa"),
                          (swa_scale, (torch.float32,), "swa_scale"), (q, _BF16, "q"), (q_idx, _BF16, "q_idx"),
                          (w_idx, (torch.float32,), "w_idx")):
            _dev(t, dts, n)
        R = rg.num_rows
        dev = q.device
        self.rg = rg
        self.inputs = (idx_k, main_kv, blk_sum, swa, swa_scale, q, q_idx, w_idx)   # keep alive
        self.out = torch.empty((R, HEADS, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((R, HEADS), dtype=torch.float32, device=dev)
        self.sel_idx = self.n_sel = self.kept = self.n_kept = self.scores = None
        if keep_intermediates:
            self.sel_idx = torch.empty((R, k), dtype=torch.int32, device=dev)
            self.n_sel = torch.empty((R,), dtype=torch.int32, device=dev)
            self.kept = torch.empty((R, n_keep + 1), dtype=torch.int32, device=dev)
            self.n_kept = torch.empty((R,), dtype=torch.int32, device=dev)
            self.scores = torch.full((R, max(1, rg.max_entries)), float("nan"), dtype=torch.float32, device=dev)
        a = _DecodeArgs()
        a.rg = rg.c()
        a.idx_k, a.main_kv, a.blk_sum = _ptr(idx_k), _ptr(main_kv), _ptr(blk_sum)
        a.swa, a.swa_scale, a.q, a.q_idx, a.w_idx = _ptr(swa), _ptr(swa_scale), _ptr(q), _ptr(q_idx), _ptr(w_idx)
        a.k, a.n_keep, a.keep_newest, a.scan_mode = k, n_keep, 1 if keep_newest else 0, scan_mode
        a.qp_route = qp_route
        a.sm_scale = float(sm_scale)
        a.out, a.lse = _ptr(self.out), _ptr(self.lse)
        a.sel_idx, a.n_sel = _ptr(self.sel_idx), _ptr(self.n_sel)
        a.kept_blocks, a.n_kept = _ptr(self.kept), _ptr(self.n_kept)
        a.scores = _ptr(self.scores)
        a.scores_ld = self.scores.shape[-1] if self.scores is not None else 0
        self._args = a
        self.ws_bytes = lib.csa2_decode_workspace_size(ctypes.byref(a))
        self.ws = torch.empty((max(self.ws_bytes, 256),), dtype=torch.uint8, device=dev)
        self._lib = lib

    def run(self, stream: int | None = None, events=None) -> None:
        """Enqueue one decode step; ``events`` is an optional ctypes array of
        DECODE_EVENTS hipEvent_t handles recorded around the stages."""
        self._args.events = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
        _check(self._lib.csa2_decode(ctypes.byref(self._args), _ptr(self.ws), self.ws_bytes,
                                     _stream() if stream is None else stream))


    def run_static(self, stream: int | None = None) -> None:
        """Enqueue one decode step through csa2_decode_static: the library's static
        per-device workspace instead of ``self.ws`` (no allocation; calls on one device
        share that workspace and must not overlap)."""
        self._args.events = None
        _check(self._lib.csa2_decode_static(ctypes.byref(self._args), _stream() if stream is None else stream))


def capture_calls(fns) -> "torch.cuda.CUDAGraph":
    """Capture the launches made by calling each of ``fns`` (in order) into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


def capture_graph(decoders, events=None) -> "torch.cuda.CUDAGraph":
    """Capture one csa2_decode launch chain per decoder (in order) into a HIP graph.

    ``events`` (optional) holds one DECODE_EVENTS handle array per decoder; the event
    records are captured with the kernels.  The decoders must have run eagerly once.
    Replaying the graph re-enqueues every captured step on the current stream.
    """
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, d in enumerate(decoders):
            d.run(events=None if events is None else events[i])
    return g


def decode(rg: Ragged, idx_k, main_kv, blk_sum, swa, swa_scale, q, q_idx, w_idx, **kw) -> Decoder:
    """Run the whole path once; returns the Decoder holding out/lse and intermediates."""
    d = Decoder(rg, idx_k, main_kv, blk_sum, swa, swa_scale, q, q_idx, w_idx, **kw)
    d.run()
    return d


def debug_stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Plain streaming read of ``src`` (a bandwidth reference; reads every byte, writes
    nothing to ``sink`` in practice)."""
    lib = load_library()
    _dev(src, (), "src")
    _dev(sink, (torch.int32,), "sink")
    nbytes = src.numel() * src.element_size()
    _check(lib.csa2_debug_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink), _stream()))


def debug_clock_trace(out: torch.Tensor, n: int, interval: int) -> None:
    """Shader-clock samples on the current stream: out[2i] = shader-clock counter,
    out[2i+1] = 100 MHz reference counter, one pair every ``interval`` reference ticks."""
    lib = load_library()
    _dev(out, (torch.int64,), "out")
    if out.numel() < 2 * n:
        raise ValueError("out holds fewer than 2n values")
    _check(lib.csa2_debug_clock_trace(_ptr(out), int(n), int(interval), _stream()))


def cache_write(rg: Ragged, row_pos, kv_tok, idx_tok, ring_kv, ring_idx, gamma_kv, gamma_idx, main_kv, idx_k,
                blk_sum, eps: float = 1e-6) -> None:
    """csa2_cache_write: pool, normalise, quantise and write the entries the rows complete
    (pools, summaries and ring slots are updated in place)."""
    lib = load_library()
    _dev(row_pos, (torch.int64,), "row_pos")
    _dev(kv_tok, _BF16, "kv_tok")
    _dev(idx_tok, _BF16, "idx_tok")
    _dev(ring_kv, _BF16, "ring_kv")
    _dev(ring_idx, _BF16, "ring_idx")
    _dev(gamma_kv, (torch.float32,), "gamma_kv")
    _dev(gamma_idx, (torch.float32,), "gamma_idx")
    _dev(main_kv, (torch.uint8,), "main_kv")
    _dev(idx_k, (torch.uint8,), "idx_k")
    _dev(blk_sum, _BF16, "blk_sum")
    if row_pos.numel() != rg.num_rows or kv_tok.numel() != rg.num_rows * D or idx_tok.numel() != rg.num_rows * IDX_D:
        raise ValueError("row_pos / kv_tok / idx_tok do not match the rows of rg")
    if ring_kv.numel() < rg.num_requests * D or ring_idx.numel() < rg.num_requests * IDX_D:
        raise ValueError("ring slots must hold one token per request")
    if gamma_kv.numel() != D or gamma_idx.numel() != IDX_D:
        raise ValueError("gamma_kv must hold 512 values and gamma_idx 128")
    _check(lib.csa2_cache_write(ctypes.byref(rg.c()), _ptr(row_pos), _ptr(kv_tok), _ptr(idx_tok), _ptr(ring_kv),
                                _ptr(ring_idx), _ptr(gamma_kv), _ptr(gamma_idx), float(eps), _ptr(main_kv), _ptr(idx_k),
                                _ptr(blk_sum), _stream()))


def debug_mxfp8(x: torch.Tensor) -> torch.Tensor:
    """The attention kernel's MXFP8 rounding over fp32 ``x`` in blocks of 32 values."""
    lib = load_library()
    _dev(x, (torch.float32,), "x")
    out = torch.empty_like(x)
    _check(lib.csa2_debug_mxfp8(_ptr(x), x.numel(), _ptr(out), _stream()))
    return out


def debug_dequant(kind: int, records: torch.Tensor, scales: torch.Tensor | None = None) -> torch.Tensor:
    """The kernels' dequantisation helpers over raw records -> fp32 values."""
    lib = load_library()
    _dev(records, (torch.uint8,), "records")
    n = records.shape[0]
    dim = IDX_D if kind == DQ_IDX else D
    out = torch.empty((n, dim), dtype=torch.float32, device=records.device)
    if scales is not None:
        _dev(scales, (torch.float32,), "scales")
    _check(lib.csa2_debug_dequant(kind, _ptr(records), _ptr(scales), n, _ptr(out), _stream()))
    return out


def version() -> int:
    return int(load_library().csa2_version())
