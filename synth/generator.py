"""Seeded synthetic workloads for the CSA2 decode-time sparse attention path.

What this module does: draw random latents, indexer keys, queries and sliding-window
tokens, and *encode* them into the cache formats the decode path reads:

* main KV entry, 288 B: 512 FP4 E2M1 codes (two per byte, element 2i in the low
  nibble of byte i) followed by 32 E8M0 scale bytes, one per 16 elements;
* indexer key entry, 68 B: 128 FP4 E2M1 codes followed by 4 E8M0 scale bytes, one per
  32 elements;
* block summaries: 128 bf16 per 64-entry block, the mean of the block's indexer keys;
* sliding window: 512 FP8 E4M3FN codes per token plus one fp32 scale per token;
* queries: bf16 bit patterns; indexer head weights: fp32.

The entry sizes (288 B main, 68 B indexer) and the stride-2 pooling of the global
cache come from the SGLang blog post "DeepSeek-V4.1 Flash on SGLang: from 35 to 873
tokens/s", section "Architecture changes and KV cache compression"; the 128-token FP8
window from the clawpit.io article on vLLM, section "SWA bounded replay".

What it does not do: decode any of these formats, score, select or attend.  Both the
HIP path and the oracle read the bytes produced here; neither imports the other.

Random streams.  Every array is drawn from ``numpy.random.default_rng`` seeded with a
tuple ``(seed, stream, request, kind, chunk)``, so chunks can be drawn in parallel and
request ``b`` of a config does not depend on how many requests follow it:

* ``(seed, 0)``                 config-level draws (ragged context lengths);
* ``(seed, 1, b, 1)``           queries of request b: per row, q [64,512] N(0,1), then
                                q_idx [8,128] N(0,1), then w [8] U(0,1);
* ``(seed, 1, b, 2)``           needle positions (distinct, uniform over [0, N_b));
* ``(seed, 1, b, 3, c)``        indexer keys [<=16384, 128] N(0,1) of chunk c;
* ``(seed, 1, b, 4, c)``        main latents [<=16384, 512] N(0,1) of chunk c;
* ``(seed, 1, b, 5)``           window tokens [T_b, 512] N(0,1).
* ``(seed, 2, 1)``              paged copies: the page permutation, then the bytes of
                                spare pages and of the unused tail rows of last pages;
* ``(seed, 3)``                 cache-write inputs: tokens, ring slots, RMSNorm gains.

All draws are float32 (page bytes: uniform uint8 / uint16).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Fixed shapes of the path (dimensions, entry sizes, block sizes).
D_LATENT = 512          # main-KV latent dim = attention K = V dim
N_HEADS = 64            # query heads
D_IDX = 128             # indexer head dim
N_IDX_HEADS = 8         # indexer heads
MAIN_BLOCK = 16         # E8M0 block of the main entry
IDX_BLOCK = 32          # E8M0 block of the indexer entry
MAIN_BYTES = D_LATENT // 2 + D_LATENT // MAIN_BLOCK   # 288
IDX_BYTES = D_IDX // 2 + D_IDX // IDX_BLOCK           # 68
SUMMARY_BLOCK = 64      # entries per coarse block
SWA_LEN = 128           # sliding-window tokens per row
TOP_K = 512
N_KEEP = 64

CHUNK = 16384           # entries per generation chunk (multiple of SUMMARY_BLOCK)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


# ---------------------------------------------------------------------------------
# Encoders (float -> stored format).  Rounding choices here do not affect parity:
# both sides read the bytes.
# ---------------------------------------------------------------------------------

# Round-half-to-even thresholds between consecutive E2M1 magnitudes
# {0, .5, 1, 1.5, 2, 3, 4, 6}: value v moves past midpoint k if v > mid_k, or if
# v == mid_k and code k+1 is even.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])


def encode_fp4_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Encode rows of ``x`` [n, D] float32 as FP4 E2M1 + E8M0 records [n, D/2 + D/block].

    Shared exponent per block: floor(log2(amax)) - 2 (E2M1's largest exponent), the
    OCP MX rule; magnitudes round half-to-even onto the E2M1 grid and saturate at 6.
    """
    n, d = x.shape
    xb = x.reshape(n, d // block, block)
    amax = np.abs(xb).max(axis=2)
    _, e = np.frexp(amax)                     # amax = f * 2**e, f in [0.5, 1)
    sexp = e.astype(np.int32) - 1 - 2
    sexp = np.where(amax > 0, sexp, -127)
    sexp = np.clip(sexp, -127, 127)
    v = np.abs(xb) * np.ldexp(np.float32(1.0), -sexp)[..., None].astype(np.float32)
    mag = np.zeros(v.shape, dtype=np.uint8)
    for k in range(7):
        mag += (v > _E2M1_MID[k]).astype(np.uint8)
        if _E2M1_TIE_UP[k]:
            mag += (v == _E2M1_MID[k]).astype(np.uint8)
    sign = ((xb < 0) & (mag > 0)).astype(np.uint8) << 3
    codes = (mag | sign).reshape(n, d)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    scales = (sexp + 127).astype(np.uint8)
    return np.ascontiguousarray(np.concatenate([packed, scales], axis=1))


def encode_e4m3_tokens(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode rows of ``x`` [t, 512] float32 as FP8 E4M3FN codes + one fp32 scale per row.

    scale = amax / 448 (fp32); each value is x / scale rounded half-to-even onto the
    E4M3FN grid (bias 7, subnormal step 2**-9, max 448), saturating.
    """
    amax = np.abs(x).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(amax > 0, scale, np.float32(1.0)).astype(np.float32)
    v = x.astype(np.float64) / scale[:, None].astype(np.float64)
    a = np.minimum(np.abs(v), 448.0)
    _, e = np.frexp(a)
    expo = e - 1                                  # floor(log2 a) for a > 0
    step = np.where(expo >= -6, np.ldexp(1.0, expo - 3), 2.0 ** -9)
    qv = np.minimum(np.rint(a / step) * step, 448.0)
    _, e2 = np.frexp(qv)
    expo2 = e2 - 1
    is_norm = qv >= 2.0 ** -6
    biased = np.where(is_norm, expo2 + 7, 0)
    mant = np.where(is_norm, qv / np.ldexp(1.0, np.where(is_norm, expo2, 0)) * 8 - 8, qv / 2.0 ** -9)
    mant = np.rint(mant).astype(np.int64)
    code = (biased.astype(np.int64) << 3) | mant
    code = np.where(qv == 0, 0, code)
    sign = ((v < 0) & (qv > 0)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8), scale


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round half to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns with a single round-half-to-even (normal range)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    # Needle keys are built from the bf16 query *values*; widening a bf16 pattern is a
    # shift, not part of the decode path's arithmetic.
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------
# Workload container
# ---------------------------------------------------------------------------------

@dataclass
class Workload:
    """One batch of decode rows over ragged per-request caches (host numpy arrays)."""
    name: str
    seed: int
    n_tokens: list            # original context length per request (info)
    entry_off: np.ndarray     # int64 [B+1]
    block_off: np.ndarray     # int64 [B+1]
    row_off: np.ndarray       # int32 [B+1] rows of request b: row_off[b] .. row_off[b+1]-1
    swa_off: np.ndarray       # int64 [B+1]
    row_req: np.ndarray       # int32 [R]
    row_swa_start: np.ndarray  # int64 [R]
    row_swa_len: np.ndarray   # int32 [R]
    idx_k: np.ndarray         # uint8 [sumN, 68]
    main_kv: np.ndarray       # uint8 [sumN, 288]
    blk_sum: np.ndarray       # uint16 (bf16 bits) [sumNB, 128]
    swa: np.ndarray           # uint8 (E4M3FN) [sumT, 512]
    swa_scale: np.ndarray     # float32 [sumT]
    q: np.ndarray             # uint16 (bf16 bits) [R, 64, 512]
    q_idx: np.ndarray         # uint16 (bf16 bits) [R, 8, 128]
    w: np.ndarray             # float32 [R, 8]
    needles: list = field(default_factory=list)  # per request: int64 positions
    page_table: np.ndarray | None = None   # int32 [B][pages_ld]: paged pools (then the pools are pages)
    total_pages: int = 0
    row_len: np.ndarray | None = None      # int64 [R]: entries each row sees (None: all)
    k: int = TOP_K
    n_keep: int = N_KEEP
    keep_newest: int = 1
    sm_scale: float = float(1.0 / np.sqrt(np.float64(D_LATENT)))

    @property
    def num_requests(self) -> int:
        return len(self.entry_off) - 1

    @property
    def num_rows(self) -> int:
        return int(self.row_req.shape[0])

    def n_entries(self, b: int) -> int:
        return int(self.entry_off[b + 1] - self.entry_off[b])

    @property
    def max_entries(self) -> int:
        return int(np.diff(self.entry_off).max()) if self.num_requests else 0

    @property
    def total_entries(self) -> int:
        return int(self.entry_off[-1])


def _gen_idx_chunk(seed, b, c, n_total, needle_pos, needle_key):
    lo = c * CHUNK
    hi = min(n_total, lo + CHUNK)
    keys = _rng(seed, 1, b, 3, c).standard_normal((hi - lo, D_IDX), dtype=np.float32)
    sel = needle_pos[(needle_pos >= lo) & (needle_pos < hi)]
    if sel.size:
        keys[sel - lo] = needle_key
    nblk = -(-(hi - lo) // SUMMARY_BLOCK)
    pad = nblk * SUMMARY_BLOCK - (hi - lo)
    kp = np.concatenate([keys.astype(np.float64), np.zeros((pad, D_IDX))]) if pad else keys.astype(np.float64)
    sums = kp.reshape(nblk, SUMMARY_BLOCK, D_IDX).sum(axis=1)
    counts = np.full(nblk, SUMMARY_BLOCK, dtype=np.float64)
    counts[-1] = SUMMARY_BLOCK - pad
    summ = bf16_bits_from_f64(sums / counts[:, None])
    return encode_fp4_blocks(keys, IDX_BLOCK), summ


def _gen_main_chunk(seed, b, c, n_total):
    lo = c * CHUNK
    hi = min(n_total, lo + CHUNK)
    lat = _rng(seed, 1, b, 4, c).standard_normal((hi - lo, D_LATENT), dtype=np.float32)
    return encode_fp4_blocks(lat, MAIN_BLOCK)


def make_workload(name: str, seed: int, n_entries: list, rows_per_req: list | int = 1,
                  n_needles: int = 16, swa_len: int | list = SWA_LEN, n_tokens: list | None = None,
                  workers: int | None = None, scan_only: bool = False) -> Workload:
    """Build a workload with request b holding ``n_entries[b]`` global entries.

    Request b has ``rows_per_req[b]`` query rows; its window buffer holds
    ``swa_len + rows - 1`` tokens and row j of the request sees tokens j .. j+swa_len-1
    (the window slides causally with the row's position).  ``swa_len`` may be a list
    (one per request, 0..128).  ``scan_only`` leaves the main-KV pool zero (for
    measuring the indexer scan alone).  Needles: ``n_needles`` distinct positions per request
    whose indexer key is 3x the head-mean of the request's first row's indexer query.
    """
    B = len(n_entries)
    rows = [rows_per_req] * B if isinstance(rows_per_req, int) else list(rows_per_req)
    swl = [swa_len] * B if isinstance(swa_len, int) else list(swa_len)
    assert len(rows) == B and len(swl) == B
    n_entries = [int(n) for n in n_entries]
    nbs = [-(-n // SUMMARY_BLOCK) for n in n_entries]
    T = [swl[b] + rows[b] - 1 if rows[b] > 0 else 0 for b in range(B)]
    entry_off = np.zeros(B + 1, dtype=np.int64)
    entry_off[1:] = np.cumsum(n_entries)
    block_off = np.zeros(B + 1, dtype=np.int64)
    block_off[1:] = np.cumsum(nbs)
    row_off = np.zeros(B + 1, dtype=np.int32)
    row_off[1:] = np.cumsum(rows)
    swa_off = np.zeros(B + 1, dtype=np.int64)
    swa_off[1:] = np.cumsum(T)
    R = int(row_off[-1])

    q = np.zeros((R, N_HEADS, D_LATENT), dtype=np.uint16)
    q_idx = np.zeros((R, N_IDX_HEADS, D_IDX), dtype=np.uint16)
    w = np.zeros((R, N_IDX_HEADS), dtype=np.float32)
    row_req = np.zeros(R, dtype=np.int32)
    row_swa_start = np.zeros(R, dtype=np.int64)
    row_swa_len = np.zeros(R, dtype=np.int32)
    idx_k = np.zeros((int(entry_off[-1]), IDX_BYTES), dtype=np.uint8)
    main_kv = np.zeros((int(entry_off[-1]), MAIN_BYTES), dtype=np.uint8)
    blk_sum = np.zeros((int(block_off[-1]), D_IDX), dtype=np.uint16)
    swa = np.zeros((int(swa_off[-1]), D_LATENT), dtype=np.uint8)
    swa_scale = np.ones(int(swa_off[-1]), dtype=np.float32)
    needles = []

    jobs = []
    for b in range(B):
        rq = _rng(seed, 1, b, 1)
        for j in range(rows[b]):
            r = int(row_off[b]) + j
            q[r] = bf16_bits_from_f32(rq.standard_normal((N_HEADS, D_LATENT), dtype=np.float32))
            q_idx[r] = bf16_bits_from_f32(rq.standard_normal((N_IDX_HEADS, D_IDX), dtype=np.float32))
            w[r] = rq.random(N_IDX_HEADS, dtype=np.float32)
            row_req[r] = b
            row_swa_start[r] = swa_off[b] + j
            row_swa_len[r] = swl[b]
        n = n_entries[b]
        nn = min(n_needles, n)
        pos = np.sort(_rng(seed, 1, b, 2).choice(n, size=nn, replace=False)).astype(np.int64) if nn else \
            np.zeros(0, dtype=np.int64)
        needles.append(pos)
        if rows[b] > 0:
            nkey = (3.0 * _bf16_bits_to_f64(q_idx[int(row_off[b])]).mean(axis=0)).astype(np.float32)
        else:
            nkey = np.zeros(D_IDX, dtype=np.float32)
        for c in range(-(-n // CHUNK)):
            jobs.append((b, c, n, pos, nkey))
        if T[b]:
            x = _rng(seed, 1, b, 5).standard_normal((T[b], D_LATENT), dtype=np.float32)
            codes, sc = encode_e4m3_tokens(x)
            swa[swa_off[b]:swa_off[b + 1]] = codes
            swa_scale[swa_off[b]:swa_off[b + 1]] = sc

    def run(job):
        b, c, n, pos, nkey = job
        ik, summ = _gen_idx_chunk(seed, b, c, n, pos, nkey)
        e0 = int(entry_off[b]) + c * CHUNK
        idx_k[e0:e0 + ik.shape[0]] = ik
        if not scan_only:
            mk = _gen_main_chunk(seed, b, c, n)
            main_kv[e0:e0 + mk.shape[0]] = mk
        b0 = int(block_off[b]) + c * (CHUNK // SUMMARY_BLOCK)
        blk_sum[b0:b0 + summ.shape[0]] = summ

    nw = workers or min(16, len(os.sched_getaffinity(0)))
    if len(jobs) > 1 and nw > 1:
        with ThreadPoolExecutor(max_workers=nw) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)

    return Workload(name=name, seed=seed, n_tokens=list(n_tokens or n_entries),
                    entry_off=entry_off, block_off=block_off, row_off=row_off, swa_off=swa_off,
                    row_req=row_req, row_swa_start=row_swa_start, row_swa_len=row_swa_len,
                    idx_k=idx_k, main_kv=main_kv, blk_sum=blk_sum, swa=swa, swa_scale=swa_scale,
                    q=q, q_idx=q_idx, w=w, needles=needles)


def to_paged(wl: Workload, seed: int | None = None, spare_pages: int | None = None) -> Workload:
    """The same logical workload over paged pools.

    The idx_k / main_kv pools are cut into 64-entry pages and the summary pool into one
    summary per page; request b's page j (entries 64j .. 64j+63, summary j) goes to a
    physical page drawn by a seeded permutation of all pages, so a request's pages are
    scattered and interleaved with other requests'.  ``spare_pages`` extra pages (default
    about 1/8 of the total) and the unused tail rows of each request's last page hold
    random bytes, so any read outside the page table's entries changes the results.
    Page-table slots past a request's last page are -1.
    """
    seed = wl.seed if seed is None else seed
    B = wl.num_requests
    nbs = [-(-wl.n_entries(b) // SUMMARY_BLOCK) for b in range(B)]
    used = int(sum(nbs))
    spare = max(1, used // 8) if spare_pages is None else int(spare_pages)
    P = used + spare
    rng = _rng(seed, 2, 1)
    perm = rng.permutation(P).astype(np.int32)
    pages_ld = max([1] + nbs)
    page_table = np.full((B, pages_ld), -1, dtype=np.int32)
    idx_k = rng.integers(0, 256, size=(P * SUMMARY_BLOCK, IDX_BYTES), dtype=np.uint8)
    main_kv = rng.integers(0, 256, size=(P * SUMMARY_BLOCK, MAIN_BYTES), dtype=np.uint8)
    blk_sum = rng.integers(0, 1 << 16, size=(P, D_IDX), dtype=np.uint16)
    i = 0
    for b in range(B):
        e0, n = int(wl.entry_off[b]), wl.n_entries(b)
        for j in range(nbs[b]):
            p = int(perm[i])
            i += 1
            page_table[b, j] = p
            lo, hi = 64 * j, min(n, 64 * j + 64)
            idx_k[64 * p:64 * p + hi - lo] = wl.idx_k[e0 + lo:e0 + hi]
            main_kv[64 * p:64 * p + hi - lo] = wl.main_kv[e0 + lo:e0 + hi]
            blk_sum[p] = wl.blk_sum[int(wl.block_off[b]) + j]
    out = Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
    out.name = wl.name + "_paged"
    out.idx_k, out.main_kv, out.blk_sum = idx_k, main_kv, blk_sum
    out.page_table, out.total_pages = page_table, P
    return out


def make_write_inputs(wl: Workload, seed: int, last_even: bool = True) -> dict:
    """Inputs of a cache write for the rows of ``wl``: the rows of request b hold
    consecutive token positions ending at 2 N_b (even: that token waits in the ring slot)
    or 2 N_b - 1 (odd: it completes entry N_b - 1), so the write fills the request's last
    entries; tokens, ring slots N(0,1) as bf16; RMSNorm gains U(0.5, 1.5).  Random stream
    ``(seed, 3)``."""
    rng = _rng(seed, 3)
    R, B = wl.num_rows, wl.num_requests
    pos = np.zeros(R, dtype=np.int64)
    for b in range(B):
        r0, r1 = int(wl.row_off[b]), int(wl.row_off[b + 1])
        last = 2 * wl.n_entries(b) if last_even else 2 * wl.n_entries(b) - 1
        pos[r0:r1] = last - (r1 - r0) + 1 + np.arange(r1 - r0)
    return dict(
        row_pos=pos,
        kv_tok=bf16_bits_from_f32(rng.standard_normal((R, D_LATENT), dtype=np.float32)),
        idx_tok=bf16_bits_from_f32(rng.standard_normal((R, D_IDX), dtype=np.float32)),
        ring_kv=bf16_bits_from_f32(rng.standard_normal((B, D_LATENT), dtype=np.float32)),
        ring_idx=bf16_bits_from_f32(rng.standard_normal((B, D_IDX), dtype=np.float32)),
        gamma_kv=rng.uniform(0.5, 1.5, D_LATENT).astype(np.float32),
        gamma_idx=rng.uniform(0.5, 1.5, D_IDX).astype(np.float32),
    )


def verify_row_len(wl: Workload) -> np.ndarray:
    """Entries each row sees when the rows of a request are consecutive verify positions.

    Row j of a request with m rows sits m-1-j tokens before the request's last row; with
    two tokens pooled per global entry and the last row completing a pair, it sees
    N_b - ceil((m-1-j)/2) entries (at least 0)."""
    rl = np.zeros(wl.num_rows, dtype=np.int64)
    for b in range(wl.num_requests):
        r0, r1 = int(wl.row_off[b]), int(wl.row_off[b + 1])
        m = r1 - r0
        for j in range(m):
            rl[r0 + j] = max(0, wl.n_entries(b) - (m - j) // 2)
    return rl


# ---------------------------------------------------------------------------------
# The five decode workloads (plus the derived bandwidth case)
# ---------------------------------------------------------------------------------

CONFIGS = {
    0: "tiny_4k",          # 1 request x 1 row, 4096 tokens pooled stride-2 -> 2048 entries, seed 0
    1: "long_128k",        # 1 x 1, 131072 tokens -> 65536 entries, seed 1
    2: "batched_32",       # 32 x 1, tokens ~ U{4096..65536} pooled, seed 2
    3: "verify_8x6",       # 8 x 6 rows, 32768 tokens -> 16384 entries, seed 3
    4: "unpooled_1m",      # 4 x 1, 1048576 tokens, one entry per token, 64 needles, seed 4
    5: "long_128k_x64",    # 64 x 1, each shaped like long_128k (scan-bandwidth case), seed 1
}


def config_lengths(i: int) -> tuple[list, list, int, int, int]:
    """(original tokens per request, entries per request, rows/request, needles, seed)."""
    if i == 0:
        return [4096], [2048], 1, 16, 0
    if i == 1:
        return [131072], [65536], 1, 16, 1
    if i == 2:
        toks = [int(t) for t in _rng(2, 0).integers(4096, 65536, size=32, endpoint=True)]
        return toks, [t // 2 for t in toks], 1, 16, 2
    if i == 3:
        return [32768] * 8, [16384] * 8, 6, 16, 3
    if i == 4:
        return [1 << 20] * 4, [1 << 20] * 4, 1, 64, 4
    if i == 5:
        return [131072] * 64, [65536] * 64, 1, 16, 1
    raise ValueError(f"unknown config {i}")


def make_config(i: int, workers: int | None = None, scan_only: bool = False) -> Workload:
    """Workload i; scan_only skips the attention-side pools (main KV, window)."""
    toks, ents, rows, needles, seed = config_lengths(i)
    return make_workload(CONFIGS[i], seed, ents, rows, n_needles=needles, n_tokens=toks, workers=workers,
                         scan_only=scan_only)
