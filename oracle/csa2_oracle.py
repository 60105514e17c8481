"""fp64 CPU oracle of the CSA2 decode-time sparse attention path.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``; nothing in the product path imports it.  It shares
no code with the HIP library or with the input generator: it receives plain numpy arrays
(raw cache bytes, bf16 bit patterns, fp32 weights and integer offsets) and decodes them
itself.

Sources (web pages, cited by title and section):
  [SGL] "DeepSeek-V4.1 Flash on SGLang: from 35 to 873 tokens/s" (sglang.io blog)
        - "Architecture changes and KV cache compression": global entries are pooled
          two tokens per entry (one per token in the last cache), stored in FP4 at 288 B
          (main KV) and 68 B (indexer key); a hierarchical candidate filter narrows the
          indexer's search so that only the top 512 global positions enter attention.
        - "DSpark adaptation and optimization": chosen candidate blocks expand straight
          into a token mask; a verify step handles up to 6 rows per request.
  [VLLM] "DeepSeek-V4.1-Flash runs 5.3x faster on vLLM after three weeks of optimization"
        - "SWA bounded replay": the sliding-window cache is FP8 and covers the most
          recent 128 positions.
  [KT]  ktransformers issue "Support for Deepseek V4.1 Flash" (mirror): the indexer is
        two-level; attention is sparse MLA.

The pages fix the structure but not the arithmetic.  The definitions below complete
them (each is restated where it is used):
  * main entry   = 512 E2M1 codes (element 2i in the low nibble of byte i) then 32 E8M0
                   scales, one per 16 elements (256 + 32 = 288 B);
  * indexer key  = 128 E2M1 codes then 4 E8M0 scales, one per 32 elements (64 + 4 = 68 B);
  * window token = 512 E4M3FN codes and one fp32 scale;
  * index score  s_t = sum_{h<8} w_h * max(0, q_h . k_t), head dim 128;
  * coarse stage = the same score on each 64-entry block's bf16 summary key; keep the
                   64 best blocks (ties to the lower block) plus the newest block;
  * fine stage   = the 512 best scores among the kept blocks' entries (ties to the
                   lower position), reported in ascending position;
  * attention    = MQA over the 512-dim latent (K = V = latent) for 64 heads, one
                   softmax jointly over the selected entries and the row's window,
                   logit scale 1/sqrt(512), no de-duplication, no sink.

[SGL] "DSpark adaptation and optimization" also names a valid-length check fused into
the candidate mask and a post-top-k step that checks scores, filters invalid positions
and translates positions into KV page addresses.  Read here as:
  * row visibility: a row may see only the first V_r entries of its request (verify
                   rows sit at consecutive positions); the row then works on the request
                   cut to V_r entries: blocks 0 .. ceil(V_r/64)-1, candidates < V_r;
  * score check  : a NaN score (possible through an E8M0 NaN scale) is never ranked;
                   since NaN would rank below every number, dropping NaN picks after the
                   top-k gives the same set;
  * invalid positions: selected positions outside 0 .. V_r-1 carry no key;
  * pages        : the pools may be cut into 64-entry pages; entry t of request b is
                   then at row 64 * page_table[b][t // 64] + t % 64 and its block's
                   summary at row page_table[b][t // 64].

[KT] contrasts full-BF16 sparse MLA with a route that rounds Q and P to MXFP8 (OCP MX:
E4M3 elements, one E8M0 scale per 32 values); joint_attention_mx states that route.

[SGL] "Small-operator fusion and GEMV" and "DSpark adaptation and optimization" name the
fused cache-write chain (pair pooling, RMSNorm, FP4 quantisation, cache write, reused for
index K; verify rows pool with the previous row, the first row with a ring buffer) but
not its arithmetic; cache_write takes the plainest reading: the mean of the two tokens,
x * gamma / sqrt(mean(x^2) + eps), OCP MX FP4, and block summaries as the bf16 mean of the
block's dequantised index keys.

Every function here is pinned by tests in tests/test_formats.py and tests/test_oracle.py
(format tables against a library decoder and the OCP MX value table, brute-force exact
rational scores, brute-force selection, the dense-attention special case, LSE merging
and invariants).
"""
from __future__ import annotations

import math

import numpy as np

D = 512            # latent dim (attention K = V)
H = 64             # query heads
D_IDX = 128        # indexer head dim
H_IDX = 8          # indexer heads
BLOCK = 64         # entries per coarse block
MAIN_BYTES = 288
IDX_BYTES = 68
SCAN_CHUNK = 65536  # entries dequantised at a time (keeps 1M-entry requests in memory)


# ---------------------------------------------------------------------------------
# O1. Formats, decoded from their bit-field definitions.
# ---------------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """OCP MX FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal (0.5 * m); otherwise 2**(e-1) * (1 + m/2).  There is
    no inf or NaN.
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e8m0_value(u: int) -> float:
    """OCP MX E8M0 scale: 2**(u - 127); code 255 is NaN."""
    return math.nan if u == 255 else 2.0 ** (u - 127)


def e4m3fn_value(c: int) -> float:
    """OCP FP8 E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.

    Exponent field 0 is subnormal (m/8 * 2**-6); exponent 15 with mantissa 7 is NaN;
    no inf (largest finite 448).
    """
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 15 and m == 7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0 = np.array([e8m0_value(u) for u in range(256)], dtype=np.float64)
E4M3 = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> their exact values (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_fp4_records(rec: np.ndarray, dim: int, block: int) -> np.ndarray:
    """Records [n, dim/2 + dim/block] of E2M1 codes + E8M0 scales -> exact values [n, dim]."""
    rec = np.asarray(rec, dtype=np.uint8)
    codes = rec[:, : dim // 2]
    vals = np.empty((rec.shape[0], dim), dtype=np.float64)
    vals[:, 0::2] = E2M1[codes & 0x0F]
    vals[:, 1::2] = E2M1[codes >> 4]
    scale = E8M0[rec[:, dim // 2: dim // 2 + dim // block]]
    return vals * np.repeat(scale, block, axis=1)


def dequant_main(rec: np.ndarray) -> np.ndarray:
    """288-B main KV records -> [n, 512] (E8M0 block 16)."""
    return dequant_fp4_records(rec, D, 16)


def dequant_idx(rec: np.ndarray) -> np.ndarray:
    """68-B indexer key records -> [n, 128] (E8M0 block 32)."""
    return dequant_fp4_records(rec, D_IDX, 32)


def dequant_swa(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E4M3FN codes [t, 512] and fp32 scales [t] -> [t, 512] (exact in fp64)."""
    return E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


# ---------------------------------------------------------------------------------
# O2/O3. Indexer score, on entries and on block summaries.
# ---------------------------------------------------------------------------------

def indexer_score(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s_t = sum_h w_h * max(0, q_h . k_t) for every row k_t of ``keys``.

    q_idx: [8, 128] exact query values, w: [8], keys: [n, 128] exact key values.
    """
    dots = keys @ np.asarray(q_idx, dtype=np.float64).T          # [n, 8]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------------------------
# O4. Coarse block filter.
# ---------------------------------------------------------------------------------

def keep_blocks(block_scores: np.ndarray, n_keep: int = 64, keep_newest: bool = True) -> np.ndarray:
    """Blocks kept by the coarse stage, ascending.

    Blocks with a NaN score are not ranked (score check).  With at most n_keep ranked
    blocks all of them are kept; otherwise order them by (score desc, block asc) and keep
    the first n_keep.  Then add the newest block (nb-1) if it is not among them.
    """
    bs = np.asarray(block_scores, dtype=np.float64)
    nb = int(bs.shape[0])
    ranked = np.flatnonzero(~np.isnan(bs))
    if ranked.size <= n_keep:
        kept = set(int(j) for j in ranked)
    else:
        order = np.lexsort((ranked, -bs[ranked]))
        kept = set(int(j) for j in ranked[order[:n_keep]])
    if keep_newest and nb > 0:
        kept.add(nb - 1)
    return np.array(sorted(kept), dtype=np.int64)


def blocks_to_entries(kept: np.ndarray, n_entries: int) -> np.ndarray:
    """Expand kept blocks into their entry positions (the newest block may be partial)."""
    parts = [np.arange(BLOCK * j, min(BLOCK * (j + 1), n_entries), dtype=np.int64) for j in kept]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------------
# O5/O6. Fine top-k.
# ---------------------------------------------------------------------------------

def top_k(positions: np.ndarray, scores: np.ndarray, k: int) -> np.ndarray:
    """The k best (score desc, position asc) of the candidates whose score is not NaN,
    reported ascending."""
    positions = np.asarray(positions, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    ok = ~np.isnan(scores)
    positions, scores = positions[ok], scores[ok]
    order = np.lexsort((positions, -scores))
    return np.sort(positions[order[:k]])


# ---------------------------------------------------------------------------------
# O7. Joint-softmax latent attention.
# ---------------------------------------------------------------------------------

def joint_attention(q: np.ndarray, keys: np.ndarray, sm_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """For each head h: z_i = sm_scale * q_h . x_i, out_h = sum_i softmax(z)_i x_i, lse_h.

    q: [64, 512] exact query values; keys: [n, 512] exact latents (K = V).  With n = 0
    the output is 0 and the log-sum-exp is -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], D)), np.full(q.shape[0], -np.inf)
    z = (q @ keys.T) * float(sm_scale)                            # [64, n]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    s = p.sum(axis=1, keepdims=True)
    out = (p @ keys) / s
    lse = (m + np.log(s))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------------
# O8. The cache write (the step before the path): [SGL] "Small-operator fusion and
# GEMV" fuses pooling, RMSNorm, FP4 quantisation and the cache write; "DSpark
# adaptation and optimization": verify rows pool with the previous row, only a
# request's first row reads the ring buffer, and the same write serves index K.
# ---------------------------------------------------------------------------------

E2M1_GRID = E2M1[:8]            # magnitudes of codes 0 .. 7: 0, .5, 1, 1.5, 2, 3, 4, 6


def fp4_encode(y: np.ndarray, block: int) -> tuple[np.ndarray, np.ndarray]:
    """OCP MX FP4 of each row of y [n, dim]: per block the E8M0 exponent
    e = floor(log2(block amax)) - 2 (E2M1's largest exponent; -127 for an all-zero
    block), clamped to -127 .. 127; each element the E2M1 code nearest to y / 2^e (ties to
    the even code, magnitudes above 6 to 6).  Returns (codes [n, dim] uint8, exponents
    [n, dim/block] int)."""
    y = np.asarray(y, dtype=np.float64)
    n, dim = y.shape
    yb = y.reshape(n, dim // block, block)
    amax = np.abs(yb).max(axis=2)
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, np.clip(fe - 1 - 2, -127, 127), -127)
    v = np.abs(yb) / np.ldexp(1.0, e)[..., None]
    d = np.abs(v[..., None] - E2M1_GRID)                          # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    ties = d == best
    # Among equally near magnitudes take the even code (codes are 0..7, ascending).
    even = ties & (np.arange(8) % 2 == 0)
    mag = np.where(even.any(axis=-1), even.argmax(axis=-1), ties.argmax(axis=-1))
    sign = (yb < 0) & (mag > 0)
    codes = (mag | (sign.astype(np.int64) << 3)).reshape(n, dim).astype(np.uint8)
    return codes, e.astype(np.int64)


def pack_fp4_record(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Records of the stored layout: element 2i in the low nibble of byte i, then the
    E8M0 bytes e + 127."""
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, (exps + 127).astype(np.uint8)], axis=1)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp64 values, one round to nearest even (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                          # x = m 2^e, |m| in [0.5, 1)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)               # 8 significant bits
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x * gamma / sqrt(mean(x^2) + eps) per row."""
    x = np.asarray(x, dtype=np.float64)
    return x * np.asarray(gamma, dtype=np.float64) / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


def cache_write(wl, row_pos, kv_tok, idx_tok, ring_kv, ring_idx, gamma_kv, gamma_idx, eps: float = 1e-6) -> dict:
    """The cache write on copies of wl's pools.  Row r (a token at position row_pos[r];
    a request's rows hold consecutive positions) at an odd position P completes entry
    t = (P-1)/2 of its request if t < N_b: pooled = mean of the token at P-1 (the previous
    row if it holds P-1, else the request's ring slot) and the row's own token; main and
    index vectors each go through rms_norm and fp4_encode (blocks 16 / 32) into the
    entry's records.  Each block that received an entry gets as summary the bf16 of the
    mean of its entries' dequantised index keys; a request whose last row has an even
    position moves that row's tokens into its ring slot.  Returns the updated pools and
    ring slots plus, per written entry, the normalised vectors ``y_kv`` / ``y_idx``."""
    main = np.array(wl.main_kv, copy=True)
    idx = np.array(wl.idx_k, copy=True)
    summ = np.array(wl.blk_sum, copy=True)
    rkv = np.array(ring_kv, copy=True)
    ridx = np.array(ring_idx, copy=True)
    written = {}
    for b in range(wl.num_requests):
        r0, r1 = int(wl.row_off[b]), int(wl.row_off[b + 1])
        n = int(wl.entry_off[b + 1] - wl.entry_off[b])
        ts = []
        for r in range(r0, r1):
            p = int(row_pos[r])
            if p < 0 or p % 2 == 0 or (p - 1) // 2 >= n:
                continue
            t = (p - 1) // 2
            if r > r0 and int(row_pos[r - 1]) == p - 1:
                pk, pi = kv_tok[r - 1], idx_tok[r - 1]
            else:
                pk, pi = ring_kv[b], ring_idx[b]
            xk = (bf16_value(pk) + bf16_value(kv_tok[r])) / 2
            xi = (bf16_value(pi) + bf16_value(idx_tok[r])) / 2
            yk = rms_norm(xk[None, :], gamma_kv, eps)
            yi = rms_norm(xi[None, :], gamma_idx, eps)
            row = int(entry_rows(wl, b, np.array([t]))[0])
            main[row] = pack_fp4_record(*fp4_encode(yk, 16))[0]
            idx[row] = pack_fp4_record(*fp4_encode(yi, 32))[0]
            written[(b, t)] = (yk[0], yi[0])
            ts.append(t)
        for j in sorted(set(t // BLOCK for t in ts)):
            cnt = min(BLOCK, n - BLOCK * j)
            keys = dequant_idx(idx[entry_rows(wl, b, np.arange(BLOCK * j, BLOCK * j + cnt))])
            summ[int(block_rows(wl, b, j + 1)[j])] = bf16_rne(keys.mean(axis=0))
        if r1 > r0 and int(row_pos[r1 - 1]) >= 0 and int(row_pos[r1 - 1]) % 2 == 0:
            rkv[b] = kv_tok[r1 - 1]
            ridx[b] = idx_tok[r1 - 1]
    return dict(main_kv=main, idx_k=idx, blk_sum=summ, ring_kv=rkv, ring_idx=ridx, written=written)


# ---------------------------------------------------------------------------------
# O7b. The MXFP8 Q/P route of the attention ([KT]: sparse MLA with Q and P rounded to
# MXFP8 instead of full BF16).
# ---------------------------------------------------------------------------------

E4M3_GRID = E4M3[:127]          # codes 0 .. 126: the non-negative finite values, ascending


def mxfp8_round(x: np.ndarray, block: int = 32) -> np.ndarray:
    """OCP MX rounding of the last axis in blocks of ``block`` values (MXFP8: E4M3
    elements, one E8M0 scale per block): shared exponent s = floor(log2(block amax)) - 8
    (8 = E4M3's largest exponent), clamped to -127 .. 127; each value becomes the E4M3
    value nearest to x / 2^s (ties to the even code, magnitudes above 448 to 448) times
    2^s.  The last axis is zero-padded to whole blocks for the scale and cut back."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    nb = -(-n // block)
    xp = np.zeros(x.shape[:-1] + (nb * block,))
    xp[..., :n] = x
    xb = xp.reshape(x.shape[:-1] + (nb, block))
    amax = np.abs(xb).max(axis=-1, keepdims=True)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))          # amax = f * 2^e, f in [0.5, 1)
    s = np.clip(e - 1 - 8, -127, 127)
    s = np.where(amax > 0, s, -127)
    y = np.minimum(np.abs(xb) / np.ldexp(1.0, s), 448.0)
    hi = np.clip(np.searchsorted(E4M3_GRID, y), 1, 126)   # first grid value >= y
    lo = hi - 1
    dl, dh = y - E4M3_GRID[lo], E4M3_GRID[hi] - y
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(y == 0, 0, code)
    r = np.sign(xb) * E4M3_GRID[code] * np.ldexp(1.0, s)
    return r.reshape(xp.shape)[..., :n]


def joint_attention_mx(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, sm_scale: float,
                       with_bound: bool = False):
    """The MXFP8 route for each head: q' = MXFP8(q) in blocks of 32 latent dims; key i is
    scales[i] * codes[i] (a main entry: its exact latent with scale 1; a window token: its
    E4M3 code values and fp32 scale); z_i = sm_scale * q' . key_i, p_i = exp(z_i - max z),
    the weight on key i's codes w_i = p_i * scales[i] is rounded to MXFP8 in blocks of 32
    consecutive keys, out = sum_i w'_i codes_i / sum_i p_i, lse = max z + log sum p.

    with_bound: also return, per (head, dim), what two independent roundings of w to E4M3
    (here and in an implementation that rounds w times a factor >= 1 and divides it out
    later) can move out by.  One rounding moves a value by at most 2^-3 of itself in
    E4M3's normal range (half a grid step is 2^-4 relative; a block maximum between 448
    and 512 grid units saturates to 448, up to 1/8 below), and in the subnormal range by
    at most 2^-10 * 2^s here and 2^-9 * 2^s there, so the bound is
    sum_i (2^-2 |w_i| + 2^-8 * 2^s_i) |codes_i| / sum p.
    """
    q = np.asarray(q, dtype=np.float64)
    codes = np.asarray(codes, dtype=np.float64)
    scales = np.asarray(scales, dtype=np.float64)
    H = q.shape[0]
    if codes.shape[0] == 0:
        out = np.zeros((H, D))
        lse = np.full(H, -np.inf)
        return (out, lse, np.zeros((H, D))) if with_bound else (out, lse)
    qm = mxfp8_round(q)
    z = (qm @ codes.T) * scales[None, :] * float(sm_scale)          # [H, n]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    w = p * scales[None, :]
    wm = mxfp8_round(w)
    out = (wm @ codes) / l
    lse = (m + np.log(l))[:, 0]
    if not with_bound:
        return out, lse
    n = w.shape[1]
    nb = -(-n // 32)
    wp = np.zeros((H, nb * 32))
    wp[:, :n] = np.abs(w)
    amax = wp.reshape(H, nb, 32).max(axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    step = np.ldexp(1.0, np.clip(e - 1 - 8, -127, 127) - 8)        # twice E4M3's subnormal step * 2^s
    step = np.repeat(np.where(amax > 0, step, 0.0), 32, axis=1)[:, :n]
    bound = ((2.0 ** -2) * np.abs(w) + step) @ np.abs(codes) / l
    return out, lse, bound


def row_key_codes(wl, r: int, sel: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The row's attention keys as (codes, scales): the selected main entries' exact
    latents with scale 1, then the window tokens' E4M3 code values and fp32 scales."""
    b = int(wl.row_req[r])
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < visible(wl, r))]
    main = dequant_main(wl.main_kv[entry_rows(wl, b, sel)])
    s0 = int(wl.row_swa_start[r])
    s1 = s0 + int(wl.row_swa_len[r])
    win = E4M3[np.asarray(wl.swa[s0:s1], dtype=np.int64)].reshape(-1, D)
    codes = np.concatenate([main, win], axis=0)
    scales = np.concatenate([np.ones(main.shape[0]), np.asarray(wl.swa_scale[s0:s1], dtype=np.float64)])
    return codes, scales


# ---------------------------------------------------------------------------------
# The whole path for one workload.
# ---------------------------------------------------------------------------------

def entry_rows(wl, b: int, t: np.ndarray) -> np.ndarray:
    """Pool rows of entries ``t`` of request b: entry_off[b] + t, or with a page table
    64 * page_table[b][t // 64] + t % 64."""
    t = np.asarray(t, dtype=np.int64)
    pt = getattr(wl, "page_table", None)
    if pt is None:
        return int(wl.entry_off[b]) + t
    return np.asarray(pt[b], dtype=np.int64)[t // BLOCK] * BLOCK + t % BLOCK


def block_rows(wl, b: int, nb: int) -> np.ndarray:
    """Summary-pool rows of blocks 0 .. nb-1 of request b."""
    j = np.arange(nb, dtype=np.int64)
    pt = getattr(wl, "page_table", None)
    if pt is None:
        return int(wl.block_off[b]) + j
    return np.asarray(pt[b], dtype=np.int64)[j]


def visible(wl, r: int) -> int:
    """Entries row r sees: N_b, or its row length clamped to 0 .. N_b."""
    b = int(wl.row_req[r])
    n = int(wl.entry_off[b + 1] - wl.entry_off[b])
    rl = getattr(wl, "row_len", None)
    return n if rl is None else min(max(int(rl[r]), 0), n)


def request_scores(wl, b: int) -> np.ndarray:
    """Index scores of every entry of request b for each of its rows: [rows_b, N_b]."""
    r0, r1 = int(wl.row_off[b]), int(wl.row_off[b + 1])
    n = int(wl.entry_off[b + 1] - wl.entry_off[b])
    out = np.zeros((r1 - r0, n), dtype=np.float64)
    qs = [bf16_value(wl.q_idx[r]) for r in range(r0, r1)]
    for c0 in range(0, n, SCAN_CHUNK):
        c1 = min(n, c0 + SCAN_CHUNK)
        keys = dequant_idx(wl.idx_k[entry_rows(wl, b, np.arange(c0, c1))])
        for j, r in enumerate(range(r0, r1)):
            out[j, c0:c1] = indexer_score(qs[j], wl.w[r], keys)
    return out


def block_scores_row(wl, r: int) -> np.ndarray:
    """Scores of the blocks row r sees (ceil(V_r / 64) of them)."""
    b = int(wl.row_req[r])
    nb = -(-visible(wl, r) // BLOCK)
    summ = bf16_value(wl.blk_sum[block_rows(wl, b, nb)])
    return indexer_score(bf16_value(wl.q_idx[r]), wl.w[r], summ)


def row_keys(wl, r: int, sel: np.ndarray) -> np.ndarray:
    """The row's attention keys: the selected main entries that are valid positions
    (0 .. V_r-1; others carry no key), then its window tokens."""
    b = int(wl.row_req[r])
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < visible(wl, r))]
    main = dequant_main(wl.main_kv[entry_rows(wl, b, sel)])
    s0 = int(wl.row_swa_start[r])
    s1 = s0 + int(wl.row_swa_len[r])
    win = dequant_swa(wl.swa[s0:s1], wl.swa_scale[s0:s1])
    return np.concatenate([main, win], axis=0)


def decode(wl, rows=None, k: int | None = None, n_keep: int | None = None, keep_newest: int | None = None,
           kept_override: dict | None = None, sel_override: dict | None = None) -> list:
    """Run the path for ``rows`` (default: all) and return one dict per row.

    Each dict holds: ``kept`` (ascending blocks), ``block_scores`` [nb], ``cand``
    (candidate positions), ``cand_scores``, ``sel`` (ascending positions), ``out``
    [64, 512], ``lse`` [64].  ``kept_override`` / ``sel_override`` map a row to a kept
    set / selected set to use instead of the oracle's own (to re-run the later steps on
    another implementation's choices).
    """
    k = wl.k if k is None else k
    n_keep = wl.n_keep if n_keep is None else n_keep
    keep_newest = wl.keep_newest if keep_newest is None else keep_newest
    R = int(wl.row_req.shape[0])
    rows = list(range(R)) if rows is None else list(rows)
    by_req: dict = {}
    for r in rows:
        by_req.setdefault(int(wl.row_req[r]), []).append(r)
    res = {}
    for b, rs in by_req.items():
        n = int(wl.entry_off[b + 1] - wl.entry_off[b])
        sc = request_scores(wl, b) if n else np.zeros((int(wl.row_off[b + 1] - wl.row_off[b]), 0))
        for r in rs:
            s = sc[r - int(wl.row_off[b])]
            bs = block_scores_row(wl, r)
            if kept_override is not None and r in kept_override:
                kept = np.asarray(kept_override[r], dtype=np.int64)
            else:
                kept = keep_blocks(bs, n_keep, bool(keep_newest))
            cand = blocks_to_entries(kept, visible(wl, r))
            cs = s[cand]
            if sel_override is not None and r in sel_override:
                sel = np.asarray(sel_override[r], dtype=np.int64)
            else:
                sel = top_k(cand, cs, k)
            out, lse = joint_attention(bf16_value(wl.q[r]), row_keys(wl, r, sel), wl.sm_scale)
            res[r] = dict(kept=kept, block_scores=bs, cand=cand, cand_scores=cs, scores=s, sel=sel,
                          out=out, lse=lse)
    return [res[r] for r in rows]
