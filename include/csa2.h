/*
 * csa2.h -- C ABI of libcsa2, the decode-time CSA2 sparse attention path on MI355X
 * (gfx950).
 *
 * For each query row the path
 *   (1) scores every global entry of the row's request through its FP4 indexer key,
 *   (2) narrows the candidates coarse-to-fine: score each 64-entry block's bf16
 *       summary key, keep the best n_keep blocks plus the newest block, then take the
 *       k best entries of the kept blocks,
 *   (3) runs 64-head latent (MQA) attention with one softmax over the k gathered FP4
 *       main entries and the row's FP8 sliding window.
 *
 * Sources: SGLang blog "DeepSeek-V4.1 Flash on SGLang: from 35 to 873 tokens/s",
 * section "Architecture changes and KV cache compression" (FP4 entries of 288 B main KV
 * and 68 B indexer key; a hierarchical candidate filter keeps the top 512 positions)
 * and section "DSpark adaptation and optimization" (kept candidate blocks expand into
 * a token mask; up to 6 verify rows per request); clawpit.io article "DeepSeek-V4.1-
 * Flash runs 5.3x faster on vLLM after three weeks of optimization", section "SWA
 * bounded replay" (an FP8 window over the 128 most recent positions).
 *
 * Formats (the pages give the sizes; the bit layouts are fixed here):
 *   main entry  (288 B): bytes 0..255  = 512 E2M1 codes, element 2i in the low nibble
 *                        of byte i; bytes 256..287 = 32 E8M0 scales, scale j covers
 *                        elements 16j..16j+15.
 *   indexer key  (68 B): bytes 0..63   = 128 E2M1 codes (same nibble order); bytes
 *                        64..67 = 4 E8M0 scales, scale j covers elements 32j..32j+31.
 *   block summary       : 128 bf16 per 64-entry block (block j covers entries
 *                        64j..64j+63 of its request).
 *   window token        : 512 E4M3FN codes + one fp32 scale.
 *   E2M1 = OCP MX FP4 (values 0, .5, 1, 1.5, 2, 3, 4, 6 and negatives); E8M0 = 2^(u-127),
 *   u = 255 is NaN; E4M3FN = OCP FP8 (bias 7, max 448, no inf).
 *
 * Conventions for every entry point:
 *   - Buffer pointers are DEVICE pointers owned by the caller; sizes and the
 *     csa2_ragged / csa2_decode_args structs themselves are host memory, read during the
 *     call only.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).  No call
 *     synchronises, allocates device memory or keeps state between calls (except the
 *     static workspace of csa2_decode_static), so calls on different streams with
 *     distinct outputs and workspaces may run concurrently.
 *   - Return value: CSA2_OK (0) or a positive CSA2_ERR_* code.  Argument checks happen on
 *     the host before anything is launched; a failed check launches nothing.  A launch
 *     failure returns CSA2_ERR_HIP.  csa2_last_error() gives a message for the calling
 *     thread's most recent failure.  Device-array contents are not validated on the host
 *     (that would need a sync); kernels clamp offsets and lengths to the pool sizes and
 *     the host-side maxima given below, so inconsistent descriptors yield wrong results
 *     rather than out-of-bounds accesses.
 *   - Positions are request-local: entry t of request b is pool row entry_off[b] + t
 *     (contiguous pools) or row 64*page_table[b*pages_ld + t/64] + t%64 (paged pools).
 *   - Score check (SGLang blog, section "DSpark adaptation and optimization": the
 *     post-top-k score check and invalid-position filter): an entry or block whose score
 *     is NaN (e.g. an E8M0 scale byte of 255) is never ranked; block selection and top-k
 *     run over the others.  NaN ranks below every number, so this equals ranking
 *     everything and dropping NaN-scored picks afterwards.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_VERSION 2

/* Fixed dimensions. */
#define CSA2_D           512   /* latent dim = attention K = V dim */
#define CSA2_HEADS       64    /* query heads */
#define CSA2_IDX_D       128   /* indexer head dim */
#define CSA2_IDX_HEADS   8     /* indexer heads */
#define CSA2_MAIN_BYTES  288   /* main-KV entry */
#define CSA2_IDX_BYTES   68    /* indexer-key entry */
#define CSA2_BLOCK       64    /* entries per coarse block */
#define CSA2_SWA_MAX     128   /* window tokens per row (at most) */

/* Supported parameter ranges. */
#define CSA2_K_MAX              2048  /* fine top-k */
#define CSA2_KEEP_MAX           128   /* coarse blocks kept (plus the newest) */
#define CSA2_ROWS_PER_REQ_MAX   16    /* rows sharing one request's caches */
#define CSA2_TOPK_ALL_MAX       8192  /* csa2_topk without kept blocks: entries per request */

/* Status codes. */
#define CSA2_OK                       0
#define CSA2_ERR_INVALID_ARG          1  /* null pointer, negative size, inconsistent sizes */
#define CSA2_ERR_UNSUPPORTED          2  /* parameter outside the supported ranges above */
#define CSA2_ERR_WORKSPACE_TOO_SMALL  3
#define CSA2_ERR_HIP                  4  /* a HIP launch or runtime call failed */

/* Ragged batch: B requests, R query rows; the rows of one request are consecutive. */
typedef struct csa2_ragged {
  int32_t num_requests;           /* B >= 0 */
  int32_t num_rows;               /* R >= 0 */
  const int64_t* entry_off;       /* device [B+1]: request b owns pool entries entry_off[b] .. entry_off[b+1]-1 */
  const int64_t* block_off;       /* device [B+1]: request b owns summaries block_off[b] .. ; must hold ceil(N_b/64) */
  const int32_t* row_off;         /* device [B+1]: rows of request b are row_off[b] .. row_off[b+1]-1 */
  const int32_t* row_req;         /* device [R]: request of each row (consistent with row_off) */
  const int64_t* row_swa_start;   /* device [R]: first window-pool token of the row's window */
  const int32_t* row_swa_len;     /* device [R]: window length, 0..128 */
  int64_t max_entries;            /* host: >= max_b N_b (entries beyond it are ignored) */
  int64_t total_entries;          /* host: rows in the idx_k / main_kv pools */
  int64_t total_blocks;           /* host: rows in the block-summary pool */
  int64_t swa_tokens;             /* host: rows in the window pool */
  int32_t max_rows_per_request;   /* host: >= max_b (row_off[b+1]-row_off[b]), <= 16 */
  /* Per-row visible length (verify rows; SGLang blog, section "DSpark adaptation and
   * optimization": the candidate mask carries each row's valid-length check).  NULL:
   * every row sees all N_b entries of its request.  Otherwise row r sees entries
   * 0 .. V_r-1, V_r = row_len[r] clamped to 0..N_b: its blocks are the first
   * ceil(V_r/64) (the newest of them is block ceil(V_r/64)-1, possibly partial), only
   * those entries are candidates, and attention skips selected positions >= V_r. */
  const int64_t* row_len;         /* nullable device [R] */
  /* Paged pools (same section: KV page-address translation).  NULL: contiguous pools as
   * above.  Otherwise the idx_k / main_kv pools are made of 64-entry pages and the
   * block-summary pool holds one summary per page: entry t of request b lives at pool
   * row 64*p + t%64 and its block's summary at row p, p = page_table[b*pages_ld + t/64];
   * entry_off then only gives the lengths N_b = entry_off[b+1] - entry_off[b], and
   * block_off is unused (may be NULL).  Page ids are clamped to 0..total_pages-1. */
  const int32_t* page_table;      /* nullable device [B][pages_ld] */
  int32_t pages_ld;               /* host: >= ceil(max_entries/64) when page_table != NULL */
  int64_t total_pages;            /* host: >= 1 when paged; 64*total_pages <= total_entries,
                                     total_pages <= total_blocks */
} csa2_ragged;

/*
 * Step (1): indexer scan.  For every row r and every entry t of its request,
 *   scores[r*ld + t] = sum_{h<8} w_idx[r*8+h] * max(0, q_h . k_t),
 * q_h = q_idx[(r*8+h)*128 .. +127] (bf16 bit patterns), k_t the dequantised 68-B key.
 * idx_k: [total_entries][68] bytes.  ld >= max_entries.
 * kept_blocks == NULL: every entry of the request is scored, also past a row's visible
 * length (the rows of one request share one read of its keys).  Otherwise only the
 * entries the row sees of the blocks kept_blocks[r*kept_ld + j], j < n_kept[r], are
 * scored (candidate-only scan); other positions of scores are left untouched.
 */
int csa2_index_score(const csa2_ragged* rg, const uint8_t* idx_k, const uint16_t* q_idx, const float* w_idx,
                     const int32_t* kept_blocks, const int32_t* n_kept, int32_t kept_ld,
                     float* scores, int64_t ld, void* stream);

/*
 * Step (2a): coarse block filter.  Block j of the row's request (nb = ceil(V/64) blocks,
 * V = the entries the row sees)
 * scores s_j = sum_h w_h * max(0, q_h . summary_j) into blk_scores[r*blk_ld + j]
 * (blk_ld >= ceil(max_entries/64)).  If nb <= n_keep every block is kept; otherwise the
 * n_keep best blocks (ties to the lower j) plus, if keep_newest, block nb-1.  The kept
 * blocks go to kept_blocks[r*(n_keep+1) + i] in ascending order, their count to
 * n_kept[r]; unused slots are -1.  blk_sum: [total_blocks][128] bf16.
 * n_keep in 1..CSA2_KEEP_MAX.
 */
int csa2_block_filter(const csa2_ragged* rg, const uint16_t* blk_sum, const uint16_t* q_idx, const float* w_idx,
                      int32_t n_keep, int32_t keep_newest,
                      int32_t* kept_blocks, int32_t* n_kept, float* blk_scores, int64_t blk_ld, void* stream);

/*
 * Step (2b): fine top-k.  Candidates are the entries the row sees of its kept blocks
 * (the newest block may be partial), NaN scores excepted; the k best scores (ties to
 * the lower position) are
 * written in ascending position to sel_idx[r*k + i], their count min(k, candidates) to
 * n_sel[r], unused slots -1; sel_score (nullable) receives the matching scores.
 * kept_blocks == NULL: every entry of the request is a candidate (max_entries <=
 * CSA2_TOPK_ALL_MAX).  k in 1..CSA2_K_MAX; kept_ld >= n_kept values.
 */
int csa2_topk(const csa2_ragged* rg, const float* scores, int64_t ld,
              const int32_t* kept_blocks, const int32_t* n_kept, int32_t kept_ld,
              int32_t k, int32_t* sel_idx, int32_t* n_sel, float* sel_score, void* stream);

/*
 * Step (3): joint-softmax latent attention.  Row r's keys are the main entries
 * sel_idx[r*sel_ld + i], i < n_sel[r] (request-local positions; negative ones and those
 * the row does not see are skipped), followed by the window tokens
 * row_swa_start[r] .. +row_swa_len[r]-1.
 * K = V = the 512-dim dequantised latent.  For each head h:
 *   z_i = sm_scale * q_h . x_i,  out[(r*64+h)*512 + d] = sum_i softmax(z)_i x_i[d],
 *   lse[r*64+h] = log sum_i exp(z_i)   (natural log; -inf and out = 0 with no keys).
 * q: [R][64][512] bf16; main_kv: [total_entries][288]; swa: [swa_tokens][512] E4M3FN;
 * swa_scale: [swa_tokens] fp32; out fp32 [R][64][512]; lse fp32 [R][64].
 * ws: device workspace of at least csa2_sparse_attn_workspace_size(rg, sel_ld) bytes
 * (with paged pools it also holds the positions translated to pool rows, which a first
 * kernel writes).
 */
int csa2_sparse_attn(const csa2_ragged* rg, const uint16_t* q, const uint8_t* main_kv,
                     const int32_t* sel_idx, const int32_t* n_sel, int32_t sel_ld,
                     const uint8_t* swa, const float* swa_scale, float sm_scale,
                     float* out, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t csa2_sparse_attn_workspace_size(const csa2_ragged* rg, int32_t sel_ld);

/* Arithmetic routes of step (3) (ktransformers issue mirror "Support for Deepseek V4.1
 * Flash": sparse MLA runs either in full BF16 or with Q and P rounded to MXFP8).
 *   CSA2_QP_BF16 : Q as given (bf16), P to about 2^-17 relative (fp32 accuracy).
 *   CSA2_QP_MXFP8: Q (per head, blocks of 32 latent dims) and P (per head, blocks of 32
 *                  consecutive keys in key order, the weight on each key's stored codes,
 *                  i.e. p times the window scale for window tokens) are rounded to MXFP8
 *                  (OCP MX: E4M3 elements, shared exponent floor(log2(block amax)) - 8,
 *                  round to nearest even, saturating at 448) before their products;
 *                  the softmax normaliser and lse use the unrounded p.  P is computed
 *                  against the running maximum of the key range a workgroup covers, so
 *                  its rounding depends on the split plan. */
#define CSA2_QP_BF16  0
#define CSA2_QP_MXFP8 1

/* The whole path on one stream: (2a) and (1), then (2b), then (3).  The fine top-k also
 * writes the picks' pool rows into the workspace (for paged pools this is the address
 * translation, fused into the selection; contiguous pools need total_entries < 2^31 for
 * it) and attention reads those, so it needs no request offsets before its first reads. */
typedef struct csa2_decode_args {
  csa2_ragged rg;
  const uint8_t* idx_k;        /* [total_entries][68] */
  const uint8_t* main_kv;      /* [total_entries][288] */
  const uint16_t* blk_sum;     /* [total_blocks][128] bf16 */
  const uint8_t* swa;          /* [swa_tokens][512] E4M3FN */
  const float* swa_scale;      /* [swa_tokens] */
  const uint16_t* q;           /* [R][64][512] bf16 */
  const uint16_t* q_idx;       /* [R][8][128] bf16 */
  const float* w_idx;          /* [R][8] */
  int32_t k;                   /* fine top-k, 1..CSA2_K_MAX (512) */
  int32_t n_keep;              /* coarse blocks kept, 1..CSA2_KEEP_MAX (64) */
  int32_t keep_newest;         /* 1: always keep block nb-1 */
  int32_t scan_mode;           /* 0: score every entry (1); 1: score only kept blocks' entries */
  float sm_scale;              /* 1/sqrt(512) */
  float* out;                  /* [R][64][512] fp32 */
  float* lse;                  /* [R][64] fp32 */
  int32_t* sel_idx;            /* nullable [R][k]: selected positions, ascending, -1 pad */
  int32_t* n_sel;              /* nullable [R] */
  int32_t* kept_blocks;        /* nullable [R][n_keep+1] */
  int32_t* n_kept;             /* nullable [R] */
  float* scores;               /* nullable [R][scores_ld]: index scores (scan_mode 1: kept entries only) */
  int64_t scores_ld;           /* >= max_entries when scores != NULL */
  void* const* events;         /* nullable: CSA2_DECODE_EVENTS hipEvent_t handles, recorded on `stream`
                                  before the first kernel and after each stage (scan, select,
                                  attention, merge) for per-stage timing; recording adds no sync */
  int32_t qp_route;            /* CSA2_QP_BF16 (default) or CSA2_QP_MXFP8; with MXFP8 and few
                                  rows the workspace also holds the rounded query (64 KB
                                  per row), which the selection launch writes and attention
                                  reads */
} csa2_decode_args;

#define CSA2_DECODE_EVENTS 5

int csa2_decode(const csa2_decode_args* a, void* ws, size_t ws_bytes, void* stream);
size_t csa2_decode_workspace_size(const csa2_decode_args* a);

/*
 * csa2_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same launch chain
 * as csa2_decode, with its workspace in a static device buffer of CSA2_STATIC_WS_BYTES
 * that the library holds on every device it runs on until the process ends.  The caller
 * passes inputs and outputs as for csa2_decode; the call allocates nothing.  Returns
 * CSA2_ERR_WORKSPACE_TOO_SMALL (nothing launched) when csa2_decode_workspace_size(a)
 * exceeds CSA2_STATIC_WS_BYTES.  Every call on one device shares that device's buffer:
 * calls that overlap on one device (other streams, other threads) race and must be
 * serialised by the caller.  `stream` must belong to the current device.  No part of
 * the buffer needs to start at zero: every value the kernels read there is written
 * earlier in the same call.
 */
#define CSA2_STATIC_WS_BYTES ((size_t)64 << 20)
int csa2_decode_static(const csa2_decode_args* a, void* stream);

/*
 * Cache write (the step before the path; SGLang blog, section "Small-operator fusion and
 * GEMV": pooling, RMSNorm, FP4 quantisation and the cache write run as one fused chain;
 * section "DSpark adaptation and optimization": verify positions are contiguous, so a
 * row's pooling partner is the previous row, and only the first row of a request needs
 * the ring buffer).  Row r is a new token at position row_pos[r] of its request (the
 * rows of a request hold consecutive positions); kv_tok[r] (512) and idx_tok[r] (128)
 * are its compressor outputs, bf16.  Global entry t pools tokens 2t and 2t+1, so a row
 * at an odd position P completes entry t = (P-1)/2:
 *   pooled = (x[P-1] + x[P]) / 2, x[P-1] = the previous row of the request if it holds
 *            position P-1, else the request's ring slot (ring_kv[b], ring_idx[b]);
 *   y      = pooled * gamma / sqrt(mean(pooled^2) + eps)     (per vector, fp32);
 *   record = OCP MX FP4 of y: per block (16 dims main, 32 dims index) the E8M0 exponent
 *            floor(log2(block amax)) - 2 (0 for an all-zero block: scale byte 0),
 *            elements y / 2^e rounded to the nearest E2M1 value (ties to the even code,
 *            6 for everything above 5), laid out as in the formats above;
 * and writes the main and index records of entry t at its pool row (t < N_b required;
 * other rows write nothing).  Then, for every block that received an entry, the
 * summary = bf16 (round to nearest even) of the mean of the dequantised index keys of
 * the block's entries 0 .. min(63, N_b - 1 - 64j); and a request whose last row sits at
 * an even position stores that row's vectors in its ring slot.  row_len and sel-related
 * fields of rg are ignored; N_b = entry_off[b+1] - entry_off[b] already counts the new
 * entries.  gamma_kv [512] / gamma_idx [128] fp32; eps > 0.  The ring slots are read
 * before any is written.  Rows whose position is negative are skipped.
 * RoPE: the same section lists a rotary embedding in the fused chain; it is not applied
 * here.  Attention in this library uses K = V = the whole 512-dim latent with no rotary
 * part (no separate RoPE dims are stored in the 288-B entry), so the write has nothing
 * to rotate; a caller whose latent carries rotary dims applies RoPE to kv_tok first.
 */
int csa2_cache_write(const csa2_ragged* rg, const int64_t* row_pos, const uint16_t* kv_tok, const uint16_t* idx_tok,
                     uint16_t* ring_kv, uint16_t* ring_idx, const float* gamma_kv, const float* gamma_idx, float eps,
                     uint8_t* main_kv, uint8_t* idx_k, uint16_t* blk_sum, void* stream);

/* Test hook: run the kernels' own dequantisation helpers over raw records.
 * kind CSA2_DQ_MAIN: records [n][288] -> out [n][512]; CSA2_DQ_IDX: [n][68] -> [n][128];
 * CSA2_DQ_SWA: records [n][512] E4M3FN with scales [n] -> out [n][512] = fp32(x * scale).
 * Outputs are exact (FP4 values and E4M3 values are representable in bf16/fp32). */
#define CSA2_DQ_MAIN 0
#define CSA2_DQ_IDX  1
#define CSA2_DQ_SWA  2
int csa2_debug_dequant(int32_t kind, const uint8_t* records, const float* scales, int64_t n, float* out,
                       void* stream);

/* Test hook: the attention kernel's MXFP8 rounding (CSA2_QP_MXFP8) over x[0 .. n-1] in
 * blocks of 32 consecutive values (n a multiple of 32), results as exact fp32 in out.
 * A block whose 32 values are all bf16 values goes through the bf16-input rounding the
 * kernel applies to the query; any other block through the fp32-input rounding it
 * applies to the probabilities. */
int csa2_debug_mxfp8(const float* x, int64_t n, float* out, void* stream);

/* Measurement hook, for callers that want the bandwidth a plain streaming read reaches
 * on this device (the reference the indexer scan is compared with): reads `bytes` bytes
 * at `src` (16-byte aligned, bytes a multiple of 16) with non-temporal 16-byte loads,
 * 16 KiB per workgroup, and writes nothing unless the bytes' XOR equals an unlikely constant, in
 * which case one word goes to `sink` (4 bytes of device memory).  Errors:
 * CSA2_ERR_INVALID_ARG for misaligned pointers or sizes. */
int csa2_debug_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Measurement hook, for callers that want the shader clock while other work runs (the
 * clock falls under sustained load): one wave records n pairs (shader-clock counter,
 * 100 MHz reference counter) into out[2i], out[2i+1], one pair every `interval`
 * reference ticks (10 ns), and ends after n x interval ticks.  Launched on a stream of
 * its own beside the work to observe; clock in GHz = 0.1 x (change of the first) /
 * (change of the second).  out: device memory of 2n uint64, owned by the caller.
 * Errors: CSA2_ERR_INVALID_ARG for n outside [0, CSA2_CLOCK_TRACE_MAX_SAMPLES], interval
 * < 1, n x interval above CSA2_CLOCK_TRACE_MAX_TICKS (2 s), or a misaligned out. */
#define CSA2_CLOCK_TRACE_MAX_SAMPLES 65536
#define CSA2_CLOCK_TRACE_MAX_TICKS 200000000
int csa2_debug_clock_trace(uint64_t* out, int32_t n, int32_t interval, void* stream);

const char* csa2_status_string(int32_t status);
const char* csa2_last_error(void);
int32_t csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
