// Host entry points of libcsa2: argument checks, workspace layout, launch chains.
// Every check runs before any launch; nothing here synchronises or allocates.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "csa2_internal.h"

using namespace csa2;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CSA2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_ragged(const csa2_ragged* rg, RaggedDev& g) {
  if (!rg) return fail(CSA2_ERR_INVALID_ARG, "ragged descriptor is NULL");
  if (rg->num_requests < 0 || rg->num_rows < 0) return fail(CSA2_ERR_INVALID_ARG, "negative request/row count");
  if (rg->num_requests > 65535 || rg->num_rows > 65535)
    return fail(CSA2_ERR_UNSUPPORTED, "at most 65535 requests and 65535 rows per call");
  if (rg->num_rows > 0 && rg->num_requests == 0) return fail(CSA2_ERR_INVALID_ARG, "rows without requests");
  if (rg->num_requests > 0 && (!rg->entry_off || !rg->row_off))
    return fail(CSA2_ERR_INVALID_ARG, "entry_off/row_off is NULL");
  if (rg->num_requests > 0 && !rg->page_table && !rg->block_off)
    return fail(CSA2_ERR_INVALID_ARG, "block_off is NULL (required for contiguous pools)");
  if (rg->num_rows > 0 && (!rg->row_req || !rg->row_swa_start || !rg->row_swa_len))
    return fail(CSA2_ERR_INVALID_ARG, "row_req/row_swa_start/row_swa_len is NULL");
  if (rg->max_entries < 0 || rg->total_entries < 0 || rg->total_blocks < 0 || rg->swa_tokens < 0)
    return fail(CSA2_ERR_INVALID_ARG, "negative pool size");
  if (rg->max_entries > rg->total_entries)
    return fail(CSA2_ERR_INVALID_ARG, "max_entries %lld exceeds total_entries %lld", (long long)rg->max_entries,
                (long long)rg->total_entries);
  if (rg->max_entries >= (int64_t(1) << 31)) return fail(CSA2_ERR_UNSUPPORTED, "max_entries must be < 2^31");
  if (rg->total_blocks >= (int64_t(1) << 31) || rg->swa_tokens >= (int64_t(1) << 31))
    return fail(CSA2_ERR_UNSUPPORTED, "total_blocks and swa_tokens must be < 2^31");
  if (rg->num_rows > 0 && (rg->max_rows_per_request < 1 || rg->max_rows_per_request > CSA2_ROWS_PER_REQ_MAX))
    return fail(CSA2_ERR_UNSUPPORTED, "max_rows_per_request must be in 1..%d", CSA2_ROWS_PER_REQ_MAX);
  if (rg->page_table) {
    if (rg->pages_ld < ceil_div(rg->max_entries, CSA2_BLOCK) || rg->pages_ld < 1)
      return fail(CSA2_ERR_INVALID_ARG, "pages_ld %d < ceil(max_entries/64)", rg->pages_ld);
    if (rg->total_pages < 1) return fail(CSA2_ERR_INVALID_ARG, "paged pools need total_pages >= 1");
    if (rg->total_pages > rg->total_blocks || rg->total_pages > rg->total_entries / CSA2_BLOCK)
      return fail(CSA2_ERR_INVALID_ARG, "total_pages %lld exceeds the pools (%lld entries, %lld summaries)",
                  (long long)rg->total_pages, (long long)rg->total_entries, (long long)rg->total_blocks);
    if (rg->total_pages >= (int64_t(1) << 31) / CSA2_BLOCK)
      return fail(CSA2_ERR_UNSUPPORTED, "paged pools must hold fewer than 2^31 entries");
  }
  g.entry_off = rg->entry_off;
  g.block_off = rg->block_off;
  g.row_off = rg->row_off;
  g.row_req = rg->row_req;
  g.row_swa_start = rg->row_swa_start;
  g.row_swa_len = rg->row_swa_len;
  g.max_entries = (int32_t)rg->max_entries;
  g.total_entries = rg->total_entries;
  g.total_blocks = (int32_t)rg->total_blocks;
  g.swa_tokens = (int32_t)rg->swa_tokens;
  g.B = rg->num_requests;
  g.R = rg->num_rows;
  g.row_len = rg->row_len;
  g.page_table = rg->page_table;
  g.pages_ld = rg->page_table ? rg->pages_ld : 0;
  g.total_pages = rg->page_table ? (int32_t)rg->total_pages : 0;
  return CSA2_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(CSA2_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(CSA2_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return CSA2_OK;
}

#define CHECK(expr)            \
  do {                         \
    int _rc = (expr);          \
    if (_rc != CSA2_OK) return _rc; \
  } while (0)

#define LAUNCH(expr, where)                     \
  do {                                          \
    hipError_t _e = (expr);                     \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

int64_t blocks_of(int64_t entries) { return ceil_div(entries, CSA2_BLOCK); }

// Workspace carve-out: a bump allocator over the caller's buffer.
struct Carve {
  char* base;
  size_t used;
  template <typename T>
  T* take(size_t count) {
    used = round_up(used, 256);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

// ---------------------------------------------------------------------------------
// Test hook: the kernels' dequantisation helpers over raw records.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_debug_dequant(int kind, const uint8_t* rec, const float* scales, int64_t n,
                                                      float* out) {
  const int groups = (kind == CSA2_DQ_IDX) ? CSA2_IDX_D / 8 : CSA2_D / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * groups) return;
  const int64_t i = t / groups;
  const int grp = (int)(t % groups);
  float v[8];
  if (kind == CSA2_DQ_MAIN) {
    const uint8_t* p = rec + i * CSA2_MAIN_BYTES;
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(p + 4 * grp);
    bf16x8_words_to_f32(fp4x8_to_bf16(codes, e8m0_operand(p[256 + grp / 2])), v);
  } else if (kind == CSA2_DQ_IDX) {
    const uint8_t* p = rec + i * CSA2_IDX_BYTES;
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(p + 4 * grp);
    bf16x8_words_to_f32(fp4x8_to_bf16(codes, e8m0_operand(p[64 + grp / 4])), v);
  } else {
    const uint8_t* p = rec + i * CSA2_D + 8 * grp;
    const bf16x4_t lo = e4m3x4_to_bf16(*reinterpret_cast<const uint32_t*>(p));
    const bf16x4_t hi = e4m3x4_to_bf16(*reinterpret_cast<const uint32_t*>(p + 4));
    bf16x8_words_to_f32(bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, v);
    const float s = scales[i];
    for (int j = 0; j < 8; ++j) v[j] *= s;
  }
  const int dim = (kind == CSA2_DQ_IDX) ? CSA2_IDX_D : CSA2_D;
  for (int j = 0; j < 8; ++j) out[i * dim + 8 * grp + j] = v[j];
}

}  // namespace

// ---------------------------------------------------------------------------------
// Static workspace of csa2_decode_static: one buffer per device, held until the process
// ends.  Host code never passes `scratch` itself to a kernel (in host code the name
// stands for a host-side shadow, not device memory): the buffer's device address is
// looked up once per device, with that device current, and only that address is used.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[CSA2_STATIC_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA2_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(CSA2_ERR_HIP, "static workspace has no valid device address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA2_OK;
}

}  // namespace

namespace csa2 {
// Plain streaming read: workgroup w reads the 16 KiB chunk w with four 16-B loads per
// thread in flight, non-temporal (the fastest of the read patterns measured: chunks of
// 8-64 KiB, 256 or 512 threads, persistent grids, with and without the hint).
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ p, int64_t n16, uint32_t* sink) {
  const int64_t b0 = (int64_t)blockIdx.x * 1024;
  const int64_t e = b0 + 1024 < n16 ? b0 + 1024 : n16;
  uint32_t acc = 0u;
  int64_t i = b0 + threadIdx.x;
  if (i + 768 < e) {
    const u32x4_t x0 = __builtin_nontemporal_load(p + i), x1 = __builtin_nontemporal_load(p + i + 256),
                  x2 = __builtin_nontemporal_load(p + i + 512), x3 = __builtin_nontemporal_load(p + i + 768);
    const u32x4_t y = x0 ^ x1 ^ x2 ^ x3;
    acc = y[0] ^ y[1] ^ y[2] ^ y[3];
  } else {
    for (; i < e; i += 256) {
      const u32x4_t x = __builtin_nontemporal_load(p + i);
      acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  k_stream_read<<<dim3((unsigned)ceil_div(n16, 1024)), dim3(256), 0, st>>>(reinterpret_cast<const u32x4_t*>(src), n16,
                                                                            sink);
  return hipGetLastError();
}

// Clock sampler: one wave reads the shader-clock counter and the 100 MHz reference
// counter every `interval` reference ticks, n times, and lane 0 stores each pair.  The
// wait between samples is bounded by the reference counter, so the kernel ends after
// n x interval ticks.
__global__ __launch_bounds__(64) void k_clock_trace(uint64_t* out, int n, int interval) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < n; ++i) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
      out[2 * i] = t;
      out[2 * i + 1] = r;
    }
    const uint64_t until = r0 + (uint64_t)(i + 1) * (uint64_t)interval;
    while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(2);
  }
}

hipError_t launch_clock_trace(uint64_t* out, int n, int interval, hipStream_t st) {
  k_clock_trace<<<dim3(1), dim3(64), 0, st>>>(out, n, interval);
  return hipGetLastError();
}

// Test hook: lane (i, g) of a wave rounds values 8g .. 8g+7 of block 16w + i (w = the
// wave's index in the grid) with the attention kernel's block helpers: blocks whose 32
// values are all bf16 values take the bf16-input rounding (the query's), the others the
// fp32-input one (the probabilities').
__global__ __launch_bounds__(256) void k_debug_mxfp8(const float* x, int64_t nblocks, float* out) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16 + (lane & 15);
  const int g = lane >> 4;
  const bool ok = blk < nblocks;
  float v[8];
  for (int j = 0; j < 8; ++j) v[j] = ok ? x[blk * 32 + 8 * g + j] : 0.f;
  uint32_t exact = 1u;
  u32x4_t w;
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = __float_as_uint(v[2 * q]), b = __float_as_uint(v[2 * q + 1]);
    exact &= ((a | b) & 0xFFFFu) == 0u ? 1u : 0u;
    w[q] = (a >> 16) | (b & 0xFFFF0000u);
  }
  exact &= __shfl_xor(exact, 16, 64);
  exact &= __shfl_xor(exact, 32, 64);
  float r[8], rb[8];
  bf16x8_words_to_f32(mx8_round_block_bf16x8(v), r);
  bf16x8_words_to_f32(mx8_round_block_bf16(as_bf16x8(w)), rb);
  if (exact)
    for (int j = 0; j < 8; ++j) r[j] = rb[j];
  if (ok)
    for (int j = 0; j < 8; ++j) out[blk * 32 + 8 * g + j] = r[j];
}

hipError_t launch_debug_mxfp8(const float* x, int64_t n, float* out, hipStream_t st) {
  const int64_t nblocks = n / 32;
  if (nblocks == 0) return hipSuccess;
  k_debug_mxfp8<<<dim3((unsigned)ceil_div(nblocks, 64)), dim3(256), 0, st>>>(x, nblocks, out);
  return hipGetLastError();
}

hipError_t launch_debug_dequant(int kind, const uint8_t* rec, const float* scales, int64_t n, float* out,
                                hipStream_t st) {
  const int groups = (kind == CSA2_DQ_IDX) ? CSA2_IDX_D / 8 : CSA2_D / 8;
  const int64_t threads = n * groups;
  if (threads == 0) return hipSuccess;
  k_debug_dequant<<<dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, st>>>(kind, rec, scales, n, out);
  return hipGetLastError();
}
}  // namespace csa2

// =================================================================================
// C ABI
// =================================================================================
extern "C" {

int csa2_index_score(const csa2_ragged* rg, const uint8_t* idx_k, const uint16_t* q_idx, const float* w_idx,
                     const int32_t* kept_blocks, const int32_t* n_kept, int32_t kept_ld, float* scores, int64_t ld,
                     void* stream) {
  RaggedDev g;
  CHECK(check_ragged(rg, g));
  if (g.R == 0) return CSA2_OK;
  CHECK(check_ptr(idx_k, 4, "idx_k"));
  CHECK(check_ptr(q_idx, 16, "q_idx"));
  CHECK(check_ptr(w_idx, 4, "w_idx"));
  CHECK(check_ptr(scores, 4, "scores"));
  if (ld < g.max_entries || ld < 1) return fail(CSA2_ERR_INVALID_ARG, "ld %lld < max_entries", (long long)ld);
  ScanArgs a{};
  a.g = g;
  a.idx_k = idx_k;
  a.q_idx = q_idx;
  a.w = w_idx;
  a.scores = scores;
  a.ld = ld;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (kept_blocks) {
    if (!n_kept) return fail(CSA2_ERR_INVALID_ARG, "n_kept is NULL");
    if (kept_ld < 1 || kept_ld > 65535) return fail(CSA2_ERR_INVALID_ARG, "kept_ld must be in 1..65535");
    a.kept = kept_blocks;
    a.n_kept = n_kept;
    a.kept_ld = kept_ld;
    LAUNCH(launch_scan_kept(a, st), "index scan (kept blocks)");
  } else {
    LAUNCH(launch_scan(a, rg->max_rows_per_request, true, false, st), "index scan");
  }
  return CSA2_OK;
}

int csa2_block_filter(const csa2_ragged* rg, const uint16_t* blk_sum, const uint16_t* q_idx, const float* w_idx,
                      int32_t n_keep, int32_t keep_newest, int32_t* kept_blocks, int32_t* n_kept, float* blk_scores,
                      int64_t blk_ld, void* stream) {
  RaggedDev g;
  CHECK(check_ragged(rg, g));
  if (n_keep < 1 || n_keep > CSA2_KEEP_MAX) return fail(CSA2_ERR_UNSUPPORTED, "n_keep must be in 1..%d", CSA2_KEEP_MAX);
  if (g.R == 0) return CSA2_OK;
  CHECK(check_ptr(blk_sum, 16, "blk_sum"));
  CHECK(check_ptr(q_idx, 16, "q_idx"));
  CHECK(check_ptr(w_idx, 4, "w_idx"));
  CHECK(check_ptr(kept_blocks, 4, "kept_blocks"));
  CHECK(check_ptr(n_kept, 4, "n_kept"));
  CHECK(check_ptr(blk_scores, 4, "blk_scores"));
  if (blk_ld < blocks_of(g.max_entries) || blk_ld < 1)
    return fail(CSA2_ERR_INVALID_ARG, "blk_ld must be >= ceil(max_entries/64)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  ScanArgs a{};
  a.g = g;
  a.blk_sum = blk_sum;
  a.q_idx = q_idx;
  a.w = w_idx;
  a.blk_scores = blk_scores;
  a.blk_ld = blk_ld;
  LAUNCH(launch_scan(a, rg->max_rows_per_request, false, true, st), "block scores");
  SelectArgs s{};
  s.g = g;
  s.blk_scores = blk_scores;
  s.blk_ld = blk_ld;
  s.n_keep = n_keep;
  s.keep_newest = keep_newest ? 1 : 0;
  s.kept = kept_blocks;
  s.n_kept = n_kept;
  s.kept_ld = n_keep + 1;
  LAUNCH(launch_block_select(s, st), "block select");
  return CSA2_OK;
}

int csa2_topk(const csa2_ragged* rg, const float* scores, int64_t ld, const int32_t* kept_blocks,
              const int32_t* n_kept, int32_t kept_ld, int32_t k, int32_t* sel_idx, int32_t* n_sel, float* sel_score,
              void* stream) {
  RaggedDev g;
  CHECK(check_ragged(rg, g));
  if (k < 1 || k > CSA2_K_MAX) return fail(CSA2_ERR_UNSUPPORTED, "k must be in 1..%d", CSA2_K_MAX);
  if (g.R == 0) return CSA2_OK;
  CHECK(check_ptr(scores, 4, "scores"));
  CHECK(check_ptr(sel_idx, 4, "sel_idx"));
  CHECK(check_ptr(n_sel, 4, "n_sel"));
  if (sel_score) CHECK(check_ptr(sel_score, 4, "sel_score"));
  if (ld < g.max_entries || ld < 1) return fail(CSA2_ERR_INVALID_ARG, "ld < max_entries");
  if (kept_blocks) {
    if (!n_kept) return fail(CSA2_ERR_INVALID_ARG, "n_kept is NULL");
    if (kept_ld < 1) return fail(CSA2_ERR_INVALID_ARG, "kept_ld must be >= 1");
  } else if (g.max_entries > CSA2_TOPK_ALL_MAX) {
    return fail(CSA2_ERR_UNSUPPORTED, "without kept blocks, max_entries must be <= %d", CSA2_TOPK_ALL_MAX);
  }
  SelectArgs s{};
  s.g = g;
  s.kept = const_cast<int32_t*>(kept_blocks);
  s.n_kept = const_cast<int32_t*>(n_kept);
  s.kept_ld = kept_ld;
  s.scores = scores;
  s.ld = ld;
  s.k = k;
  s.sel = sel_idx;
  s.n_sel = n_sel;
  s.sel_score = sel_score;
  LAUNCH(launch_topk(s, kept_blocks == nullptr, reinterpret_cast<hipStream_t>(stream)), "top-k");
  return CSA2_OK;
}

// Standalone attention workspace: the split partials, then (paged pools) the selected
// positions translated to pool rows.
size_t csa2_sparse_attn_workspace_size(const csa2_ragged* rg, int32_t sel_ld) {
  if (!rg || rg->num_rows <= 0 || sel_ld < 1) return 0;
  size_t n = round_up(attn_workspace_bytes(rg->num_rows, sel_ld), 256);
  if (rg->page_table) n += round_up((size_t)rg->num_rows * sel_ld * sizeof(int32_t), 256);
  return n;
}

static int attn_args(const RaggedDev& g, const uint16_t* q, const uint8_t* main_kv, const int32_t* sel_idx,
                     const int32_t* n_sel, int32_t sel_ld, const uint8_t* swa, const float* swa_scale, float sm_scale,
                     float* out, float* lse, void* ws, size_t ws_bytes, AttnArgs& a) {
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(main_kv, 16, "main_kv"));
  CHECK(check_ptr(sel_idx, 4, "sel_idx"));
  CHECK(check_ptr(n_sel, 4, "n_sel"));
  CHECK(check_ptr(out, 16, "out"));
  CHECK(check_ptr(lse, 4, "lse"));
  if (g.swa_tokens > 0) {
    CHECK(check_ptr(swa, 16, "swa"));
    CHECK(check_ptr(swa_scale, 4, "swa_scale"));
  }
  if (sel_ld < 1 || sel_ld > CSA2_K_MAX) return fail(CSA2_ERR_UNSUPPORTED, "sel_ld must be in 1..%d", CSA2_K_MAX);
  if (!isfinite(sm_scale)) return fail(CSA2_ERR_INVALID_ARG, "sm_scale is not finite");
  a.g = g;
  a.q = q;
  a.main_kv = main_kv;
  a.sel = sel_idx;
  a.n_sel = n_sel;
  a.sel_ld = sel_ld;
  a.swa = swa;
  a.swa_scale = swa_scale;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  attn_plan(g.R, sel_ld, a.tile_keys, a.split_keys, a.splits, a.head_split);
  const size_t need = attn_workspace_bytes(g.R, sel_ld);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(CSA2_ERR_WORKSPACE_TOO_SMALL, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 256)) return fail(CSA2_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    Carve c{static_cast<char*>(ws), 0};
    const size_t parts = (size_t)g.R * a.splits * CSA2_HEADS;
    a.opart = c.take<float>(parts * CSA2_D);
    a.mpart = c.take<float>(parts);
    a.lpart = c.take<float>(parts);
  }
  return CSA2_OK;
}

int csa2_sparse_attn(const csa2_ragged* rg, const uint16_t* q, const uint8_t* main_kv, const int32_t* sel_idx,
                     const int32_t* n_sel, int32_t sel_ld, const uint8_t* swa, const float* swa_scale, float sm_scale,
                     float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  RaggedDev g;
  CHECK(check_ragged(rg, g));
  if (g.R == 0) return CSA2_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AttnArgs a{};
  if (!g.page_table) {
    CHECK(attn_args(g, q, main_kv, sel_idx, n_sel, sel_ld, swa, swa_scale, sm_scale, out, lse, ws, ws_bytes, a));
    LAUNCH(launch_attn(a, st), "sparse attention");
    return CSA2_OK;
  }
  // Paged pools: translate the positions to pool rows first.
  CHECK(check_ptr(sel_idx, 4, "sel_idx"));
  CHECK(check_ptr(n_sel, 4, "n_sel"));
  if (sel_ld < 1 || sel_ld > CSA2_K_MAX) return fail(CSA2_ERR_UNSUPPORTED, "sel_ld must be in 1..%d", CSA2_K_MAX);
  const size_t need = csa2_sparse_attn_workspace_size(rg, sel_ld);
  if (!ws || ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE_TOO_SMALL, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(CSA2_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int32_t* rows = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             round_up(attn_workspace_bytes(g.R, sel_ld), 256));
  CHECK(attn_args(g, q, main_kv, rows, n_sel, sel_ld, swa, swa_scale, sm_scale, out, lse, ws, ws_bytes, a));
  a.sel_rows = 1;
  LAUNCH(launch_sel_rows(g, sel_idx, n_sel, sel_ld, rows, st), "position translation");
  LAUNCH(launch_attn(a, st), "sparse attention");
  return CSA2_OK;
}

// Workspace of csa2_decode, in carve order.
struct SliceBufs {
  int32_t n_slices = 0;
  int32_t* blk = nullptr;
  float* sc = nullptr;
  int32_t* n = nullptr;
};

static size_t decode_layout(const csa2_decode_args* a, char* base, float** scores, float** blk_scores,
                            int32_t** kept, int32_t** n_kept, int32_t** sel, int32_t** n_sel, int32_t** sel_rows,
                            char** attn_ws, size_t* attn_bytes, SliceBufs* slices = nullptr,
                            uint16_t** q_mx = nullptr) {
  const csa2_ragged& rg = a->rg;
  const int64_t R = rg.num_rows;
  const int64_t ld = round_up((size_t)(rg.max_entries > 0 ? rg.max_entries : 1), 64);
  const int64_t blk_ld = round_up((size_t)(blocks_of(rg.max_entries) > 0 ? blocks_of(rg.max_entries) : 1), 64);
  Carve c{base, 0};
  float* s = a->scores ? nullptr : c.take<float>((size_t)R * ld);
  if (scores) *scores = a->scores ? a->scores : s;
  float* bs = c.take<float>((size_t)R * blk_ld);
  if (blk_scores) *blk_scores = bs;
  int32_t* kp = a->kept_blocks ? nullptr : c.take<int32_t>((size_t)R * (a->n_keep + 1));
  if (kept) *kept = a->kept_blocks ? a->kept_blocks : kp;
  int32_t* nk = a->n_kept ? nullptr : c.take<int32_t>((size_t)R);
  if (n_kept) *n_kept = a->n_kept ? a->n_kept : nk;
  int32_t* sl = a->sel_idx ? nullptr : c.take<int32_t>((size_t)R * a->k);
  if (sel) *sel = a->sel_idx ? a->sel_idx : sl;
  int32_t* ns = a->n_sel ? nullptr : c.take<int32_t>((size_t)R);
  if (n_sel) *n_sel = a->n_sel ? a->n_sel : ns;
  // Pool rows of the picks (int32): written by the fine top-k so that attention reads
  // records without first looking up its request's offsets.
  const bool rows = rg.page_table || rg.total_entries < (int64_t(1) << 31);
  int32_t* sr = rows ? c.take<int32_t>((size_t)R * a->k) : nullptr;
  if (sel_rows) *sel_rows = sr;
  const size_t ab = attn_workspace_bytes(R, a->k);
  char* aw = c.take<char>(ab);
  if (attn_ws) *attn_ws = aw;
  if (attn_bytes) *attn_bytes = ab;
  // Sliced coarse stage (full scans of rows with many blocks).
  const int32_t nsl = a->scan_mode == 0 ? select_slices(blocks_of(rg.max_entries), a->n_keep) : 0;
  if (nsl > 0) {
    const size_t cand = (size_t)R * nsl * a->n_keep;
    int32_t* cb = c.take<int32_t>(cand);
    float* cs = c.take<float>(cand);
    int32_t* cn = c.take<int32_t>((size_t)R * nsl);
    if (slices) *slices = SliceBufs{nsl, cb, cs, cn};
  }
  // MXFP8 route with a head-split attention plan (few rows): the rounded query, written
  // by the selection launch.  Larger launches round it inside the attention, where the
  // first tile's record loads hide that work.
  int32_t p_tk, p_sk, p_splits, p_hs;
  attn_plan(R, a->k, p_tk, p_sk, p_splits, p_hs);
  uint16_t* qm = a->qp_route == CSA2_QP_MXFP8 && p_hs ? c.take<uint16_t>((size_t)R * CSA2_HEADS * CSA2_D) : nullptr;
  if (q_mx) *q_mx = qm;
  return round_up(c.used, 256);
}

size_t csa2_decode_workspace_size(const csa2_decode_args* a) {
  if (!a || a->rg.num_rows <= 0 || a->k < 1 || a->n_keep < 1) return 0;
  return decode_layout(a, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
}

int csa2_decode(const csa2_decode_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (!a) return fail(CSA2_ERR_INVALID_ARG, "args is NULL");
  RaggedDev g;
  CHECK(check_ragged(&a->rg, g));
  if (a->k < 1 || a->k > CSA2_K_MAX) return fail(CSA2_ERR_UNSUPPORTED, "k must be in 1..%d", CSA2_K_MAX);
  if (a->n_keep < 1 || a->n_keep > CSA2_KEEP_MAX)
    return fail(CSA2_ERR_UNSUPPORTED, "n_keep must be in 1..%d", CSA2_KEEP_MAX);
  if (a->scan_mode != 0 && a->scan_mode != 1) return fail(CSA2_ERR_UNSUPPORTED, "scan_mode must be 0 or 1");
  if (a->qp_route != CSA2_QP_BF16 && a->qp_route != CSA2_QP_MXFP8)
    return fail(CSA2_ERR_UNSUPPORTED, "qp_route must be CSA2_QP_BF16 or CSA2_QP_MXFP8");
  if (g.R == 0) return CSA2_OK;
  CHECK(check_ptr(a->idx_k, 4, "idx_k"));
  CHECK(check_ptr(a->blk_sum, 16, "blk_sum"));
  CHECK(check_ptr(a->q_idx, 16, "q_idx"));
  CHECK(check_ptr(a->w_idx, 4, "w_idx"));
  if (a->scores && a->scores_ld < g.max_entries) return fail(CSA2_ERR_INVALID_ARG, "scores_ld < max_entries");
  if ((a->kept_blocks == nullptr) != (a->n_kept == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "kept_blocks and n_kept must both be set or both be NULL");
  if ((a->sel_idx == nullptr) != (a->n_sel == nullptr))
    return fail(CSA2_ERR_INVALID_ARG, "sel_idx and n_sel must both be set or both be NULL");
  const size_t need = csa2_decode_workspace_size(a);
  if (!ws || ws_bytes < need) return fail(CSA2_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu",
                                          need, ws_bytes);
  if (!aligned(ws, 256)) return fail(CSA2_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  float *scores, *blk_scores;
  int32_t *kept, *n_kept, *sel, *n_sel, *sel_rows;
  char* attn_ws;
  size_t attn_bytes;
  SliceBufs slices;
  uint16_t* q_mx;
  decode_layout(a, static_cast<char*>(ws), &scores, &blk_scores, &kept, &n_kept, &sel, &n_sel, &sel_rows, &attn_ws,
                &attn_bytes, &slices, &q_mx);
  const int64_t ld = a->scores ? a->scores_ld : (int64_t)round_up((size_t)(g.max_entries > 0 ? g.max_entries : 1), 64);
  const int64_t blk_ld = (int64_t)round_up((size_t)(blocks_of(g.max_entries) > 0 ? blocks_of(g.max_entries) : 1), 64);

  // The fine top-k also writes the picks' pool rows (for paged pools the page
  // translation is fused into the selection), and attention reads those.
  AttnArgs at{};
  CHECK(attn_args(g, a->q, a->main_kv, sel_rows ? sel_rows : sel, n_sel, a->k, a->swa, a->swa_scale, a->sm_scale,
                  a->out, a->lse, attn_ws, attn_bytes, at));
  at.sel_rows = sel_rows ? 1 : 0;
  at.qp_route = a->qp_route;
  if (q_mx) {
    // The query is rounded once per row by the selection launch (in parallel with it)
    // instead of in every attention workgroup.
    at.q = q_mx;
    at.q_rounded = 1;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  ScanArgs sa{};
  sa.g = g;
  sa.idx_k = a->idx_k;
  sa.blk_sum = a->blk_sum;
  sa.q_idx = a->q_idx;
  sa.w = a->w_idx;
  sa.scores = scores;
  sa.ld = ld;
  sa.blk_scores = blk_scores;
  sa.blk_ld = blk_ld;

  SelectArgs se{};
  se.g = g;
  se.blk_scores = blk_scores;
  se.blk_ld = blk_ld;
  se.n_keep = a->n_keep;
  se.keep_newest = a->keep_newest ? 1 : 0;
  se.kept = kept;
  se.n_kept = n_kept;
  se.kept_ld = a->n_keep + 1;
  se.scores = scores;
  se.ld = ld;
  se.k = a->k;
  se.sel = sel;
  se.n_sel = n_sel;
  se.sel_rows = sel_rows;
  se.n_slices = slices.n_slices;
  se.cand_blk = slices.blk;
  se.cand_sc = slices.sc;
  se.cand_n = slices.n;
  se.q = a->q;
  se.q_mx = q_mx;

  auto mark = [&](int i) -> hipError_t {
    return a->events ? hipEventRecord(static_cast<hipEvent_t>(a->events[i]), st) : hipSuccess;
  };
  LAUNCH(mark(0), "event record");
  if (a->scan_mode == 0) {
    // One launch scores every entry and every block summary; one launch selects.
    LAUNCH(launch_scan(sa, a->rg.max_rows_per_request, true, true, st), "scan");
    LAUNCH(mark(1), "event record");
    // Rows with many blocks: slices of blocks are ranked in parallel first.
    LAUNCH(launch_block_slices(se, st), "block slices");
    LAUNCH(launch_select_fused(se, st), "select");
  } else {
    // Coarse stage first, then score only the kept blocks' entries.
    LAUNCH(launch_scan(sa, a->rg.max_rows_per_request, false, true, st), "block scores");
    LAUNCH(launch_block_select(se, st), "block select");
    sa.kept = kept;
    sa.n_kept = n_kept;
    sa.kept_ld = a->n_keep + 1;
    LAUNCH(launch_scan_kept(sa, st), "index scan (kept blocks)");
    LAUNCH(mark(1), "event record");
    LAUNCH(launch_topk(se, false, st), "top-k");
  }
  LAUNCH(mark(2), "event record");
  LAUNCH(launch_attn_main(at, st), "sparse attention");
  LAUNCH(mark(3), "event record");
  LAUNCH(launch_attn_merge(at, st), "attention merge");
  LAUNCH(mark(4), "event record");
  return CSA2_OK;
}

int csa2_decode_static(const csa2_decode_args* a, void* stream) {
  if (!a) return fail(CSA2_ERR_INVALID_ARG, "args is NULL");
  const size_t need = csa2_decode_workspace_size(a);
  if (need > CSA2_STATIC_WS_BYTES)
    return fail(CSA2_ERR_WORKSPACE_TOO_SMALL,
                "decode needs %zu workspace bytes; the static workspace holds %zu (CSA2_STATIC_WS_BYTES)", need,
                (size_t)CSA2_STATIC_WS_BYTES);
  void* ws = nullptr;
  CHECK(static_workspace(&ws));
  return csa2_decode(a, ws, CSA2_STATIC_WS_BYTES, stream);
}

int csa2_debug_dequant(int32_t kind, const uint8_t* records, const float* scales, int64_t n, float* out,
                       void* stream) {
  if (kind != CSA2_DQ_MAIN && kind != CSA2_DQ_IDX && kind != CSA2_DQ_SWA)
    return fail(CSA2_ERR_INVALID_ARG, "unknown dequant kind %d", kind);
  if (n < 0) return fail(CSA2_ERR_INVALID_ARG, "negative record count");
  if (n == 0) return CSA2_OK;
  CHECK(check_ptr(records, 4, "records"));
  CHECK(check_ptr(out, 4, "out"));
  if (kind == CSA2_DQ_SWA) CHECK(check_ptr(scales, 4, "scales"));
  LAUNCH(launch_debug_dequant(kind, records, scales, n, out, reinterpret_cast<hipStream_t>(stream)), "dequant");
  return CSA2_OK;
}

int csa2_cache_write(const csa2_ragged* rg, const int64_t* row_pos, const uint16_t* kv_tok, const uint16_t* idx_tok,
                     uint16_t* ring_kv, uint16_t* ring_idx, const float* gamma_kv, const float* gamma_idx, float eps,
                     uint8_t* main_kv, uint8_t* idx_k, uint16_t* blk_sum, void* stream) {
  RaggedDev g;
  CHECK(check_ragged(rg, g));
  if (g.R == 0) return CSA2_OK;
  if (!(eps > 0.f) || !isfinite(eps)) return fail(CSA2_ERR_INVALID_ARG, "eps must be positive and finite");
  CHECK(check_ptr(row_pos, 8, "row_pos"));
  CHECK(check_ptr(kv_tok, 16, "kv_tok"));
  CHECK(check_ptr(idx_tok, 4, "idx_tok"));
  CHECK(check_ptr(ring_kv, 16, "ring_kv"));
  CHECK(check_ptr(ring_idx, 4, "ring_idx"));
  CHECK(check_ptr(gamma_kv, 4, "gamma_kv"));
  CHECK(check_ptr(gamma_idx, 4, "gamma_idx"));
  CHECK(check_ptr(main_kv, 16, "main_kv"));
  CHECK(check_ptr(idx_k, 4, "idx_k"));
  CHECK(check_ptr(blk_sum, 4, "blk_sum"));
  LAUNCH(launch_cache_write(g, rg->max_rows_per_request, row_pos, kv_tok, idx_tok, ring_kv, ring_idx, gamma_kv,
                            gamma_idx, eps, main_kv, idx_k, blk_sum, reinterpret_cast<hipStream_t>(stream)),
         "cache write");
  return CSA2_OK;
}

int csa2_debug_mxfp8(const float* x, int64_t n, float* out, void* stream) {
  if (n < 0 || n % 32 != 0) return fail(CSA2_ERR_INVALID_ARG, "n must be a non-negative multiple of 32");
  if (n == 0) return CSA2_OK;
  if (n / 32 / 64 >= (int64_t)0x7FFFFFFF) return fail(CSA2_ERR_UNSUPPORTED, "too many values for one launch");
  CHECK(check_ptr(x, 4, "x"));
  CHECK(check_ptr(out, 4, "out"));
  LAUNCH(launch_debug_mxfp8(x, n, out, reinterpret_cast<hipStream_t>(stream)), "mxfp8 rounding");
  return CSA2_OK;
}

int csa2_debug_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(CSA2_ERR_INVALID_ARG, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return CSA2_OK;
  if (bytes / 16 / 1024 >= (int64_t)0x7FFFFFFF) return fail(CSA2_ERR_UNSUPPORTED, "too many bytes for one launch");
  CHECK(check_ptr(src, 16, "src"));
  CHECK(check_ptr(sink, 4, "sink"));
  LAUNCH(launch_stream_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream)), "stream read");
  return CSA2_OK;
}

int csa2_debug_clock_trace(uint64_t* out, int32_t n, int32_t interval, void* stream) {
  if (n < 0 || n > CSA2_CLOCK_TRACE_MAX_SAMPLES) return fail(CSA2_ERR_INVALID_ARG, "n out of range");
  if (interval < 1 || (int64_t)n * interval > CSA2_CLOCK_TRACE_MAX_TICKS)
    return fail(CSA2_ERR_INVALID_ARG, "interval out of range");
  if (n == 0) return CSA2_OK;
  CHECK(check_ptr(out, 8, "out"));
  LAUNCH(launch_clock_trace(out, n, interval, reinterpret_cast<hipStream_t>(stream)), "clock trace");
  return CSA2_OK;
}

const char* csa2_status_string(int32_t status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported parameter";
    case CSA2_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CSA2_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* csa2_last_error(void) { return g_err; }

int32_t csa2_version(void) { return CSA2_VERSION; }

}  // extern "C"
