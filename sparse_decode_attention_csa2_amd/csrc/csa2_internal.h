// Internal interfaces between libcsa2's host entry points and its kernels.
#pragma once

#include "csa2_dev.h"

namespace csa2 {

// The ragged descriptor as the kernels see it: device offset arrays plus host maxima
// used both for grid sizing and to clamp every device-provided offset.
// Every kernel receives it by value, so it is kept small (the host checks that the
// counts held in 32 bits fit).
struct RaggedDev {
  const int64_t* entry_off;
  const int64_t* block_off;
  const int32_t* row_off;
  const int32_t* row_req;
  const int64_t* row_swa_start;
  const int32_t* row_swa_len;
  const int64_t* row_len;      // nullable [R]: entries visible to each row
  const int32_t* page_table;   // nullable [B][pages_ld]: paged pools
  int64_t total_entries;
  int32_t max_entries;
  int32_t total_blocks;
  int32_t swa_tokens;
  int32_t total_pages;
  int32_t pages_ld;
  int32_t B;
  int32_t R;
};

__device__ __forceinline__ bool paged(const RaggedDev& g) { return g.page_table != nullptr; }

// Entries of request b, clamped to max_entries and (contiguous pools) to the pool; e0
// is the first pool row (contiguous pools only; 0 when paged).  Branch-free, so the
// loads issue together with the caller's other start-up loads.
// Kernels instantiated per pool layout pass `pg` as a constant; the default reads the
// descriptor.
__device__ __forceinline__ void req_entries(const RaggedDev& g, int b, int64_t& e0, int64_t& n, bool pg) {
  const int64_t a0 = g.entry_off[b], z0 = g.entry_off[b + 1];
  const int64_t a = pg ? a0 : clamp64(a0, 0, g.total_entries);
  const int64_t z = pg ? (z0 < a ? a : z0) : clamp64(z0, a, g.total_entries);
  e0 = pg ? 0 : a;
  n = (z - a) < g.max_entries ? (z - a) : g.max_entries;
}
__device__ __forceinline__ void req_entries(const RaggedDev& g, int b, int64_t& e0, int64_t& n) {
  req_entries(g, b, e0, n, paged(g));
}

// Entries row r sees out of its request's n, in two steps: row_len_raw loads the row's
// value (unconditionally, from a valid address either way, and before anything that
// depends on the request, so that it joins the first round of loads), row_visible
// applies it.
__device__ __forceinline__ int64_t row_len_raw(const RaggedDev& g, int r) {
  return *(g.row_len ? g.row_len + r : g.entry_off);
}
__device__ __forceinline__ int64_t row_visible(const RaggedDev& g, int64_t raw, int64_t n) {
  return g.row_len ? clamp64(raw, 0, n) : n;
}

// Physical page of logical page (block) j of request b; j < ceil(max_entries/64) <=
// pages_ld is the caller's to ensure.
__device__ __forceinline__ int64_t page_of(const RaggedDev& g, int b, int64_t j) {
  const int p = g.page_table[(int64_t)b * g.pages_ld + j];
  return p < 0 ? 0 : (p >= g.total_pages ? g.total_pages - 1 : p);
}

// First summary of request b and how many of its ceil(n/64) summaries the pool holds
// (paged pools: bl0 is unused and every summary is addressed through its page).
__device__ __forceinline__ void req_blocks(const RaggedDev& g, int b, int64_t n, int64_t& bl0, int64_t& nb_avail,
                                           bool pg) {
  const int64_t nb = (n + CSA2_BLOCK - 1) / CSA2_BLOCK;
  if (pg) {
    bl0 = 0;
    nb_avail = nb;
    return;
  }
  bl0 = clamp64(g.block_off[b], 0, g.total_blocks);
  nb_avail = (g.total_blocks - bl0) < nb ? (g.total_blocks - bl0) : nb;
}
__device__ __forceinline__ void req_blocks(const RaggedDev& g, int b, int64_t n, int64_t& bl0, int64_t& nb_avail) {
  req_blocks(g, b, n, bl0, nb_avail, paged(g));
}

// Pool row of entry t (< n) of request b, and of the summary of its block j.
__device__ __forceinline__ int64_t entry_row(const RaggedDev& g, int b, int64_t e0, int64_t t) {
  return paged(g) ? page_of(g, b, t / CSA2_BLOCK) * CSA2_BLOCK + (t % CSA2_BLOCK) : e0 + t;
}
__device__ __forceinline__ int64_t block_row(const RaggedDev& g, int b, int64_t bl0, int64_t j) {
  return paged(g) ? page_of(g, b, j) : bl0 + j;
}

// Rows of request b, clamped to [0, R) and to at most `cap` rows.
__device__ __forceinline__ void req_rows(const RaggedDev& g, int b, int cap, int& r0, int& r1) {
  int a = g.row_off[b], z = g.row_off[b + 1];
  a = a < 0 ? 0 : (a > g.R ? g.R : a);
  z = z < a ? a : (z > g.R ? g.R : z);
  if (z - a > cap) z = a + cap;
  r0 = a;
  r1 = z;
}

__device__ __forceinline__ int row_request(const RaggedDev& g, int r) {
  int b = g.row_req[r];
  return b < 0 ? 0 : (b >= g.B ? g.B - 1 : b);
}

// --------------------------------------------------------------------------------
// Launchers (each returns the launch's hipError_t).
// --------------------------------------------------------------------------------

struct ScanArgs {
  RaggedDev g;
  const uint8_t* idx_k;
  const uint16_t* blk_sum;
  const uint16_t* q_idx;
  const float* w;
  float* scores;          // [R][ld]   (entry part)
  int64_t ld;
  float* blk_scores;      // [R][blk_ld] (block part)
  int64_t blk_ld;
  int32_t entry_tiles;    // workgroups of the entry part (grid.x after the block part)
  int32_t iters;          // 64-entry chunks per wave in the entry part
  int32_t blk_groups;     // 16-summary groups per wave in the block part
  int32_t block_tiles;    // workgroups of the block part (first in grid.x)
  const int32_t* kept;    // candidate-only scan: [R][kept_ld]
  const int32_t* n_kept;
  int32_t kept_ld;
};

hipError_t launch_scan(ScanArgs a, int max_rows_per_req, bool entries, bool blocks, hipStream_t st);
hipError_t launch_scan_kept(ScanArgs a, hipStream_t st);

struct SelectArgs {
  RaggedDev g;
  const float* blk_scores;   // [R][blk_ld]
  int64_t blk_ld;
  int32_t n_keep;
  int32_t keep_newest;
  int32_t* kept;             // [R][kept_ld]
  int32_t* n_kept;           // [R]
  int32_t kept_ld;
  const float* scores;       // [R][ld]
  int64_t ld;
  int32_t k;
  int32_t* sel;              // [R][k]
  int32_t* n_sel;            // [R]
  float* sel_score;          // nullable [R][k]
  int32_t* sel_rows;         // nullable [R][k]: pool rows of the selected entries (-1 pad)
  // Sliced coarse stage (many blocks per row): slice s of row r keeps its n_keep best
  // blocks in cand_blk / cand_sc [R][n_slices][n_keep] (ascending), cand_n [R][n_slices].
  int32_t n_slices;          // 0: the coarse stage ranks all of a row's blocks at once
  int32_t* cand_blk;
  float* cand_sc;
  int32_t* cand_n;
  // MXFP8 route: the query [R][64][512] bf16, and where its MXFP8-rounded copy goes
  // (nullable: no rounding).  The selection launch that precedes attention rounds it in
  // extra workgroups (16 heads each), beside the rows' own workgroups.
  const uint16_t* q;
  uint16_t* q_mx;
};

// Blocks per slice of the sliced coarse stage, and when it is used: rows with more than
// kSelSliceFrom blocks, as long as the candidates fit the select's key buffer.
#ifndef CSA2_SEL_SLICE
#define CSA2_SEL_SLICE 1024
#endif
constexpr int kSelSlice = CSA2_SEL_SLICE;
constexpr int kSelSliceFrom = 4096;
constexpr int kSelSliceCand = 4096;
inline int32_t select_slices(int64_t max_nb, int32_t n_keep) {
  if (max_nb <= kSelSliceFrom) return 0;
  const int64_t s = (max_nb + kSelSlice - 1) / kSelSlice;
  return s * n_keep <= kSelSliceCand ? (int32_t)s : 0;
}

hipError_t launch_block_select(SelectArgs a, hipStream_t st);
hipError_t launch_topk(SelectArgs a, bool all_entries, hipStream_t st);
hipError_t launch_select_fused(SelectArgs a, hipStream_t st);
hipError_t launch_block_slices(SelectArgs a, hipStream_t st);

struct AttnArgs {
  RaggedDev g;
  const uint16_t* q;
  const uint8_t* main_kv;
  const int32_t* sel;        // request-local positions, or pool rows when sel_rows != 0
  const int32_t* n_sel;
  int32_t sel_ld;
  int32_t sel_rows;
  int32_t qp_route;          // CSA2_QP_BF16 or CSA2_QP_MXFP8
  const uint8_t* swa;
  const float* swa_scale;
  float sm_scale_log2;       // sm_scale * log2(e)
  int32_t tile_keys;         // keys per tile (64)
  int32_t split_keys;        // keys per split: a multiple of 32, at least one tile
  int32_t splits;
  float* opart;              // [R][splits][8 waves][16 d-tiles][64 lanes][4]
  float* mpart;              // [R][splits][64]
  float* lpart;              // [R][splits][64]
  float* out;                // [R][64][512]
  float* lse;                // [R][64]
  int32_t head_split;        // 1: four workgroups per split, one per head group
  int32_t q_rounded;         // MXFP8 route: q already holds the MXFP8-rounded query
};

void attn_plan(int64_t R, int32_t sel_ld, int32_t& tile_keys, int32_t& split_keys, int32_t& splits,
               int32_t& head_split);
size_t attn_workspace_bytes(int64_t R, int32_t sel_ld);
hipError_t launch_attn(AttnArgs a, hipStream_t st);
hipError_t launch_attn_main(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t st);
// Request-local selected positions -> pool rows (-1 for empty slots and positions the
// row does not see), for attention over paged pools.
hipError_t launch_sel_rows(const RaggedDev& g, const int32_t* sel, const int32_t* n_sel, int32_t sel_ld,
                           int32_t* rows, hipStream_t st);

hipError_t launch_cache_write(const RaggedDev& g, int32_t max_rows_per_request, const int64_t* row_pos,
                              const uint16_t* kv_tok, const uint16_t* idx_tok, uint16_t* ring_kv, uint16_t* ring_idx,
                              const float* gamma_kv, const float* gamma_idx, float eps, uint8_t* main_kv,
                              uint8_t* idx_k, uint16_t* blk_sum, hipStream_t st);
hipError_t launch_debug_mxfp8(const float* x, int64_t n, float* out, hipStream_t st);
hipError_t launch_clock_trace(uint64_t* out, int n, int interval, hipStream_t st);
hipError_t launch_debug_dequant(int kind, const uint8_t* rec, const float* scales, int64_t n, float* out,
                                hipStream_t st);

}  // namespace csa2
