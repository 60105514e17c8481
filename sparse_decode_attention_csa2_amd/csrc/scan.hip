// Indexer scan and block-summary scoring on gfx950.
//
// Score of entry t for a query row (SGLang blog "DeepSeek-V4.1 Flash on SGLang",
// section "Architecture changes and KV cache compression": FP4 indexer keys of 68 B
// feed a hierarchical filter):  s_t = sum_{h<8} w_h * max(0, q_h . k_t), dim 128.
//
// Work mapping.  A wave handles 16 entries per MFMA group: lane l loads the 16 code
// bytes [16g, 16g+16) (dims 32g..32g+31, g = l/16) of entry l%16 plus that block's E8M0
// byte, and converts them in registers to bf16 (exact).  The contraction over the 128
// dims runs as four bf16 16x16x32 MFMAs whose K index is permuted (step c takes dims
// 32g + 8c + j from lane group g); the query operand uses the same permutation.  The A
// operand holds two query rows (8 heads each), so the rows of one request (verify
// rows) share a single read of its keys.  The ReLU and the head weights are applied to
// the fp32 MFMA output and the two half-sums meet with one cross-lane add.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kGroups = 4;                          // 16-entry groups per wave per tile
constexpr int kTile = kWaves * kGroups * 16;        // 256 entries (or blocks) per WG

template <int MAXPAIRS>
__device__ __forceinline__ void load_query(const ScanArgs& a, int r0, int r1, bf16x8_t (&qa)[MAXPAIRS][4],
                                           float (&wv)[MAXPAIRS][4]) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int p = 0; p < MAXPAIRS; ++p) {
    const int row = r0 + 2 * p + (m >> 3);
    const bool ok = row < r1;
    const uint16_t* qp = a.q_idx + ((int64_t)(ok ? row : r0) * CSA2_IDX_HEADS + (m & 7)) * CSA2_IDX_D + 32 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4_t v = ok ? load16(qp + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
      qa[p][c] = as_bf16x8(v);
    }
    const int orow = r0 + 2 * p + (g >> 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[p][i] = orow < r1 ? a.w[(int64_t)orow * CSA2_IDX_HEADS + 4 * (g & 1) + i] : 0.f;
  }
}

// Weighted ReLU over the lane's 4 heads, then the partner half (lane ^ 16).
__device__ __forceinline__ float head_sum(const f32x4_t& acc, const float (&wv)[4]) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) part = fmaf(wv[i], fmaxf(acc[i], 0.f), part);
  return part + shfl_xor_f(part, 16);
}

template <int MAXPAIRS>
__device__ __forceinline__ void score_group(const bf16x8_t (&kb)[4], const bf16x8_t (&qa)[MAXPAIRS][4],
                                            const float (&wv)[MAXPAIRS][4], int npairs, int r0, int r1,
                                            int64_t pos, int64_t n, float* out, int64_t ld) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
  for (int p = 0; p < MAXPAIRS; ++p) {
    if (p < npairs) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma16x16x32(qa[p][c], kb[c], acc);
      const float s = head_sum(acc, wv[p]);
      const int orow = r0 + 2 * p + (g >> 1);
      if ((g & 1) == 0 && orow < r1 && pos < n) out[(int64_t)orow * ld + pos] = s;
    }
  }
}

// PARTS: 1 = entries only, 2 = block summaries only, 3 = both in one launch (distinct
// instantiations keep the variants apart in kernel traces).
template <int MAXPAIRS, int PARTS>
__global__ __launch_bounds__(256) void k_scan(ScanArgs a) {
  const int b = blockIdx.y;
  int64_t e0, n;
  req_entries(a.g, b, e0, n);
  int r0, r1;
  req_rows(a.g, b, 2 * MAXPAIRS, r0, r1);
  if (r1 <= r0) return;
  const int npairs = (r1 - r0 + 1) >> 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 15, g = lane >> 4;

  // Block-summary tiles come first in the grid so that they start early and do not
  // trail the (many more) entry tiles.
  if ((int)blockIdx.x >= a.block_tiles) {
    const int64_t base = (int64_t)(blockIdx.x - a.block_tiles) * kTile + wave * (kGroups * 16);
    if (base >= n) return;
    // Issue every load of the wave's tile before any conversion.
    u32x4_t kc[kGroups];
    uint32_t ks[kGroups];
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      int64_t e = base + gi * 16 + m;
      e = e < n ? e : n - 1;
      const uint8_t* rec = a.idx_k + (e0 + e) * CSA2_IDX_BYTES;
      kc[gi] = load16_a4(rec + 16 * g);
      ks[gi] = rec[64 + g];
    }
    bf16x8_t qa[MAXPAIRS][4];
    float wv[MAXPAIRS][4];
    load_query<MAXPAIRS>(a, r0, r1, qa, wv);
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const float sc = e8m0_operand(ks[gi]);
      bf16x8_t kb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[c] = fp4x8_to_bf16(kc[gi][c], sc);
      score_group<MAXPAIRS>(kb, qa, wv, npairs, r0, r1, base + gi * 16 + m, n, a.scores, a.ld);
    }
  } else {
    int64_t bl0, nb;
    req_blocks(a.g, b, n, bl0, nb);
    const int64_t base = (int64_t)blockIdx.x * kTile + wave * (kGroups * 16);
    if (base >= nb) return;
    bf16x8_t qa[MAXPAIRS][4];
    float wv[MAXPAIRS][4];
    load_query<MAXPAIRS>(a, r0, r1, qa, wv);
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      int64_t j = base + gi * 16 + m;
      const int64_t jl = j < nb ? j : nb - 1;
      const uint16_t* sp = a.blk_sum + (bl0 + jl) * CSA2_IDX_D + 32 * g;
      bf16x8_t kb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[c] = as_bf16x8(load16(sp + 8 * c));
      score_group<MAXPAIRS>(kb, qa, wv, npairs, r0, r1, j, nb, a.blk_scores, a.blk_ld);
    }
  }
}

// Candidate-only scan: one wave per (kept block slot, row); scores the block's <= 64
// entries for that row only.
__global__ __launch_bounds__(64) void k_scan_kept(ScanArgs a) {
  const int r = blockIdx.y;
  const int slot = blockIdx.x;
  int nk = a.n_kept[r];
  nk = nk < 0 ? 0 : (nk > a.kept_ld ? a.kept_ld : nk);
  if (slot >= nk) return;
  const int b = row_request(a.g, r);
  int64_t e0, n;
  req_entries(a.g, b, e0, n);
  const int64_t blk = a.kept[(int64_t)r * a.kept_ld + slot];
  if (blk < 0 || blk * CSA2_BLOCK >= n) return;
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int64_t base = blk * CSA2_BLOCK;
  u32x4_t kc[4];
  uint32_t ks[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    int64_t e = base + gi * 16 + m;
    e = e < n ? e : n - 1;
    const uint8_t* rec = a.idx_k + (e0 + e) * CSA2_IDX_BYTES;
    kc[gi] = load16_a4(rec + 16 * g);
    ks[gi] = rec[64 + g];
  }
  bf16x8_t qa[1][4];
  float wv[1][4];
  load_query<1>(a, r, r + 1, qa, wv);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const float sc = e8m0_operand(ks[gi]);
    bf16x8_t kb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kb[c] = fp4x8_to_bf16(kc[gi][c], sc);
    score_group<1>(kb, qa, wv, 1, r, r + 1, base + gi * 16 + m, n, a.scores, a.ld);
  }
}

}  // namespace

template <int PARTS>
static void launch_scan_parts(const ScanArgs& a, int max_rows_per_req, dim3 grid, hipStream_t st) {
  if (max_rows_per_req <= 2)
    k_scan<1, PARTS><<<grid, dim3(256), 0, st>>>(a);
  else if (max_rows_per_req <= 4)
    k_scan<2, PARTS><<<grid, dim3(256), 0, st>>>(a);
  else if (max_rows_per_req <= 8)
    k_scan<4, PARTS><<<grid, dim3(256), 0, st>>>(a);
  else
    k_scan<8, PARTS><<<grid, dim3(256), 0, st>>>(a);
}

hipError_t launch_scan(ScanArgs a, int max_rows_per_req, bool entries, bool blocks, hipStream_t st) {
  const int64_t max_nb = (a.g.max_entries + CSA2_BLOCK - 1) / CSA2_BLOCK;
  a.entry_tiles = entries ? (int32_t)((a.g.max_entries + kTile - 1) / kTile) : 0;
  a.block_tiles = blocks ? (int32_t)((max_nb + kTile - 1) / kTile) : 0;
  const int gx = a.entry_tiles + a.block_tiles;
  if (gx == 0 || a.g.B == 0 || a.g.R == 0) return hipSuccess;
  const dim3 grid(gx, a.g.B);
  if (entries && blocks)
    launch_scan_parts<3>(a, max_rows_per_req, grid, st);
  else if (entries)
    launch_scan_parts<1>(a, max_rows_per_req, grid, st);
  else
    launch_scan_parts<2>(a, max_rows_per_req, grid, st);
  return hipGetLastError();
}

hipError_t launch_scan_kept(ScanArgs a, hipStream_t st) {
  if (a.g.R == 0 || a.kept_ld == 0) return hipSuccess;
  k_scan_kept<<<dim3(a.kept_ld, a.g.R), dim3(64), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa2
