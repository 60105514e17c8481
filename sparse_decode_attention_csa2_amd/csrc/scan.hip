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
#include <algorithm>
#include <type_traits>

#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kGroups = 4;                          // 16-entry groups per wave per tile
constexpr int kTile = kWaves * kGroups * 16;        // 256 entries (or blocks) per WG
constexpr int kRsrcWord3 = 0x00020000;             // raw buffer descriptor, gfx9 family
typedef float f32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));

#ifndef CSA2_SCAN_DEPTH
#define CSA2_SCAN_DEPTH 3
#endif
// Chunks per wave, at most: 4 (workgroups of 1,024 entries) measured fastest on the
// 64 x 65,536-entry scan (56-57 us against 58-59 us at 8, 59 at 16, 63-64 at 1).
#ifndef CSA2_SCAN_MAX_ITERS
#define CSA2_SCAN_MAX_ITERS 4
#endif
#ifndef CSA2_SCAN_WG_STAGE
#define CSA2_SCAN_WG_STAGE 1
#endif
constexpr int kMaxIters = CSA2_SCAN_MAX_ITERS;      // chunks per wave, at most
// Entry-only scans on the contiguous-read path: up to 13 chunks per wave, so that the
// score stage (13 KiB) and the key slots (18 KiB) leave room for kLdskWgsPerCu
// workgroups per CU in 160 KiB of LDS.
constexpr int kMaxItersLdsk = 13;
constexpr int kLdskWgsPerCu = 5;
#ifndef CSA2_SCAN_ONE_ROUND
#define CSA2_SCAN_ONE_ROUND 1
#endif
constexpr int kWgRows = 4;                          // rows staged per workgroup
#ifndef CSA2_SCAN_WAVES_PER_EU
#define CSA2_SCAN_WAVES_PER_EU 4
#endif
#ifndef CSA2_SCAN_LDSK_WAVES
#define CSA2_SCAN_LDSK_WAVES CSA2_SCAN_WAVES_PER_EU
#endif

// Waits until at most N vector-memory operations of this wave are outstanding (s_waitcnt
// with the other counters left alone).  The compiler sees the wait and counts on it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

// Weighted ReLU over the lane's 4 heads, then the partner half (lane ^ 16).  The ReLU
// is an integer max on the fp32 bits (negative floats are negative integers), and the
// exchange is a row swap (VALU; every lane gets the same sum).
__device__ __forceinline__ float head_sum(const f32x4_t& acc, const float (&wv)[4]) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) part = fmaf(wv[i], __int_as_float(max(__float_as_int(acc[i]), 0)), part);
  return xor16_add(part);
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

// Entry path: the group's scores go to the wave's LDS staging rows (row t of the
// request's rows, 64 entries of the chunk) and leave with one wide store per row.
template <int MAXPAIRS>
__device__ __forceinline__ void score_group_lds(const bf16x8_t (&kb)[4], const bf16x8_t (&qa)[MAXPAIRS][4],
                                                const float (&wv)[MAXPAIRS][4], int npairs, int gi,
                                                float (*sb)[64]) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int p = 0; p < MAXPAIRS; ++p) {
    if (p < npairs) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma16x16x32(qa[p][c], kb[c], acc);
      const float s = head_sum(acc, wv[p]);
      if ((g & 1) == 0) sb[2 * p + (g >> 1)][16 * gi + m] = s;
    }
  }
}

// Stores the staged scores of a 64-entry chunk starting at pos0: lane (t, j) writes
// entries 4j .. 4j+3 of row r0 + t, so a row leaves as 256 contiguous bytes.
template <int MAXPAIRS>
__device__ __forceinline__ void flush_chunk(float (*sb)[64], int nrows, int r0, int64_t pos0, int64_t n, float* out,
                                            int64_t ld) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int lane = threadIdx.x & 63, j = lane & 15;
#pragma unroll
  for (int t0 = 0; t0 < 2 * MAXPAIRS; t0 += 4) {
    const int t = t0 + (lane >> 4);
    if (t < nrows) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&sb[t][4 * j]);
      const int64_t pos = pos0 + 4 * j;
      float* o = out + (int64_t)(r0 + t) * ld + pos;
      if (pos + 4 <= n) {
        store16_a4(o, v);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (pos + i < n) o[i] = v[i];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// PARTS: 1 = entries only, 2 = block summaries only, 3 = both in one launch (distinct
// instantiations keep the variants apart in kernel traces).  PAGED: the pools are
// 64-entry pages reached through the page table (a chunk is exactly one page).
// LDSK: each wave reads its 64-entry chunk of keys as one contiguous 4,352-byte run of
// whole cache lines, with the non-temporal hint, and regroups it into the MFMA layout
// through LDS (otherwise lanes load that layout directly: 16-byte pieces 68 bytes
// apart plus scale bytes, partial lines that the L2 completes across loads, which the
// non-temporal hint defeats).
template <int MAXPAIRS, int PARTS, bool PAGED, bool LDSK = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    LDSK ? CSA2_SCAN_LDSK_WAVES : (MAXPAIRS == 1 ? CSA2_SCAN_WAVES_PER_EU : (MAXPAIRS == 8 ? 1 : 2))))) void k_scan(ScanArgs a) {
  const int b = blockIdx.y;
  int64_t e0, n;
  req_entries(a.g, b, e0, n, PAGED);
  int r0, r1;
  req_rows(a.g, b, 2 * MAXPAIRS, r0, r1);
  if (r1 <= r0) return;
  const int npairs = (r1 - r0 + 1) >> 1;
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave

  // Block-summary tiles come first in the grid so that they start early and do not
  // trail the (many more) entry tiles.  Some launches that also score entries have none:
  // their entry workgroups score their own blocks (see launch_scan).
  if ((int)blockIdx.x >= a.block_tiles) {
    // A workgroup takes iters x 4 consecutive 64-entry chunks; on step c wave w scores
    // chunk 4c + w, so the four waves of a step read 17 KB of contiguous keys.  Each
    // wave keeps kDepth chunks of loads in flight (a ring in registers): a chunk's slot
    // is refilled with the loads of the chunk kDepth steps ahead as soon as it has been
    // converted.  Keys are read through a buffer descriptor over the workgroup's
    // entries (per-lane offset = the lane's offset plus the chunk's, group offset
    // immediate); reads past the request's end return zeros (never stored).
    // Chunks of loads in flight per wave (fewer with more query rows held in registers).
    // The contiguous path (LDSK) keeps one, which leaves registers for five waves per
    // SIMD (64 x 65,536-entry scan 51.6 us with one, 54.0-54.5 with two, 56.6-57.8 with
    // three; decode steps also fastest with one).
    constexpr int kDepth = LDSK ? 1 : (MAXPAIRS <= 2 ? CSA2_SCAN_DEPTH : (MAXPAIRS == 4 ? 2 : 1));
    const int iters = a.iters;
    const int64_t wg_base = (int64_t)(blockIdx.x - a.block_tiles) * (kWaves * 64) * iters;
    if (wg_base >= n) return;   // uniform over the workgroup
    const int wg_n = (int)min<int64_t>(n - wg_base, (int64_t)kWaves * 64 * iters);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.idx_k + (e0 + wg_base) * CSA2_IDX_BYTES), (short)0, wg_n * CSA2_IDX_BYTES, kRsrcWord3);
    const int voff_c = m * CSA2_IDX_BYTES + 16 * g, voff_s = m * CSA2_IDX_BYTES + 64 + g;
    // Paged pools: lane c holds the page of the wave's chunk c (logical page
    // (wg_base + 64 wave)/64 + 4c); each chunk then gets a descriptor over its own page,
    // limited to the entries the request has there.
    int pv = 0;
    if constexpr (PAGED) {
      const int64_t lp = (wg_base + (int64_t)wave * 64) / CSA2_BLOCK + 4 * lane;
      if (lane < a.iters && lp * CSA2_BLOCK < n) pv = (int)page_of(a.g, b, lp);
    }
    constexpr bool kLdsKeys = LDSK;
    constexpr int kNonTemporal = 2;   // buffer-load cache policy: nt
    constexpr int kChunkLoads = kLdsKeys ? kGroups + 1 : 2 * kGroups;   // load instructions per chunk
    struct Chunk {
      u32x4_t kc[kLdsKeys ? kGroups + 1 : kGroups];
      uint32_t ks[kLdsKeys ? 1 : kGroups];
    };
    // The chunk offset goes into the per-lane offset (the scalar offset stays 0), so the
    // descriptor's range check, which covers the per-lane and instruction offsets,
    // bounds every read by the workgroup's (or, paged, the page's) entries.
    auto issue = [&](Chunk& ck, int lb) {
      __amdgpu_buffer_rsrc_t r = rs;
      int co = lb * CSA2_IDX_BYTES;
      if constexpr (PAGED) {
        // The chunk index, page and entry count are the same on every lane; readfirstlane
        // says so, which keeps the descriptor in scalar registers (otherwise every load
        // becomes a loop over the lanes' distinct descriptors).
        const int c = __builtin_amdgcn_readfirstlane((lb - wave * 64) / (kWaves * 64));
        const int64_t page = __builtin_amdgcn_readlane(pv, c);
        const int cnt = __builtin_amdgcn_readfirstlane(max(0, min(64, wg_n - lb)));
        r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.idx_k + page * (CSA2_BLOCK * CSA2_IDX_BYTES)),
                                              (short)0, cnt * CSA2_IDX_BYTES, kRsrcWord3);
        co = 0;
      }
      if constexpr (kLdsKeys) {
        // The chunk's 64 x 68 bytes in order: lane l takes bytes 16l + 1024q (q < 4) and
        // 4096 + 16(l mod 16).
        const int vo = co + 16 * lane;
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
          ck.kc[q] = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 1024 * q, 0, kNonTemporal);
        ck.kc[kGroups] = __builtin_amdgcn_raw_buffer_load_b128(r, co + 4096 + 16 * (lane & 15), 0, kNonTemporal);
      } else {
        const int vc = co + voff_c, vs = co + voff_s;
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
          ck.kc[gi] = __builtin_amdgcn_raw_buffer_load_b128(r, vc + gi * 16 * CSA2_IDX_BYTES, 0, 0);
          ck.ks[gi] = __builtin_amdgcn_raw_buffer_load_b8(r, vs + gi * 16 * CSA2_IDX_BYTES, 0, 0);
        }
      }
    };
    // Contiguous reads: each wave's loaded chunk is stored to its LDS slot of 64 x 68
    // bytes and read back in the MFMA lane layout.  Every 4 entries (17 16-byte pieces)
    // the slot skips one piece: the read-back's dword pairs (entries 68 bytes apart)
    // otherwise meet in the same banks two by two (32 conflict cycles per chunk in a
    // probe of the pattern; none with the skip, which leaves 14 in the stores).
    constexpr int kStageWords = 64 * CSA2_IDX_BYTES / 4 + 4 * 15;
    __shared__ __align__(16) uint32_t kstage[kLdsKeys ? kWaves : 1][kLdsKeys ? kStageWords : 4];
    // First word of 16-byte piece pc (< 272) of a chunk in its slot: pc + pc / 17 pieces
    // (pc * 241 >> 12 == pc / 17 for pc < 4,096).
    auto stage_word = [](int pc) { return 4 * (pc + ((pc * 241) >> 12)); };
    bf16x8_t qa[MAXPAIRS][4];
    float wv[MAXPAIRS][4];
    const int nrows = r1 - r0;
    // Scores are staged in LDS: with at most kWgRows rows the whole workgroup's scores
    // stay until the end and leave as contiguous row segments (one write burst per
    // workgroup); with more rows each wave flushes every chunk.
    // The contiguous path runs one row per request (a single stage row).
    constexpr bool kWgStage = CSA2_SCAN_WG_STAGE && 2 * MAXPAIRS <= kWgRows;
    constexpr int kStageRows = kWgStage ? (LDSK ? 1 : 2 * MAXPAIRS) : 1;
    // Entry-only contiguous-read scans size their stage at launch (dynamic LDS of
    // iters x 1 KiB): their chunks per wave are chosen so that the grid is one round.
    constexpr bool kDynStage = LDSK && PARTS == 1;
    constexpr int kStageLen = kWgStage && !kDynStage ? kWaves * 64 * kMaxIters : 1;
    __shared__ __align__(16) float wstage_s[kStageRows][kStageLen];
    extern __shared__ __align__(16) float scan_dyn_stage[];
    float* const wst = kDynStage ? scan_dyn_stage : &wstage_s[0][0];
    const int wst_ld = kDynStage ? kWaves * 64 * iters : kStageLen;
    __shared__ __align__(16) float sbuf[kWgStage ? 1 : kWaves][2 * MAXPAIRS][64];
    float (*sb)[64] = sbuf[kWgStage ? 0 : wave];
    // Scores of one chunk (16 x kGroups entries) from its codes and scale bytes in the
    // MFMA lane layout.
    // Scores of one chunk (16 x kGroups entries) from its codes in the MFMA lane layout
    // and each group's scale as the cvt operand (an fp32 whose exponent field is the
    // E8M0 code).
    __shared__ float wtrash[kWgStage && MAXPAIRS == 1 ? 64 : 1];
    auto score_chunk = [&](const u32x4_t (&kcv)[kGroups], const float (&sc)[kGroups], int lb) {
      if constexpr (MAXPAIRS == 1 && kWgStage) {
        // One row pair: the groups' four-step MFMA chains run interleaved (no result is
        // read right after the MFMA that writes it); the two half-sums meet through a
        // row swap of the wave (first = rows 0 and 2, second = rows 1 and 3, so every
        // lane ends with its pair's sum); every lane stores, the lanes that hold no
        // staged score to a scratch word, so no store is branched around.
        f32x4_t acc[kGroups];
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) acc[gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int gi = 0; gi < kGroups; ++gi) acc[gi] = mfma16x16x32(qa[0][c], fp4x8_to_bf16(kcv[gi][c], sc[gi]), acc[gi]);
        }
        // Two groups share one row swap: swapping group gi's partial sums (first operand)
        // with group gi + 1's leaves rows 0 and 2 with gi's pair of rows and rows 1 and 3
        // with gi + 1's, so lane row g adds the pair of group gi + (g & 1) for query row
        // g >> 1 (the same two terms as a swap of each group with itself).
        const int srow = LDSK ? 0 : (g >> 1);
        const bool real = LDSK ? g < 2 : true;
        static_assert(kGroups % 2 == 0, "groups in pairs");
#pragma unroll
        for (int gi = 0; gi < kGroups; gi += 2) {
          float part[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            part[j] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              part[j] = fmaf(wv[0][i], __int_as_float(max(__float_as_int(acc[gi + j][i]), 0)), part[j]);
          }
          const auto sw =
              __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
          float* dst = real ? &wst[srow * wst_ld + lb + 16 * (gi + (g & 1)) + m] : &wtrash[lane];
          *dst = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
      } else {
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
          bf16x8_t kb[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) kb[c] = fp4x8_to_bf16(kcv[gi][c], sc[gi]);
#pragma unroll
          for (int p = 0; p < MAXPAIRS; ++p) {
            if (p < npairs) {
              f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int c = 0; c < 4; ++c) acc = mfma16x16x32(qa[p][c], kb[c], acc);
              const float sv = head_sum(acc, wv[p]);
              if ((g & 1) == 0) {
                if constexpr (kWgStage)
                  wst[(2 * p + (g >> 1)) * wst_ld + lb + 16 * gi + m] = sv;
                else
                  sb[2 * p + (g >> 1)][16 * gi + m] = sv;
              }
            }
          }
        }
        if constexpr (!kWgStage) flush_chunk<MAXPAIRS>(sb, nrows, r0, wg_base + lb, n, a.scores, a.ld);
      }
    };
    // A chunk in a slot, read in the MFMA lane layout: lane (m, g) of group gi takes
    // entry 16gi + m's bytes 16g .. 16g+15 and its scale byte g (read as a byte and
    // shifted into the fp32 exponent field: one instruction, against a rotate and a
    // mask for a byte taken from the scale word).
    auto score_slot = [&](const uint32_t* kst, int lb) {
      u32x4_t kcv[kGroups];
      float sc[kGroups];
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) {
        const int e = 16 * gi + m;   // entry of the chunk; 17 words each, a piece skipped per 4
        const uint32_t* w = kst + e * (CSA2_IDX_BYTES / 4) + 4 * (e >> 2);
        kcv[gi] = u32x4_t{w[4 * g], w[4 * g + 1], w[4 * g + 2], w[4 * g + 3]};
        sc[gi] = e8m0_operand(reinterpret_cast<const uint8_t*>(w + 16)[g]);   // scale byte g
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      score_chunk(kcv, sc, lb);
    };
    // Register path of the contiguous reads: the loaded chunk goes to the wave's slot.
    auto stage = [&](const Chunk& ck) {
      if constexpr (kLdsKeys) {
        uint32_t* kst = kstage[wave];
#pragma unroll
        for (int q = 0; q < kGroups; ++q) *reinterpret_cast<u32x4_t*>(kst + stage_word(lane + 64 * q)) = ck.kc[q];
        if (lane < 16) *reinterpret_cast<u32x4_t*>(kst + stage_word(256 + lane)) = ck.kc[kGroups];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    };
    auto consume = [&](const Chunk& ck, int lb) {
      if constexpr (kLdsKeys) {
        stage(ck);
        score_slot(kstage[wave], lb);
      } else {
        u32x4_t kcv[kGroups];
        float sc[kGroups];
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
          kcv[gi] = ck.kc[gi];
          sc[gi] = e8m0_operand(ck.ks[gi]);
        }
        score_chunk(kcv, sc, lb);
      }
    };
    constexpr int kStep = kWaves * 64;
    const int lb0 = wave * 64;
    if (lb0 < wg_n) {
      // Start: the first chunks' loads, then the query (and wave 0's own block
      // summaries), then one wait for all of them, so that inside the loop no register
      // loaded before it makes the compiler wait for every load in flight.  ALL: every
      // ring slot is filled (chunks past the workgroup's entries read zeros through the
      // descriptor and are never scored).
      Chunk ring[kDepth];
      bf16x8_t kbs[4];
      int64_t jb0 = 0, jend = 0;
      // Both parts in one launch without block tiles: the workgroup's own 64-entry
      // blocks (4 x iters <= 16, one MFMA group) are scored by wave 0.
      bool own_blocks = PARTS == 3 && a.block_tiles == 0 && wave == 0;   // uniform per wave
      auto start = [&](auto all) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
          if (decltype(all)::value || d < iters) issue(ring[d], lb0 + d * kStep);
        if constexpr (PARTS == 3) {
          int64_t bl0 = 0;
          if (own_blocks) {
            int64_t nb;
            req_blocks(a.g, b, n, bl0, nb, PAGED);
            jb0 = wg_base / CSA2_BLOCK;
            jend = min<int64_t>(nb, (wg_base + wg_n + CSA2_BLOCK - 1) / CSA2_BLOCK);
            // None of the workgroup's blocks in the pool: nothing to score (this also
            // keeps the clamped row below in bounds).
            own_blocks = jend > jb0;
          }
          if (own_blocks) {
            const int64_t j = jb0 + m;
            const int64_t jl = j < jend ? j : jend - 1;
            const int64_t row = PAGED ? page_of(a.g, b, jl) : bl0 + jl;
            const uint16_t* sp = a.blk_sum + row * CSA2_IDX_D + 32 * g;
#pragma unroll
            for (int c = 0; c < 4; ++c) kbs[c] = as_bf16x8(load16(sp + 8 * c));
          }
        }
        load_query<MAXPAIRS>(a, r0, r1, qa, wv);
        wait_vmcnt<0>();
        if constexpr (PARTS == 3) {
          if (own_blocks) score_group<MAXPAIRS>(kbs, qa, wv, npairs, r0, r1, jb0 + m, jend, a.blk_scores, a.blk_ld);
        }
      };
      if (iters <= kDepth) {
        // Every chunk of the wave fits the ring: no refills.
        start(std::false_type{});
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          const int lb = lb0 + d * kStep;
          if (d < iters && lb < wg_n) consume(ring[d], lb);
        }
      } else if constexpr (kLdsKeys) {
        // One chunk in registers: once it is staged to LDS the next chunk's loads go out
        // before this chunk is scored (64 x 65,536-entry scan 53.1-55.2 -> 51.8-53.6 us
        // over runs of 200 launches; scoring first and then loading was the slower order).
        // The compiler would sink the loads below the scoring (their registers are free
        // for the conversions there); a memory clobber keeps them ahead of it, at 96
        // VGPRs (still five waves per SIMD): 52.2 -> 51.8 us, 1M-context batch 52.0 ->
        // 51.1 us (medians of eight alternating runs of 200 launches).
        start(std::true_type{});
        for (int c = 0; c < iters; ++c) {
          const int lb = lb0 + c * kStep;
          if (lb >= wg_n) break;
          wait_vmcnt<0>();
          stage(ring[0]);
          issue(ring[0], lb + kStep);
          asm volatile("" ::: "memory");
          score_slot(kstage[wave], lb);
        }
      } else {
        // The ring's slots are consumed in turn (no data-dependent exit inside the
        // unrolled ring) and every slot is refilled right after, so the waits before a
        // chunk leave the kDepth - 1 chunks issued after it in flight.
        start(std::true_type{});
        for (int c0 = 0; c0 < iters; c0 += kDepth) {
#pragma unroll
          for (int d = 0; d < kDepth; ++d) {
            const int lb = lb0 + (c0 + d) * kStep;
            if (c0 + d < iters && lb < wg_n) consume(ring[d], lb);
            issue(ring[d], lb + kDepth * kStep);
          }
        }
      }
    }
    if constexpr (kWgStage) {
      __syncthreads();
      for (int t = 0; t < nrows; ++t) {
        float* orow = a.scores + (int64_t)(r0 + t) * a.ld + wg_base;
        for (int i = 4 * (int)threadIdx.x; i < wg_n; i += 4 * kWaves * 64) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&wst[t * wst_ld + i]);
          if (i + 4 <= wg_n) {
            // A scan that only produces scores (PARTS 1) hands them to the caller: stream
            // them past the caches.  In the decode chain the select reads them next.
            if constexpr (PARTS == 1)
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4a4_t*>(orow + i));
            else
              store16_a4(orow + i, v);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (i + k < wg_n) orow[i + k] = v[k];
          }
        }
      }
    }
  } else {
    int64_t bl0, nb;
    req_blocks(a.g, b, n, bl0, nb, PAGED);
    // 16 x bgroups summaries per wave.  A summary is 256 B (3.8x an entry's 68 B), so
    // with one entry chunk per wave the block tiles take one group per wave and finish
    // with the entry tiles; larger scans give them up to four.
    const int bgroups = a.blk_groups;
    const int64_t base = (int64_t)blockIdx.x * (kWaves * 16) * bgroups + wave * 16 * bgroups;
    if (base >= nb) return;
    bf16x8_t qa[MAXPAIRS][4];
    float wv[MAXPAIRS][4];
    load_query<MAXPAIRS>(a, r0, r1, qa, wv);
    for (int gi = 0; gi < bgroups; ++gi) {
      const int64_t j = base + gi * 16 + m;
      const int64_t jl = j < nb ? j : nb - 1;
      const int64_t row = PAGED ? page_of(a.g, b, jl) : bl0 + jl;
      const uint16_t* sp = a.blk_sum + row * CSA2_IDX_D + 32 * g;
      bf16x8_t kb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[c] = as_bf16x8(load16(sp + 8 * c));
      score_group<MAXPAIRS>(kb, qa, wv, npairs, r0, r1, j, nb, a.blk_scores, a.blk_ld);
    }
  }
}

// Candidate-only scan: one wave per (kept block slot, row); scores the block's entries
// that the row sees (<= 64), for that row only.
__global__ __launch_bounds__(64) void k_scan_kept(ScanArgs a) {
  const int r = blockIdx.y;
  const int slot = blockIdx.x;
  int nk = a.n_kept[r];
  nk = nk < 0 ? 0 : (nk > a.kept_ld ? a.kept_ld : nk);
  if (slot >= nk) return;
  const int64_t vis = row_len_raw(a.g, r);
  const int b = row_request(a.g, r);
  int64_t e0, n;
  req_entries(a.g, b, e0, n);
  n = row_visible(a.g, vis, n);
  const int64_t blk = a.kept[(int64_t)r * a.kept_ld + slot];
  if (blk < 0 || blk * CSA2_BLOCK >= n) return;
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int64_t base = blk * CSA2_BLOCK;
  const int64_t row0 = paged(a.g) ? page_of(a.g, b, blk) * CSA2_BLOCK : e0 + base;   // the block is one page
  u32x4_t kc[4];
  uint32_t ks[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    int64_t e = base + gi * 16 + m;
    e = e < n ? e : n - 1;
    const uint8_t* rec = a.idx_k + (row0 + (e - base)) * CSA2_IDX_BYTES;
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

// Compute units of the current device (queried once per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus[dev];
}

template <int PARTS, bool PAGED>
static void launch_scan_rows(const ScanArgs& a, int max_rows_per_req, dim3 grid, hipStream_t st) {
  // Contiguous key reads (LDSK) where they measured faster: long workgroups, one row
  // pair per request, contiguous pools (64 x 65,536-entry scan 54.9 -> 50.8 us; decode
  // steps 117.7 -> 110.9 us at 64 x 128K, 105.7 -> 97.7 us at 1M context; short
  // workgroups were slower with them).
  if constexpr ((PARTS == 3 || PARTS == 1) && !PAGED) {
    if (max_rows_per_req == 1 && a.iters >= kMaxIters) {
      const size_t dyn = PARTS == 1 ? (size_t)kWaves * 64 * a.iters * sizeof(float) : 0;
      k_scan<1, PARTS, PAGED, true><<<grid, dim3(256), dyn, st>>>(a);
      return;
    }
  }
  if (max_rows_per_req <= 2)
    k_scan<1, PARTS, PAGED><<<grid, dim3(256), 0, st>>>(a);
  else if (max_rows_per_req <= 4)
    k_scan<2, PARTS, PAGED><<<grid, dim3(256), 0, st>>>(a);
  else if (max_rows_per_req <= 8)
    k_scan<4, PARTS, PAGED><<<grid, dim3(256), 0, st>>>(a);
  else
    k_scan<8, PARTS, PAGED><<<grid, dim3(256), 0, st>>>(a);
}

template <int PARTS>
static void launch_scan_parts(const ScanArgs& a, int max_rows_per_req, dim3 grid, hipStream_t st) {
  if (a.g.page_table)
    launch_scan_rows<PARTS, true>(a, max_rows_per_req, grid, st);
  else
    launch_scan_rows<PARTS, false>(a, max_rows_per_req, grid, st);
}

#ifndef CSA2_SCAN_TARGET_WGS
#define CSA2_SCAN_TARGET_WGS 2048
#endif

hipError_t launch_scan(ScanArgs a, int max_rows_per_req, bool entries, bool blocks, hipStream_t st) {
  const int64_t max_nb = (a.g.max_entries + CSA2_BLOCK - 1) / CSA2_BLOCK;
  // Chunks per wave: 1 while the entry part has at most CSA2_SCAN_TARGET_WGS workgroups
  // of 256 entries, then doubled (up to 8) so that large scans run as fewer, longer
  // workgroups that keep loads in flight across chunks.
  const int64_t tiles1 = (a.g.max_entries + kTile - 1) / kTile;
  int iters = 1;
  while (iters < kMaxIters && tiles1 * a.g.B >= (int64_t)CSA2_SCAN_TARGET_WGS * 2 * iters) iters *= 2;
  // Entry-only scans that take the contiguous-read path (see launch_scan_rows) run as
  // one round of workgroups: kLdskWgsPerCu per CU, each wave taking as many chunks as
  // that needs (a second, partly occupied round of workgroups would end the launch).
  if (entries && !blocks && !a.g.page_table && max_rows_per_req == 1 && iters >= kMaxIters) {
#if CSA2_SCAN_ONE_ROUND
    const int64_t chunks = (a.g.max_entries + CSA2_BLOCK - 1) / CSA2_BLOCK;
    const int64_t per_req = std::max<int64_t>(1, (int64_t)kLdskWgsPerCu * device_cus() / a.g.B);
    const int64_t it = (chunks + kWaves * per_req - 1) / (kWaves * per_req);
    iters = (int)std::min<int64_t>(std::max<int64_t>(it, kMaxIters), kMaxItersLdsk);
#else
    while (iters < 8 && tiles1 * a.g.B >= (int64_t)CSA2_SCAN_TARGET_WGS * 2 * iters) iters *= 2;
#endif
  }
  a.iters = iters;
  a.entry_tiles = entries ? (int32_t)((a.g.max_entries + (int64_t)kTile * iters - 1) / ((int64_t)kTile * iters)) : 0;
  a.blk_groups = iters < kGroups ? iters : kGroups;
  const int64_t blk_tile = (int64_t)kWaves * 16 * a.blk_groups;
  // With both parts, the entry workgroups score their own blocks instead of separate
  // block tiles when their workgroups are long (4 chunks per wave) or hold several row
  // pairs (where the block tiles would push the grid past one round of workgroups);
  // short one-row workgroups keep the block tiles off their critical path.
  const bool own_blocks = entries && blocks && (iters >= kMaxIters || max_rows_per_req > 2);
  a.block_tiles = (blocks && !own_blocks) ? (int32_t)((max_nb + blk_tile - 1) / blk_tile) : 0;
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
