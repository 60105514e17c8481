// Coarse block filter and fine top-k on gfx950 (one workgroup per query row).
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Architecture changes and KV
// cache compression": a hierarchical candidate filter leaves the top 512 global
// positions; section "DSpark adaptation and optimization": the chosen candidate blocks
// expand straight into a token mask.  Here: keep the n_keep best 64-entry blocks by
// summary score (ties to the lower block) plus the newest block, expand them into their
// entries, and keep the k best entries (ties to the lower position), ascending.
//
// Selection is exact.  Items (block scores, or the entries of the kept blocks) are
// gathered once into LDS as order-preserving 32-bit keys (0 = empty item), in chunks of
// 64; each wave owns a contiguous range of chunks, so item order is (wave, chunk, lane).
//  - k-th largest key: a first histogram (2048 LDS bins) bins the scores linearly
//    between the smallest and largest valid score; one wave scans the bins; the
//    members of a threshold bin with at most 64 of them are ranked by (key desc, order
//    asc) by one wave.  A larger bin (or a range without finite bins) continues with
//    11-bit digits of the key bits: keys normalised by the workgroup minimum, the
//    highest bits that vary first.
//  - output: the member collection also counts each wave's keys above the threshold
//    bin, the ranking wave adds its members' share, and per-chunk ballots then give each
//    item its rank among the selected items, so positions come out ascending without
//    sorting.
// These kernels run once per row and are latency-bound: loops stay rolled (small
// unroll factors, as instruction fetch of a large straight-line kernel would dominate),
// and every load in a loop is unconditional (key buffers are zero-padded to whole
// chunks, global indices are clamped) so the compiler can keep several in flight; a
// guarded load becomes a branch plus a wait per element.
#include "csa2_internal.h"

namespace csa2 {
namespace {

// Threads per row's workgroup: 1,024 (16 waves) walks each pass over a one-row fine
// stage's 4,160 candidates in half the chunks per wave of 512 (one-row step 29.0 ->
// 28.5 us, 1M-context step 85.3 -> 83.7 us, identical results).
#ifndef CSA2_SEL_THREADS
#define CSA2_SEL_THREADS 1024
#endif
constexpr int NT = CSA2_SEL_THREADS;
constexpr int NW = NT / kWave;
#ifndef CSA2_SEL_DIGIT
#define CSA2_SEL_DIGIT 11
#endif
// A threshold bin of at most CSA2_SEL_MEMMAX (<= 64) keys is resolved from its members
// by one wave; larger bins take another histogram pass over the next digit.  64 measured
// fastest: one-row step 35.8 -> 35.4 us against 256 (bins of 65-256 keys resolved by a
// radix-4 descent); 11-bit digits beat 10 and 12.
#ifndef CSA2_SEL_MEMMAX
#define CSA2_SEL_MEMMAX 64
#endif
constexpr int kDigit = CSA2_SEL_DIGIT;                       // key bits ranked per histogram pass
constexpr int kBins = 1 << kDigit;
static_assert(kBins >= 4 * kWave && kBins <= kWave * kWave, "bins per lane: 4 .. 64");
constexpr int kMemMax = CSA2_SEL_MEMMAX;                     // bin members resolved directly
static_assert(kMemMax >= 1 && kMemMax <= 64, "members are ranked one per lane");
constexpr int kMaxCand = (CSA2_KEEP_MAX + 1) * CSA2_BLOCK;   // 8256 candidate slots
constexpr int kLdsBlocks = 16384;                            // block keys held in LDS
// Gather batch per thread: enough for a fine stage of up to 72 kept blocks (4,608
// candidates) in one round of loads (5 at 1,024 threads).  Every load of a batch is issued
// (clamped), so a larger batch only adds loads: 16 made the one-row step 1.5 us slower.
#ifndef CSA2_SEL_GATHER_BATCH
#define CSA2_SEL_GATHER_BATCH ((4608 + NT - 1) / NT)
#endif
constexpr int kGB = CSA2_SEL_GATHER_BATCH;                   // gather batch per thread
// Rows of at most this many block slots rank their blocks after one round of loads
// (kSmallRowBlocks / NT per thread, issued before the row's offsets are known).
constexpr int kSmallRowBlocks = 1024;
static_assert(kSmallRowBlocks % NT == 0, "whole loads per thread");
static_assert(kMaxCand >= CSA2_TOPK_ALL_MAX, "candidate buffer");
static_assert(kLdsBlocks >= kMaxCand, "shared key buffer");
static_assert(kLdsBlocks >= kSelSliceCand && kSelSlice % kWave == 0, "sliced coarse stage buffers");

struct SelShared {
  alignas(16) uint32_t hist[2][kBins];
  uint32_t red[2 * NW];
  uint32_t cnt[NW];
  uint32_t wgt[NW], weq[NW];
  uint32_t mkey[kMemMax];
  uint32_t mwave[kMemMax];            // wave that holds each member
  uint32_t digit, above;
  int32_t m, mcnt;
  uint32_t T;
  int32_t n_gt;
  int32_t flag;
  int32_t nk;
  int32_t kl[CSA2_KEEP_MAX + 2];
  int32_t kpage[CSA2_KEEP_MAX + 2];   // pool page of each kept block (paged pools)
};

__device__ __forceinline__ void wave_chunks(int n, int& c0, int& c1) {
  const int nch = (n + kWave - 1) / kWave, w = threadIdx.x / kWave;
  c0 = w * nch / NW;
  c1 = (w + 1) * nch / NW;
}

// Key range and count of the valid (non-zero) items, reduced per wave into sh.red and
// sh.cnt by the gather (one barrier later every thread reads the workgroup figures).
__device__ __forceinline__ void range_publish(uint32_t lo, uint32_t hi, uint32_t cnt, SelShared& sh) {
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), kWave - 1);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.red[2 * (threadIdx.x / kWave)] = lo;
    sh.red[2 * (threadIdx.x / kWave) + 1] = hi;
    sh.cnt[threadIdx.x / kWave] = cnt;
  }
}

// Valid items published by range_publish (after a barrier).
__device__ __forceinline__ int valid_count(const SelShared& sh) {
  int c = 0;
  for (int w = 0; w < NW; ++w) c += (int)sh.cnt[w];
  return c;
}

// Score of a key (inverse of score_key for non-zero keys).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// k-th largest key among the valid items (1 <= k < valid count): T and n_gt = number of
// keys > T.  key(i), defined for every i in the whole chunks covering n, returns 0 for
// an empty item.  Expects the per-wave key ranges in sh.red and sh.hist[0] zeroed,
// both behind a barrier.  Returns true when it has also left each wave's count of keys
// > T and == T (over the wave's chunks) in sh.wgt / sh.weq, behind a barrier.
template <class KeyF>
__device__ bool sel_kth(KeyF key, int n, int k, SelShared& sh, uint32_t& T, int& n_gt) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int c0, c1;
  wave_chunks(n, c0, c1);
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, sh.red[2 * w]);
    hi = max(hi, sh.red[2 * w + 1]);
  }

  // Wave 0: the bin of hist holding the rem-th largest key (bins ascend with the keys)
  // into sh.digit, the keys in higher bins into sh.above, the bin's count into sh.m.
  auto find_bin = [&](const uint32_t* hist, int rem) {
    // Lane l owns the kPer bins below kBins - kPer * l (highest first); find the bin
    // holding the rem-th key.
    constexpr int kPer = kBins / kWave;
    const uint32_t* hb = hist + kBins - kPer * (lane + 1);
    uint32_t tot = 0u;
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(hb + 4 * q);
      tot += v[0] + v[1] + v[2] + v[3];
    }
    const uint32_t before = wave_incl_scan(tot) - tot;
    // The lane whose kPer bins hold the rem-th key; its bins are then examined by
    // lanes 0 .. kPer-1 in parallel (lane x takes the x-th bin in descending order).
    const uint64_t owner = __ballot(before < (uint32_t)rem && before + tot >= (uint32_t)rem);
    const int tl = owner ? (int)__builtin_ctzll(owner) : kWave - 1;
    const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)before, tl);
    const int x = lane & (kPer - 1);
    const uint32_t bin = (uint32_t)(kBins - kPer * (tl + 1) + (kPer - 1 - x));
    const uint32_t cnt = lane < kPer ? hist[bin] : 0u;
    const uint32_t incl = tb + wave_incl_scan(cnt);
    const uint64_t hit = __ballot(lane < kPer && incl >= (uint32_t)rem);
    if (lane == (int)__builtin_ctzll(hit)) {
      sh.digit = bin;
      sh.above = incl - cnt;
      sh.m = (int)cnt;
    }
  };

  // Members of the threshold bin (member(key) true) into sh.mkey / sh.mwave / sh.mcnt,
  // and each wave's count of keys above the bin (above(key) true) into sh.wgt; the
  // caller then needs one barrier.
  auto collect = [&](auto member, auto above) {
    uint32_t gtc = 0u;   // per lane: no cross-lane operation in the loop, so it unrolls
#pragma unroll 4
    for (int c = c0; c < c1; ++c) {
      const int i = c * kWave + lane;
      const uint32_t kk = key(i);
      gtc += (kk && above(kk)) ? 1u : 0u;
      if (kk && member(kk)) {
        const int slot = min(atomicAdd(&sh.mcnt, 1), kMemMax - 1);   // < m <= kMemMax by construction
        sh.mkey[slot] = kk;
        sh.mwave[slot] = (uint32_t)wave;
      }
    }
    gtc = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(gtc), kWave - 1);
    if (lane == 0) {
      sh.wgt[wave] = gtc;
      sh.weq[wave] = 0u;
    }
  };

  // Wave 0, at most 64 members: lane i ranks member i against all of them (keys > and
  // ==); the rem-th largest is held by the lane with n_greater < rem <= n_greater +
  // n_equal.  Then each wave's members > T join its count of keys above the bin, and its
  // members == T give its count of ties.
  auto rank_members = [&](int rem, int above_total) {
    const int m = __builtin_amdgcn_readfirstlane(sh.mcnt);
    const uint32_t kk = lane < m ? sh.mkey[lane] : 0u;
    const uint32_t kw = lane < m ? sh.mwave[lane] : (uint32_t)NW;
    uint32_t gt = 0u, eq = 0u;
    for (int j = 0; j < m; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kk, j);
      gt += kj > kk ? 1u : 0u;
      eq += kj == kk ? 1u : 0u;
    }
    const uint64_t hit = __ballot(lane < m && gt < (uint32_t)rem && (uint32_t)rem <= gt + eq);
    const int src = hit ? (int)__builtin_ctzll(hit) : 0;
    const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)kk, src);
    const uint32_t tg = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
    if (lane < m) atomicAdd(kk > t ? &sh.wgt[kw] : &sh.weq[kw], kk >= t ? 1u : 0u);
    if (lane == 0) {
      sh.T = t;
      sh.n_gt = above_total + (int)tg;
    }
  };

  // First pass: bins linear in the score between the smallest and the largest valid
  // score.  The float keys' leading bits are mostly exponent, so an 11-bit digit of them
  // puts a row's scores into a few dozen of the 2,048 bins and the threshold bin often
  // holds over a hundred keys (one more histogram pass); bins linear in the value leave a
  // few keys in it.  The bin is a non-decreasing function of the key (one rounding of
  // s * scale + off, clamped), so bins ascend with the keys and the threshold bin's
  // members are exactly the keys that map to it.  A bin of more than 64 keys, or a range
  // that does not give finite bins, continues with the digits of the key bits.
  int buf = 0;
  {
    const float slo = key_score(lo), shi = key_score(hi);
    const float range = shi - slo;
    const float scale = (float)kBins / range;
    const float off = -slo * scale;
    const bool lin_ok = range > 0.f && scale < __builtin_inff() && off < __builtin_inff() && off > -__builtin_inff();
    if (lin_ok) {
      auto lbin = [&](uint32_t kk) {
        return (uint32_t)__builtin_amdgcn_fmed3f(__builtin_fmaf(key_score(kk), scale, off), 0.f, (float)(kBins - 1));
      };
      uint32_t* hist = sh.hist[0];
#pragma unroll 4
      for (int c = c0; c < c1; ++c) {
        const uint32_t kk = key(c * kWave + lane);
        atomicAdd(&hist[lbin(kk) & (kBins - 1)], kk ? 1u : 0u);   // unconditional: no branch per key
      }
      for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[1][i] = 0u;
      if (threadIdx.x == 0) sh.mcnt = 0;
      __syncthreads();
      if (wave == 0) find_bin(hist, k);
      __syncthreads();
      if (sh.m <= kMemMax) {
        const uint32_t d = sh.digit;
        collect([&](uint32_t kk) { return lbin(kk) == d; }, [&](uint32_t kk) { return lbin(kk) > d; });
        __syncthreads();
        if (wave == 0) rank_members(k - (int)sh.above, (int)sh.above);
        __syncthreads();
        T = sh.T;
        n_gt = sh.n_gt;
        return true;
      }
      buf = 1;   // sh.hist[1] is zeroed
    }
  }

  const uint32_t span = hi - lo;
  int L = span ? 32 - __builtin_clz(span) : 0;   // bits of (key - lo) that vary
  uint32_t prefix = 0u;                           // (key - lo) >> L of the keys in play
  int rem = k, above_total = 0;
  while (true) {
    const int shift = L > kDigit ? L - kDigit : 0;
    const uint32_t dmask = (1u << (L - shift)) - 1u;
    uint32_t* hist = sh.hist[buf];
#pragma unroll 4
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = key(c * kWave + lane);
      const uint32_t v = kk - lo;
      atomicAdd(&hist[(v >> shift) & dmask], (kk && ((uint64_t)v >> L) == prefix) ? 1u : 0u);
    }
    for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[buf ^ 1][i] = 0u;
    if (threadIdx.x == 0) sh.mcnt = 0;
    __syncthreads();
    if (wave == 0) find_bin(hist, rem);
    __syncthreads();
    const int m = sh.m;
    rem -= (int)sh.above;
    above_total += (int)sh.above;
    prefix = (prefix << (L - shift)) | sh.digit;
    L = shift;
    buf ^= 1;
    if (L == 0) {   // every key left is equal: the first rem of them by order
      T = lo + prefix;
      n_gt = above_total;
      return false;
    }
    if (m <= kMemMax) break;
  }
  // Collect the bin's members; one wave then finds the rem-th largest member key and
  // counts the members above it.
  collect([&](uint32_t kk) { return ((uint64_t)(kk - lo) >> L) == prefix; },
          [&](uint32_t kk) { return ((uint64_t)(kk - lo) >> L) > prefix; });
  __syncthreads();
  if (wave == 0) rank_members(rem, above_total);
  __syncthreads();
  T = sh.T;
  n_gt = sh.n_gt;
  return true;
}

// Emit (output position, item, key, aux(item)) for every valid key > T and the first
// need_eq keys == T, positions ascending with item order.  aux(i) (any i in the whole
// chunks covering n) is read with the key, ahead of the test, so the emit waits on no
// read of its own.  counted: each wave's counts of keys > T and == T are already in
// sh.wgt / sh.weq (behind a barrier).  All threads must call it.
template <class KeyF, class AuxF, class EmitF>
__device__ void sel_emit(KeyF key, int n, uint32_t T, int need_eq, bool counted, SelShared& sh, AuxF aux,
                         EmitF emit) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int c0, c1;
  wave_chunks(n, c0, c1);
  if (!counted) {
    uint32_t gtc = 0u, eqc = 0u;
#pragma unroll 4
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = key(c * kWave + lane);
      gtc += __popcll(__ballot(kk > T));
      eqc += __popcll(__ballot(kk && kk == T));
    }
    if (lane == 0) {
      sh.wgt[wave] = gtc;
      sh.weq[wave] = eqc;
    }
    __syncthreads();
  }
  uint32_t gb = 0u, eb = 0u;
  for (int w = 0; w < wave; ++w) {
    gb += sh.wgt[w];
    eb += sh.weq[w];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c = c0; c < c1; ++c) {
    const int i = c * kWave + lane;
    const uint32_t kk = key(i);
    const auto ax = aux(i);
    const bool g = kk > T, e = kk && kk == T;
    const uint64_t bg = __ballot(g), be = __ballot(e);
    const uint32_t gbl = gb + __popcll(bg & below), ebl = eb + __popcll(be & below);
    // An item > T follows the ties taken before it; a tie is taken while ebl < need_eq,
    // where min(ebl, need_eq) = ebl: one position formula for both.
    if (g || (e && ebl < (uint32_t)need_eq)) emit((int)(gbl + min(ebl, (uint32_t)need_eq)), i, kk, ax);
    gb += __popcll(bg);
    eb += __popcll(be);
  }
}

// Item aux for emits that need none.
struct NoAux {
  __device__ int operator()(int) const { return 0; }
};

// The `take` best of n items (everything valid when n_valid <= take); returns the count.
template <class KeyF, class AuxF, class EmitF>
__device__ int sel_top(KeyF key, int n, int n_valid, int take, SelShared& sh, AuxF aux, EmitF emit) {
  uint32_t T = 0u;
  int n_gt = 0;
  bool counted = false;
  if (n_valid > take) {
    counted = sel_kth(key, n, take, sh, T, n_gt);
  } else {
    take = n_valid;
  }
  sel_emit(key, n, T, take - n_gt, counted, sh, aux, emit);
  return take;
}

// Gather item scores into kbuf as keys: load(i, ok) reads item i's score (a safe
// address when !ok) and ok(i) tells whether item i < n exists; kGB independent loads in
// flight per thread; kbuf is zero-padded to whole chunks.  Publishes the per-wave key
// range and zeroes the first histogram buffer; the caller then needs one barrier.
template <int GB = kGB, class ValidF, class LoadF>
__device__ void gather(int n, ValidF valid, LoadF load, uint32_t* kbuf, SelShared& sh,
                       const float* pre = nullptr) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, cnt = 0u;
  auto keys = [&](int base, const float (&v)[GB], const bool (&ok)[GB]) {
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      const uint32_t kk = score_key(v[u]) & (0u - (uint32_t)ok[u]);   // masked, not branched
      if (i < n) kbuf[i] = kk;
      // Branch-free: an empty key (0) leaves the minimum, maximum and count alone.
      lo = min(lo, kk ? kk : 0xFFFFFFFFu);
      hi = max(hi, kk);
      cnt += kk ? 1u : 0u;
    }
  };
  int base0 = 0;
  if (pre) {   // the first batch was loaded by the caller
    float v[GB];
    bool ok[GB];
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int i = u * NT + (int)threadIdx.x;
      ok[u] = (i < n) & valid(i);
      v[u] = pre[u];
    }
    keys(0, v, ok);
    base0 = NT * GB;
  }
  for (int base = base0; base < n; base += NT * GB) {
    float v[GB];
    bool ok[GB];
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      ok[u] = (i < n) & valid(i);   // valid() must accept any i (clamped reads)
      v[u] = load(i, ok[u]);
    }
    keys(base, v, ok);
  }
  const int padded = (n + kWave - 1) / kWave * kWave;
  for (int i = n + (int)threadIdx.x; i < padded; i += NT) kbuf[i] = 0u;
  range_publish(lo, hi, cnt, sh);
  for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[0][i] = 0u;
}

template <bool PAGED>
__device__ __forceinline__ int row_blocks(const SelectArgs& a, int r, int64_t& n, int64_t& e0) {
  const int64_t vis = row_len_raw(a.g, r);
  const int b = row_request(a.g, r);
  int64_t bl0, nb;
  req_entries(a.g, b, e0, n, PAGED);
  n = row_visible(a.g, vis, n);
  req_blocks(a.g, b, n, bl0, nb, PAGED);
  return (int)nb;
}

// First gather batch of row r's block scores, loaded before the row's offsets are known
// (the loads are clamped to the row's blk_ld <= kLdsBlocks slots).
template <int GB>
__device__ __forceinline__ void prefetch_blocks(const SelectArgs& a, int r, float (&pre)[GB]) {
  const float* bs = a.blk_scores + (int64_t)r * a.blk_ld;
  const int lim = (int)a.blk_ld - 1;
#pragma unroll
  for (int u = 0; u < GB; ++u) pre[u] = bs[min(u * NT + (int)threadIdx.x, lim)];
  // Keep the loads here, ahead of the offset loads' waits.
  asm volatile("" ::: "memory");
}

// Coarse stage of row r: kept blocks (ascending) into sh.kl / sh.nk and, if given, the
// global kept list.  BIG: blk_ld may exceed kLdsBlocks (rows with more blocks rank
// straight from global memory); otherwise pre holds the first gather batch.
template <bool BIG, int GB = kGB>
__device__ void coarse(const SelectArgs& a, int r, int nb, SelShared& sh, uint32_t* kbuf, const float* pre) {
  const float* bs = a.blk_scores + (int64_t)r * a.blk_ld;
  int32_t* kout = a.kept ? a.kept + (int64_t)r * a.kept_ld : nullptr;
  if (threadIdx.x == 0) sh.flag = 0;
  auto emit = [&](int pos, int i, uint32_t, int) {
    sh.kl[pos] = i;
    if (kout) kout[pos] = i;
    if (i == nb - 1) sh.flag = 1;
  };
  int cnt;
  if (!BIG || nb <= kLdsBlocks) {
    // The gather runs over the row's blk_ld slots (a launch constant, >= nb) with its
    // loads clamped to them, so they need not wait for the request's offsets; items at
    // or past nb are masked to empty keys.
    const int lim = (int)(a.blk_ld < kLdsBlocks ? a.blk_ld : kLdsBlocks);
    gather<GB>(lim, [&](int i) { return i < nb; }, [&](int i, bool) { return bs[min(i, lim - 1)]; }, kbuf, sh,
               BIG ? nullptr : pre);
    __syncthreads();
    cnt = sel_top([&](int i) { return kbuf[i]; }, nb, valid_count(sh), a.n_keep, sh, NoAux(), emit);
  } else {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, nv = 0u;
    for (int i = threadIdx.x; i < nb; i += NT) {
      const uint32_t kk = score_key(bs[i]);
      lo = min(lo, kk ? kk : 0xFFFFFFFFu);
      hi = max(hi, kk);
      nv += kk ? 1u : 0u;
    }
    range_publish(lo, hi, nv, sh);
    for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[0][i] = 0u;
    __syncthreads();
    auto gkey = [&](int i) {
      const float v = bs[i < nb ? i : 0];
      return i < nb ? score_key(v) : 0u;
    };
    cnt = sel_top(gkey, nb, valid_count(sh), a.n_keep, sh, NoAux(), emit);
  }
  __syncthreads();
  // The newest block joins if the ranking left it out (it is the largest index, so the
  // list stays ascending).
  if (nb > 0 && a.keep_newest && sh.flag == 0) {
    if (threadIdx.x == 0) {
      sh.kl[cnt] = nb - 1;
      if (kout) kout[cnt] = nb - 1;
    }
    ++cnt;
  }
  if (kout) {
    for (int i = cnt + threadIdx.x; i < a.kept_ld; i += NT) kout[i] = -1;
    if (threadIdx.x == 0) a.n_kept[r] = cnt;
  }
  if (threadIdx.x == 0) sh.nk = cnt;
}

// Sliced coarse stage, second level: rank the slices' candidates for row r (slot-major,
// which is ascending block order, so ties still go to the lower block) and keep the
// n_keep best plus the newest block, as coarse() does for all blocks at once.  The
// n_keep best of a row are among the n_keep best of their slices.
__device__ void coarse_cand(const SelectArgs& a, int r, int nb, SelShared& sh, uint32_t* kbuf) {
  int32_t* kout = a.kept ? a.kept + (int64_t)r * a.kept_ld : nullptr;
  const int K = a.n_keep, items = a.n_slices * K;
  const float* cs = a.cand_sc + (int64_t)r * items;
  const int32_t* cb = a.cand_blk + (int64_t)r * items;
  const int32_t* cn = a.cand_n + (int64_t)r * a.n_slices;
  if (threadIdx.x == 0) sh.flag = 0;
  auto emit = [&](int pos, int i, uint32_t, int) {
    const int blk = cb[i];
    sh.kl[pos] = blk;
    if (kout) kout[pos] = blk;
    if (blk == nb - 1) sh.flag = 1;
  };
  // gather() evaluates valid(i) for every i of its last whole batch (up to
  // kSelSliceCand - 1, past `items`), so the slice index is clamped to the row's slices: cand_n is the
  // last buffer of the decode workspace and must not be read past its end.
  const int last_slice = a.n_slices - 1;
  static_assert(kSelSliceCand % NT == 0, "candidate gather: one batch of whole rows");
  gather<kSelSliceCand / NT>(items, [&](int i) { return i % K < cn[min(i / K, last_slice)]; },
                             [&](int i, bool ok) { return cs[ok ? i : 0]; }, kbuf, sh);
  __syncthreads();
  int cnt = sel_top([&](int i) { return kbuf[i]; }, items, valid_count(sh), K, sh, NoAux(), emit);
  __syncthreads();
  if (nb > 0 && a.keep_newest && sh.flag == 0) {
    if (threadIdx.x == 0) {
      sh.kl[cnt] = nb - 1;
      if (kout) kout[cnt] = nb - 1;
    }
    ++cnt;
  }
  if (kout) {
    for (int i = cnt + threadIdx.x; i < a.kept_ld; i += NT) kout[i] = -1;
    if (threadIdx.x == 0) a.n_kept[r] = cnt;
  }
  if (threadIdx.x == 0) sh.nk = cnt;
}

// Fine stage of row r over the kept blocks sh.kl[0 .. nk) (chunk s = kept block s,
// lane = entry) or, with all_entries, over entries 0 .. n-1.  Candidates are the items
// with a key: positions the row sees whose score is not NaN.  When a.sel_rows is set
// the picks' pool rows go there too: e0 + position for contiguous pools, the page
// table's row for paged ones (PAGED).
template <bool PAGED>
__device__ void fine(const SelectArgs& a, int r, int64_t n, int64_t e0, int nk, bool all_entries, SelShared& sh,
                     uint32_t* kbuf) {
  const float* sc = a.scores + (int64_t)r * a.ld;
  const int k = a.k;
  int32_t* sel = a.sel + (int64_t)r * k;
  float* ss = a.sel_score ? a.sel_score + (int64_t)r * k : nullptr;
  const int nk_c = nk > 0 ? nk : 1;   // slot index clamp for unconditional reads
  // Pool rows of the picks (attention over paged pools): thread s looks up the page of
  // kept block s (nk <= 129 < NT) once, with its load in flight together with the
  // gather's, and the emit below translates from LDS.
  static_assert(CSA2_KEEP_MAX + 1 <= NT, "one kept block per thread");
  int32_t* rows = (a.sel_rows && !all_entries) ? a.sel_rows + (int64_t)r * k : nullptr;
  int32_t kpage = 0;
  if (PAGED && rows && (int)threadIdx.x < nk) {
    const int64_t kb = sh.kl[threadIdx.x];
    const bool ok = kb >= 0 && kb * CSA2_BLOCK < n;
    const int64_t lp = ok ? kb : 0;   // an in-range page-table slot either way
    const int64_t pg = page_of(a.g, row_request(a.g, r), lp) * CSA2_BLOCK;
    kpage = ok ? (int32_t)pg : 0;
  }
  int items;
  if (all_entries) {
    items = (int)(n < kMaxCand ? n : kMaxCand);
    gather(items, [](int) { return true; }, [&](int i, bool ok) { return sc[ok ? i : 0]; }, kbuf, sh);
  } else {
    items = nk * CSA2_BLOCK;
    auto slot_pos = [&](int i) {
      const int sl = min(i / CSA2_BLOCK, nk_c - 1);
      return (int64_t)sh.kl[sl] * CSA2_BLOCK + (i % CSA2_BLOCK);
    };
    auto valid = [&](int i) {
      const int64_t p = slot_pos(i);
      return p >= 0 && p < n;
    };
    gather(items, valid, [&](int i, bool ok) { return sc[ok ? slot_pos(i) : 0]; }, kbuf, sh);
  }
  if (PAGED && rows && (int)threadIdx.x < nk) sh.kpage[threadIdx.x] = kpage;
  __syncthreads();
  // aux of item i: its kept block's first position and, over paged pools, the block's
  // first pool row.
  auto aux = [&](int i) {
    const int sl = min(i / CSA2_BLOCK, nk_c - 1);
    return make_int2(sh.kl[sl] * CSA2_BLOCK, PAGED ? sh.kpage[sl] : 0);
  };
  const int take = sel_top([&](int i) { return kbuf[i]; }, items, valid_count(sh), k, sh, aux,
                           [&](int pos, int i, uint32_t kk, int2 ax) {
    const int j = i % CSA2_BLOCK;
    sel[pos] = all_entries ? i : ax.x + j;
    if (ss) ss[pos] = key_score(kk);
    if (rows) rows[pos] = PAGED ? ax.y + j : (int32_t)(e0 + ax.x + j);
  });
  for (int i = take + threadIdx.x; i < k; i += NT) {
    sel[i] = -1;
    if (ss) ss[i] = 0.f;
    if (rows) rows[i] = -1;
  }
  if (threadIdx.x == 0) a.n_sel[r] = take;
}

// MXFP8 route: workgroup `part` (4 per row) rounds 16 heads of its row's query; wave w
// takes one head, lane l its 8 dims at 32 (l & 15) + 8 (l >> 4), so that the lanes l,
// l ^ 16, l ^ 32 and l ^ 48 hold one 32-dim block between them.
constexpr int kQParts = CSA2_HEADS / (NT / 64);
static_assert(kQParts * (NT / 64) == CSA2_HEADS, "whole heads per workgroup");
__device__ __forceinline__ void round_query_part(const SelectArgs& a, int part) {
  const int r = part / kQParts;
  const int head = (part % kQParts) * (NT / 64) + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t off = ((int64_t)r * CSA2_HEADS + head) * CSA2_D + 32 * (lane & 15) + 8 * (lane >> 4);
  const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(a.q + off);
  *reinterpret_cast<bf16x8_t*>(a.q_mx + off) = mx8_round_block_bf16(x);
}
__host__ __device__ inline int query_parts(const SelectArgs& a) { return a.q_mx ? kQParts * a.g.R : 0; }

template <bool PAGED, bool BIG>
__global__ __launch_bounds__(NT) void k_block_select(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kLdsBlocks];
  float pre[kGB];
  if (!BIG) prefetch_blocks<kGB>(a, blockIdx.x, pre);
  int64_t n, e0;
  const int nb = row_blocks<PAGED>(a, blockIdx.x, n, e0);
  coarse<BIG>(a, blockIdx.x, nb, sh, kbuf, pre);
}

// QR: the launch also carries the MXFP8 query-rounding workgroups (after the rows').
template <bool PAGED, bool QR>
__global__ __launch_bounds__(NT) void k_topk(SelectArgs a, int all_entries) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kMaxCand];
  const int r = blockIdx.x;
  if (QR && r >= a.g.R) {
    round_query_part(a, r - a.g.R);
    return;
  }
  int64_t n, e0;
  row_blocks<PAGED>(a, r, n, e0);
  int nk = 0;
  if (!all_entries) {
    nk = a.n_kept[r];
    nk = nk < 0 ? 0 : (nk > a.kept_ld ? a.kept_ld : nk);
    nk = nk > CSA2_KEEP_MAX + 1 ? CSA2_KEEP_MAX + 1 : nk;
    for (int i = threadIdx.x; i < nk; i += NT) sh.kl[i] = a.kept[(int64_t)r * a.kept_ld + i];
    __syncthreads();
  }
  fine<PAGED>(a, r, n, e0, nk, all_entries != 0, sh, kbuf);
}

// Sliced coarse stage, first level: workgroup (s, r) ranks blocks s*kSelSlice ..
// of row r and writes its n_keep best (ascending) with their scores.
template <bool PAGED>
__global__ __launch_bounds__(NT) void k_block_slices(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kSelSlice];
  const int s = blockIdx.x, r = blockIdx.y;
  int64_t n, e0;
  const int nb = row_blocks<PAGED>(a, r, n, e0);
  const int j0 = s * kSelSlice;
  const int items = min(kSelSlice, nb - j0);
  const int64_t slot = ((int64_t)r * a.n_slices + s) * a.n_keep;
  if (items <= 0) {
    if (threadIdx.x == 0) a.cand_n[(int64_t)r * a.n_slices + s] = 0;
    return;
  }
  const float* bs = a.blk_scores + (int64_t)r * a.blk_ld + j0;
  static_assert(kSelSlice % NT == 0, "slice gather: one batch of whole rows");
  gather<kSelSlice / NT>(items, [](int) { return true; }, [&](int i, bool ok) { return bs[ok ? i : 0]; }, kbuf, sh);
  __syncthreads();
  const int cnt = sel_top([&](int i) { return kbuf[i]; }, items, valid_count(sh), a.n_keep, sh, NoAux(),
                          [&](int pos, int i, uint32_t kk, int) {
    a.cand_blk[slot + pos] = j0 + i;
    a.cand_sc[slot + pos] = key_score(kk);
  });
  if (threadIdx.x == 0) a.cand_n[(int64_t)r * a.n_slices + s] = cnt;
}

// Both stages for one row; the block keys and the candidate keys share one LDS buffer.
// CMODE 0: all blocks ranked from LDS (first batch prefetched); 1: rows may have more
// blocks than LDS holds; 2: the sliced coarse stage's candidates; 3: as 0 for rows of at
// most kSmallRowBlocks block slots, whose whole gather is one round of loads (a batch
// sized for more blocks would issue loads that only repeat the last slot).
template <bool PAGED, int CMODE, bool QR>
__global__ __launch_bounds__(NT) void k_select_fused(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kLdsBlocks];
  constexpr int GBC = CMODE == 3 ? kSmallRowBlocks / NT : kGB;
  const int r = blockIdx.x;
  if (QR && r >= a.g.R) {
    round_query_part(a, r - a.g.R);
    return;
  }
  float pre[GBC];
  if (CMODE == 0 || CMODE == 3) prefetch_blocks(a, r, pre);
  int64_t n, e0;
  const int nb = row_blocks<PAGED>(a, r, n, e0);
  if (CMODE == 2)
    coarse_cand(a, r, nb, sh, kbuf);
  else
    coarse<CMODE == 1, GBC>(a, r, nb, sh, kbuf, pre);
  __syncthreads();
  fine<PAGED>(a, r, n, e0, sh.nk, false, sh, kbuf);
}

}  // namespace

hipError_t launch_block_select(SelectArgs a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  const bool big = a.blk_ld > kLdsBlocks;
  if (a.g.page_table)
    big ? k_block_select<true, true><<<dim3(a.g.R), dim3(NT), 0, st>>>(a)
        : k_block_select<true, false><<<dim3(a.g.R), dim3(NT), 0, st>>>(a);
  else
    big ? k_block_select<false, true><<<dim3(a.g.R), dim3(NT), 0, st>>>(a)
        : k_block_select<false, false><<<dim3(a.g.R), dim3(NT), 0, st>>>(a);
  return hipGetLastError();
}

template <bool QR>
hipError_t topk_launch(SelectArgs a, bool all_entries, hipStream_t st) {
  const dim3 grid(a.g.R + query_parts(a));
  if (a.g.page_table)
    k_topk<true, QR><<<grid, dim3(NT), 0, st>>>(a, all_entries ? 1 : 0);
  else
    k_topk<false, QR><<<grid, dim3(NT), 0, st>>>(a, all_entries ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_topk(SelectArgs a, bool all_entries, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  return a.q_mx ? topk_launch<true>(a, all_entries, st) : topk_launch<false>(a, all_entries, st);
}

#ifndef CSA2_SEL_SMALL_ROWS
#define CSA2_SEL_SMALL_ROWS 1
#endif
template <bool QR>
hipError_t select_fused_launch(SelectArgs a, hipStream_t st) {
  const int mode = a.n_slices > 0 ? 2 : (a.blk_ld > kLdsBlocks ? 1 : (CSA2_SEL_SMALL_ROWS && a.blk_ld <= kSmallRowBlocks ? 3 : 0));
  const dim3 grid(a.g.R + query_parts(a)), block(NT);
  if (a.g.page_table) {
    if (mode == 2) k_select_fused<true, 2, QR><<<grid, block, 0, st>>>(a);
    else if (mode == 1) k_select_fused<true, 1, QR><<<grid, block, 0, st>>>(a);
    else if (mode == 3) k_select_fused<true, 3, QR><<<grid, block, 0, st>>>(a);
    else k_select_fused<true, 0, QR><<<grid, block, 0, st>>>(a);
  } else {
    if (mode == 2) k_select_fused<false, 2, QR><<<grid, block, 0, st>>>(a);
    else if (mode == 1) k_select_fused<false, 1, QR><<<grid, block, 0, st>>>(a);
    else if (mode == 3) k_select_fused<false, 3, QR><<<grid, block, 0, st>>>(a);
    else k_select_fused<false, 0, QR><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_select_fused(SelectArgs a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  return a.q_mx ? select_fused_launch<true>(a, st) : select_fused_launch<false>(a, st);
}

hipError_t launch_block_slices(SelectArgs a, hipStream_t st) {
  if (a.g.R == 0 || a.n_slices == 0) return hipSuccess;
  const dim3 grid(a.n_slices, a.g.R);
  if (a.g.page_table)
    k_block_slices<true><<<grid, dim3(NT), 0, st>>>(a);
  else
    k_block_slices<false><<<grid, dim3(NT), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa2
