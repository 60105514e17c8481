// Coarse block filter and fine top-k on gfx950 (one workgroup per query row).
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Architecture changes and KV
// cache compression": a hierarchical candidate filter leaves the top 512 global
// positions; section "DSpark adaptation and optimization": the chosen candidate blocks
// expand straight into a token mask.  Here: keep the n_keep best 64-entry blocks by
// summary score (ties to the lower block) plus the newest block, expand them into their
// entries, and keep the k best entries (ties to the lower position), ascending.
//
// Selection is exact.  Scores map to order-preserving 32-bit keys, cached in LDS.  The
// keys are normalised by the workgroup minimum, so that an 11-bit radix digit taken
// from the highest bits that actually vary spreads the keys over 2048 LDS histogram
// bins (raw float keys of similar magnitude share their top bits and would pile into a
// few bins).  A descending scan of the histogram gives the bin holding the k-th key;
// when that bin has at most kRankMax members they are ranked directly by (key desc,
// position asc), otherwise the next digit is examined.  The result is the k-th key T and
// the number of keys above it; an ordered compaction then emits every key > T and the
// lowest-position keys == T, in ascending position.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int NT = 512;                                      // threads per workgroup
constexpr int kBins = 2048;                                  // 11-bit digits
constexpr int kDigit = 11;
constexpr int kRankMax = 128;                                // bin members ranked directly
constexpr int kMaxCand = (CSA2_KEEP_MAX + 1) * CSA2_BLOCK;   // 8256 >= CSA2_TOPK_ALL_MAX
static_assert(kMaxCand >= CSA2_TOPK_ALL_MAX, "candidate buffer");

struct SelShared {
  alignas(16) uint32_t hist[2][kBins];  // double-buffered: zero one while filling the other
  uint64_t scan_tmp[NT / kWave + 1];
  uint32_t red[2 * (NT / kWave)];
  uint32_t rkey[kRankMax];
  int32_t ridx[kRankMax];
  int32_t rrank[kRankMax];
  int32_t rgt[kRankMax];
  uint32_t kmin, kmax;
  uint32_t digit;
  uint32_t above;
  uint32_t T;
  int32_t n_gt;
  int32_t m;
  int32_t cnt;
  int32_t flag;
  int32_t slot_off[CSA2_KEEP_MAX + 2];
};

// Per-thread running min/max of keys, reduced over the workgroup into sh.kmin/kmax
// (and the first histogram buffer zeroed) behind one barrier.
struct KeyRange {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  __device__ __forceinline__ void add(uint32_t k) {
    lo = min(lo, k);
    hi = max(hi, k);
  }
  __device__ __forceinline__ void reduce(SelShared& sh) {
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
      sh.red[2 * wave] = lo;
      sh.red[2 * wave + 1] = hi;
    }
    for (int i = threadIdx.x; i < kBins; i += NT) sh.hist[0][i] = 0u;
    __syncthreads();
    uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      a = min(a, sh.red[2 * w]);
      b = max(b, sh.red[2 * w + 1]);
    }
    lo = a;
    hi = b;
  }
};

// k-th largest key (1 <= k <= n): T, and n_gt = number of keys > T.  `rg` holds the
// workgroup-wide key range (after reduce(), which also zeroed hist[0]).
template <class KeyF>
__device__ void radix_kth(KeyF key, int n, int k, const KeyRange& rg, SelShared& sh, uint32_t& T, int& n_gt) {
  const uint32_t lo = rg.lo;
  const uint32_t span = rg.hi - lo;
  int L = span ? 32 - __builtin_clz(span) : 0;       // bits of (key - lo) that vary
  uint32_t prefix = 0u;                               // (key - lo) >> L of the keys still in play
  int rem = k;
  int above_total = 0;
  int buf = 0;
  int m = n;
  while (true) {
    const int shift = L > kDigit ? L - kDigit : 0;
    const uint32_t dmask = (1u << (L - shift)) - 1u;  // L - shift in 0..11
    uint32_t* hist = sh.hist[buf];
    uint32_t* next = sh.hist[buf ^ 1];
    for (int base = 0; base < n; base += NT * 8) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        v[u] = i < n ? key(i) - lo : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        if (i < n && ((uint64_t)v[u] >> L) == prefix) atomicAdd(&hist[(v[u] >> shift) & dmask], 1u);
      }
    }
    for (int i = threadIdx.x; i < kBins; i += NT) next[i] = 0u;
    if (threadIdx.x == 0) sh.cnt = 0;
    __syncthreads();
    // One wave finds the bin holding the rem-th key, scanning bins in descending order:
    // lane l owns bins kBins-1-32l .. kBins-32-32l.
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const uint32_t* hb = hist + kBins - 32 * (lane + 1);   // ascending 32 bins
      uint32_t c[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(hb + 4 * q);
        c[4 * q] = v[0];
        c[4 * q + 1] = v[1];
        c[4 * q + 2] = v[2];
        c[4 * q + 3] = v[3];
      }
      uint32_t tot = 0u;
#pragma unroll
      for (int q = 0; q < 32; ++q) tot += c[q];
      uint32_t before = wave_incl_scan(tot) - tot;
#pragma unroll
      for (int q = 31; q >= 0; --q) {
        if (before < (uint32_t)rem && before + c[q] >= (uint32_t)rem) {
          sh.digit = (uint32_t)(kBins - 32 * (lane + 1) + q);
          sh.above = before;
          sh.m = (int)c[q];
        }
        before += c[q];
      }
    }
    __syncthreads();
    const uint32_t d = sh.digit;
    m = sh.m;
    rem -= (int)sh.above;
    above_total += (int)sh.above;
    prefix = (prefix << (L - shift)) | d;
    L = shift;
    buf ^= 1;
    if (L == 0) {
      // Every key left has the same value: take the first rem of them by position.
      T = lo + prefix;
      n_gt = above_total;
      return;
    }
    if (m <= kRankMax) break;
  }
  // Collect the m members of the bin, then rank them by (key desc, position asc) with
  // P threads per member.
  for (int base = 0; base < n; base += NT * 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      v[u] = i < n ? key(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < n && ((uint64_t)(v[u] - lo) >> L) == prefix) {
        const int slot = atomicAdd(&sh.cnt, 1);
        sh.rkey[slot] = v[u];
        sh.ridx[slot] = i;
      }
    }
  }
  for (int i = threadIdx.x; i < kRankMax; i += NT) {
    sh.rrank[i] = 0;
    sh.rgt[i] = 0;
  }
  __syncthreads();
  {
    const int P = NT / m;                         // m <= kRankMax <= NT/4
    const int i = threadIdx.x / P, part = threadIdx.x % P;
    if (i < m) {
      const uint32_t ki = sh.rkey[i];
      const int ii = sh.ridx[i];
      const int j0 = part * m / P, j1 = (part + 1) * m / P;
      int rank = 0, gt = 0;
      for (int j = j0; j < j1; j += 8) {
        uint32_t kj[8];
        int ij[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          kj[u] = j + u < j1 ? sh.rkey[j + u] : 0u;
          ij[u] = j + u < j1 ? sh.ridx[j + u] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j + u < j1) {
            gt += kj[u] > ki;
            rank += (kj[u] > ki) || (kj[u] == ki && ij[u] < ii);
          }
        }
      }
      if (rank) atomicAdd(&sh.rrank[i], rank);
      if (gt) atomicAdd(&sh.rgt[i], gt);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += NT) {
    if (sh.rrank[i] == rem - 1) {
      sh.T = sh.rkey[i];
      sh.n_gt = above_total + sh.rgt[i];
    }
  }
  __syncthreads();
  T = sh.T;
  n_gt = sh.n_gt;
}

// Emit (output position, candidate index) for every key > T and for the first need_eq
// keys == T, in ascending candidate index.  All threads must call it.
template <class KeyF, class EmitF>
__device__ void ordered_emit(KeyF key, int n, uint32_t T, int need_eq, SelShared& sh, EmitF emit) {
  const int per = (n + NT - 1) / NT;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  uint32_t gt = 0u, eq = 0u;
  for (int b = lo; b < hi; b += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = b + u < hi ? key(b + u) : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b + u < hi) {
        gt += v[u] > T;
        eq += v[u] == T;
      }
    }
  }
  uint64_t tot;
  const uint64_t before = block_excl_scan<NT>(((uint64_t)gt << 32) | eq, sh.scan_tmp, tot);
  uint32_t gtb = (uint32_t)(before >> 32), eqb = (uint32_t)before;
  for (int b = lo; b < hi; b += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = b + u < hi ? key(b + u) : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b + u < hi) {
        if (v[u] > T) {
          emit((int)(gtb + min(eqb, (uint32_t)need_eq)), b + u);
          ++gtb;
        } else if (v[u] == T) {
          if (eqb < (uint32_t)need_eq) emit((int)(gtb + eqb), b + u);
          ++eqb;
        }
      }
    }
  }
}

// Gather n selection keys into LDS with 16 independent loads in flight per thread.
// load(i) returns the i-th score.
constexpr int kGather = 16;
template <class LoadF>
__device__ __forceinline__ void gather_keys(int n, LoadF load, uint32_t* kbuf, KeyRange& rg) {
  for (int base = 0; base < n; base += NT * kGather) {
    float v[kGather];
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      v[u] = i < n ? load(i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < n) {
        const uint32_t kk = score_key(v[u]);
        kbuf[i] = kk;
        rg.add(kk);
      }
    }
  }
}

// Coarse stage for row r over nb block scores; out(pos, block) receives the kept blocks
// in ascending order.  Returns the count (uniform across the workgroup).  kbuf (LDS,
// kcap entries) caches the keys when they fit.
template <class OutF>
__device__ int block_select(const SelectArgs& a, int r, int nb, SelShared& sh, uint32_t* kbuf, int kcap,
                            OutF out) {
  if (nb <= 0) return 0;
  if (nb <= a.n_keep) {
    for (int i = threadIdx.x; i < nb; i += NT) out(i, i);
    return nb;
  }
  const float* bs = a.blk_scores + (int64_t)r * a.blk_ld;
  uint32_t T;
  int n_gt;
  if (threadIdx.x == 0) sh.flag = 0;
  auto emit = [&](int pos, int i) {
    out(pos, i);
    if (i == nb - 1) sh.flag = 1;
  };
  KeyRange rg;
  if (nb <= kcap) {
    gather_keys(nb, [&](int i) { return bs[i]; }, kbuf, rg);
    rg.reduce(sh);
    auto key = [&](int i) { return kbuf[i]; };
    radix_kth(key, nb, a.n_keep, rg, sh, T, n_gt);
    ordered_emit(key, nb, T, a.n_keep - n_gt, sh, emit);
  } else {
    auto key = [&](int i) { return score_key(bs[i]); };
    for (int i = threadIdx.x; i < nb; i += NT) rg.add(key(i));
    rg.reduce(sh);
    radix_kth(key, nb, a.n_keep, rg, sh, T, n_gt);
    ordered_emit(key, nb, T, a.n_keep - n_gt, sh, emit);
  }
  __syncthreads();
  int cnt = a.n_keep;
  if (a.keep_newest && sh.flag == 0) {
    if (threadIdx.x == 0) out(cnt, nb - 1);
    ++cnt;
  }
  return cnt;
}

// Fine stage for row r: candidates are the entries of the kept blocks (kl, in LDS, nk
// of them) or all n entries; results go to sel/n_sel/sel_score.  With `ordered` the
// kept list is known to be ascending, in range and partial only in its last block
// (as the coarse stage produces it), so candidate c is entry 64*kl[c/64] + c%64.
__device__ void fine_topk(const SelectArgs& a, int r, int64_t n, const int32_t* kl, int nk, bool all_entries,
                          bool ordered, SelShared& sh, uint32_t* ckey, int32_t* cpos) {
  const float* sc = a.scores + (int64_t)r * a.ld;
  int ncand;
  KeyRange rg;
  if (all_entries) {
    ncand = (int)(n < kMaxCand ? n : kMaxCand);
    gather_keys(ncand, [&](int i) { return sc[i]; }, ckey, rg);
    for (int i = threadIdx.x; i < ncand; i += NT) cpos[i] = i;
  } else {
    if (ordered) {
      if (threadIdx.x <= nk) {
        const int s = threadIdx.x;
        sh.slot_off[s] = s * CSA2_BLOCK;
        if (s == nk && nk > 0) {
          const int64_t left = n - (int64_t)kl[nk - 1] * CSA2_BLOCK;
          sh.slot_off[s] = (nk - 1) * CSA2_BLOCK + (int)(left < CSA2_BLOCK ? left : CSA2_BLOCK);
        }
      }
    } else if (threadIdx.x < kWave) {
      // Slot offsets: a kept block contributes min(64, n - 64*block) entries.
      const int lane = threadIdx.x;
      int carry = 0;
      for (int s0 = 0; s0 < nk; s0 += kWave) {
        const int s = s0 + lane;
        int cnt = 0;
        if (s < nk) {
          const int64_t kb = kl[s];
          if (kb >= 0 && kb * CSA2_BLOCK < n) {
            const int64_t left = n - kb * CSA2_BLOCK;
            cnt = (int)(left < CSA2_BLOCK ? left : CSA2_BLOCK);
          }
        }
        const int incl = wave_incl_scan(cnt);
        if (s < nk) sh.slot_off[s] = carry + incl - cnt;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) sh.slot_off[nk] = carry;
    }
    __syncthreads();
    ncand = sh.slot_off[nk];
    const int total = nk * CSA2_BLOCK;
    for (int base = 0; base < total; base += NT * kGather) {
      float v[kGather];
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        const int s = i / CSA2_BLOCK, j = i % CSA2_BLOCK;
        v[u] = (i < total && sh.slot_off[s] + j < sh.slot_off[s + 1]) ? sc[(int64_t)kl[s] * CSA2_BLOCK + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        const int s = i / CSA2_BLOCK, j = i % CSA2_BLOCK;
        if (i < total) {
          const int c = sh.slot_off[s] + j;
          if (c < sh.slot_off[s + 1]) {
            cpos[c] = (int32_t)((int64_t)kl[s] * CSA2_BLOCK + j);
            const uint32_t kk = score_key(v[u]);
            ckey[c] = kk;
            rg.add(kk);
          }
        }
      }
    }
  }
  rg.reduce(sh);
  const int k = a.k;
  int32_t* sel = a.sel + (int64_t)r * k;
  float* ss = a.sel_score ? a.sel_score + (int64_t)r * k : nullptr;
  int nsel;
  if (ncand <= k) {
    for (int i = threadIdx.x; i < ncand; i += NT) {
      sel[i] = cpos[i];
      if (ss) ss[i] = sc[cpos[i]];
    }
    nsel = ncand;
  } else {
    auto key = [&](int i) { return ckey[i]; };
    uint32_t T;
    int n_gt;
    radix_kth(key, ncand, k, rg, sh, T, n_gt);
    ordered_emit(key, ncand, T, k - n_gt, sh, [&](int pos, int i) {
      sel[pos] = cpos[i];
      if (ss) ss[pos] = sc[cpos[i]];
    });
    nsel = k;
  }
  for (int i = nsel + threadIdx.x; i < k; i += NT) {
    sel[i] = -1;
    if (ss) ss[i] = 0.f;
  }
  if (threadIdx.x == 0) a.n_sel[r] = nsel;
}

__device__ __forceinline__ int row_blocks(const SelectArgs& a, int r, int64_t& n) {
  const int b = row_request(a.g, r);
  int64_t e0, bl0, nb;
  req_entries(a.g, b, e0, n);
  req_blocks(a.g, b, n, bl0, nb);
  return (int)nb;
}

constexpr int kBlockCap = 16384;   // block keys cached in LDS (N up to 1M entries)

__global__ __launch_bounds__(NT) void k_block_select(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kBlockCap];
  const int r = blockIdx.x;
  int64_t n;
  const int nb = row_blocks(a, r, n);
  int32_t* kout = a.kept + (int64_t)r * a.kept_ld;
  const int cnt = block_select(a, r, nb, sh, kbuf, kBlockCap, [&](int pos, int blk) { kout[pos] = blk; });
  for (int i = cnt + threadIdx.x; i < a.kept_ld; i += NT) kout[i] = -1;
  if (threadIdx.x == 0) a.n_kept[r] = cnt;
}

__global__ __launch_bounds__(NT) void k_topk(SelectArgs a, int all_entries) {
  __shared__ SelShared sh;
  __shared__ uint32_t ckey[kMaxCand];
  __shared__ int32_t cpos[kMaxCand];
  __shared__ int32_t kl[CSA2_KEEP_MAX + 1];
  const int r = blockIdx.x;
  int64_t n;
  row_blocks(a, r, n);
  int nk = 0;
  if (!all_entries) {
    nk = a.n_kept[r];
    nk = nk < 0 ? 0 : (nk > a.kept_ld ? a.kept_ld : nk);
    nk = nk > CSA2_KEEP_MAX + 1 ? CSA2_KEEP_MAX + 1 : nk;
    for (int i = threadIdx.x; i < nk; i += NT) kl[i] = a.kept[(int64_t)r * a.kept_ld + i];
    __syncthreads();
  }
  fine_topk(a, r, n, kl, nk, all_entries != 0, false, sh, ckey, cpos);
}

// Block keys and candidate keys share one LDS region: the block stage is finished
// (barrier) before the candidates are gathered.
__global__ __launch_bounds__(NT) void k_select_fused(SelectArgs a) {
  __shared__ SelShared sh;
  __shared__ uint32_t kbuf[kBlockCap];
  __shared__ int32_t cpos[kMaxCand];
  __shared__ int32_t kl[CSA2_KEEP_MAX + 1];
  static_assert(kBlockCap >= kMaxCand, "shared key buffer");
  const int r = blockIdx.x;
  int64_t n;
  const int nb = row_blocks(a, r, n);
  int32_t* kout = a.kept ? a.kept + (int64_t)r * a.kept_ld : nullptr;
  const int cnt = block_select(a, r, nb, sh, kbuf, kBlockCap, [&](int pos, int blk) {
    kl[pos] = blk;
    if (kout) kout[pos] = blk;
  });
  if (kout) {
    for (int i = cnt + threadIdx.x; i < a.kept_ld; i += NT) kout[i] = -1;
    if (threadIdx.x == 0) a.n_kept[r] = cnt;
  }
  __syncthreads();
  fine_topk(a, r, n, kl, cnt, false, true, sh, kbuf, cpos);
}

}  // namespace

hipError_t launch_block_select(SelectArgs a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  k_block_select<<<dim3(a.g.R), dim3(NT), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk(SelectArgs a, bool all_entries, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  k_topk<<<dim3(a.g.R), dim3(NT), 0, st>>>(a, all_entries ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_select_fused(SelectArgs a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  k_select_fused<<<dim3(a.g.R), dim3(NT), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa2
