// Coarse block filter and fine top-k on gfx950 (one workgroup per query row).
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Architecture changes and KV
// cache compression": a hierarchical candidate filter leaves the top 512 global
// positions; section "DSpark adaptation and optimization": the chosen candidate blocks
// expand straight into a token mask.  Here: keep the n_keep best 64-entry blocks by
// summary score (ties to the lower block) plus the newest block, expand them into their
// entries, and keep the k best entries (ties to the lower position), ascending.
//
// Selection is exact: scores map to order-preserving 32-bit keys; a 4-pass 8-bit radix
// descent over LDS histograms finds the k-th largest key T and how many keys exceed it;
// an ordered compaction (per-thread contiguous segments + a workgroup prefix sum of
// (greater, equal) counts) then emits every key > T and the lowest-position keys == T,
// in ascending position.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int NT = 256;
constexpr int kMaxCand = (CSA2_KEEP_MAX + 1) * CSA2_BLOCK;   // 8256 >= CSA2_TOPK_ALL_MAX
static_assert(kMaxCand >= CSA2_TOPK_ALL_MAX, "candidate buffer");

struct SelShared {
  uint32_t hist[256];
  uint64_t scan_tmp[NT / kWave + 1];
  uint32_t digit;
  uint32_t gt_count;
  int32_t flag;
  int32_t count;
  int32_t slot_off[CSA2_KEEP_MAX + 2];
};

// k-th largest key (1 <= k <= n): T, and n_gt = number of keys > T.
template <class KeyF>
__device__ void radix_kth(KeyF key, int n, int k, SelShared& sh, uint32_t& T, int& n_gt) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t kk = key(i);
      if ((kk & mask) == prefix) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      uint32_t c[4], s = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        c[t] = sh.hist[255 - 4 * lane - t];
        s += c[t];
      }
      uint32_t before = wave_incl_scan(s) - s;   // keys with a larger digit (digits descend with lane)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (before < (uint32_t)rem && before + c[t] >= (uint32_t)rem) {
          sh.digit = 255u - 4u * lane - t;
          sh.gt_count = before;
        }
        before += c[t];
      }
    }
    __syncthreads();
    rem -= (int)sh.gt_count;
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
  }
  T = prefix;
  n_gt = k - rem;
}

// Emit (output position, candidate index) for every key > T and for the first need_eq
// keys == T, in ascending candidate index.  All threads must call it.
template <class KeyF, class EmitF>
__device__ void ordered_emit(KeyF key, int n, uint32_t T, int need_eq, SelShared& sh, EmitF emit) {
  const int per = (n + NT - 1) / NT;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  uint32_t gt = 0u, eq = 0u;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key(i);
    gt += kk > T;
    eq += kk == T;
  }
  uint64_t tot;
  const uint64_t before = block_excl_scan<NT>(((uint64_t)gt << 32) | eq, sh.scan_tmp, tot);
  uint32_t gtb = (uint32_t)(before >> 32), eqb = (uint32_t)before;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key(i);
    if (kk > T) {
      emit((int)(gtb + min(eqb, (uint32_t)need_eq)), i);
      ++gtb;
    } else if (kk == T) {
      if (eqb < (uint32_t)need_eq) emit((int)(gtb + eqb), i);
      ++eqb;
    }
  }
}

// Gather n selection keys into LDS with 8 independent loads in flight per thread.
// load(i) returns the i-th score.
template <class LoadF>
__device__ __forceinline__ void gather_keys(int n, LoadF load, uint32_t* kbuf) {
  for (int base = 0; base < n; base += NT * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      v[u] = i < n ? load(i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < n) kbuf[i] = score_key(v[u]);
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
  if (nb <= kcap) {
    gather_keys(nb, [&](int i) { return bs[i]; }, kbuf);
    __syncthreads();
    auto key = [&](int i) { return kbuf[i]; };
    radix_kth(key, nb, a.n_keep, sh, T, n_gt);
    ordered_emit(key, nb, T, a.n_keep - n_gt, sh, emit);
  } else {
    auto key = [&](int i) { return score_key(bs[i]); };
    radix_kth(key, nb, a.n_keep, sh, T, n_gt);
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
// of them) or all n entries; results go to sel/n_sel/sel_score.
__device__ void fine_topk(const SelectArgs& a, int r, int64_t n, const int32_t* kl, int nk, bool all_entries,
                          SelShared& sh, uint32_t* ckey, int32_t* cpos) {
  const float* sc = a.scores + (int64_t)r * a.ld;
  int ncand;
  if (all_entries) {
    ncand = (int)(n < kMaxCand ? n : kMaxCand);
    gather_keys(ncand, [&](int i) { return sc[i]; }, ckey);
    for (int i = threadIdx.x; i < ncand; i += NT) cpos[i] = i;
  } else {
    // Slot offsets: a kept block contributes min(64, n - 64*block) entries.
    if (threadIdx.x < kWave) {
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
    for (int base = 0; base < total; base += NT * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        const int s = i / CSA2_BLOCK, j = i % CSA2_BLOCK;
        v[u] = (i < total && sh.slot_off[s] + j < sh.slot_off[s + 1]) ? sc[(int64_t)kl[s] * CSA2_BLOCK + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + (int)threadIdx.x;
        const int s = i / CSA2_BLOCK, j = i % CSA2_BLOCK;
        if (i < total) {
          const int c = sh.slot_off[s] + j;
          if (c < sh.slot_off[s + 1]) {
            cpos[c] = (int32_t)((int64_t)kl[s] * CSA2_BLOCK + j);
            ckey[c] = score_key(v[u]);
          }
        }
      }
    }
  }
  __syncthreads();
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
    radix_kth(key, ncand, k, sh, T, n_gt);
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
  fine_topk(a, r, n, kl, nk, all_entries != 0, sh, ckey, cpos);
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
  fine_topk(a, r, n, kl, cnt, false, sh, kbuf, cpos);
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
