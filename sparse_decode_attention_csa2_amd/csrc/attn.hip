// Joint-softmax latent attention over the selected FP4 entries and the FP8 window.
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Architecture changes and KV
// cache compression": only the top 512 global positions (FP4, 288 B per entry) take
// part in attention; clawpit.io vLLM article, section "SWA bounded replay": the
// sliding-window cache is FP8 over the 128 most recent positions.  Each head h of the
// row computes one softmax over both key sets (K = V = the 512-dim latent):
//   z_i = sm_scale * q_h . x_i,  out_h = sum_i softmax(z)_i x_i,  lse_h = log sum_i e^z_i.
//
// Kernel structure.  A workgroup of 8 waves takes a range of 64-key tiles of one row.
// Per tile, each thread owns two keys x 32 dims: it loads their records during the
// previous tile (the positions first, then the records, all addresses clamped so no
// load waits on a branch) and dequantises them exactly to bf16 into one key-major LDS
// copy Kl[key][dim].  Wave (hg, dh) owns heads 16hg..16hg+15 and latent dims
// 256dh..256dh+255: it contracts its half of the dims for S^T = K Q^T (query fragments
// stay in registers for all tiles) and the two halves meet through LDS; O^T = V^T P^T
// reads its V^T operand from the same key-major copy with transposing LDS loads.
// Window tokens enter as their exact E4M3 values; their fp32 scale multiplies the
// logits and the probabilities instead.  Both products run on bf16 16x16x32 MFMAs with
// fp32 accumulation and an online softmax between them; probabilities enter PV as
// bf16 hi + lo parts.  Workgroups of one row write (unnormalised O, running max,
// running sum) partials that a second kernel merges by log-sum-exp; with a single
// split the kernel writes the result directly.  Launches with few rows spread each
// split's four head groups over four workgroups (head-split, below).
#include <math.h>

#include "csa2_internal.h"

namespace csa2 {
namespace {

#ifndef CSA2_ATTN_KLS
#define CSA2_ATTN_KLS 528
#endif
constexpr int KLS = CSA2_ATTN_KLS;   // Kl row stride in bf16 (512 + 16: rows 32 B apart modulo 256 B)
static_assert(KLS >= 512 && KLS % 8 == 0, "Kl rows hold 512 bf16, 16-byte aligned");

// Column of dim d (a multiple of 4) in row `row` of Kl: each 32-dim (64-B) chunk holds
// its four 16-B pieces in the order piece ^ ((row >> 2) & 3).  The dequantising threads
// write 16-B pieces of rows 2 apart at the same chunk, which without the swizzle fall
// into the same banks (measured 23.6 conflict cycles per 16-B store); with it every
// 16-B store, the QK^T reads (rows 16b + lane % 16) and the transposing PV reads (rows
// 4g + ...) are conflict-free.
__device__ __forceinline__ int kl_col(int row, int d) { return d ^ (((row >> 2) & 3) << 3); }
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplitKeys = CSA2_K_MAX + CSA2_SWA_MAX;   // positions of one split staged in LDS
constexpr int kAttnTileKeys = 64;

#ifndef CSA2_ATTN_TARGET_WGS
#define CSA2_ATTN_TARGET_WGS 256
#endif

struct RowKeys {
  int64_t e0, n;     // pool row of position 0 and the positions the row sees (pool rows
                     // themselves, 0 .. total_entries-1, when sel holds pool rows)
  int n_main;        // selected main entries (slots)
  int64_t s0;        // first window token
  int n_swa;
};

// ROWS: the selection holds pool rows (a.sel_rows != 0), so the request's offsets are
// not needed and not loaded.
template <bool ROWS = false>
__device__ __forceinline__ RowKeys row_keys(const AttnArgs& a, int r) {
  RowKeys k;
  if (ROWS) {
    k.e0 = 0;
    k.n = a.g.total_entries;
  } else {
    const int64_t vis = row_len_raw(a.g, r);
    const int b = row_request(a.g, r);
    int64_t e0, n;
    req_entries(a.g, b, e0, n);
    n = row_visible(a.g, vis, n);
    k.e0 = a.sel_rows ? 0 : e0;
    k.n = a.sel_rows ? a.g.total_entries : n;
  }
  // All loads first, then selects (a branch here would let the compiler sink a load
  // into it, behind the others).
  const int ns = a.n_sel[r];
  const int64_t s0 = a.g.row_swa_start[r];
  int len = a.g.row_swa_len[r];
  k.n_main = ns < 0 ? 0 : (ns > a.sel_ld ? a.sel_ld : ns);
  len = len < 0 ? 0 : (len > CSA2_SWA_MAX ? CSA2_SWA_MAX : len);
  const bool bad = s0 < 0 || s0 >= a.g.swa_tokens;
  const int64_t room = a.g.swa_tokens - s0;
  k.s0 = bad ? 0 : s0;
  k.n_swa = bad ? 0 : (int)(len < room ? len : room);
  return k;
}

// One key's raw record slice as loaded by its thread (dims 32ch .. 32ch+31).
struct KeyRegs {
  u32x4_t c0, c1;     // main: c0 = 16 code bytes; window: c0, c1 = 32 E4M3 bytes
  uint32_t sc;        // as loaded: main: the 4 E8M0 bytes of blocks 4(ch/2) .. 4(ch/2)+3;
                      // window: fp32 scale bits.  Nothing reads it before convert_key, so
                      // the loads stay in flight while the previous tile computes.
  int kind;           // 0 empty, 1 main entry, 2 window token
};

// E8M0 scales of a main key's blocks 2ch and 2ch+1 (from the loaded scale word).
__device__ __forceinline__ uint32_t main_scales(const KeyRegs& k, int ch) { return k.sc >> (16 * (ch & 1)); }

// Exact bf16 values of a key's 32 dims (dims 32ch .. 32ch+31) as 16 packed words
// (element 2q in the low half).
__device__ __forceinline__ void convert_key(const KeyRegs& k, int ch, uint32_t (&w)[16]) {
  if (k.kind == 1) {
    const uint32_t s2 = main_scales(k, ch);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4_t x = __builtin_bit_cast(u32x4_t, fp4x8_to_bf16(k.c0[d], e8m0_operand((s2 >> (8 * (d >> 1))) & 255u)));
      w[4 * d] = x[0];
      w[4 * d + 1] = x[1];
      w[4 * d + 2] = x[2];
      w[4 * d + 3] = x[3];
    }
  } else if (k.kind == 2) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t c = d < 4 ? k.c0[d] : k.c1[d - 4];
      const u32x2_t x = __builtin_bit_cast(u32x2_t, e4m3x4_to_bf16(c));
      w[2 * d] = x[0];
      w[2 * d + 1] = x[1];
    }
  } else {
#pragma unroll
    for (int d = 0; d < 16; ++d) w[d] = 0u;
  }
}

// 16 bf16 of the key-major tile read transposed: with lane (g, i) (i = lane % 16)
// pointing at 4 consecutive elements, lane (g, j) receives element j % 4 of lanes
// (g, 4k + j / 4), k = 0..3 (ds_read_b64_tr_b16).
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(__attribute__((address_space(3))) uint16_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// One workgroup of 8 waves per split: wave (hg, dh) = (wave % 4, wave / 4) owns heads
// 16hg .. 16hg+15 and latent dims 256dh .. 256dh+255 of the output.  Per 64-key tile:
// the 512 threads dequantise the tile into the key-major LDS copy (each thread 2 keys x
// 32 dims; the records of the next tile are loaded before the current tile computes);
// each wave contracts its half of the dims for S^T = K Q^T and the two halves meet
// through LDS; the online softmax runs identically in both waves of a head group; PV
// reads its A operand (V^T) from the same key-major copy with transposing LDS loads.
// MX: the MXFP8 route (Q and P rounded to MXFP8 before their products); otherwise Q as
// given and P as exact-to-2^-17 bf16 hi + lo parts.
// HALF: the plan ends some splits with a half-full tile (split_keys not a multiple of
// the tile), so tiles check for it; other plans get no trace of that path.
// HS (launches with few workgroups, such as one row's 10 splits): a split's heads are
// spread over four workgroups, one per head group (blockIdx.x = 4 split + hg).  Wave
// (kb, dh) = (wave % 4, wave / 4) then contracts key block kb over dims 256dh.. for
// S^T, every wave reads the whole 64-key S^T of the head group back from LDS, and wave
// w owns dims 64w .. 64w+63 of O.  Every product and sum is the one the full workgroup
// makes, in the same order, so the results are identical; each workgroup has a quarter
// of the MFMA and LDS work per tile.
template <bool MX, bool ROWS, bool HALF, bool HS = false>
__global__ __launch_bounds__(512) void k_attn(AttnArgs a) {
  constexpr int TK = kAttnTileKeys;   // 64
  constexpr int KB = TK / 32;         // 32-key groups
  constexpr int NB = TK / 16;         // 16-key blocks
  __shared__ __align__(16) uint16_t Kl[TK * KLS];
  __shared__ __align__(16) float Sx[8][4 * NB][64];
  __shared__ float ksc[TK];
  __shared__ float kbias[TK];   // 0 for a key of the split, -inf for an empty slot

  static_assert(!(HS && HALF), "head-split launches plan whole tiles");
  constexpr int NO = HS ? 4 : 16;     // 16-dim O tiles per wave
  const int r = blockIdx.y, split = HS ? (int)(blockIdx.x >> 2) : (int)blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), dh = wave >> 2;
  const int hg = HS ? (int)(blockIdx.x & 3) : (wave & 3);
  const int h = hg * 16 + ln;
  const int k_begin = split * a.split_keys;

  // Dequant role: keys 32u + 2kp + e (e < 2) of a tile, dims 32ch .. 32ch+31.  A tile's
  // keys are fetched in two steps that every thread takes without branching (so no load
  // waits on another path's registers): the selected positions (sel_pos), then the
  // records (load_keys), each address clamped to valid memory and the key's kind
  // deciding afterwards what the loaded bytes mean.  Positions are read clamped to the
  // row's sel_ld slots rather than its count, so the first tile's positions load
  // alongside the row's counts.
  const int kp = tid & 15, ch = (tid >> 4) & 15, u = tid >> 8;
  const int32_t* sel_row = a.sel + (int64_t)r * a.sel_ld;
  int32_t pos_raw[2];
  auto sel_pos = [&](int kt) {
#pragma unroll
    for (int e = 0; e < 2; ++e) pos_raw[e] = sel_row[min(kt + 32 * u + 2 * kp + e, a.sel_ld - 1)];
  };
  sel_pos(k_begin);
  // Query fragments of this wave's dims (B operand of S^T = K Q^T): lane holds
  // q[h][256dh + 32st + 8g + j].  Loaded before anything that depends on the row.
  bf16x8_t qb[8];
  {
    const uint16_t* qp = a.q + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + 256 * dh + 8 * g;
#pragma unroll
    for (int st = 0; st < 8; ++st) qb[st] = as_bf16x8(load16(qp + 32 * st));
  }
  // Keep these loads ahead of the row checks below (the compiler would otherwise sink
  // them past the early exits, behind the counts they do not depend on).
  asm volatile("" ::: "memory");
  const RowKeys rk = row_keys<ROWS>(a, r);
  const int n_keys = rk.n_main + rk.n_swa;

  if (n_keys == 0) {
    if (blockIdx.x == 0) {
      for (int i = tid; i < CSA2_HEADS * CSA2_D; i += 512) a.out[(int64_t)r * CSA2_HEADS * CSA2_D + i] = 0.f;
      if (tid < CSA2_HEADS) a.lse[(int64_t)r * CSA2_HEADS + tid] = -INFINITY;
    }
    return;
  }
  if (k_begin >= n_keys) return;
  const int k_end = min(n_keys, k_begin + a.split_keys);

  f32x4_t o[NO];
#pragma unroll
  for (int t = 0; t < NO; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint8_t* safe = reinterpret_cast<const uint8_t*>(a.q);   // any readable 16-B aligned bytes
  KeyRegs kr[2];
  auto load_keys = [&](int kt) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = kt + 32 * u + 2 * kp + e;
      const bool live = i < k_end;
      const int64_t pos = pos_raw[e];
      const bool is_main = live && i < rk.n_main && pos >= 0 && pos < rk.n;
      const bool is_win = live && i >= rk.n_main;
      const int64_t tok = rk.s0 + (is_win ? i - rk.n_main : 0);
      const uint8_t* mrec = a.main_kv + (rk.e0 + (is_main ? pos : 0)) * CSA2_MAIN_BYTES;
      const uint8_t* wrec = a.swa + tok * CSA2_D + 32 * ch;
      const uint8_t* pa = is_main ? mrec + 16 * ch : (is_win ? wrec : safe);
      const uint8_t* pb = is_win ? wrec + 16 : pa;
      const uint8_t* ps = is_main ? mrec + 256 + 4 * (ch >> 1)
                                  : (is_win ? reinterpret_cast<const uint8_t*>(a.swa_scale + tok) : safe);
      KeyRegs k;
      k.c0 = load16(pa);
      k.c1 = load16(pb);
      k.sc = *reinterpret_cast<const uint32_t*>(ps);
      k.kind = is_main ? 1 : (is_win ? 2 : 0);
      kr[e] = k;
    }
  };
  load_keys(k_begin);
  if constexpr (MX) {
    // MXFP8 route, unless the selection launch before this one rounded the query
    // already: block st of 32 dims = this lane's 8 values and those of lanes xor 16 and
    // xor 32 (rounded while the first tile's records are in flight).
    if (!a.q_rounded) {
#pragma unroll
      for (int st = 0; st < 8; ++st) qb[st] = mx8_round_block_bf16(qb[st]);
    }
  }

  // Kl offsets with the swizzle (kl_col) folded in.  QK^T: lane (g, ln) reads dims 8g..
  // of a 32-dim chunk of row 16b + ln, whose swizzle term is (ln >> 2) & 3 for every b.
  const int qk_g = kl_col(ln, 8 * g);
  // Transposed reads: lane (g, i = 4k + q) points at key 4g + k of a 16-key half and dims
  // 4q .. 4q+3 of a 16-dim tile; those rows' swizzle term is g, which moves the lane's
  // 8 bytes within the tile's 64-B chunk differently for even and odd 16-dim tiles.
  const int tr_row = (4 * g + (ln >> 2)) * KLS + (HS ? 64 * wave : 256 * dh);
  const int tr_off[2] = {tr_row + kl_col(4 * g, 4 * (ln & 3)), tr_row + kl_col(4 * g, 16 + 4 * (ln & 3)) - 16};

  for (int kt = k_begin; kt < k_end; kt += TK) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t w[16];
      convert_key(kr[e], ch, w);
      const int row = 32 * u + 2 * kp + e;
      uint16_t* k0 = Kl + row * KLS;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4_t*>(k0 + kl_col(row, 32 * ch + 8 * q)) =
            u32x4_t{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
      if (ch == 0) {
        const int key = 32 * u + 2 * kp + e;
        ksc[key] = kr[e].kind == 2 ? __uint_as_float(kr[e].sc) : (kr[e].kind == 1 ? 1.f : 0.f);
        kbias[key] = kr[e].kind != 0 ? 0.f : -INFINITY;
      }
    }
    __syncthreads();
    // The next tile's positions now, its records after the softmax.
    const bool more = kt + TK < k_end;
    if (more) sel_pos(kt + TK);

    // Partial S^T over this wave's 256 dims: 16-key blocks b, 8 K steps of 32 dims.  A
    // tile holding at most 32 keys (the end of a split) skips its empty second half here
    // and in PV: those keys are empty (zero records, masked logits), so the skipped
    // products are exact zeros.
    const bool half = HALF && kt + TK / 2 >= k_end;   // uniform
    f32x4_t s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (HS) {
      // This wave's key block over its 256 dims; all eight partial blocks meet in LDS.
      const int kb = wave & 3;
      f32x4_t sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8_t ak =
            as_bf16x8(*reinterpret_cast<const u32x4_t*>(Kl + (16 * kb + ln) * KLS + 256 * dh + 32 * st + qk_g));
        sk = mfma16x16x32(ak, qb[st], sk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Sx[wave][i][lane] = sk[i];
    } else if (half) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
#pragma unroll
        for (int b = 0; b < NB / 2; ++b) {
          const bf16x8_t ak =
              as_bf16x8(*reinterpret_cast<const u32x4_t*>(Kl + (16 * b + ln) * KLS + 256 * dh + 32 * st + qk_g));
          s[b] = mfma16x16x32(ak, qb[st], s[b]);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t ak =
              as_bf16x8(*reinterpret_cast<const u32x4_t*>(Kl + (16 * b + ln) * KLS + 256 * dh + 32 * st + qk_g));
          s[b] = mfma16x16x32(ak, qb[st], s[b]);
        }
      }
    }
    // The two dim halves of a head group meet in LDS.
    if constexpr (HS) {
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[b][i] = Sx[b][i][lane] + Sx[b + 4][i][lane];
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sx[wave][4 * b + i][lane] = s[b][i];
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[b][i] += Sx[wave ^ 4][4 * b + i][lane];
    }

    // Lane holds keys 16b + 4g + i for head h (the same values in both waves of the
    // head group: a + b == b + a).
    float z[4 * NB], sc[4 * NB];
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * b + 4 * g + i;
        sc[4 * b + i] = ksc[key];
        // An fma with a zero addend rounds like the product alone; an empty slot (zero
        // record and scale) gets -inf.
        z[4 * b + i] = fmaf(s[b][i] * sc[4 * b + i], a.sm_scale_log2, kbias[key]);
        mx = fmaxf(mx, z[4 * b + i]);
      }
    }
    mx = xor32_max(xor16_max(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    // Probabilities enter PV as bf16 hi + lo parts: one bf16 would round each weight
    // by up to 2^-9 relative, the whole error budget of the output.  MX route: each
    // 32-key group's weights (p times the key's window scale, the factor on its stored
    // codes) are rounded to MXFP8, which is exact in one bf16; the normaliser keeps the
    // unrounded p.
    float psum = 0.f;
    bf16x8_t pb_hi[KB], pb_lo[KB];
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int zi = 8 * c + j;   // blocks 2c (j < 4) and 2c+1 (j >= 4)
        const float p = exp2f(z[zi] - m_use);
        psum += p;
        pv[j] = p * sc[zi];
      }
      if constexpr (MX)
        pb_hi[c] = mx8_round_block_bf16x8(pv);
      else
        split_bf16x8(pv, pb_hi[c], pb_lo[c]);
    }
    l_run = l_run * alpha + psum;
    // Rescale the accumulators only when a head's running maximum moved.
    if (__ballot(m_new != m_run && m_run != -INFINITY)) {
#pragma unroll
      for (int t = 0; t < NO; ++t) o[t] *= alpha;
    }
    m_run = m_new;
    if (more) load_keys(kt + TK);

    // O^T[dim][head] += V^T[dim][key] P^T[key][head] over this wave's 16 d-tiles: per
    // 32-key group c the lane's eight K elements are keys 32c + 4g + {0..3} and
    // 32c + 16 + 4g + {0..3} (the order of pb), read transposed from the key-major tile.
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      if (half && c > 0) break;   // uniform: the second 32-key group is empty
#pragma unroll
      for (int t0 = 0; t0 < NO; t0 += 4) {
        bf16x8_t av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint16_t* p = Kl + tr_off[(t0 + v) & 1] + 32 * c * KLS + 16 * (t0 + v);
          const u32x2_t lo = lds_read_tr16(p);
          const u32x2_t hi = lds_read_tr16(p + 16 * KLS);
          av[v] = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) o[t0 + v] = mfma16x16x32(av[v], pb_hi[c], o[t0 + v]);
        if constexpr (!MX) {
#pragma unroll
          for (int v = 0; v < 4; ++v) o[t0 + v] = mfma16x16x32(av[v], pb_lo[c], o[t0 + v]);
        }
      }
    }
    __syncthreads();   // LDS reads of this tile are done before the next tile's writes
  }

  const float l_tot = xor32_add(xor16_add(l_run));
  // Lane holds O^T[d0 + 16t + 4g + i][h] with d0 = 256dh (HS: 64 wave).
  const int d0 = HS ? 64 * wave : 256 * dh;
  const bool stat_writer = g == 0 && (HS ? wave == 0 : dh == 0);
  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = a.out + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + d0 + 4 * g;
#pragma unroll
    for (int t = 0; t < NO; ++t) *reinterpret_cast<f32x4_t*>(op + 16 * t) = o[t] * inv;
    if (stat_writer)
      a.lse[(int64_t)r * CSA2_HEADS + h] = (m_run == -INFINITY) ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
  } else {
    // Partials keep the accumulator fragment layout, [split][hg + 4 dh][t][lane][4]
    // (dims 256dh + 16t), so every store instruction writes 1 KB of contiguous memory.
    const int64_t ps = (int64_t)r * a.splits + split;
    const int slot = HS ? hg + 4 * (wave >> 2) : wave;
    const int t0 = HS ? 4 * (wave & 3) : 0;
    float* op = a.opart + ((ps * 8 + slot) * 16 + t0) * 256 + 4 * lane;
#pragma unroll
    for (int t = 0; t < NO; ++t) *reinterpret_cast<f32x4_t*>(op + 256 * t) = o[t];
    if (stat_writer) {
      a.mpart[ps * CSA2_HEADS + h] = m_run;
      a.lpart[ps * CSA2_HEADS + h] = l_tot;
    }
  }
}

// Merge of the split partials by log-sum-exp.  Workgroup (w, tg) of a row takes heads
// 16w .. 16w+15 and d-tiles 4tg .. 4tg+3; thread (tt, lane) owns the fragment slot
// (t = 4tg + tt, lane) of every split, so the partial loads are contiguous 1 KB per
// wave.  The 16 heads' per-split statistics are staged in LDS first (one load per
// thread), and the partial loads are issued before the statistics are combined.
constexpr int kMaxSplits = (CSA2_K_MAX + CSA2_SWA_MAX + 31) / 32;

// KB: partial loads issued in one round per thread (>= the launch's splits).  Launches
// with at most 8 splits (many rows) take KB = 8: 64 VGPRs, 8 waves per SIMD, so a
// 64-row launch's 2,048 workgroups are all resident at once (KB = 16 holds 82 VGPRs,
// 5 waves per SIMD).
template <int KB>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  touch_kernargs<sizeof(AttnArgs)>();
  __shared__ float msh[kMaxSplits][16], lsh[kMaxSplits][16];
  const int r = blockIdx.y, w = blockIdx.x >> 3, tg = blockIdx.x & 7;
  const RowKeys rk = row_keys(a, r);
  const int n_keys = rk.n_main + rk.n_swa;
  if (n_keys == 0) return;
  const int per = a.split_keys;
  const int ns = (n_keys + per - 1) / per;
  const int tid = threadIdx.x, lane = tid & 63, tt = tid >> 6, ln = lane & 15, g = lane >> 4;
  const int h = 16 * w + ln, t = 4 * tg + tt;
  const int64_t base = (int64_t)r * a.splits;
  for (int i = tid; i < ns * 16; i += 256) {
    const int s = i >> 4, hh = 16 * w + (i & 15);
    msh[s][i & 15] = a.mpart[(base + s) * CSA2_HEADS + hh];
    lsh[s][i & 15] = a.lpart[(base + s) * CSA2_HEADS + hh];
  }
  // Split partial layout [split][wave = hg + 4 dh][16 d-tiles][lane][4].
  const float* src = a.opart + ((base * 8 + w + 4 * (t >> 4)) * 16 + (t & 15)) * 256 + 4 * lane;
  constexpr int64_t kStride = 8 * 16 * 256;   // floats per split
  constexpr int kBatch = KB;
  f32x4_t v[kBatch];
  // Every load issues (clamped to the launch's last split; only u < ns are used): a
  // guarded load made the compiler wait for the first ones before issuing the rest.
#pragma unroll
  for (int u = 0; u < kBatch; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(src + min(u, a.splits - 1) * kStride);
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, msh[s][ln]);
  float* op = a.out + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + 16 * t + 4 * g;
  const bool lse_writer = tg == 0 && tt == 0 && g == 0;
  if (M == -INFINITY) {
    *reinterpret_cast<f32x4_t*>(op) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (lse_writer) a.lse[(int64_t)r * CSA2_HEADS + h] = -INFINITY;
    return;
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    if (u < ns) {
      const float e = exp2f(msh[u][ln] - M);
      acc += e * v[u];
      L += e * lsh[u][ln];
    }
  }
  for (int s = kBatch; s < ns; ++s) {
    const float e = exp2f(msh[s][ln] - M);
    acc += e * *reinterpret_cast<const f32x4_t*>(src + s * kStride);
    L += e * lsh[s][ln];
  }
  *reinterpret_cast<f32x4_t*>(op) = L > 0.f ? acc * (1.f / L) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (lse_writer) a.lse[(int64_t)r * CSA2_HEADS + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

// Splits per row: enough workgroups to cover the GPU; a split takes its 64-key tiles
// one after another.  The number of splits comes from whole tiles; the keys are then
// spread over them in 32-key units (at least one tile each), which shortens the longest
// split where whole tiles divide unevenly (640 keys in 4 splits: 160 each, the last tile
// of a split half-full, instead of 3 + 3 + 3 + 1 tiles; 64-row attention 33.2 -> 32.3 us).
// A tile holding at most 32 keys runs only its first half.  Finer plans with more splits
// measured slower (32 rows: 7 splits of 96 keys against 5 of 128, +2 us per step).
// Head-split launches (see k_attn): 1 = when four workgroups per split of the plan above
// still fit one per CU (up to 6 rows at 640 keys); 2 = also plan whole-tile splits for
// head-split workgroups when that fits (fewer, longer splits, down to one split per row
// and no merge).  2 measured slower where it differs: batched 32 rows 49.6 -> 52.7 us,
// verify 48 rows 50.4 -> 60.4 us, 64-row attention 32.4 -> 39.0 us (every head-group
// workgroup converts the whole tile, four times the conversion work under load).
#ifndef CSA2_ATTN_HS
#define CSA2_ATTN_HS 1
#endif

void attn_plan(int64_t R, int32_t sel_ld, int32_t& tile_keys, int32_t& split_keys, int32_t& splits,
               int32_t& head_split) {
  const int max_keys = sel_ld + CSA2_SWA_MAX;
  const int tk = kAttnTileKeys;
  const int tiles = (max_keys + tk - 1) / tk;
  int64_t want = R > 0 ? (CSA2_ATTN_TARGET_WGS + R - 1) / R : 1;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  tile_keys = tk;
  const int64_t tps = (tiles + want - 1) / want;
  const int64_t n = (tiles + tps - 1) / tps;
  int64_t per = (max_keys + n - 1) / n;
  per = (per + tk / 2 - 1) / (tk / 2) * (tk / 2);
  if (per < tk) per = tk;
  split_keys = (int32_t)per;
  splits = (int32_t)((max_keys + per - 1) / per);
  head_split = 0;
  if (CSA2_ATTN_HS >= 1 && split_keys % tk == 0 && R * splits * 4 <= CSA2_ATTN_TARGET_WGS) {
    head_split = 1;
  } else if (CSA2_ATTN_HS >= 2) {
    int64_t w4 = R > 0 ? (CSA2_ATTN_TARGET_WGS / 4) / R : 1;
    if (w4 < 1) w4 = 1;
    if (w4 > tiles) w4 = tiles;
    const int64_t tps4 = (tiles + w4 - 1) / w4;
    const int64_t per4 = tps4 * tk;
    const int64_t n4 = (max_keys + per4 - 1) / per4;
    if (R * n4 * 4 <= CSA2_ATTN_TARGET_WGS) {
      split_keys = (int32_t)per4;
      splits = (int32_t)n4;
      head_split = 1;
    }
  }
}

size_t attn_workspace_bytes(int64_t R, int32_t sel_ld) {
  int32_t tk, per, splits, hs;
  attn_plan(R, sel_ld, tk, per, splits, hs);
  if (splits <= 1) return 0;
  const size_t parts = (size_t)R * splits * CSA2_HEADS;
  return parts * CSA2_D * sizeof(float) + 2 * parts * sizeof(float) + 3 * 256;
}

template <bool HALF, bool HS>
static void launch_attn_variant(const AttnArgs& a, dim3 grid, hipStream_t st) {
  if (a.qp_route == CSA2_QP_MXFP8) {
    if (a.sel_rows)
      k_attn<true, true, HALF, HS><<<grid, dim3(512), 0, st>>>(a);
    else
      k_attn<true, false, HALF, HS><<<grid, dim3(512), 0, st>>>(a);
  } else {
    if (a.sel_rows)
      k_attn<false, true, HALF, HS><<<grid, dim3(512), 0, st>>>(a);
    else
      k_attn<false, false, HALF, HS><<<grid, dim3(512), 0, st>>>(a);
  }
}

hipError_t launch_attn_main(const AttnArgs& a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  const bool half = a.split_keys % kAttnTileKeys != 0;
  const bool hs = a.head_split != 0 && !half;
  if (hs)
    launch_attn_variant<false, true>(a, dim3(a.splits * 4, a.g.R), st);
  else if (half)
    launch_attn_variant<true, false>(a, dim3(a.splits, a.g.R), st);
  else
    launch_attn_variant<false, false>(a, dim3(a.splits, a.g.R), st);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t st) {
  if (a.g.R == 0 || a.splits == 1) return hipSuccess;
  const dim3 grid(32, a.g.R), block(256);
  if (a.splits <= 8)
    k_attn_merge<8><<<grid, block, 0, st>>>(a);
  else
    k_attn_merge<16><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

// Selected positions -> pool rows, one thread per slot.
__global__ __launch_bounds__(256) void k_sel_rows(RaggedDev g, const int32_t* sel, const int32_t* n_sel,
                                                 int32_t sel_ld, int32_t* rows) {
  const int r = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= sel_ld) return;
  int ns = n_sel[r];
  ns = ns < 0 ? 0 : (ns > sel_ld ? sel_ld : ns);
  const int64_t vis = row_len_raw(g, r);
  const int b = row_request(g, r);
  int64_t e0, n;
  req_entries(g, b, e0, n);
  n = row_visible(g, vis, n);
  const int64_t pos = sel[(int64_t)r * sel_ld + i];
  rows[(int64_t)r * sel_ld + i] = (i < ns && pos >= 0 && pos < n) ? (int32_t)entry_row(g, b, e0, pos) : -1;
}

hipError_t launch_sel_rows(const RaggedDev& g, const int32_t* sel, const int32_t* n_sel, int32_t sel_ld,
                           int32_t* rows, hipStream_t st) {
  if (g.R == 0) return hipSuccess;
  k_sel_rows<<<dim3((sel_ld + 255) / 256, g.R), dim3(256), 0, st>>>(g, sel, n_sel, sel_ld, rows);
  return hipGetLastError();
}

hipError_t launch_attn(AttnArgs a, hipStream_t st) {
  hipError_t e = launch_attn_main(a, st);
  return e != hipSuccess ? e : launch_attn_merge(a, st);
}

}  // namespace csa2
