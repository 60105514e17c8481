// Cache write on gfx950: pair pooling, RMSNorm, FP4/E8M0 quantisation, main-KV and
// index-K record writes, block-summary update, ring-slot update.
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Small-operator fusion and
// GEMV" (pooling, RMSNorm, FP4 quantisation and the cache write feed one another and
// are fused) and section "DSpark adaptation and optimization" (verify positions are
// contiguous: a row pools with the previous row, only a request's first row reads the
// ring buffer; the same fused write serves main KV and index K).
//
// One workgroup per request, one launch: a wave per row builds both records of the
// entry the row completes (lane l holds main dims 8l..8l+7 and index dims 2l, 2l+1, so
// a 16-dim main block spans two lanes and a 32-dim index block sixteen); after a
// workgroup barrier (the new records are then visible to the whole workgroup) four
// waves per block sum a quarter of the records of each block that received entries,
// the quarters meet in LDS, one wave per block stores the summary, and one moves the
// ring slot, which every row that reads it has read before the barrier.
#include <climits>

#include "csa2_internal.h"

namespace csa2 {
namespace {

// E2M1 code of v = y / 2^e (|v| < 8): the nearest of 0, .5, 1, 1.5, 2, 3, 4, 6 with
// ties to the even code, above 5 saturating to 6; sign in bit 3 (none for zero).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | ((v < 0.f && m) ? 8u : 0u);
}

// OCP MX shared exponent for FP4: floor(log2(amax)) - 2 (E2M1's largest exponent),
// clamped to E8M0's range; -127 for an all-zero block.
__device__ __forceinline__ int fp4_scale_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Twice the value of an E2M1 code, as a signed integer: the magnitudes 0, .5, 1, 1.5,
// 2, 3, 4, 6 of codes 0..7 doubled are 0, 1, 2, 3, 4, 6, 8, 12 (one nibble each of a
// packed constant); bit 3 is the sign.
__device__ __forceinline__ int e2m1_twice(uint32_t c) {
  const int k = (int)((0xC8643210u >> (4u * (c & 7u))) & 15u);
  return (c & 8u) ? -k : k;
}

// 2^(e - 128) for an E8M0 byte e (0..255) as a double, from its exponent field; with
// the doubled E2M1 value above, k * 2^(e - 128) is an element's exact value.
__device__ __forceinline__ double e8m0_half_scale(uint32_t e) {
  return __longlong_as_double((long long)(e + 895u) << 52);
}

typedef float f32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));

// Cross-lane steps on the VALU (no LDS round trips): lanes l and l ^ 32 / l ^ 16 through
// gfx950's permlane swaps; within a 16-lane row, DPP rotations by 8 (lane l ^ 8) and by
// 4, and quad permutes for l ^ 2 and l ^ 1.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

// Sum over the wave, as the butterfly over lanes l ^ 32, 16, 8, 4, 2, 1 adds it (each
// step adds the same two values; after the step over l ^ 8, lanes l and l ^ 8 agree, so
// the rotation by 4 reads lane l ^ 4's value).
__device__ __forceinline__ float wave_sum_f(float v) {
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  v += __uint_as_float(dpp<kRowRor8>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kRowRor4>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kQuadXor1>(__float_as_uint(v)));
  return v;
}

// Maximum over each 16-lane row (order does not matter for a maximum).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kQuadXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kQuadXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kRowRor4>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp<kRowRor8>(__float_as_uint(v))));
}

// Minimum and maximum over the wave.
__device__ __forceinline__ void wave_minmax_i(int& lo, int& hi) {
  const auto a32 = __builtin_amdgcn_permlane32_swap((uint32_t)lo, (uint32_t)lo, false, false);
  const auto b32 = __builtin_amdgcn_permlane32_swap((uint32_t)hi, (uint32_t)hi, false, false);
  lo = min((int)a32[0], (int)a32[1]);
  hi = max((int)b32[0], (int)b32[1]);
  const auto a16 = __builtin_amdgcn_permlane16_swap((uint32_t)lo, (uint32_t)lo, false, false);
  const auto b16 = __builtin_amdgcn_permlane16_swap((uint32_t)hi, (uint32_t)hi, false, false);
  lo = min((int)a16[0], (int)a16[1]);
  hi = max((int)b16[0], (int)b16[1]);
  lo = min(lo, (int)dpp<kRowRor8>((uint32_t)lo));
  hi = max(hi, (int)dpp<kRowRor8>((uint32_t)hi));
  lo = min(lo, (int)dpp<kRowRor4>((uint32_t)lo));
  hi = max(hi, (int)dpp<kRowRor4>((uint32_t)hi));
  lo = min(lo, (int)dpp<kQuadXor2>((uint32_t)lo));
  hi = max(hi, (int)dpp<kQuadXor2>((uint32_t)hi));
  lo = min(lo, (int)dpp<kQuadXor1>((uint32_t)lo));
  hi = max(hi, (int)dpp<kQuadXor1>((uint32_t)hi));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// bf16 bits of a double, one round to nearest even (normal bf16 range; outside it the
// value goes through fp32).
__device__ __forceinline__ uint32_t bf16_rne_from_double(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int exp = (int)((u >> 52) & 0x7FF);
  const int eb = exp - 1023 + 127;
  if (d == 0.0) return sign;
  if (exp == 0 || exp == 0x7FF || eb < 1 || eb > 254) return bf16_bits_rne((float)d);
  const uint64_t mant = (u & ((1ull << 52) - 1)) | (1ull << 52);             // 53 bits
  uint64_t r = (mant + ((1ull << 44) - 1) + ((mant >> 45) & 1)) >> 45;        // 8 bits, RNE
  int e2 = eb;
  if (r == 256) {
    r = 128;
    ++e2;
  }
  if (e2 > 254) return bf16_bits_rne((float)d);
  return sign | ((uint32_t)e2 << 7) | (uint32_t)(r & 0x7F);
}

struct WriteArgs {
  RaggedDev g;
  const int64_t* row_pos;
  const uint16_t* kv_tok;
  const uint16_t* idx_tok;
  uint16_t* ring_kv;
  uint16_t* ring_idx;
  const float* gamma_kv;
  const float* gamma_idx;
  float eps;
  uint8_t* main_kv;
  uint8_t* idx_k;
  uint16_t* blk_sum;
};

// Records of the entry that row r of request b (rows from r0) completes; one wave, lane
// = its lane.  Every input is loaded before any record is written (the stores could
// otherwise hold back the index vector's loads).
__device__ void write_entry(const WriteArgs& a, int b, int r0, int r, int lane) {
  int64_t e0, n;
  req_entries(a.g, b, e0, n);
  const int64_t p = a.row_pos[r];
  const int64_t pprev = a.row_pos[r > 0 ? r - 1 : 0];
  // Both partner candidates (the previous row's tokens and the ring slot) are loaded
  // with the row's own, so no token load waits for the positions.
  const int rq = r > 0 ? r - 1 : 0;
  const uint16_t* xk = a.kv_tok + (int64_t)r * CSA2_D;
  const uint16_t* xi = a.idx_tok + (int64_t)r * CSA2_IDX_D;
  const u32x4_t vq = load16(a.kv_tok + (int64_t)rq * CSA2_D + 8 * lane);
  const u32x4_t vr = load16(a.ring_kv + (int64_t)b * CSA2_D + 8 * lane);
  const u32x4_t vb = load16(xk + 8 * lane);
  const uint32_t wq = *reinterpret_cast<const uint32_t*>(a.idx_tok + (int64_t)rq * CSA2_IDX_D + 2 * lane);
  const uint32_t wr = *reinterpret_cast<const uint32_t*>(a.ring_idx + (int64_t)b * CSA2_IDX_D + 2 * lane);
  const uint32_t wb = *reinterpret_cast<const uint32_t*>(xi + 2 * lane);
  const f32x4a4_t gk0 = *reinterpret_cast<const f32x4a4_t*>(a.gamma_kv + 8 * lane);
  const f32x4a4_t gk1 = *reinterpret_cast<const f32x4a4_t*>(a.gamma_kv + 8 * lane + 4);
  const float gi0 = a.gamma_idx[2 * lane], gi1 = a.gamma_idx[2 * lane + 1];
  asm volatile("" ::: "memory");   // keep the loads here, ahead of the checks below
  const bool prev_row = r - 1 >= r0 && pprev == p - 1;
  const u32x4_t va = prev_row ? vq : vr;
  const uint32_t wa = prev_row ? wq : wr;
  // Entry completed by the row: t = (P-1)/2 for an odd position P with t < N_b.
  if (p < 0 || (p & 1) == 0) return;
  const int64_t t = (p - 1) / 2;
  if (t >= n) return;
  const int64_t row = entry_row(a.g, b, e0, t);

  // Main vector: dims 8 lane .. 8 lane + 7.
  {
    const float gk[8] = {gk0[0], gk0[1], gk0[2], gk0[3], gk1[0], gk1[1], gk1[2], gk1[3]};
    float y[8];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] = (bf16_lo(va[q]) + bf16_lo(vb[q])) * 0.5f;
      y[2 * q + 1] = (bf16_hi(va[q]) + bf16_hi(vb[q])) * 0.5f;
      ss = fmaf(y[2 * q], y[2 * q], ss);
      ss = fmaf(y[2 * q + 1], y[2 * q + 1], ss);
    }
    const float rs = 1.f / sqrtf(wave_sum_f(ss) / (float)CSA2_D + a.eps);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = y[i] * rs * gk[i];
      amax = fmaxf(amax, fabsf(y[i]));
    }
    amax = fmaxf(amax, __uint_as_float(dpp<kQuadXor1>(__float_as_uint(amax))));   // 16-dim block = lanes 2k, 2k+1
    const int e = fp4_scale_exp(amax);
    uint32_t codes = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) codes |= e2m1_code(__builtin_ldexpf(y[i], -e)) << (4 * i);
    uint8_t* rec = a.main_kv + row * CSA2_MAIN_BYTES;
    *reinterpret_cast<uint32_t*>(rec + 4 * lane) = codes;
    if ((lane & 1) == 0) rec[256 + lane / 2] = (uint8_t)(e + 127);
  }
  // Index vector: dims 2 lane, 2 lane + 1.
  {
    float y0 = (bf16_lo(wa) + bf16_lo(wb)) * 0.5f, y1 = (bf16_hi(wa) + bf16_hi(wb)) * 0.5f;
    const float ss = fmaf(y1, y1, y0 * y0);
    const float rs = 1.f / sqrtf(wave_sum_f(ss) / (float)CSA2_IDX_D + a.eps);
    y0 = y0 * rs * gi0;
    y1 = y1 * rs * gi1;
    float amax = fmaxf(fabsf(y0), fabsf(y1));
    amax = row16_max(amax);   // 32-dim block = 16 lanes
    const int e = fp4_scale_exp(amax);
    const uint32_t c = e2m1_code(__builtin_ldexpf(y0, -e)) | (e2m1_code(__builtin_ldexpf(y1, -e)) << 4);
    uint8_t* rec = a.idx_k + row * CSA2_IDX_BYTES;
    rec[lane] = (uint8_t)c;
    if ((lane & 15) == 0) rec[64 + lane / 16] = (uint8_t)(e + 127);
  }
}

// Summary of block `which` (0 or 1) of the (at most two) blocks request b's rows wrote
// into, and the request's ring slot.  summary_prepare, before the records are written:
// the rows' positions, the block and (ring) the ring slot's tokens, all kernel inputs;
// summary_part, after: a quarter of the block's records summed; summary_finish: the
// quarters added and the stores.
struct SummaryPrep {
  const uint8_t* blk;   // the block's first index record
  uint16_t* dst;        // its summary, dims 2 lane, 2 lane + 1
  int cnt;              // entries in the block (0: no block to summarise)
  bool ring;            // the last row waits for its partner: move its tokens to the ring
  u32x4_t rk;
  uint32_t ri;
};

__device__ SummaryPrep summary_prepare(const WriteArgs& a, int b, int which, bool ring, int lane) {
  SummaryPrep sp{};
  int r0, r1;
  req_rows(a.g, b, CSA2_ROWS_PER_REQ_MAX, r0, r1);
  if (r1 <= r0) return sp;
  int64_t e0, n, bl0, nb;
  req_entries(a.g, b, e0, n);
  req_blocks(a.g, b, n, bl0, nb);
  // Lane l looks at row r0 + l (a request has at most 16 rows): one load round for all.
  static_assert(CSA2_ROWS_PER_REQ_MAX <= 64, "one row per lane");
  int64_t tl = -1;
  if (r0 + lane < r1) {
    const int64_t p = a.row_pos[r0 + lane];
    tl = (p >= 0 && (p & 1) != 0 && (p - 1) / 2 < n) ? (p - 1) / 2 : -1;
  }
  // Entries are below max_entries (32 bits).
  int tmin = tl >= 0 ? (int)tl : INT_MAX, tmax = (int)tl;
  wave_minmax_i(tmin, tmax);
  if (tmin != INT_MAX) {
    const int64_t j = tmin / CSA2_BLOCK + which;
    if (j <= tmax / CSA2_BLOCK && j < nb) {
      // A block's entries are consecutive pool rows (a page, with paged pools).
      sp.cnt = (int)min<int64_t>(CSA2_BLOCK, n - j * CSA2_BLOCK);
      sp.blk = a.idx_k + entry_row(a.g, b, e0, j * CSA2_BLOCK) * CSA2_IDX_BYTES;
      sp.dst = a.blk_sum + block_row(a.g, b, bl0, j) * CSA2_IDX_D + 2 * lane;
    }
  }
  // Ring slot: the last row's token when it waits for its partner (even position).
  if (ring) {
    const int64_t p = a.row_pos[r1 - 1];
    if (p >= 0 && (p & 1) == 0) {
      sp.ring = true;
      sp.rk = load16(a.kv_tok + (int64_t)(r1 - 1) * CSA2_D + 8 * lane);
      sp.ri = *reinterpret_cast<const uint32_t*>(a.idx_tok + (int64_t)(r1 - 1) * CSA2_IDX_D + 2 * lane);
    }
  }
  return sp;
}

// Part q (of kSumParts) of a block's sum: entries [16q, 16q + 16), loaded at once
// (clamped to the block's last entry); each element's exact value (a small integer times
// a power of two) is summed in entry order, entries past the block's count adding zero.
constexpr int kSumParts = 4;
constexpr int kSumPart = CSA2_BLOCK / kSumParts;
__device__ void summary_part(const SummaryPrep& sp, int q, int lane, double& s0, double& s1) {
  s0 = 0.0;
  s1 = 0.0;
  if (sp.cnt <= 0) return;
  uint32_t c[kSumPart], sb[kSumPart];
#pragma unroll
  for (int u = 0; u < kSumPart; ++u) {
    const uint8_t* rec = sp.blk + min(kSumPart * q + u, sp.cnt - 1) * CSA2_IDX_BYTES;
    c[u] = rec[lane];
    sb[u] = rec[64 + lane / 16];
  }
#pragma unroll
  for (int u = 0; u < kSumPart; ++u) {
    const double sc = kSumPart * q + u < sp.cnt ? e8m0_half_scale(sb[u]) : 0.0;
    s0 += (double)e2m1_twice(c[u] & 15u) * sc;
    s1 += (double)e2m1_twice(c[u] >> 4) * sc;
  }
}

// The block's summary from its parts' sums (added in part order) and the ring slot.
__device__ void summary_finish(const WriteArgs& a, int b, const SummaryPrep& sp, const double (*part)[2], int lane) {
  if (sp.cnt > 0) {
    double s0 = part[0][0], s1 = part[0][1];
#pragma unroll
    for (int q = 1; q < kSumParts; ++q) {
      s0 += part[q][0];
      s1 += part[q][1];
    }
    const uint32_t w = bf16_rne_from_double(s0 / sp.cnt) | (bf16_rne_from_double(s1 / sp.cnt) << 16);
    *reinterpret_cast<uint32_t*>(sp.dst) = w;
  }
  if (sp.ring) {
    *reinterpret_cast<u32x4_t*>(a.ring_kv + (int64_t)b * CSA2_D + 8 * lane) = sp.rk;
    *reinterpret_cast<uint32_t*>(a.ring_idx + (int64_t)b * CSA2_IDX_D + 2 * lane) = sp.ri;
  }
}

// Workgroup b (at least 2 x kSumParts waves): the request's rows (wave w takes rows
// r0 + w, r0 + w + waves, ...), then its block summaries: wave w < 2 kSumParts sums
// part w / 2 of block w % 2 (the preparation, which reads only kernel inputs, runs before
// the rows), the parts meet in LDS, and waves 0 and 1 add them in part order and store
// the summaries (and, wave 0, the ring slot).
__global__ __launch_bounds__(64 * CSA2_ROWS_PER_REQ_MAX) void k_write(WriteArgs a) {
  __shared__ double psum[2][kSumParts][64][2];
  const int b = blockIdx.x;
  const int nw = (int)(blockDim.x >> 6);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool summer = wave < 2 * kSumParts;
  SummaryPrep sp{};
  if (summer) sp = summary_prepare(a, b, wave & 1, wave == 0, lane);   // wave 0 moves the ring slot
  int r0, r1;
  req_rows(a.g, b, CSA2_ROWS_PER_REQ_MAX, r0, r1);
  for (int r = r0 + wave; r < r1; r += nw) write_entry(a, b, r0, r, lane);
  __syncthreads();
  if (summer) {
    double s0, s1;
    summary_part(sp, wave >> 1, lane, s0, s1);
    psum[wave & 1][wave >> 1][lane][0] = s0;
    psum[wave & 1][wave >> 1][lane][1] = s1;
  }
  __syncthreads();
  if (wave < 2) {
    double part[kSumParts][2];
#pragma unroll
    for (int q = 0; q < kSumParts; ++q) {
      part[q][0] = psum[wave][q][lane][0];
      part[q][1] = psum[wave][q][lane][1];
    }
    summary_finish(a, b, sp, part, lane);
  }
}

}  // namespace

hipError_t launch_cache_write(const RaggedDev& g, int32_t max_rows_per_request, const int64_t* row_pos,
                              const uint16_t* kv_tok, const uint16_t* idx_tok, uint16_t* ring_kv, uint16_t* ring_idx,
                              const float* gamma_kv, const float* gamma_idx, float eps, uint8_t* main_kv,
                              uint8_t* idx_k, uint16_t* blk_sum, hipStream_t st) {
  if (g.R == 0 || g.B == 0) return hipSuccess;
  WriteArgs a{g, row_pos, kv_tok, idx_tok, ring_kv, ring_idx, gamma_kv, gamma_idx, eps, main_kv, idx_k, blk_sum};
  // A wave per row of the largest request, and at least one per part of the two
  // summaries.
  static_assert(2 * kSumParts <= CSA2_ROWS_PER_REQ_MAX, "summary waves fit the workgroup");
  const int nw = max_rows_per_request < 2 * kSumParts
                     ? 2 * kSumParts
                     : (max_rows_per_request > CSA2_ROWS_PER_REQ_MAX ? CSA2_ROWS_PER_REQ_MAX : max_rows_per_request);
  k_write<<<dim3(g.B), dim3(64 * nw), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa2
