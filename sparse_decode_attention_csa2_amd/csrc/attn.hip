// Joint-softmax latent attention over the selected FP4 entries and the FP8 window.
//
// SGLang blog "DeepSeek-V4.1 Flash on SGLang", section "Architecture changes and KV
// cache compression": only the top 512 global positions (FP4, 288 B per entry) take
// part in attention; clawpit.io vLLM article, section "SWA bounded replay": the
// sliding-window cache is FP8 over the 128 most recent positions.  Each head h of the
// row computes one softmax over both key sets (K = V = the 512-dim latent):
//   z_i = sm_scale * q_h . x_i,  out_h = sum_i softmax(z)_i x_i,  lse_h = log sum_i e^z_i.
//
// Kernel structure.  A workgroup (4 waves) takes a range of 32-key tiles of one row.
// Per tile, the 256 threads gather the keys' records and dequantise them (exactly) to
// bf16 in LDS twice: key-major Kl[key][dim] for S^T = K Q^T and dim-major Vt[dim][key]
// for O^T = V^T P^T.  Window tokens enter as their exact E4M3 values; their fp32 scale
// multiplies the logits and the probabilities instead.  Wave w owns heads 16w..16w+15
// (query fragments stay in registers for all tiles); both products run on bf16 16x16x32
// MFMAs with fp32 accumulation, with an online softmax between them.  Workgroups of one
// row write (unnormalised O, running max, running sum) partials that a second kernel
// merges by log-sum-exp; with a single split the kernel writes the result directly.
#include <math.h>

#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int TK = kAttnTile;   // 32 keys per tile
constexpr int KLS = 520;        // Kl row stride in bf16 (512 + 8: 16-B aligned rows, spread banks)
constexpr int VTS = 36;         // Vt row stride in bf16 (32 + 4)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowKeys {
  int64_t e0, n;     // request's first pool entry and entry count
  int n_main;        // selected main entries (slots)
  int64_t s0;        // first window token
  int n_swa;
};

__device__ __forceinline__ RowKeys row_keys(const AttnArgs& a, int r) {
  RowKeys k;
  const int b = row_request(a.g, r);
  req_entries(a.g, b, k.e0, k.n);
  int ns = a.n_sel[r];
  k.n_main = ns < 0 ? 0 : (ns > a.sel_ld ? a.sel_ld : ns);
  int64_t s0 = a.g.row_swa_start[r];
  int len = a.g.row_swa_len[r];
  len = len < 0 ? 0 : (len > CSA2_SWA_MAX ? CSA2_SWA_MAX : len);
  if (s0 < 0 || s0 >= a.g.swa_tokens) {
    s0 = 0;
    len = 0;
  } else if (s0 + len > a.g.swa_tokens) {
    len = (int)(a.g.swa_tokens - s0);
  }
  k.s0 = s0;
  k.n_swa = len;
  return k;
}

__device__ __forceinline__ void st_b128(uint16_t* p, bf16x8_t v) {
  *reinterpret_cast<u32x4_t*>(p) = __builtin_bit_cast(u32x4_t, v);
}

__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  __shared__ __align__(16) uint16_t Kl[TK * KLS];
  __shared__ __align__(16) uint16_t Vt[CSA2_D * VTS];
  __shared__ float ksc[TK];
  __shared__ int kval[TK];

  const int r = blockIdx.y, split = blockIdx.x;
  const RowKeys rk = row_keys(a, r);
  const int n_keys = rk.n_main + rk.n_swa;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;
  const int h = wave * 16 + ln;

  if (n_keys == 0) {
    if (split == 0) {
      for (int i = tid; i < CSA2_HEADS * CSA2_D; i += 256) a.out[(int64_t)r * CSA2_HEADS * CSA2_D + i] = 0.f;
      if (tid < CSA2_HEADS) a.lse[(int64_t)r * CSA2_HEADS + tid] = -INFINITY;
    }
    return;
  }
  const int k_begin = split * a.tiles_per_split * TK;
  if (k_begin >= n_keys) return;
  const int k_end = min(n_keys, k_begin + a.tiles_per_split * TK);

  // Query fragments (B operand of S^T = K Q^T): lane holds q[h][32*st + 8g + j].
  bf16x8_t qb[16];
  {
    const uint16_t* qp = a.q + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + 8 * g;
#pragma unroll
    for (int st = 0; st < 16; ++st) qb[st] = as_bf16x8(load16(qp + 32 * st));
  }

  f32x4_t o[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int kk = tid & (TK - 1);   // dequant role: key kk of the tile ...
  const int ch = tid >> 5;         // ... dims 64ch .. 64ch+63

  for (int kt = k_begin; kt < k_end; kt += TK) {
    __syncthreads();   // the previous tile's LDS reads are done
    {
      const int i = kt + kk;
      bf16x8_t x[8];
      bool valid = false;
      float scale = 0.f;
      if (i < k_end) {
        if (i < rk.n_main) {
          const int64_t pos = a.sel[(int64_t)r * a.sel_ld + i];
          if (pos >= 0 && pos < rk.n) {
            const uint8_t* rec = a.main_kv + (rk.e0 + pos) * CSA2_MAIN_BYTES;
            const u32x4_t c0 = load16(rec + 32 * ch);
            const u32x4_t c1 = load16(rec + 32 * ch + 16);
            const uint32_t s4 = *reinterpret_cast<const uint32_t*>(rec + 256 + 4 * ch);
            const uint32_t wd[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
            for (int w = 0; w < 8; ++w) x[w] = fp4x8_to_bf16(wd[w], e8m0_operand((s4 >> (8 * (w >> 1))) & 255u));
            valid = true;
            scale = 1.f;
          }
        } else {
          const int64_t tok = rk.s0 + (i - rk.n_main);
          const uint8_t* rec = a.swa + tok * CSA2_D + 64 * ch;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4_t c = load16(rec + 16 * u);
            const bf16x4_t lo0 = e4m3x4_to_bf16(c[0]), hi0 = e4m3x4_to_bf16(c[1]);
            const bf16x4_t lo1 = e4m3x4_to_bf16(c[2]), hi1 = e4m3x4_to_bf16(c[3]);
            x[2 * u] = bf16x8_t{lo0[0], lo0[1], lo0[2], lo0[3], hi0[0], hi0[1], hi0[2], hi0[3]};
            x[2 * u + 1] = bf16x8_t{lo1[0], lo1[1], lo1[2], lo1[3], hi1[0], hi1[1], hi1[2], hi1[3]};
          }
          valid = true;
          scale = a.swa_scale[tok];
        }
      }
      if (!valid) {
#pragma unroll
        for (int w = 0; w < 8; ++w) x[w] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
      }
      uint16_t* kr = Kl + kk * KLS + 64 * ch;
#pragma unroll
      for (int w = 0; w < 8; ++w) st_b128(kr + 8 * w, x[w]);
      // Transposed copy, one 16-bit element at a time.  The halves are split from the
      // 32-bit words with integer shifts: element extraction from a bf16 vector into a
      // 16-bit store is mis-selected by this compiler (every store took the low half of
      // the first word).
      uint16_t* vc = Vt + (64 * ch) * VTS + kk;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const u32x4_t xw = __builtin_bit_cast(u32x4_t, x[w]);
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          vc[(8 * w + 2 * q2) * VTS] = (uint16_t)(xw[q2] & 0xFFFFu);
          vc[(8 * w + 2 * q2 + 1) * VTS] = (uint16_t)(xw[q2] >> 16);
        }
      }
      if (ch == 0) {
        ksc[kk] = valid ? scale : 0.f;
        kval[kk] = valid ? 1 : 0;
      }
    }
    __syncthreads();

    // S^T[key][head] for the tile's 32 keys (two 16-key M tiles) and this wave's 16 heads.
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Kl + ln * KLS + 32 * st + 8 * g));
      const bf16x8_t a1 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Kl + (16 + ln) * KLS + 32 * st + 8 * g));
      s0 = mfma16x16x32(a0, qb[st], s0);
      s1 = mfma16x16x32(a1, qb[st], s1);
    }
    // Lane holds keys 4g+i (s0) and 16+4g+i (s1) for head h.
    float z[8];
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4));
      const float s = (j < 4) ? s0[j] : s1[j - 4];
      const bool ok = (kt + key < k_end) && kval[key];
      sc[j] = ksc[key];
      z[j] = ok ? s * sc[j] * a.sm_scale_log2 : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, z[j]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    // Probabilities enter PV as bf16 hi + lo parts: one bf16 would round each weight
    // by up to 2^-9 relative, the whole error budget of the output.
    float psum = 0.f, pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(z[j] - m_use);
      psum += p;
      pv[j] = p * sc[j];
    }
    bf16x8_t pb_hi, pb_lo;
    split_bf16x8(pv, pb_hi, pb_lo);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 32; ++t) o[t] *= alpha;

    // O^T[dim][head] += V^T[dim][key] P^T[key][head]; the K order matches pb's keys.
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const uint16_t* vr = Vt + (16 * t + ln) * VTS;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr + 4 * g);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + 16 + 4 * g);
      const bf16x8_t av = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
      o[t] = mfma16x16x32(av, pb_hi, o[t]);
      o[t] = mfma16x16x32(av, pb_lo, o[t]);
    }
  }

  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  // Lane holds O^T[16t + 4g + i][h].
  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = a.out + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + 4 * g;
#pragma unroll
    for (int t = 0; t < 32; ++t) *reinterpret_cast<f32x4_t*>(op + 16 * t) = o[t] * inv;
    if (g == 0)
      a.lse[(int64_t)r * CSA2_HEADS + h] = (m_run == -INFINITY) ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
  } else {
    const int64_t ps = (int64_t)r * a.splits + split;
    float* op = a.opart + (ps * CSA2_HEADS + h) * CSA2_D + 4 * g;
#pragma unroll
    for (int t = 0; t < 32; ++t) *reinterpret_cast<f32x4_t*>(op + 16 * t) = o[t];
    if (g == 0) {
      a.mpart[ps * CSA2_HEADS + h] = m_run;
      a.lpart[ps * CSA2_HEADS + h] = l_tot;
    }
  }
}

// One workgroup per (head, row): 128 threads x 4 dims.  The per-split statistics are
// loaded in parallel into LDS; the partial outputs are then summed with independent
// loads in flight.
constexpr int kMaxSplits = (CSA2_K_MAX + CSA2_SWA_MAX + TK - 1) / TK;

__global__ __launch_bounds__(128) void k_attn_merge(AttnArgs a) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float msh[kMaxSplits];
  __shared__ float red[2];
  const int h = blockIdx.x, r = blockIdx.y;
  const RowKeys rk = row_keys(a, r);
  const int n_keys = rk.n_main + rk.n_swa;
  if (n_keys == 0) return;
  const int per = a.tiles_per_split * TK;
  const int ns = (n_keys + per - 1) / per;
  const int64_t base = (int64_t)r * a.splits;
  const int tid = threadIdx.x;
  for (int s = tid; s < ns; s += 128) {
    msh[s] = a.mpart[(base + s) * CSA2_HEADS + h];
    wsh[s] = a.lpart[(base + s) * CSA2_HEADS + h];
  }
  __syncthreads();
  if (tid < 64) {
    float M = -INFINITY;
    for (int s = tid; s < ns; s += 64) M = fmaxf(M, msh[s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float L = 0.f;
    if (M != -INFINITY)
      for (int s = tid; s < ns; s += 64) L += wsh[s] * exp2f(msh[s] - M);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
    if (tid == 0) {
      red[0] = M;
      red[1] = L;
    }
  }
  __syncthreads();
  const float M = red[0], L = red[1];
  const int d = 4 * tid;
  float* op = a.out + ((int64_t)r * CSA2_HEADS + h) * CSA2_D + d;
  if (M == -INFINITY || !(L > 0.f)) {
    *reinterpret_cast<f32x4_t*>(op) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tid == 0) a.lse[(int64_t)r * CSA2_HEADS + h] = -INFINITY;
    return;
  }
  const float* src = a.opart + (base * CSA2_HEADS + h) * CSA2_D + d;
  const int64_t stride = (int64_t)CSA2_HEADS * CSA2_D;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    f32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(src + (s + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += exp2f(msh[s + u] - M) * v[u];
  }
  for (; s < ns; ++s) acc += exp2f(msh[s] - M) * *reinterpret_cast<const f32x4_t*>(src + s * stride);
  *reinterpret_cast<f32x4_t*>(op) = acc * (1.f / L);
  if (tid == 0) a.lse[(int64_t)r * CSA2_HEADS + h] = (M + log2f(L)) * kLn2;
}

}  // namespace

void attn_plan(int64_t R, int32_t sel_ld, int32_t& tiles_per_split, int32_t& splits) {
  const int max_keys = sel_ld + CSA2_SWA_MAX;
  const int tiles = (max_keys + TK - 1) / TK;
  int64_t want = R > 0 ? (512 + R - 1) / R : 1;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  tiles_per_split = (int32_t)((tiles + want - 1) / want);
  splits = (tiles + tiles_per_split - 1) / tiles_per_split;
}

size_t attn_workspace_bytes(int64_t R, int32_t sel_ld) {
  int32_t tps, splits;
  attn_plan(R, sel_ld, tps, splits);
  if (splits <= 1) return 0;
  const size_t parts = (size_t)R * splits * CSA2_HEADS;
  return parts * CSA2_D * sizeof(float) + 2 * parts * sizeof(float) + 3 * 256;
}

hipError_t launch_attn_main(const AttnArgs& a, hipStream_t st) {
  if (a.g.R == 0) return hipSuccess;
  k_attn<<<dim3(a.splits, a.g.R), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t st) {
  if (a.g.R == 0 || a.splits == 1) return hipSuccess;
  k_attn_merge<<<dim3(CSA2_HEADS, a.g.R), dim3(128), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn(AttnArgs a, hipStream_t st) {
  hipError_t e = launch_attn_main(a, st);
  return e != hipSuccess ? e : launch_attn_merge(a, st);
}

}  // namespace csa2
