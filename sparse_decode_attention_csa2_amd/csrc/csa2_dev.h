// Device helpers shared by the gfx950 kernels of libcsa2: cache-format dequantisation
// (FP4 E2M1 with E8M0 scales, FP8 E4M3FN), the bf16 MFMA, order-preserving score keys
// and wave/workgroup scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace csa2 {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------
// Dequantisation.  E2M1 values times an E8M0 power of two, and E4M3FN values, are
// exact in bf16 (bf16 keeps fp32's exponent range), so every converted operand below is
// the exact value of the stored code.
// ---------------------------------------------------------------------------------

// The scaled converts of gfx950 take the scale as an fp32 whose exponent field is the
// E8M0 code (value 2^(u-127)).
__device__ __forceinline__ float e8m0_operand(uint32_t u) { return __uint_as_float(u << 23); }

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16 x scale.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t codes, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 4 E4M3FN codes (one dword, element i in byte i) -> 4 bf16 (unscaled, exact).
__device__ __forceinline__ bf16x4_t e4m3x4_to_bf16(uint32_t codes) {
  const float one = 1.0f;
  bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, one, false);
  bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, one, true);
  return bf16x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// fp32 -> bf16 bit pattern, round half to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> two bf16 (round half to even; a in the low half): one v_cvt_pk_bf16_f32.
// Equal to bf16_bits_rne on both for finite inputs (fp32 denormals are preserved).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{a, b}), b2_t));
}

// Split 8 fp32 values into bf16 hi + lo parts (v ~= hi + lo to about 2^-17 relative),
// packed as MFMA operands: hi = RNE(v), lo = RNE(v - hi).
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t hw, lw;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t h = pack_bf16x2_rne(v[2 * q], v[2 * q + 1]);
    const float r0 = v[2 * q] - __uint_as_float(h << 16);
    const float r1 = v[2 * q + 1] - __uint_as_float(h & 0xFFFF0000u);
    hw[q] = h;
    lw[q] = pack_bf16x2_rne(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8_t, hw);
  lo = __builtin_bit_cast(bf16x8_t, lw);
}

// Max / sum of x over lanes l and l ^ 16, and over lanes l and l ^ 32, through gfx950's
// row and half swaps (VALU, no LDS round trip).  v_permlane16_swap of x with itself
// gives every lane the values of its 16-lane row pair (even row first), and
// v_permlane32_swap those of its two 32-lane halves (lower half first); max and sum are
// symmetric, so every lane gets the same bits as x op shuffle(x).
__device__ __forceinline__ float xor16_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_add(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ---------------------------------------------------------------------------------
// MXFP8 (OCP MX v1.0: E4M3 elements sharing one E8M0 scale per 32-value block).
// The block's shared exponent is floor(log2(amax)) - 8 (E4M3's largest exponent),
// clamped to E8M0's range; each value x becomes RNE_E4M3(x / 2^s) * 2^s, saturating at
// 448.  The rounding is done in fp32 arithmetic (exact scalings, one round-to-nearest-
// even of a value with the grid step brought to 1), not by a conversion instruction.
// ---------------------------------------------------------------------------------
#ifndef CSA2_MX_HW_CVT
#define CSA2_MX_HW_CVT 1
#endif

__device__ __forceinline__ int mx8_scale_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1;   // floor(log2(amax)), subnormals included
  const int s = e - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

__device__ __forceinline__ float mx8_round(float x, int s) {
  const float y = fminf(__builtin_ldexpf(fabsf(x), -s), 448.f);   // |x| / 2^s, < 2^9
  // Grid step 2^(e-3) with e = floor(log2 y), and 2^-9 (subnormals) below 2^-6.
  const int e = max(__builtin_amdgcn_frexp_expf(y) - 1, -6);
  const float r = __builtin_ldexpf(__builtin_rintf(__builtin_ldexpf(y, 3 - e)), e - 3);
  return copysignf(__builtin_ldexpf(fminf(r, 448.f), s), x);
}

// MXFP8-round 8 fp32 values of a block with shared exponent s, packed as an exact bf16
// MFMA operand (element q in the low half of word q / 2).
__device__ __forceinline__ bf16x8_t mx8_round8_bf16x8(const float (&v)[8], int s) {
  u32x4_t w;
#if CSA2_MX_HW_CVT
  // gfx950's scaled FP8 conversions: x / 2^s to E4M3FN (round to nearest even) and back
  // times 2^s straight to bf16 (exact: an E4M3 value times 2^s), after clamping to the largest grid value (448 units) so nothing overflows.
  typedef short v2s __attribute__((ext_vector_type(2)));
  const float sc = __builtin_ldexpf(1.f, s), lim = __builtin_ldexpf(448.f, s);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = __builtin_amdgcn_fmed3f(v[2 * q], -lim, lim), b = __builtin_amdgcn_fmed3f(v[2 * q + 1], -lim, lim);
    const v2s p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, a, b, sc, false);
    w[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                            (uint32_t)__builtin_bit_cast(int, p), sc, false));
  }
#else
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = bf16_bits_rne(mx8_round(v[2 * q], s)) | (bf16_bits_rne(mx8_round(v[2 * q + 1], s)) << 16);
#endif
  return __builtin_bit_cast(bf16x8_t, w);
}

// MXFP8-round 8 fp32 values of a 32-value block whose other 24 values sit in the lanes
// xor 16 and xor 32 (a lane's 8 values are one quarter of the block).
__device__ __forceinline__ bf16x8_t mx8_round_block_bf16x8(const float (&v)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = xor32_max(xor16_max(amax));
  return mx8_round8_bf16x8(v, mx8_scale_exp(amax));
}

// Packed 16-bit unsigned max / min of two words (v_pk_max_u16, v_pk_min_u16).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}

// The same MXFP8 rounding for a block of bf16 values (the query), without leaving bf16:
// a bf16 magnitude's bits order like its value, so the block maximum is a packed 16-bit
// integer max (then over lanes xor 16 and xor 32), its exponent field f gives the shared
// exponent s = max(f, 8) - 135 (f - 127 = floor(log2 amax) for normal amax; zero and
// subnormal maxima give f = 0 and s = -127), the saturation at 448 * 2^s is a packed
// integer min of the magnitudes against that value's bits (exponent field s + 135,
// mantissa 0x60), and gfx950's scaled conversions take bf16 pairs to E4M3FN (round to
// nearest even) and back.
__device__ __forceinline__ bf16x8_t mx8_round_block_bf16(bf16x8_t x) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const u32x4_t w = __builtin_bit_cast(u32x4_t, x);
  u32x4_t mag;
#pragma unroll
  for (int q = 0; q < 4; ++q) mag[q] = w[q] & 0x7FFF7FFFu;
  uint32_t mm = pk_max_u16(pk_max_u16(mag[0], mag[1]), pk_max_u16(mag[2], mag[3]));
  const auto p16 = __builtin_amdgcn_permlane16_swap(mm, mm, false, false);
  mm = pk_max_u16(p16[0], p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(mm, mm, false, false);
  mm = pk_max_u16(p32[0], p32[1]);
  const uint32_t f = max(max(mm & 0xFFFFu, mm >> 16) >> 7, 8u);   // s + 135
  const float sc = e8m0_operand(f - 8u);                           // 2^s
  const uint32_t lim = (f << 7) | 0x60u;                           // bf16 bits of 448 * 2^s
  const uint32_t lim2 = lim | (lim << 16);
  u32x4_t out;
#pragma unroll
  for (int q = 0; q < 4; q += 2) {
    const uint32_t c0 = (w[q] & 0x80008000u) | pk_min_u16(mag[q], lim2);
    const uint32_t c1 = (w[q + 1] & 0x80008000u) | pk_min_u16(mag[q + 1], lim2);
    v2s e = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, __builtin_bit_cast(bf16x2_t, c0), sc, false);
    e = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(e, __builtin_bit_cast(bf16x2_t, c1), sc, true);
    const uint32_t codes = __builtin_bit_cast(uint32_t, e);
    out[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, sc, false));
    out[q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, sc, true));
  }
  return __builtin_bit_cast(bf16x8_t, out);
}

// Widen 8 bf16 to fp32 through the packed 32-bit words (integer shifts only).
__device__ __forceinline__ void bf16x8_words_to_f32(bf16x8_t x, float (&v)[8]) {
  const u32x4_t w = __builtin_bit_cast(u32x4_t, x);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x4_t as_bf16x4(u32x2_t v) { return __builtin_bit_cast(bf16x4_t, v); }

// 16-byte load from an address that is only 4-byte aligned (68-B records); gfx950
// global loads accept it.
__device__ __forceinline__ u32x4_t load16_a4(const uint8_t* p) {
  typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
  return *reinterpret_cast<const u32x4a4_t*>(p);
}
__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void store16_a4(float* p, f32x4_t v) {
  typedef float f32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
  *reinterpret_cast<f32x4a4_t*>(p) = v;
}

// ---------------------------------------------------------------------------------
// MFMA: D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16] (j < 8), and receives
// D[4*(l/16) + i][l%16] (i < 4).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------
// Selection keys: larger score -> larger unsigned key; +0 and -0 map to one key; NaN
// maps to 0, the key of an empty item (a NaN score never takes part in a ranking).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return s != s ? 0u : key;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }


// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves (no LDS round
// trips): row_shr 1/2/4/8 scans each row of 16 lanes, then row_bcast15 and row_bcast31
// carry row totals into the following rows.  Lanes a move has no source for add 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Wave-wide max / min of 32-bit unsigned values on DPP moves; lane 63 ends with the
// result, which readlane makes uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return ~wave_max_u32(~x);
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v);

template <>
__device__ __forceinline__ uint32_t wave_incl_scan<uint32_t>(uint32_t v) { return wave_incl_scan_u32(v); }

template <>
__device__ __forceinline__ int wave_incl_scan<int>(int v) { return (int)wave_incl_scan_u32((uint32_t)v); }

// 64-bit values as two 32-bit halves (each half's sum must stay below 2^32).
template <>
__device__ __forceinline__ uint64_t wave_incl_scan<uint64_t>(uint64_t v) {
  const uint32_t lo = wave_incl_scan_u32((uint32_t)v), hi = wave_incl_scan_u32((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Exclusive prefix sum over a workgroup of NT threads; `tmp` is LDS of NT/64 + 1 entries.
// Also returns the total.  Contains two barriers.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* tmp, T& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  T incl = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    T x = tmp[w];
    if (w < wave) before += x;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

#ifndef CSA2_TOUCH_KERNARGS
#define CSA2_TOUCH_KERNARGS 1
#endif

// Reads one dword of each 64-byte line of the first BYTES of the kernel's argument
// segment, all in the kernel's first round of scalar loads.  A kernel's arguments are
// otherwise fetched as it needs them, and a line first touched after a dependent load
// costs another full memory round trip on the kernel's critical path.
template <int BYTES>
__device__ __forceinline__ void touch_kernargs() {
#if CSA2_TOUCH_KERNARGS
  static_assert(BYTES <= 256, "at most four argument lines");
  const uint32_t __attribute__((address_space(4)))* p =
      (const uint32_t __attribute__((address_space(4)))*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t v0 = p[0];
  const uint32_t v1 = BYTES > 64 ? p[16] : 0u;
  const uint32_t v2 = BYTES > 128 ? p[32] : 0u;
  const uint32_t v3 = BYTES > 192 ? p[48] : 0u;
  asm volatile("" ::"s"(v0), "s"(v1), "s"(v2), "s"(v3));
#endif
}

}  // namespace csa2
