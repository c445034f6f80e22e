// Shared device helpers for the gfx950 MLA decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_fp8.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ conversions

// 4 fp8 E4M3 bytes (one dword, byte 0 first) -> 4 bf16, exactly (E4M3 fits
// in bf16).  v_cvt_scalef32_pk_bf16_fp8 converts bytes {0,1} (word 0) or
// {2,3} (word 1) with a binary32 scale of 1.
__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  bf16x4 a = fp8x4_to_bf16x4(w[0]);
  bf16x4 b = fp8x4_to_bf16x4(w[1]);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 8 E2M1 codes (one dword: byte k holds elements 2k (low nibble) and 2k+1)
// times a binary32 scale -> 8 bf16.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E8M0 scale byte -> binary32 2^(b-127) (b = 0 is the subnormal 2^-127,
// b = 255 NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b == 0 ? 0x00400000u : (b == 255 ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// binary32 -> fp8 E4M3 (OCP fn): round to nearest even, saturate to +-448,
// NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  float av = __uint_as_float(a);
  uint32_t code;
  if (av < 0.015625f) {
    // subnormal range: quantum 2^-9; rint rounds ties to even; 8 -> 0x08 (2^-6)
    code = (uint32_t)__builtin_rintf(av * 512.0f);
  } else {
    // keep 3 mantissa bits, nearest even (carry may bump the exponent)
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    int e = (int)(r >> 23) - 127 + 7;
    uint32_t m = (r >> 20) & 7u;
    if (e > 15 || (e == 15 && m == 7)) {
      code = 0x7Eu;  // saturate (448)
    } else {
      code = ((uint32_t)e << 3) | m;
    }
  }
  return code | sign;
}

// 8 bf16 (dword k holds elements 2k, 2k+1 in its low, high half) -> the
// 8 fp8 E4M3 codes of x / scale (correctly rounded divisions), element 0
// in the low byte of the first dword.
__device__ __forceinline__ u32x2 encode_fp8x8(const uint32_t w[4], float scale) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b = f32_to_fp8_e4m3(bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) / scale);
    if (e < 4)
      lo |= b << (8 * e);
    else
      hi |= b << (8 * (e - 4));
  }
  return u32x2{lo, hi};
}

// 4 bf16 (w0: elements 0, 1; w1: elements 2, 3; low half first) -> the 4
// fp8 E4M3 codes encode_fp8x8 gives for them (of x / scale, the division
// correctly rounded), element 0 in the low byte; rscale = 1 / scale rounded
// to nearest.  With rscale normal and finite, q = |x| * rscale carries two
// roundings of relative size 2^-24 at most, so the correctly rounded
// quotient lies within 8 binary32 steps of q (6 at most, where q and the
// quotient fall in neighbouring binades), and the encoder is monotone in
// the magnitude: where the
// magnitudes 8 steps below and above q get the same code, that code is the
// quotient's.  The codes come from v_cvt_pk_fp8_f32 on magnitudes held to
// [0, 448] (where it rounds as f32_to_fp8_e4m3 does, to nearest even, for
// every binary32 input).  Near a boundary of the fp8 grid (about one value
// in 10^5), for a NaN, and for every value when rscale is subnormal or
// infinite (scale above 2^126 or below 2^-126), the division and
// f32_to_fp8_e4m3 decide.
__device__ __forceinline__ uint32_t encode_fp8x4_fast(uint32_t w0, uint32_t w1, float scale, float rscale) {
  constexpr uint32_t kMax = 0x43E00000u;  // 448
  const uint32_t e[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
  float lo[4], hi[4];
  bool ok = rscale >= 0x1p-126f && rscale <= 0x1.fffffep127f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t mag = (e[k] & 0x7FFFu) << 16;  // |x| as binary32
    ok = ok && mag <= 0x7F800000u;                 // not a NaN
    const uint32_t m = __float_as_uint(__uint_as_float(mag) * rscale);
    lo[k] = __uint_as_float(min(max(m, 8u) - 8u, kMax));
    hi[k] = __uint_as_float(min(m + 8u, kMax));
  }
  // codes of lo[2h+t], hi[2h+t] in bytes 2t, 2t+1 of d[h]
  uint32_t d[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2 * h], hi[2 * h], 0, false);
    d[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo[2 * h + 1], hi[2 * h + 1], v0, true);
    ok = ok && ((d[h] ^ (d[h] >> 8)) & 0x00FF00FFu) == 0;
  }
  if (!ok) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) c |= f32_to_fp8_e4m3(bf16_bits_to_f32(e[k]) / scale) << (8 * k);
    return c;
  }
  const uint32_t code = (d[0] & 0xFFu) | ((d[0] >> 8) & 0xFF00u) | ((d[1] & 0xFFu) << 16) | ((d[1] << 8) & 0xFF000000u);
  const uint32_t sign = ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) | (w1 & 0x80000000u);
  return code | sign;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------ MFMA

// C[16x16] += A[16x32] * B[32x16], bf16 in, f32 accumulate.  Lane l holds
// A row l%16, k 8*(l/16)..+7; B column l%16, same k; C rows 4*(l/16)..+3 of
// column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask));
}

// max that returns NaN if either operand is NaN
__device__ __forceinline__ float nan_max(float a, float b) {
  return (a != a || b != b) ? __builtin_nanf("") : fmaxf(a, b);
}

// ------------------------------------------------------------ split plan

// The split partition of mla_decode_partial, shared by the device kernel
// and the host helper: `chunk` from the partition stream's length T (the
// tokens plus MLA_PIECE_TOKENS per request), the longest request and the
// caller's bounds.
__host__ __device__ __forceinline__ int64_t split_chunk(int64_t T, int64_t lmax, int32_t num_splits,
                                                        int32_t num_workers, int32_t split_min) {
  int64_t chunk = split_min > 1 ? split_min : 1;
  if (num_splits > 1) {
    int64_t a = (T + num_workers - 1) / num_workers;
    int64_t b = (lmax + num_splits - 2) / (num_splits - 1);
    if (a > chunk) chunk = a;
    if (b > chunk) chunk = b;
  } else if (T > chunk) {
    chunk = T;
  }
  return chunk;
}

}  // namespace mla
