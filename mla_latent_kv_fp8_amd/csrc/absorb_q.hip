// The absorbed query of the decode runtime's `pre`: the W_UK product
// (batched_gemm_a16wfp4 with transpose_bm and prequant: the bf16 q_nope is
// quantised to MXFP4 per 32 along k, and multiplied by the per-head MXFP4
// W_K [512][128]), concatenated with q_pe into the 576-wide query row, in
// bf16 or as fp8 E4M3 codes of value / q_scale (the y_scale path).
//
// Workgroup = (16 query rows, one head), 4 waves; wave w computes outputs
// n in [128w, 128w + 128) for the 16 rows as C[n][t] = W[h][n][:] . xq[t][:]
// on 16x16x32 bf16 MFMAs (4 K-steps).  Both operands are MXFP4 values,
// which bf16 holds exactly, so the products are exact and the sums are f32.
// The MXFP4 quantisation of a row's 32-element block happens in the four
// lanes that hold it as the B operand of one K-step (lane groups of one
// lane row), with a lane-swap maximum.  The 16 x 576 output tile is
// assembled in LDS and stored as whole rows.
#include "common.hpp"

namespace mla {

// max over the lane groups {l, l^16, l^32, l^48}
__device__ __forceinline__ float absorb_group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// MXFP4 quantisation of one 32-element block held 8 per lane by the four
// lanes of a lane row, dequantised (exactly) back to bf16: shared exponent
// X = floor(log2 max|v|) - 2 held to [-127, 127]; each v / 2^X is rounded to
// the nearest E2M1 value (ties to the even code; the E2M1 grid has step 0.5
// below 2, 1 below 4 and 2 up to 6, and an even code is an even multiple of
// its step), values past 6 take 6.  A block with a NaN or an infinity gives
// NaN; an all-zero block gives zeros.
__device__ __forceinline__ bf16x8 mxfp4_block_dequant(const bf16x8& x) {
  float v[8];
  float amax = 0.0f, bad = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (float)x[i];
    amax = fmaxf(amax, fabsf(v[i]));
    bad = (__builtin_isfinite(v[i]) ? bad : 1.0f);
  }
  amax = absorb_group_max4(amax);
  bad = absorb_group_max4(bad);
  bf16x8 out;
  if (bad != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __builtin_bit_cast(__bf16, (uint16_t)0x7FC0);
    return out;
  }
  // amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1; below the least
  // normal binary32 the exponent is under -128 and X is held at -127
  int X = amax < 0x1p-126f ? -127 : __builtin_amdgcn_frexp_expf(amax) - 3;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = __builtin_ldexpf(fabsf(v[i]), -X);  // exact power-of-two scaling
    const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
    const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
    float q = __builtin_rintf(a * inv) * step;  // exact scalings by powers of two; rint: ties to even
    q = fminf(q, 6.0f);
    const float d = __builtin_copysignf(__builtin_ldexpf(q, X), v[i]);  // exact in bf16
    out[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(d) >> 16));
  }
  if (amax == 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __builtin_bit_cast(__bf16, (uint16_t)0);
  }
  return out;
}

constexpr int AQ_ROWS = 16;
constexpr int AQ_PITCH = MLA_D_QK * 2 + 16;  // bytes per staged output row (bf16 case; +16: bank stagger)

template <bool FP8>
__global__ void __launch_bounds__(256) absorb_q_kernel(const uint16_t* __restrict__ q_nope, int64_t qn_row,
                                                       int64_t qn_head, const uint16_t* __restrict__ q_pe,
                                                       int64_t qp_row, int64_t qp_head,
                                                       const uint8_t* __restrict__ w_k, int64_t wk_head,
                                                       int64_t wk_n, const uint8_t* __restrict__ wk_scale,
                                                       int64_t wks_head, int64_t wks_n, int32_t rows,
                                                       int32_t heads, float q_scale, void* __restrict__ out,
                                                       int64_t out_row, int64_t out_head) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[AQ_ROWS * AQ_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * AQ_ROWS;
  const int t = t0 + lr < rows ? t0 + lr : rows - 1;  // rows past the end compute on the last row
  // B operands: the row's 4 K-steps (k = 32 ks + 8 lg .. +7), MXFP4-quantised
  bf16x8 xq[4];
  {
    const uint16_t* xr = q_nope + (int64_t)t * qn_row + (int64_t)h * qn_head + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xq[ks] = *reinterpret_cast<const bf16x8*>(xr + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xq[ks] = mxfp4_block_dequant(xq[ks]);
  }
  // A operands: W rows n = 128 wave + 16 j + lr, decoded from E2M1 with their
  // E8M0 scale (v_cvt_scalef32_pk_bf16_fp4 multiplies by the scale)
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = 128 * wave + 16 * j + lr;
    const uint8_t* wr = w_k + (int64_t)h * wk_head + (int64_t)n * wk_n + 4 * lg;
    const uint32_t s4 = *reinterpret_cast<const uint32_t*>(wk_scale + (int64_t)h * wks_head + (int64_t)n * wks_n);
    uint32_t codes[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) codes[ks] = *reinterpret_cast<const uint32_t*>(wr + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 wf = fp4x8_to_bf16x8(codes[ks], e8m0_to_f32((s4 >> (8 * ks)) & 0xFF));
      acc[j] = mfma16(wf, xq[ks], acc[j]);
    }
  }
  // outputs n .. n+3 (C rows 4 lg ..) of row lr into the LDS tile
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = 128 * wave + 16 * j + 4 * lg;
    if constexpr (FP8) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) b |= f32_to_fp8_e4m3(acc[j][i] / q_scale) << (8 * i);  // correctly rounded division
      *reinterpret_cast<uint32_t*>(tile + lr * AQ_PITCH + n) = b;
    } else {
      *reinterpret_cast<u32x2*>(tile + lr * AQ_PITCH + 2 * n) =
          u32x2{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])};
    }
  }
  // q_pe: 16 rows x 64 -> 128 threads of 8 values
  if (tid < AQ_ROWS * 8) {
    const int r = tid >> 3, c = 8 * (tid & 7);
    const int tt = t0 + r < rows ? t0 + r : rows - 1;
    const u32x4 pe = *reinterpret_cast<const u32x4*>(q_pe + (int64_t)tt * qp_row + (int64_t)h * qp_head + c);
    if constexpr (FP8) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= f32_to_fp8_e4m3(bf16_bits_to_f32((pe[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) / q_scale) << (8 * i);
        hi |= f32_to_fp8_e4m3(bf16_bits_to_f32((pe[2 + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu) / q_scale)
              << (8 * i);
      }
      *reinterpret_cast<u32x2*>(tile + r * AQ_PITCH + MLA_D_LATENT + c) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<u32x4*>(tile + r * AQ_PITCH + 2 * (MLA_D_LATENT + c)) = pe;
    }
  }
  __syncthreads();
  // whole rows out: 16-byte chunks (72 per bf16 row, 36 per fp8 row)
  constexpr int CH = FP8 ? MLA_D_QK / 16 : MLA_D_QK * 2 / 16;
  const int nrows = rows - t0 < AQ_ROWS ? rows - t0 : AQ_ROWS;
  for (int i = tid; i < nrows * CH; i += 256) {
    const int r = i / CH, c = i - CH * r;
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * AQ_PITCH + 16 * c);
    const int64_t off = (int64_t)(t0 + r) * out_row + (int64_t)h * out_head;  // in output elements
    if constexpr (FP8)
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(out) + off + 16 * c) = v;
    else
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + off + 8 * c) = v;
  }
}

}  // namespace mla

extern "C" int mla_absorb_query(const uint16_t* q_nope, int64_t qn_row, int64_t qn_head, const uint16_t* q_pe,
                                int64_t qp_row, int64_t qp_head, const uint8_t* w_k, int64_t wk_head, int64_t wk_n,
                                const uint8_t* wk_scale, int64_t wks_head, int64_t wks_n, int32_t rows,
                                int32_t heads, int32_t out_fp8, float q_scale, void* out, int64_t out_row,
                                int64_t out_head, void* stream) {
  if (rows < 0 || heads < 1 || (out_fp8 != 0 && out_fp8 != 1)) return MLA_ERR_INVALID;
  if (rows == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_k || !wk_scale || !out) return MLA_ERR_INVALID;
  if (out_fp8 && (!(q_scale > 0.0f) || q_scale == INFINITY)) return MLA_ERR_INVALID;
  if (heads > 65535) return MLA_ERR_UNSUPPORTED;
  // 16-byte row chunks of the bf16 inputs and of the output, 4-byte code
  // words and scale words of W_K
  if ((qn_row | qn_head | qp_row | qp_head) % 8 != 0 || ((uintptr_t)q_nope | (uintptr_t)q_pe) % 16 != 0)
    return MLA_ERR_UNSUPPORTED;
  if ((wk_head | wk_n | wks_head | wks_n) % 4 != 0 || ((uintptr_t)w_k | (uintptr_t)wk_scale) % 4 != 0)
    return MLA_ERR_UNSUPPORTED;
  if ((out_row | out_head) % (out_fp8 ? 16 : 8) != 0 || ((uintptr_t)out) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  const dim3 grid((rows + mla::AQ_ROWS - 1) / mla::AQ_ROWS, heads);
  hipStream_t s = (hipStream_t)stream;
  if (out_fp8)
    hipLaunchKernelGGL(mla::absorb_q_kernel<true>, grid, dim3(256), 0, s, q_nope, qn_row, qn_head, q_pe, qp_row,
                       qp_head, w_k, wk_head, wk_n, wk_scale, wks_head, wks_n, rows, heads, q_scale, out, out_row,
                       out_head);
  else
    hipLaunchKernelGGL(mla::absorb_q_kernel<false>, grid, dim3(256), 0, s, q_nope, qn_row, qn_head, q_pe, qp_row,
                       qp_head, w_k, wk_head, wk_n, wk_scale, wks_head, wks_n, rows, heads, q_scale, out, out_row,
                       out_head);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
