// The fp8 encodes of the decode runtime's `pre`: the cache write of new
// tokens (do_kv_cache_update: bf16 [kv_c | k_pe] rows -> fp8 E4M3 cache
// rows) and the query's concat + quantisation (_decode_concat_quant_fp8_op:
// bf16 [ql_nope | q_pe] -> fp8 E4M3 query rows).
#include "common.hpp"

namespace mla {

// One thread per 8 consecutive columns of one token: 72 threads per row.
// The row's 8 values are loaded together with the token's slot (one memory
// round trip, not two: a row is read even when its slot is skipped); VEC:
// one 16-byte load (both sources 16-byte aligned, strides multiples of 8).
template <bool VEC>
__global__ void __launch_bounds__(256) kv_write_kernel(const uint16_t* __restrict__ kv_c,
                                                       int64_t kv_c_stride,
                                                       const uint16_t* __restrict__ k_pe,
                                                       int64_t k_pe_stride,
                                                       const int64_t* __restrict__ slots, int32_t n,
                                                       uint8_t* __restrict__ cache, int64_t num_slots,
                                                       float kv_scale) {
  int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (int64_t)n * 72) return;
  int64_t i = item / 72;
  int c0 = (int)(item % 72) * 8;
  const uint16_t* src = c0 < MLA_D_LATENT ? kv_c + i * kv_c_stride + c0
                                          : k_pe + i * k_pe_stride + (c0 - MLA_D_LATENT);
  uint32_t w[4];
  if constexpr (VEC) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = raw[k];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
  }
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  *reinterpret_cast<u32x2*>(cache + slot * MLA_D_QK + c0) = encode_fp8x8(w, kv_scale);
}

// One thread per 8 consecutive columns of one (row, head) query vector:
// 72 threads per 576-wide row, [ql_nope (512) | q_pe (64)] / q_scale -> E.
__global__ void __launch_bounds__(256) concat_quant_kernel(const uint16_t* __restrict__ ql_nope, int64_t ln_row,
                                                           int64_t ln_head, const uint16_t* __restrict__ q_pe,
                                                           int64_t pe_row, int64_t pe_head, float q_scale,
                                                           int64_t vectors, int32_t heads,
                                                           uint8_t* __restrict__ q8, int64_t q8_row,
                                                           int64_t q8_head) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= vectors * 72) return;
  const int64_t th = item / 72;
  const int c0 = (int)(item - 72 * th) * 8;
  const int64_t t = th / heads, h = th - (int64_t)heads * t;
  const uint16_t* src = c0 < MLA_D_LATENT ? ql_nope + t * ln_row + h * ln_head + c0
                                          : q_pe + t * pe_row + h * pe_head + (c0 - MLA_D_LATENT);
  const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = (raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    const uint32_t b = f32_to_fp8_e4m3(bf16_bits_to_f32(bits) / q_scale);  // correctly rounded division
    if (e < 4)
      lo |= b << (8 * e);
    else
      hi |= b << (8 * (e - 4));
  }
  *reinterpret_cast<u32x2*>(q8 + t * q8_row + h * q8_head + c0) = u32x2{lo, hi};
}

}  // namespace mla

extern "C" const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int mla_kv_write(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                            int64_t k_pe_stride, const int64_t* slot_mapping, int32_t n,
                            uint8_t* kv_cache, int64_t num_slots, float kv_scale, void* stream) {
  if (n < 0 || num_slots < 0) return MLA_ERR_INVALID;
  if (n == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping || !kv_cache) return MLA_ERR_INVALID;
  if (kv_c_stride < MLA_D_LATENT || k_pe_stride < MLA_D_ROPE) return MLA_ERR_INVALID;
  if (!(kv_scale > 0.0f) || !__builtin_isfinite(kv_scale)) return MLA_ERR_INVALID;
  int64_t items = (int64_t)n * 72;
  int64_t blocks = (items + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_UNSUPPORTED;
  const bool vec = ((((uintptr_t)kv_c) | ((uintptr_t)k_pe)) % 16 == 0) && ((kv_c_stride | k_pe_stride) % 8 == 0);
  if (vec)
    hipLaunchKernelGGL(mla::kv_write_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       kv_c, kv_c_stride, k_pe, k_pe_stride, slot_mapping, n, kv_cache, num_slots, kv_scale);
  else
    hipLaunchKernelGGL(mla::kv_write_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       kv_c, kv_c_stride, k_pe, k_pe_stride, slot_mapping, n, kv_cache, num_slots, kv_scale);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" int mla_concat_quant_fp8(const uint16_t* ql_nope, int64_t ln_row, int64_t ln_head, const uint16_t* q_pe,
                                    int64_t pe_row, int64_t pe_head, float q_scale, int32_t rows, int32_t heads,
                                    uint8_t* q8, int64_t q8_row, int64_t q8_head, void* stream) {
  if (rows < 0 || heads < 1) return MLA_ERR_INVALID;
  if (rows == 0) return MLA_OK;
  if (!ql_nope || !q_pe || !q8) return MLA_ERR_INVALID;
  if (!(q_scale > 0.0f) || !__builtin_isfinite(q_scale)) return MLA_ERR_INVALID;
  // 16-byte loads of 8 bf16, 8-byte stores of 8 codes
  if ((ln_row | ln_head | pe_row | pe_head) % 8 != 0 || (((uintptr_t)ql_nope) | ((uintptr_t)q_pe)) % 16 != 0)
    return MLA_ERR_UNSUPPORTED;
  if ((q8_row | q8_head) % 8 != 0 || ((uintptr_t)q8) % 8 != 0) return MLA_ERR_UNSUPPORTED;
  const int64_t vectors = (int64_t)rows * heads;
  const int64_t blocks = (vectors * 72 + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mla::concat_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, ql_nope,
                     ln_row, ln_head, q_pe, pe_row, pe_head, q_scale, vectors, heads, q8, q8_row, q8_head);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
