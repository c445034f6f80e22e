// LSE merge of split-KV partials (the split merge after the decode
// partials; the same combine the runtime applies across ranks).
#include "common.hpp"

namespace mla {

// Reductions over the 64 lanes of a wave without LDS traffic: rotations
// within each 16-lane row (DPP), then the swaps across rows.
__device__ __forceinline__ float dpp_ror(float x, int n) {
  const int v = __float_as_int(x);
  int r;
  switch (n) {
    case 8: r = __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(v, v, 0x122, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(v, v, 0x121, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

template <typename F>
__device__ __forceinline__ float wave_reduce(float x, F op) {
  x = op(x, dpp_ror(x, 8));
  x = op(x, dpp_ror(x, 4));
  x = op(x, dpp_ror(x, 2));
  x = op(x, dpp_ror(x, 1));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One wave per (row, head): lane l owns latent columns 8l..8l+7.  Lane k
// holds split k's LSE (64 splits per pass); the finite splits are gathered
// with a ballot and their rows loaded four at a time.
__global__ void __launch_bounds__(256) merge_lse_kernel(
    const uint16_t* __restrict__ o_part, int64_t os_split, int64_t os_row, int64_t os_head,
    const float* __restrict__ lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
    int32_t num_splits, int32_t rows, int32_t heads, uint16_t* __restrict__ o, int64_t o_row,
    int64_t o_head, float* __restrict__ lse, int64_t l_row, int64_t l_head) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)rows * heads) return;
  const int64_t t = pair / heads, h = pair % heads;
  const float* lp = lse_part + t * ls_row + h * ls_head;

  // max over splits; a NaN LSE propagates so a poisoned split poisons the row
  float m = -INFINITY;
  for (int k = lane; k < num_splits; k += 64) m = nan_max(m, lp[k * ls_split]);
  m = wave_reduce(m, [](float a, float b) { return nan_max(a, b); });

  uint16_t* op = o + t * o_row + h * o_head + lane * 8;
  if (m == -INFINITY) {
    *reinterpret_cast<u32x4*>(op) = u32x4{0, 0, 0, 0};
    if (lse != nullptr && lane == 0) lse[t * l_row + h * l_head] = -INFINITY;
    return;
  }
  float s = 0.0f;
  for (int k = lane; k < num_splits; k += 64) {
    const float l = lp[k * ls_split];
    if (l != -INFINITY) s += expf(l - m);
  }
  s = wave_reduce(s, [](float a, float b) { return a + b; });
  const float total = m + logf(s);

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = o_part + t * os_row + h * os_head + lane * 8;
  for (int k0 = 0; k0 < num_splits; k0 += 64) {
    const int k = k0 + lane;
    const float l = k < num_splits ? lp[k * ls_split] : -INFINITY;
    const float w = expf(l - total);  // 0 for empty splits, NaN if poisoned
    uint64_t live = __ballot(l != -INFINITY);
    while (live) {
      int ks[4];
      int n = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ks[j] = live ? __builtin_ctzll(live) : -1;
        if (live) {
          live &= live - 1;
          ++n;
        }
      }
      u32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ks[j] >= 0) v[j] = *reinterpret_cast<const u32x4*>(base + (int64_t)(k0 + ks[j]) * os_split);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ks[j] < 0) continue;
        const float wj = __shfl(w, ks[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += wj * __uint_as_float(v[j][e] << 16);
          acc[2 * e + 1] += wj * __uint_as_float(v[j][e] & 0xFFFF0000u);
        }
      }
      (void)n;
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
  *reinterpret_cast<u32x4*>(op) = out;
  if (lse != nullptr && lane == 0) lse[t * l_row + h * l_head] = total;
}

}  // namespace mla

extern "C" int mla_merge_lse(const uint16_t* o_part, int64_t os_split, int64_t os_row,
                             int64_t os_head, const float* lse_part, int64_t ls_split,
                             int64_t ls_row, int64_t ls_head, int32_t num_splits, int32_t rows,
                             int32_t heads, uint16_t* o, int64_t o_row, int64_t o_head, float* lse,
                             int64_t l_row, int64_t l_head, void* stream) {
  if (rows < 0 || heads < 1 || num_splits < 1) return MLA_ERR_INVALID;
  if (rows == 0) return MLA_OK;
  if (!o_part || !lse_part || !o) return MLA_ERR_INVALID;
  // 16-byte vector access of each (split,row,head) latent row
  if ((os_split | os_row | os_head | o_row | o_head) % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if ((((uintptr_t)o_part) | ((uintptr_t)o)) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  int64_t pairs = (int64_t)rows * heads;
  int64_t blocks = (pairs + 3) / 4;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mla::merge_lse_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     o_part, os_split, os_row, os_head, lse_part, ls_split, ls_row, ls_head,
                     num_splits, rows, heads, o, o_row, o_head, lse, l_row, l_head);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
