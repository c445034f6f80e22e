// LSE merge of split-KV partials (the split merge after the decode
// partials; the same combine the runtime applies across ranks).
#include "post_common.hpp"

namespace mla {

// One wave per (row, head): lane l owns latent columns 8l..8l+7.
__global__ void __launch_bounds__(256) merge_lse_kernel(
    const uint16_t* __restrict__ o_part, int64_t os_split, int64_t os_row, int64_t os_head,
    const float* __restrict__ lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
    int32_t num_splits, int32_t rows, int32_t heads, uint16_t* __restrict__ o, int64_t o_row,
    int64_t o_head, float* __restrict__ lse, int64_t l_row, int64_t l_head) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)rows * heads) return;
  const int64_t t = pair / heads, h = pair % heads;
  const float* lp[1] = {lse_part + t * ls_row + h * ls_head};
  const uint16_t* base[1] = {o_part + t * os_row + h * os_head + lane * 8};
  u32x4 out[1];
  float total[1];
  float l1[1];
  merge_lse_load<1>(lp, ls_split, num_splits, lane, l1);
  merge_rows<1>(lp, base, ls_split, os_split, num_splits, lane, l1, out, total);
  *reinterpret_cast<u32x4*>(o + t * o_row + h * o_head + lane * 8) = out[0];
  if (lse != nullptr && lane == 0) lse[t * l_row + h * l_head] = total[0];
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
