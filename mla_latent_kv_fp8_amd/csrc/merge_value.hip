// The LSE merge of the split partials fused with the W_UV value projection
// and the FP32 sigmoid gate (the runtime's `post`; [VALUE] `MlaValue`, whose
// weight fragments load before the latent is ready).  The merged latent
// never leaves the workgroup.
#include "post_common.hpp"

namespace mla {

constexpr int MV_ROWS = 16;          // rows per workgroup (one MFMA N tile)
constexpr int MV_WAVES = 16;         // one merged row each; waves 0..7 also compute 16 outputs each
constexpr int MV_PITCH = 512 + 8;    // LDS row pitch in bf16 (1040 B)

// Workgroup = (16-row block, head), 16 waves.  Wave w merges row w of the
// block (the same device code as mla_merge_lse, so the latent is the bf16
// value that call writes) into LDS.  Waves 0..7 first issue the loads of
// the W_UV fragments of outputs 16w..16w+15 for all 16 K-steps, and after
// the merge compute C[v][t] = W[h][v][:] . latent[t][h][:] on 16x16x32 bf16
// MFMAs and apply the gate epilogue.
// The row blocks of a head share an XCD, so its W is read once from HBM.
template <int FMT>
__global__ void __launch_bounds__(MV_WAVES * 64) merge_value_kernel(
    const uint16_t* __restrict__ o_part, int64_t os_split, int64_t os_row, int64_t os_head,
    const float* __restrict__ lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head, int32_t num_splits,
    const void* __restrict__ w_uv, int64_t w_head, int64_t w_v, const uint8_t* __restrict__ w_scale,
    int64_t ws_head, int64_t ws_v, const uint16_t* __restrict__ gate, int64_t g_row,
    const int32_t* __restrict__ lengths, int32_t rows, int32_t qlen, int32_t heads, int32_t nrb,
    uint16_t* __restrict__ out, int64_t out_row, float* __restrict__ lse, int64_t l_row, int64_t l_head) {
  __shared__ __attribute__((aligned(16))) uint16_t lat[MV_ROWS * MV_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  int h, rb;
  {
    const int bid = blockIdx.x, slot = bid >> 3;
    h = (bid & 7) + 8 * (slot / nrb);
    rb = slot % nrb;
  }
  if (h >= heads) return;
  const int t0 = rb * MV_ROWS;
  const bool mfma_wave = wave < 8;  // wave-uniform

  // the MFMA waves: W fragments (lane: output v, latents 32s + 8lg .. +7),
  // then the epilogue's gate values and row lengths
  bf16x8 a[16];
  const int tg = min(t0 + lr, rows - 1);  // rows past the end: a real row, not stored
  const int col = h * MLA_D_V + 16 * (wave & 7) + 4 * lg;
  int len = 0;
  u32x2 gv = u32x2{0, 0};
  if (mfma_wave) {
    load_w_frags<FMT>(w_uv, w_head, w_v, w_scale, ws_head, ws_v, h, 16 * wave + lr, lg, a);
    len = lengths[tg / qlen];
    gv = *reinterpret_cast<const u32x2*>(gate + tg * g_row + col);
  }

  // merge row w of the block (a row past the end merges a copy of a real
  // row and is stored as zeros)
  {
    const int r = t0 + wave;
    const int rr = min(r, rows - 1);
    const float* lp[1] = {lse_part + (int64_t)rr * ls_row + (int64_t)h * ls_head};
    const uint16_t* base[1] = {o_part + (int64_t)rr * os_row + (int64_t)h * os_head + lane * 8};
    u32x4 o[1];
    float total[1], l1[1];
    merge_lse_load<1>(lp, ls_split, num_splits, lane, l1);
    if (num_splits <= 64)
      merge_rows<1, true>(lp, base, ls_split, os_split, num_splits, lane, l1, o, total);
    else
      merge_rows<1>(lp, base, ls_split, os_split, num_splits, lane, l1, o, total);
    const bool live = r < rows;
    *reinterpret_cast<u32x4*>(&lat[wave * MV_PITCH + 8 * lane]) = live ? o[0] : u32x4{0, 0, 0, 0};
    if (lse != nullptr && live && lane == 0) lse[(int64_t)r * l_row + (int64_t)h * l_head] = total[0];
  }
  __syncthreads();
  if (!mfma_wave) return;

  f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(&lat[lr * MV_PITCH + 32 * s + 8 * lg]);
    acc = mfma16(a[s], b, acc);
  }
  const int t = t0 + lr;
  if (t < rows) *reinterpret_cast<u32x2*>(out + (int64_t)t * out_row + col) = gate_out(acc, gv, len);
}

}  // namespace mla

extern "C" int mla_merge_value_gate(const uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                                    const float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                                    int32_t num_splits, int32_t w_format, const void* w_uv, int64_t w_head,
                                    int64_t w_v, const uint8_t* w_scale, int64_t ws_head, int64_t ws_v,
                                    const uint16_t* gate, int64_t g_row, const int32_t* lengths, int32_t rows,
                                    int32_t qlen, int32_t heads, uint16_t* out, int64_t out_row, float* lse,
                                    int64_t l_row, int64_t l_head, void* stream) {
  if (rows < 0 || qlen < 1 || heads < 1 || num_splits < 1) return MLA_ERR_INVALID;
  if (rows % qlen != 0) return MLA_ERR_INVALID;
  if (rows == 0) return MLA_OK;
  if (!o_part || !lse_part || !w_uv || !gate || !lengths || !out) return MLA_ERR_INVALID;
  if (g_row < (int64_t)heads * MLA_D_V || out_row < (int64_t)heads * MLA_D_V) return MLA_ERR_INVALID;
  // 16-byte partial rows, 8-byte gate / output stores
  if ((os_split | os_row | os_head) % 8 != 0 || ((uintptr_t)o_part) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if ((g_row | out_row) % 4 != 0 || (((uintptr_t)gate) | ((uintptr_t)out)) % 8 != 0) return MLA_ERR_UNSUPPORTED;
  const int nrb = (rows + mla::MV_ROWS - 1) / mla::MV_ROWS;
  const int64_t blocks = ((int64_t)heads + 7) / 8 * 8 * nrb;  // every head slot up to a multiple of 8
  if (blocks > 0x7FFFFFFF) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (w_format == MLA_W_BF16) {
    if (w_v < MLA_D_LATENT || w_head < (int64_t)MLA_D_V * w_v) return MLA_ERR_INVALID;
    if ((w_head | w_v) % 8 != 0 || ((uintptr_t)w_uv) % 16 != 0) return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla::merge_value_kernel<MLA_W_BF16>, dim3((unsigned)blocks), dim3(mla::MV_WAVES * 64), 0, s,
                       o_part, os_split, os_row, os_head, lse_part, ls_split, ls_row, ls_head, num_splits, w_uv,
                       w_head, w_v, w_scale, ws_head, ws_v, gate, g_row, lengths, rows, qlen, heads, nrb, out,
                       out_row, lse, l_row, l_head);
  } else if (w_format == MLA_W_MXFP4) {
    if (!w_scale) return MLA_ERR_INVALID;
    if (w_v < MLA_D_LATENT / 2 || w_head < (int64_t)MLA_D_V * w_v) return MLA_ERR_INVALID;
    if (ws_v < MLA_D_LATENT / 32 || ws_head < (int64_t)MLA_D_V * ws_v) return MLA_ERR_INVALID;
    if ((w_head | w_v) % 4 != 0 || ((uintptr_t)w_uv) % 4 != 0) return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla::merge_value_kernel<MLA_W_MXFP4>, dim3((unsigned)blocks), dim3(mla::MV_WAVES * 64), 0, s,
                       o_part, os_split, os_row, os_head, lse_part, ls_split, ls_row, ls_head, num_splits, w_uv,
                       w_head, w_v, w_scale, ws_head, ws_v, gate, g_row, lengths, rows, qlen, heads, nrb, out,
                       out_row, lse, l_row, l_head);
  } else {
    return MLA_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
