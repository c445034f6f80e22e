// W_UV value projection fused with the gate epilogue (the value step of the
// decode runtime's `post`; the gate rule of the CuTe-DSL value page, classes
// MlaValue and MlaGate):  out = len_r > 0 ? bf16(f32(bf16(acc)) * sigma_f32(g))
// : +0, with acc = sum_l latent[l] * W[v][l].
#include "post_common.hpp"

namespace mla {

constexpr int VG_ROWS = 64;            // rows per workgroup (fewer rows re-read W more often)
constexpr int VG_RG = VG_ROWS / 16;    // 16-row groups (MFMA N tiles) per workgroup
constexpr int VG_LD = VG_ROWS / 4;     // 16-B latent loads per thread
constexpr int VG_PITCH = 512 + 8;      // LDS row pitch in bf16 (1040 B: conflict-free b128 reads)

// Workgroup = (row block of VG_ROWS, head, half of the 128 outputs).  Wave w
// computes outputs v in [64*half + 16w, +16) for all rows of the block as
// C[v][t] = W[h][v][:] . latent[t][h][:] on 16x16x32 bf16 MFMAs.  Each
// lane prefetches its W fragments for all 16 K-steps up front (every W
// element is read once); the latent block is staged once in LDS and read as
// the B operand.
template <int FMT>
__global__ void __launch_bounds__(256) value_gate_kernel(
    const uint16_t* __restrict__ latent, int64_t l_row, int64_t l_head, const void* __restrict__ w_uv,
    int64_t w_head, int64_t w_v, const uint8_t* __restrict__ w_scale, int64_t ws_head, int64_t ws_v,
    const uint16_t* __restrict__ gate, int64_t g_row, const int32_t* __restrict__ lengths,
    int32_t rows, int32_t qlen, uint16_t* __restrict__ out, int64_t out_row) {
  __shared__ __attribute__((aligned(16))) uint16_t lat[VG_ROWS * VG_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * VG_ROWS;
  const int lr = lane & 15, lg = lane >> 4;
  const int v = 64 * blockIdx.z + 16 * wave + lr;  // the A-operand row of this lane

  // W fragments of all 16 K-steps (lane: output v, latents 32s + 8lg .. +7)
  bf16x8 a[16];
  load_w_frags<FMT>(w_uv, w_head, w_v, w_scale, ws_head, ws_v, h, v, lg, a);

  // stage the latent block (VG_ROWS rows x 64 chunks of 16 B) with all loads in
  // flight at once; the epilogue's gate values and row lengths are fetched
  // here too, so their latency hides behind the staging and the MFMAs
  {
    u32x4 x[VG_LD];
#pragma unroll
    for (int i = 0; i < VG_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 6, part = c & 63;
      x[i] = u32x4{0, 0, 0, 0};
      if (t0 + r < rows)
        x[i] = *reinterpret_cast<const u32x4*>(latent + (int64_t)(t0 + r) * l_row + h * l_head + part * 8);
    }
#pragma unroll
    for (int i = 0; i < VG_LD; ++i) {
      const int c = tid + 256 * i, r = c >> 6, part = c & 63;
      *reinterpret_cast<u32x4*>(&lat[r * VG_PITCH + part * 8]) = x[i];
    }
  }
  const int col = h * MLA_D_V + 64 * blockIdx.z + 16 * wave + 4 * lg;
  u32x2 gv[VG_RG];
  int len[VG_RG];
#pragma unroll
  for (int rg = 0; rg < VG_RG; ++rg) {
    const int t = min(t0 + 16 * rg + lr, rows - 1);  // rows past the end: a real row, not stored
    len[rg] = lengths[t / qlen];
    gv[rg] = *reinterpret_cast<const u32x2*>(gate + t * g_row + col);
  }
  __syncthreads();

  f32x4 acc[VG_RG];
#pragma unroll
  for (int rg = 0; rg < VG_RG; ++rg) acc[rg] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
#pragma unroll
    for (int rg = 0; rg < VG_RG; ++rg) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&lat[(16 * rg + lr) * VG_PITCH + 32 * s + 8 * lg]);
      acc[rg] = mfma16(a[s], b, acc[rg]);
    }
  }

  // epilogue: lane holds v = 64*half + 16w + 4lg + i for row t = t0 + 16rg + lr
#pragma unroll
  for (int rg = 0; rg < VG_RG; ++rg) {
    const int t = t0 + 16 * rg + lr;
    if (t >= rows) continue;
    *reinterpret_cast<u32x2*>(out + t * out_row + col) = gate_out(acc[rg], gv[rg], len[rg]);
  }
}

}  // namespace mla

extern "C" int mla_value_gate(const uint16_t* latent, int64_t l_row, int64_t l_head, int32_t w_format,
                              const void* w_uv, int64_t w_head, int64_t w_v, const uint8_t* w_scale,
                              int64_t ws_head, int64_t ws_v, const uint16_t* gate, int64_t g_row,
                              const int32_t* lengths, int32_t rows, int32_t qlen, int32_t heads,
                              uint16_t* out, int64_t out_row, void* stream) {
  if (rows < 0 || qlen < 1 || heads < 1) return MLA_ERR_INVALID;
  if (rows % qlen != 0) return MLA_ERR_INVALID;
  if (rows == 0) return MLA_OK;
  if (!latent || !w_uv || !gate || !lengths || !out) return MLA_ERR_INVALID;
  if (g_row < (int64_t)heads * MLA_D_V || out_row < (int64_t)heads * MLA_D_V) return MLA_ERR_INVALID;
  if ((l_row | l_head) % 8 != 0 || ((uintptr_t)latent) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if ((g_row | out_row) % 4 != 0 || (((uintptr_t)gate) | ((uintptr_t)out)) % 8 != 0)
    return MLA_ERR_UNSUPPORTED;
  dim3 grid((unsigned)((rows + mla::VG_ROWS - 1) / mla::VG_ROWS), (unsigned)heads, 2);
  hipStream_t s = (hipStream_t)stream;
  if (w_format == MLA_W_BF16) {
    if (w_v < MLA_D_LATENT || w_head < (int64_t)MLA_D_V * w_v) return MLA_ERR_INVALID;
    if ((w_head | w_v) % 8 != 0 || ((uintptr_t)w_uv) % 16 != 0) return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla::value_gate_kernel<MLA_W_BF16>, grid, dim3(256), 0, s, latent, l_row, l_head,
                       w_uv, w_head, w_v, w_scale, ws_head, ws_v, gate, g_row, lengths, rows, qlen, out,
                       out_row);
  } else if (w_format == MLA_W_MXFP4) {
    if (!w_scale) return MLA_ERR_INVALID;
    if (w_v < MLA_D_LATENT / 2 || w_head < (int64_t)MLA_D_V * w_v) return MLA_ERR_INVALID;
    if (ws_v < MLA_D_LATENT / 32 || ws_head < (int64_t)MLA_D_V * ws_v) return MLA_ERR_INVALID;
    if ((w_head | w_v) % 4 != 0 || ((uintptr_t)w_uv) % 4 != 0) return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla::value_gate_kernel<MLA_W_MXFP4>, grid, dim3(256), 0, s, latent, l_row, l_head,
                       w_uv, w_head, w_v, w_scale, ws_head, ws_v, gate, g_row, lengths, rows, qlen, out,
                       out_row);
  } else {
    return MLA_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
