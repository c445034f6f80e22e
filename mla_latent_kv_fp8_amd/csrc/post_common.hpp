// Device code of the steps after the partial attention: the LSE merge of
// the split partials, and the W_UV fragments and gate epilogue of the value
// projection.
#pragma once

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

// LSE merge of R (row, head) latent rows by one wave, the rows in lockstep
// so that their loads are in flight together.  lp[r] points at row r's split
// LSEs (stride ls_split), base[r] at its split-0 latent row (stride
// os_split).  Lane l produces latent columns 8l..8l+7 as bf16 pairs in
// out[r]; total[r] is the merged LSE.
//   m = max_k lse_k (a NaN propagates);  total = m + ln sum_{lse_k > -inf} e^(lse_k - m)
//   o = bf16( sum_{lse_k > -inf} e^(lse_k - total) * o_k ),  accumulated in
//   ascending k, four splits per step
// A row with every split empty gives o = 0 and total = -inf; its latent rows
// are never read.
// Up to 64 splits (the common case) each lane's LSE is loaded once, by
// merge_lse_load, and kept in a register; beyond that merge_rows re-reads
// the LSEs in every pass.  ONE = true asserts at most 64 splits: that
// variant has no loads before the latent rows', so a caller's loads issued
// after merge_lse_load are not waited for until then.
// The *_at forms take the split loads as functors: lse_at(r, k) loads row
// r's split-k LSE, o_at(r, k) this lane's 8 columns (16 bytes) of its split-k
// latent row; the strided forms below read the usual [split][row] layout.
template <int R, class LA>
__device__ __forceinline__ void merge_lse_load_at(LA lse_at, int num_splits, int lane, float (&l1)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) l1[r] = num_splits <= 64 && lane < num_splits ? lse_at(r, lane) : -INFINITY;
}

template <int R, bool ONE, class LA, class OA>
__device__ __forceinline__ void merge_rows_at(LA lse_at, OA o_at, int num_splits, int lane, const float (&l1)[R],
                                              u32x4 (&out)[R], float (&total)[R]) {
  float m[R], s[R], acc[R][8];
  const bool one_pass = ONE || num_splits <= 64;
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = one_pass ? l1[r] : -INFINITY;
  if (!one_pass) {
    for (int k = lane; k < num_splits; k += 64) {
#pragma unroll
      for (int r = 0; r < R; ++r) m[r] = nan_max(m[r], lse_at(r, k));
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = wave_reduce(m[r], [](float a, float b) { return nan_max(a, b); });
    s[r] = 0.0f;
  }
  for (int k = lane; k < num_splits; k += 64) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float l = one_pass ? l1[r] : lse_at(r, k);
      if (l != -INFINITY) s[r] += expf(l - m[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    s[r] = wave_reduce(s[r], [](float a, float b) { return a + b; });
    // every split empty: m = -inf, s = 0, total = -inf and nothing is live
    total[r] = m[r] == -INFINITY ? -INFINITY : m[r] + logf(s[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  }
  for (int k0 = 0; k0 < num_splits; k0 += 64) {
    const int k = k0 + lane;
    float w[R];
    uint64_t live[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float l = one_pass ? l1[r] : (k < num_splits ? lse_at(r, k) : -INFINITY);
      w[r] = expf(l - total[r]);  // NaN if poisoned (a live split's weight)
      live[r] = __ballot(l != -INFINITY);
    }
    bool any = false;
#pragma unroll
    for (int r = 0; r < R; ++r) any |= live[r] != 0;
    while (any) {
      // up to four live splits of every row: all loads first, then the sums
      int ks[R][4];
      u32x4 v[R][4];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ks[r][j] = live[r] ? __builtin_ctzll(live[r]) : -1;
          if (live[r]) live[r] &= live[r] - 1;
        }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (ks[r][j] >= 0) v[r][j] = o_at(r, k0 + ks[r][j]);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ks[r][j] < 0) continue;
          const float wj = __shfl(w[r], ks[r][j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[r][2 * e] += wj * __uint_as_float(v[r][j][e] << 16);
            acc[r][2 * e + 1] += wj * __uint_as_float(v[r][j][e] & 0xFFFF0000u);
          }
        }
      any = false;
#pragma unroll
      for (int r = 0; r < R; ++r) any |= live[r] != 0;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) out[r][e] = pack_bf16x2(acc[r][2 * e], acc[r][2 * e + 1]);
}

template <int R>
__device__ __forceinline__ void merge_lse_load(const float* const* lp, int64_t ls_split, int num_splits, int lane,
                                               float (&l1)[R]) {
  merge_lse_load_at<R>([&](int r, int k) { return lp[r][k * ls_split]; }, num_splits, lane, l1);
}

template <int R, bool ONE = false>
__device__ __forceinline__ void merge_rows(const float* const* lp, const uint16_t* const* base, int64_t ls_split,
                                           int64_t os_split, int num_splits, int lane, const float (&l1)[R],
                                           u32x4 (&out)[R], float (&total)[R]) {
  merge_rows_at<R, ONE>([&](int r, int k) { return lp[r][k * ls_split]; },
                        [&](int r, int k) { return *reinterpret_cast<const u32x4*>(base[r] + (int64_t)k * os_split); },
                        num_splits, lane, l1, out,
                        total);
}

// W_UV fragments of all 16 K-steps for output row v of head h: lane group lg
// holds latents 32s + 8lg .. +7 of K-step s (the A operand of C[v][t]).
template <int FMT>
__device__ __forceinline__ void load_w_frags(const void* w_uv, int64_t w_head, int64_t w_v, const uint8_t* w_scale,
                                             int64_t ws_head, int64_t ws_v, int h, int v, int lg, bf16x8 (&a)[16]) {
  if (FMT == MLA_W_BF16) {
    const uint16_t* wp = reinterpret_cast<const uint16_t*>(w_uv) + h * w_head + v * w_v + 8 * lg;
#pragma unroll
    for (int s = 0; s < 16; ++s) a[s] = *reinterpret_cast<const bf16x8*>(wp + 32 * s);
  } else {
    const uint8_t* wp = reinterpret_cast<const uint8_t*>(w_uv) + h * w_head + v * w_v + 4 * lg;
    const uint8_t* sp = w_scale + h * ws_head + v * ws_v;
    uint32_t codes[16];
    u32x4 sc4[4];
#pragma unroll
    for (int s = 0; s < 16; ++s) codes[s] = *reinterpret_cast<const uint32_t*>(wp + 16 * s);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc4[i] = u32x4{sp[4 * i], sp[4 * i + 1], sp[4 * i + 2], sp[4 * i + 3]};
#pragma unroll
    for (int s = 0; s < 16; ++s) a[s] = fp4x8_to_bf16x8(codes[s], e8m0_to_f32(sc4[s >> 2][s & 3]));
  }
}

// Gate epilogue for one lane's four outputs (C rows 4lg..4lg+3):
// len > 0 ? bf16(f32(bf16(acc)) * sigma_f32(f32(g))) : +0 (a NaN gate or
// value of an empty request's row is not propagated).
__device__ __forceinline__ u32x2 gate_out(const f32x4& acc, const u32x2& gv, int len) {
  if (len <= 0) return u32x2{0, 0};
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float val = bf16_bits_to_f32(f32_to_bf16_bits(acc[i]));
    const uint32_t gb = (i & 1) ? (gv[i >> 1] >> 16) : (gv[i >> 1] & 0xFFFFu);
    const float gl = bf16_bits_to_f32(gb);
    const float sig = 1.0f / (1.0f + expf(-gl));
    o[i] = val * sig;
  }
  return u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

}  // namespace mla
