// Split-KV partial attention of absorbed queries over a paged fp8 E4M3
// latent cache (the decode partials of the runtime's `attend` /
// `m1c_inputs`: o [splits, S, H, 512] bf16 and LSE [splits, S, H] f32).
//
// Design (gfx950, wave64, one 256-thread workgroup per CU):
//  * Work: the KV token stream is cut into `chunk`-token units; worker u
//    processes the pieces of unit u (token balanced), for one block of
//    16*NRG <= 48 query rows (rows = (qlen position, head) pairs of a
//    request; more rows take more blocks, which share the tile through L2).
//    All rows of a request share the same cache rows, so one staged tile
//    feeds every head: QK and PV are dense MFMA contractions.
//  * Per 64-token tile: the gathered fp8 rows (576 B each) are staged once in
//    LDS in swizzled 1 KB blocks of 16 tokens x 64 bytes, by asynchronous
//    global->LDS loads into a double buffer (tile i+1 streams in while tile
//    i is computed); the cache indices of a piece are staged in LDS first
//    (2048 at a time).
//  * QK on 16x16x32 bf16 MFMAs as S^T = K . Q^T: A = 16 tokens x 32 dims of
//    the staged tile (fp8 -> bf16 in registers), B = Q^T held in registers
//    for the whole piece.  Wave w owns token quarter w of every tile for all
//    row groups, so each staged byte is converted to bf16 once per block.
//  * Softmax: base-2 online softmax with a lazy reference max (rescale only
//    when the running max grows by more than 2^8); per-tile row maxima are
//    exchanged through LDS so every wave uses the same reference.
//  * PV as O^T = V^T . P^T: wave w owns latent columns [128w, 128w+128).
//    The A operand (8 tokens of one column) comes straight from the
//    staged tile with ds_read_b64_tr_b8; the B operand is P^T, written to
//    LDS by the S-tile owners directly in MFMA operand order (the S^T
//    accumulator layout gives each lane 4 consecutive tokens, so the PV
//    contraction uses the matching token permutation).
#include "common.hpp"

namespace mla {

constexpr int NT = 64;             // tokens per tile
constexpr int TILE_BYTES = 36864;  // one staged tile: 36 blocks of 1 KB
constexpr float kLazy = 8.0f;  // rescale threshold, log2 units

struct PartialArgs {
  const uint16_t* q;
  int64_t q_sr, q_sh;
  int32_t batch, qlen, heads, M, n_rb;
  const uint8_t* kv;
  int64_t num_slots;
  const int32_t* indptr;
  const int32_t* indices;
  float c_log2;  // sm_scale * kv_scale * log2(e)
  float kv_scale;
  int32_t num_splits, num_workers, split_min;
  uint16_t* o;
  int64_t os_s, os_r, os_h;
  float* lse;
  int64_t ls_s, ls_r, ls_h;
};

// LDS layout of a staged tile (64 tokens x 36 chunks of 16 B): block
// (t/16, c/4) of 1 KB holds 16 tokens x 4 chunks; inside it, chunk c of
// token t sits at 16-B slot 4*(t%16) + ((c%4) ^ h(t)).  With 32 banks the
// QK fragment read (8 consecutive tokens, one chunk) and the transposed V
// read (tokens {4G..4G+3} and {16+4G..16+4G+3}, one chunk) both hit 8
// distinct 16-byte bank groups.
__device__ __forceinline__ int hsw(int t) { return ((t >> 1) & 3) ^ (((t >> 4) & 1) << 1); }
__device__ __forceinline__ int tile_off(int t, int c) {
  return 16 * (64 * (9 * (t >> 4) + (c >> 2)) + 4 * (t & 15) + ((c & 3) ^ hsw(t)));
}

// Query fragments of one 16-row group: K-step 2p uses dims 64p+16g..+7 and
// K-step 2p+1 dims 64p+16g+8..+15 for lane group g (the same permutation
// the K fragments use), so each lane loads 32 contiguous bytes per p.
__device__ __forceinline__ void load_q(const PartialArgs& p, int r, int m, int lg, bf16x8 (&qf)[18]) {
  if (m < p.M) {
    const int j = m / p.heads, h = m % p.heads;
    const uint16_t* src = p.q + (int64_t)(r * p.qlen + j) * p.q_sr + (int64_t)h * p.q_sh + 16 * lg;
#pragma unroll
    for (int pp = 0; pp < 9; ++pp) {
      qf[2 * pp] = *reinterpret_cast<const bf16x8*>(src + 64 * pp);
      qf[2 * pp + 1] = *reinterpret_cast<const bf16x8*>(src + 64 * pp + 8);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 18; ++s) qf[s] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// K fragment pair of (quarter qq, p): 16 bytes of token 16qq + lr at chunk
// 4p + lg -> bf16 for K-steps 2p (lo) and 2p+1 (hi).  The 64 lanes read one
// whole 1 KB block.
__device__ __forceinline__ void load_k(const MLA_LDS uint8_t* kt, int qq, int pp, int lr, int lg,
                                       bf16x8& lo, bf16x8& hi) {
  const int t = 16 * qq + lr;
  const u32x4 raw = *(const MLA_LDS u32x4*)(kt + tile_off(t, 4 * pp + lg));
  lo = fp8x8_to_bf16x8(u32x2{raw[0], raw[1]});
  hi = fp8x8_to_bf16x8(u32x2{raw[2], raw[3]});
}

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// LDS byte address lds_base + 16*l.  Issued through inline assembly so that
// the compiler does not make later LDS reads (of the other buffer) wait for
// it; the kernel waits for these loads itself (vmcnt) before the barrier
// that publishes a tile.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const uint8_t* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issue the direct global->LDS loads of one 64-token tile.  Wave w loads the
// 16 tokens of quarter w: load instruction cg fills block (w, cg), lane l
// carrying token 16w + l/4, chunk 4cg + ((l%4) ^ h(t)).  Tokens past the
// tile end and tokens with an invalid index load `safe_row` (masked, or
// poisoned through the score).
__device__ __forceinline__ void issue_tile(const uint8_t* kv, const MLA_LDS int32_t* idx_lds, int ntok,
                                           int safe_row, MLA_LDS uint8_t* dst, int wave, int lane) {
  const int t = 16 * wave + (lane >> 2);
  int row = t < ntok ? idx_lds[t] : -1;
  row = row < 0 ? safe_row : row;
  const uint8_t* src = kv + (int64_t)row * MLA_D_QK + 16 * ((lane & 3) ^ hsw(t));
  const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + 1024 * 9 * wave));
#pragma unroll
  for (int cg = 0; cg < 9; ++cg) lds_dma16(src + 64 * cg, d + 1024 * cg);
}

constexpr int IDX_CAP = 2048;  // tokens whose cache indices are staged at once

template <int NRG>
__global__ void __launch_bounds__(256, 1) partial_kernel(PartialArgs p) {
  constexpr int RB = 16 * NRG;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf_[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t pt[2 * NRG * 64 * 8];
  __shared__ __attribute__((aligned(16))) float redmax[RB * 4];
  __shared__ __attribute__((aligned(16))) float redsum[RB * 4];
  __shared__ __attribute__((aligned(16))) int32_t idx[IDX_CAP];
  __shared__ int32_t red_i[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  MLA_LDS uint8_t* kbuf = (MLA_LDS uint8_t*)kbuf_;
  MLA_LDS int32_t* idxl = (MLA_LDS int32_t*)idx;

  // ---- block -> (worker, row block); the row blocks of a worker share an
  // XCD (and its L2), workers interleave across the 8 XCDs
  int u, rb;
  {
    const int bid = blockIdx.x;
    if (p.num_workers % 8 == 0) {
      const int slot = bid >> 3;
      u = (bid & 7) + 8 * (slot / p.n_rb);
      rb = slot % p.n_rb;
    } else {
      u = bid / p.n_rb;
      rb = bid % p.n_rb;
    }
  }

  // ---- the split partition: T, L_max -> chunk
  int lmax = 0;
  for (int r = tid; r < p.batch; r += 256) lmax = max(lmax, p.indptr[r + 1] - p.indptr[r]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) lmax = max(lmax, __shfl_xor(lmax, s));
  if (lane == 0) red_i[wave] = lmax;
  __syncthreads();
  lmax = max(max(red_i[0], red_i[1]), max(red_i[2], red_i[3]));
  const int base = p.indptr[0];
  const int64_t T = (int64_t)p.indptr[p.batch] - base;
  const int64_t chunk = split_chunk(T, lmax, p.num_splits, p.num_workers, p.split_min);
  const int64_t nunits = T > 0 ? (T + chunk - 1) / chunk : 1;
  if (u >= nunits) return;
  const int64_t g0 = (int64_t)u * chunk;
  const int64_t g1 = g0 + chunk < T ? g0 + chunk : T;
  const bool last_unit = (u == nunits - 1);
  const int m_lo = rb * RB;  // first row (of the request's qlen*heads) of this block

  // first request whose stream end is >= g0
  int r;
  {
    int lo = 0, hi = p.batch;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if ((int64_t)p.indptr[mid + 1] - base >= g0) hi = mid; else lo = mid + 1;
    }
    r = lo;
  }

  auto fill_neginf = [&](int req, int k_from) {
    // LSE = -inf for splits [k_from, num_splits) of every row of this block
    const int nrows = min(RB, p.M - m_lo);
    const int n = (p.num_splits - k_from) * nrows;
    for (int i = tid; i < n; i += 256) {
      const int k = k_from + i / nrows, m = m_lo + i % nrows;
      const int t = req * p.qlen + m / p.heads, h = m % p.heads;
      p.lse[k * p.ls_s + (int64_t)t * p.ls_r + (int64_t)h * p.ls_h] = -INFINITY;
    }
  };

  for (; r < p.batch; ++r) {
    const int64_t P = (int64_t)p.indptr[r] - base;
    const int L = p.indptr[r + 1] - p.indptr[r];
    if (P >= g1 && !(last_unit && P == T)) break;
    if (L == 0) {
      const int64_t owner = P / chunk < nunits - 1 ? P / chunk : nunits - 1;
      if (owner == u) fill_neginf(r, 0);
      continue;
    }
    const int a = (int)((g0 > P ? g0 : P) - P);
    const int b = (int)((g1 < P + L ? g1 : P + L) - P);
    if (b <= a) continue;
    const int k = (a == 0) ? 0 : (int)((P + a) / chunk - P / chunk);
    if (k == 0) {
      const int nsplit = (int)((P + L - 1) / chunk - P / chunk + 1);
      if (nsplit < p.num_splits) fill_neginf(r, nsplit);
    }

    // ---------------------------------------------------------- one piece
    // wave w owns token quarter w of every tile, for all NRG row groups
    bf16x8 qf[NRG][18];
    int lim[NRG];  // visible tokens of row (g, lr), as an end in request tokens
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const int m = m_lo + 16 * g + lr;
      load_q(p, r, m, lg, qf[g]);
      const int vis = m < p.M ? L - p.qlen + m / p.heads + 1 : 0;
      lim[g] = min(b, vis);
    }

    f32x4 O[8][NRG];
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int g = 0; g < NRG; ++g) O[d][g] = f32x4{0, 0, 0, 0};
    float mref[NRG], lsum[NRG];
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      mref[g] = -INFINITY;
      lsum[g] = 0.0f;
    }
    const int32_t* rows_r = p.indices + p.indptr[r];

    for (int s0 = a; s0 < b; s0 += IDX_CAP) {
      // ---- stage this segment's cache indices (invalid -> -1)
      const int slen = min(IDX_CAP, b - s0);
      __syncthreads();  // the previous segment's tiles are done with idx
      {
        int rowv[IDX_CAP / 256];
#pragma unroll
        for (int j = 0; j < IDX_CAP / 256; ++j) {
          const int i = tid + 256 * j;
          rowv[j] = i < slen ? rows_r[s0 + i] : -1;
        }
#pragma unroll
        for (int j = 0; j < IDX_CAP / 256; ++j) {
          const int i = tid + 256 * j;
          if (i < slen) idx[i] = (uint32_t)rowv[j] < (uint64_t)p.num_slots ? rowv[j] : -1;
        }
      }
      __syncthreads();
      int safe_row = 0;  // a valid row of this segment, for padding loads
      {
        int v = idx[0];
        if (v < 0) {
          for (int i = 1; i < slen; ++i)
            if (idx[i] >= 0) { v = idx[i]; break; }
        }
        safe_row = v < 0 ? 0 : v;
      }
      const int ntiles = (slen + NT - 1) / NT;
      issue_tile(p.kv, idxl, min(NT, slen), safe_row, kbuf, wave, lane);

      for (int it = 0; it < ntiles; ++it) {
        const int t0 = s0 + NT * it;
        MLA_LDS uint8_t* kt = kbuf + (it & 1) * TILE_BYTES;
        wait_vm_all();                   // this wave's loads of tile `it` have landed
        __syncthreads();                 // ... and every wave's; PV(it-1) is done
        if (it + 1 < ntiles)
          issue_tile(p.kv, idxl + NT * (it + 1), min(NT, slen - NT * (it + 1)), safe_row,
                     kbuf + ((it + 1) & 1) * TILE_BYTES, wave, lane);

        // ---- QK: S^T (quarter `wave`, row group g) over the 576 dims
        f32x4 S[NRG];
#pragma unroll
        for (int g = 0; g < NRG; ++g) S[g] = f32x4{0, 0, 0, 0};
        {
          // K fragments read one step ahead of their use
          const int tq = 16 * wave + lr;
          u32x4 raw[2];
          raw[0] = *(const MLA_LDS u32x4*)(kt + tile_off(tq, lg));
#pragma unroll
          for (int pp = 0; pp < 9; ++pp) {
            if (pp + 1 < 9) raw[(pp + 1) & 1] = *(const MLA_LDS u32x4*)(kt + tile_off(tq, 4 * (pp + 1) + lg));
            const u32x4 cur = raw[pp & 1];
            const bf16x8 klo = fp8x8_to_bf16x8(u32x2{cur[0], cur[1]});
            const bf16x8 khi = fp8x8_to_bf16x8(u32x2{cur[2], cur[3]});
#pragma unroll
            for (int g = 0; g < NRG; ++g) {
              S[g] = mfma16(klo, qf[g][2 * pp], S[g]);
              S[g] = mfma16(khi, qf[g][2 * pp + 1], S[g]);
            }
          }
        }

        // ---- scale, mask (an invalid index poisons with NaN), per-(row, quarter) max
        const int32_t* ti = idx + NT * it + 16 * wave + 4 * lg;
        bool bad[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bad[e] = ti[e] < 0;
#pragma unroll
        for (int g = 0; g < NRG; ++g) {
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = t0 + 16 * wave + 4 * lg + e;
            float x = tok < lim[g] ? S[g][e] * p.c_log2 : -INFINITY;
            if (bad[e] && tok < lim[g]) x = __builtin_nanf("");
            S[g][e] = x;
            mx = fmaxf(mx, x);
          }
          mx = wave_max_xor(mx, 16);
          mx = wave_max_xor(mx, 32);
          if (lg == 0) redmax[(16 * g + lr) * 4 + wave] = mx;
        }
        __syncthreads();

        // ---- reference max update (identical in every wave), rescale
        bool rescale = false;
        float alpha[NRG];
#pragma unroll
        for (int g = 0; g < NRG; ++g) {
          const f32x4 q4 = *reinterpret_cast<const f32x4*>(&redmax[(16 * g + lr) * 4]);
          const float mx = fmaxf(fmaxf(q4[0], q4[1]), fmaxf(q4[2], q4[3]));
          alpha[g] = 1.0f;
          if (mx > mref[g] + kLazy) {
            alpha[g] = __builtin_amdgcn_exp2f(mref[g] - mx);
            mref[g] = mx;
            rescale = true;
          }
          lsum[g] *= alpha[g];
        }
        if (__any(rescale)) {
#pragma unroll
          for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int g = 0; g < NRG; ++g) O[d][g] *= alpha[g];
        }

        // ---- P = exp2(x - mref) -> bf16 P^T fragments in LDS; row sums in f32
        // (the PV contraction slot of lane-group G, element e is token
        // 32*(quarter/2) + 16*(quarter%2) + 4G + e)
#pragma unroll
        for (int g = 0; g < NRG; ++g) {
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = S[g][e];
            pv[e] = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - mref[g]);
            lsum[g] += pv[e];
          }
          *reinterpret_cast<u32x2*>(&pt[(((wave >> 1) * NRG + g) * 64 + lane) * 8 + 4 * (wave & 1)]) =
              u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        }
        __syncthreads();

        // ---- PV: O^T[128w + 16d .., rows] += V^T . P^T
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
          // transposed V operand: source lane s of group G points at token
          // slot (G, s/2), columns 16*chunk + 8*(s&1)
          const int s2 = lr >> 1;
          const int tt = 32 * kap + (s2 < 4 ? 4 * lg + s2 : 16 + 4 * lg + s2 - 4);
          const MLA_LDS uint8_t* vrow = kt + 8 * (lr & 1);
          i32x2 vraw[8];
#pragma unroll
          for (int d = 0; d < 8; ++d)
            vraw[d] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(vrow + tile_off(tt, 8 * wave + d)));
          bf16x8 pf[NRG];
#pragma unroll
          for (int g = 0; g < NRG; ++g)
            pf[g] = *reinterpret_cast<const bf16x8*>(&pt[((kap * NRG + g) * 64 + lane) * 8]);
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            const bf16x8 vf = fp8x8_to_bf16x8(u32x2{(uint32_t)vraw[d][0], (uint32_t)vraw[d][1]});
#pragma unroll
            for (int g = 0; g < NRG; ++g) O[d][g] = mfma16(vf, pf[g], O[d][g]);
          }
        }
      }
    }

    // ---------------------------------------------------- piece epilogue
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      float l = lsum[g];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      if (lg == 0) redsum[(16 * g + lr) * 4 + wave] = l;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(&redsum[(16 * g + lr) * 4]);
      const float l = ((s4[0] + s4[1]) + s4[2]) + s4[3];
      const int m = m_lo + 16 * g + lr;
      if (m >= p.M) continue;
      const int t = r * p.qlen + m / p.heads, h = m % p.heads;
      // l == 0: no visible token in this split.  A NaN l (NaN cache bytes or
      // an invalid index) is written through, so it poisons the row.
      if (l != 0.0f) {
        const float inv = p.kv_scale / l;
        uint16_t* orow =
            p.o + k * p.os_s + (int64_t)t * p.os_r + (int64_t)h * p.os_h + 128 * wave + 4 * lg;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const f32x4 v = O[d][g];
          *reinterpret_cast<u32x2*>(orow + 16 * d) =
              u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
        }
      }
      if (wave == 0 && lg == 0)
        p.lse[k * p.ls_s + (int64_t)t * p.ls_r + (int64_t)h * p.ls_h] =
            l != 0.0f ? (mref[g] + __log2f(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();
  }
}

template <int NRG>
static int launch(const PartialArgs& a, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(partial_kernel<NRG>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla

extern "C" int mla_split_plan(const int32_t* indptr, int32_t batch, int32_t num_splits,
                              int32_t num_workers, int32_t split_min_tokens, int32_t* bounds,
                              int64_t* chunk_out) {
  if (!indptr || !bounds || batch < 0 || num_splits < 1 || num_workers < 1) return MLA_ERR_INVALID;
  int64_t T = (int64_t)indptr[batch] - indptr[0], lmax = 0;
  for (int r = 0; r < batch; ++r) {
    int64_t L = (int64_t)indptr[r + 1] - indptr[r];
    if (L < 0) return MLA_ERR_INVALID;
    if (L > lmax) lmax = L;
  }
  const int64_t chunk = mla::split_chunk(T, lmax, num_splits, num_workers, split_min_tokens);
  for (int r = 0; r < batch; ++r) {
    const int64_t P = (int64_t)indptr[r] - indptr[0], L = (int64_t)indptr[r + 1] - indptr[r];
    int32_t* b = bounds + (int64_t)r * (num_splits + 1);
    int k = 0;
    b[k++] = 0;
    for (int64_t c = (P / chunk + 1) * chunk; c < P + L; c += chunk) {
      if (k >= num_splits) return MLA_ERR_INVALID;
      b[k++] = (int32_t)(c - P);
    }
    while (k <= num_splits) b[k++] = (int32_t)L;
  }
  if (chunk_out) *chunk_out = chunk;
  return MLA_OK;
}

extern "C" int mla_decode_partial(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                                  int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                                  int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                                  float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                                  int32_t split_min_tokens, uint16_t* o_part, int64_t os_split,
                                  int64_t os_row, int64_t os_head, float* lse_part, int64_t ls_split,
                                  int64_t ls_row, int64_t ls_head, void* stream) {
  if (batch < 0 || qlen < 1 || heads < 1 || num_splits < 1 || num_splits > 1024 || num_workers < 1)
    return MLA_ERR_INVALID;
  if (batch == 0) return MLA_OK;
  if (!q || !kv_cache || !kv_indptr || !kv_indices || !o_part || !lse_part) return MLA_ERR_INVALID;
  if (num_slots < 1 || num_slots > 0x7FFFFFFFLL) return MLA_ERR_INVALID;
  if (!(kv_scale > 0.0f) || !(sm_scale > 0.0f)) return MLA_ERR_INVALID;
  // 16-byte query fragments, 8-byte partial stores, 16-byte cache rows
  if ((q_stride_row | q_stride_head) % 8 != 0 || ((uintptr_t)q) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if ((os_split | os_row | os_head) % 4 != 0 || ((uintptr_t)o_part) % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if (((uintptr_t)kv_cache) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)qlen * heads;
  if (M > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  // rows per block: 16, 32 or 48 (larger requests take several blocks)
  const int nrg = M <= 16 ? 1 : (M <= 32 ? 2 : 3);
  const int n_rb = (int)((M + 16 * nrg - 1) / (16 * nrg));
  const int64_t blocks = (int64_t)num_workers * n_rb;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_UNSUPPORTED;

  mla::PartialArgs a;
  a.q = q; a.q_sr = q_stride_row; a.q_sh = q_stride_head;
  a.batch = batch; a.qlen = qlen; a.heads = heads; a.M = (int32_t)M; a.n_rb = n_rb;
  a.kv = kv_cache; a.num_slots = num_slots; a.indptr = kv_indptr; a.indices = kv_indices;
  a.c_log2 = sm_scale * kv_scale * mla::kLog2e;
  a.kv_scale = kv_scale;
  a.num_splits = num_splits; a.num_workers = num_workers; a.split_min = split_min_tokens;
  a.o = o_part; a.os_s = os_split; a.os_r = os_row; a.os_h = os_head;
  a.lse = lse_part; a.ls_s = ls_split; a.ls_r = ls_row; a.ls_h = ls_head;
  hipStream_t s = (hipStream_t)stream;
  switch (nrg) {
    case 1: return mla::launch<1>(a, (int)blocks, s);
    case 2: return mla::launch<2>(a, (int)blocks, s);
    default: return mla::launch<3>(a, (int)blocks, s);
  }
}
