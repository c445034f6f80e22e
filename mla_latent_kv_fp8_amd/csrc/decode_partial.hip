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
//    global->LDS loads, triple buffered (the loads of tile i+2 are issued
//    while tile i is computed).  A piece's cache indices (2048 at a time)
//    and its query rows are staged by the same direct loads; the first two
//    tiles are issued as soon as the indices have landed.
//  * QK on 16x16x32 bf16 MFMAs as S^T = K . Q^T: A = 16 tokens x 32 dims of
//    the staged tile (fp8 -> bf16 in registers), B = Q^T, loaded once per
//    piece into accumulation registers (the 48-row block too: its whole
//    query, 216 registers, with O in 96 arch registers).  Wave
//    w owns token quarter w of every tile for all row groups, so each staged
//    byte is converted to bf16 once per block.  An fp8 query skips the
//    conversion: its QK runs on the scaled 16x16x128 fp8 MFMA with K and Q
//    both E4M3 codes (exact products, f32 sums), q_scale in the score
//    constant.
//  * Softmax: base-2, P = 2^(s*c - ref) in bf16, sums in f32, with a
//    per-row reference ref that starts at 0.  Each lane keeps the running
//    maximum of its scores; at the end of a piece the four quarters' row
//    maxima are exchanged with the row sums, and a row whose maximum lies
//    more than 64 log2 units from its reference takes the maximum as its
//    reference and the piece runs again (P <= 2^64 then bounds bf16 P and
//    the f32 sums).  No tile waits for a decision about the reference, and
//    O is never rescaled.  Two barriers per tile: the first frees the
//    buffer of tile i-1 for the loads of tile i+2, which issue one per QK
//    step (so the address unit works through them while the MFMAs run); the
//    second publishes P^T.
//  * PV as O^T = V^T . P^T: wave w owns latent columns [128w, 128w+128).
//    The A operand (8 tokens of one column) comes straight from the
//    staged tile with ds_read_b64_tr_b8; the B operand is P^T, written to
//    LDS by the S-tile owners directly in MFMA operand order (the S^T
//    accumulator layout gives each lane 4 consecutive tokens, so the PV
//    contraction uses the matching token permutation).
//  * Epilogue: O is normalised into LDS as bf16 rows and written out one
//    whole 1 KB row per store instruction.
//  * The fused call (mla_decode_attend) also merges: a request of one split
//    goes straight to the merged latent; the pieces of a split request go to
//    workspace slots, and the block that completes a request's count (a
//    system-scope atomic) merges its splits with the LSE merge's own code.
#include <hip/hip_ext.h>

#include <mutex>
#include <type_traits>

#include "post_common.hpp"

namespace mla {

constexpr int NT = 64;             // tokens per tile
constexpr int TILE_BYTES = 36864;  // one staged tile: 36 blocks of 1 KB
constexpr float kLazy = 64.0f;  // restart threshold, log2 units (P <= 2^64 in bf16 / f32 sums)

struct PartialArgs {
  const uint16_t* q;   // bf16 query, or
  const uint8_t* q8;   // fp8 E4M3 query codes (the fp8-query variant)
  int64_t q_sr, q_sh;
  int32_t batch, qlen, heads, M, n_rb;
  const uint8_t* kv;
  int64_t num_slots;
  const int32_t* indptr;
  const int32_t* indices;
  float c_log2;  // sm_scale * kv_scale (* q_scale for an fp8 query) * log2(e)
  float kv_scale;
  int32_t num_splits, num_workers, split_min;
  uint16_t* o;
  int64_t os_s, os_r, os_h;
  float* lse;
  int64_t ls_s, ls_r, ls_h;
  // the fused call: the merged latent and LSE (lat_lse may be null), and the
  // workspace (counters, then the split partials by unit slot)
  uint16_t* lat;
  int64_t lat_r, lat_h;
  float* lat_lse;
  int64_t ll_r, ll_h;
  int32_t* ws_cnt;      // one counter per (request, row block)
  uint8_t* ws;          // base of the partial area
  int32_t ws_lse_off;   // byte offset of the partial LSEs [slot][RB] in ws
  int32_t ws_o_off;     // byte offset of the partial rows [slot][RB][512] bf16 in ws
};

// The cache write fused into the call (the WRITE variant; empty otherwise,
// so the plain kernel's arguments do not change).  The batch * k new
// tokens are the last k of each request: token r * k + j is request r's
// token L_r - k + j, with bf16 rows c [.][512] and pe [.][64] (16-byte
// aligned, row strides in elements) and cache slot slot[.] (skipped
// outside [0, num_slots)).  The rows go to the cache the call reads
// (PartialArgs::kv, written through cache_w): no pointer of their own, one
// scalar pair fewer for the argument reads to compete for.
template <bool WRITE>
struct NewArgs {};
template <>
struct NewArgs<true> {
  const uint16_t* c;
  const uint16_t* pe;
  int64_t c_r, pe_r;
  const int64_t* slot;
  int32_t k;
};

// the cache the fused write stores to: the one the call reads
__device__ __forceinline__ uint8_t* cache_w(const PartialArgs& p) { return const_cast<uint8_t*>(p.kv); }

// new tokens per request the fused cache write stages in LDS
constexpr int NEW_MAX = 8;

// The fused cache write for new tokens j0..j1-1 of request r that no piece
// attends (positions before the request's first token): read, encoded and
// stored straight from global memory by the first row block's workgroup.
__device__ __forceinline__ void write_new_direct(const PartialArgs& p, const NewArgs<true>& nw, int r, int j0,
                                                 int j1, int tid) {
  for (int i = tid; i < (j1 - j0) * 72; i += 256) {
    const int64_t t = (int64_t)r * nw.k + j0 + i / 72;
    const int c8 = i % 72;  // columns 8*c8 .. 8*c8+7
    const int64_t slot = nw.slot[t];
    if (slot < 0 || slot >= p.num_slots) continue;
    const uint16_t* src = c8 < 64 ? nw.c + t * nw.c_r + 8 * c8 : nw.pe + t * nw.pe_r + 8 * (c8 - 64);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
    const uint32_t w[4] = {raw[0], raw[1], raw[2], raw[3]};
    *reinterpret_cast<u32x2*>(cache_w(p) + slot * MLA_D_QK + 8 * c8) = encode_fp8x8(w, p.kv_scale);
  }
}

// The fused cache write of a piece's cnt new tokens, staged in LDS as bf16
// (latent rows of 1 KB from nraw, then a block of 128-byte rope rows) with
// their slots (two dwords each) in nslot: encoded and stored, 8 columns per
// thread and step.
__device__ __forceinline__ void store_new_rows(const PartialArgs& p, const NewArgs<true>& nw,
                                               const MLA_LDS uint8_t* nraw, const MLA_LDS int32_t* nslot, int cnt,
                                               int tid) {
  const float rscale = 1.0f / p.kv_scale;
  for (int i = tid; i < cnt * 72; i += 256) {
    const int jj = i / 72, c8 = i - 72 * jj;  // columns 8*c8 .. 8*c8+7 of staged token jj
    const int64_t slot = (int64_t)(uint32_t)nslot[2 * jj] | ((int64_t)nslot[2 * jj + 1] << 32);
    if (slot < 0 || slot >= p.num_slots) continue;
    const MLA_LDS uint8_t* src = c8 < 64 ? nraw + 1024 * jj + 16 * c8 : nraw + 1024 * NEW_MAX + 128 * jj + 16 * (c8 - 64);
    const u32x4 raw = *(const MLA_LDS u32x4*)src;
    *reinterpret_cast<u32x2*>(cache_w(p) + slot * MLA_D_QK + 8 * c8) =
        u32x2{encode_fp8x4_fast(raw[0], raw[1], p.kv_scale, rscale), encode_fp8x4_fast(raw[2], raw[3], p.kv_scale, rscale)};
  }
}

// The split partition computed on the host (the one the kernel derives from
// kv_indptr, unit by unit), passed in the kernel arguments: a workgroup then
// starts its first piece without first reading the request offsets and
// searching them.
constexpr int PLAN_UNITS = 256;  // units one plan holds (the arguments stay under 4 KB)
constexpr int PLAN_RP = 128;     // request offsets of a unit staged in LDS (2 waves x 64)
template <bool PLAN>
struct UnitPlan {};
template <>
struct UnitPlan<true> {
  int64_t chunk, nunits, Tv;
  int32_t base, pad_;
  int32_t r[PLAN_UNITS];      // first request of unit u
  int32_t p0[PLAN_UNITS];     // kv_indptr[r] - kv_indptr[0]
  int32_t len0[PLAN_UNITS];   // L_r
  uint16_t nreq[PLAN_UNITS];  // requests the unit covers: r .. r + nreq
};

// LDS layout of a staged tile (64 tokens x 36 chunks of 16 B): block
// (t/16, c/4) of 1 KB holds 16 tokens x 4 chunks; inside it, chunk c of
// token t sits at 16-B slot 4*(t%16) + ((c%4) ^ h(t)).  This h makes both
// the QK fragment reads (16 tokens of a quarter, one chunk each) and the
// transposed V reads (tokens {4G..4G+3} and {16+4G..16+4G+3}, 8-byte
// halves) free of bank conflicts on gfx950 (measured with the LDS
// bank-conflict counter: flipping only bit 1 for the second 16 tokens
// left the V reads 2-way conflicted).
__device__ __forceinline__ int hsw(int t) { return ((t >> 1) & 3) ^ (((t >> 4) & 1) * 3); }
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
// 4-byte variant: lane l writes lds_base + 4l
__device__ __forceinline__ void lds_dma4(const int32_t* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// floor(x / c) for x >= 0, c > 0: one 32-bit division when both fit (the
// stream positions of up to 2^32 tokens), the 64-bit one otherwise
__device__ __forceinline__ int64_t div_pos(int64_t x, int64_t c) {
  if ((((uint64_t)x | (uint64_t)c) >> 32) == 0) return (int64_t)((uint32_t)x / (uint32_t)c);
  return x / c;
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issue the direct global->LDS loads of one 64-token tile.  Wave w loads the
// 16 tokens of quarter w: load instruction cg fills block (w, cg), lane l
// carrying token 16w + l/4, chunk 4cg + ((l%4) ^ h(t)).  `row` is the cache
// row of that token (tile_row); tokens past the tile end and tokens with an
// index outside [0, num_slots) load `safe_row` (masked, or poisoned through
// the score).
__device__ __forceinline__ int tile_row(const MLA_LDS int32_t* idx_lds, int ntok, int wave, int lane) {
  const int t = 16 * wave + (lane >> 2);
  return t < ntok ? idx_lds[t] : -1;
}

__device__ __forceinline__ void issue_tile(const uint8_t* kv, int64_t num_slots, int row, int safe_row,
                                           MLA_LDS uint8_t* dst, int wave, int lane) {
  const int t = 16 * wave + (lane >> 2);
  row = (uint32_t)row < (uint64_t)num_slots ? row : safe_row;
  const uint8_t* src = kv + (int64_t)row * MLA_D_QK + 16 * ((lane & 3) ^ hsw(t));
  const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + 1024 * 9 * wave));
#pragma unroll
  for (int cg = 0; cg < 9; ++cg) lds_dma16(src + 64 * cg, d + 1024 * cg);
}

// The same loads one instruction at a time: tile_dma(...)(cg) fills block
// (w, cg), so a tile's 9 loads per wave can be spread over other work.
struct TileDma {
  const uint8_t* src;
  uint32_t d;
  __device__ __forceinline__ void operator()(int cg) const { lds_dma16(src + 64 * cg, d + 1024 * cg); }
};
struct NoDma {
  __device__ __forceinline__ void operator()(int) const {}
};
__device__ __forceinline__ TileDma tile_dma(const uint8_t* kv, int64_t num_slots, int row, int safe_row,
                                            MLA_LDS uint8_t* dst, int wave, int lane) {
  const int t = 16 * wave + (lane >> 2);
  row = (uint32_t)row < (uint64_t)num_slots ? row : safe_row;
  return TileDma{kv + (int64_t)row * MLA_D_QK + 16 * ((lane & 3) ^ hsw(t)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + 1024 * 9 * wave))};
}

constexpr int IDX_CAP = 2048;  // tokens whose cache indices are staged at once
constexpr int NBUF = 3;        // staged tiles in flight (triple buffering)
// max over the 4 lane groups {l, l^16, l^32, l^48} with VALU lane swaps
__device__ __forceinline__ float group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// sum over the 4 lane groups {l, l^16, l^32, l^48}
__device__ __forceinline__ float group_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// minimum over the 64 lanes, returned in a scalar register: rotations within
// each 16-lane row (DPP), then the lane-group swaps
__device__ __forceinline__ int wave_min64(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = min((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return __builtin_amdgcn_readfirstlane(min((int)b[0], (int)b[1]));
}

// max(a, b, c) on one v_max3_f32.  Every score here is a number or a quiet
// NaN (MFMA results, the mask's NaN), and a quiet NaN operand is passed
// over, so this is fmaxf(a, fmaxf(b, c)) without the compiler's
// signaling-NaN quieting of each operand.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Whether any of the first n staged cache indices in this wave's share
// (entries 64*wave + lane, stepping by 256) lies outside [0, num_slots).
__device__ __forceinline__ bool idx_share_bad(const MLA_LDS int32_t* idx, int n, uint32_t ns, int wave, int lane) {
  bool bad = false;
  for (int i = 64 * wave + lane; i < n; i += 256) bad |= (uint32_t)idx[i] >= ns;
  return __any(bad);
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Direct global->LDS staging of n (1 <= n <= IDX_CAP) cache indices, one
// per lane per load; entries past n repeat entry n-1, so nothing past the
// source range is read.
__device__ __forceinline__ void stage_idx(const int32_t* src, int n, MLA_LDS int32_t* idx_lds, int wave, int lane) {
  // rolled on purpose: the per-lane addresses are recomputed in place
  // rather than hoisted (and spilled) across the piece loop
#pragma unroll 1
  for (int j = 0; j < IDX_CAP / 256; ++j) {
    const int blk = wave + 4 * j;  // 64 indices per load instruction
    const int i = 64 * blk + lane;
    const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(idx_lds + 64 * blk));
    if (64 * blk < n) lds_dma4(src + (i < n ? i : n - 1), d);
  }
}

// Query staging.  A block's query reaches LDS by direct loads in fragment
// order: for a bf16 query, 1 KB block (g, s) holds at 16*lane the fragment
// of K-step s = 2pp + h that lane (lr, lg) reads, dims 64pp + 16lg + 8h ..
// +7 of row 16g + lr; an fp8 query takes one block per (g, pp), with dims
// 64pp + 16lg .. +15 (both K-steps of the pair).  Each lane's row offsets
// are computed once, so a load costs one address add, and the reads into
// registers are contiguous.  Blocks 0..35 go to tile buffer 2, the rest to
// the query area.
template <int NRG, bool QF8> constexpr int q_blocks() { return (QF8 ? 9 : 18) * NRG; }
template <int NRG, bool QF8> constexpr int q_area_bytes() {
  return q_blocks<NRG, QF8>() * 1024 > TILE_BYTES ? q_blocks<NRG, QF8>() * 1024 - TILE_BYTES : 16;
}
__device__ __forceinline__ MLA_LDS uint8_t* q_block(MLA_LDS uint8_t* buf2, MLA_LDS uint8_t* qarea, int j) {
  return j < TILE_BYTES / 1024 ? buf2 + 1024 * j : qarea + 1024 * (j - TILE_BYTES / 1024);
}
// The first segment's cache indices, then this wave's share of the query
// blocks, all by direct global->LDS loads; returns how many of this wave's
// loads are the query's (the caller waits for the indices alone first).
// rowq[g]: offset of this lane's row (g, lr) in the query (elements).
template <int NRG, bool QF8, class AfterIdx>
__device__ __forceinline__ int stage_q_and_idx(const PartialArgs& p, const int64_t (&rowq)[NRG],
                                               const int32_t* idx_src, int nidx, MLA_LDS uint8_t* buf2,
                                               MLA_LDS uint8_t* qarea, MLA_LDS int32_t* idx_lds, int wave,
                                               int lane, AfterIdx after_idx) {
  constexpr int NT_G = QF8 ? 9 : 18;  // blocks per row group
  const int lg = lane >> 4;
  // the indices go first: the caller waits for them alone and issues the
  // first tiles while the query is still in flight; after_idx issues loads
  // the same wait covers (the returned count is the query's loads only)
  stage_idx(idx_src, nidx, idx_lds, wave, lane);
  after_idx();
  int n = 0;
#pragma unroll
  for (int g = 0; g < NRG; ++g) {
    const uint8_t* base = QF8 ? p.q8 + rowq[g] + 16 * lg
                              : reinterpret_cast<const uint8_t*>(p.q + rowq[g] + 16 * lg);
#pragma unroll 1
    for (int t = wave; t < NT_G; t += 4) {
      // bf16: K-step t = 2pp + h at dims 64pp + 8h (bytes 128pp + 16h); fp8: pair t at byte 64t
      const int off = QF8 ? 64 * t : 128 * (t >> 1) + 16 * (t & 1);
      lds_dma16(base + off, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)q_block(buf2, qarea, NT_G * g + t)));
      ++n;
    }
  }
  return n;
}

// The fp8 query's QK runs on the fp8 MFMA: its fragments stay E4M3 codes,
// 16 bytes per 64-dim group pp (dims 64pp + 16lg .. +15), the same bytes
// the K chunk of that group holds for the token; q_scale is folded into the
// score constant.
template <int NRG>
__device__ __forceinline__ void read_q(MLA_LDS uint8_t* buf2, MLA_LDS uint8_t* qarea, int lane,
                                       u32x4 (&qf)[NRG][9]) {
#pragma unroll
  for (int g = 0; g < NRG; ++g)
#pragma unroll
    for (int pp = 0; pp < 9; ++pp) qf[g][pp] = *(const MLA_LDS u32x4*)(q_block(buf2, qarea, 9 * g + pp) + 16 * lane);
}

// The staged bf16 query -> this wave's query fragments qf[g][s] (K-step s
// of row group g).
template <int NRG>
__device__ __forceinline__ void read_q(MLA_LDS uint8_t* buf2, MLA_LDS uint8_t* qarea, int lane,
                                       bf16x8 (&qf)[NRG][18]) {
#pragma unroll
  for (int g = 0; g < NRG; ++g)
#pragma unroll
    for (int s = 0; s < 18; ++s) qf[g][s] = *(const MLA_LDS bf16x8*)(q_block(buf2, qarea, 18 * g + s) + 16 * lane);
}

// A valid cache row among the first n staged indices (0 if there is none),
// loaded in place of padding and invalid entries.
__device__ __forceinline__ int first_valid_row(const int32_t* idx, int n, int64_t num_slots) {
  int v = idx[0];
  if ((uint32_t)v >= (uint64_t)num_slots) {
    v = 0;
    for (int i = 1; i < n; ++i)
      if ((uint32_t)idx[i] < (uint64_t)num_slots) { v = idx[i]; break; }
  }
  return v;
}

// s_waitcnt vmcnt(n) for a wave-uniform n: at most n of this wave's loads
// may still be in flight (loads complete in issue order)
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
#define MLA_WAIT_CASE(k) \
  case k:                \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    MLA_WAIT_CASE(0) MLA_WAIT_CASE(1) MLA_WAIT_CASE(2) MLA_WAIT_CASE(3) MLA_WAIT_CASE(4) MLA_WAIT_CASE(5)
    MLA_WAIT_CASE(6) MLA_WAIT_CASE(7) MLA_WAIT_CASE(8) MLA_WAIT_CASE(9) MLA_WAIT_CASE(10) MLA_WAIT_CASE(11)
    MLA_WAIT_CASE(12) MLA_WAIT_CASE(13) MLA_WAIT_CASE(14) MLA_WAIT_CASE(15) MLA_WAIT_CASE(16)
#undef MLA_WAIT_CASE
    default:
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // more than 16: wait for everything
  }
}

// Scheduling hint for one unrolled step: NM groups of (1 MFMA, a share of NV
// VALU instructions, a share of ND LDS reads), so the conversions and reads
// issue in the shadow of the matrix pipe instead of around it.
template <int NM, int NV, int ND, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NM) {
    constexpr int nv = NV / NM + (I < NV % NM ? 1 : 0);
    constexpr int nd = ND / NM + (I < ND % NM ? 1 : 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);
    interleave<NM, NV, ND, I + 1>();
  }
}

// PV of one tile: O^T[128w + 16d .., rows] += V^T . P^T over 2 K-steps of
// 32 tokens.  The transposed V operand: source lane s of lane-group G points
// at token slot (G, s/2), columns 16*chunk + 8*(s&1).  read_v issues the 8
// transposed reads of one K-step; pv_tile takes those of K-step 0 already
// in flight (issued before the barrier that publishes P^T), issues K-step
// 1's before K-step 0's MFMAs, and converts block d+1 while the MFMAs of d
// run.
// Per-lane byte offsets of the transposed V reads within a tile, for
// columns chunk 8*wave + j (j < 4) of K-step 0; chunk 8*wave + j + 4 is
// 1 KB further and K-step 1 (tokens + 32) is 18 KB further, so 4 registers
// address all 16 reads of a tile (the rest are immediate offsets).
struct VOffsets {
  int o[4];
};
__device__ __forceinline__ VOffsets v_offsets(int wave, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int s2 = lr >> 1;
  const int tt = s2 < 4 ? 4 * lg + s2 : 16 + 4 * lg + s2 - 4;
  VOffsets v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v.o[j] = tile_off(tt, 8 * wave + j) + 8 * (lr & 1);
  return v;
}

__device__ __forceinline__ void read_v(const MLA_LDS uint8_t* kt, int kap, const VOffsets& vo, i32x2 (&v)[8]) {
  const MLA_LDS uint8_t* b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = kt + vo.o[j];
#pragma unroll
  for (int d = 0; d < 8; ++d)
    v[d] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(b[d & 3] + 1024 * (d >> 2) + 18432 * kap));
}

template <int NRG>
__device__ __forceinline__ void pv_tile(const MLA_LDS uint8_t* kt, const uint16_t* pt, f32x4 (&O)[8][NRG],
                                        const i32x2 (&v0)[8], const VOffsets& vo, int lane) {
  bf16x8 pf[2][NRG];
#pragma unroll
  for (int g = 0; g < NRG; ++g) pf[0][g] = *reinterpret_cast<const bf16x8*>(&pt[(g * 64 + lane) * 8]);
  i32x2 v1[8];
  read_v(kt, 1, vo, v1);
#pragma unroll
  for (int g = 0; g < NRG; ++g) pf[1][g] = *reinterpret_cast<const bf16x8*>(&pt[((NRG + g) * 64 + lane) * 8]);
#pragma unroll
  for (int kap = 0; kap < 2; ++kap) {
    const i32x2(&vr)[8] = kap == 0 ? v0 : v1;
    bf16x8 vf = fp8x8_to_bf16x8(u32x2{(uint32_t)vr[0][0], (uint32_t)vr[0][1]});
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      bf16x8 vn = vf;
      if (d + 1 < 8) vn = fp8x8_to_bf16x8(u32x2{(uint32_t)vr[d + 1][0], (uint32_t)vr[d + 1][1]});
#pragma unroll
      for (int g = 0; g < NRG; ++g) O[d][g] = mfma16(vf, pf[kap][g], O[d][g]);
      vf = vn;
      interleave<NRG, 4, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// QK of one tile for this wave's 16-token quarter and all row groups:
// S[g] (16 tokens x 16 rows, C layout: tokens 4*(l/16).. of row l%16) =
// K . Q^T over the 576 dims, as 9 K-step pairs.  Step pp uses chunk 4pp+lg
// of token 16*wave+lr (block (wave, pp) of the staged tile); K reads run
// two steps ahead of their conversion, and each step interleaves its MFMAs
// with the conversions of the next step.
template <int NRG, typename DMA>
__device__ __forceinline__ void qk_tile(const MLA_LDS uint8_t* kt, const bf16x8 (&qf)[NRG][18], int wave, int lane,
                                        f32x4 (&S)[NRG], const DMA& dma) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int g = 0; g < NRG; ++g) S[g] = f32x4{0, 0, 0, 0};
  const MLA_LDS uint8_t* kq = kt + tile_off(16 * wave + lr, lg);
  u32x4 raw[3];
  raw[0] = *(const MLA_LDS u32x4*)kq;
  raw[1] = *(const MLA_LDS u32x4*)(kq + 1024);
  bf16x8 klo = fp8x8_to_bf16x8(u32x2{raw[0][0], raw[0][1]});
  bf16x8 khi = fp8x8_to_bf16x8(u32x2{raw[0][2], raw[0][3]});
#pragma unroll
  for (int pp = 0; pp < 9; ++pp) {
    if (pp == 0) { dma(0); dma(1); dma(2); }
    if (pp >= 1 && pp <= 3) { dma(2 * pp + 1); dma(2 * pp + 2); }
    if (pp + 2 < 9) raw[(pp + 2) % 3] = *(const MLA_LDS u32x4*)(kq + 1024 * (pp + 2));
    bf16x8 nlo = klo, nhi = khi;
    if (pp + 1 < 9) {
      nlo = fp8x8_to_bf16x8(u32x2{raw[(pp + 1) % 3][0], raw[(pp + 1) % 3][1]});
      nhi = fp8x8_to_bf16x8(u32x2{raw[(pp + 1) % 3][2], raw[(pp + 1) % 3][3]});
    }
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      S[g] = mfma16(klo, qf[g][2 * pp], S[g]);
      S[g] = mfma16(khi, qf[g][2 * pp + 1], S[g]);
    }
    klo = nlo;
    khi = nhi;
    interleave<2 * NRG, 8, 1>();
    __builtin_amdgcn_sched_barrier(0);  // keep the steps (and their read-ahead) in order
  }
}

// QK of one tile for an fp8 query, on the fp8 MFMA straight from the
// staged E4M3 bytes (no conversion of K): the 576 dims as four 128-dim
// steps, step s taking 64-dim groups 2s and 2s+1 (the chunk lane group lg
// reads from each, 32 bytes per lane; the query fragment holds the same
// dims), then the 64 rope dims as a fifth step whose other half is zero.
// Operand and accumulator layouts as in qk_tile; the products are exact and
// accumulate in f32.
template <int NRG, typename DMA>
__device__ __forceinline__ void qk_tile_f8(const MLA_LDS uint8_t* kt, const u32x4 (&qf)[NRG][9], int wave, int lane,
                                           f32x4 (&S)[NRG], const DMA& dma) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int g = 0; g < NRG; ++g) S[g] = f32x4{0, 0, 0, 0};
  const MLA_LDS uint8_t* kq = kt + tile_off(16 * wave + lr, lg);
  u32x4 raw[9];
#pragma unroll
  for (int pp = 0; pp < 9; ++pp) raw[pp] = *(const MLA_LDS u32x4*)(kq + 1024 * pp);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    dma(2 * st);
    dma(2 * st + 1);
    const i32x8 a = __builtin_bit_cast(i32x8, u32x8{raw[2 * st][0], raw[2 * st][1], raw[2 * st][2], raw[2 * st][3],
                                                    raw[2 * st + 1][0], raw[2 * st + 1][1], raw[2 * st + 1][2],
                                                    raw[2 * st + 1][3]});
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const u32x4 q0 = qf[g][2 * st], q1 = qf[g][2 * st + 1];
      const i32x8 bq = __builtin_bit_cast(i32x8, u32x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]});
      // E4M3 operands (format 0), unit E8M0 scales (127)
      S[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bq, S[g], 0, 0, 0, 127, 0, 127);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  dma(8);
  // the rope dims: group 8's chunk in the low 16 bytes of both operands,
  // zeros in the high 16 (one MFMA type along the whole accumulation chain)
  const i32x8 ar = __builtin_bit_cast(i32x8, u32x8{raw[8][0], raw[8][1], raw[8][2], raw[8][3], 0u, 0u, 0u, 0u});
#pragma unroll
  for (int g = 0; g < NRG; ++g) {
    const u32x4 q8 = qf[g][8];
    const i32x8 bq = __builtin_bit_cast(i32x8, u32x8{q8[0], q8[1], q8[2], q8[3], 0u, 0u, 0u, 0u});
    S[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ar, bq, S[g], 0, 0, 0, 127, 0, 127);
  }
}

// P = 2^(c*S - ref) of this wave's quarter (S in raw score units, nmb =
// -ref) -> bf16 P^T fragments in LDS (in the PV B-operand order), and the
// per-lane partial row sums.
template <int NRG>
__device__ __forceinline__ void p_tile(const f32x4 (&S)[NRG], float c, const float (&nmb)[NRG], uint16_t* ptb,
                                       int wave, int lane, float (&ps)[NRG]) {
#pragma unroll
  for (int g = 0; g < NRG; ++g) {
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(S[g][e], c, nmb[g]));
    ps[g] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
    *reinterpret_cast<u32x2*>(&ptb[(((wave >> 1) * NRG + g) * 64 + lane) * 8 + 4 * (wave & 1)]) =
        u32x2{pk_bf16(pv[0], pv[1]), pk_bf16(pv[2], pv[3])};
  }
}

// Per-workgroup wall-clock marks of the partial kernel, in the measurement
// build libmla_fp8_timeline.so only (compiled with MLA_WG_TIMELINE; the
// marks compile to nothing otherwise): s_memrealtime, a 100 MHz counter
// common to every CU, at
//   0 the workgroup's start, 1 its end, 2 (a count) its pieces,
//   3 / 7 the start of its first / second piece, 4 / 8 their first ready
//   tile (staged and waited for), 5 / 9 the end of their tile loop (the
//   last pass's, after a restart), 6 / 10 (a count) their tiles,
//   11, 12, 13 in its last piece's epilogue: row sums and maxima exchanged,
//   rows normalised into LDS, partial rows stored,
//   14 the late new rows of the fused cache write encoded and stored (first
//   piece), 15 the first piece's cache indices landed.
// Workgroup record i is linear block id i; mla_wg_timeline reads them.
#ifdef MLA_WG_TIMELINE
constexpr bool kTimeline = true;
constexpr int TL_MAX = 4096;  // workgroups with a record
__device__ uint64_t g_timeline[TL_MAX][16];
#else
constexpr bool kTimeline = false;
#endif
__device__ __forceinline__ uint64_t tl_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
  return t;
}

template <int NRG, bool QF8, bool PLAN, bool FUSE, bool WRITE>
__global__ void __launch_bounds__(256, 1) partial_kernel(PartialArgs p, UnitPlan<PLAN> pl, NewArgs<WRITE> nw) {
  static_assert(!FUSE || PLAN, "the fused call takes the host-built partition");
  constexpr int RB = 16 * NRG;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf_[NBUF * TILE_BYTES];
  constexpr int PT_ELEMS = 2 * NRG * 64 * 8;  // P^T of one tile (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t pt[2 * PT_ELEMS];  // double buffered by tile parity
  __shared__ __attribute__((aligned(16))) float redmax[RB * 4];
  __shared__ __attribute__((aligned(16))) float redsum[RB * 4];
  __shared__ __attribute__((aligned(16))) int32_t idx[IDX_CAP];
  __shared__ __attribute__((aligned(16))) uint8_t qarea_[q_area_bytes<NRG, QF8>()];  // query staging, past tile buffer 2
  __shared__ int32_t red_i[4];
  __shared__ int32_t segbad_[4];  // per wave: a bad cache index in its share of the segment
  __shared__ int64_t rowoff[RB];  // output offset of block row i within its request, -1 past M
  __shared__ int64_t latoff[FUSE ? RB : 1];  // the same in the merged latent
  __shared__ int32_t last_[1];               // fused call: the counter value this block saw
  // the fused cache write: a piece's new tokens as bf16 (latent rows, then
  // a block of rope rows) and their slots (two dwords each)
  __shared__ __attribute__((aligned(16))) uint8_t nraw_[WRITE ? NEW_MAX * 1024 + 1024 : 16];
  __shared__ __attribute__((aligned(16))) int32_t nslot_[WRITE ? 64 : 1];
  // the normalised O rows are staged as bf16 [RB][O_PITCH] in the tile buffers
  constexpr int O_PITCH = MLA_D_LATENT + 16;  // +32 B: rows start 8 banks apart
  static_assert(RB * O_PITCH * 2 <= NBUF * TILE_BYTES, "O staging fits the tile buffers");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  MLA_LDS uint8_t* kbuf = (MLA_LDS uint8_t*)kbuf_;
  MLA_LDS int32_t* idxl = (MLA_LDS int32_t*)idx;
  MLA_LDS uint8_t* qarea = (MLA_LDS uint8_t*)qarea_;
  MLA_LDS uint8_t* nraw = (MLA_LDS uint8_t*)nraw_;
  MLA_LDS int32_t* nslot = (MLA_LDS int32_t*)nslot_;
  const VOffsets vo = v_offsets(wave, lane);
  uint64_t tl[kTimeline ? 16 : 1] = {};  // the timeline marks (measurement build)
  int tl_piece = 0;
  // mark i of the first piece, or i + 4 of the second (constant indices:
  // the marks stay in registers)
  auto tl_piece_mark = [&](int i, uint64_t v, bool add) {
    if constexpr (kTimeline) {
      if (tl_piece == 0)
        tl[i] = add ? tl[i] + v : v;
      else if (tl_piece == 1)
        tl[i + 4] = add ? tl[i + 4] + v : v;
    }
  };
  if constexpr (kTimeline) tl[0] = tl_now();

  // ---- block -> (worker, row block), from the block indices alone, so
  // that no argument read waits for another (the grid's size is an
  // argument read too): the grid is (8, row blocks, ceil(workers / 8)), and
  // the workgroups past the last worker find no unit and leave.  Workgroups
  // go to the 8 XCDs round robin in linear order (x first), so the row
  // blocks of a worker (linear ids 8 apart) share an XCD and its L2, start
  // together, and workers interleave across the XCDs.
  const int u = blockIdx.x + 8 * blockIdx.z, rb = blockIdx.y;

  // ---- the split partition: T, L_max -> chunk, and the requests this
  // unit covers
  constexpr int64_t W = MLA_PIECE_TOKENS;
  const int m_lo = rb * RB;  // first row (of the request's qlen*heads) of this block
  constexpr int RMAX = 64;
  __shared__ int32_t rP[RMAX + 1];
  __shared__ __attribute__((aligned(16))) int32_t rPraw[PLAN_RP];
  int base = 0, r = 0, r_end = 0, nreq = 0;
  int64_t Tv = 0, chunk = 1, nunits = 1;
  int plan_p0 = 0, plan_len0 = 0;  // the first piece's offset and length, from the plan
  if constexpr (PLAN) {
    base = pl.base;
    Tv = pl.Tv;
    chunk = pl.chunk;
    nunits = pl.nunits;
    // this unit's plan entries, read with the other arguments (u < 8 *
    // ceil(workers / 8) <= PLAN_UNITS), and all used here, so that none of
    // the reads is left for later: the first piece's cache indices wait on
    // plan_p0 and plan_len0
    const int plan_r = pl.r[u], plan_n = pl.nreq[u];
    plan_p0 = pl.p0[u];
    plan_len0 = pl.len0[u];
    asm volatile("" ::"s"(plan_r), "s"(plan_n), "s"(plan_p0), "s"(plan_len0));
    if (u < nunits) {
      r = plan_r;
      r_end = r + plan_n;
      // kv_indptr[r + i] (i < PLAN_RP, clamped to the last entry) to LDS by
      // direct loads; the first piece takes its offsets from the plan, and
      // these loads, issued before its staging, have landed by its first wait
      if (wave < PLAN_RP / 64) {
        const int i = min(r + 64 * wave + lane, p.batch);
        lds_dma4(p.indptr + i, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(rPraw + 64 * wave)));
      }
    }
  } else {
    // the request offsets are staged in LDS (the tile buffers are still
    // free) when they fit
    const bool ip_lds = (int64_t)(p.batch + 1) * 4 <= (int64_t)NBUF * TILE_BYTES;
    MLA_LDS int32_t* ipl = (MLA_LDS int32_t*)kbuf;
    if (ip_lds) {
      for (int i0 = 0; i0 <= p.batch; i0 += 1024) {
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + tid + 256 * j;
          v[j] = i <= p.batch ? p.indptr[i] : 0;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + tid + 256 * j;
          if (i <= p.batch) ipl[i] = v[j];
        }
      }
      __syncthreads();
    }
    auto ip = [&](int i) -> int { return ip_lds ? ipl[i] : p.indptr[i]; };
    int lmax = 0;
    for (int rr = tid; rr < p.batch; rr += 256) lmax = max(lmax, ip(rr + 1) - ip(rr));
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) lmax = max(lmax, __shfl_xor(lmax, s));
    if (lane == 0) red_i[wave] = lmax;
    __syncthreads();
    lmax = max(max(red_i[0], red_i[1]), max(red_i[2], red_i[3]));
    base = ip(0);
    // the partition's stream: request r takes MLA_PIECE_TOKENS positions,
    // then its tokens; Vs(r) = ip(r) - base + W r is where it starts
    Tv = (int64_t)ip(p.batch) - base + W * p.batch;
    chunk = split_chunk(Tv, lmax, p.num_splits, p.num_workers, p.split_min);
    nunits = Tv > 0 ? (Tv + chunk - 1) / chunk : 1;
    const int64_t s0 = (int64_t)u * chunk;
    const int64_t s1 = s0 + chunk < Tv ? s0 + chunk : Tv;
    // first request whose stream end is >= s0, and the requests this unit covers
    if (u < nunits) {
      int lo = 0, hi = p.batch;
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)ip(mid + 1) - base + W * (mid + 1) >= s0) hi = mid; else lo = mid + 1;
      }
      r = lo;
      r_end = r;
      while (r_end < p.batch) {
        const int64_t Vs = (int64_t)ip(r_end) - base + W * r_end;
        if (Vs >= s1 && !(u == nunits - 1 && Vs == Tv)) break;
        ++r_end;
      }
    }
    // (P, L) of the covered requests, read before the tile buffers are reused
    nreq = min(r_end - r, RMAX);
    for (int i = tid; i <= nreq; i += 256) rP[i] = ip(r + i) - base;
  }
  const int64_t g0 = (int64_t)u * chunk;
  const int64_t g1 = g0 + chunk < Tv ? g0 + chunk : Tv;
  if (tid < RB) {
    const int m = m_lo + tid;
    rowoff[tid] = FUSE ? 0 : (m < p.M ? (int64_t)(m / p.heads) * p.os_r + (int64_t)(m % p.heads) * p.os_h : -1);
    if constexpr (FUSE) latoff[tid] = m < p.M ? (int64_t)(m / p.heads) * p.lat_r + (int64_t)(m % p.heads) * p.lat_h : -1;
  }
  __syncthreads();
  if (u >= nunits) return;

  // this lane's rows (row group g, lane row lr) as (position in the qlen
  // window, head); rows past M take the block's first row
  int rj[NRG], rh[NRG];
#pragma unroll
  for (int g = 0; g < NRG; ++g) {
    const int m0 = m_lo + 16 * g + lr;
    const int m = m0 < p.M ? m0 : m_lo;
    rj[g] = m / p.heads;
    rh[g] = m - p.heads * rj[g];
  }
  auto fill_neginf = [&](int req, int k_from) {
    // LSE = -inf for splits [k_from, num_splits) of every row of this block
    const int nrows = min(RB, p.M - m_lo);
    if (tid < nrows) {
      const int m = m_lo + tid;
      const int t = req * p.qlen + m / p.heads, h = m % p.heads;
      float* dst = p.lse + (int64_t)t * p.ls_r + (int64_t)h * p.ls_h;
      for (int k = k_from; k < p.num_splits; ++k) dst[k * p.ls_s] = -INFINITY;
    }
  };

  bool rp_ready = !PLAN;  // the planned offsets in rPraw have landed and are visible
  for (int ri = 0; r < r_end; ++r, ++ri) {
    int64_t P;
    int L;
    if constexpr (PLAN) {
      if (ri == 0) {
        P = plan_p0;
        L = plan_len0;
      } else {
        if (!rp_ready) {  // the first piece was empty: wait for the offsets here
          wait_vm_all();
          __syncthreads();
          rp_ready = true;
        }
        if (ri + 1 < PLAN_RP) {
          P = (int64_t)rPraw[ri] - base;
          L = rPraw[ri + 1] - rPraw[ri];
        } else {
          P = (int64_t)p.indptr[r] - base;
          L = p.indptr[r + 1] - p.indptr[r];
        }
      }
    } else if (ri < nreq) {
      P = rP[ri];
      L = rP[ri + 1] - rP[ri];
    } else {
      P = (int64_t)p.indptr[r] - base;
      L = p.indptr[r + 1] - p.indptr[r];
    }
    const int64_t V = P + W * (r + 1);  // stream position of the request's first token
    const int64_t vq = div_pos(V, chunk);  // the unit that holds it
    if (L == 0) {
      const int64_t owner = vq < nunits - 1 ? vq : nunits - 1;
      if constexpr (WRITE)
        if (__builtin_expect(owner == u && rb == 0, 0)) write_new_direct(p, nw, r, 0, nw.k, tid);
      if (owner == u) {
        if constexpr (FUSE) {
          // an empty request's merged rows: latent 0, LSE -inf
          const int nrows = min(RB, p.M - m_lo);
          uint16_t* lbase = p.lat + (int64_t)r * p.qlen * p.lat_r + 8 * lane;
          for (int i = wave; i < nrows; i += 4) *reinterpret_cast<u32x4*>(lbase + latoff[i]) = u32x4{0, 0, 0, 0};
          if (p.lat_lse && tid < nrows) {
            const int m = m_lo + tid;
            p.lat_lse[((int64_t)r * p.qlen + m / p.heads) * p.ll_r + (int64_t)(m % p.heads) * p.ll_h] = -INFINITY;
          }
        } else {
          fill_neginf(r, 0);
        }
      }
      continue;
    }
    const int a = (int)((g0 > V ? g0 : V) - V);
    const int b = (int)((g1 < V + L ? g1 : V + L) - V);
    if (b <= a) continue;
    const int k = (a == 0) ? 0 : (int)(u - vq);  // a > 0: the piece starts at this unit's start
    // fused call: the request's split count, and this piece's workspace
    // slot (split 0 is the last piece of unit vq: slot 1 of it; a later split
    // is the first piece of its unit: slot 0)
    const int nsplit = (int)(div_pos(V + L - 1, chunk) - vq + 1);
    const int64_t su = k == 0 ? vq : (int64_t)u;
    const int slot = (int)((su * 2 + (k == 0 ? 1 : 0)) * p.n_rb + rb);
    if (FUSE && (k >= p.num_splits || su < 0 || su >= nunits)) continue;  // a host copy that differs from kv_indptr
    if (!FUSE && PLAN && k >= p.num_splits) {
      // only a host copy of the offsets that differs from kv_indptr gets
      // here: poison the rows' last split instead of writing past it
      const int nrows = min(RB, p.M - m_lo);
      if (tid < nrows) {
        const int m = m_lo + tid;
        p.lse[(int64_t)(p.num_splits - 1) * p.ls_s + (int64_t)(r * p.qlen + m / p.heads) * p.ls_r +
              (int64_t)(m % p.heads) * p.ls_h] = __builtin_nanf("");
      }
      continue;
    }
    if (!FUSE && k == 0 && nsplit < p.num_splits) fill_neginf(r, nsplit);
    // the fused cache write: new tokens before the request's first token
    // (a request shorter than nw_k) are written by its first piece's owner
    if constexpr (WRITE)
      if (__builtin_expect(a == 0 && rb == 0 && L < nw.k, 0)) write_new_direct(p, nw, r, 0, nw.k - L, tid);

    // ---------------------------------------------------------- one piece
    if constexpr (kTimeline) tl_piece_mark(3, tl_now(), false);
    bool tl_ready = false;
    const int32_t* rows_r = p.indices + (PLAN ? base + (int)P : p.indptr[r]);
    int lim[NRG];  // visible tokens of row (g, lr), as an end in request tokens
    int lim_min = b;
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const int m = m_lo + 16 * g + lr;
      // rows past M compute on a copy of a real row; their results are discarded
      const int vis = m < p.M ? L - p.qlen + rj[g] + 1 : b;
      lim[g] = min(b, vis);
      lim_min = min(lim_min, lim[g]);
    }
    lim_min = wave_min64(lim_min);  // wave-uniform: keep the mask test scalar

    // ---- stage the first segment's cache indices and the block's query in
    // LDS by direct loads (the query in tile buffer 2 and the query area;
    // tile 2 is issued only after every wave has read it).  Only the indices
    // are waited for here: tiles 0 and 1 are issued while the query is still
    // in flight.
    // ---- the fused cache write: this piece's new tokens (nw_cnt of them,
    // from request token j0 on) as bf16 rows, and their slots, to LDS by
    // direct loads issued between the indices and the query, so the wait
    // for the indices covers them
    int nw_cnt = 0, nw_j0 = 0;
    bool nw_late = false;  // stored after tiles 0 and 1 are issued (see below)
    if constexpr (WRITE) {
      const int pos0 = L - nw.k;  // position of the request's new token 0
      const int j0 = max(0, a - pos0), j1 = min(nw.k, b - pos0);
      if (j1 > j0) {
        nw_cnt = j1 - j0;
        nw_j0 = j0;
        nw_late = max(pos0, a) - a >= 3 * NT;
      }
    }
    auto stage_new = [&]() {
      if constexpr (WRITE) {
        if (nw_cnt == 0) return;
        const int64_t tn = (int64_t)r * nw.k + nw_j0;  // the first of them
        for (int jj = wave; jj < nw_cnt; jj += 4)
          lds_dma16(reinterpret_cast<const uint8_t*>(nw.c + (tn + jj) * nw.c_r) + 16 * lane,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(nraw + 1024 * jj)));
        if (wave == 0) {
          // lane l: rope chunk l%8 of token l/8 (lanes past the last token
          // load its last chunk again); dword l of the slots likewise
          const int jr = min(lane >> 3, nw_cnt - 1);
          lds_dma16(reinterpret_cast<const uint8_t*>(nw.pe + (tn + jr) * nw.pe_r) + 16 * (lane & 7),
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(nraw + 1024 * NEW_MAX)));
          lds_dma4(reinterpret_cast<const int32_t*>(nw.slot + tn) + min(lane, 2 * nw_cnt - 1),
                   __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)nslot));
        }
      }
    };

    int64_t rowq[NRG];
#pragma unroll
    for (int g = 0; g < NRG; ++g) rowq[g] = ((int64_t)r * p.qlen + rj[g]) * p.q_sr + (int64_t)rh[g] * p.q_sh;
    const int nq = stage_q_and_idx<NRG, QF8>(p, rowq, rows_r + a, min(IDX_CAP, b - a), kbuf + 2 * TILE_BYTES, qarea,
                                             idxl, wave, lane, stage_new);
    wait_vm_upto(__builtin_amdgcn_readfirstlane(nq));
    __syncthreads();
    rp_ready = true;  // the planned offsets were loaded before this staging
    if constexpr (kTimeline)
      if (tl_piece == 0) tl[15] = tl_now();
    if constexpr (WRITE) {
      // The new tokens go into their cache slots before any tile that holds
      // them is loaded, from every row block's workgroup (the same bytes):
      // the tiles' loads then read them, as this CU's own stores keep its
      // L1 current and reach the XCD's L2 first.  When tiles 0-2 hold one,
      // they are stored here and waited for (stores and loads share one
      // counter, so this also waits for the query); otherwise after tiles 0
      // and 1 are issued and before tile 2 is: global loads and stores
      // report completion to a wave in issue order, so the wait for tile 1
      // (after tile 2 is issued) covers them too, and the barrier after it
      // comes before tile 3 is issued.
      if (__builtin_expect(nw_cnt > 0 && !nw_late, 0)) {
        store_new_rows(p, nw, nraw, nslot, nw_cnt, tid);
        wait_vm_all();
        __syncthreads();
      }
    }
    {
      const int slen = min(IDX_CAP, b - a);
      const int safe_row = first_valid_row(idx, slen, p.num_slots);
      issue_tile(p.kv, p.num_slots, tile_row(idxl, min(NT, slen), wave, lane), safe_row, kbuf, wave, lane);
      if (slen > NT)
        issue_tile(p.kv, p.num_slots, tile_row(idxl + NT, min(NT, slen - NT), wave, lane), safe_row,
                   kbuf + TILE_BYTES, wave, lane);
      {
        const bool bad = idx_share_bad(idxl, slen, (uint32_t)p.num_slots, wave, lane);
        if (lane == 0) segbad_[wave] = bad;  // read after the barrier below
      }
      // the late new rows, encoded while the tiles load (with their stores
      // the youngest, no more than 9 outstanding still means tile 0 has
      // landed)
      if constexpr (WRITE)
        if (nw_late) {
          store_new_rows(p, nw, nraw, nslot, nw_cnt, tid);
          if constexpr (kTimeline)
            if (tl_piece == 0) tl[14] = tl_now();
        }
      // the query (issued before the tiles) and tile 0 have landed; tile 1's
      // 9 loads may still fly
      if (slen > NT)
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else
        wait_vm_all();
      __syncthreads();
    }
    // the query fragments: K-step 2pp uses dims 64pp+16lg..+7, 2pp+1 the
    // next 8 (the K fragments use the same order); kept in AGPRs (they are
    // only MFMA B operands), so the arch VGPRs hold the per-tile working set
    typename std::conditional<QF8, u32x4[NRG][9], bf16x8[NRG][18]>::type qf;
    read_q<NRG>(kbuf + 2 * TILE_BYTES, qarea, lane, qf);
#pragma unroll
    for (int g = 0; g < NRG; ++g)
#pragma unroll
      for (int ss = 0; ss < (QF8 ? 9 : 18); ++ss) asm volatile("" : "+a"(qf[g][ss]));

    f32x4 O[8][NRG];
    // per row: the softmax reference (log2 units) and its negation, the
    // lane's share of the row sum, and the lane's running maximum score
    // (raw score units)
    float mref[NRG], nmb[NRG], lsum[NRG], rmax[NRG];
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      mref[g] = 0.0f;
      nmb[g] = 0.0f;
    }

    // Every row starts with reference 0: P = 2^(s*c - ref) stays within
    // 2^(+-64) of the row's largest term unless the row's maximum lies more
    // than 64 log2 units away from the reference.  Whether it does is known
    // at the end of the piece, from the exchanged row maxima: such a row
    // takes its maximum as the reference and the piece runs again from its
    // first token (once: the maxima do not change).  O is never rescaled,
    // and no tile waits for a decision about the reference.
    bool again = true;
    bool restaged = false;  // the first segment's indices must be staged again
    while (again) {
    again = false;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int g = 0; g < NRG; ++g) O[d][g] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      lsum[g] = 0.0f;
      rmax[g] = -INFINITY;
    }

    for (int s0 = a; s0 < b; s0 += IDX_CAP) {
      const int slen = min(IDX_CAP, b - s0);
      const bool first_seg = s0 == a && !restaged;  // staged and issued with the query
      if (!first_seg) {
        // ---- a later segment (or a restart): stage its cache indices
        __syncthreads();  // the previous segment's tiles are done with idx / kbuf
        stage_idx(rows_r + s0, slen, idxl, wave, lane);
        wait_vm_all();
        __syncthreads();
      }
      const int safe_row = first_valid_row(idx, slen, p.num_slots);
      const int ntiles = (slen + NT - 1) / NT;
      if (!first_seg) {
        issue_tile(p.kv, p.num_slots, tile_row(idxl, min(NT, slen), wave, lane), safe_row, kbuf, wave, lane);
        if (ntiles > 1)
          issue_tile(p.kv, p.num_slots, tile_row(idxl + NT, min(NT, slen - NT), wave, lane), safe_row,
                     kbuf + TILE_BYTES, wave, lane);
        {
          const bool bad = idx_share_bad(idxl, slen, (uint32_t)p.num_slots, wave, lane);
          if (lane == 0) segbad_[wave] = bad;  // read after the barrier below
        }
        if (ntiles > 1)
          asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // tile 0's 9 loads (tile 1's may fly)
        else
          wait_vm_all();
        __syncthreads();
      }

      // a bad cache index anywhere in this segment sends every tile through
      // the masking path (which then finds it); written before the barrier
      // that follows tile 0's wait
      const bool seg_bad = (segbad_[0] | segbad_[1] | segbad_[2] | segbad_[3]) != 0;
      if constexpr (kTimeline) {
        if (!tl_ready) tl_piece_mark(4, tl_now(), false);
        tl_ready = true;
        tl_piece_mark(6, (uint64_t)ntiles, true);
      }
      // P^T is double buffered by tile parity.
      for (int it = 0; it < ntiles; ++it) {
        const int t0 = s0 + NT * it;
        const MLA_LDS uint8_t* kt = kbuf + (it % NBUF) * TILE_BYTES;
        uint16_t* ptb = pt + (it & 1) * PT_ELEMS;
        // tile it+2's rows, read ahead of QK
        const bool more = it + 2 < ntiles;
        const int nrow = more ? tile_row(idxl + NT * (it + 2), min(NT, slen - NT * (it + 2)), wave, lane) : 0;
        // every wave is past PV of tile it-1 (and, at the first tile, past
        // its query reads): that buffer takes tile it+2, whose loads issue
        // one per QK step
        __syncthreads();
        f32x4 S[NRG];
        if (more) {
          const TileDma dma =
              tile_dma(p.kv, p.num_slots, nrow, safe_row, kbuf + ((it + 2) % NBUF) * TILE_BYTES, wave, lane);
          if constexpr (QF8)
            qk_tile_f8<NRG>(kt, qf, wave, lane, S, dma);
          else
            qk_tile<NRG>(kt, qf, wave, lane, S, dma);
        } else {
          if constexpr (QF8)
            qk_tile_f8<NRG>(kt, qf, wave, lane, S, NoDma{});
          else
            qk_tile<NRG>(kt, qf, wave, lane, S, NoDma{});
        }
        // ---- mask (raw score units) only where a row's visible range or a
        // bad index reaches into this quarter
        {
          const int tq0 = t0 + 16 * wave;
          if (!(tq0 + 16 <= lim_min && !seg_bad)) {
            const i32x4 ids = *(const MLA_LDS i32x4*)(idxl + NT * it + 16 * wave + 4 * lg);
            const uint32_t ns = (uint32_t)p.num_slots;
            const bool bad0 = (uint32_t)ids[0] >= ns, bad1 = (uint32_t)ids[1] >= ns;
            const bool bad2 = (uint32_t)ids[2] >= ns, bad3 = (uint32_t)ids[3] >= ns;
#pragma unroll
            for (int g = 0; g < NRG; ++g)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int tok = tq0 + 4 * lg + e;
                const bool bad = e == 0 ? bad0 : e == 1 ? bad1 : e == 2 ? bad2 : bad3;
                S[g][e] = tok < lim[g] ? (bad ? __builtin_nanf("") : S[g][e]) : -INFINITY;
              }
          }
        }
        // ---- the running maxima (a NaN score leaves them; it poisons the sum)
#pragma unroll
        for (int g = 0; g < NRG; ++g)
          rmax[g] = max3f(max3f(rmax[g], S[g][0], S[g][1]), S[g][2], S[g][3]);
        float ps[NRG];
        p_tile<NRG>(S, p.c_log2, nmb, ptb, wave, lane, ps);
        i32x2 v0[8];
        read_v(kt, 0, vo, v0);               // in flight across the barrier
        // tile it+1 has landed (this wave's part; tile it+2's 9 loads may fly)
        if (more)
          asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else if (it + 1 < ntiles)
          wait_vm_all();
        __syncthreads();  // P^T of tile it; tile it+1 visible
#pragma unroll
        for (int g = 0; g < NRG; ++g) lsum[g] += ps[g];
        pv_tile<NRG>(kt, ptb, O, v0, vo, lane);
      }
    }
    if constexpr (kTimeline) tl_piece_mark(5, tl_now(), false);
    // ---- end of the piece: the row sums and maxima of the four quarters;
    // rows whose maximum lies more than 64 log2 units from their reference
    // take it as the new reference and the piece runs again (a block-uniform
    // decision: every wave reads the same maxima)
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const float l = group_sum4(lsum[g]);
      const float lm = group_max4(rmax[g]) * p.c_log2;
      if (lg == 0) {
        redsum[(16 * g + lr) * 4 + wave] = l;
        redmax[(16 * g + lr) * 4 + wave] = lm;
      }
    }
    __syncthreads();
    if constexpr (kTimeline) tl[11] = tl_now();
    bool moved = false;
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(&redmax[(16 * g + lr) * 4]);
      const float mx = fmaxf(fmaxf(q4[0], q4[1]), fmaxf(q4[2], q4[3]));
      if (mx > mref[g] + kLazy || (mx != -INFINITY && mx < mref[g] - kLazy)) {
        mref[g] = mx;
        nmb[g] = -mx;
        moved = true;
      }
    }
    if (__any(moved)) {
      again = true;
      restaged = true;
    }
    }  // while (again)
    if constexpr (kTimeline) ++tl_piece;

    // ---------------------------------------------------- piece epilogue
    // The row sums; O normalised to bf16 into LDS (every wave is past its
    // last PV after the first barrier, so the tile buffers are free), then
    // written out one whole 1 KB row per store instruction.
    // The fused call writes a request of one split straight into the merged
    // latent (what the merge makes of one split: rows with no visible token
    // are 0, NaN rows the canonical NaN) and the pieces of a split request
    // into its workspace slot; the last of them to finish merges them.
    const bool direct = FUSE && nsplit == 1;
    MLA_LDS uint16_t* ost = (MLA_LDS uint16_t*)kbuf;
    uint64_t wmask = 0;  // block rows to write (a finite or NaN sum, row < M; every row < M when direct)
    const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(p.ws, 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(&redsum[(16 * g + lr) * 4]);
      const float l = ((s4[0] + s4[1]) + s4[2]) + s4[3];
      // l == 0: no visible token in this split (the row is not written).  A
      // NaN l (NaN cache bytes or an invalid index) is written through, so
      // it poisons the row.
      const float inv = direct && l == 0.0f ? 0.0f : p.kv_scale * __builtin_amdgcn_rcpf(l);
      const bool nan_row = direct && l != l;
      MLA_LDS uint16_t* orow = ost + (16 * g + lr) * O_PITCH + 128 * wave + 4 * lg;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const f32x4 v = O[d][g];
        u32x2 w2 = u32x2{pk_bf16(v[0] * inv, v[1] * inv), pk_bf16(v[2] * inv, v[3] * inv)};
        if (nan_row) w2 = u32x2{0x7FC07FC0u, 0x7FC07FC0u};
        *reinterpret_cast<MLA_LDS u32x2*>(orow + 16 * d) = w2;
      }
      const int m = m_lo + 16 * g + lr;
      wmask |= (__ballot((direct || l != 0.0f) && m < p.M) & 0xFFFFull) << (16 * g);  // lanes lg == 0: rows 16g + lr
      if (wave == 0 && lg == 0 && m < p.M) {
        const int t = r * p.qlen + rj[g], h = rh[g];
        const float lv = l != 0.0f ? (mref[g] + __log2f(l)) * kLn2 : -INFINITY;
        if constexpr (!FUSE) {
          p.lse[k * p.ls_s + (int64_t)t * p.ls_r + (int64_t)h * p.ls_h] = lv;
        } else if (direct) {
          if (p.lat_lse) p.lat_lse[(int64_t)t * p.ll_r + (int64_t)h * p.ll_h] = lv;
        } else {
          // system-coherent store: the merging block may run on another XCD
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lv), wsr,
                                                p.ws_lse_off + (slot * RB + 16 * g + lr) * 4, 0, 17);
        }
      }
    }
    __syncthreads();
    {
      if constexpr (kTimeline) tl[12] = tl_now();
      // this wave's rows wave, wave+4, ...: all LDS reads first, then the stores
      uint16_t* obase = FUSE ? p.lat + (int64_t)r * p.qlen * p.lat_r + 8 * lane
                             : p.o + k * p.os_s + (int64_t)r * p.qlen * p.os_r + 8 * lane;
      const int wu = __builtin_amdgcn_readfirstlane(wave);
      u32x4 ov[RB / 4];
      int64_t off[RB / 4];
#pragma unroll
      for (int j = 0; j < RB / 4; ++j) {
        ov[j] = *reinterpret_cast<const MLA_LDS u32x4*>(ost + (wu + 4 * j) * O_PITCH + 8 * lane);
        off[j] = FUSE ? latoff[wu + 4 * j] : rowoff[wu + 4 * j];
      }
      // keep the reads together, ahead of the (conditional) stores
#pragma unroll
      for (int j = 0; j < RB / 4; ++j) asm volatile("" : "+v"(ov[j]), "+v"(off[j]));
      if (!FUSE || direct) {
#pragma unroll
        for (int j = 0; j < RB / 4; ++j)
          if ((wmask >> (wu + 4 * j)) & 1) *reinterpret_cast<u32x4*>(obase + off[j]) = ov[j];
      } else {
#pragma unroll
        for (int j = 0; j < RB / 4; ++j)
          if ((wmask >> (wu + 4 * j)) & 1)
            __builtin_amdgcn_raw_buffer_store_b128(ov[j], wsr, p.ws_o_off + (slot * RB + wu + 4 * j) * 1024 + 16 * lane,
                                                   0, 17);
      }
    }
    if constexpr (kTimeline) tl[13] = tl_now();
    if constexpr (FUSE) {
      if (!direct) {
        // Count this piece in once its rows are complete in memory (every
        // wave waits for its own system-coherent stores before the barrier);
        // the block that completes the count merges the request's splits,
        // reading them with system-coherent loads, and clears the counter
        // for the next call.
        wait_vm_all();
        __syncthreads();
        int32_t* cnt = p.ws_cnt + (int64_t)r * p.n_rb + rb;
        if (tid == 0) last_[0] = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __syncthreads();
        if (last_[0] == nsplit - 1) {
          const int nrows = min(RB, p.M - m_lo);
          auto slot_of = [&](int kk) -> int {
            return (int)((((kk == 0 ? vq : vq + kk) * 2) + (kk == 0 ? 1 : 0)) * p.n_rb + rb);
          };
#pragma unroll 1
          for (int gi = 0; gi < RB / 16; ++gi) {
            int rw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = wave + 4 * (4 * gi + j);
              rw[j] = row < nrows ? row : 0;
            }
            auto lse_at = [&](int j, int kk) -> float {
              return __builtin_bit_cast(
                  float, __builtin_amdgcn_raw_buffer_load_b32(wsr, p.ws_lse_off + (slot_of(kk) * RB + rw[j]) * 4, 0, 17));
            };
            auto o_at = [&](int j, int kk) -> u32x4 {
              return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   wsr, p.ws_o_off + (slot_of(kk) * RB + rw[j]) * 1024 + 16 * lane, 0, 17));
            };
            float l1[4];
            merge_lse_load_at<4>(lse_at, nsplit, lane, l1);
            u32x4 out[4];
            float total[4];
            merge_rows_at<4, false>(lse_at, o_at, nsplit, lane, l1, out, total);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = wave + 4 * (4 * gi + j);
              if (row < nrows) {
                *reinterpret_cast<u32x4*>(p.lat + (int64_t)r * p.qlen * p.lat_r + latoff[row] + 8 * lane) = out[j];
                if (p.lat_lse && lane == 0) {
                  const int m = m_lo + row;
                  p.lat_lse[((int64_t)r * p.qlen + m / p.heads) * p.ll_r + (int64_t)(m % p.heads) * p.ll_h] = total[j];
                }
              }
            }
          }
          if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
      }
    }
    __syncthreads();
  }
#ifdef MLA_WG_TIMELINE
  tl[1] = tl_now();
  tl[2] = (uint64_t)tl_piece;
  const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if (tid == 0 && lin < TL_MAX)
    for (int i = 0; i < 16; ++i) g_timeline[lin][i] = tl[i];
#endif
}

// The events that the next launch of the partial kernel records at its own
// start and end (mla_time_next_partial); taken by that launch.
static std::mutex g_time_mu;
static hipEvent_t g_time_ev[2] = {nullptr, nullptr};

template <int NRG, bool QF8, bool PLAN, bool FUSE = false, bool WRITE = false>
static int launch(const PartialArgs& a, const UnitPlan<PLAN>& pl, hipStream_t s,
                  const NewArgs<WRITE>& nw = NewArgs<WRITE>{}) {
  static_assert(sizeof(PartialArgs) + sizeof(UnitPlan<PLAN>) <= 4096, "kernel arguments over 4 KB");
  const dim3 grid(8, (unsigned)a.n_rb, ((unsigned)a.num_workers + 7) / 8);
  hipEvent_t ev[2];
  {
    std::lock_guard<std::mutex> lock(g_time_mu);
    ev[0] = g_time_ev[0];
    ev[1] = g_time_ev[1];
    g_time_ev[0] = g_time_ev[1] = nullptr;
  }
  if (ev[0] || ev[1])
    hipExtLaunchKernelGGL((partial_kernel<NRG, QF8, PLAN, FUSE, WRITE>), grid, dim3(256), 0, s, ev[0], ev[1], 0, a, pl, nw);
  else
    hipLaunchKernelGGL((partial_kernel<NRG, QF8, PLAN, FUSE, WRITE>), grid, dim3(256), 0, s, a, pl, nw);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// The kernel's split partition, unit by unit, on the host: the same chunk,
// and for each unit the first request whose stream end reaches the unit's
// start and the requests it covers (the kernel's search and scan).
static int make_plan(const int32_t* ip, int32_t batch, int32_t num_splits, int32_t num_workers,
                     int32_t split_min, UnitPlan<true>& pl) {
  constexpr int64_t W = MLA_PIECE_TOKENS;
  const int64_t base = ip[0];
  int64_t lmax = 0;
  for (int r = 0; r < batch; ++r) {
    const int64_t L = (int64_t)ip[r + 1] - ip[r];
    if (L < 0) return MLA_ERR_INVALID;
    if (L > lmax) lmax = L;
  }
  const int64_t Tv = (int64_t)ip[batch] - base + W * batch;
  const int64_t chunk = split_chunk(Tv, lmax, num_splits, num_workers, split_min);
  const int64_t nunits = Tv > 0 ? (Tv + chunk - 1) / chunk : 1;
  if (nunits > num_workers || nunits > PLAN_UNITS) return MLA_ERR_UNSUPPORTED;
  pl.chunk = chunk;
  pl.nunits = nunits;
  pl.Tv = Tv;
  pl.base = (int32_t)base;
  pl.pad_ = 0;
  int r = 0;
  for (int64_t u = 0; u < nunits; ++u) {
    const int64_t g0 = u * chunk, g1 = g0 + chunk < Tv ? g0 + chunk : Tv;
    while (r < batch && (int64_t)ip[r + 1] - base + W * (r + 1) < g0) ++r;  // ends only grow with r
    int r_end = r;
    while (r_end < batch) {
      const int64_t Vs = (int64_t)ip[r_end] - base + W * r_end;
      if (Vs >= g1 && !(u == nunits - 1 && Vs == Tv)) break;
      ++r_end;
    }
    if (r_end - r > 0xFFFF) return MLA_ERR_UNSUPPORTED;  // the count is 16-bit
    pl.r[u] = r;
    pl.nreq[u] = (uint16_t)(r_end - r);
    pl.p0[u] = r < batch ? (int32_t)(ip[r] - base) : 0;
    pl.len0[u] = r < batch ? ip[r + 1] - ip[r] : 0;
  }
  for (int64_t u = nunits; u < PLAN_UNITS; ++u) {
    pl.r[u] = pl.p0[u] = pl.len0[u] = 0;
    pl.nreq[u] = 0;
  }
  return MLA_OK;
}

}  // namespace mla

extern "C" int mla_split_plan(const int32_t* indptr, int32_t batch, int32_t num_splits,
                              int32_t num_workers, int32_t split_min_tokens, int32_t* bounds,
                              int64_t* chunk_out) {
  if (!indptr || !bounds || batch < 0 || num_splits < 1 || num_workers < 1) return MLA_ERR_INVALID;
  constexpr int64_t W = MLA_PIECE_TOKENS;
  int64_t T = (int64_t)indptr[batch] - indptr[0], lmax = 0;
  for (int r = 0; r < batch; ++r) {
    int64_t L = (int64_t)indptr[r + 1] - indptr[r];
    if (L < 0) return MLA_ERR_INVALID;
    if (L > lmax) lmax = L;
  }
  const int64_t chunk = mla::split_chunk(T + W * batch, lmax, num_splits, num_workers, split_min_tokens);
  for (int r = 0; r < batch; ++r) {
    const int64_t L = (int64_t)indptr[r + 1] - indptr[r];
    const int64_t V = (int64_t)indptr[r] - indptr[0] + W * (r + 1);  // first token's stream position
    int32_t* b = bounds + (int64_t)r * (num_splits + 1);
    int k = 0;
    b[k++] = 0;
    for (int64_t c = (V / chunk + 1) * chunk; c < V + L; c += chunk) {
      if (k >= num_splits) return MLA_ERR_INVALID;
      b[k++] = (int32_t)(c - V);
    }
    while (k <= num_splits) b[k++] = (int32_t)L;
  }
  if (chunk_out) *chunk_out = chunk;
  return MLA_OK;
}

namespace mla {

// Argument checks and kernel arguments shared by the partial and the fused
// entry points (bf16 or fp8 query).  q_scale multiplies every score (1 for
// bf16).  Sets the row-block geometry.
static int common_args(PartialArgs& a, int& nrg, const void* q, bool q_fp8, int64_t q_stride_row,
                       int64_t q_stride_head, float q_scale, int32_t batch, int32_t qlen, int32_t heads,
                       const uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                       const int32_t* kv_indices, float sm_scale, float kv_scale, int32_t num_splits,
                       int32_t num_workers, int32_t split_min_tokens) {
  if (!q || !kv_cache || !kv_indptr || !kv_indices) return MLA_ERR_INVALID;
  if (num_slots < 1 || num_slots > 0x7FFFFFFFLL) return MLA_ERR_INVALID;
  if (!(kv_scale > 0.0f) || !(sm_scale > 0.0f) || kv_scale == INFINITY || sm_scale == INFINITY)
    return MLA_ERR_INVALID;
  if (!(q_scale > 0.0f) || q_scale == INFINITY) return MLA_ERR_INVALID;
  // 16-byte query chunks (8 bf16 or 16 fp8 elements), 16-byte cache rows
  const int64_t q_align = q_fp8 ? 16 : 8;
  if ((q_stride_row | q_stride_head) % q_align != 0 || ((uintptr_t)q) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (((uintptr_t)kv_cache) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)qlen * heads;
  if (M > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  // rows per block: 16, 32 or 48 (larger requests take several blocks)
  nrg = M <= 16 ? 1 : (M <= 32 ? 2 : 3);
  const int n_rb = (int)((M + 16 * nrg - 1) / (16 * nrg));
  // the grid is (8, n_rb, ceil(num_workers / 8)) (n_rb <= 21846 here)
  if (((int64_t)num_workers + 7) / 8 > 65535) return MLA_ERR_UNSUPPORTED;
  a = PartialArgs{};
  a.q = q_fp8 ? nullptr : (const uint16_t*)q;
  a.q8 = q_fp8 ? (const uint8_t*)q : nullptr;
  a.q_sr = q_stride_row; a.q_sh = q_stride_head;
  a.batch = batch; a.qlen = qlen; a.heads = heads; a.M = (int32_t)M; a.n_rb = n_rb;
  a.kv = kv_cache; a.num_slots = num_slots; a.indptr = kv_indptr; a.indices = kv_indices;
  a.c_log2 = sm_scale * kv_scale * q_scale * kLog2e;  // q_scale = 1: sm_scale * kv_scale * log2(e)
  a.kv_scale = kv_scale;
  a.num_splits = num_splits; a.num_workers = num_workers; a.split_min = split_min_tokens;
  return MLA_OK;
}

// the new tokens of the fused cache write (per_request of them for each
// request, the request's last ones), written to the call's kv_cache
struct NewRows {
  const uint16_t* kv_c;
  int64_t kv_c_stride;
  const uint16_t* k_pe;
  int64_t k_pe_stride;
  const int64_t* slots;
  int32_t per_request;
};

static int decode_partial_impl(const void* q, bool q_fp8, int64_t q_stride_row, int64_t q_stride_head,
                               float q_scale, int32_t batch, int32_t qlen, int32_t heads,
                               const uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                               const int32_t* kv_indices, float sm_scale, float kv_scale,
                               int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                               uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                               float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                               void* stream, const int32_t* indptr_host = nullptr,
                               const NewRows* nw = nullptr) {
  if (batch < 0 || qlen < 1 || heads < 1 || num_splits < 1 || num_splits > 1024 || num_workers < 1)
    return MLA_ERR_INVALID;
  if (nw) {
    if (!nw->kv_c || !nw->k_pe || !nw->slots || nw->kv_c_stride < MLA_D_LATENT || nw->k_pe_stride < MLA_D_ROPE)
      return MLA_ERR_INVALID;
    if (nw->per_request < 1 || nw->per_request > NEW_MAX) return MLA_ERR_INVALID;
    // 16-byte row loads
    if (((uintptr_t)nw->kv_c | (uintptr_t)nw->k_pe) % 16 != 0 || (nw->kv_c_stride | nw->k_pe_stride) % 8 != 0)
      return MLA_ERR_UNSUPPORTED;
  }
  if (batch == 0) return MLA_OK;
  if (!o_part || !lse_part) return MLA_ERR_INVALID;
  PartialArgs a;
  int nrg = 3;
  int st = common_args(a, nrg, q, q_fp8, q_stride_row, q_stride_head, q_scale, batch, qlen, heads, kv_cache,
                       num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits, num_workers, split_min_tokens);
  if (st != MLA_OK) return st;
  // 8-byte partial stores
  if ((os_split | os_row | os_head) % 4 != 0 || ((uintptr_t)o_part) % 8 != 0) return MLA_ERR_UNSUPPORTED;
  a.o = o_part; a.os_s = os_split; a.os_r = os_row; a.os_h = os_head;
  a.lse = lse_part; a.ls_s = ls_split; a.ls_r = ls_row; a.ls_h = ls_head;
  hipStream_t s = (hipStream_t)stream;
  UnitPlan<true> pl;
  if (indptr_host)
    for (int32_t r = 0; r < batch; ++r)
      if (indptr_host[r + 1] < indptr_host[r]) return MLA_ERR_INVALID;
  st = indptr_host && num_workers <= PLAN_UNITS
           ? make_plan(indptr_host, batch, num_splits, num_workers, split_min_tokens, pl)
           : MLA_ERR_UNSUPPORTED;
  if (st == MLA_ERR_INVALID) return st;
  const bool wr = nw != nullptr;
  NewArgs<true> nwa{};
  if (nw) nwa = NewArgs<true>{nw->kv_c, nw->k_pe, nw->kv_c_stride, nw->k_pe_stride, nw->slots, nw->per_request};
  if (st == MLA_OK) {
    if (q_fp8) {
      switch (nrg) {
        case 1: return wr ? launch<1, true, true, false, true>(a, pl, s, nwa) : launch<1, true, true>(a, pl, s);
        case 2: return wr ? launch<2, true, true, false, true>(a, pl, s, nwa) : launch<2, true, true>(a, pl, s);
        default: return wr ? launch<3, true, true, false, true>(a, pl, s, nwa) : launch<3, true, true>(a, pl, s);
      }
    }
    switch (nrg) {
      case 1: return wr ? launch<1, false, true, false, true>(a, pl, s, nwa) : launch<1, false, true>(a, pl, s);
      case 2: return wr ? launch<2, false, true, false, true>(a, pl, s, nwa) : launch<2, false, true>(a, pl, s);
      default: return wr ? launch<3, false, true, false, true>(a, pl, s, nwa) : launch<3, false, true>(a, pl, s);
    }
  }
  const UnitPlan<false> none;
  if (q_fp8) {
    switch (nrg) {
      case 1: return wr ? launch<1, true, false, false, true>(a, none, s, nwa) : launch<1, true, false>(a, none, s);
      case 2: return wr ? launch<2, true, false, false, true>(a, none, s, nwa) : launch<2, true, false>(a, none, s);
      default: return wr ? launch<3, true, false, false, true>(a, none, s, nwa) : launch<3, true, false>(a, none, s);
    }
  }
  switch (nrg) {
    case 1: return wr ? launch<1, false, false, false, true>(a, none, s, nwa) : launch<1, false, false>(a, none, s);
    case 2: return wr ? launch<2, false, false, false, true>(a, none, s, nwa) : launch<2, false, false>(a, none, s);
    default: return wr ? launch<3, false, false, false, true>(a, none, s, nwa) : launch<3, false, false>(a, none, s);
  }
}

// The fused call's workspace: the counters (one int32 per request and row
// block), then the partial LSEs [slot][RB] f32 and rows [slot][RB][512] bf16
// of two slots per unit and row block, each part 256-byte aligned.
struct AttendLayout {
  int64_t cnt_bytes, lse_bytes, o_bytes, total;
};
static AttendLayout attend_layout(int32_t batch, int32_t qlen, int32_t heads, int32_t num_workers) {
  const int64_t M = (int64_t)qlen * heads;
  const int nrg = M <= 16 ? 1 : (M <= 32 ? 2 : 3);
  const int64_t rb_rows = 16 * nrg, n_rb = (M + rb_rows - 1) / rb_rows;
  const int64_t slots = 2 * (int64_t)(num_workers < PLAN_UNITS ? num_workers : PLAN_UNITS) * n_rb;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  AttendLayout l;
  l.cnt_bytes = al(4 * (int64_t)batch * n_rb);
  l.lse_bytes = al(4 * slots * rb_rows);
  l.o_bytes = slots * rb_rows * 1024;
  l.total = l.cnt_bytes + l.lse_bytes + l.o_bytes;
  return l;
}

static int attend_impl(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head, int32_t batch, int32_t qlen,
                       int32_t heads, const uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                       const int32_t* kv_indices, float sm_scale, float kv_scale, int32_t num_splits,
                       int32_t num_workers, int32_t split_min_tokens, const int32_t* indptr_host, uint16_t* o,
                       int64_t o_row, int64_t o_head, float* lse, int64_t l_row, int64_t l_head, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (batch < 0 || qlen < 1 || heads < 1 || num_splits < 1 || num_splits > 1024 || num_workers < 1)
    return MLA_ERR_INVALID;
  if (batch == 0) return MLA_OK;
  if (!o || !workspace || !indptr_host) return MLA_ERR_INVALID;
  PartialArgs a;
  int nrg = 3;
  int st = common_args(a, nrg, q, false, q_stride_row, q_stride_head, 1.0f, batch, qlen, heads, kv_cache,
                       num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits, num_workers, split_min_tokens);
  if (st != MLA_OK) return st;
  if (num_workers > PLAN_UNITS) return MLA_ERR_UNSUPPORTED;
  // 16-byte latent row stores; a 256-byte aligned workspace addressed with
  // 32-bit offsets
  if ((o_row | o_head) % 8 != 0 || ((uintptr_t)o) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (((uintptr_t)workspace) % 256 != 0) return MLA_ERR_UNSUPPORTED;
  const AttendLayout lay = attend_layout(batch, qlen, heads, num_workers);
  if (lay.total > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < lay.total) return MLA_ERR_INVALID;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr_host[r + 1] < indptr_host[r]) return MLA_ERR_INVALID;
  UnitPlan<true> pl;
  st = make_plan(indptr_host, batch, num_splits, num_workers, split_min_tokens, pl);
  if (st != MLA_OK) return st;
  a.lat = o; a.lat_r = o_row; a.lat_h = o_head;
  a.lat_lse = lse; a.ll_r = l_row; a.ll_h = l_head;
  a.ws_cnt = reinterpret_cast<int32_t*>(workspace);
  a.ws = reinterpret_cast<uint8_t*>(workspace);
  a.ws_lse_off = (int32_t)lay.cnt_bytes;
  a.ws_o_off = (int32_t)(lay.cnt_bytes + lay.lse_bytes);
  hipStream_t s = (hipStream_t)stream;
  switch (nrg) {
    case 1: return launch<1, false, true, true>(a, pl, s);
    case 2: return launch<2, false, true, true>(a, pl, s);
    default: return launch<3, false, true, true>(a, pl, s);
  }
}

// The no-allocation call's workspace: one array per GPU in the library's
// device memory.  Its device address is taken once per device, with that
// device current, at the first call there; kernels only ever see that
// address (the array's name is a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[MLA_ATTEND_NOALLOC_MAX_BYTES];
constexpr int MAX_DEVICES = 64;
static void* g_scratch[MAX_DEVICES];
static std::mutex g_scratch_mu;

static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MLA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace mla

extern "C" int mla_decode_partial(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                                  int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                                  int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                                  float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                                  int32_t split_min_tokens, uint16_t* o_part, int64_t os_split,
                                  int64_t os_row, int64_t os_head, float* lse_part, int64_t ls_split,
                                  int64_t ls_row, int64_t ls_head, void* stream) {
  return mla::decode_partial_impl(q, false, q_stride_row, q_stride_head, 1.0f, batch, qlen, heads, kv_cache,
                                  num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream);
}

extern "C" int mla_decode_partial_fp8q(const uint8_t* q8, int64_t q_stride_row, int64_t q_stride_head,
                                       float q_scale, int32_t batch, int32_t qlen, int32_t heads,
                                       const uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                                       const int32_t* kv_indices, float sm_scale, float kv_scale,
                                       int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                                       uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                                       float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                                       void* stream) {
  return mla::decode_partial_impl(q8, true, q_stride_row, q_stride_head, q_scale, batch, qlen, heads,
                                  kv_cache, num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream);
}

extern "C" int mla_decode_partial_hostplan(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                                           int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                                           int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                                           float sm_scale, float kv_scale, int32_t num_splits,
                                           int32_t num_workers, int32_t split_min_tokens, uint16_t* o_part,
                                           int64_t os_split, int64_t os_row, int64_t os_head, float* lse_part,
                                           int64_t ls_split, int64_t ls_row, int64_t ls_head,
                                           const int32_t* kv_indptr_host, void* stream) {
  if (!kv_indptr_host && batch > 0) return MLA_ERR_INVALID;
  return mla::decode_partial_impl(q, false, q_stride_row, q_stride_head, 1.0f, batch, qlen, heads, kv_cache,
                                  num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream, kv_indptr_host);
}

extern "C" int mla_decode_partial_fp8q_hostplan(const uint8_t* q8, int64_t q_stride_row, int64_t q_stride_head,
                                                float q_scale, int32_t batch, int32_t qlen, int32_t heads,
                                                const uint8_t* kv_cache, int64_t num_slots,
                                                const int32_t* kv_indptr, const int32_t* kv_indices,
                                                float sm_scale, float kv_scale, int32_t num_splits,
                                                int32_t num_workers, int32_t split_min_tokens, uint16_t* o_part,
                                                int64_t os_split, int64_t os_row, int64_t os_head,
                                                float* lse_part, int64_t ls_split, int64_t ls_row,
                                                int64_t ls_head, const int32_t* kv_indptr_host, void* stream) {
  if (!kv_indptr_host && batch > 0) return MLA_ERR_INVALID;
  return mla::decode_partial_impl(q8, true, q_stride_row, q_stride_head, q_scale, batch, qlen, heads,
                                  kv_cache, num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream, kv_indptr_host);
}

extern "C" int mla_kv_write_decode_partial_hostplan(
    const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe, int64_t k_pe_stride,
    const int64_t* slot_mapping, int32_t new_per_request, const uint16_t* q, int64_t q_stride_row,
    int64_t q_stride_head, int32_t batch, int32_t qlen, int32_t heads, uint8_t* kv_cache, int64_t num_slots,
    const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float kv_scale, int32_t num_splits,
    int32_t num_workers, int32_t split_min_tokens, uint16_t* o_part, int64_t os_split, int64_t os_row,
    int64_t os_head, float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
    const int32_t* kv_indptr_host, void* stream) {
  if (!kv_indptr_host && batch > 0) return MLA_ERR_INVALID;
  const mla::NewRows nw{kv_c, kv_c_stride, k_pe, k_pe_stride, slot_mapping, new_per_request};
  return mla::decode_partial_impl(q, false, q_stride_row, q_stride_head, 1.0f, batch, qlen, heads, kv_cache,
                                  num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream, kv_indptr_host, &nw);
}

extern "C" int mla_kv_write_decode_partial_fp8q_hostplan(
    const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe, int64_t k_pe_stride,
    const int64_t* slot_mapping, int32_t new_per_request, const uint8_t* q8, int64_t q_stride_row,
    int64_t q_stride_head, float q_scale, int32_t batch, int32_t qlen, int32_t heads, uint8_t* kv_cache,
    int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float kv_scale,
    int32_t num_splits, int32_t num_workers, int32_t split_min_tokens, uint16_t* o_part, int64_t os_split,
    int64_t os_row, int64_t os_head, float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
    const int32_t* kv_indptr_host, void* stream) {
  if (!kv_indptr_host && batch > 0) return MLA_ERR_INVALID;
  const mla::NewRows nw{kv_c, kv_c_stride, k_pe, k_pe_stride, slot_mapping, new_per_request};
  return mla::decode_partial_impl(q8, true, q_stride_row, q_stride_head, q_scale, batch, qlen, heads,
                                  kv_cache, num_slots, kv_indptr, kv_indices, sm_scale, kv_scale, num_splits,
                                  num_workers, split_min_tokens, o_part, os_split, os_row, os_head, lse_part,
                                  ls_split, ls_row, ls_head, stream, kv_indptr_host, &nw);
}

extern "C" int64_t mla_decode_attend_workspace_bytes(int32_t batch, int32_t qlen, int32_t heads, int32_t num_workers) {
  if (batch < 0 || qlen < 1 || heads < 1 || num_workers < 1) return -MLA_ERR_INVALID;
  return mla::attend_layout(batch, qlen, heads, num_workers).total;
}

extern "C" int mla_decode_attend(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head, int32_t batch,
                                 int32_t qlen, int32_t heads, const uint8_t* kv_cache, int64_t num_slots,
                                 const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float kv_scale,
                                 int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                                 const int32_t* kv_indptr_host, uint16_t* o, int64_t o_row, int64_t o_head,
                                 float* lse, int64_t l_row, int64_t l_head, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  return mla::attend_impl(q, q_stride_row, q_stride_head, batch, qlen, heads, kv_cache, num_slots, kv_indptr,
                          kv_indices, sm_scale, kv_scale, num_splits, num_workers, split_min_tokens, kv_indptr_host,
                          o, o_row, o_head, lse, l_row, l_head, workspace, workspace_bytes, stream);
}

extern "C" int mla_decode_attend_noalloc(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                                         int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                                         int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                                         float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                                         int32_t split_min_tokens, const int32_t* kv_indptr_host, uint16_t* o,
                                         int64_t o_row, int64_t o_head, float* lse, int64_t l_row, int64_t l_head,
                                         void* stream) {
  if (batch < 0 || qlen < 1 || heads < 1 || num_workers < 1) return MLA_ERR_INVALID;
  if (batch == 0) return MLA_OK;
  if (mla::attend_layout(batch, qlen, heads, num_workers).total > MLA_ATTEND_NOALLOC_MAX_BYTES)
    return MLA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const int st = mla::scratch_address(&ws);
  if (st != MLA_OK) return st;
  return mla::attend_impl(q, q_stride_row, q_stride_head, batch, qlen, heads, kv_cache, num_slots, kv_indptr,
                          kv_indices, sm_scale, kv_scale, num_splits, num_workers, split_min_tokens, kv_indptr_host,
                          o, o_row, o_head, lse, l_row, l_head, ws, MLA_ATTEND_NOALLOC_MAX_BYTES, stream);
}

extern "C" int mla_time_next_partial(void* start_event, void* stop_event) {
  std::lock_guard<std::mutex> lock(mla::g_time_mu);
  mla::g_time_ev[0] = (hipEvent_t)start_event;
  mla::g_time_ev[1] = (hipEvent_t)stop_event;
  return MLA_OK;
}

#ifdef MLA_WG_TIMELINE
// The measurement build's timeline (the marks described at g_timeline):
// records 0 .. n-1 (n <= 4096) to host memory, 16 uint64 each; and a clear
// of every record (a workgroup that finds no unit writes none).  Both wait
// for the device.
extern "C" int mla_wg_timeline(uint64_t* host, int32_t n) {
  if (!host || n < 0 || n > mla::TL_MAX) return MLA_ERR_INVALID;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(mla::g_timeline), sizeof(uint64_t) * 16 * (size_t)n) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

extern "C" int mla_wg_timeline_clear() {
  static uint64_t zero[mla::TL_MAX][16];
  return hipMemcpyToSymbol(HIP_SYMBOL(mla::g_timeline), zero, sizeof(zero)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
#endif
