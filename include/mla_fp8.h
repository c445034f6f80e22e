/*
 * mla_fp8.h — C ABI of the MLA decode hot path over an fp8 latent KV cache
 * (gfx950 / MI355X).
 *
 * The path, as the vLLM pages "vllm.models.kimi_k3.amd.specialized_decode.
 * runtime.mla" (sections `pre`, `attend`, `m1c_inputs`, `post`) and
 * "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.mla.value"
 * (classes `MlaValue`, `MlaGate`) describe it:
 *
 *   mla_kv_write        new tokens' [kv_c | k_pe] rows -> fp8 cache rows
 *   mla_absorb_query    q_nope x W_UK (MXFP4) concatenated with q_pe -> the
 *                       absorbed query rows (bf16, or fp8 with q_scale)
 *   mla_concat_quant_fp8  absorbed query [ql_nope | q_pe] -> fp8 query rows
 *   mla_decode_partial  absorbed queries attend over the paged fp8 cache:
 *                       split-KV partials o (bf16) and LSE (f32)
 *   mla_decode_partial_fp8q  the same for an fp8 query with a per-tensor scale
 *   mla_decode_partial_hostplan, mla_decode_partial_fp8q_hostplan  the two
 *                       above with the split partition computed on the host
 *   mla_kv_write_decode_partial_hostplan, _fp8q_hostplan  the cache write
 *                       and the host-planned partials in one launch
 *   mla_decode_attend   the attention and the LSE merge in one launch ->
 *                       latent (bf16) and LSE, with a caller's workspace
 *   mla_decode_attend_noalloc  the same with the library's own workspace
 *   mla_merge_lse       LSE merge of the splits -> latent (bf16)
 *   mla_value_gate      per-head W_UV (bf16 or MXFP4) + FP32 sigmoid gate
 *   mla_merge_value_gate  the merge, W_UV and gate in one call (no latent written)
 *   mla_time_next_partial  (measurement) events the next partial launch records
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     the argument says "host".  The library keeps no pointer after a call
 *     returns (mla_time_next_partial's event handles excepted), allocates
 *     nothing, and never synchronizes: work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream).
 *   - bf16 data is passed as uint16_t (raw bits), fp8 E4M3 (OCP "fn": bias
 *     7, max 448, 0x7F/0xFF NaN, no infinities) as uint8_t.
 *   - Strides are in ELEMENTS of the pointed-to type; the innermost axis of
 *     every array is contiguous.
 *   - Return value: MLA_OK, or an error code from the list below.  Argument
 *     checks happen on the host before anything is enqueued; on an error
 *     nothing is enqueued.  MLA_ERR_HIP reports a failed launch.
 *   - Index validity (slot_mapping, kv_indices inside [0, num_slots)) is the
 *     caller's guarantee; a cache index outside that range reads as fp8 NaN
 *     (so it poisons the rows that use it instead of faulting).
 */
#ifndef MLA_FP8_H
#define MLA_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID 1     /* a null pointer, bad size or bad stride   */
#define MLA_ERR_UNSUPPORTED 2 /* valid but outside what the kernels cover */
#define MLA_ERR_HIP 3         /* the HIP runtime reported an error        */

#define MLA_D_LATENT 512 /* kv_lora_rank: value width of a cache row */
#define MLA_D_ROPE 64    /* rope width */
#define MLA_D_QK 576     /* one cache row: 512 latent then 64 rope   */
#define MLA_D_V 128      /* v_head_dim: W_UV output width per head    */

/* Partition weight: in the token stream the split partition cuts, each
 * request takes this many positions before its tokens, so that units which
 * start more pieces (each with a fixed start-up cost) get fewer tokens. */
#define MLA_PIECE_TOKENS 320

#define MLA_W_BF16 0
#define MLA_W_MXFP4 1

/* Text for a status code (static storage; never NULL). */
const char* mla_status_string(int status);

/*
 * Cache write of new tokens ([MLA] `pre`: do_kv_cache_update(kv_c, k_pe,
 * kv_cache, slots, ..., k_scale)).  Token i's cache row is
 *   kv_cache[slot_mapping[i]][c] = E(x_c / kv_scale),  c < 576,
 * with x = [kv_c[i][0:512] | k_pe[i][0:64]] (bf16), the division a correctly
 * rounded binary32 division, and E the fp8 E4M3 encoder rounding to nearest
 * even and saturating to +-448 (NaN -> 0x7F).  A negative slot skips the
 * token.  Slots must be distinct.
 *   kv_c         [n][kv_c_stride] bf16, first 512 used (e.g. a view of a
 *                fused projection output, stride >= 512)
 *   k_pe         [n][k_pe_stride] bf16, first 64 used
 *   slot_mapping [n] int64
 *   kv_cache     [num_slots][576] u8, rows contiguous
 * n = 0 is a no-op.
 * Errors: MLA_ERR_INVALID for n < 0, num_slots < 0, a null pointer,
 * kv_c_stride < 512, k_pe_stride < 64, or kv_scale not positive and finite;
 * MLA_ERR_UNSUPPORTED when n * 72 threads exceed one launch grid.
 */
int mla_kv_write(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                 int64_t k_pe_stride, const int64_t* slot_mapping, int32_t n, uint8_t* kv_cache,
                 int64_t num_slots, float kv_scale, void* stream);

/*
 * The absorbed query ([MLA] `pre`: ql_nope = batched_gemm_a16wfp4(q_nope^T,
 * W_K, W_K_scale, transpose_bm, prequant, y_scale), then the concat with q_pe
 * and, on the fp8 path, the quantisation).  For row t < rows, head h < heads:
 *   xq = q_nope[t][h][0:128] quantised to MXFP4 in blocks of 32 (OCP MX:
 *        shared exponent X = floor(log2 max|v|) - 2 held to [-127, 127], each
 *        v / 2^X rounded to the nearest E2M1 value with ties to the even code,
 *        past 6 clamped to 6; a block holding NaN or inf gives NaN),
 *   y[n] = sum_k xq[k] * W_K[h][n][k]   (n < 512, W_K decoded exactly;
 *        products exact, sums in binary32),
 *   out_fp8 = 0:  out[t][h][0:512] = bf16(y),  out[t][h][512:576] = q_pe[t][h]
 *   out_fp8 = 1:  out[t][h][0:512] = E(y / q_scale),
 *                 out[t][h][512:576] = E(q_pe[t][h] / q_scale)
 * (correctly rounded binary32 divisions, E the encoder of mla_kv_write), so
 * the fp8 rows are the q8 of mla_decode_partial_fp8q with this q_scale.
 *   q_nope   [rows][heads][128] bf16, strides (qn_row, qn_head)
 *   q_pe     [rows][heads][64] bf16, strides (qp_row, qp_head) (e.g. the two
 *            slices of a [rows][heads][192] projection output); strides
 *            multiples of 8, both 16-byte aligned
 *   w_k      [heads][512][64] u8: row n of head h holds 128 E2M1 codes, two
 *            per byte, element 2j in the low nibble; strides (wk_head, wk_n)
 *            in bytes
 *   wk_scale [heads][512][4] u8 E8M0 (2^(s-127); 0xFF NaN), one per 32 along
 *            k; strides (wks_head, wks_n) in bytes; strides of w_k and
 *            wk_scale multiples of 4, both 4-byte aligned
 *   out      [rows][heads][576] bf16 (out_fp8 = 0) or u8 codes (out_fp8 = 1),
 *            strides (out_row, out_head) in its elements, multiples of 8
 *            (bf16) or 16 (fp8), 16-byte aligned (e.g. the query buffer of
 *            mla_decode_partial with padded heads)
 * Errors: MLA_ERR_INVALID for rows < 0, heads < 1, out_fp8 not 0 or 1, a null
 * pointer, or (out_fp8 = 1) q_scale not > 0 and finite; MLA_ERR_UNSUPPORTED
 * for the alignment rules above or heads > 65535.  rows = 0 is a no-op.
 */
int mla_absorb_query(const uint16_t* q_nope, int64_t qn_row, int64_t qn_head, const uint16_t* q_pe,
                     int64_t qp_row, int64_t qp_head, const uint8_t* w_k, int64_t wk_head, int64_t wk_n,
                     const uint8_t* wk_scale, int64_t wks_head, int64_t wks_n, int32_t rows, int32_t heads,
                     int32_t out_fp8, float q_scale, void* out, int64_t out_row, int64_t out_head,
                     void* stream);

/*
 * The fp8 query ([MLA] `pre`: _decode_concat_quant_fp8_op(ql_nope, q_pe,
 * q_scale), whose output `attend` decodes on).  For row t < rows, head
 * h < heads, c < 576, with x = [ql_nope[t][h][0:512] | q_pe[t][h][0:64]] (bf16):
 *   q8[t][h][c] = E(x_c / q_scale),
 * the division a correctly rounded binary32 division and E the encoder of
 * mla_kv_write (round to nearest even, saturate to +-448, NaN -> 0x7F).  The
 * result is the q8 of mla_decode_partial_fp8q, with the same q_scale.
 *   ql_nope [rows][heads][512] bf16, strides (ln_row, ln_head), multiples of 8
 *   q_pe    [rows][heads][64] bf16, strides (pe_row, pe_head), multiples of 8
 *           (e.g. the rope slice of a [rows][heads][192] projection output)
 *           both 16-byte aligned
 *   q8      [rows][heads][576] u8, strides (q8_row, q8_head), multiples of 8,
 *           8-byte aligned (otherwise MLA_ERR_UNSUPPORTED)
 *   q_scale > 0 and finite (otherwise MLA_ERR_INVALID)
 * rows = 0 is a no-op.
 */
int mla_concat_quant_fp8(const uint16_t* ql_nope, int64_t ln_row, int64_t ln_head, const uint16_t* q_pe,
                         int64_t pe_row, int64_t pe_head, float q_scale, int32_t rows, int32_t heads,
                         uint8_t* q8, int64_t q8_row, int64_t q8_head, void* stream);

/*
 * Split-KV partial attention ([MLA] `attend`, `m1c_inputs`: partials
 * o [splits, S, H, 512] bf16 and LSE [splits, S, H] f32, merged afterwards).
 *
 * Rows: S = batch * qlen query rows; row t = r*qlen + j belongs to request
 * r.  Request r's cache rows are kv_indices[kv_indptr[r] .. kv_indptr[r+1])
 * (page size 1, CSR), L_r = kv_indptr[r+1] - kv_indptr[r] tokens; the
 * cache already holds the request's qlen newest tokens, and row j sees its
 * first L_r - qlen + j + 1 tokens (causal within the speculative window).
 *
 * For head h < heads, over a token range [a, b) of the row's visible tokens:
 *   s_i = sm_scale * kv_scale * sum_{d<576} q[t][h][d] * fp8(kv[row_i][d])
 *   LSE = ln sum_i exp(s_i),   o = kv_scale * sum_i exp(s_i - LSE) * fp8(kv[row_i][0:512])
 * The ranges are the splits.  In a stream where request r (kv_indices
 * order) takes MLA_PIECE_TOKENS positions followed by its L_r tokens (its
 * first token at V_r = kv_indptr[r] - kv_indptr[0] + MLA_PIECE_TOKENS*(r+1)),
 * of length T_v = T + MLA_PIECE_TOKENS*batch, a cut falls every `chunk`
 * positions,
 *   chunk = max(split_min_tokens, ceil(T_v / num_workers), ceil(L_max / (num_splits-1)))
 *   (chunk = max(split_min_tokens, T_v) when num_splits == 1),
 * T the total tokens and L_max the longest request; split k of request r is
 * its k-th piece between cuts (mla_split_plan computes the same partition
 * on the host).  One workgroup set processes one chunk, so the work, counted
 * as tokens plus a fixed cost per piece, is balanced across num_workers
 * workers.
 *
 * Outputs, for every k < num_splits, t < S, h < heads:
 *   lse_part[k*ls_split + t*ls_row + h*ls_head]          f32, -inf if split k is
 *                                                         empty for row t
 *   o_part[k*os_split + t*os_row + h*os_head + d]        bf16 (d < 512), written only
 *                                                         where the LSE is finite
 * q: [S][...][576] bf16 with strides (q_stride_row, q_stride_head); the
 * query buffer may carry padded heads beyond `heads` (never read).
 * kv_cache: [num_slots][576] u8.  Requires 1 <= num_splits <= 1024,
 * num_workers >= 1, qlen >= 1, heads >= 1.  batch = 0 is a no-op.
 * Errors: MLA_ERR_INVALID for a size outside those ranges, batch < 0, a null
 * pointer, num_slots outside [1, 2^31 - 1], or sm_scale or kv_scale not
 * positive and finite; MLA_ERR_UNSUPPORTED unless q is 16-byte aligned with strides
 * that are multiples of 8, o_part is 8-byte aligned with strides that are
 * multiples of 4 and kv_cache is 16-byte aligned, or when qlen * heads
 * exceeds 2^20 or num_workers exceeds one launch grid (524280).
 */
int mla_decode_partial(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                       int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                       int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                       float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                       int32_t split_min_tokens, uint16_t* o_part, int64_t os_split, int64_t os_row,
                       int64_t os_head, float* lse_part, int64_t ls_split, int64_t ls_row,
                       int64_t ls_head, void* stream);

/*
 * The same split-KV partials for an fp8 query ([MLA] `pre` quantises the
 * absorbed query to fp8 E4M3 with one per-tensor scale, and `attend` decodes
 * on that quantised query).  Query element d of row t, head h stands for
 *   q_scale * fp8(q8[t][h][d]),
 * so every score is the bf16-query formula above with q replaced by that
 * value:  s_i = sm_scale * kv_scale * q_scale * sum_d fp8(q8) * fp8(kv).
 * Everything else (rows, causal rule, split partition, outputs, errors) is
 * as for mla_decode_partial.
 *   q8       [S][...][576] u8 E4M3 codes, strides (q_stride_row,
 *            q_stride_head) in bytes, both multiples of 16, q8 16-byte
 *            aligned (otherwise MLA_ERR_UNSUPPORTED)
 *   q_scale  > 0 and finite (otherwise MLA_ERR_INVALID)
 */
int mla_decode_partial_fp8q(const uint8_t* q8, int64_t q_stride_row, int64_t q_stride_head, float q_scale,
                            int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                            int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                            float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                            int32_t split_min_tokens, uint16_t* o_part, int64_t os_split,
                            int64_t os_row, int64_t os_head, float* lse_part, int64_t ls_split,
                            int64_t ls_row, int64_t ls_head, void* stream);

/*
 * mla_decode_partial for a bf16 query, with the split partition computed on
 * the host.  Same arguments, outputs and errors as mla_decode_partial, plus
 *   kv_indptr_host [batch+1] int32 (HOST): the same offsets as kv_indptr,
 *                  which stays a device pointer (the kernel still reads the
 *                  offsets of requests beyond a unit's first from it)
 * The host computes each unit's first request and range (the partition
 * described at mla_decode_partial) and passes them in the kernel
 * arguments, so a workgroup starts its first piece without reading and
 * searching the offsets.  The results are bit for bit those of
 * mla_decode_partial.  Up to 256 workers, and units of up to 65535
 * requests; beyond either, the call runs as mla_decode_partial.
 * kv_indptr_host is read during the call only.  It must hold exactly the
 * offsets of kv_indptr: a host copy that differs is undefined behaviour
 * (the first piece of a unit takes its range from the host copy and could
 * read kv_indices outside the request).  A split index that the mismatch
 * would push past num_splits is never written: that piece sets LSE NaN in
 * split num_splits-1 of its rows instead.
 * Errors: those of mla_decode_partial, and MLA_ERR_INVALID for a null
 * kv_indptr_host (batch > 0) or a decreasing offset in it (checked for any
 * worker count).
 */
int mla_decode_partial_hostplan(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head,
                                int32_t batch, int32_t qlen, int32_t heads, const uint8_t* kv_cache,
                                int64_t num_slots, const int32_t* kv_indptr, const int32_t* kv_indices,
                                float sm_scale, float kv_scale, int32_t num_splits, int32_t num_workers,
                                int32_t split_min_tokens, uint16_t* o_part, int64_t os_split,
                                int64_t os_row, int64_t os_head, float* lse_part, int64_t ls_split,
                                int64_t ls_row, int64_t ls_head, const int32_t* kv_indptr_host,
                                void* stream);

/*
 * mla_decode_partial_fp8q with the split partition computed on the host, as
 * mla_decode_partial_hostplan does for a bf16 query: the same arguments,
 * outputs and errors as mla_decode_partial_fp8q, plus kv_indptr_host
 * [batch+1] int32 (HOST), under the same rules.  The results are bit for
 * bit those of mla_decode_partial_fp8q.
 */
int mla_decode_partial_fp8q_hostplan(const uint8_t* q8, int64_t q_stride_row, int64_t q_stride_head,
                                     float q_scale, int32_t batch, int32_t qlen, int32_t heads,
                                     const uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                                     const int32_t* kv_indices, float sm_scale, float kv_scale,
                                     int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                                     uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                                     float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                                     const int32_t* kv_indptr_host, void* stream);

/*
 * The cache write of the new tokens ([MLA] `pre`: do_kv_cache_update) and
 * the split-KV partials over the updated cache ([MLA] `attend`) in one
 * launch: the cache bytes of mla_kv_write followed by the partials of
 * mla_decode_partial_hostplan, bit for bit.  Arguments: those of
 * mla_kv_write for the new tokens (without n, num_slots and kv_scale, which
 * are the partials' own), new_per_request, then those of
 * mla_decode_partial_hostplan, with kv_cache written.
 *   new_per_request  k, 1..8: the batch * k new tokens are the last k
 *                tokens of each request, request-major: kv_c, k_pe and
 *                slot_mapping row r * k + j is request r's token at
 *                position L_r - k + j (kv_indices[kv_indptr[r] + L_r - k + j]
 *                normally names slot_mapping[r * k + j]).  A token at a
 *                negative position (L_r < k) is written and not attended.
 *   kv_c, k_pe   16-byte aligned, strides multiples of 8 elements.
 * Each workgroup that attends a new token writes that token's row itself,
 * and has the store completed before it loads the tile that holds the
 * token, so the launch needs no ordering between workgroups.  In return, a slot this call writes must be
 * named in kv_indices at no position other than its own token's (as a slot
 * freshly given to a request is); where it is, which row such a read sees
 * is unspecified.  Slots must be distinct, as for mla_kv_write; a slot
 * outside [0, num_slots) skips its token.
 * Errors: those of mla_decode_partial_hostplan, and MLA_ERR_INVALID for a
 * null kv_c, k_pe or slot_mapping, kv_c_stride < 512, k_pe_stride < 64 or
 * new_per_request outside 1..8; MLA_ERR_UNSUPPORTED for rows that are not
 * 16-byte aligned.  batch = 0 is a no-op.
 */
int mla_kv_write_decode_partial_hostplan(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                                         int64_t k_pe_stride, const int64_t* slot_mapping,
                                         int32_t new_per_request, const uint16_t* q, int64_t q_stride_row,
                                         int64_t q_stride_head, int32_t batch, int32_t qlen, int32_t heads,
                                         uint8_t* kv_cache, int64_t num_slots, const int32_t* kv_indptr,
                                         const int32_t* kv_indices, float sm_scale, float kv_scale,
                                         int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                                         uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                                         float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                                         const int32_t* kv_indptr_host, void* stream);

/*
 * mla_kv_write_decode_partial_hostplan for an fp8 query: the new tokens'
 * arguments as there, then those of mla_decode_partial_fp8q_hostplan (with
 * kv_cache written); the partials are those of
 * mla_decode_partial_fp8q_hostplan after mla_kv_write, bit for bit.
 */
int mla_kv_write_decode_partial_fp8q_hostplan(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                                              int64_t k_pe_stride, const int64_t* slot_mapping,
                                              int32_t new_per_request, const uint8_t* q8, int64_t q_stride_row,
                                              int64_t q_stride_head, float q_scale, int32_t batch, int32_t qlen,
                                              int32_t heads, uint8_t* kv_cache, int64_t num_slots,
                                              const int32_t* kv_indptr, const int32_t* kv_indices,
                                              float sm_scale, float kv_scale, int32_t num_splits,
                                              int32_t num_workers, int32_t split_min_tokens, uint16_t* o_part,
                                              int64_t os_split, int64_t os_row, int64_t os_head,
                                              float* lse_part, int64_t ls_split, int64_t ls_row,
                                              int64_t ls_head, const int32_t* kv_indptr_host, void* stream);

/*
 * The attention and its LSE merge in one launch ([MLA] `m1c_inputs`: the
 * mono kernel runs the partials, then merges the splits): the merged latent
 * and LSE of mla_decode_partial_hostplan followed by mla_merge_lse, bit for
 * bit, without the partials as outputs.
 *   o    [S][...][512] bf16, strides (o_row, o_head): row t, head h gets
 *        bf16(sum_k e^(LSE_k - LSE) o_k) over the splits k of its request
 *        (0 where every split is empty, the canonical NaN 0x7FC0 where a
 *        split is NaN)
 *   lse  [S][...] f32, strides (l_row, l_head), or NULL: the merged LSE
 *        (natural log; -inf for a row that sees no token)
 *   workspace  device memory of at least mla_decode_attend_workspace_bytes
 *        bytes, 256-byte aligned: a counter per (request, 48-row block),
 *        then the partials of the requests that take more than one split.
 *        Its first part (the counters, 4*batch*row_blocks bytes rounded up
 *        to 256) must be zero before the first call on it; every call that
 *        completes with a consistent kv_indptr_host leaves it zero again.
 *        Calls that overlap on one workspace race.
 * The other arguments, the split partition and the query layout are those
 * of mla_decode_partial_hostplan (bf16 query).  A request whose tokens fall
 * in one split is written straight to o; for a split request, the last of
 * its pieces to finish (counted with a system-scope atomic, the partial rows
 * written and read with system-coherent accesses) merges its splits in the
 * LSE merge's order.
 * Errors: those of mla_decode_partial_hostplan; MLA_ERR_INVALID for a null
 * o, workspace or kv_indptr_host (batch > 0) or workspace_bytes below the
 * size it needs; MLA_ERR_UNSUPPORTED for more than 256 workers, a unit of
 * more than 65535 requests, o not 16-byte aligned with strides that are
 * multiples of 8, a workspace not 256-byte aligned, or a workspace of 2 GiB
 * or more.
 */
int mla_decode_attend(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head, int32_t batch,
                      int32_t qlen, int32_t heads, const uint8_t* kv_cache, int64_t num_slots,
                      const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float kv_scale,
                      int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                      const int32_t* kv_indptr_host, uint16_t* o, int64_t o_row, int64_t o_head, float* lse,
                      int64_t l_row, int64_t l_head, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The workspace mla_decode_attend needs for these sizes (bytes), or
 * -MLA_ERR_INVALID for batch < 0, qlen < 1, heads < 1 or num_workers < 1.
 * Host only; it depends on the sizes alone (not on the request lengths).
 */
int64_t mla_decode_attend_workspace_bytes(int32_t batch, int32_t qlen, int32_t heads, int32_t num_workers);

/*
 * mla_decode_attend for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, outputs and errors, without the workspace
 * arguments.  The workspace is an array of MLA_ATTEND_NOALLOC_MAX_BYTES in
 * the library's own device memory, one per GPU, held until the process ends;
 * the first call on a device takes its address there.  The call allocates
 * nothing and never synchronizes.  Sizes whose workspace
 * (mla_decode_attend_workspace_bytes) exceeds MLA_ATTEND_NOALLOC_MAX_BYTES
 * give MLA_ERR_UNSUPPORTED; a failed device query gives MLA_ERR_HIP.  The
 * array starts zeroed and every completed call leaves its counters zero
 * again; all calls on one GPU share it, so calls that overlap on one GPU
 * (different streams, concurrent host threads) race.
 */
#define MLA_ATTEND_NOALLOC_MAX_BYTES (32 << 20)
int mla_decode_attend_noalloc(const uint16_t* q, int64_t q_stride_row, int64_t q_stride_head, int32_t batch,
                              int32_t qlen, int32_t heads, const uint8_t* kv_cache, int64_t num_slots,
                              const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale, float kv_scale,
                              int32_t num_splits, int32_t num_workers, int32_t split_min_tokens,
                              const int32_t* kv_indptr_host, uint16_t* o, int64_t o_row, int64_t o_head,
                              float* lse, int64_t l_row, int64_t l_head, void* stream);

/*
 * Host helper: the split partition mla_decode_partial uses.
 *   kv_indptr_host [batch+1] (host), split_bounds_host [batch][num_splits+1]
 *   (host, written): split k of request r covers request-local tokens
 *   [bounds[r][k], bounds[r][k+1]); unused splits are empty (= L_r).
 *   *chunk_out (host, nullable) receives chunk.
 * Pure host code: no device work, usable without a GPU.
 */
int mla_split_plan(const int32_t* kv_indptr_host, int32_t batch, int32_t num_splits,
                   int32_t num_workers, int32_t split_min_tokens, int32_t* split_bounds_host,
                   int64_t* chunk_out);

/*
 * LSE merge of the split partials ([MLA] `m1c_inputs`: the step after the
 * partials combines the splits; `post` applies the same combine across
 * ranks).  For row t, head h:
 *   m = max_k lse_k;  m = -inf  ->  o = 0, lse = -inf;  otherwise
 *   lse = m + ln sum_k exp(lse_k - m),   o = bf16( sum_k exp(lse_k - lse) * o_k )
 * Splits with lse_k = -inf are skipped and their o_k is never read.
 *   o_part   [num_splits][rows][heads][512] bf16 (strides os_split, os_row, os_head)
 *   lse_part [num_splits][rows][heads] f32 (strides ls_split, ls_row, ls_head)
 *   o        [rows][heads][512] bf16 (strides o_row, o_head)
 *   lse      [rows][heads] f32 (strides l_row, l_head), nullable
 * rows = 0 is a no-op.
 * Errors: MLA_ERR_INVALID for rows < 0, heads < 1, num_splits < 1 or a null
 * pointer (lse aside); MLA_ERR_UNSUPPORTED unless os_split, os_row, os_head,
 * o_row and o_head are multiples of 8 and o_part and o are 16-byte aligned,
 * or when rows * heads exceeds one launch grid.
 */
int mla_merge_lse(const uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                  const float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                  int32_t num_splits, int32_t rows, int32_t heads, uint16_t* o, int64_t o_row,
                  int64_t o_head, float* lse, int64_t l_row, int64_t l_head, void* stream);

/*
 * W_UV value projection + sigmoid gate ([VALUE] `MlaValue` and `MlaGate`;
 * [MLA] `post`).  For row t (request t / qlen), head h, v < 128:
 *   acc = sum_{l<512} latent[t][h][l] * W(h, v, l)          (f32 accumulation)
 *   out[t][h*128 + v] = bf16( f32(bf16(acc)) * sigmoid_f32(gate[t][h*128 + v]) )
 * when lengths[t / qlen] > 0, and +0 otherwise (even for a NaN gate).
 *   latent [rows][heads][512] bf16 (strides l_row, l_head)
 *   w_format MLA_W_BF16: w_uv = bf16 [heads][128][512] (strides w_head, w_v;
 *            the latent axis contiguous, as the absorbed kv_b_proj view)
 *   w_format MLA_W_MXFP4: w_uv = u8 E2M1 codes [heads][128][256] (strides in
 *            bytes w_head, w_v; element 2k in the low nibble of byte k),
 *            w_scale = u8 E8M0 [heads][128][16] (strides ws_head, ws_v), one
 *            scale per 32 consecutive latents: W = e2m1 * 2^(e8m0 - 127)
 *   gate   [rows][heads*128] bf16 logits (stride g_row)
 *   lengths [rows / qlen] int32
 *   out    [rows][heads*128] bf16 (stride out_row)
 * rows must be a multiple of qlen; rows = 0 is a no-op.
 * Errors: MLA_ERR_INVALID for rows < 0, qlen < 1, heads < 1, rows not a
 * multiple of qlen, a null pointer (w_scale is needed for MXFP4 only),
 * g_row or out_row < heads*128, W strides smaller than one [128][512]
 * head, or an unknown w_format; MLA_ERR_UNSUPPORTED unless l_row and l_head
 * are multiples of 8 with latent 16-byte aligned, g_row and out_row are
 * multiples of 4 with gate and out 8-byte aligned, and the W strides are
 * multiples of 8 with w_uv 16-byte aligned (bf16) or multiples of 4 with
 * w_uv 4-byte aligned (MXFP4).
 */
int mla_value_gate(const uint16_t* latent, int64_t l_row, int64_t l_head, int32_t w_format,
                   const void* w_uv, int64_t w_head, int64_t w_v, const uint8_t* w_scale,
                   int64_t ws_head, int64_t ws_v, const uint16_t* gate, int64_t g_row,
                   const int32_t* lengths, int32_t rows, int32_t qlen, int32_t heads,
                   uint16_t* out, int64_t out_row, void* stream);

/*
 * mla_merge_lse followed by mla_value_gate in one call ([MLA] `post`; [VALUE]
 * `MlaValue`, which loads its weight fragments before the latent is ready).
 * For row t, head h: the latent row is the merge of the split partials,
 * exactly the bf16 value mla_merge_lse writes, and
 *   out[t][h*128 + v] = bf16( f32(bf16(sum_l latent[t][h][l] * W(h, v, l))) * sigmoid_f32(gate[t][h*128 + v]) )
 * when lengths[t / qlen] > 0, +0 otherwise: the output of mla_value_gate on
 * that latent, bit for bit.  The latent is not written.
 *   o_part, lse_part, num_splits  as for mla_merge_lse (rows x heads)
 *   w_format, w_uv, w_scale, gate, lengths, out  as for mla_value_gate (the
 *            value heads are the attention heads)
 *   lse      [rows][heads] f32 (strides l_row, l_head), the merged LSE; nullable
 * rows must be a multiple of qlen; rows = 0 is a no-op.
 * Errors: those of mla_value_gate for the weights, gate, lengths and out;
 * also MLA_ERR_INVALID for num_splits < 1 or a null o_part or lse_part, and
 * MLA_ERR_UNSUPPORTED unless os_split, os_row and os_head are multiples of
 * 8 and o_part is 16-byte aligned, or when the grid exceeds one launch.
 */
int mla_merge_value_gate(const uint16_t* o_part, int64_t os_split, int64_t os_row, int64_t os_head,
                         const float* lse_part, int64_t ls_split, int64_t ls_row, int64_t ls_head,
                         int32_t num_splits, int32_t w_format, const void* w_uv, int64_t w_head, int64_t w_v,
                         const uint8_t* w_scale, int64_t ws_head, int64_t ws_v, const uint16_t* gate,
                         int64_t g_row, const int32_t* lengths, int32_t rows, int32_t qlen, int32_t heads,
                         uint16_t* out, int64_t out_row, float* lse, int64_t l_row, int64_t l_head, void* stream);

/*
 * Measurement aid, for a harness that times the partial kernel itself.  The
 * next launch of the partial kernel by this process (by any of
 * mla_decode_partial, mla_decode_partial_hostplan, mla_decode_partial_fp8q,
 * mla_decode_partial_fp8q_hostplan, mla_decode_attend,
 * mla_decode_attend_noalloc) records start_event when the kernel starts and
 * stop_event when it ends (hipExtLaunchKernelGGL), so that
 * hipEventElapsedTime of the two is the kernel's own duration and not that
 * of the queue around it.  The events are the caller's: hipEvent_t handles
 * created with timing (the default flags), on the device of that launch,
 * alive until it has run.  Either may be NULL; NULL, NULL clears a pending
 * pair.  The library holds the two handles until that one launch takes them
 * (the only pointers it keeps across calls).  One pending pair per process:
 * calls from concurrent host threads race for it.  Returns MLA_OK.
 */
int mla_time_next_partial(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MLA_FP8_H */
