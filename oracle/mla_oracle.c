/*
 * CPU oracle for MLA decode over an fp8 latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the GPU library: every conversion and
 * every reduction below is written out from its definition, accumulates in
 * IEEE double, and runs in plain loops with no blocking or fusion.
 *
 * Sources (the pages are vLLM API documentation of the Kimi decode runtime):
 *   [MLA]   "vllm.models.kimi_k3.amd.specialized_decode.runtime.mla"
 *           sections `attend`, `m1c_inputs`, `post`, `pre`.
 *   [VALUE] "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.mla.value"
 *           classes `MlaValue`, `MlaGate`.
 * Where the pages leave a step open, the reading taken is named at the
 * function that takes it.
 *
 * Parity status of each function: every function here is pinned by the
 * CPU tests (closed forms, library routines, brute force, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D_LATENT 512 /* kv_lora width: the value part of a cache row */
#define ORC_D_ROPE 64
#define ORC_D_QK 576 /* one cache row: 512 latent then 64 rope ([MLA] `pre`) */
#define ORC_D_V 128  /* per-head output width of W_UV ([VALUE] `MlaValue`) */

/* ---------------------------------------------------------------- codecs */

/* fp8 E4M3 in the OCP "fn" flavour (no infinities): sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent field 0 is subnormal; 0x7F / 0xFF
 * are NaN.  Reading taken: the cache dtype of [MLA] `attend` is this
 * format (the one the target GPU converts natively). */
double orc_fp8_decode(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 7;
  double mag;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -6 - 3); /* m/8 * 2^-6 */
  else
    mag = ldexp(8.0 + m, e - 7 - 3); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* Round a double to the nearest value with `p` significant bits whose
 * exponent is at least `emin` (so subnormals keep a fixed quantum), ties to
 * even.  No range limit is applied here. */
static double round_to_precision(double x, int p, int emin) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e); /* |x| = f * 2^e with f in [0.5, 1): leading bit is 2^(e-1) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  double quantum = ldexp(1.0, lead - (p - 1));
  /* x / quantum is exact (power-of-two scaling); nearbyint rounds ties to
   * even in the default rounding mode. */
  return nearbyint(x / quantum) * quantum;
}

/* Encoder E of the cache write: round to nearest even among fp8 E4M3
 * values, saturating to +-448, NaN -> 0x7F.  Reading taken: [MLA] `pre`
 * stores the scaled row in fp8 without saying how it rounds; nearest-even
 * with saturation is the plain choice. */
uint8_t orc_fp8_encode(double x) {
  if (isnan(x)) return 0x7F;
  int neg = signbit(x) ? 1 : 0;
  double a = fabs(x);
  double r = round_to_precision(a, 4, -6);
  if (r > 448.0) r = 448.0;
  int code;
  if (r < ldexp(1.0, -6)) {
    code = (int)(r / ldexp(1.0, -9)); /* subnormal: r = m * 2^-9, m in 0..7 */
  } else {
    int e;
    double f = frexp(r, &e); /* r = f * 2^e, f in [0.5, 1) */
    int mant = (int)((2.0 * f - 1.0) * 8.0); /* r = (1 + mant/8) * 2^(e-1) */
    if (mant == 8) { mant = 0; e += 1; } /* not reached: r has 4 significant bits */
    code = ((e - 1 + 7) << 3) | mant;
  }
  return (uint8_t)(code | (neg << 7));
}

/* bf16: the upper half of an IEEE binary32. */
double orc_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to bf16 (8 significant bits, emin -126, overflow -> inf),
 * ties to even; NaN -> 0x7FC0. */
uint16_t orc_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  double r = round_to_precision(x, 8, -126);
  /* largest finite bf16 is (2 - 2^-7) * 2^127; beyond it rounds to inf */
  double maxf = ldexp(255.0, 127 - 7);
  float f;
  if (fabs(r) > maxf)
    f = signbit(x) ? -INFINITY : INFINITY;
  else
    f = (float)r; /* exact: r has 8 significant bits and a binary32 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* fp4 E2M1 (OCP MX): sign, 2 exponent bits with bias 1, 1 mantissa bit. */
double orc_e2m1_decode(uint8_t nib) {
  int sign = (nib >> 3) & 1;
  int e = (nib >> 1) & 3;
  int m = nib & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* E8M0 shared scale (OCP MX): 2^(b - 127); 0xFF is NaN. */
double orc_e8m0_decode(uint8_t b) {
  if (b == 0xFF) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------- kv write */

/* The cache write of [MLA] `pre` (do_kv_cache_update of kv_c and k_pe): new
 * token i's row is [kv_c (512) | k_pe (64)], each value divided by kv_scale
 * in binary32 and encoded with E, stored at row slot_mapping[i].  A negative
 * slot skips the token.  Reading taken: the division is a correctly rounded
 * binary32 division of each value by the scale. */
void orc_kv_write(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                  int64_t k_pe_stride, const int64_t* slot_mapping, int32_t n,
                  uint8_t* kv_cache, float kv_scale) {
  for (int32_t i = 0; i < n; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    for (int c = 0; c < ORC_D_QK; ++c) {
      uint16_t h = c < ORC_D_LATENT ? kv_c[i * kv_c_stride + c]
                                    : k_pe[i * k_pe_stride + (c - ORC_D_LATENT)];
      float x = (float)orc_bf16_decode(h);
      float scaled = x / kv_scale; /* binary32 division */
      kv_cache[slot * ORC_D_QK + c] = orc_fp8_encode((double)scaled);
    }
  }
}

/* ------------------------------------------------- query concat + quant */

/* The fp8 query of [MLA] `pre` (_decode_concat_quant_fp8_op(ql_nope, q_pe,
 * q_scale)): the absorbed query row of (t, h) is [ql_nope (512) | q_pe (64)],
 * each value divided by q_scale in binary32 and encoded with E.  Readings
 * taken: the op's inputs are the bf16 ql_nope and q_pe (the pages show the
 * call, not the op), and its division and rounding are those of the cache
 * write above.  ql_nope [rows][heads][512], q_pe [rows][heads][64] (bf16
 * bits), q8 [rows][heads][576], all contiguous. */
void orc_concat_quant_fp8(const uint16_t* ql_nope, const uint16_t* q_pe, float q_scale, int32_t rows,
                          int32_t heads, uint8_t* q8) {
  for (int64_t th = 0; th < (int64_t)rows * heads; ++th) {
    for (int c = 0; c < ORC_D_QK; ++c) {
      uint16_t h = c < ORC_D_LATENT ? ql_nope[th * ORC_D_LATENT + c]
                                    : q_pe[th * ORC_D_ROPE + (c - ORC_D_LATENT)];
      float x = (float)orc_bf16_decode(h);
      float scaled = x / q_scale; /* binary32 division */
      q8[th * ORC_D_QK + c] = orc_fp8_encode((double)scaled);
    }
  }
}

/* ---------------------------------------- absorbed-query producer (W_UK) */

/* The E2M1 magnitudes in code order (OCP MX v1.0): codes 0..7 are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static double e2m1_magnitude(int code) { return orc_e2m1_decode((uint8_t)code); }

/* MXFP4 quantisation of one block of 32 values, dequantised (OCP MX v1.0,
 * conversion to an MX format): the shared exponent is
 *   X = floor(log2(max_i |v_i|)) - 2   (2: the largest E2M1 exponent),
 * held to the E8M0 range [-127, 127]; each element is v_i / 2^X rounded to
 * the nearest E2M1 value (ties to the even code), values beyond the largest
 * (6) taking 6.  out_i = (that value, with the sign of v_i) * 2^X.  Readings
 * taken where the spec leaves it to the implementation: a block holding a
 * NaN or an infinity dequantises to NaN; an all-zero block to zeros. */
void orc_mxfp4_block(const double* v, double* out) {
  double amax = 0.0;
  int bad = 0;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(v[i])) bad = 1;
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  }
  if (bad) {
    for (int i = 0; i < 32; ++i) out[i] = NAN;
    return;
  }
  if (amax == 0.0) {
    for (int i = 0; i < 32; ++i) out[i] = 0.0;
    return;
  }
  int e;
  frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1 */
  int X = (e - 1) - 2;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  for (int i = 0; i < 32; ++i) {
    double a = ldexp(fabs(v[i]), -X); /* exact: a power-of-two scaling */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
      double dc = fabs(a - e2m1_magnitude(c)), db = fabs(a - e2m1_magnitude(best));
      if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    double q = ldexp(e2m1_magnitude(best), X);
    out[i] = signbit(v[i]) ? -q : q;
  }
}

/* The absorbed query of [MLA] `pre`: ql_nope = batched_gemm_a16wfp4(
 * q_nope^T, W_K, W_K_scale, transpose_bm=True, prequant=True,
 * y_scale=q_scale or None), then the concat with q_pe (and, on the fp8
 * path, its quantisation).  Readings taken (the page shows the call, not
 * what its flags compute):
 *   - W_K of head h is a [512][128] MXFP4 matrix: row n holds 128 E2M1 codes
 *     (two per byte, element 2k in the low nibble) and one E8M0 scale per 32
 *     along k; y[t][h][n] = sum_k x[t][h][k] * W_K[h][n][k].
 *   - transpose_bm: the per-head product [H][S][512] is laid out [S][H][512].
 *   - prequant: the bf16 activation q_nope[t][h][:] is first quantised to
 *     MXFP4 in blocks of 32 along k (orc_mxfp4_block), so both operands are
 *     MXFP4; the product is computed exactly here.
 *   - y_scale given (out_fp8 = 1): the product leaves as fp8 E4M3 codes
 *     E(f32(y) / q_scale) (binary32 division, the encoder E of the cache
 *     write) and the concat encodes q_pe the same way; absent (out_fp8 = 0),
 *     y is rounded to bf16 and q_pe is copied.
 * q_nope [rows][heads][128] and q_pe [rows][heads][64] are bf16 bits;
 * w_k [heads][512][64] bytes, w_scale [heads][512][4]; out is
 * [rows][heads][576] (bf16 bits or fp8 codes); y_out (nullable)
 * [rows][heads][512] receives the exact products. */
void orc_absorb_query(const uint16_t* q_nope, const uint16_t* q_pe, const uint8_t* w_k, const uint8_t* w_scale,
                      int32_t rows, int32_t heads, int32_t out_fp8, float q_scale, void* out, double* y_out) {
  int64_t n_th = (int64_t)rows * heads;
#pragma omp parallel for schedule(static)
  for (int64_t th = 0; th < n_th; ++th) {
    int64_t h = th % heads;
    double x[128], xq[128];
    for (int k = 0; k < 128; ++k) x[k] = orc_bf16_decode(q_nope[th * 128 + k]);
    for (int b = 0; b < 4; ++b) orc_mxfp4_block(x + 32 * b, xq + 32 * b);
    for (int n = 0; n < ORC_D_LATENT; ++n) {
      double y = 0.0;
      for (int k = 0; k < 128; ++k) {
        uint8_t byte = w_k[(h * ORC_D_LATENT + n) * 64 + k / 2];
        uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
        double w = orc_e2m1_decode(nib) * orc_e8m0_decode(w_scale[(h * ORC_D_LATENT + n) * 4 + k / 32]);
        y += xq[k] * w;
      }
      if (y_out) y_out[th * ORC_D_LATENT + n] = y;
      if (out_fp8) {
        float scaled = (float)y / q_scale; /* binary32 division */
        ((uint8_t*)out)[th * ORC_D_QK + n] = orc_fp8_encode((double)scaled);
      } else {
        ((uint16_t*)out)[th * ORC_D_QK + n] = orc_bf16_round(y);
      }
    }
    for (int c = 0; c < ORC_D_ROPE; ++c) {
      uint16_t pe = q_pe[th * ORC_D_ROPE + c];
      if (out_fp8) {
        float scaled = (float)orc_bf16_decode(pe) / q_scale;
        ((uint8_t*)out)[th * ORC_D_QK + ORC_D_LATENT + c] = orc_fp8_encode((double)scaled);
      } else {
        ((uint16_t*)out)[th * ORC_D_QK + ORC_D_LATENT + c] = pe;
      }
    }
  }
}

/* ---------------------------------------------------------- split bounds */

static int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Split-KV partition.  [MLA] `m1c_inputs` gives only the shape of the
 * partials, o [splits, S, H, 512] and LSE [splits, S, H].  Reading taken:
 * a stream in which request r takes ORC_PIECE_TOKENS positions followed by
 * its L_r tokens (in kv_indices order) is cut every `chunk` positions, with
 *   T_v   = T + ORC_PIECE_TOKENS * batch
 *   chunk = max(split_min_tokens, ceil(T_v / num_workers),
 *               ceil(L_max / (num_splits - 1)))   (num_splits > 1)
 *   chunk = max(1, T_v)                            (num_splits == 1)
 * where T is the total number of tokens and L_max the longest request.  A
 * request's splits are its pieces between consecutive cuts, in order; the
 * third term keeps every request within num_splits pieces.  bounds[r][k] is
 * the first token (within request r) of split k; bounds[r][num_splits] =
 * L_r and unused splits are empty (bounds equal to L_r).
 * Returns chunk. */
#define ORC_PIECE_TOKENS 320

int64_t orc_split_bounds(const int32_t* indptr, int32_t batch, int32_t num_splits,
                         int32_t num_workers, int32_t split_min_tokens, int32_t* bounds) {
  int64_t T = (int64_t)indptr[batch] - indptr[0];
  int64_t Tv = T + (int64_t)ORC_PIECE_TOKENS * batch;
  int64_t lmax = 0;
  for (int32_t r = 0; r < batch; ++r) {
    int64_t L = (int64_t)indptr[r + 1] - indptr[r];
    if (L > lmax) lmax = L;
  }
  int64_t chunk = split_min_tokens > 1 ? split_min_tokens : 1;
  if (num_splits > 1) {
    int64_t a = num_workers > 0 ? ceil_div64(Tv, num_workers) : Tv;
    int64_t b = ceil_div64(lmax, num_splits - 1);
    if (a > chunk) chunk = a;
    if (b > chunk) chunk = b;
  } else {
    if (Tv > chunk) chunk = Tv;
  }
  for (int32_t r = 0; r < batch; ++r) {
    /* V: stream position of request r's first token */
    int64_t V = (int64_t)indptr[r] - indptr[0] + (int64_t)ORC_PIECE_TOKENS * (r + 1);
    int64_t L = (int64_t)indptr[r + 1] - indptr[r];
    int32_t* b = bounds + (int64_t)r * (num_splits + 1);
    int k = 0;
    b[k++] = 0;
    /* every multiple of chunk strictly inside (V, V + L) starts a split */
    for (int64_t c = (V / chunk + 1) * chunk; c < V + L; c += chunk) b[k++] = (int32_t)(c - V);
    while (k <= num_splits) b[k++] = (int32_t)L;
  }
  return chunk;
}

/* ----------------------------------------------------- attention (exact) */

/* Exact softmax attention of one query row of one head over tokens
 * [lo, hi) of request r (definition behind [MLA] `attend` / `m1c_inputs`),
 * with the query row already decoded to real values q[d]:
 *   s_i = sm_scale * kv_scale * sum_{d<576} q[d] * D(kv[row_i][d])
 *   LSE = ln sum_i exp(s_i),   o = kv_scale * sum_i exp(s_i - LSE) * D(kv[row_i][0:512])
 * An empty range gives LSE = -inf and o = 0. */
static void attend_row(const double* qd, const uint8_t* kv_cache, const int32_t* rows,
                       int64_t lo, int64_t hi, double sm_scale, double kv_scale, double* s,
                       double* lse_out, double* o_out) {
  for (int d = 0; d < ORC_D_LATENT; ++d) o_out[d] = 0.0;
  if (hi <= lo) {
    *lse_out = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t i = lo; i < hi; ++i) {
    const uint8_t* kr = kv_cache + (int64_t)rows[i] * ORC_D_QK;
    double dot = 0.0;
    for (int d = 0; d < ORC_D_QK; ++d) dot += qd[d] * orc_fp8_decode(kr[d]);
    s[i - lo] = sm_scale * kv_scale * dot;
    if (s[i - lo] > m) m = s[i - lo];
  }
  double sum = 0.0;
  for (int64_t i = lo; i < hi; ++i) sum += exp(s[i - lo] - m);
  double lse = m + log(sum);
  for (int64_t i = lo; i < hi; ++i) {
    const uint8_t* kr = kv_cache + (int64_t)rows[i] * ORC_D_QK;
    double p = exp(s[i - lo] - lse);
    for (int d = 0; d < ORC_D_LATENT; ++d) o_out[d] += p * orc_fp8_decode(kr[d]);
  }
  for (int d = 0; d < ORC_D_LATENT; ++d) o_out[d] *= kv_scale;
  *lse_out = lse;
}

/* The query of row t, head h as real values: a bf16 query is its bf16
 * value; an fp8 query (q8 of [MLA] `pre`, the query quantised with the
 * per-tensor scale q_scale, which `attend` hands to the decode as is) is
 * q_scale * D(q8), D the E4M3 decode above.  Reading taken: the quantised
 * query stands for q_scale times its decoded value, as the cache row stands
 * for kv_scale times its own. */
static void decode_query(const void* q, int q_fp8, double q_scale, int64_t off, double* qd) {
  for (int d = 0; d < ORC_D_QK; ++d)
    qd[d] = q_fp8 ? q_scale * orc_fp8_decode(((const uint8_t*)q)[off + d])
                  : orc_bf16_decode(((const uint16_t*)q)[off + d]);
}

/* Split-KV partial attention ([MLA] `m1c_inputs`: o [splits, S, H, 512]
 * and LSE [splits, S, H]).  q is [S, H, 576] contiguous with S = batch*qlen;
 * row t = r*qlen + j belongs to request r.  Reading taken for qlen > 1 (the
 * pages run qlen 4 / 8 without stating the mask): the cache already holds
 * the request's qlen new tokens, and row j sees the first
 * L_r - qlen + j + 1 tokens (causal within the window).  Split k of row t is
 * the exact attention over [bounds[r][k], bounds[r][k+1]) intersected with
 * the visible prefix; o_out / lse_out are [num_splits][S][H][512] / [..][H]
 * in double (rounding o to bf16 is a separate step). */
static void decode_partial(const void* q, int q_fp8, double q_scale, int32_t batch, int32_t qlen,
                           int32_t heads, const uint8_t* kv_cache, const int32_t* indptr,
                           const int32_t* indices, const int32_t* bounds, int32_t num_splits,
                           double sm_scale, double kv_scale, double* o_out, double* lse_out) {
  int64_t S = (int64_t)batch * qlen;
  int64_t lmax = 0;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr[r + 1] - indptr[r] > lmax) lmax = indptr[r + 1] - indptr[r];
  int64_t total = (int64_t)num_splits * S * heads;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(lmax > 0 ? lmax : 1));
    double qd[ORC_D_QK];
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < total; ++w) {
      int64_t h = w % heads;
      int64_t t = (w / heads) % S;
      int64_t k = w / (heads * S);
      int64_t r = t / qlen, j = t % qlen;
      int64_t L = (int64_t)indptr[r + 1] - indptr[r];
      int64_t visible = L - qlen + j + 1;
      if (visible < 0) visible = 0;
      const int32_t* b = bounds + r * (num_splits + 1);
      int64_t lo = b[k], hi = b[k + 1];
      if (hi > visible) hi = visible;
      const int32_t* rows = indices + indptr[r];
      decode_query(q, q_fp8, q_scale, (t * heads + h) * ORC_D_QK, qd);
      attend_row(qd, kv_cache, rows, lo, hi, sm_scale, kv_scale, s, lse_out + (k * S + t) * heads + h,
                 o_out + ((k * S + t) * heads + h) * ORC_D_LATENT);
    }
    free(s);
  }
}

/* bf16 query [S, H, 576] (the bf16 query of [MLA] `m1c_inputs`). */
void orc_decode_partial(const uint16_t* q, int32_t batch, int32_t qlen, int32_t heads,
                        const uint8_t* kv_cache, const int32_t* indptr, const int32_t* indices,
                        const int32_t* bounds, int32_t num_splits, double sm_scale,
                        double kv_scale, double* o_out, double* lse_out) {
  decode_partial(q, 0, 1.0, batch, qlen, heads, kv_cache, indptr, indices, bounds, num_splits, sm_scale,
                 kv_scale, o_out, lse_out);
}

/* fp8 E4M3 query q8 [S, H, 576] with its per-tensor scale ([MLA] `pre`
 * returns it, `attend` decodes with it). */
void orc_decode_partial_q8(const uint8_t* q8, double q_scale, int32_t batch, int32_t qlen, int32_t heads,
                           const uint8_t* kv_cache, const int32_t* indptr, const int32_t* indices,
                           const int32_t* bounds, int32_t num_splits, double sm_scale,
                           double kv_scale, double* o_out, double* lse_out) {
  decode_partial(q8, 1, q_scale, batch, qlen, heads, kv_cache, indptr, indices, bounds, num_splits,
                 sm_scale, kv_scale, o_out, lse_out);
}

/* -------------------------------------------------------------- merge */

/* LSE merge of split partials ([MLA] `m1c_inputs`: the step after the
 * partials combines the splits; `post` applies the same combine across
 * ranks).  For each (row, head):
 *   m = max_k LSE_k; if m = -inf: o = 0, LSE = -inf; otherwise
 *   LSE = m + ln sum_k exp(LSE_k - m),  o = sum_k exp(LSE_k - LSE) * o_k
 * where o_k is the stored bf16 partial.  Splits with LSE_k = -inf contribute
 * nothing and their o_k is never read (it may hold anything).
 * o_part [num_splits][rows][heads][512] bf16, lse_part [num_splits][rows][heads]. */
void orc_merge_lse(const uint16_t* o_part, const float* lse_part, int32_t num_splits, int64_t rows,
                   int32_t heads, double* o_out, double* lse_out) {
  int64_t n = rows * heads;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double m = -INFINITY;
    for (int k = 0; k < num_splits; ++k) {
      double l = lse_part[k * n + i];
      if (l > m) m = l;
    }
    double* o = o_out + i * ORC_D_LATENT;
    for (int d = 0; d < ORC_D_LATENT; ++d) o[d] = 0.0;
    if (m == -INFINITY) {
      lse_out[i] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int k = 0; k < num_splits; ++k) {
      double l = lse_part[k * n + i];
      if (l != -INFINITY) sum += exp(l - m);
    }
    double lse = m + log(sum);
    for (int k = 0; k < num_splits; ++k) {
      double l = lse_part[k * n + i];
      if (l == -INFINITY) continue;
      double wgt = exp(l - lse);
      const uint16_t* ok = o_part + (k * n + i) * ORC_D_LATENT;
      for (int d = 0; d < ORC_D_LATENT; ++d) o[d] += wgt * orc_bf16_decode(ok[d]);
    }
    lse_out[i] = lse;
  }
}

/* ------------------------------------------------------- value + gate */

/* W_UV value projection and sigmoid gate ([VALUE] `MlaValue`, `MlaGate`;
 * [MLA] `post`).  For row t (request t / qlen), head h, output v < 128:
 *   acc = sum_{l<512} latent[t][h][l] * W(h, v, l)
 *   out[t][h*128 + v] = bf16( f32(bf16(acc)) * sigmoid(f32(gate[t][h*128+v])) )
 * when lengths[t / qlen] > 0, and +0 otherwise (even for a NaN gate or a
 * NaN latent).  W is bf16 [H][128][512] (latent axis contiguous), or, when
 * w_fp4 != NULL, MXFP4: codes [H][128][256] bytes (element 2k in the low
 * nibble) with E8M0 scales [H][128][16], one per 32 consecutive latents.
 * acc_out (may be NULL) receives acc in double; out receives bf16 bits. */
void orc_value_gate(const uint16_t* latent, const uint16_t* w_bf16, const uint8_t* w_fp4,
                    const uint8_t* w_scale, const uint16_t* gate, const int32_t* lengths,
                    int32_t batch, int32_t qlen, int32_t heads, double* acc_out, uint16_t* out) {
  int64_t S = (int64_t)batch * qlen;
  int64_t n = S * heads;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = i / heads, h = i % heads;
    int64_t r = t / qlen;
    const uint16_t* lat = latent + i * ORC_D_LATENT;
    for (int v = 0; v < ORC_D_V; ++v) {
      double acc = 0.0;
      for (int l = 0; l < ORC_D_LATENT; ++l) {
        double w;
        if (w_fp4) {
          uint8_t byte = w_fp4[((h * ORC_D_V + v) * ORC_D_LATENT + l) / 2];
          uint8_t nib = (l & 1) ? (byte >> 4) : (byte & 0xF);
          w = orc_e2m1_decode(nib) * orc_e8m0_decode(w_scale[(h * ORC_D_V + v) * 16 + l / 32]);
        } else {
          w = orc_bf16_decode(w_bf16[(h * ORC_D_V + v) * ORC_D_LATENT + l]);
        }
        acc += orc_bf16_decode(lat[l]) * w;
      }
      int64_t col = h * ORC_D_V + v;
      if (acc_out) acc_out[t * heads * ORC_D_V + col] = acc;
      if (lengths[r] > 0) {
        double value = orc_bf16_decode(orc_bf16_round(acc));
        float g = (float)orc_bf16_decode(gate[t * heads * ORC_D_V + col]);
        double sig = 1.0 / (1.0 + exp(-(double)g));
        out[t * heads * ORC_D_V + col] = orc_bf16_round(value * sig);
      } else {
        out[t * heads * ORC_D_V + col] = 0; /* +0 */
      }
    }
  }
}

/* elementwise array forms of the codecs above */
void orc_bf16_round_array(const double* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(in[i]);
}
void orc_fp8_encode_array(const double* in, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(in[i]);
}

/* number of OpenMP threads the oracle runs on (for reporting) */
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
