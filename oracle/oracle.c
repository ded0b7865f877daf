/*
 * Plain fp64 CPU oracle for attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the HIP library is
 * compared against.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or helper with
 * the HIP library under mha_mla_kv_amd/ and never calls it.
 *
 * Every routine is the plain definition, written as loops, accumulated in
 * double precision.  Inputs are float32 arrays: bf16 and fp32 values are held
 * exactly in float32, so widening them to double is exact and both sides see
 * the same numbers.  OpenMP spreads independent output rows over host threads;
 * nothing inside a row is blocked, fused or reordered.
 *
 * Sources (page title, then the part of the page that fixes the step):
 *  - "模型架构｜MQA & GQA 调研" (MQA & GQA survey), section
 *    "Grouped-query attention": query heads are split into G groups and every
 *    group shares one key head and one value head; G = 1 is MQA, G = H is MHA.
 *  - same page, code section: repeat_kv expands KV head g to the n_rep
 *    consecutive query heads g*n_rep .. g*n_rep+n_rep-1 (its docstring names
 *    repeat_interleave along the head axis), so query head h reads KV head
 *    floor(h / n_rep); Attention.forward writes the new K/V at start_pos,
 *    reads the cache up to start_pos+seqlen, scores Q K^T / sqrt(head_dim),
 *    adds the additive mask, takes the softmax in fp32, multiplies by V.
 *  - qqstock DeepSeek MLA article, sections 1-4 and the MultiHeadLatentAttention
 *    listing: only the latent c (kv_lora_rank wide) and one rotated key part
 *    k_rope shared by all heads are cached; keys are [W_UK c , k_rope], values
 *    are W_UV c; the score width is nope+rope, so the default softmax scale of
 *    scaled_dot_product_attention is 1/sqrt(nope_head_dim + rope_dim).  With
 *    W_UK folded into the query and W_UV applied after the weighted sum, the
 *    same numbers come out (sections 2 and 4).
 *
 * Readings where the pages are silent:
 *  - cache_lens[b] counts the valid cached tokens including the newest one;
 *    decode attends to t in [0, L_b) with no mask.  Values are clamped to
 *    [0, T_max].  L_b = 0 gives an output row of zeros.
 *  - Causal prefill lets query i see keys j <= i (no cached prefix, so the
 *    top-left and bottom-right alignments coincide).  With a cached prefix of
 *    P positions, new token i sits at position P + i and sees keys j <= P + i
 *    (bottom-right alignment).
 *  - softmax_scale <= 0 selects the default scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int clamp_len(int32_t L, int T_max) {
  if (L < 0) return 0;
  if (L > T_max) return T_max;
  return (int)L;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Softmax-weighted sum over n scores: out[d] = sum_t p_t * rows(t)[d],
 * p_t = exp(s_t - max s) / sum exp(s_u - max s).  rows(t) = base + t*stride. */
static void softmax_weighted_sum(const double* s, int n, const float* base,
                                 long stride, int D, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) return;
  double m = s[0];
  for (int t = 1; t < n; ++t)
    if (s[t] > m) m = s[t];
  double denom = 0.0;
  for (int t = 0; t < n; ++t) denom += exp(s[t] - m);
  for (int t = 0; t < n; ++t) {
    double p = exp(s[t] - m) / denom;
    const float* row = base + (long)t * stride;
    for (int d = 0; d < D; ++d) out[d] += p * (double)row[d];
  }
}

/*
 * GQA decode: one new query token per sequence against its cached K/V.
 *   q   [B, Hq, D]            k, v [B, T_max, Hkv, D]     out [B, Hq, D]
 *   out[b,h] = softmax_t( scale * q[b,h] . k[b,t,g] ) . v[b,t,g],
 *   g = floor(h / (Hq/Hkv)), t < L_b.
 * Hkv must divide Hq (checked by the caller).
 */
void oracle_gqa_decode(const float* q, const float* k, const float* v,
                       const int32_t* cache_lens, double* out, int B, int Hq,
                       int Hkv, int D, int T_max, double scale) {
  const int n_rep = Hq / Hkv;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int g = h / n_rep;
      const int L = clamp_len(cache_lens[b], T_max);
      double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
      const float* qv = q + ((long)b * Hq + h) * D;
      for (int t = 0; t < L; ++t) {
        const float* kr = k + (((long)b * T_max + t) * Hkv + g) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += (double)qv[d] * (double)kr[d];
        s[t] = scale * dot;
      }
      const float* vbase = v + ((long)b * T_max * Hkv + g) * D;
      softmax_weighted_sum(s, L, vbase, (long)Hkv * D, D,
                           out + ((long)b * Hq + h) * D);
      free(s);
    }
  }
}

/*
 * Causal GQA prefill, no cached prefix.
 *   q, out [B, S, Hq, D]      k, v [B, S, Hkv, D]
 *   out[b,i,h] = softmax_{j<=i}( scale * q[b,i,h] . k[b,j,g] ) . v[b,j,g].
 * rows/n_rows (optional): when rows != NULL only the listed query positions
 * i = rows[r] are computed (all b, h); other output rows are left untouched.
 */
void oracle_gqa_prefill_causal(const float* q, const float* k, const float* v,
                               double* out, int B, int S, int Hq, int Hkv,
                               int D, double scale, const int32_t* rows,
                               int n_rows) {
  const int n_rep = Hq / Hkv;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const int NI = rows ? n_rows : S;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int r = 0; r < NI; ++r) {
      for (int h = 0; h < Hq; ++h) {
        const int i = rows ? rows[r] : r;
        if (i < 0 || i >= S) continue;
        const int g = h / n_rep;
        const int n = i + 1; /* keys 0..i */
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        const float* qv = q + (((long)b * S + i) * Hq + h) * D;
        for (int j = 0; j < n; ++j) {
          const float* kr = k + (((long)b * S + j) * Hkv + g) * D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += (double)qv[d] * (double)kr[d];
          s[j] = scale * dot;
        }
        const float* vbase = v + ((long)b * S * Hkv + g) * D;
        softmax_weighted_sum(s, n, vbase, (long)Hkv * D, D,
                             out + (((long)b * S + i) * Hq + h) * D);
        free(s);
      }
    }
  }
}

/*
 * Causal GQA prefill after a cached prefix (chunked prefill), per sequence.
 *   q, out [B, S, Hq, D] (the new tokens)   k, v [B, T_max, Hkv, D] (the cache,
 *   the new tokens' rows already written at positions P_b .. P_b + n_b - 1)
 *   start_pos [B] = P_b, q_lens [B] = n_b new tokens (NULL: S each)
 *   out[b,i,h] = softmax_{j <= P_b + i}( scale * q[b,i,h] . k[b,j,g] ) . v[b,j,g]
 *   for i < n_b; rows i >= n_b are zero.
 * This is Attention.forward of the MQA & GQA survey page with start_pos > 0:
 * the new K/V are written at start_pos first, the keys are the cache up to
 * start_pos + seqlen, and the additive mask spans cache_len + seqlen; its
 * plainest reading (bottom-right alignment) lets new token i, at position
 * start_pos + i, see every cached position up to its own.
 * P_b is clamped to [0, T_max] and n_b to [0, min(S, T_max - P_b)].
 */
void oracle_gqa_prefill_cached(const float* q, const float* k, const float* v,
                               const int32_t* start_pos, const int32_t* q_lens,
                               double* out, int B, int S, int Hq, int Hkv,
                               int D, int T_max, double scale) {
  const int n_rep = Hq / Hkv;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < S; ++i) {
      for (int h = 0; h < Hq; ++h) {
        const int P = clamp_len(start_pos[b], T_max);
        int nq = q_lens ? (int)q_lens[b] : S;
        if (nq > S) nq = S;
        if (nq > T_max - P) nq = T_max - P;
        double* o = out + (((long)b * S + i) * Hq + h) * D;
        if (i >= nq) {
          for (int d = 0; d < D; ++d) o[d] = 0.0;
          continue;
        }
        const int g = h / n_rep;
        const int n = P + i + 1; /* keys 0 .. P + i */
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        const float* qv = q + (((long)b * S + i) * Hq + h) * D;
        for (int j = 0; j < n; ++j) {
          const float* kr = k + (((long)b * T_max + j) * Hkv + g) * D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += (double)qv[d] * (double)kr[d];
          s[j] = scale * dot;
        }
        const float* vbase = v + ((long)b * T_max * Hkv + g) * D;
        softmax_weighted_sum(s, n, vbase, (long)Hkv * D, D, o);
        free(s);
      }
    }
  }
}

/*
 * MLA decode, decompressed form (keys and values rebuilt from the latent).
 *   q_nope [B, H, dn]   q_rope [B, H, dR]   (q_rope already rotated)
 *   w_uk [H, dn, r]     rows h*dn.. of the k-nope up-projection weight
 *   w_uv [H, dv, r]     rows h*dv.. of the value up-projection weight
 *   c_kv [B, T_max, r]  k_rope [B, T_max, dR] (already rotated, one per token)
 *   out [B, H, dv]
 *   k_nope[h,t] = w_uk[h] c_kv[b,t];  v[h,t] = w_uv[h] c_kv[b,t]
 *   s_t = scale * (q_nope . k_nope[h,t] + q_rope . k_rope[b,t])
 *   out[b,h] = sum_t softmax(s)_t v[h,t]
 * bh_list/n_bh (optional): only the listed (b, h) pairs, flattened b*H+h.
 */
void oracle_mla_decode_decompressed(const float* q_nope, const float* q_rope,
                                    const float* w_uk, const float* w_uv,
                                    const float* c_kv, const float* k_rope,
                                    const int32_t* cache_lens, double* out,
                                    int B, int H, int dn, int dR, int dv, int r,
                                    int T_max, double scale,
                                    const int32_t* bh_list, int n_bh) {
  if (scale <= 0.0) scale = 1.0 / sqrt((double)(dn + dR));
  const int N = bh_list ? n_bh : B * H;
#pragma omp parallel for schedule(dynamic)
  for (int idx = 0; idx < N; ++idx) {
    const int bh = bh_list ? bh_list[idx] : idx;
    const int b = bh / H, h = bh % H;
    if (b < 0 || b >= B) continue;
    const int L = clamp_len(cache_lens[b], T_max);
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double* vrow = (double*)malloc(sizeof(double) * (size_t)dv);
    double* acc = out + ((long)b * H + h) * dv;
    const float* qn = q_nope + ((long)b * H + h) * dn;
    const float* qr = q_rope + ((long)b * H + h) * dR;
    const float* Wk = w_uk + (long)h * dn * r;
    const float* Wv = w_uv + (long)h * dv * r;
    for (int t = 0; t < L; ++t) {
      const float* c = c_kv + ((long)b * T_max + t) * r;
      const float* kr = k_rope + ((long)b * T_max + t) * dR;
      double dot = 0.0;
      for (int i = 0; i < dn; ++i) {
        double kn = 0.0; /* k_nope[h,t][i] */
        for (int j = 0; j < r; ++j) kn += (double)Wk[(long)i * r + j] * (double)c[j];
        dot += (double)qn[i] * kn;
      }
      for (int e = 0; e < dR; ++e) dot += (double)qr[e] * (double)kr[e];
      s[t] = scale * dot;
    }
    for (int i = 0; i < dv; ++i) acc[i] = 0.0;
    if (L > 0) {
      double m = s[0];
      for (int t = 1; t < L; ++t)
        if (s[t] > m) m = s[t];
      double denom = 0.0;
      for (int t = 0; t < L; ++t) denom += exp(s[t] - m);
      for (int t = 0; t < L; ++t) {
        const double p = exp(s[t] - m) / denom;
        const float* c = c_kv + ((long)b * T_max + t) * r;
        for (int i = 0; i < dv; ++i) { /* v[h,t][i] */
          double vi = 0.0;
          for (int j = 0; j < r; ++j) vi += (double)Wv[(long)i * r + j] * (double)c[j];
          vrow[i] = vi;
        }
        for (int i = 0; i < dv; ++i) acc[i] += p * vrow[i];
      }
    }
    free(vrow);
    free(s);
  }
}

/*
 * MLA causal prefill, decompressed form: the scaled_dot_product_attention
 * (is_causal=True) call of the MultiHeadLatentAttention listing on the qqstock
 * DeepSeek MLA article, with the keys and values rebuilt from the latent cache.
 *   q_nope [B, S, H, dn]   q_rope [B, S, H, dR]   (the new tokens; q_rope rotated)
 *   w_uk [H, dn, r]   w_uv [H, dv, r]   (per-head rows of the up-projections)
 *   c_kv [B, T_max, r]   k_rope [B, T_max, dR]   (the new tokens' rows already
 *   written at start_pos[b] ..)   start_pos [B] or NULL (0)   q_lens [B] or NULL (S)
 *   out [B, S, H, dv]
 *   k_nope[h,t] = w_uk[h] c_kv[b,t];  v[h,t] = w_uv[h] c_kv[b,t]
 *   s_j = scale * (q_nope[b,i,h] . k_nope[h,j] + q_rope[b,i,h] . k_rope[b,j])
 *   out[b,i,h] = sum_{j <= P + i} softmax(s)_j v[h,j]   for i < n_b; zeros after.
 * P = start_pos[b] clamped to [0, T_max]; n_b = q_lens[b] clamped to
 * [0, min(S, T_max - P)].  The rebuilt keys and values of a (sequence, head)
 * are computed once, as the listing materialises key_nope and value.
 */
void oracle_mla_prefill_causal(const float* q_nope, const float* q_rope,
                               const float* w_uk, const float* w_uv,
                               const float* c_kv, const float* k_rope,
                               const int32_t* start_pos, const int32_t* q_lens,
                               double* out, int B, int S, int H, int dn, int dR,
                               int dv, int r, int T_max, double scale) {
  if (scale <= 0.0) scale = 1.0 / sqrt((double)(dn + dR));
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int P = start_pos ? clamp_len(start_pos[b], T_max) : 0;
      int nq = q_lens ? (int)q_lens[b] : S;
      if (nq > S) nq = S;
      if (nq > T_max - P) nq = T_max - P;
      if (nq < 0) nq = 0;
      for (int i = nq; i < S; ++i) {
        double* o = out + (((long)b * S + i) * H + h) * dv;
        for (int e = 0; e < dv; ++e) o[e] = 0.0;
      }
      if (nq == 0) continue;
      const int L = P + nq; /* cache rows any new token of this sequence sees */
      const float* Wk = w_uk + (long)h * dn * r;
      const float* Wv = w_uv + (long)h * dv * r;
      double* kn = (double*)malloc(sizeof(double) * (size_t)L * dn);
      double* vv = (double*)malloc(sizeof(double) * (size_t)L * dv);
      double* sc = (double*)malloc(sizeof(double) * (size_t)L);
      for (int t = 0; t < L; ++t) {
        const float* c = c_kv + ((long)b * T_max + t) * r;
        for (int i = 0; i < dn; ++i) {
          double a = 0.0;
          for (int j = 0; j < r; ++j) a += (double)Wk[(long)i * r + j] * (double)c[j];
          kn[(long)t * dn + i] = a;
        }
        for (int e = 0; e < dv; ++e) {
          double a = 0.0;
          for (int j = 0; j < r; ++j) a += (double)Wv[(long)e * r + j] * (double)c[j];
          vv[(long)t * dv + e] = a;
        }
      }
      for (int i = 0; i < nq; ++i) {
        const float* qn = q_nope + (((long)b * S + i) * H + h) * dn;
        const float* qr = q_rope + (((long)b * S + i) * H + h) * dR;
        const int n = P + i + 1; /* keys 0 .. P + i */
        for (int t = 0; t < n; ++t) {
          const float* kr = k_rope + ((long)b * T_max + t) * dR;
          double dot = 0.0;
          for (int d = 0; d < dn; ++d) dot += (double)qn[d] * kn[(long)t * dn + d];
          for (int e = 0; e < dR; ++e) dot += (double)qr[e] * (double)kr[e];
          sc[t] = scale * dot;
        }
        double m = sc[0];
        for (int t = 1; t < n; ++t)
          if (sc[t] > m) m = sc[t];
        double denom = 0.0;
        for (int t = 0; t < n; ++t) denom += exp(sc[t] - m);
        double* o = out + (((long)b * S + i) * H + h) * dv;
        for (int e = 0; e < dv; ++e) o[e] = 0.0;
        for (int t = 0; t < n; ++t) {
          const double p = exp(sc[t] - m) / denom;
          for (int e = 0; e < dv; ++e) o[e] += p * vv[(long)t * dv + e];
        }
      }
      free(sc);
      free(vv);
      free(kn);
    }
  }
}

/*
 * MLA decode, absorbed form: the k-nope up-projection is folded into the query
 * and the value up-projection is applied once after the weighted sum.
 *   q_abs[j] = sum_i w_uk[h][i][j] q_nope[b,h][i]           (j < r)
 *   s_t      = scale * (q_abs . c_kv[b,t] + q_rope . k_rope[b,t])
 *   o_lat    = sum_t softmax(s)_t c_kv[b,t]                  (r wide)
 *   out[i]   = sum_j w_uv[h][i][j] o_lat[j]
 * Same arguments as the decompressed form.
 */
void oracle_mla_decode_absorbed(const float* q_nope, const float* q_rope,
                                const float* w_uk, const float* w_uv,
                                const float* c_kv, const float* k_rope,
                                const int32_t* cache_lens, double* out, int B,
                                int H, int dn, int dR, int dv, int r, int T_max,
                                double scale, const int32_t* bh_list, int n_bh) {
  if (scale <= 0.0) scale = 1.0 / sqrt((double)(dn + dR));
  const int N = bh_list ? n_bh : B * H;
#pragma omp parallel for schedule(dynamic)
  for (int idx = 0; idx < N; ++idx) {
    const int bh = bh_list ? bh_list[idx] : idx;
    const int b = bh / H, h = bh % H;
    if (b < 0 || b >= B) continue;
    const int L = clamp_len(cache_lens[b], T_max);
    double* q_abs = (double*)malloc(sizeof(double) * (size_t)r);
    double* o_lat = (double*)malloc(sizeof(double) * (size_t)r);
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    const float* qn = q_nope + ((long)b * H + h) * dn;
    const float* qr = q_rope + ((long)b * H + h) * dR;
    const float* Wk = w_uk + (long)h * dn * r;
    const float* Wv = w_uv + (long)h * dv * r;
    for (int j = 0; j < r; ++j) {
      double a = 0.0;
      for (int i = 0; i < dn; ++i) a += (double)Wk[(long)i * r + j] * (double)qn[i];
      q_abs[j] = a;
    }
    for (int t = 0; t < L; ++t) {
      const float* c = c_kv + ((long)b * T_max + t) * r;
      const float* kr = k_rope + ((long)b * T_max + t) * dR;
      double dot = 0.0;
      for (int j = 0; j < r; ++j) dot += q_abs[j] * (double)c[j];
      for (int e = 0; e < dR; ++e) dot += (double)qr[e] * (double)kr[e];
      s[t] = scale * dot;
    }
    softmax_weighted_sum(s, L, c_kv + (long)b * T_max * r, (long)r, r, o_lat);
    double* o = out + ((long)b * H + h) * dv;
    for (int i = 0; i < dv; ++i) {
      double a = 0.0;
      for (int j = 0; j < r; ++j) a += (double)Wv[(long)i * r + j] * o_lat[j];
      o[i] = a;
    }
    free(s);
    free(o_lat);
    free(q_abs);
  }
}

/* Rotary position embedding of head vectors.
 *
 * The pages call it without printing it: Attention.forward on the "模型架构｜MQA &
 * GQA 调研" page (code section) applies apply_rotary_emb(xq, xk, freqs_cis) to
 * the new tokens' queries and keys before the cache write, and the
 * MultiHeadLatentAttention listing of the qqstock DeepSeek MLA article applies
 * apply_rope(query_rope, key_rope, cis=freqs_cis) to the rotated parts only
 * (section 3: decoupled RoPE).  Reading: the rotation of LLaMA-2, whose
 * Attention class the GQA page prints.  A head vector x of width d (even) is
 * taken as d/2 consecutive pairs (x[2j], x[2j+1]), each the complex number
 * x[2j] + i x[2j+1], which is multiplied by exp(i m theta_j) with
 * theta_j = base^(-2j/d) and m the token's absolute position:
 *   out[2j]   = x[2j] cos(m theta_j) - x[2j+1] sin(m theta_j)
 *   out[2j+1] = x[2j] sin(m theta_j) + x[2j+1] cos(m theta_j)
 * x [N, H, d] float32 (N tokens of H heads), pos [N] int32, out [N, H, d].
 */
void oracle_rope(const float* x, const int32_t* pos, int N, int H, int d, double base, double* out) {
#pragma omp parallel for schedule(static)
  for (long n = 0; n < N; ++n) {
    const double m = (double)pos[n];
    for (int h = 0; h < H; ++h) {
      const float* xr = x + (n * H + h) * (long)d;
      double* o = out + (n * H + h) * (long)d;
      for (int j = 0; j < d / 2; ++j) {
        const double theta = pow(base, -2.0 * (double)j / (double)d);
        const double a = m * theta;
        const double re = (double)xr[2 * j], im = (double)xr[2 * j + 1];
        o[2 * j] = re * cos(a) - im * sin(a);
        o[2 * j + 1] = re * sin(a) + im * cos(a);
      }
    }
  }
}
