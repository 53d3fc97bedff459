/*
 * CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library and includes nothing from it.
 *
 * It evaluates the plain definitions, slowly and in wide arithmetic:
 *
 *  - Lightning indexer ("DeepSeek V3.2 and the lightning indexer", section
 *    "How the lightning indexer works"; DeepSeek-V3.2 spec sheet, design
 *    overview / section 2.1): a few indexer heads score the query against each
 *    preceding token as a weighted sum of ReLU-activated dot products, in FP8:
 *        I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]),  s <= pos(t).
 *    Every FP8 e4m3 value is an integer multiple of 2^-9 with at most 4
 *    significant bits, so each dot product over d_I <= 2^10 terms is exact in
 *    double precision.  The weighted head sum is accumulated in double and
 *    rounded once to fp32; it is exact whenever the terms w * ReLU(.) need at
 *    most 53 bits, which always holds on the 0.25-step input grids.  The
 *    accumulator starts at +0, so the result is never -0.
 *  - Top-k (same sections): each query keeps its k best-scoring preceding
 *    tokens.  Ties go to the lower token index, the kept indices are written
 *    in ascending order, and unused slots hold -1 (readings of points the
 *    pages leave open).
 *  - Sparse attention in the MQA mode of MLA (lightning-indexer post, same
 *    section: one latent per token, shared by all query heads, selection made
 *    once per query position): softmax attention of every query head over the
 *    selected latents only, in double precision; the value is the first
 *    d_latent columns of each latent row and the scores use all
 *    d_latent + d_rope columns.
 *  - Masked mode for short prefill (DeepSeek-V3.2 spec sheet, design overview
 *    and "Inference efficiency" table: a masked MHA mode simulates DSA for
 *    short-sequence prefill; the pages do not specify it).  Reading: the same
 *    heads attend densely to every token s <= pos(t) and the scores of the
 *    tokens outside the selection are set to -inf before the softmax.  It is
 *    written here as that dense masked softmax, separately from the sparse
 *    function above, so that the two formulations can be checked against
 *    each other.
 *  - Backward of the sparse attention over fixed indices (the sparse training
 *    stage trains every parameter with the selection on: DeepSeek-V3.2 spec
 *    sheet, design overview; lightning-indexer post, section on training).
 *    With o = sum_i p_i v_i and p = softmax(z), z_i = scale * q . kv_i, for an
 *    upstream gradient dout of o: D = dout . o, dp_i = dout . v_i,
 *    dz_i = p_i (dp_i - D); then dq = scale * sum_i dz_i kv_i and each listed
 *    row gets dkv[s_i] += scale * dz_i q, plus p_i dout on its value columns.
 *    Each index entry is one term, as in the forward.  The gradient does not
 *    flow into the selection (the indices are fixed).
 *  - Dense warm-up objective (DeepSeek-V3.2 spec sheet, design overview and
 *    the curriculum row of its training table; "DeepSeek V3.2 and the
 *    lightning indexer", training section): only the indexer is trained, so
 *    that its softmax over the scores of a query matches the main attention's
 *    distribution summed over the heads, under a KL loss.  Readings: the main
 *    attention here is dense over s <= pos(t) (the warm-up keeps it dense);
 *    the summed distribution is divided by the head count so that it is a
 *    distribution, p[t,s] = (1/H) sum_h softmax_s(z[t,h,s]); the loss of a
 *    row is KL(p_t || softmax(I_t)) with the target first, and its gradient
 *    with respect to the scores is softmax(I_t) - p_t.  Back through the
 *    indexer, with u = q_I[t,j] . k_I[s] and the ReLU's derivative taken as 0
 *    at u = 0: dw[t,j] = sum_s dI[t,s] ReLU(u), dq_I[t,j] = w[t,j] sum_s
 *    dI[t,s] [u > 0] k_I[s], dk_I[s] = sum_(t,j) dI[t,s] w[t,j] [u > 0] q_I[t,j].
 *
 * Query rows are given explicitly (batch index, absolute position and the
 * row's own query data), so any subset of a workload's rows can be evaluated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * Number formats
 * ------------------------------------------------------------------------- */

/* OCP FP8 e4m3fn: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 * exponent 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; no infinities. */
double dsa_oracle_e4m3_to_double(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  if (e == 15 && m == 7) return NAN;
  const double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return sign ? -mag : mag;
}

/* bfloat16: the top 16 bits of an IEEE binary32. */
static double bf16_to_double(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------------
 * Lightning indexer
 * ------------------------------------------------------------------------- */

/* scores[r, s] for s in [0, min(pos_r, Lk-1)]; other entries are untouched.
 *   q_idx_rows [nrows, H_I, d_I] e4m3fn, w_rows [nrows, H_I] fp32,
 *   k_idx [B, Lk, d_I] e4m3fn, scores [nrows, Lk] fp32. */
void dsa_oracle_index_scores(int32_t kv_len, int32_t idx_heads, int32_t idx_dim, int64_t nrows,
                             const int32_t* row_batch, const int32_t* row_pos,
                             const uint8_t* q_idx_rows, const float* w_rows,
                             const uint8_t* k_idx, float* scores) {
  double table[256];
  for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_to_double((uint8_t)c);

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const uint8_t* keys = k_idx + (int64_t)row_batch[r] * kv_len * idx_dim;
    const uint8_t* qr = q_idx_rows + r * idx_heads * idx_dim;
    const float* wr = w_rows + r * idx_heads;
    const int64_t last = row_pos[r] < kv_len - 1 ? row_pos[r] : kv_len - 1;
    for (int64_t s = 0; s <= last; ++s) {
      const uint8_t* ks = keys + s * idx_dim;
      double score = 0.0;
      for (int j = 0; j < idx_heads; ++j) {
        const uint8_t* qj = qr + (int64_t)j * idx_dim;
        double dot = 0.0;
        for (int d = 0; d < idx_dim; ++d) dot += table[qj[d]] * table[ks[d]];
        const double relu = dot > 0.0 ? dot : 0.0;
        score += (double)wr[j] * relu;
      }
      scores[r * kv_len + s] = (float)score;
    }
  }
}

/* ---------------------------------------------------------------------------
 * Top-k
 * ------------------------------------------------------------------------- */

typedef struct { float score; int32_t index; } cand_t;

/* Order: higher score first; equal scores -> lower index first. */
static int by_score_then_index(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->index > y->index) - (x->index < y->index);
}

static int by_index(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* indices[r, :] = the min(k, pos_r + 1) best candidates s <= pos_r of row r,
 * ascending, padded with -1.  scores [nrows, Lk] fp32 (only s <= pos_r read). */
void dsa_oracle_topk(int32_t kv_len, int32_t topk, int64_t nrows, const int32_t* row_pos,
                     const float* scores, int32_t* indices) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t n = (row_pos[r] < kv_len - 1 ? row_pos[r] : kv_len - 1) + 1;
    int32_t* out = indices + r * topk;
    const int64_t keep = n < topk ? n : topk;
    cand_t* c = (cand_t*)malloc((size_t)n * sizeof(cand_t));
    for (int64_t s = 0; s < n; ++s) {
      c[s].score = scores[r * kv_len + s];
      c[s].index = (int32_t)s;
    }
    qsort(c, (size_t)n, sizeof(cand_t), by_score_then_index);
    for (int64_t i = 0; i < keep; ++i) out[i] = c[i].index;
    qsort(out, (size_t)keep, sizeof(int32_t), by_index);
    for (int64_t i = keep; i < topk; ++i) out[i] = -1;
    free(c);
  }
}

/* ---------------------------------------------------------------------------
 * Sparse attention, MQA mode of MLA
 * ------------------------------------------------------------------------- */

/* For each row r and head h, over the selected tokens s (entries of
 * indices[r, :] that lie in [0, Lk); -1 and out-of-range entries are skipped):
 *   z_s   = scale * sum_{d < D_v + D_r} q[r,h,d] * kv[b_r, s, d]
 *   p_s   = exp(z_s - max z) / Z,   Z = sum exp(z_s - max z)
 *   out   = sum_s p_s * kv[b_r, s, 0:D_v]
 *   lse   = max z + ln Z
 * A row with no selected token gives out = 0 and lse = -inf.
 *   q_rows [nrows, H, D_v+D_r] bf16, kv [B, Lk, D_v+D_r] bf16,
 *   indices [nrows, k] int32, out [nrows, H, D_v] fp32, lse [nrows, H] fp32 (nullable). */
void dsa_oracle_sparse_mla_attn(int32_t kv_len, int32_t heads, int32_t d_latent, int32_t d_rope,
                                int32_t topk, float softmax_scale, int64_t nrows,
                                const int32_t* row_batch, const uint16_t* q_rows,
                                const uint16_t* kv, const int32_t* indices, float* out,
                                float* lse) {
  const int32_t dqk = d_latent + d_rope;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int32_t h = 0; h < heads; ++h) {
      const uint16_t* cache = kv + (int64_t)row_batch[r] * kv_len * dqk;
      const int32_t* sel = indices + r * topk;
      double* z = (double*)malloc((size_t)topk * sizeof(double));
      double* acc = (double*)calloc((size_t)d_latent, sizeof(double));
      double* qh = (double*)malloc((size_t)dqk * sizeof(double));
      for (int d = 0; d < dqk; ++d) qh[d] = bf16_to_double(q_rows[(r * heads + h) * dqk + d]);
      double zmax = -INFINITY;
      for (int i = 0; i < topk; ++i) {
        const int32_t s = sel[i];
        if (s < 0 || s >= kv_len) { z[i] = -INFINITY; continue; }
        const uint16_t* row = cache + (int64_t)s * dqk;
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += qh[d] * bf16_to_double(row[d]);
        z[i] = (double)softmax_scale * dot;
        if (z[i] > zmax) zmax = z[i];
      }
      double Z = 0.0;
      for (int i = 0; i < topk; ++i) {
        const int32_t s = sel[i];
        if (s < 0 || s >= kv_len) continue;
        const double p = exp(z[i] - zmax);
        Z += p;
        const uint16_t* row = cache + (int64_t)s * dqk;
        for (int d = 0; d < d_latent; ++d) acc[d] += p * bf16_to_double(row[d]);
      }
      float* o = out + (r * heads + h) * d_latent;
      for (int d = 0; d < d_latent; ++d) o[d] = Z > 0.0 ? (float)(acc[d] / Z) : 0.0f;
      if (lse) lse[r * heads + h] = Z > 0.0 ? (float)(zmax + log(Z)) : -INFINITY;
      free(qh);
      free(z);
      free(acc);
    }
  }
}

/* Dense causal attention of each (row, head) over s = 0 .. min(pos, kv_len - 1)
 * with the scores of the tokens not listed in the row's indices set to -inf
 * (entries outside that range are ignored; a listed token counts once). */
void dsa_oracle_masked_mha_attn(int32_t kv_len, int32_t heads, int32_t d_latent, int32_t d_rope,
                                int32_t topk, float softmax_scale, int64_t nrows,
                                const int32_t* row_batch, const int32_t* row_pos,
                                const uint16_t* q_rows, const uint16_t* kv, const int32_t* indices,
                                float* out, float* lse) {
  const int32_t dqk = d_latent + d_rope;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int32_t h = 0; h < heads; ++h) {
      const uint16_t* cache = kv + (int64_t)row_batch[r] * kv_len * dqk;
      const int32_t n = row_pos[r] + 1 < kv_len ? row_pos[r] + 1 : kv_len;
      unsigned char* keep = (unsigned char*)calloc((size_t)n, 1);
      double* z = (double*)malloc((size_t)n * sizeof(double));
      double* acc = (double*)calloc((size_t)d_latent, sizeof(double));
      double* qh = (double*)malloc((size_t)dqk * sizeof(double));
      for (int i = 0; i < topk; ++i) {
        const int32_t s = indices[r * topk + i];
        if (s >= 0 && s < n) keep[s] = 1;
      }
      for (int d = 0; d < dqk; ++d) qh[d] = bf16_to_double(q_rows[(r * heads + h) * dqk + d]);
      /* the dense scores, then the mask */
      double zmax = -INFINITY;
      for (int32_t s = 0; s < n; ++s) {
        const uint16_t* row = cache + (int64_t)s * dqk;
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += qh[d] * bf16_to_double(row[d]);
        z[s] = keep[s] ? (double)softmax_scale * dot : -INFINITY;
        if (z[s] > zmax) zmax = z[s];
      }
      double Z = 0.0;
      if (zmax > -INFINITY)
        for (int32_t s = 0; s < n; ++s) {
          const double p = exp(z[s] - zmax);
          Z += p;
          const uint16_t* row = cache + (int64_t)s * dqk;
          for (int d = 0; d < d_latent; ++d) acc[d] += p * bf16_to_double(row[d]);
        }
      float* o = out + (r * heads + h) * d_latent;
      for (int d = 0; d < d_latent; ++d) o[d] = Z > 0.0 ? (float)(acc[d] / Z) : 0.0f;
      if (lse) lse[r * heads + h] = Z > 0.0 ? (float)(zmax + log(Z)) : -INFINITY;
      free(keep);
      free(qh);
      free(z);
      free(acc);
    }
  }
}

/* Gradients of dsa_oracle_sparse_mla_attn for the given rows and upstream
 * gradient dout [nrows, heads, d_latent]: dq [nrows, heads, dqk] (written) and
 * dkv [batch, kv_len, dqk] (accumulated into; the caller zeroes it), in double
 * precision.  Entries outside [0, kv_len) are skipped, as in the forward. */
void dsa_oracle_sparse_mla_attn_bwd(int32_t kv_len, int32_t heads, int32_t d_latent, int32_t d_rope,
                                    int32_t topk, float softmax_scale, int64_t nrows,
                                    const int32_t* row_batch, const uint16_t* q_rows,
                                    const uint16_t* kv, const int32_t* indices, const double* dout,
                                    double* dq, double* dkv) {
  const int32_t dqk = d_latent + d_rope;
  const double scale = (double)softmax_scale;
  double* pz = (double*)malloc((size_t)nrows * heads * topk * 2 * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int32_t h = 0; h < heads; ++h) {
      const uint16_t* cache = kv + (int64_t)row_batch[r] * kv_len * dqk;
      const int32_t* sel = indices + r * topk;
      const double* g = dout + (r * heads + h) * d_latent;
      double* p = pz + ((r * heads + h) * topk) * 2;  /* p_i, dz_i interleaved */
      double* qh = (double*)malloc((size_t)dqk * sizeof(double));
      double* o = (double*)calloc((size_t)d_latent, sizeof(double));
      for (int d = 0; d < dqk; ++d) qh[d] = bf16_to_double(q_rows[(r * heads + h) * dqk + d]);
      /* forward: softmax over the listed entries */
      double zmax = -INFINITY;
      for (int i = 0; i < topk; ++i) {
        const int32_t s = sel[i];
        p[2 * i] = -INFINITY;
        if (s < 0 || s >= kv_len) continue;
        const uint16_t* row = cache + (int64_t)s * dqk;
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += qh[d] * bf16_to_double(row[d]);
        p[2 * i] = scale * dot;
        if (p[2 * i] > zmax) zmax = p[2 * i];
      }
      double Z = 0.0;
      for (int i = 0; i < topk; ++i)
        if (p[2 * i] > -INFINITY) Z += exp(p[2 * i] - zmax);
      for (int i = 0; i < topk; ++i) {
        p[2 * i] = p[2 * i] > -INFINITY ? exp(p[2 * i] - zmax) / Z : 0.0;
        p[2 * i + 1] = 0.0;
        if (p[2 * i] == 0.0) continue;
        const uint16_t* row = cache + (int64_t)sel[i] * dqk;
        for (int d = 0; d < d_latent; ++d) o[d] += p[2 * i] * bf16_to_double(row[d]);
      }
      /* backward */
      double D = 0.0;
      for (int d = 0; d < d_latent; ++d) D += g[d] * o[d];
      double* dqh = dq + (r * heads + h) * dqk;
      for (int d = 0; d < dqk; ++d) dqh[d] = 0.0;
      for (int i = 0; i < topk; ++i) {
        const int32_t s = sel[i];
        if (s < 0 || s >= kv_len) continue;
        const uint16_t* row = cache + (int64_t)s * dqk;
        double dp = 0.0;
        for (int d = 0; d < d_latent; ++d) dp += g[d] * bf16_to_double(row[d]);
        const double dz = p[2 * i] * (dp - D);
        p[2 * i + 1] = dz;
        for (int d = 0; d < dqk; ++d) dqh[d] += scale * dz * bf16_to_double(row[d]);
      }
      free(qh);
      free(o);
    }
  }
  /* dkv: rows may list the same token, so the scatter runs in order */
  for (int64_t r = 0; r < nrows; ++r)
    for (int32_t h = 0; h < heads; ++h) {
      const int32_t* sel = indices + r * topk;
      const double* g = dout + (r * heads + h) * d_latent;
      const double* p = pz + ((r * heads + h) * topk) * 2;
      for (int i = 0; i < topk; ++i) {
        const int32_t s = sel[i];
        if (s < 0 || s >= kv_len) continue;
        double* dst = dkv + ((int64_t)row_batch[r] * kv_len + s) * dqk;
        for (int d = 0; d < dqk; ++d) {
          const double qd = bf16_to_double(q_rows[(r * heads + h) * dqk + d]);
          dst[d] += scale * p[2 * i + 1] * qd + (d < d_latent ? p[2 * i] * g[d] : 0.0);
        }
      }
    }
  free(pz);
}

/* ---------------------------------------------------------------------------
 * Dense warm-up objective
 * ------------------------------------------------------------------------- */

/* target[r, s] = (1/heads) sum_h softmax over s' <= pos_r of
 * softmax_scale * q_rows[r,h,:] . kv[b_r, s', :], for s in [0, min(pos_r, Lk-1)];
 * other entries are untouched.  Double precision throughout. */
void dsa_oracle_warmup_target(int32_t kv_len, int32_t heads, int32_t dqk, float softmax_scale,
                              int64_t nrows, const int32_t* row_batch, const int32_t* row_pos,
                              const uint16_t* q_rows, const uint16_t* kv, double* target) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const uint16_t* cache = kv + (int64_t)row_batch[r] * kv_len * dqk;
    const int32_t n = row_pos[r] + 1 < kv_len ? row_pos[r] + 1 : kv_len;
    double* z = (double*)malloc((size_t)n * sizeof(double));
    double* qh = (double*)malloc((size_t)dqk * sizeof(double));
    double* t = target + r * kv_len;
    for (int32_t s = 0; s < n; ++s) t[s] = 0.0;
    for (int32_t h = 0; h < heads; ++h) {
      for (int d = 0; d < dqk; ++d) qh[d] = bf16_to_double(q_rows[(r * heads + h) * dqk + d]);
      double zmax = -INFINITY;
      for (int32_t s = 0; s < n; ++s) {
        const uint16_t* row = cache + (int64_t)s * dqk;
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += qh[d] * bf16_to_double(row[d]);
        z[s] = (double)softmax_scale * dot;
        if (z[s] > zmax) zmax = z[s];
      }
      double Z = 0.0;
      for (int32_t s = 0; s < n; ++s) Z += exp(z[s] - zmax);
      for (int32_t s = 0; s < n; ++s) t[s] += exp(z[s] - zmax) / Z / heads;
    }
    free(z);
    free(qh);
  }
}

/* Per row r over s in [0, min(pos_r, Lk-1)]: with the indexer distribution
 * pi = softmax(scores[r, .]), loss[r] = sum_s target (log target - log pi)
 * (terms with target = 0 are 0) and dscores[r, s] = pi_s - target_s, the
 * gradient of the summed loss.  Other dscores entries are untouched. */
void dsa_oracle_warmup_kl(int32_t kv_len, int64_t nrows, const int32_t* row_pos, const float* scores,
                          const float* target, double* loss, double* dscores) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t n = row_pos[r] + 1 < kv_len ? row_pos[r] + 1 : kv_len;
    const float* I = scores + r * kv_len;
    const float* p = target + r * kv_len;
    double m = -INFINITY;
    for (int32_t s = 0; s < n; ++s) m = (double)I[s] > m ? (double)I[s] : m;
    double Z = 0.0;
    for (int32_t s = 0; s < n; ++s) Z += exp((double)I[s] - m);
    const double logZ = m + log(Z);
    double l = 0.0;
    for (int32_t s = 0; s < n; ++s) {
      const double log_pi = (double)I[s] - logZ;
      const double ps = (double)p[s];
      if (ps > 0.0) l += ps * (log(ps) - log_pi);
      dscores[r * kv_len + s] = exp(log_pi) - ps;
    }
    loss[r] = l;
  }
}

/* Gradients of the indexer scores with respect to its inputs, for the given
 * rows and a gradient dscores [nrows, kv_len] of the scores (entries past
 * pos_r are not read): dq_idx [nrows, H_I, d_I] and dw [nrows, H_I] written,
 * dk_idx [B, kv_len, d_I] accumulated into.  The ReLU's derivative is 0 at 0. */
void dsa_oracle_index_scores_bwd(int32_t kv_len, int32_t idx_heads, int32_t idx_dim, int64_t nrows,
                                 const int32_t* row_batch, const int32_t* row_pos,
                                 const uint8_t* q_idx_rows, const float* w_rows, const uint8_t* k_idx,
                                 const double* dscores, double* dq_idx, double* dw, double* dk_idx) {
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = dsa_oracle_e4m3_to_double((uint8_t)c);
  /* per row in parallel; the key gradient is summed serially afterwards */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const uint8_t* keys = k_idx + (int64_t)row_batch[r] * kv_len * idx_dim;
    const int32_t n = row_pos[r] + 1 < kv_len ? row_pos[r] + 1 : kv_len;
    for (int32_t j = 0; j < idx_heads; ++j) {
      const uint8_t* q = q_idx_rows + (r * idx_heads + j) * idx_dim;
      const double wj = (double)w_rows[r * idx_heads + j];
      double* dq = dq_idx + (r * idx_heads + j) * idx_dim;
      double dwj = 0.0;
      for (int d = 0; d < idx_dim; ++d) dq[d] = 0.0;
      for (int32_t s = 0; s < n; ++s) {
        const uint8_t* k = keys + (int64_t)s * idx_dim;
        double u = 0.0;
        for (int d = 0; d < idx_dim; ++d) u += lut[q[d]] * lut[k[d]];
        if (u > 0.0) {
          const double g = dscores[r * kv_len + s];
          dwj += g * u;
          for (int d = 0; d < idx_dim; ++d) dq[d] += g * wj * lut[k[d]];
        }
      }
      dw[r * idx_heads + j] = dwj;
    }
  }
  for (int64_t r = 0; r < nrows; ++r) {
    const uint8_t* keys = k_idx + (int64_t)row_batch[r] * kv_len * idx_dim;
    double* dk_seq = dk_idx + (int64_t)row_batch[r] * kv_len * idx_dim;
    const int32_t n = row_pos[r] + 1 < kv_len ? row_pos[r] + 1 : kv_len;
#pragma omp parallel for schedule(static)
    for (int32_t s = 0; s < n; ++s) {
      const uint8_t* k = keys + (int64_t)s * idx_dim;
      const double g = dscores[r * kv_len + s];
      for (int32_t j = 0; j < idx_heads; ++j) {
        const uint8_t* q = q_idx_rows + (r * idx_heads + j) * idx_dim;
        double u = 0.0;
        for (int d = 0; d < idx_dim; ++d) u += lut[q[d]] * lut[k[d]];
        if (u > 0.0) {
          const double c = g * (double)w_rows[r * idx_heads + j];
          for (int d = 0; d < idx_dim; ++d) dk_seq[(int64_t)s * idx_dim + d] += c * lut[q[d]];
        }
      }
    }
  }
}

int dsa_oracle_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
