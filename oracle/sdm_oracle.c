/*
 * sdm_oracle.c -- plain single-threaded fp32 CPU oracle for Sparse Delta Memory.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
 * shares no code with the HIP library and must never sit on the product path.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -shared -fPIC -lm
 * (no FMA contraction, so each expression below is the rounding sequence its
 * comment states).
 *
 * What is computed, and where it comes from (pages: gist.science summaries of
 * "Sparse Delta Memory", paper 2607.07386; Spanish page = ES, French = FR):
 *
 *  1. Addressing (ES "Mecanismo Central" item 2, FR "Mecanisme Central",
 *     "Selection de Cles Creuses"): the projected key k' and query q' are cut
 *     into two halves; the outer sum of the two half-score vectors gives one
 *     score per slot (N = n_sub^2 slots, product-key memory); top-W slots are
 *     written and top-R slots are read; the N-vector is never formed, using
 *     topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)).
 *     Readings where the pages are silent: the halves are the first and last
 *     d_k/2 elements; each half is dotted with its own table of n_sub
 *     sub-keys (product-key memory); slot = i*n_sub + j; ties go to the lower
 *     index; lists are in rank order; one sub-key table pair per head serves
 *     both queries and keys.
 *  2. Write weights (ES item 3, the per-slot factor k_t^(i) of the delta
 *     update, left undefined by the pages): softmax over the selected top-W
 *     sums, temperature 1, max subtracted.  Read weights likewise over top-R.
 *  3. Gated delta write on the W selected slots only (ES item 3, forget gate
 *     then delta update; unselected slots unchanged):
 *        m~ = alpha * M[s];  M[s] = m~ + beta*w*(v - m~)
 *     evaluated in the algebraically equal form M[s] = (1-c)*m~ + c*v with
 *     c = beta*w, so that c = 1 stores v exactly and c = 0 keeps m~ exactly.
 *  4. Sparse read (ES item 4): o_t = sum over the R read slots of r_j M[j],
 *     taken after the token's write.
 *  5. Dense gated-delta baseline: S = a S + b (v - a S k) k^T, o = S q.
 */
#include "sdm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* exact widening */
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float load_elem(const void* base, int32_t dtype, int64_t i) {
  if (dtype == SDM_REF_BF16) return bf16_to_f32(((const uint16_t*)base)[i]);
  return ((const float*)base)[i];
}

/* Strict total order used everywhere: a ranks ahead of b iff its score is
 * larger, or the scores are equal (as floats, so -0 == +0) and its index is
 * smaller. */
static int ranks_ahead(float sa, int64_t ia, float sb, int64_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

typedef struct {
  float s;
  int64_t id;
} cand_t;

/* Offer (s, id) to a best-first list of current length *len and capacity cap
 * (insertion; the worst entry falls off when full). */
static void offer(cand_t* list, int32_t* len, int32_t cap, float s, int64_t id) {
  int32_t n = *len;
  if (n == cap) {
    if (!ranks_ahead(s, id, list[n - 1].s, list[n - 1].id)) return;
    n--;
  }
  int32_t p = n;
  while (p > 0 && ranks_ahead(s, id, list[p - 1].s, list[p - 1].id)) {
    list[p] = list[p - 1];
    p--;
  }
  list[p].s = s;
  list[p].id = id;
  *len = n + 1;
}

static int cmp_cand(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (ranks_ahead(x->s, x->id, y->s, y->id)) return -1;
  if (ranks_ahead(y->s, y->id, x->s, x->id)) return 1;
  return 0;
}

/* ------------------------------------------------------------ addressing */

int sdm_ref_half_scores(const float* x, const float* C, int32_t n_sub, int32_t dh, float* s) {
  if (!x || !C || !s) return SDM_REF_ERR_NULL;
  if (n_sub < 1 || dh < 1) return SDM_REF_ERR_SHAPE;
  for (int32_t i = 0; i < n_sub; i++) {
    float acc = 0.0f;
    for (int32_t e = 0; e < dh; e++) {
      float p = x[e] * C[(int64_t)i * dh + e];
      acc = acc + p;
    }
    s[i] = acc;
  }
  return SDM_REF_OK;
}

int sdm_ref_topk_bruteforce(const float* s1, const float* s2, int32_t n_sub, int32_t k,
                            int32_t* idx, float* score) {
  if (!s1 || !s2 || !idx || !score) return SDM_REF_ERR_NULL;
  if (n_sub < 1 || (int64_t)n_sub * n_sub > 0x7fffffffLL) return SDM_REF_ERR_SHAPE;
  int64_t N = (int64_t)n_sub * n_sub;
  if (k < 1 || k > N) return SDM_REF_ERR_SHAPE;
  cand_t* all = (cand_t*)malloc((size_t)N * sizeof(cand_t));
  if (!all) return SDM_REF_ERR_NOMEM;
  for (int64_t i = 0; i < n_sub; i++)
    for (int64_t j = 0; j < n_sub; j++) {
      all[i * n_sub + j].s = s1[i] + s2[j];
      all[i * n_sub + j].id = i * n_sub + j;
    }
  qsort(all, (size_t)N, sizeof(cand_t), cmp_cand);
  for (int32_t r = 0; r < k; r++) {
    idx[r] = (int32_t)all[r].id;
    score[r] = all[r].s;
  }
  free(all);
  return SDM_REF_OK;
}

/* Core of the two-stage selection.  Writes the best `keep` outer-sum
 * candidates (keep <= k+1) into out[] and returns how many were produced. */
static int32_t two_stage(const float* s1, const float* s2, int32_t n_sub, int32_t k, cand_t* l1,
                         cand_t* l2, cand_t* out) {
  int32_t m = k + 1 < n_sub ? k + 1 : n_sub; /* stage-1 list length */
  int32_t n1 = 0, n2 = 0;
  for (int32_t i = 0; i < n_sub; i++) offer(l1, &n1, m, s1[i], i);
  for (int32_t j = 0; j < n_sub; j++) offer(l2, &n2, m, s2[j], j);
  int64_t grid = (int64_t)m * m;
  int32_t keep = (int64_t)(k + 1) < grid ? k + 1 : (int32_t)grid;
  int32_t n = 0;
  for (int32_t a = 0; a < m; a++)
    for (int32_t b = 0; b < m; b++) {
      float s = l1[a].s + l2[b].s;
      int64_t slot = l1[a].id * n_sub + l2[b].id;
      offer(out, &n, keep, s, slot);
    }
  return n;
}

static float rel_gap(float a, float b) {
  /* a ranks at position k, b at k+1, so a >= b */
  if (a == b) return 0.0f;
  float fa = fabsf(a), fb = fabsf(b);
  float den = fa > fb ? fa : fb;
  return (a - b) / den;
}

int sdm_ref_two_stage_topk(const float* s1, const float* s2, int32_t n_sub, int32_t k,
                           int32_t* idx, float* score, float* gap) {
  if (!s1 || !s2 || !idx || !score) return SDM_REF_ERR_NULL;
  if (n_sub < 1 || (int64_t)n_sub * n_sub > 0x7fffffffLL) return SDM_REF_ERR_SHAPE;
  int64_t N = (int64_t)n_sub * n_sub;
  if (k < 1 || k > N) return SDM_REF_ERR_SHAPE;
  int32_t m = k + 1 < n_sub ? k + 1 : n_sub;
  cand_t* l1 = (cand_t*)malloc((size_t)m * sizeof(cand_t));
  cand_t* l2 = (cand_t*)malloc((size_t)m * sizeof(cand_t));
  cand_t* out = (cand_t*)malloc((size_t)(k + 1) * sizeof(cand_t));
  if (!l1 || !l2 || !out) {
    free(l1), free(l2), free(out);
    return SDM_REF_ERR_NOMEM;
  }
  int32_t n = two_stage(s1, s2, n_sub, k, l1, l2, out);
  for (int32_t r = 0; r < k; r++) {
    idx[r] = (int32_t)out[r].id;
    score[r] = out[r].s;
  }
  if (gap) *gap = n > k ? rel_gap(out[k - 1].s, out[k].s) : INFINITY;
  free(l1), free(l2), free(out);
  return SDM_REF_OK;
}

int sdm_ref_softmax(const float* score, int32_t k, float* w) {
  if (!score || !w) return SDM_REF_ERR_NULL;
  if (k < 1) return SDM_REF_ERR_SHAPE;
  float mx = score[0]; /* rank order: the first score is the largest */
  float z = 0.0f;
  for (int32_t r = 0; r < k; r++) {
    w[r] = expf(score[r] - mx);
    z = z + w[r];
  }
  for (int32_t r = 0; r < k; r++) w[r] = w[r] / z;
  return SDM_REF_OK;
}

static int check_dims(const sdm_ref_dims* d) {
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->d_k < 2 || (d->d_k & 1) || d->n_sub < 1 ||
      d->d_v < 1)
    return SDM_REF_ERR_SHAPE;
  int64_t N = (int64_t)d->n_sub * d->n_sub;
  if (N > 0x7fffffffLL) return SDM_REF_ERR_SHAPE;
  if (d->W < 1 || d->W > N || d->R < 1 || d->R > N) return SDM_REF_ERR_SHAPE;
  return SDM_REF_OK;
}

int sdm_ref_score_topk(const sdm_ref_dims* d, int32_t dtype, const void* qp, const void* kp,
                       const void* subkeys, int32_t* widx, float* wwt, float* wgap,
                       int32_t* ridx, float* rwt, float* rgap) {
  if (!d || !qp || !kp || !subkeys || !widx || !wwt || !ridx || !rwt) return SDM_REF_ERR_NULL;
  if (dtype != SDM_REF_F32 && dtype != SDM_REF_BF16) return SDM_REF_ERR_DTYPE;
  int rc = check_dims(d);
  if (rc) return rc;
  const int32_t dh = d->d_k / 2, n_sub = d->n_sub;
  const int32_t kmax = d->W > d->R ? d->W : d->R;
  const int32_t mmax = kmax + 1 < n_sub ? kmax + 1 : n_sub;
  float* x = (float*)malloc((size_t)dh * sizeof(float));
  float* C = (float*)malloc((size_t)n_sub * dh * sizeof(float));
  float* s1 = (float*)malloc((size_t)n_sub * sizeof(float));
  float* s2 = (float*)malloc((size_t)n_sub * sizeof(float));
  float* C2 = (float*)malloc((size_t)n_sub * dh * sizeof(float));
  cand_t* l1 = (cand_t*)malloc((size_t)mmax * sizeof(cand_t));
  cand_t* l2 = (cand_t*)malloc((size_t)mmax * sizeof(cand_t));
  cand_t* out = (cand_t*)malloc((size_t)(kmax + 1) * sizeof(cand_t));
  float* sc = (float*)malloc((size_t)kmax * sizeof(float));
  if (!x || !C || !s1 || !s2 || !C2 || !l1 || !l2 || !out || !sc) {
    free(x), free(C), free(s1), free(s2), free(C2), free(l1), free(l2), free(out), free(sc);
    return SDM_REF_ERR_NOMEM;
  }
  for (int32_t b = 0; b < d->B; b++)
    for (int32_t h = 0; h < d->H; h++) {
      /* this head's two sub-key tables, widened to fp32 */
      int64_t cbase = (int64_t)h * 2 * n_sub * dh;
      for (int64_t e = 0; e < (int64_t)n_sub * dh; e++) {
        C[e] = load_elem(subkeys, dtype, cbase + e);
        C2[e] = load_elem(subkeys, dtype, cbase + (int64_t)n_sub * dh + e);
      }
      for (int32_t t = 0; t < d->T; t++) {
        int64_t tok = ((int64_t)b * d->H + h) * d->T + t;
        for (int pass = 0; pass < 2; pass++) { /* 0: key -> write, 1: query -> read */
          const void* src = pass == 0 ? kp : qp;
          int32_t k = pass == 0 ? d->W : d->R;
          int32_t* oidx = pass == 0 ? widx + tok * d->W : ridx + tok * d->R;
          float* owt = pass == 0 ? wwt + tok * d->W : rwt + tok * d->R;
          float* ogap = pass == 0 ? wgap : rgap;
          /* half 1: elements [0, dh); half 2: [dh, d_k) */
          for (int32_t e = 0; e < dh; e++) x[e] = load_elem(src, dtype, tok * d->d_k + e);
          sdm_ref_half_scores(x, C, n_sub, dh, s1);
          for (int32_t e = 0; e < dh; e++) x[e] = load_elem(src, dtype, tok * d->d_k + dh + e);
          sdm_ref_half_scores(x, C2, n_sub, dh, s2);
          int32_t n = two_stage(s1, s2, n_sub, k, l1, l2, out);
          for (int32_t r = 0; r < k; r++) {
            oidx[r] = (int32_t)out[r].id;
            sc[r] = out[r].s;
          }
          sdm_ref_softmax(sc, k, owt);
          if (ogap) ogap[tok] = n > k ? rel_gap(out[k - 1].s, out[k].s) : INFINITY;
        }
      }
    }
  free(x), free(C), free(s1), free(s2), free(C2), free(l1), free(l2), free(out), free(sc);
  return SDM_REF_OK;
}

/* ------------------------------------------------------------------ scan */

int sdm_ref_scan(const sdm_ref_dims* d, int32_t v_dtype, float* M, const int32_t* widx,
                 const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
                 const float* alpha, const float* beta, float* out) {
  if (!d || !M || !widx || !wwt || !ridx || !rwt || !v || !alpha || !beta || !out)
    return SDM_REF_ERR_NULL;
  if (v_dtype != SDM_REF_F32 && v_dtype != SDM_REF_BF16) return SDM_REF_ERR_DTYPE;
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->n_sub < 1 || d->d_v < 1) return SDM_REF_ERR_SHAPE;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  if (N > 0x7fffffffLL || d->W < 1 || d->W > N || d->R < 1 || d->R > N) return SDM_REF_ERR_SHAPE;
  const int32_t dv = d->d_v;
  float* vt = (float*)malloc((size_t)dv * sizeof(float));
  if (!vt) return SDM_REF_ERR_NOMEM;
  /* slot indices are checked before anything is written */
  const int64_t ntok = (int64_t)d->B * d->H * d->T;
  for (int64_t i = 0; i < ntok * d->W; i++)
    if (widx[i] < 0 || widx[i] >= N) return free(vt), SDM_REF_ERR_SHAPE;
  for (int64_t i = 0; i < ntok * d->R; i++)
    if (ridx[i] < 0 || ridx[i] >= N) return free(vt), SDM_REF_ERR_SHAPE;

  for (int64_t st = 0; st < (int64_t)d->B * d->H; st++) { /* one (b, h) stream */
    float* Ms = M + st * N * dv;
    for (int32_t t = 0; t < d->T; t++) {
      const int64_t tok = st * d->T + t;
      const float a = alpha[tok], be = beta[tok];
      for (int32_t e = 0; e < dv; e++) vt[e] = load_elem(v, v_dtype, tok * dv + e);
      /* gated delta write on the W selected rows, rank order */
      for (int32_t r = 0; r < d->W; r++) {
        float* row = Ms + (int64_t)widx[tok * d->W + r] * dv;
        const float c = be * wwt[tok * d->W + r];
        const float omc = 1.0f - c;
        for (int32_t e = 0; e < dv; e++) {
          const float mt = a * row[e];        /* forget gate */
          const float keep = omc * mt;         /* (1 - c) m~ */
          const float put = c * vt[e];         /* c v */
          row[e] = keep + put;
        }
      }
      /* sparse read of the post-write rows, rank order */
      float* o = out + tok * dv;
      for (int32_t e = 0; e < dv; e++) {
        float acc = 0.0f;
        for (int32_t r = 0; r < d->R; r++) {
          const float* row = Ms + (int64_t)ridx[tok * d->R + r] * dv;
          acc = acc + rwt[tok * d->R + r] * row[e];
        }
        o[e] = acc;
      }
    }
  }
  free(vt);
  return SDM_REF_OK;
}

/* ------------------------------------------------------- dense baseline */

int sdm_ref_gdn_scan(int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t d_v, int32_t dtype,
                     float* S, const void* k, const void* q, const void* v, const float* alpha,
                     const float* beta, float* out) {
  if (!S || !k || !q || !v || !alpha || !beta || !out) return SDM_REF_ERR_NULL;
  if (dtype != SDM_REF_F32 && dtype != SDM_REF_BF16) return SDM_REF_ERR_DTYPE;
  if (B < 1 || H < 1 || T < 0 || d_k < 1 || d_v < 1) return SDM_REF_ERR_SHAPE;
  float* kt = (float*)malloc((size_t)d_k * sizeof(float));
  float* qt = (float*)malloc((size_t)d_k * sizeof(float));
  float* err = (float*)malloc((size_t)d_v * sizeof(float));
  if (!kt || !qt || !err) {
    free(kt), free(qt), free(err);
    return SDM_REF_ERR_NOMEM;
  }
  for (int64_t st = 0; st < (int64_t)B * H; st++) {
    float* Ss = S + st * (int64_t)d_v * d_k; /* S[a][b]: row a is a value dim */
    for (int32_t t = 0; t < T; t++) {
      const int64_t tok = st * T + t;
      const float a_t = alpha[tok], b_t = beta[tok];
      for (int32_t b = 0; b < d_k; b++) {
        kt[b] = load_elem(k, dtype, tok * d_k + b);
        qt[b] = load_elem(q, dtype, tok * d_k + b);
      }
      /* prediction p = S_{t-1} k and scaled error e = b (v - a p) */
      for (int32_t a = 0; a < d_v; a++) {
        float p = 0.0f;
        for (int32_t b = 0; b < d_k; b++) p = p + Ss[(int64_t)a * d_k + b] * kt[b];
        const float ap = a_t * p;
        const float diff = load_elem(v, dtype, tok * d_v + a) - ap;
        err[a] = b_t * diff;
      }
      /* S_t = a S_{t-1} + e k^T */
      for (int32_t a = 0; a < d_v; a++)
        for (int32_t b = 0; b < d_k; b++) {
          float* sab = Ss + (int64_t)a * d_k + b;
          const float decayed = a_t * *sab;
          const float add = err[a] * kt[b];
          *sab = decayed + add;
        }
      /* read after the update: o = S_t q */
      for (int32_t a = 0; a < d_v; a++) {
        float o = 0.0f;
        for (int32_t b = 0; b < d_k; b++) o = o + Ss[(int64_t)a * d_k + b] * qt[b];
        out[tok * d_v + a] = o;
      }
    }
  }
  free(kt), free(qt), free(err);
  return SDM_REF_OK;
}
