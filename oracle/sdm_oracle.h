/*
 * sdm_oracle.h -- CPU oracle for the Sparse Delta Memory (SDM) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * Plain, single-threaded fp32 C, compiled with -ffp-contract=off: every
 * floating-point operation is one IEEE-754 binary32 operation, evaluated in
 * the order the comments state.  All pointers are HOST pointers owned by the
 * caller.  Every entry point returns 0 on success and a nonzero code on a bad
 * argument (in which case nothing has been written).
 *
 * Method source: "Sparse Delta Memory" technical summaries (gist.science
 * paper 2607.07386, Spanish page "Mecanismo Central" items 1-4 and "Diseno
 * IsoFLOP"; French page "Mecanisme Central").  The dense gated-delta baseline
 * follows the dense gated DeltaNet update S_t = a_t S + b_t (v_t - a_t S k_t) k_t^T
 * with the read o_t = S_t q_t taken after the update.
 */
#ifndef SDM_ORACLE_H
#define SDM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem sizes.  N = n_sub * n_sub slots; slot s = i * n_sub + j where i is
 * the sub-key index of the first half and j the sub-key index of the second. */
typedef struct {
  int32_t B, H, T, d_k, n_sub, d_v, W, R;
} sdm_ref_dims;

/* Element type of q', k', sub-keys and v: 0 = fp32, 1 = bf16 (raw uint16 bits,
 * widened to fp32 exactly). */
enum { SDM_REF_F32 = 0, SDM_REF_BF16 = 1 };

enum {
  SDM_REF_OK = 0,
  SDM_REF_ERR_NULL = 1,
  SDM_REF_ERR_SHAPE = 2,
  SDM_REF_ERR_DTYPE = 3,
  SDM_REF_ERR_NOMEM = 4
};

/* Scores of one half-vector x[0..dh) against n_sub sub-keys C[n_sub][dh]:
 * s[i] = sum over e ascending of x[e]*C[i][e] (fp32, accumulator starts at 0). */
int sdm_ref_half_scores(const float* x, const float* C, int32_t n_sub, int32_t dh, float* s);

/* Top-k over ALL n_sub^2 outer sums s1[i] + s2[j] (materialised), ordered by
 * (score descending, slot ascending).  idx[k] receives slots, score[k] sums. */
int sdm_ref_topk_bruteforce(const float* s1, const float* s2, int32_t n_sub, int32_t k,
                            int32_t* idx, float* score);

/* Two-stage top-k: stage 1 keeps the best min(k+1, n_sub) of each half, stage 2
 * ranks their outer sums.  Same output as above.  *gap (may be NULL) receives
 * the relative gap between the k-th and (k+1)-th sums, 0 for an exact tie, and
 * +inf when k = n_sub^2 (nothing is left out). */
int sdm_ref_two_stage_topk(const float* s1, const float* s2, int32_t n_sub, int32_t k,
                           int32_t* idx, float* score, float* gap);

/* Slot weights: softmax (temperature 1) of rank-ordered scores, max first. */
int sdm_ref_softmax(const float* score, int32_t k, float* w);

/* Full addressing for [B][H][T] tokens.
 *   qp, kp  : [B][H][T][d_k]      (dtype)
 *   subkeys : [H][2][n_sub][d_k/2] (dtype), shared by queries and keys
 *   widx, wwt, wgap : [B][H][T][W], [B][H][T][W], [B][H][T]
 *   ridx, rwt, rgap : [B][H][T][R], [B][H][T][R], [B][H][T]
 * wgap / rgap may be NULL. */
int sdm_ref_score_topk(const sdm_ref_dims* d, int32_t dtype, const void* qp, const void* kp,
                       const void* subkeys, int32_t* widx, float* wwt, float* wgap,
                       int32_t* ridx, float* rwt, float* rgap);

/* Sparse gated-delta scan, in place on M[B][H][N][d_v] (fp32).
 *   widx/wwt [B][H][T][W], ridx/rwt [B][H][T][R], v [B][H][T][d_v] (v_dtype),
 *   alpha/beta [B][H][T] fp32, out [B][H][T][d_v] fp32.
 * Within one token the W write slots must be distinct and in [0, N). */
int sdm_ref_scan(const sdm_ref_dims* d, int32_t v_dtype, float* M, const int32_t* widx,
                 const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
                 const float* alpha, const float* beta, float* out);

/* Dense gated-delta scan, in place on S[B][H][d_v][d_k] (fp32, maps k -> v).
 *   k, q [B][H][T][d_k], v [B][H][T][d_v] (dtype), alpha/beta [B][H][T],
 *   out [B][H][T][d_v]. */
int sdm_ref_gdn_scan(int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t d_v, int32_t dtype,
                     float* S, const void* k, const void* q, const void* v, const float* alpha,
                     const float* beta, float* out);

#ifdef __cplusplus
}
#endif
#endif
