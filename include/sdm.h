/*
 * sdm.h -- C ABI of libsdm, the MI355X (gfx950) Sparse Delta Memory hot path.
 *
 * Sparse Delta Memory (SDM) replaces the small dense state of a gated
 * DeltaNet layer with an explicit table M of N = n_sub^2 rows of d_v floats
 * per (batch, head) stream, addressed through product keys.  Source of the
 * method: the gist.science technical summaries of paper 2607.07386, "Sparse
 * Delta Memory" (Spanish page, section "Mecanismo Central", items 1-4, and
 * section "Diseno IsoFLOP"; French page, section "Mecanisme Central").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (HBM of the current HIP device)
 *    owned by the caller; the library never allocates, frees or copies
 *    caller memory and never synchronises the host.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and the call returns at once; results are ready
 *    when the stream reaches that point.  Calls are stateless and reentrant.
 *  - Tensors are dense, row-major (C order), with the shapes given below and
 *    no padding.  Addresses must be 16-byte aligned.  When T == 0 the tensors
 *    with a T axis hold no elements and their pointers may be NULL.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    nonzero return nothing has been enqueued and no output was written.
 *    SDM_ERR_HIP reports a failed launch; faults inside a kernel surface at
 *    the caller's next synchronisation, as with any HIP kernel.
 *  - Inputs are assumed finite.  NaN scores give unspecified selections.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDM_OK = 0,
  SDM_ERR_NULL = 1,        /* a required pointer is NULL */
  SDM_ERR_SHAPE = 2,       /* sizes inconsistent (odd d_k, W > N, N >= 2^31, ...) */
  SDM_ERR_DTYPE = 3,       /* unknown element type */
  SDM_ERR_UNSUPPORTED = 4, /* valid problem outside the kernels' limits */
  SDM_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  SDM_ERR_HIP = 6,         /* a HIP launch or runtime call failed */
  SDM_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
  SDM_ERR_SCRATCH = 8      /* needs more than the library's static scratch */
} sdm_status;

typedef enum {
  SDM_F32 = 0,  /* IEEE binary32 */
  SDM_BF16 = 1  /* bfloat16 (upper half of a binary32), widened exactly to fp32 */
} sdm_dtype;

/* Sizes of one SDM problem.  N = n_sub * n_sub slots per stream.
 * B batches x H heads = B*H independent streams of T tokens each. */
typedef struct {
  int32_t B, H, T;   /* batch, heads, tokens per stream */
  int32_t d_k;       /* projected key/query width (even); halves of d_k/2 */
  int32_t n_sub;     /* sub-keys per half */
  int32_t d_v;       /* value width = row width of M */
  int32_t W, R;      /* write and read slots per token */
} sdm_dims;

/*
 * sdm_score_topk -- product-key addressing (Spanish page "Mecanismo Central"
 * item 2; French page "Mecanisme Central", "Selection de Cles Creuses").
 *
 * For each token of each stream (b,h), the projected key k' and query q' are
 * cut into halves x1 = x[0:d_k/2) and x2 = x[d_k/2:d_k).  Each half is scored
 * against its own sub-key table of head h:  s_c[i] = <x_c, C[h][c][i]>.  The
 * score of slot s = i*n_sub + j is s_1[i] + s_2[j].  The W best slots of k'
 * (write set) and the R best slots of q' (read set) are found with the
 * two-stage identity topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)); the
 * N-vector of slot scores is never formed.  Order: score descending, ties to
 * the lower index at both stages.  Weights: softmax (temperature 1) over the
 * selected slot scores, separately for the write and read sets.
 *
 *   qp, kp   [B][H][T][d_k]        in_dtype   projected query / key
 *   subkeys  [H][2][n_sub][d_k/2]  in_dtype   shared by queries and keys
 *   widx     [B][H][T][W]  int32   out: write slots, rank order
 *   wwt      [B][H][T][W]  fp32    out: write weights
 *   ridx     [B][H][T][R]  int32   out: read slots, rank order
 *   rwt      [B][H][T][R]  fp32    out: read weights
 *   workspace                       device scratch of at least
 *                                   sdm_score_topk_workspace_size(dims, in_dtype)
 *                                   bytes (may be NULL when that size is 0);
 *                                   its contents on entry do not matter.
 *
 * Scores are accumulated in fp32 (bf16 products are exact in fp32).
 * Candidate set: the (k+1) x (k+1) grid of the two halves' top-(k+1) lists.
 * fp32 inputs are scored in sequential order and ranked on that whole grid,
 * ties included.  bf16 inputs are scored on the matrix cores, in another
 * summation order; there a pair holding a half's (k+1)-th sub-key whose fp32
 * sum exactly ties the k-th selected sum may lose to a higher slot index.
 * Kernel limits (else SDM_ERR_UNSUPPORTED): n_sub a multiple of 16 and
 * <= 1024, d_k/2 a multiple of 16 and <= 256, W, R <= min(n_sub, 128).
 * Inputs must be finite.
 */
int sdm_score_topk(const sdm_dims* dims, sdm_dtype in_dtype, const void* qp, const void* kp,
                   const void* subkeys, int32_t* widx, float* wwt, int32_t* ridx, float* rwt,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdm_score_topk_noalloc -- sdm_score_topk for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes no workspace.  The matrix-core copy of the
 * sub-key tables that sdm_score_topk writes into the caller's workspace goes
 * instead into a static device array of the library, 16 MiB per device, held
 * from the library's load until the process ends.  Nothing is allocated or
 * freed, on the device or the host.
 *
 * Arguments, layouts, results, limits and errors are sdm_score_topk's, plus:
 * sizes whose sdm_score_topk_workspace_size exceeds 16 MiB return
 * SDM_ERR_SCRATCH without enqueuing anything (bf16 needs 2 KiB per 16
 * sub-keys per half per 32 elements of the half: up to 16 heads of 1024
 * sub-keys with halves of 256; fp32 inputs need none).  The first call on a
 * device looks up the array's address there (SDM_ERR_HIP if that fails).
 * Every call on one device shares that device's array and rewrites it
 * completely before reading it; two calls that overlap on one device (on
 * different streams, or from several host threads) race on it.
 */
int sdm_score_topk_noalloc(const sdm_dims* dims, sdm_dtype in_dtype, const void* qp,
                           const void* kp, const void* subkeys, int32_t* widx, float* wwt,
                           int32_t* ridx, float* rwt, void* stream);

/* Bytes of device workspace sdm_score_topk needs for these sizes and input
 * type (0 when none, or when the sizes are invalid).  Pure host function.
 * With bf16 inputs the call first copies the sub-key tables there in the
 * order the matrix cores read them (about n_sub*d_k*2 bytes per head). */
size_t sdm_score_topk_workspace_size(const sdm_dims* dims, sdm_dtype in_dtype);

/*
 * sdm_pack_subkeys / sdm_score_topk_packed -- the same addressing split in two,
 * for callers that score many short calls against fixed sub-key tables (one
 * token per stream per call when decoding; Spanish page "Resultados
 * Experimentales", ablations, efficiency at inference).
 *
 * sdm_pack_subkeys writes the matrix-core copy of `subkeys` into `workspace`
 * (the copy sdm_score_topk makes on every call); only dims->H, d_k and n_sub
 * are used.  With fp32 inputs nothing needs packing and it returns SDM_OK
 * without touching the workspace.  sdm_score_topk_packed then scores as
 * sdm_score_topk does, reading the packed tables from `workspace` (read only;
 * the caller keeps it unchanged and owns it) instead of repacking them.  The
 * workspace must have been filled by sdm_pack_subkeys for the same H, d_k,
 * n_sub and sub-key values, on this stream or one ordered before it; results
 * are otherwise undefined.  `subkeys` is still passed (fp32 inputs read it).
 * Arguments, limits and errors are those of sdm_score_topk.
 */
int sdm_pack_subkeys(const sdm_dims* dims, sdm_dtype in_dtype, const void* subkeys,
                     void* workspace, size_t workspace_bytes, void* stream);
int sdm_score_topk_packed(const sdm_dims* dims, sdm_dtype in_dtype, const void* qp,
                          const void* kp, const void* subkeys, int32_t* widx, float* wwt,
                          int32_t* ridx, float* rwt, const void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * sdm_decode_step -- one decoding step in one launch: sdm_score_topk_packed's
 * addressing of one new token per stream, then, in the same workgroups, that
 * token's gated delta write and sparse read as sdm_scan does them (Spanish
 * page "Mecanismo Central" items 2 to 4).
 *
 * dims describe the addressing problem; every one of its B*H*T tokens is a
 * scan stream of its own holding that one token: token t of addressing stream
 * st = b*H + h is scan stream s = st*T + t.  For the decoding layout (dims
 * B = 1, H heads, T = the batch of sequences), s = h*T + t, i.e. head-major
 * [H][batch] streams, as sdm_scan sees them when decoding.
 *   qp, kp, subkeys, widx, wwt, ridx, rwt, workspace   as sdm_score_topk_packed
 *                            (slot lists and weights are written, [S][T][W/R])
 *   M      [B*H*T][N][d_v]  fp32      in/out, the streams' tables
 *   v      [B*H*T][d_v]     v_dtype
 *   alpha, beta [B*H*T]     fp32
 *   out    [B*H*T][d_v]     fp32      the read of each token
 * Tables are bit-identical to sdm_score_topk_packed followed by sdm_scan (the
 * same write in the same roundings); outputs agree with sdm_scan's to fp32
 * rounding (the read is summed in another order).  Slots outside [0, N) are
 * ignored as in sdm_scan.  Limits: those of sdm_score_topk, and d_v one of
 * 16, 32, 64, 128, 256 (else SDM_ERR_UNSUPPORTED); M, v and out 16-byte
 * aligned.
 */
int sdm_decode_step(const sdm_dims* dims, sdm_dtype in_dtype, const void* qp, const void* kp,
                    const void* subkeys, sdm_dtype v_dtype, float* M, const void* v,
                    const float* alpha, const float* beta, int32_t* widx, float* wwt,
                    int32_t* ridx, float* rwt, float* out, const void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * sdm_scan -- sparse gated-delta write and sparse read over the memory table
 * (Spanish page "Mecanismo Central" items 1, 3 and 4; French page
 * "Mecanisme Central").
 *
 * For every stream, tokens t = 0..T-1 in order:
 *   write: for each of the W write slots s with weight w, c = beta_t * w,
 *          M[s] <- (1 - c) * (alpha_t * M[s]) + c * v_t
 *          (= m~ + beta_t w (v_t - m~) with m~ = alpha_t M[s]), each product
 *          and the sum rounded separately in fp32; every other row is left
 *          bit-for-bit unchanged;
 *   read:  out_t = sum over the R read slots s of r_s * M[s], using the rows
 *          as they are AFTER token t's write.
 *
 *   M        [B][H][N][d_v]  fp32        in/out: memory table (M0 in, M_T out)
 *   widx/wwt [B][H][T][W]    int32/fp32  write slots (distinct within a token)
 *   ridx/rwt [B][H][T][R]    int32/fp32  read slots
 *   v        [B][H][T][d_v]  v_dtype
 *   alpha    [B][H][T]       fp32        forget gate
 *   beta     [B][H][T]       fp32        write strength
 *   out      [B][H][T][d_v]  fp32        output
 *   workspace                            device scratch of at least
 *                                        sdm_scan_workspace_size(dims) bytes
 *                                        (may be NULL when that size is 0);
 *                                        its contents on entry do not matter.
 *
 * An event whose slot lies outside [0, N) is ignored: nothing is read or
 * written for it, so its write changes no row and its read adds nothing to
 * the output (the table can never be touched outside the stream's rows).
 * The W write slots of one token must be distinct (not checked).  Results
 * are deterministic (the read sums use a fixed order).  Scanning [0,T1) and then [T1,T) with the same
 * M leaves a table bit-identical to one scan of [0,T), and bit-identical
 * outputs as well, except for tokens whose write plus read slots in one slot
 * partition exceed what a wave holds in registers (between 32 and 256 events,
 * sized from W, R and the partition count for three standard deviations above
 * the mean), whose outputs then agree to fp32 rounding.
 * Two calls that overlap on one device must not share M, out or workspace.
 * Kernel limits (else SDM_ERR_UNSUPPORTED): d_v a multiple of 16 and <= 512,
 * W, R <= 256.
 */
int sdm_scan(const sdm_dims* dims, sdm_dtype v_dtype, float* M, const int32_t* widx,
             const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
             const float* alpha, const float* beta, float* out, void* workspace,
             size_t workspace_bytes, void* stream);

/* Bytes of device workspace sdm_scan needs for these sizes (0 when none, or
 * when the sizes are invalid).  Pure host function. */
size_t sdm_scan_workspace_size(const sdm_dims* dims);

/*
 * sdm_scan_timeparallel -- the same scan as sdm_scan, evaluated slot by slot
 * instead of token by token.  Rows never interact: a row sees exactly the
 * write and read events that name it, in time order (a token's write of a
 * slot before its read of it).  The events of every stream are sorted by
 * (slot, time); each touched row is then loaded once, its writes applied in
 * time order, the row it holds at each read recorded, and each token's output
 * summed over its reads in rank order.  The parallelism is the number of
 * touched rows, not the number of streams.  Events whose slot lies outside
 * [0, N) are ignored as in sdm_scan (such a read adds its weight times a
 * zero row).
 *
 * Arguments, layouts and results as sdm_scan, with this workspace:
 *   workspace  sdm_scan_timeparallel_workspace_size(dims) bytes, 256-byte
 *              aligned: two buffers of slots and positions (16 bytes per
 *              event, events = B*H*T*(W+R)), the sort's digit counts (4
 *              bytes per 4096 events per digit, at most 1024 digits) and a
 *              read buffer of B*H*T*R*d_v floats.
 * The table and the outputs are bit-identical to the sequential scan's
 * definition (each element's fp32 operations in the same order).  Rows that
 * only reads touch are not stored.  Kernel limits (else
 * SDM_ERR_UNSUPPORTED): d_v a power of two in [16, 256]; B*H*T*(W+R) < 2^31.
 */
int sdm_scan_timeparallel(const sdm_dims* dims, sdm_dtype v_dtype, float* M,
                          const int32_t* widx, const float* wwt, const int32_t* ridx,
                          const float* rwt, const void* v, const float* alpha,
                          const float* beta, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of device workspace sdm_scan_timeparallel needs (0 when the sizes
 * are invalid or unsupported).  Pure host function. */
size_t sdm_scan_timeparallel_workspace_size(const sdm_dims* dims);

/*
 * Training: the gradients of the path (SDM is trained end to end, Spanish page
 * "Resultados Experimentales", and its initial table M0 is a learned parameter,
 * "Estado Inicial Aprendido").  The slot selections are piecewise constant, so
 * these are the gradients with the forward's slots held fixed.  A training
 * step runs sdm_score_topk, sdm_scan_record, then (with the loss gradient dout)
 * sdm_scan_backward and sdm_score_topk_backward.
 *
 * sdm_scan_record -- sdm_scan that also stores, for every write event, the
 * row as it was before the write:
 *   tape     [B][H][T][W][d_v]  fp32  out: tape[b,h,t,r] = M_{t-1}[widx[b,h,t,r]]
 * Everything else (arguments, workspace, limits, results) is sdm_scan's.
 */
int sdm_scan_record(const sdm_dims* dims, sdm_dtype v_dtype, float* M, const int32_t* widx,
                    const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
                    const float* alpha, const float* beta, float* out, float* tape,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdm_scan_backward -- reverse sweep of the scan.  With L a loss, dout = dL/do
 * and dM holding dL/dM_T on entry, it walks t = T-1..0 and for each token
 * takes the read's adjoint, then the write's:
 *   read:  drwt_r = <dout_t, M_t[ridx_r]>,  dM[ridx_r] += rwt_r * dout_t
 *   write: G = dM[s_r], old = tape_t[r], c = beta_t * wwt_r,
 *          dwwt_r = beta_t * <G, v_t - alpha_t old>,
 *          dbeta_t = sum_r wwt_r <G, v_t - alpha_t old>,
 *          dalpha_t = sum_r (1 - c) <G, old>,   dv_t = sum_r c G,
 *          dM[s_r] = (1 - c) alpha_t G,   M[s_r] = old.
 *
 *   M        [B][H][N][d_v]  fp32  in: the table after the forward (the one
 *                                  sdm_scan_record left); out: M0, restored
 *   dM       [B][H][N][d_v]  fp32  in: dL/dM_T (zeros if the final table is
 *                                  not used); out: dL/dM0
 *   widx, wwt, ridx, rwt, v, alpha, beta   the forward's inputs, unchanged
 *   tape     [B][H][T][W][d_v] fp32  from sdm_scan_record
 *   dout     [B][H][T][d_v]  fp32
 *   dv       [B][H][T][d_v]  fp32  out (fp32 whatever v_dtype is)
 *   dalpha, dbeta [B][H][T]  fp32  out
 *   dwwt     [B][H][T][W]    fp32  out: dL/dwwt
 *   drwt     [B][H][T][R]    fp32  out: dL/drwt
 *   workspace                       sdm_scan_backward_workspace_size(dims) bytes
 *
 * Write slots must be distinct within a token (as for sdm_scan); read slots
 * may repeat, and each read then adds its own share to the row's gradient (a
 * block of 8 tokens holding such a token is swept one read at a time, which
 * is slow but exact).  Events whose slot lies outside [0, N) are skipped, as
 * in the forward scan, and get dwwt / drwt = 0.
 * Results are deterministic.  The restored M equals M0 bit for bit (each
 * written row gets back its recorded value).  Kernel limits (else
 * SDM_ERR_UNSUPPORTED): d_v a power of two in [16, 256]; W, R <= 256.
 */
int sdm_scan_backward(const sdm_dims* dims, sdm_dtype v_dtype, float* M, float* dM,
                      const int32_t* widx, const float* wwt, const int32_t* ridx,
                      const float* rwt, const void* v, const float* alpha, const float* beta,
                      const float* tape, const float* dout, float* dv, float* dalpha,
                      float* dbeta, float* dwwt, float* drwt, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of device workspace sdm_scan_backward needs (0 when none, or when
 * the sizes are invalid or unsupported).  Pure host function. */
size_t sdm_scan_backward_workspace_size(const sdm_dims* dims);

/*
 * sdm_score_topk_backward -- adjoint of the addressing (Spanish page
 * "Mecanismo Central" item 2, softmax weights over the selected slot scores).
 * For each token and each side (writes: k', widx, wwt, dwwt; reads: q', ridx,
 * rwt, drwt), with slot s_r = i_r*n_sub + j_r:
 *   dsigma_r = w_r (dw_r - sum_u w_u dw_u)
 *   dx[0:d_k/2) = sum_r dsigma_r C[h][0][i_r],  dx[d_k/2:d_k) = sum_r dsigma_r C[h][1][j_r]
 *   dsubkeys[h][0][i_r] += dsigma_r x[0:d_k/2),  dsubkeys[h][1][j_r] += dsigma_r x[d_k/2:d_k)
 *
 *   qp, kp, subkeys           in_dtype, as given to sdm_score_topk
 *   widx, wwt, ridx, rwt      sdm_score_topk's outputs
 *   dwwt, drwt                fp32 gradients of the weights (sdm_scan_backward's)
 *   dq, dk    [B][H][T][d_k]  fp32 out (overwritten)
 *   dsubkeys  [H][2][n_sub][d_k/2] fp32 in/out: the gradient is ADDED (the
 *                             caller clears it, or accumulates over calls)
 *
 *   workspace                 device scratch of at least
 *                             sdm_score_topk_backward_workspace_size(dims)
 *                             bytes, 256-byte aligned; contents not kept
 *
 * Every output is deterministic: each sum is taken in a fixed order.  The
 * sub-key gradient is a sum per table row over the (token, side) pairs whose
 * slots use that row; the library groups those contributions by row with a
 * stable sort instead of accumulating them with atomics.  Kernel limits (else
 * SDM_ERR_UNSUPPORTED): n_sub <= 1024, d_k/2 a multiple of 16 and <= 256,
 * W, R <= 128, 4*B*H*T*max(W, R) < 2^31.  qp, kp, subkeys, dq, dk and
 * dsubkeys must be 16-byte aligned (SDM_ERR_ALIGN).
 */
int sdm_score_topk_backward(const sdm_dims* dims, sdm_dtype in_dtype, const void* qp,
                            const void* kp, const void* subkeys, const int32_t* widx,
                            const float* wwt, const int32_t* ridx, const float* rwt,
                            const float* dwwt, const float* drwt, float* dq, float* dk,
                            float* dsubkeys, void* workspace, size_t workspace_bytes,
                            void* stream);
/* Workspace bytes for sdm_score_topk_backward (0 when T == 0 or the problem
 * is invalid). */
size_t sdm_score_topk_backward_workspace_size(const sdm_dims* dims);

/*
 * sdm_route_topk -- router of routed-slot writes with selective decay (Spanish
 * page "Resumen Tecnico: Raven", section 2.2), a second workload on the same
 * table and scan.  Per token and side, over M slot logits z:
 *   m = sigmoid(z); keep the K largest (selected on z: sigmoid is strictly
 *   increasing; ties to the lower slot); r = m / (sum of the kept m);
 *   write side: wcoef = 1 - exp(a_t * r)  (a_t <= 0; computed as -expm1);
 *   read side:  rwt = r.
 * Lists are in rank order (logit descending, slot ascending).  With them,
 * sdm_scan(alpha = beta = 1, wwt = wcoef, rwt, v = u) applies the page's
 * S[i] = exp(a r_i) S[i] + (1 - exp(a r_i)) u_t on the routed slots only and
 * reads the query side's routed slots after the write.
 *
 *   zk, zq   [B][H][T][M]  fp32   write-side and read-side router logits
 *   a        [B][H][T]     fp32   decay (<= 0)
 *   widx     [B][H][T][K]  int32  out;  wcoef [B][H][T][K] fp32 out
 *   ridx     [B][H][T][K]  int32  out;  rwt   [B][H][T][K] fp32 out
 *
 * Inputs must be finite.  Kernel limits (else SDM_ERR_UNSUPPORTED): M <= 8192,
 * K <= 128.  For sdm_scan the table needs N = M = n_sub^2.
 */
int sdm_route_topk(int32_t B, int32_t H, int32_t T, int32_t M, int32_t K, const float* zk,
                   const float* zq, const float* a, int32_t* widx, float* wcoef, int32_t* ridx,
                   float* rwt, void* stream);

/*
 * sdm_gdn_scan -- the dense gated DeltaNet recurrence that SDM extends
 * (Spanish page "Planteamiento del Problema", "Metodologia"; its state
 * starts at zero, "Estado Inicial Aprendido"), used as the IsoFLOP baseline:
 *   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
 *   out_t = S_t q_t  (read after the update).
 *
 *   S        [B][H][d_v][d_k]  fp32   in/out: state (maps k to v)
 *   k, q     [B][H][T][d_k]    dtype
 *   v        [B][H][T][d_v]    dtype
 *   alpha, beta [B][H][T]      fp32
 *   out      [B][H][T][d_v]    fp32
 *
 * Kernel limits (else SDM_ERR_UNSUPPORTED): d_k = d_v = 128.
 */
int sdm_gdn_scan(int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t d_v, sdm_dtype dtype,
                 float* S, const void* k, const void* q, const void* v, const float* alpha,
                 const float* beta, float* out, void* stream);

/* Static string naming a status code. */
const char* sdm_status_str(int status);

/* Library version, e.g. "0.1.0". */
const char* sdm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SDM_H */
