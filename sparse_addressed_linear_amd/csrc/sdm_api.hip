// C ABI of libsdm: argument validation and dispatch.  Every pointer is a
// caller-owned device pointer; nothing is allocated or synchronised here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "sdm.h"
#include "sdm_internal.h"

namespace sdm {
size_t score_topk_lds_bytes(int n_sub, int W, int R);
}

namespace {

constexpr int64_t kMaxN = 0x7fffffffLL;
constexpr size_t kMaxLds = 160 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const sdm_dims* d) {
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->d_k < 2 || (d->d_k & 1) || d->n_sub < 1 ||
      d->d_v < 1)
    return SDM_ERR_SHAPE;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  if (N > kMaxN) return SDM_ERR_SHAPE;
  if (d->W < 1 || d->W > N || d->R < 1 || d->R > N) return SDM_ERR_SHAPE;
  if ((int64_t)d->B * d->H > 0x7fffffffLL) return SDM_ERR_SHAPE;
  return SDM_OK;
}

bool valid_dtype(int t) { return t == SDM_F32 || t == SDM_BF16; }

// Scratch of sdm_score_topk_noalloc: the matrix-core copy of the sub-key
// tables, in a file-scope device array instead of a caller's workspace.  Each
// device holds its own copy at its own address; host code uses only the
// address looked up per device below, never the array's name (which on the
// host is a stand-in, not a device address).
constexpr size_t kNoallocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call there and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SDM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SDM_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SDM_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SDM_OK;
}

}  // namespace

extern "C" {

size_t sdm_score_topk_workspace_size(const sdm_dims* d, sdm_dtype in_dtype) {
  if (!d || check_dims(d) != SDM_OK || !valid_dtype(in_dtype)) return 0;
  return sdm::score_topk_workspace_bytes(d->H, d->n_sub, d->d_k, in_dtype == SDM_BF16);
}

// checks shared by the addressing entry points (everything but the workspace)
static int check_score(const sdm_dims* d, sdm_dtype in_dtype, const void* qp, const void* kp,
                       const void* subkeys, const void* widx, const void* wwt,
                       const void* ridx, const void* rwt) {
  if (!d || !subkeys) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  // tensors with a T axis have no elements when T == 0 and may then be NULL
  if (d->T > 0 && (!qp || !kp || !widx || !wwt || !ridx || !rwt)) return SDM_ERR_NULL;
  if (!valid_dtype(in_dtype)) return SDM_ERR_DTYPE;
  const int dh = d->d_k / 2;
  if (d->n_sub > 1024 || d->n_sub % 16 != 0 || dh % 16 != 0 || dh > 256 || d->W > d->n_sub || d->R > d->n_sub ||
      d->W > 128 || d->R > 128)
    return SDM_ERR_UNSUPPORTED;
  if (sdm::score_topk_lds_bytes(d->n_sub, d->W, d->R) > kMaxLds) return SDM_ERR_UNSUPPORTED;
  if (!aligned16(qp) || !aligned16(kp) || !aligned16(subkeys) || !aligned16(widx) ||
      !aligned16(wwt) || !aligned16(ridx) || !aligned16(rwt))
    return SDM_ERR_ALIGN;
  return SDM_OK;
}

static int run_score(const sdm_dims* d, sdm_dtype in_dtype, const void* qp, const void* kp,
                     const void* subkeys, int32_t* widx, float* wwt, int32_t* ridx, float* rwt,
                     const void* workspace, size_t workspace_bytes, bool pack, void* stream) {
  int rc = check_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt);
  if (rc) return rc;
  if (d->T == 0) return SDM_OK;
  const size_t need =
      sdm::score_topk_workspace_bytes(d->H, d->n_sub, d->d_k, in_dtype == SDM_BF16);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SDM_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return SDM_ERR_ALIGN;
  sdm::ScoreArgs a{};
  a.packed = const_cast<void*>(workspace);  // written only when pack is set
  a.qp = qp;
  a.kp = kp;
  a.subkeys = subkeys;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.S = d->B * d->H;
  a.H = d->H;
  a.T = d->T;
  a.d_k = d->d_k;
  a.n_sub = d->n_sub;
  a.W = d->W;
  a.R = d->R;
  hipError_t e = sdm::launch_score_topk(a, in_dtype == SDM_BF16, pack, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_score_topk(const sdm_dims* d, sdm_dtype in_dtype, const void* qp, const void* kp,
                   const void* subkeys, int32_t* widx, float* wwt, int32_t* ridx, float* rwt,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return run_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt, workspace,
                   workspace_bytes, true, stream);
}

int sdm_pack_subkeys(const sdm_dims* d, sdm_dtype in_dtype, const void* subkeys, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!d || !subkeys) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (!valid_dtype(in_dtype)) return SDM_ERR_DTYPE;
  const int dh = d->d_k / 2;
  if (d->n_sub > 1024 || d->n_sub % 16 != 0 || dh % 16 != 0 || dh > 256) return SDM_ERR_UNSUPPORTED;
  if (!aligned16(subkeys)) return SDM_ERR_ALIGN;
  const size_t need =
      sdm::score_topk_workspace_bytes(d->H, d->n_sub, d->d_k, in_dtype == SDM_BF16);
  if (need == 0) return SDM_OK;  // fp32 sub-keys are read as they are
  if (!workspace || workspace_bytes < need) return SDM_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SDM_ERR_ALIGN;
  sdm::ScoreArgs a{};
  a.packed = workspace;
  a.subkeys = subkeys;
  a.H = d->H;
  a.d_k = d->d_k;
  a.n_sub = d->n_sub;
  hipError_t e = sdm::launch_pack_subkeys(a, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_score_topk_packed(const sdm_dims* d, sdm_dtype in_dtype, const void* qp, const void* kp,
                          const void* subkeys, int32_t* widx, float* wwt, int32_t* ridx,
                          float* rwt, const void* workspace, size_t workspace_bytes,
                          void* stream) {
  return run_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt, workspace,
                   workspace_bytes, false, stream);
}

int sdm_decode_step(const sdm_dims* d, sdm_dtype in_dtype, const void* qp, const void* kp,
                    const void* subkeys, sdm_dtype v_dtype, float* M, const void* v,
                    const float* alpha, const float* beta, int32_t* widx, float* wwt,
                    int32_t* ridx, float* rwt, float* out, const void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = check_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt);
  if (rc) return rc;
  if (d->T > 0 && (!M || !v || !alpha || !beta || !out)) return SDM_ERR_NULL;
  if (!valid_dtype(v_dtype)) return SDM_ERR_DTYPE;
  // one lane group of d_v/4 lanes per row (a power of two dividing 64)
  if (d->d_v != 16 && d->d_v != 32 && d->d_v != 64 && d->d_v != 128 && d->d_v != 256)
    return SDM_ERR_UNSUPPORTED;
  if (d->T == 0) return SDM_OK;
  const size_t need =
      sdm::score_topk_workspace_bytes(d->H, d->n_sub, d->d_k, in_dtype == SDM_BF16);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SDM_ERR_WORKSPACE;
  if ((need > 0 && !aligned16(workspace)) || !aligned16(M) || !aligned16(v) || !aligned16(out))
    return SDM_ERR_ALIGN;
  sdm::ScoreArgs a{};
  a.packed = const_cast<void*>(workspace);  // read only: the sub-keys are packed already
  a.qp = qp;
  a.kp = kp;
  a.subkeys = subkeys;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.S = d->B * d->H;
  a.H = d->H;
  a.T = d->T;
  a.d_k = d->d_k;
  a.n_sub = d->n_sub;
  a.W = d->W;
  a.R = d->R;
  a.M = M;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.N = (int64_t)d->n_sub * d->n_sub;
  a.d_v = d->d_v;
  a.v_bf16 = v_dtype == SDM_BF16 ? 1 : 0;
  a.fuse = 1;
  hipError_t e = sdm::launch_score_topk(a, in_dtype == SDM_BF16, false, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_score_topk_noalloc(const sdm_dims* d, sdm_dtype in_dtype, const void* qp,
                           const void* kp, const void* subkeys, int32_t* widx, float* wwt,
                           int32_t* ridx, float* rwt, void* stream) {
  int rc = check_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt);
  if (rc) return rc;
  if (d->T == 0) return SDM_OK;
  const size_t need =
      sdm::score_topk_workspace_bytes(d->H, d->n_sub, d->d_k, in_dtype == SDM_BF16);
  if (need > kNoallocScratchBytes) return SDM_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return run_score(d, in_dtype, qp, kp, subkeys, widx, wwt, ridx, rwt, ws, need, true, stream);
}

size_t sdm_scan_workspace_size(const sdm_dims* d) {
  if (!d || check_dims(d) != SDM_OK) return 0;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  return sdm::plan_scan(d->B * d->H, d->T, N, d->d_v, d->W, d->R).work_bytes;
}

// kernel limits of the addressing adjoint (record positions are 32-bit)
static int score_bwd_shape_ok(const sdm_dims* d) {
  const int dh = d->d_k / 2;
  if (d->n_sub > 1024 || dh > 256 || dh % 16 != 0 || d->W > 128 || d->R > 128 ||
      d->W > d->n_sub * d->n_sub || sdm::score_bwd_lds_bytes(d->W > d->R ? d->W : d->R) > kMaxLds ||
      sdm::score_bwd_records(d->B * d->H, d->T, d->W, d->R) > 0x7fffffffLL ||
      (int64_t)d->H * 2 * d->n_sub >= 0x7fffffffLL)  // record keys (h, half, row) in 31 bits
    return SDM_ERR_UNSUPPORTED;
  return SDM_OK;
}

size_t sdm_score_topk_backward_workspace_size(const sdm_dims* d) {
  if (!d || check_dims(d) != SDM_OK || score_bwd_shape_ok(d) != SDM_OK) return 0;
  if (d->T == 0) return 0;
  return sdm::score_bwd_workspace_bytes(d->B * d->H, d->T, d->H, d->n_sub, d->W, d->R);
}

int sdm_score_topk_backward(const sdm_dims* d, sdm_dtype in_dtype, const void* qp,
                            const void* kp, const void* subkeys, const int32_t* widx,
                            const float* wwt, const int32_t* ridx, const float* rwt,
                            const float* dwwt, const float* drwt, float* dq, float* dk,
                            float* dsubkeys, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!d || !subkeys || !dsubkeys) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->T > 0 && (!qp || !kp || !widx || !wwt || !ridx || !rwt || !dwwt || !drwt || !dq || !dk))
    return SDM_ERR_NULL;
  if (!valid_dtype(in_dtype)) return SDM_ERR_DTYPE;
  rc = score_bwd_shape_ok(d);
  if (rc) return rc;
  // rows of the inputs, of dq / dk and of the sub-key gradient move 16 bytes per lane
  if (!aligned16(qp) || !aligned16(kp) || !aligned16(subkeys) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dsubkeys))
    return SDM_ERR_ALIGN;
  if (d->T == 0) return SDM_OK;
  const size_t need = sdm::score_bwd_workspace_bytes(d->B * d->H, d->T, d->H, d->n_sub, d->W, d->R);
  if (!workspace || workspace_bytes < need) return SDM_ERR_WORKSPACE;
  if (((uintptr_t)workspace) & 255) return SDM_ERR_ALIGN;
  sdm::ScoreBwdArgs a{};
  a.qp = qp;
  a.kp = kp;
  a.subkeys = subkeys;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.dwwt = dwwt;
  a.drwt = drwt;
  a.dq = dq;
  a.dk = dk;
  a.dsub = dsubkeys;
  a.S = d->B * d->H;
  a.H = d->H;
  a.T = d->T;
  a.d_k = d->d_k;
  a.n_sub = d->n_sub;
  a.W = d->W;
  a.R = d->R;
  hipError_t e = sdm::launch_score_bwd(a, in_dtype == SDM_BF16, workspace, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_route_topk(int32_t B, int32_t H, int32_t T, int32_t M, int32_t K, const float* zk,
                   const float* zq, const float* a, int32_t* widx, float* wcoef, int32_t* ridx,
                   float* rwt, void* stream) {
  if (B < 1 || H < 1 || T < 0 || M < 1 || K < 1 || K > M) return SDM_ERR_SHAPE;
  if (T > 0 && (!zk || !zq || !a || !widx || !wcoef || !ridx || !rwt)) return SDM_ERR_NULL;
  if (M > 8192 || K > 128 || sdm::route_lds_bytes(M, K) > kMaxLds) return SDM_ERR_UNSUPPORTED;
  if (T == 0) return SDM_OK;
  sdm::RouteArgs r{};
  r.zk = zk;
  r.zq = zq;
  r.a = a;
  r.widx = widx;
  r.wcoef = wcoef;
  r.ridx = ridx;
  r.rwt = rwt;
  r.units = (int64_t)B * H * T;
  r.M = M;
  r.K = K;
  hipError_t e = sdm::launch_route(r, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

static int run_scan(const sdm_dims* d, sdm_dtype v_dtype, float* M, const int32_t* widx,
                    const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
                    const float* alpha, const float* beta, float* out, float* tape,
                    bool want_tape, void* workspace, size_t workspace_bytes, void* stream) {
  if (!d || !M) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->T > 0 && (!widx || !wwt || !ridx || !rwt || !v || !alpha || !beta || !out ||
                   (want_tape && !tape)))
    return SDM_ERR_NULL;
  if (!valid_dtype(v_dtype)) return SDM_ERR_DTYPE;
  if (d->d_v % 16 != 0 || d->d_v > 512 || d->W > 256 || d->R > 256) return SDM_ERR_UNSUPPORTED;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  const sdm::ScanPlan p =
      sdm::plan_scan(d->B * d->H, d->T, N, d->d_v, d->W, d->R, want_tape);
  if (p.lds > kMaxLds) return SDM_ERR_UNSUPPORTED;
  // one workgroup per (stream, column slice, partition): a 32-bit grid
  if ((int64_t)d->B * d->H * p.CS * p.P > 0x7fffffffLL) return SDM_ERR_UNSUPPORTED;
  if (p.work_bytes > 0 && (!workspace || workspace_bytes < p.work_bytes))
    return SDM_ERR_WORKSPACE;
  if (!aligned16(M) || !aligned16(v) || !aligned16(out) ||
      (p.work_bytes && !aligned16(workspace)) || (want_tape && !aligned16(tape)))
    return SDM_ERR_ALIGN;
  if (d->T == 0) return SDM_OK;
  sdm::ScanArgs a{};
  a.M = M;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.work = static_cast<float*>(workspace);
  a.tape = want_tape ? tape : nullptr;
  a.N = N;
  a.S = d->B * d->H;
  a.T = d->T;
  a.d_v = d->d_v;
  a.W = d->W;
  a.R = d->R;
  hipError_t e = sdm::launch_scan(a, p, v_dtype == SDM_BF16, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_scan(const sdm_dims* d, sdm_dtype v_dtype, float* M, const int32_t* widx,
             const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
             const float* alpha, const float* beta, float* out, void* workspace,
             size_t workspace_bytes, void* stream) {
  return run_scan(d, v_dtype, M, widx, wwt, ridx, rwt, v, alpha, beta, out, nullptr, false,
                  workspace, workspace_bytes, stream);
}

int sdm_scan_record(const sdm_dims* d, sdm_dtype v_dtype, float* M, const int32_t* widx,
                    const float* wwt, const int32_t* ridx, const float* rwt, const void* v,
                    const float* alpha, const float* beta, float* out, float* tape,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return run_scan(d, v_dtype, M, widx, wwt, ridx, rwt, v, alpha, beta, out, tape, true,
                  workspace, workspace_bytes, stream);
}

// time-parallel scan: whole rows per lane group (d_v/4 lanes), events of all
// streams counted and placed in int32
static int tp_shape_ok(const sdm_dims* d) {
  const bool dv_ok = d->d_v >= 16 && d->d_v <= 256 && (d->d_v & (d->d_v - 1)) == 0;
  if (!dv_ok || !sdm::tp_sizes_ok(d->B * d->H, d->T, d->W, d->R))
    return SDM_ERR_UNSUPPORTED;
  return SDM_OK;
}

size_t sdm_scan_timeparallel_workspace_size(const sdm_dims* d) {
  if (!d || check_dims(d) != SDM_OK || tp_shape_ok(d) != SDM_OK) return 0;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  return sdm::tp_workspace_bytes(d->B * d->H, d->T, N, d->d_v, d->W, d->R);
}

int sdm_scan_timeparallel(const sdm_dims* d, sdm_dtype v_dtype, float* M, const int32_t* widx,
                          const float* wwt, const int32_t* ridx, const float* rwt,
                          const void* v, const float* alpha, const float* beta, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!d || !M) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->T > 0 && (!widx || !wwt || !ridx || !rwt || !v || !alpha || !beta || !out))
    return SDM_ERR_NULL;
  if (!valid_dtype(v_dtype)) return SDM_ERR_DTYPE;
  rc = tp_shape_ok(d);
  if (rc) return rc;
  if (d->T == 0) return SDM_OK;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  const size_t need = sdm::tp_workspace_bytes(d->B * d->H, d->T, N, d->d_v, d->W, d->R);
  if (!workspace || workspace_bytes < need) return SDM_ERR_WORKSPACE;
  if (!aligned16(M) || !aligned16(v) || !aligned16(out) || (((uintptr_t)workspace) & 255))
    return SDM_ERR_ALIGN;
  sdm::TpArgs a{};
  a.M = M;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.N = N;
  a.S = d->B * d->H;
  a.T = d->T;
  a.d_v = d->d_v;
  a.W = d->W;
  a.R = d->R;
  hipError_t e = sdm::launch_scan_tp(a, v_dtype == SDM_BF16, workspace, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

// whole rows per workgroup: d_v = 4 * (lanes per row), a power of two up to 256
static bool bwd_dv_ok(int d_v) { return d_v >= 16 && d_v <= 256 && (d_v & (d_v - 1)) == 0; }

size_t sdm_scan_backward_workspace_size(const sdm_dims* d) {
  if (!d || check_dims(d) != SDM_OK || !bwd_dv_ok(d->d_v)) return 0;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  return sdm::plan_scan_bwd(d->B * d->H, d->T, N, d->d_v, d->W, d->R).work_bytes;
}

int sdm_scan_backward(const sdm_dims* d, sdm_dtype v_dtype, float* M, float* dM,
                      const int32_t* widx, const float* wwt, const int32_t* ridx,
                      const float* rwt, const void* v, const float* alpha, const float* beta,
                      const float* tape, const float* dout, float* dv, float* dalpha,
                      float* dbeta, float* dwwt, float* drwt, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!d || !M || !dM) return SDM_ERR_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->T > 0 && (!widx || !wwt || !ridx || !rwt || !v || !alpha || !beta || !tape || !dout ||
                   !dv || !dalpha || !dbeta || !dwwt || !drwt))
    return SDM_ERR_NULL;
  if (!valid_dtype(v_dtype)) return SDM_ERR_DTYPE;
  if (!bwd_dv_ok(d->d_v) || d->W > 256 || d->R > 256) return SDM_ERR_UNSUPPORTED;
  const int64_t N = (int64_t)d->n_sub * d->n_sub;
  const sdm::ScanBwdPlan p = sdm::plan_scan_bwd(d->B * d->H, d->T, N, d->d_v, d->W, d->R);
  if (p.lds > kMaxLds) return SDM_ERR_UNSUPPORTED;
  // one workgroup per (stream, partition): a 32-bit grid
  if ((int64_t)d->B * d->H * p.P > 0x7fffffffLL) return SDM_ERR_UNSUPPORTED;
  if (p.work_bytes > 0 && (!workspace || workspace_bytes < p.work_bytes))
    return SDM_ERR_WORKSPACE;
  if (!aligned16(M) || !aligned16(dM) || !aligned16(v) || !aligned16(tape) || !aligned16(dout) ||
      !aligned16(dv) || (p.work_bytes && !aligned16(workspace)))
    return SDM_ERR_ALIGN;
  if (d->T == 0) return SDM_OK;
  sdm::ScanBwdArgs a{};
  a.M = M;
  a.dM = dM;
  a.widx = widx;
  a.wwt = wwt;
  a.ridx = ridx;
  a.rwt = rwt;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.tape = tape;
  a.dout = dout;
  a.dv = dv;
  a.dalpha = dalpha;
  a.dbeta = dbeta;
  a.dwwt = dwwt;
  a.drwt = drwt;
  a.work = static_cast<float*>(workspace);
  a.N = N;
  a.S = d->B * d->H;
  a.T = d->T;
  a.d_v = d->d_v;
  a.W = d->W;
  a.R = d->R;
  hipError_t e = sdm::launch_scan_bwd(a, p, v_dtype == SDM_BF16, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

int sdm_gdn_scan(int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t d_v, sdm_dtype dtype,
                 float* S, const void* k, const void* q, const void* v, const float* alpha,
                 const float* beta, float* out, void* stream) {
  if (!S) return SDM_ERR_NULL;
  if (B < 1 || H < 1 || T < 0 || d_k < 1 || d_v < 1) return SDM_ERR_SHAPE;
  if (T > 0 && (!k || !q || !v || !alpha || !beta || !out)) return SDM_ERR_NULL;
  if (!valid_dtype(dtype)) return SDM_ERR_DTYPE;
  if (d_k != 128 || d_v != 128) return SDM_ERR_UNSUPPORTED;
  if (!aligned16(S) || !aligned16(k) || !aligned16(q) || !aligned16(v) || !aligned16(out))
    return SDM_ERR_ALIGN;
  if (T == 0) return SDM_OK;
  sdm::GdnArgs a{};
  a.S = S;
  a.k = k;
  a.q = q;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.nS = B * H;
  a.T = T;
  a.d_k = d_k;
  a.d_v = d_v;
  hipError_t e = sdm::launch_gdn(a, dtype == SDM_BF16, (hipStream_t)stream);
  return e == hipSuccess ? SDM_OK : SDM_ERR_HIP;
}

const char* sdm_status_str(int s) {
  switch (s) {
    case SDM_OK: return "ok";
    case SDM_ERR_NULL: return "null pointer";
    case SDM_ERR_SHAPE: return "inconsistent sizes";
    case SDM_ERR_DTYPE: return "unknown element type";
    case SDM_ERR_UNSUPPORTED: return "outside the kernels' limits";
    case SDM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SDM_ERR_HIP: return "HIP launch failed";
    case SDM_ERR_WORKSPACE: return "workspace missing or too small";
    case SDM_ERR_SCRATCH: return "needs more than the library's static scratch";
    default: return "unknown status";
  }
}

const char* sdm_version(void) { return "0.1.0"; }

}  // extern "C"
