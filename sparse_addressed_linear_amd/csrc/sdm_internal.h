// Internal declarations shared by the libsdm translation units (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdm {

// Workgroups the scan aims to spread one launch over (one per CU of a
// 256-CU MI355X).
constexpr int kTargetWorkgroups = 256;

// Orders a wave's earlier LDS writes before its later LDS reads by other
// lanes of the same wave (code-motion barrier plus wavefront-scope fence).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// v from lane (lane ^ m) of the same wave, m a power of two below 64 known
// after unrolling.  Cross-lane moves without the LDS crossbar: DPP quad
// permutes (1, 2), row shifts (4), row rotate (8), the swizzle unit (16) and
// the gfx950 32-lane swap (32).
// (mov_dpp leaves lanes without a source undefined: the permutes and the
// rotate have none, and of the two shifts only lanes that have one are kept)
__device__ __forceinline__ uint32_t xor_shuffle(uint32_t v, int m, int lane) {
  switch (m) {
    case 1: return __builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    case 2: return __builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    case 4: {
      const uint32_t up = __builtin_amdgcn_mov_dpp((int)v, 0x104, 0xF, 0xF, false);  // row_shl:4
      const uint32_t dn = __builtin_amdgcn_mov_dpp((int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
      return (lane & 4) ? dn : up;
    }
    case 8: return __builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);    // xor 16 in 32
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return lane < 32 ? r[1] : r[0];
    }
  }
}

__device__ __forceinline__ float xor_shuffle(float v, int m, int lane) {
  return __uint_as_float(xor_shuffle(__float_as_uint(v), m, lane));
}

// 64-bit form: the DPP moves write both halves of the destination pair
// directly (no repacking moves).
__device__ __forceinline__ uint64_t xor_shuffle(uint64_t v, int m, int lane) {
  switch (m) {
    case 1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    case 4: {
      const uint64_t up = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, false);
      const uint64_t dn = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, false);
      return (lane & 4) ? dn : up;
    }
    case 8: return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
    default: {
      const uint32_t lo = xor_shuffle((uint32_t)v, m, lane);
      const uint32_t hi = xor_shuffle((uint32_t)(v >> 32), m, lane);
      return ((uint64_t)hi << 32) | lo;
    }
  }
}

struct ScanArgs {
  float* M;                // [S][N][d_v]
  const int32_t* widx;     // [S][T][W]
  const float* wwt;
  const int32_t* ridx;     // [S][T][R]
  const float* rwt;
  const void* v;           // [S][T][d_v]
  const float* alpha;      // [S][T]
  const float* beta;
  float* out;              // [S][T][d_v]
  float* work;             // [P][S][T][d_v] partial reads (P > 1)
  float* tape;             // [S][T][W][d_v] pre-write rows, or nullptr (not recorded)
  int64_t N;
  int32_t S, T, d_v, W, R;
  int32_t CS, P, hsize, lcap, xcd_map;
};

// Time-parallel form of the scan (events sorted by slot, then time).
struct TpArgs {
  float* M;                // [S][N][d_v] in/out
  const int32_t* widx;     // [S][T][W]
  const float* wwt;
  const int32_t* ridx;     // [S][T][R]
  const float* rwt;
  const void* v;           // [S][T][d_v]
  const float* alpha;      // [S][T]
  const float* beta;
  float* out;              // [S][T][d_v]
  int64_t N;
  int32_t S, T, d_v, W, R;
};

bool tp_sizes_ok(int S, int T, int W, int R);
size_t tp_workspace_bytes(int S, int T, int64_t N, int d_v, int W, int R);
hipError_t launch_scan_tp(const TpArgs& a, bool vbf16, void* ws, hipStream_t stream);

// Router of routed-slot writes (sigmoid top-K over M slot logits).
struct RouteArgs {
  const float* zk;         // [units][M] write-side logits
  const float* zq;         // [units][M] read-side logits
  const float* a;          // [units] decay (<= 0)
  int32_t* widx;           // [units][K]
  float* wcoef;            // [units][K] write strength 1 - exp(a*r)
  int32_t* ridx;           // [units][K]
  float* rwt;              // [units][K] read gates
  int64_t units;           // stream-tokens
  int32_t M, K;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t stream);
size_t route_lds_bytes(int M, int K);

// Adjoint of the addressing: weight gradients to dq', dk' and the sub-keys.
struct ScoreBwdArgs {
  const void* qp;          // [S][T][d_k]
  const void* kp;
  const void* subkeys;     // [H][2][n_sub][dh]
  const int32_t* widx;     // [S][T][W]
  const float* wwt;
  const int32_t* ridx;     // [S][T][R]
  const float* rwt;
  const float* dwwt;       // [S][T][W]
  const float* drwt;       // [S][T][R]
  float* dq;               // [S][T][d_k]
  float* dk;
  float* dsub;             // [H][2][n_sub][dh], accumulated (added to)
  int32_t S, H, T, d_k, n_sub, W, R;
};

// ws: score_bwd_workspace_bytes (records, their sorted copy, row bounds, sort scratch)
hipError_t launch_score_bwd(const ScoreBwdArgs& a, bool bf16, void* ws, hipStream_t stream);
size_t score_bwd_lds_bytes(int kmax);  // kmax = max(W, R)
int64_t score_bwd_records(int S, int T, int W, int R);
size_t score_bwd_workspace_bytes(int S, int T, int H, int n_sub, int W, int R);

// Reverse sweep of the scan (gradients).  Rows are whole (d_v = 4*LPR floats).
struct ScanBwdArgs {
  float* M;                // [S][N][d_v] in: table after the last token; out: M0
  float* dM;               // [S][N][d_v] in: dL/dM_T; out: dL/dM_0
  const int32_t* widx;     // [S][T][W]   forward's slots and weights
  const float* wwt;
  const int32_t* ridx;     // [S][T][R]
  const float* rwt;
  const void* v;           // [S][T][d_v]
  const float* alpha;      // [S][T]
  const float* beta;
  const float* tape;       // [S][T][W][d_v] pre-write rows from the forward
  const float* dout;       // [S][T][d_v]
  float* dv;               // [S][T][d_v]
  float* dalpha;           // [S][T]
  float* dbeta;
  float* dwwt;             // [S][T][W]
  float* drwt;             // [S][T][R]
  float* work;             // P > 1: [P][S][T][d_v] partial dv, then [P][S][T][2] dalpha, dbeta
  int64_t N;
  int32_t S, T, d_v, W, R;
  int32_t P, hsize, lcap, xcd_map;
};

struct ScanBwdPlan {
  int lpr;      // lanes per row (d_v / 4)
  int P;        // slot partitions
  int epl;      // events per lane group held in registers
  int hsize;    // LDS hash size (power of two)
  int lcap;     // per-wave event list capacity
  size_t lds;
  size_t work_bytes;
};

ScanBwdPlan plan_scan_bwd(int S, int T, int64_t N, int d_v, int W, int R);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, const ScanBwdPlan& p, bool vbf16,
                           hipStream_t stream);

struct ScanPlan {
  int lpr;      // lanes per row slice (slice = 4*lpr columns)
  int CS;       // column slices per stream
  int P;        // slot partitions
  int nw;       // waves per workgroup = tokens per block
  int epl;      // row slices per lane group held in registers
  int hsize;    // LDS hash size (power of two)
  int lcap;     // per-wave event list capacity
  size_t lds;   // dynamic LDS bytes
  size_t work_bytes;
};

ScanPlan plan_scan(int S, int T, int64_t N, int d_v, int W, int R, bool tape = false);
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& p, bool vbf16, hipStream_t stream);

struct ScoreArgs {
  const void* qp;          // [S][T][d_k]
  const void* kp;
  const void* subkeys;     // [H][2][n_sub][dh]
  void* packed;            // bf16: sub-key MFMA fragments (workspace)
  int32_t* widx;           // [S][T][W]
  float* wwt;
  int32_t* ridx;           // [S][T][R]
  float* rwt;
  int32_t S, H, T, d_k, n_sub, W, R;
  // fused decoding step (fuse != 0): token t of addressing stream st is scan
  // stream st*T + t with one token, table M + (st*T + t)*N*d_v
  float* M;
  const void* v;           // [S*T][d_v] (bf16 when v_bf16)
  const float* alpha;      // [S*T]
  const float* beta;
  float* out;              // [S*T][d_v]
  int64_t N;
  int32_t d_v, v_bf16, fuse;
};

// pack: repack the bf16 sub-keys into `packed` first (else it already holds them)
hipError_t launch_score_topk(const ScoreArgs& a, bool bf16, bool pack, hipStream_t stream);
hipError_t launch_pack_subkeys(const ScoreArgs& a, hipStream_t stream);
size_t score_topk_workspace_bytes(int H, int n_sub, int d_k, bool bf16);

struct GdnArgs {
  float* S;                // [S][d_v][d_k]
  const void* k;           // [S][T][d_k]
  const void* q;
  const void* v;           // [S][T][d_v]
  const float* alpha;
  const float* beta;
  float* out;              // [S][T][d_v]
  int32_t nS, T, d_k, d_v;
};

hipError_t launch_gdn(const GdnArgs& a, bool bf16, hipStream_t stream);

}  // namespace sdm
