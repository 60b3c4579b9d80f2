// Kernel templates of the product-key addressing (included by the score_topk*.hip units).
//
// Method ("Sparse Delta Memory", gist.science summaries of paper 2607.07386;
// Spanish page "Mecanismo Central" item 2, French page "Mecanisme Central"):
// the projected key (query) is cut into two halves; each half is scored
// against its own table of n_sub sub-keys (product-key memory); slot
// s = i*n_sub + j scores s1[i] + s2[j]; the top-W (top-R) slots are found
// through topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)) without forming the
// N = n_sub^2 scores.  Weights: softmax over the selected sums.  Order: score
// descending, ties to the lower index (sub-key index in stage 1, slot in
// stage 2).
//
// One workgroup of 8 waves handles kTT tokens of one (b,h) stream, keys and
// queries together: column c < kTT is the key of token t0 + c (write list),
// column kTT + c its query (read list).  Keys and queries are scored against
// the same sub-key tables, so the 2*kTT = 16 columns fill the N side of a
// 16x16 MFMA tile and each sub-key is read once per workgroup and half.
//   1. half scores: sub-keys x columns on v_mfma_f32_16x16x32_bf16 (bf16
//      inputs, fp32 accumulate) or on the VALU in the sequential order of a
//      scalar loop (fp32 inputs).  The scores stay in the accumulator
//      registers: lane (tl, kq) of wave w holds column tl's sub-keys
//      16*(w + 8*j) + 4*kq + r.
//   2. stage 1 per column: a threshold t with k <= #{key >= t} <= cap is found
//      by counting over all waves (first guess from the column's mean and
//      spread, then bisection on keys), the keys >= t are packed into the
//      column's LDS candidate buffer and one wave sorts them.
//   3. stage 2 per column: top-k of the outer sums over the pruned rank grid
//      {(a,b): (a+1)(b+1) <= k} -- a pair outside it is beaten by at least k
//      pairs of its dominating rectangle.  With ties in the fp32 sums that
//      argument can fail, so the best pair just outside the grid is checked
//      and, if it could compete, the full m x m grid is ranked.
// Keys are unique 64-bit values (order-preserving score bits, then the
// complemented index), so every selection is exact and bisection on keys
// always ends.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "scan_common.h"
#include "sdm_internal.h"

namespace sdm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTT = 8;          // tokens per workgroup
constexpr int kCols = 2 * kTT;  // key and query columns
constexpr int kWaves = 8;       // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kCapMax = 256;    // largest candidate set sorted at once
constexpr int kGridMax = 704;   // largest pruned grid held in registers (11 per lane)

// K steps of 32 per sub-key row in the packed fragments: the MFMA template
// count for dh (1, 2, 4 or 8; rows are zero-padded to it)
__host__ __device__ inline int score_ksteps(int dh) {
  return dh <= 32 ? 1 : dh <= 64 ? 2 : dh <= 128 ? 4 : 8;
}

// candidates kept for a top-k: between k and this many
__host__ __device__ inline int cap_for(int k) {
  const int c = 2 * k > 64 ? 2 * k : 64;
  return c < kCapMax ? c : kCapMax;
}

// order-preserving code of a finite float: sign bit flipped for s >= 0, all
// bits flipped for s < 0; adding +0 first turns -0 into +0, so both zeros
// rank equal
__device__ __forceinline__ uint32_t ord32(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// larger key = ranks ahead: higher score, then lower index
__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)ord32(s) << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ float key_score(uint64_t k) { return unord32((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xffffffffu - (uint32_t)k; }

// stage-1 list entry: score bits in the low word, sub-key id in the high word
__device__ __forceinline__ uint64_t list_entry(uint64_t key) {
  return ((uint64_t)key_id(key) << 32) | __float_as_uint(key_score(key));
}
__device__ __forceinline__ float entry_score(uint64_t e) { return __uint_as_float((uint32_t)e); }
__device__ __forceinline__ uint32_t entry_id(uint64_t e) { return (uint32_t)(e >> 32); }

// sum over e ascending of x[e]*c[e], each product and sum rounded in fp32
__device__ __forceinline__ float dot_seq(const float* x, const float* c, int n) {
#pragma clang fp contract(off)
  float acc = 0.f;
  for (int e = 0; e < n; e++) {
    const float p = x[e] * c[e];
    acc = acc + p;
  }
  return acc;
}

__device__ __forceinline__ float wave_sum(float x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += xor_shuffle(x, o, lane);
  return x;
}
__device__ __forceinline__ uint32_t wave_max32(uint32_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, xor_shuffle(x, o, lane));
  return x;
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = xor_shuffle(x, o, lane);
    x = y > x ? y : x;
  }
  return x;
}

template <int NPL>
__device__ __forceinline__ int count_ge(const uint64_t (&key)[NPL], uint64_t t) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < NPL; j++) c += __popcll(__ballot(key[j] >= t));
  return c;
}

// Threshold t with k <= #{key >= t} <= cap.  Requires #{key >= lo} >= k and
// #{key >= hi} < k.  Keys are unique, so bisection ends with #{key >= t} == k
// at the latest.
template <int NPL>
__device__ uint64_t find_threshold(const uint64_t (&key)[NPL], int k, int cap, uint64_t guess,
                                   uint64_t lo, uint64_t hi) {
  uint64_t t = (guess > lo && guess < hi) ? guess : lo + (hi - lo) / 2;
  for (int it = 0; it < 96; it++) {
    const int c = count_ge(key, t);
    if (c >= k && c <= cap) return t;
    if (c < k) hi = t;
    else lo = t;
    if (hi - lo <= 1) return lo;
    t = lo + (hi - lo) / 2;
  }
  return lo;
}

// Ascending-index bitonic network over 64*E keys held E per lane (element
// i = lane*E + r), sorting into DESCENDING order.  Stage S, step J are template
// parameters, so each step's lane pattern (which lanes keep the larger key of
// an exchange) is a compile-time 64-bit constant that becomes the select
// condition directly (inverse ballot): no per-lane arithmetic, and nothing
// for the register allocator to keep live (or spill) across the network.
constexpr uint64_t keep_max_lanes(int E, int J, int S) {
  // lanes whose element keeps the larger key of a cross-lane exchange: the
  // lower slot of a descending run or the upper slot of an ascending one
  // (J, S >= E, so the register index r does not change either bit)
  uint64_t m = 0;
  for (int l = 0; l < 64; l++) {
    const int i = l * E;
    if (((i & J) == 0) == ((i & S) == 0)) m |= 1ull << l;
  }
  return m;
}

constexpr uint64_t desc_lanes(int E, int r, int S) {  // element lane*E + r in a descending run
  uint64_t m = 0;
  for (int l = 0; l < 64; l++)
    if (((l * E + r) & S) == 0) m |= 1ull << l;
  return m;
}

template <typename K, int E, int S, int J>
__device__ __forceinline__ void bitonic_step(K (&v)[E], int lane) {
  if constexpr (J >= E) {
    constexpr uint64_t km_bits = keep_max_lanes(E, J, S);
    const bool km = __builtin_amdgcn_inverse_ballot_w64(km_bits);
#pragma unroll
    for (int r = 0; r < E; r++) {
      const K o = xor_shuffle(v[r], J / E, lane);
      // equal keys are equal values, so one compare decides
      v[r] = ((o > v[r]) == km) ? o : v[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; r++) {
      if ((r & J) == 0) {
        const bool desc = __builtin_amdgcn_inverse_ballot_w64(desc_lanes(E, r, S));
        const K p = v[r], q = v[r | J];
        const bool swap = (q > p) == desc;  // equal keys: swapping changes nothing
        v[r] = swap ? q : p;
        v[r | J] = swap ? p : q;
      }
    }
  }
  if constexpr (J > 1) bitonic_step<K, E, S, J / 2>(v, lane);
}

template <typename K, int E, int S>
__device__ __forceinline__ void bitonic_stage(K (&v)[E], int lane) {
  bitonic_step<K, E, S, S / 2>(v, lane);
  if constexpr (S < 64 * E) bitonic_stage<K, E, S * 2>(v, lane);
}

template <int E>
__device__ __forceinline__ void bitonic_desc(uint64_t (&v)[E], int lane) {
  bitonic_stage<uint64_t, E, 2>(v, lane);
}

// Sort the c (<= kCapMax) keys in buf descending; lanes then write the first k
// through `emit(rank, key)`.
template <int E, typename Emit>
__device__ __forceinline__ void sort_emit_e(uint64_t* buf, int c, int k, int lane, Emit emit) {
  uint64_t v[E];
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    v[r] = i < c ? buf[i] : 0ull;
  }
  bitonic_desc<E>(v, lane);
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    if (i < k) emit(i, v[r]);
  }
}

template <typename Emit>
__device__ __forceinline__ void sort_emit(uint64_t* buf, int c, int k, int lane, Emit emit) {
  if (c <= 64) sort_emit_e<1>(buf, c, k, lane, emit);
  else if (c <= 128) sort_emit_e<2>(buf, c, k, lane, emit);
  else sort_emit_e<4>(buf, c, k, lane, emit);
}

// The same network on 32-bit keys.
template <int E>
__device__ __forceinline__ void bitonic_desc32(uint32_t (&v)[E], int lane) {
  bitonic_stage<uint32_t, E, 2>(v, lane);
}

__device__ __forceinline__ int bitlen32(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

// Sorted order of the c (<= 64*E) keys in buf, all with score part in
// [obase, omax], into v (position p = lane*E + r, descending).  Fast path: a
// 32-bit network on compressed keys -- score part minus obase, shifted right
// just enough to fit 32 - IB bits, then IB bits of the key's position in buf --
// after which the full keys are gathered by position.  Compressed scores are
// monotone in the true ones, so the order is exact unless two neighbours share
// a compressed score; then the full 64-bit keys are sorted instead (fp32 ties,
// or scores a few ulps apart when the range needs a shift).
template <int E>
__device__ __forceinline__ void sort_keys(const uint64_t* buf, int c, int lane, uint32_t obase,
                                          uint32_t omax, uint64_t (&v)[E]) {
  constexpr int IB = E <= 2 ? 7 : 8;  // position bits (c <= 2^IB)
  constexpr uint32_t PM = (1u << IB) - 1u;
  const int sh = max(0, bitlen32(omax - obase) - (32 - IB));
  uint32_t w[E];
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int i = lane * E + r;
    w[r] = 0u;  // padding sorts last: a real key has position bits PM - i >= 1 or score bits
    if (i < c) {
      const uint32_t o = (uint32_t)(buf[i] >> 32);
      w[r] = (((o - obase) >> sh) << IB) | (PM - (uint32_t)i);
    }
  }
  bitonic_desc32<E>(w, lane);
  bool tie = false;
#pragma unroll
  for (int r = 0; r + 1 < E; r++) tie |= lane * E + r + 1 < c && (w[r] >> IB) == (w[r + 1] >> IB);
  const uint32_t nx = (uint32_t)__shfl_down((int)w[0], 1);  // lane + 1's first
  tie |= lane < 63 && lane * E + E < c && (w[E - 1] >> IB) == (nx >> IB);
  if (__ballot(tie) == 0ull) {
#pragma unroll
    for (int r = 0; r < E; r++) v[r] = lane * E + r < c ? buf[PM - (w[r] & PM)] : 0ull;
  } else {
#pragma unroll
    for (int r = 0; r < E; r++) {
      const int i = lane * E + r;
      v[r] = i < c ? buf[i] : 0ull;
    }
    bitonic_desc<E>(v, lane);
  }
}

// sort_emit for keys with score part in [obase, omax] (see sort_keys); buf may
// be overwritten by emit (every key is read before the first write).
template <typename Emit>
__device__ __forceinline__ void sort_emit_range(uint64_t* buf, int c, int k, int lane,
                                                uint32_t obase, uint32_t omax, Emit emit) {
  auto run = [&](auto tag) {
    constexpr int E = decltype(tag)::value;
    uint64_t v[E];
    sort_keys<E>(buf, c, lane, obase, omax, v);
#pragma unroll
    for (int r = 0; r < E; r++) {
      const int i = lane * E + r;
      if (i < k) emit(i, v[r]);
    }
  };
  if (c <= 64) run(std::integral_constant<int, 1>{});
  else if (c <= 128) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 4>{});
}

// Compact keys >= t into buf (ballot order); returns the count.
template <int NPL>
__device__ __forceinline__ int compact_ge(const uint64_t (&key)[NPL], uint64_t t, uint64_t* buf,
                                          int lane) {
  int base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < NPL; j++) {
    const bool f = key[j] >= t;
    const uint64_t m = __ballot(f);
    if (f) buf[base + __popcll(m & below)] = key[j];
    base += __popcll(m);
  }
  return base;
}

}  // namespace

// Shared-memory layout (bytes) for W write and R read slots.  Column c owns
// a block of 2*capmax keys: stage-1 candidates of half h at [h*capmax, ...),
// then, once sorted, the two rank-ordered lists at [0, m) and [m, 2m) and
// stage 2's scratch at [2m, 2m + capmax) (capmax >= 2m).
struct ScoreSmem {
  size_t cand, grid, rowoff, dump, total;
  int m, capmax, gW, gR;  // list length, candidate stride, grid sizes
};

// size of the pruned rank grid {(a,b) : (a+1)(b+1) <= k} over k x k ranks
__host__ __device__ inline int pruned_grid_size(int k) {
  int g = 0;
  for (int a = 0; a < k; a++) g += (k / (a + 1) < k ? k / (a + 1) : k);
  return g;
}

__host__ __device__ inline ScoreSmem score_smem(int W, int R) {
  ScoreSmem s;
  s.m = W > R ? W : R;
  s.capmax = cap_for(s.m);
  s.gW = pruned_grid_size(W);
  s.gR = W == R ? 0 : pruned_grid_size(R);
  size_t o = 0;
  s.cand = o;   o += (size_t)kCols * 2 * s.capmax * 8;
  s.grid = o;   o += (size_t)(s.gW + s.gR) * 4;  // (ra << 16) | rb, W grid then R grid
  s.rowoff = o; o += (size_t)2 * (s.m + 1) * 4;
  o = (o + 15) & ~(size_t)15;
  s.dump = o;   o += (size_t)kWaves * 64 * 8;  // one slot per lane for discarded stores
  s.total = o;
  return s;
}

namespace {

// Half scores of the 16 columns against this wave's sub-key tiles
// i0 = 16*(wave + 8*j), j < NT: D[sub-key][column] = sum_e C[sub-key][e] *
// x[column][e] on v_mfma_f32_16x16x32_bf16.  The A fragments come from the
// packed copy of this head-half's sub-keys ([tile][K step][lane] x 16 bytes,
// dh padded with zeros to a multiple of 32), so each load instruction reads
// 1 KB contiguous; tiles past n_sub fall outside the buffer resource and read
// as zero (n_sub is a multiple of 16, so such tiles are wholly outside and
// their scores are discarded by the caller).  There is no branch, and each
// batch's loads are all in flight before its first MFMA.  xcol points at this
// lane's column half (any valid row when !col_ok).
template <int NT, int KS, int TBMAX>
__device__ __forceinline__ void mfma_scores(const uint16_t* xcol, bool col_ok,
                                            const unsigned char* Pb, int n_tiles, int dh,
                                            int wave, int lane, float (&sc)[NT][4]) {
  // sub-key tiles loaded together (up to 16 loads, at most TBMAX tiles)
  constexpr int TB0 = 16 / KS < NT ? 16 / KS : NT;
  constexpr int TB = TB0 < TBMAX ? TB0 : TBMAX;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int kq = lane >> 4;  // which 8-wide K chunk of the 32
  bf16x8 bfrag[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    const int d0 = ks * 32 + kq * 8;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(xcol + min(d0, dh - 8));
    bfrag[ks] = (col_ok && d0 < dh) ? v : bf16x8{};
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Pb, (short)0, n_tiles * KS * 1024, 0x00020000);
  const int voff = (wave * KS * 64 + lane) * 16;  // tile j = 0, K step 0
  constexpr int tstep = kWaves * KS * 1024;       // bytes from tile j to j + 1
#pragma unroll
  for (int j0 = 0; j0 < NT; j0 += TB) {
    u32x4 af[TB][KS];
#pragma unroll
    for (int t = 0; t < TB; t++)
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        if (j0 + t < NT)
          af[t][ks] =
              __builtin_amdgcn_raw_buffer_load_b128(rs, voff + (j0 + t) * tstep + ks * 1024, 0, 0);
#pragma unroll
    for (int t = 0; t < TB; t++) {
      if (j0 + t < NT) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[t][ks]),
                                                        bfrag[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; r++) sc[j0 + t][r] = acc[r];
      }
    }
  }
}

// fp32 inputs: the same layout, each score a sequential dot product.
template <int NT>
__device__ __forceinline__ void valu_scores(const float* xcol, const float* Cf, int n_sub, int dh,
                                            int wave, int lane, float (&sc)[NT][4]) {
  const int kq = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; j++) {
    const int i0 = 16 * (wave + kWaves * j);
#pragma unroll
    for (int r = 0; r < 4; r++)
      sc[j][r] = i0 < n_sub ? dot_seq(xcol, Cf + (int64_t)(i0 + 4 * kq + r) * dh, dh) : 0.f;
  }
}

// #{own keys >= t}; o == 0 marks an empty position.  base_id is the sub-key
// id of (j = 0, r = 0); position (j, r) holds id base_id + 128*j + r.
template <int NT>
__device__ __forceinline__ int count_own(const uint32_t (&o)[NT][4], uint32_t base_id,
                                         uint64_t t) {
  int c = 0;
  const uint32_t th = (uint32_t)(t >> 32);
  if ((uint32_t)t == 0u) {
    // keys >= (th, 0) exactly when the score part is >= th
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) c += o[j][r] >= th ? 1 : 0;
  } else {
    // (o, ~id) >= (th, tlo) with 32-bit compares; o == 0 never reaches th
    const uint32_t tlo = (uint32_t)t;
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint32_t lid = 0xffffffffu - (base_id + kWaves * 16 * j + r);
        c += (o[j][r] > th || (o[j][r] == th && lid >= tlo)) ? 1 : 0;
      }
  }
  return c;
}

// Sorted positions p = lane*E + r < k of stage 2: slot ids and softmax
// weights straight from the registers of the sort.
template <int E>
__device__ __forceinline__ void emit_slots(const uint64_t (&v)[E], int k, int lane,
                                           int32_t* dst_i, float* dst_w) {
  const uint32_t top_hi = __builtin_amdgcn_readfirstlane((uint32_t)(v[0] >> 32));
  const float top = unord32(top_hi);
  float e[E];
  float z = 0.f;
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int p = lane * E + r;
    e[r] = p < k ? __expf(key_score(v[r]) - top) : 0.f;
    z += e[r];
  }
  const float iz = __builtin_amdgcn_rcpf(wave_sum(z));
#pragma unroll
  for (int r = 0; r < E; r++) {
    const int p = lane * E + r;
    if (p < k) {
      dst_i[p] = (int32_t)key_id(v[r]);
      dst_w[p] = e[r] * iz;
    }
  }
}

// Stage 2 tail once the c candidates in buf are known: sort them in
// registers, check the frontier outside the pruned grid, write the result.
// Returns false when the frontier could compete (the caller then ranks the
// full grid).
template <int E, bool TIEK>
__device__ __forceinline__ bool stage2_sorted(const uint64_t* buf, int c, uint32_t obase,
                                              uint32_t omax, const uint64_t* L1,
                                              const uint64_t* L2, const int32_t* rowoff, int m,
                                              int k, const uint64_t* lk, int lane,
                                              int32_t* dst_i, float* dst_w) {
  uint64_t v[E];
  sort_keys<E>(buf, c, lane, obase, omax, v);
  // k-th best key: position k-1 = lane (k-1)/E, register (k-1)%E
  uint64_t kv = v[0];
#pragma unroll
  for (int r = 1; r < E; r++) kv = ((k - 1) % E == r) ? v[r] : kv;
  const int src = (k - 1) / E;
  const uint32_t klo = __shfl((uint32_t)kv, src), khi = __shfl((uint32_t)(kv >> 32), src);
  const float kth_score = unord32(khi);
  (void)klo;
  // best pair just outside the pruned grid within the first k ranks, row by
  // row: exact if it cannot outrank the k-th (compare scores: a score tie
  // with a lower slot would)
  float fr = -INFINITY;
  bool any = false;
  for (int ra = lane; ra < k; ra += 64) {
    const int rb = rowoff[ra + 1] - rowoff[ra];  // row ra of the grid: ranks 0 .. rb-1
    if (rb < k) {
      const float s = entry_score(L1[ra]) + entry_score(L2[rb]);
      fr = any ? fmaxf(fr, s) : s;
      any = true;
    }
  }
  // the pairs holding a list's rank-k entry (lk[0] of L1, lk[1] of L2;
  // present when m > k) lie outside the k x k grid: (0, k) and (k, 0) bound
  // them all, as a sum never grows with either rank
  bool edge = false;
  if constexpr (TIEK) {
    if (m > k) {
      const float f1 = entry_score(L1[0]) + entry_score(lk[1]);
      const float f2 = entry_score(lk[0]) + entry_score(L2[0]);
      edge = !(f1 < kth_score) || !(f2 < kth_score);
    }
  }
  const bool compete = edge || __ballot(any && !(fr < kth_score)) != 0ull;
  if (compete) return false;
  emit_slots<E>(v, k, lane, dst_i, dst_w);
  return true;
}

// Stage 2 for one column whose stage-1 lists (rank order, list_entry form)
// are L1, L2 (ranks 0 .. k-1) and lk[0], lk[1] (rank k): the k best slots over the
// pruned grid (row offsets rowoff), written in rank order with their softmax
// weights.  The selection is defined on the m x m grid of the stage-1 lists
// (m = k+1, or n_sub when that is smaller); a pair outside the pruned grid
// can only enter it through an fp32 tie, and then the full m x m grid is
// ranked.  buf holds cap_for(k) keys of scratch.
template <int NPL2, bool TIEK>
__device__ __forceinline__ void stage2(const uint64_t* L1, const uint64_t* L2, const uint64_t* lk,
                                       int m, int k, int n_sub,
                                       const uint32_t* grid, const int32_t* rowoff, int G,
                                       float z, uint64_t* buf, int lane, int32_t* dst_i,
                                       float* dst_w) {
  uint64_t key[NPL2];
  float sum = 0.f, sq = 0.f;
  uint32_t mo = 0u;  // largest score code
#pragma unroll
  for (int j = 0; j < NPL2; j++) {
    const int c = j * 64 + lane;
    key[j] = 0ull;
    if (c < G) {
      const uint32_t ab = grid[c];
      const uint64_t a1 = L1[ab >> 16], a2 = L2[ab & 0xffff];
      const float s = entry_score(a1) + entry_score(a2);
      const uint32_t o = ord32(s);
      key[j] = ((uint64_t)o << 32) | (0xffffffffu - (entry_id(a1) * (uint32_t)n_sub + entry_id(a2)));
      mo = max(mo, o);
      sum += s;
      sq += s * s;
    }
  }
  const int cap = cap_for(k);
  mo = wave_max32(mo);
  // first threshold from the mean and spread of the G sums
  sum = wave_sum(sum);
  sq = wave_sum(sq);
  const float mean = sum / G;
  const float sd = sqrtf(fmaxf(sq / G - mean * mean, 0.f));
  const uint64_t guess = (uint64_t)ord32(mean + z * sd) << 32;
  const uint64_t t = find_threshold(key, k, cap, guess, 0ull, ((uint64_t)mo + 1ull) << 32);
  const int c = compact_ge(key, t, buf, lane);
  wave_lds_sync();
  bool done;
  const uint32_t ob = (uint32_t)(t >> 32);
  if (c <= 64)
    done = stage2_sorted<1, TIEK>(buf, c, ob, mo, L1, L2, rowoff, m, k, lk, lane, dst_i, dst_w);
  else if (c <= 128)
    done = stage2_sorted<2, TIEK>(buf, c, ob, mo, L1, L2, rowoff, m, k, lk, lane, dst_i, dst_w);
  else
    done = stage2_sorted<4, TIEK>(buf, c, ob, mo, L1, L2, rowoff, m, k, lk, lane, dst_i, dst_w);
  if (done) return;

  // rare: rank the full m x m grid.  The k-th key of the pruned grid is a
  // lower bound; bisect upward until at most cap keys remain.
  wave_lds_sync();
  auto full_key = [&](int q) {
    const int qa = q / m, qb = q % m;
    uint64_t a1, a2;
    if constexpr (TIEK) {
      a1 = qa < k ? L1[qa] : lk[0];
      a2 = qb < k ? L2[qb] : lk[1];
    } else {
      a1 = L1[qa];
      a2 = L2[qb];
    }
    return make_key(entry_score(a1) + entry_score(a2), entry_id(a1) * (uint32_t)n_sub + entry_id(a2));
  };
  auto cnt = [&](uint64_t tt) {
    int n = 0;
    for (int base = 0; base < m * m; base += 64) {
      const int q = base + lane;
      n += __popcll(__ballot(q < m * m && full_key(q) >= tt));
    }
    return n;
  };
  uint64_t lo = 0ull, hi = ~0ull, tt = t;
  for (int it = 0; it < 96; it++) {
    const int n = cnt(tt);
    if (n >= k && n <= cap) break;
    if (n < k) hi = tt;
    else lo = tt;
    if (hi - lo <= 1) {
      tt = lo;
      break;
    }
    tt = lo + (hi - lo) / 2;
  }
  int base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int b0 = 0; b0 < m * m; b0 += 64) {
    const int q = b0 + lane;
    const uint64_t kk = q < m * m ? full_key(q) : 0ull;
    const bool f = q < m * m && kk >= tt;
    const uint64_t msk = __ballot(f);
    if (f) buf[base + __popcll(msk & below)] = kk;
    base += __popcll(msk);
  }
  wave_lds_sync();
  sort_emit(buf, base, k, lane, [&](int r, uint64_t kk) { buf[r] = kk; });
  wave_lds_sync();
  const float top = key_score(buf[0]);
  float zs = 0.f;
  for (int r = lane; r < k; r += 64) zs += __expf(key_score(buf[r]) - top);
  const float iz = __builtin_amdgcn_rcpf(wave_sum(zs));
  for (int r = lane; r < k; r += 64) {
    const uint64_t kk = buf[r];
    dst_i[r] = (int32_t)key_id(kk);
    dst_w[r] = __expf(key_score(kk) - top) * iz;
  }
}

// Row offsets of the pruned grid for k (k <= 128 rows, two per lane) by a
// prefix sum over one wave.
__device__ __forceinline__ void grid_rowoff(int k, int32_t* rowoff, int lane) {
  const int len0 = lane < k ? min(k, k / (lane + 1)) : 0;
  const int len1 = lane + 64 < k ? min(k, k / (lane + 65)) : 0;
  int s0 = len0, s1 = len1;
  for (int o = 1; o < 64; o <<= 1) {
    const int y0 = __shfl_up(s0, o), y1 = __shfl_up(s1, o);
    if (lane >= o) s0 += y0, s1 += y1;
  }
  // both totals are read with every lane active (a lane shuffle from a lane
  // that is switched off does not return that lane's value)
  const int tot0 = __shfl(s0, 63);
  const int tot1 = __shfl(s1, 63);
  if (lane < k) rowoff[lane] = s0 - len0;
  if (lane + 64 < k) rowoff[lane + 64] = tot0 + s1 - len1;
  if (lane == 0) rowoff[k] = tot0 + tot1;
}

__device__ __forceinline__ void grid_fill(int k, const int32_t* rowoff, uint32_t* grid, int wave,
                                          int lane) {
  for (int ra = wave; ra < k; ra += kWaves) {
    const int off = rowoff[ra], len = rowoff[ra + 1] - off;
    for (int rb = lane; rb < len; rb += 64) grid[off + rb] = ((uint32_t)ra << 16) | rb;
  }
}

// First-guess quantiles: a Gaussian model puts about 1.4k of the n stage-1
// scores (of the G stage-2 sums) above mean + z * sd.
struct ScoreZ {
  float w1, r1, w2, r2;
};

// TT: tokens per tile, 8 (every column used, each wave owns the key and query
// columns of one token) or 4 for launches too small to fill the GPU (columns
// of tokens 4..7 stay empty, and each wave owns one column: waves 0-3 the keys,
// 4-7 the queries), which halves each wave's share of the serial per-column
// work (sorts, stage 2) and so the latency of a tile.
// Waves per SIMD the kernel is compiled for.  With 8-token tiles and grids
// of at most 5 keys a lane (k <= 71) a workgroup needs at most 46 KB of LDS
// (40 KB at k = 64), so three fit on a CU if registers allow: the kernel is held to 80 VGPRs
// (6 waves a SIMD; the stage-1 score codes then partly spill to scratch) and
// loads its sub-key fragments two tiles at a time.  The extra workgroup covers
// more of the dependent latency of the sorts and stage 2 than the spills cost.
// Larger grids need more LDS (two workgroups a CU either way) and decoding
// launches use too few workgroups for occupancy to matter: there 128 VGPRs.
// The fused decoding step's gated delta write of one element, as the scan's:
// c = beta*w, then (1-c)*(alpha*m) + c*v, every product and the sum rounded
// separately (no contraction), so tables match the scan's bit for bit.
__device__ __forceinline__ void dec_gate(float beta, float w, float& c, float& omc) {
#pragma clang fp contract(off)
  c = beta * w;
  omc = 1.0f - c;
}

__device__ __forceinline__ float dec_upd(float m, float al, float omc, float c, float v) {
#pragma clang fp contract(off)
  const float mt = al * m;
  const float keep = omc * mt;
  const float put = c * v;
  return keep + put;
}

template <int NPL2, int TT>
constexpr bool score_high_occ() {
  return TT == kTT && NPL2 <= 5;
}

template <bool BF16, int NT, int NPL2, int TT, bool FUSE>
__global__ void __launch_bounds__(kThreads, (score_high_occ<NPL2, TT>() ? 6 : 4))
    sdm_score_topk_kernel(ScoreArgs a, int tiles_per_wg, ScoreZ z) {
  static_assert(TT == kTT || TT == kTT / 2, "tile of 8 or 4 tokens");
  constexpr int NCW = TT == kTT ? 2 : 1;  // columns each wave owns
  // the o-th column owned by wave w
  auto owned = [](int w, int o) { return TT == kTT ? w + o * kTT : (w & 3) + (w >> 2) * kTT; };
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float2 s_stat[kWaves][kCols];    // per wave: sum, sum of squares
  __shared__ uint32_t s_max[kWaves][kCols];   // per wave: largest score part
  __shared__ int s_cnt[2][kWaves][kCols];     // per wave: #{keys >= t}, two rounds
  __shared__ uint32_t s_range[2][kCols];      // per column: score part of t, largest score part
  __shared__ uint64_t s_last[kCols][2];       // per column and half: the rank-k list entry
  const ScoreSmem L = score_smem(a.W, a.R);
  const int m = L.m, cm = L.capmax;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L.cand);
  uint32_t* grid = reinterpret_cast<uint32_t*>(smem + L.grid);
  int32_t* rowoff = reinterpret_cast<int32_t*>(smem + L.rowoff);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int st = blockIdx.y;
  const int h = st % a.H;

  // pruned rank grids (R's only when R != W), built once per workgroup; the
  // row fill is ordered before stage 2 by the barriers of stage 1
  if (wave == 0) {
    grid_rowoff(a.W, rowoff, lane);
    if (L.gR) grid_rowoff(a.R, rowoff + (m + 1), lane);
  }
  __syncthreads();
  grid_fill(a.W, rowoff, grid, wave, lane);
  if (L.gR) grid_fill(a.R, rowoff + (m + 1), grid + L.gW, wave, lane);

  const int ntiles = (a.T + TT - 1) / TT;
  const int tile_end = min(ntiles, (int)(blockIdx.x + 1) * tiles_per_wg);
  for (int tile = blockIdx.x * tiles_per_wg; tile < tile_end; tile++) {
    const int t0 = tile * TT;
    for (int half = 0; half < 2; half++) {
      // Everything below is derived afresh from these in each half: values
      // kept live across halves would not fit in the register budget.
      int n_sub = a.n_sub, dh = a.d_k / 2, hw = wave, hl = lane;
      asm volatile("" : "+s"(n_sub), "+s"(dh), "+s"(hw), "+v"(hl));
      const int tl = hl & 15;  // this lane's column
      const int kq = hl >> 4;
      const bool is_q = tl >= kTT;
      const int tok = t0 + (tl & (kTT - 1));
      const bool col_ok = (tl & (kTT - 1)) < TT && tok < a.T;
      // fp32: stage 1 keeps k+1 entries (at most n_sub), the rank-k one to
      // bound the pairs just outside stage 2's grid when fp32 sums tie
      const int kc0 = is_q ? a.R : a.W;
      const int capc = cap_for(kc0);
      const int kc = (!BF16 && kc0 < n_sub) ? kc0 + 1 : kc0;
      const float zc = is_q ? z.r1 : z.w1;
      const uint32_t base_id = 16u * hw + 4u * kq;  // sub-key id of this lane's first score

      // ---- 1. half scores ---------------------------------------------------
      float sc[NT][4];
      if (BF16) {
        const uint16_t* xcol = static_cast<const uint16_t*>(is_q ? a.qp : a.kp) +
                               ((int64_t)st * a.T + (col_ok ? tok : 0)) * a.d_k + half * dh;
        const int n_tiles = n_sub / 16;
        const int ksteps = score_ksteps(dh);
        const unsigned char* Pb = static_cast<const unsigned char*>(a.packed) +
                                  ((int64_t)h * 2 + half) * n_tiles * ksteps * 1024;
        constexpr int TBM = score_high_occ<NPL2, TT>() ? 2 : 16;
        if (dh <= 32) mfma_scores<NT, 1, TBM>(xcol, col_ok, Pb, n_tiles, dh, hw, hl, sc);
        else if (dh <= 64) mfma_scores<NT, 2, TBM>(xcol, col_ok, Pb, n_tiles, dh, hw, hl, sc);
        else if (dh <= 128) mfma_scores<NT, 4, TBM>(xcol, col_ok, Pb, n_tiles, dh, hw, hl, sc);
        else mfma_scores<NT, 8, TBM>(xcol, col_ok, Pb, n_tiles, dh, hw, hl, sc);
      } else {
        const float* xcol = static_cast<const float*>(is_q ? a.qp : a.kp) +
                            ((int64_t)st * a.T + (col_ok ? tok : 0)) * a.d_k + half * dh;
        const float* Cf =
            static_cast<const float*>(a.subkeys) + ((int64_t)h * 2 + half) * n_sub * dh;
        valu_scores<NT>(xcol, Cf, n_sub, dh, hw, hl, sc);
      }

      // ---- 2. stage 1: threshold over all waves, pack, sort -----------------
      uint32_t o[NT][4];
      float sum = 0.f, sq = 0.f;
      uint32_t omax = 0u;
#pragma unroll
      for (int j = 0; j < NT; j++) {
        const bool valid = 16 * (hw + kWaves * j) < n_sub;  // whole tiles
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float s = sc[j][r];
          o[j][r] = valid ? ord32(s) : 0u;
          sum += valid ? s : 0.f;
          sq += valid ? s * s : 0.f;
          omax = o[j][r] > omax ? o[j][r] : omax;
        }
      }
      sum += xor_shuffle(sum, 16, hl);
      sq += xor_shuffle(sq, 16, hl);
      omax = max(omax, xor_shuffle(omax, 16, hl));
      sum += xor_shuffle(sum, 32, hl);
      sq += xor_shuffle(sq, 32, hl);
      omax = max(omax, xor_shuffle(omax, 32, hl));
      if (kq == 0) {
        s_stat[hw][tl] = make_float2(sum, sq);
        s_max[hw][tl] = omax;
      }
      __syncthreads();
      sum = 0.f, sq = 0.f, omax = 0u;
#pragma unroll
      for (int w = 0; w < kWaves; w++) {
        const float2 v = s_stat[w][tl];
        sum += v.x;
        sq += v.y;
        omax = max(omax, s_max[w][tl]);
      }
      const float mean = sum / n_sub;
      const float sd = sqrtf(fmaxf(sq / n_sub - mean * mean, 0.f));
      uint64_t lo = 0ull, hi = ((uint64_t)omax + 1ull) << 32;
      const uint64_t guess = (uint64_t)ord32(mean + zc * sd) << 32;
      uint64_t t = (guess > lo && guess < hi) ? guess : lo + (hi - lo) / 2;
      int it = 0, own = 0;
      for (;;) {
        // keys are rebuilt from o in every round, not kept live across rounds
#pragma unroll
        for (int j = 0; j < NT; j++)
#pragma unroll
          for (int r = 0; r < 4; r++) asm volatile("" : "+v"(o[j][r]));
        own = count_own<NT>(o, base_id, t);
        int ws = own + (int)xor_shuffle((uint32_t)own, 16, hl);
        ws += (int)xor_shuffle((uint32_t)ws, 32, hl);
        if (kq == 0) s_cnt[it & 1][hw][tl] = ws;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; w++) tot += s_cnt[it & 1][w][tl];
        const bool ok = !col_ok || (tot >= kc && tot <= capc);
        if (__ballot(!ok) == 0ull || it >= 127) break;  // same decision in every wave
        if (!ok) {
          if (tot < kc) hi = t;
          else lo = t;
          t = hi - lo <= 1 ? lo : lo + (hi - lo) / 2;
        }
        it++;
      }
      const int fin = it & 1;
      if (hw == 0 && kq == 0) s_range[0][tl] = (uint32_t)(t >> 32), s_range[1][tl] = omax;
      // pack this lane's keys >= t behind those of earlier waves and lanes
      int pos = 0;
      for (int w = 0; w < hw; w++) pos += s_cnt[fin][w][tl];
      {
        const int x16 = (int)xor_shuffle((uint32_t)own, 16, hl);  // kq ^ 1
        const int x32 = (int)xor_shuffle((uint32_t)own, 32, hl);  // kq ^ 2
        const int x48 = (int)xor_shuffle((uint32_t)x16, 32, hl);  // kq ^ 3
        pos += kq == 0 ? 0 : kq == 1 ? x16 : kq == 2 ? x32 + x48 : x16 + x32 + x48;
      }
      {
        // every position stores: kept keys to the column's block, the others
        // to this lane's own discard slot (no branches, no exec-mask churn)
        uint64_t* cb = cand + (tl * 2 + half) * cm;
        uint64_t* dump = reinterpret_cast<uint64_t*>(smem + L.dump) + hw * 64 + hl;
        const uint32_t th = (uint32_t)(t >> 32), tlo = (uint32_t)t;
        const int lim = col_ok ? cm : 0;
        if (tlo == 0u && __ballot(tlo != 0u) == 0ull) {
          // threshold on the score part alone (the usual case)
#pragma unroll
          for (int j = 0; j < NT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const uint32_t ov = o[j][r];
              const bool keep = ov >= th && pos < lim;
              uint64_t* dst = keep ? cb + pos : dump;
              *dst = ((uint64_t)ov << 32) | (0xffffffffu - (base_id + kWaves * 16 * j + r));
              pos += keep ? 1 : 0;
            }
        } else {
#pragma unroll
          for (int j = 0; j < NT; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const uint32_t ov = o[j][r];
              const uint32_t lid = 0xffffffffu - (base_id + kWaves * 16 * j + r);
              const bool keep = (ov > th || (ov == th && lid >= tlo)) && pos < lim;
              uint64_t* dst = keep ? cb + pos : dump;
              *dst = ((uint64_t)ov << 32) | lid;
              pos += keep ? 1 : 0;
            }
        }
      }
      __syncthreads();
      // one wave per column sorts (the columns `owned` by the wave); the
      // rank-ordered list of half h goes to [h*m, h*m + k) of the column's
      // block (in place for h = 0: read before written)
#pragma unroll
      for (int o = 0; o < NCW; o++) {
        const int cc = owned(hw, o);
        if (t0 + (cc & (kTT - 1)) < a.T) {
          const int k = cc >= kTT ? a.R : a.W;
          int c = 0;
#pragma unroll
          for (int w = 0; w < kWaves; w++) c += s_cnt[fin][w][cc];
          c = min(c, cm);
          uint64_t* lst = cand + cc * 2 * cm + half * m;
          if constexpr (BF16) {
            sort_emit_range(cand + (cc * 2 + half) * cm, c, k, hl, s_range[0][cc],
                            s_range[1][cc], [&](int r, uint64_t kk) { lst[r] = list_entry(kk); });
          } else {
            uint64_t* last = &s_last[cc][half];
            sort_emit_range(cand + (cc * 2 + half) * cm, c, k < a.n_sub ? k + 1 : k, hl,
                            s_range[0][cc], s_range[1][cc], [&](int r, uint64_t kk) {
                              if (r < k) lst[r] = list_entry(kk);
                              else *last = list_entry(kk);
                            });
          }
        }
      }
    }

    // ---- 3. stage 2: this wave's columns (lists written by this wave) ------
    wave_lds_sync();
    for (int o = 0; o < NCW; o++) {
      const int cc = owned(wave, o);
      const int tw = t0 + (cc & (kTT - 1));
      const bool q = cc >= kTT;
      if (tw < a.T) {
        const int k = q ? a.R : a.W;
        const bool own_grid = q && L.gR;
        uint64_t* blk = cand + cc * 2 * cm;
        stage2<NPL2, !BF16>(blk, blk + m, &s_last[cc][0], (!BF16 && k < a.n_sub) ? k + 1 : k, k,
                     a.n_sub, own_grid ? grid + L.gW : grid,
                     own_grid ? rowoff + (m + 1) : rowoff, own_grid ? L.gR : L.gW,
                     q ? z.r2 : z.w2, blk + 2 * m, lane,
                     (q ? a.ridx : a.widx) + ((int64_t)st * a.T + tw) * k,
                     (q ? a.rwt : a.wwt) + ((int64_t)st * a.T + tw) * k);
      }
    }

    // ---- 4. fused decoding step: each token of the tile is a stream of its
    // own holding this one token.  The wave owning a token's key column
    // applies its gated delta writes; after a barrier, the wave owning its
    // query column sums its reads, taken after the write (Spanish page
    // "Mecanismo Central" items 3 and 4).  A lane group of d_v/4 lanes takes
    // one row at a time, 8 rows' loads in flight.  A build of its own (FUSE,
    // 4-token tiles), so that the other builds' registers are not touched.
    if constexpr (FUSE) {
      static_assert(!FUSE || TT == kTT / 2, "the fused step takes 4-token tiles");
      __syncthreads();  // the tile's slot lists are written
      const int lpr = a.d_v >> 2;  // a power of two, at most 64
      const int gpw = 64 / lpr;
      const int rg = lane / lpr, rl = lane - rg * lpr;
      // 4-token tiles: waves 0-3 own the tokens' key columns, 4-7 their query
      // columns (one each)
      const int cc = owned(wave, 0);
      const bool isq = cc >= kTT;
      const int tw = t0 + (cc & (kTT - 1));
      const bool live = (cc & (kTT - 1)) < TT && tw < a.T;  // wave-uniform
      const int64_t s = (int64_t)st * a.T + tw;  // slot-list row and stream of the token
      const int K = isq ? a.R : a.W;
      const int32_t* idx = (isq ? a.ridx : a.widx) + s * K;
      const float* wt = (isq ? a.rwt : a.wwt) + s * K;
      float* Ms = a.M + s * a.N * a.d_v + 4 * rl;
      // rows in batches of kEB per lane group, every row load of a batch in
      // flight before its first use (positions past the list, or naming no
      // slot of the table, load row 0 and are not used)
      constexpr int kEB = 8;
      for (int ph = 0; ph < 2; ph++) {  // 0: the writes, 1: the reads
        if (live && isq == (ph == 1)) {
          float al = 0.f, be = 0.f;
          float4 vv = make_float4(0.f, 0.f, 0.f, 0.f), acc = vv;
          if (ph == 0) {
            al = a.alpha[s];
            be = a.beta[s];
            vv = scanc::load_v4(a.v, a.v_bf16 != 0, s * a.d_v + 4 * rl);
          }
          for (int j0 = rg; j0 < K; j0 += gpw * kEB) {
            int32_t sl[kEB];
            float wv[kEB];
            float4 m[kEB];
#pragma unroll
            for (int u = 0; u < kEB; u++) {
              const int j = j0 + u * gpw;
              sl[u] = j < K ? idx[j] : -1;
              wv[u] = j < K ? wt[j] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kEB; u++) {
              const bool ok = (uint32_t)sl[u] < (uint32_t)a.N;
              m[u] = *reinterpret_cast<const float4*>(Ms + (int64_t)(ok ? sl[u] : 0) * a.d_v);
            }
#pragma unroll
            for (int u = 0; u < kEB; u++) {
              if ((uint32_t)sl[u] >= (uint32_t)a.N) continue;
              if (ph == 0) {
                float c, omc;
                dec_gate(be, wv[u], c, omc);
                *reinterpret_cast<float4*>(Ms + (int64_t)sl[u] * a.d_v) = make_float4(
                    dec_upd(m[u].x, al, omc, c, vv.x), dec_upd(m[u].y, al, omc, c, vv.y),
                    dec_upd(m[u].z, al, omc, c, vv.z), dec_upd(m[u].w, al, omc, c, vv.w));
              } else {
                acc = scanc::fma4(wv[u], m[u], acc);
              }
            }
          }
          if (ph == 1) {
            for (int off = lpr; off < 64; off <<= 1)
              acc = scanc::add4(acc, scanc::shfl_xor4(acc, off));
            if (rg == 0) *reinterpret_cast<float4*>(a.out + s * a.d_v + 4 * rl) = acc;
          }
        }
        __syncthreads();  // writes before reads; reads before the next tile's lists
      }
    }
  }
}

// Inverse of the standard normal CDF (P. J. Acklam's published rational
// approximation, relative error about 1e-9); it only steers the first
// threshold guess.
static inline double norm_quantile(double p) {
  static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02,
                             -2.759285104469687e+02, 1.383577518672690e+02,
                             -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02,
                             -1.556989798598866e+02, 6.680131188771972e+01,
                             -1.328068155288572e+01};
  static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01,
                             -2.400758277161838e+00, -2.549671010115749e+00,
                             4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01,
                             2.445134137142996e+00, 3.754408661907416e+00};
  if (p <= 0.0) return -8.0;
  if (p >= 1.0) return 8.0;
  const double pl = 0.02425;
  if (p < pl) {
    const double q = sqrt(-2 * log(p));
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  }
  if (p > 1 - pl) {
    const double q = sqrt(-2 * log(1 - p));
    return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  }
  const double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1);
}

// threshold z such that about 1.4*k of n Gaussian scores lie above mean + z*sd
static inline float guess_z(int k, int n) {
  double f = 1.4 * k / n;
  if (f > 0.95) f = 0.95;
  return (float)norm_quantile(1.0 - f);
}

template <bool BF16, int NT, int NPL2>
static inline hipError_t launch_t(const ScoreArgs& a, hipStream_t stream) {
  const ScoreSmem L = score_smem(a.W, a.R);
  // tiles of 8 tokens unless they would leave CUs idle (decoding, short
  // sequences): then tiles of 4, twice the workgroups, shorter per-tile chains
  const bool small = (int64_t)((a.T + kTT - 1) / kTT) * a.S < kTargetWorkgroups;
  // the fused decoding step always takes 4-token tiles
  auto k = a.fuse ? sdm_score_topk_kernel<BF16, NT, NPL2, kTT / 2, true>
                  : small ? sdm_score_topk_kernel<BF16, NT, NPL2, kTT / 2, false>
                          : sdm_score_topk_kernel<BF16, NT, NPL2, kTT, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
  if (e != hipSuccess) return e;
  // token tiles per workgroup (one grid build serves them all) while the
  // launch still has at least 2048 workgroups: up to 8, or up to 16 for the
  // large pruned grids (more than 5 keys a lane, k > 71), whose build costs
  // more (Long: 11.7 against 12.4 ms with 4)
  const int tt = (small || a.fuse) ? kTT / 2 : kTT;
  const int ntiles = (a.T + tt - 1) / tt;
  const int per_max = NPL2 <= 5 ? 8 : 16;
  int per = 1;
  while (per < per_max && (int64_t)((ntiles + 2 * per - 1) / (2 * per)) * a.S >= 2048) per *= 2;
  dim3 grid((ntiles + per - 1) / per, a.S);
  const ScoreZ z{guess_z(a.W, a.n_sub), guess_z(a.R, a.n_sub), guess_z(a.W, pruned_grid_size(a.W)),
                 guess_z(a.R, pruned_grid_size(a.R))};
  hipLaunchKernelGGL(k, grid, dim3(kThreads), L.total, stream, a, per, z);
  return hipGetLastError();
}

}  // namespace

// Launch for NT sub-key tiles per wave (n_sub <= 128*NT), any grid width.
template <int NT>
hipError_t launch_score_t(const ScoreArgs& a, bool bf16, int npl2, hipStream_t stream) {
#define SDM_SCORE_CASE(M_)                                                      \
  if (npl2 <= M_) return bf16 ? launch_t<true, NT, M_>(a, stream) : launch_t<false, NT, M_>(a, stream);
  SDM_SCORE_CASE(2)
  SDM_SCORE_CASE(5)
  SDM_SCORE_CASE(11)
#undef SDM_SCORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdm
