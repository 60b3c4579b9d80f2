// Device helpers shared by the forward scan and its reverse (gradient) sweep.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {
namespace scanc {

constexpr uint64_t kEmpty = 0x00000000ffffffffull;  // LDS hash entry: key -1, empty mask

// integer finaliser: a slot's hash for LDS tables and slot partitions.  The
// shift/multiply constants are the published "lowbias32" finaliser of Chris
// Wellons' hash-prospector search (a 32-bit xorshift-multiply mixer).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float4 load_v4(const void* v, bool bf16, int64_t off) {
  if (bf16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(v) + off);
    float4 r;
    r.x = __uint_as_float(raw.x << 16);
    r.y = __uint_as_float(raw.x & 0xffff0000u);
    r.z = __uint_as_float(raw.y << 16);
    r.w = __uint_as_float(raw.y & 0xffff0000u);
    return r;
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(v) + off);
}

__device__ __forceinline__ float4 fma4(float w, float4 x, float4 acc) {
  return make_float4(__fmaf_rn(w, x.x, acc.x), __fmaf_rn(w, x.y, acc.y),
                     __fmaf_rn(w, x.z, acc.z), __fmaf_rn(w, x.w, acc.w));
}

__device__ __forceinline__ float4 shfl_xor4(float4 a, int m) {
  return make_float4(__shfl_xor(a.x, m), __shfl_xor(a.y, m), __shfl_xor(a.z, m),
                     __shfl_xor(a.w, m));
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// writer mask of slot s in table h (0 when absent)
__device__ __forceinline__ uint32_t probe(const uint64_t* h, int hmsk, int32_t s) {
  int p = (int)(mix32((uint32_t)s) & (uint32_t)hmsk);
  while (true) {
    const uint64_t ent = h[p];
    const int32_t k = (int32_t)(uint32_t)ent;
    if (k == s) return (uint32_t)(ent >> 32);
    if (k == -1) return 0u;
    p = (p + 1) & hmsk;
  }
}

}  // namespace scanc
}  // namespace sdm
