// Shared device and host helpers of the gfx950 kernels: element types, 16-byte vector
// access, wave64/workgroup reductions, argument checks and launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "fo.h"

namespace fo {

typedef __bf16 bf16;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// element <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// gfx950 converts with v_cvt_pk_bf16_f32: round to nearest even, NaN kept NaN.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// elements per 16-byte vector
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

// A 16-byte register image of N elements of T.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
union Pack {
  u32x4 raw;
  T v[Vec<T>::N];
};

// Streaming load (data read once): non-temporal hint.
template <typename T>
__device__ __forceinline__ Pack<T> load_pack(const T* p) {
  Pack<T> r;
  r.raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return r;
}
// Cached load for data that is read again soon (weights, a row read twice).
template <typename T>
__device__ __forceinline__ Pack<T> load_pack_cached(const T* p) {
  Pack<T> r;
  r.raw = *reinterpret_cast<const u32x4*>(p);
  return r;
}
template <typename T>
__device__ __forceinline__ void store_pack(T* p, const Pack<T>& r) {
  __builtin_nontemporal_store(r.raw, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// reductions (fixed order: deterministic)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Merge two (max, sum-of-exp relative to max) pairs of an online logsumexp.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) { s = 0.f; m = mn; return; }
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}
__device__ __forceinline__ void wave_lse(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, kWave);
    float s2 = __shfl_xor(s, o, kWave);
    lse_merge(m, s, m2, s2);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FO_OK : FO_ERR_HIP;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace fo
