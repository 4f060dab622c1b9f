// Measurement probes: a streaming copy and a register-only bf16 MFMA loop.  They run
// beside the ops in the same process, so each op's rate can be stated against the
// ceilings this device reaches in practice as well as against the published peaks
// (HBM 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s).  Neither is part of any op.
#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kCopyUnroll = 4;

// dst = src, 16-byte non-temporal loads and stores, kCopyUnroll vectors per thread in
// flight, one pass (every vector is read once and written once).
__global__ __launch_bounds__(256) void probe_copy_k(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (base + u * 256 < n) v[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (base + u * 256 < n) __builtin_nontemporal_store(v[u], dst + base + u * 256);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kMfmaChains = 4;  // independent accumulators per wave
constexpr int kMfmaWaves = 4;   // waves per workgroup; two workgroups per CU

// Every wave runs `iters` rounds of kMfmaChains independent 32x32x16 bf16 MFMAs on
// register operands; launched as two 4-wave workgroups per CU (2 waves per SIMD, as
// in the GEMM).  The accumulator sums are written out so the loop is not removed.
__global__ __launch_bounds__(kMfmaWaves * 64) void probe_mfma_k(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (float)threadIdx.x + (float)e);
    b[e] = (bf16)(0.5f * (float)e);
  }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * kMfmaWaves + threadIdx.x / 64] = s;
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" int fo_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return FO_OK;
  if (!src || !dst) return FO_ERR_NULL;
  if (bytes % 16 != 0 || !aligned16(src) || !aligned16(dst)) return FO_ERR_STRIDE;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t blocks = ceil_div(n, 256 * kCopyUnroll);
  if (blocks > INT32_MAX) return FO_ERR_SHAPE;
  probe_copy_k<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return launch_status();
}

extern "C" int fo_probe_mfma(int32_t n_cu, int64_t iters, float* out, void* stream) {
  if (n_cu < 1 || iters < 1 || iters > INT32_MAX) return FO_ERR_SHAPE;
  if (!out) return FO_ERR_NULL;
  probe_mfma_k<<<dim3((unsigned)(2 * n_cu)), dim3(kMfmaWaves * 64), 0, as_stream(stream)>>>(
      (int)iters, out);
  return launch_status();
}
