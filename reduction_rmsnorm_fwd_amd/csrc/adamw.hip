// Fused AdamW step over many fp32 tensors in one launch, for gfx950.
//
// Definition (the Triton Adam kernel of "Fast-LLM: 高效大语言模型训练框架", 关键实现细节:
// one fused pass that scales the gradient by a device scalar, updates both moments,
// applies weight decay and the parameter update, and skips the whole update while a
// device no-op flag is set; the host passes step_size, bias_correction and
// decay_factor), read as AdamW with decoupled weight decay, per element:
//   g' = scale g;  m = b1 m + (1 - b1) g';  v = b2 v + (1 - b2) g'^2
//   p = decay_factor p - step_size m / (sqrt(v) / bias_correction + eps)
// The page notes that this kernel exists for one tensor at a time only; here one launch
// covers up to kMaxTensors tensors (a table in the kernel arguments), so the optimizer
// step of a model is a handful of launches instead of one per parameter tensor.
//
// Memory: 28 bytes per element (read p, g, m, v; write p, m, v), nothing else.  Each
// workgroup owns a chunk of kChunk consecutive elements of one tensor; every thread
// issues all its 16-byte loads (4 vectors of each of the four arrays) before any
// arithmetic, then writes back; loads and stores are non-temporal (every byte is
// touched once).  A tensor whose four pointers are not all 16-byte aligned goes
// element by element (same arithmetic, same results).
#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kAdamThreads = 256;
constexpr int kAdamVecs = 4;  // 16-byte vectors per thread and array
constexpr int64_t kChunk = (int64_t)kAdamThreads * kAdamVecs * 4;  // elements per workgroup
constexpr int kMaxTensors = 36;

struct TensorTable {
  float* p[kMaxTensors];
  const float* g[kMaxTensors];
  float* m[kMaxTensors];
  float* v[kMaxTensors];
  int64_t n[kMaxTensors];
  int64_t first_chunk[kMaxTensors + 1];  // chunk index where tensor i starts
  int32_t vec[kMaxTensors];              // 1: all four arrays 16-byte aligned
  int32_t count;
};

struct Hyper {
  float step_size, beta1, beta2, bias_correction, decay_factor, eps;
  const int32_t* noop;  // device flag; nonzero: no update at all (may be null)
  const float* scale;   // device gradient scale (null: 1)
};

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, const Hyper& h,
                                          float gs) {
  g *= gs;
  m = h.beta1 * m + (1.f - h.beta1) * g;
  v = h.beta2 * v + (1.f - h.beta2) * (g * g);
  p = h.decay_factor * p - h.step_size * m / (sqrtf(v) / h.bias_correction + h.eps);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(TensorTable tt, Hyper h) {
  if (h.noop != nullptr && *h.noop != 0) return;
  const float gs = h.scale != nullptr ? *h.scale : 1.f;
  const int64_t c = blockIdx.x;
  int t = 0;  // the tensor owning chunk c (tensors without chunks are skipped)
  while (t + 1 < tt.count && tt.first_chunk[t + 1] <= c) ++t;
  const int64_t n = tt.n[t];
  const int64_t e0 = (c - tt.first_chunk[t]) * kChunk;
  const int64_t e1 = e0 + kChunk < n ? e0 + kChunk : n;
  float* __restrict__ P = tt.p[t];
  const float* __restrict__ G = tt.g[t];
  float* __restrict__ M = tt.m[t];
  float* __restrict__ V = tt.v[t];
  const int tid = threadIdx.x;
  if (tt.vec[t]) {
    const int64_t nv = (e1 - e0) / 4;  // whole vectors in the chunk (e0 % 4 == 0)
    f32x4 p[kAdamVecs], g[kAdamVecs], m[kAdamVecs], v[kAdamVecs];
#pragma unroll
    for (int i = 0; i < kAdamVecs; ++i) {
      const int64_t k = (int64_t)i * kAdamThreads + tid;
      if (k < nv) {
        const int64_t e = e0 + 4 * k;
        p[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(P + e));
        g[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(G + e));
        m[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(M + e));
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(V + e));
      }
    }
#pragma unroll
    for (int i = 0; i < kAdamVecs; ++i) {
      const int64_t k = (int64_t)i * kAdamThreads + tid;
      if (k < nv) {
        const int64_t e = e0 + 4 * k;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pj = p[i][j], mj = m[i][j], vj = v[i][j];
          adam_elem(pj, g[i][j], mj, vj, h, gs);
          p[i][j] = pj; m[i][j] = mj; v[i][j] = vj;
        }
        __builtin_nontemporal_store(p[i], reinterpret_cast<f32x4*>(P + e));
        __builtin_nontemporal_store(m[i], reinterpret_cast<f32x4*>(M + e));
        __builtin_nontemporal_store(v[i], reinterpret_cast<f32x4*>(V + e));
      }
    }
    // the tensor's last 1..3 elements past its last whole vector
    const int64_t e = e0 + 4 * nv + tid;
    if (tid < 4 && e < e1) {
      float pj = P[e], mj = M[e], vj = V[e];
      adam_elem(pj, G[e], mj, vj, h, gs);
      P[e] = pj; M[e] = mj; V[e] = vj;
    }
  } else {
    for (int64_t e = e0 + tid; e < e1; e += kAdamThreads) {
      float pj = P[e], mj = M[e], vj = V[e];
      adam_elem(pj, G[e], mj, vj, h, gs);
      P[e] = pj; M[e] = mj; V[e] = vj;
    }
  }
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" int fo_adamw_step(int32_t n_tensors, const int64_t* numel, float* const* params,
                             const float* const* grads, float* const* exp_avgs,
                             float* const* exp_avg_sqs, const int32_t* noop_flag,
                             const float* grad_scale, float step_size, float beta1, float beta2,
                             float bias_correction, float decay_factor, float eps,
                             void* stream) {
  if (n_tensors < 0) return FO_ERR_SHAPE;
  if (n_tensors == 0) return FO_OK;
  if (!numel || !params || !grads || !exp_avgs || !exp_avg_sqs) return FO_ERR_NULL;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (numel[i] < 0) return FO_ERR_SHAPE;
    if (numel[i] > 0 && (!params[i] || !grads[i] || !exp_avgs[i] || !exp_avg_sqs[i]))
      return FO_ERR_NULL;
  }
  const Hyper h{step_size, beta1, beta2, bias_correction, decay_factor, eps, noop_flag,
                grad_scale};
  hipStream_t st = as_stream(stream);
  for (int32_t b = 0; b < n_tensors; b += kMaxTensors) {
    TensorTable tt{};
    tt.count = (n_tensors - b < kMaxTensors) ? n_tensors - b : kMaxTensors;
    int64_t chunks = 0;
    for (int i = 0; i < tt.count; ++i) {
      const int32_t s = b + i;
      tt.p[i] = params[s];
      tt.g[i] = grads[s];
      tt.m[i] = exp_avgs[s];
      tt.v[i] = exp_avg_sqs[s];
      tt.n[i] = numel[s];
      tt.vec[i] = aligned16(params[s]) && aligned16(grads[s]) && aligned16(exp_avgs[s]) &&
                  aligned16(exp_avg_sqs[s]);
      tt.first_chunk[i] = chunks;
      chunks += ceil_div(numel[s], kChunk);
      if (chunks > INT32_MAX) return FO_ERR_SHAPE;
    }
    tt.first_chunk[tt.count] = chunks;
    if (chunks == 0) continue;
    adamw_kernel<<<dim3((unsigned)chunks), dim3(kAdamThreads), 0, st>>>(tt, h);
    if (hipGetLastError() != hipSuccess) return FO_ERR_HIP;
  }
  return FO_OK;
}
