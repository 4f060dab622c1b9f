// Rotary position embedding on Q and K, forward and backward, in place, for gfx950.
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构: the attention mixer
// carries RoPE; 训练配置示例 gives rotary type default with theta, and the head
// counts heads / head_groups / head_size; "LLaMA-Factory Kernels 系统" and the Liger
// section of "Kernels（自定义内核）" list it as a fused op).  Half-split pairing:
//   a[t,i] = pos[t] * theta^(-2i/D),  (x_i, x_{i+D/2}) <- R(a) (x_i, x_{i+D/2})
// The backward applies R(-a).
//
// A workgroup owns kTok consecutive tokens.  It first computes cos/sin of every
// (token, pair) once into LDS: the angle is the fp64 product of the position and the
// host-computed fp64 frequency, range-reduced against 2*pi in fp64, and only the
// reduced angle (|r| <= pi) is rounded to fp32 for sincosf.  That keeps the angle
// error near 1e-7 rad at any position, where an fp32 product would be off by 1e-3 rad
// at position 16383.  Then the workgroup streams every head of Q and K of its tokens:
// a unit is one 16-byte vector of the low half and the matching vector of the high
// half of one head, read once and written once.  A token at position 0 is the
// identity rotation: it is skipped (neither read nor written), so its data stays
// bit-identical, signed zeros included.
#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kMaxHeadDim = 512;
constexpr int kTok = 4;          // tokens per workgroup
constexpr int kThreads = 256;

struct Freqs {
  double f[kMaxHeadDim / 2];  // theta^(-2i/D), fp64, computed on the host
};

__device__ __forceinline__ void rope_cs(double a, float& c, float& s) {
  // a - n*2pi with 2pi split in two doubles (Cody-Waite); |result| <= pi (+ tiny)
  constexpr double kTwoPiHi = 6.28318530717958623200e+00;
  constexpr double kTwoPiLo = 2.44929359829470635445e-16;
  constexpr double kInvTwoPi = 1.59154943091895345608e-01;
  const double n = rint(a * kInvTwoPi);
  double r = fma(-n, kTwoPiHi, a);
  r = fma(-n, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// VEC elements per access (16-byte vectors, or 1 for the scalar path)
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void rope_kernel(
    int64_t T_, int nq, int nkv, int D, T* q, int64_t ldq, T* k, int64_t ldk,
    const int64_t* __restrict__ pos, Freqs fr, float sgn) {
  __shared__ float cs[kTok][kMaxHeadDim / 2][2];
  __shared__ int ident[kTok];
  const int P = D / 2;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int ntok = (T_ - t0 < kTok) ? (int)(T_ - t0) : kTok;
  if (threadIdx.x < ntok) ident[threadIdx.x] = pos[t0 + threadIdx.x] == 0;
  for (int u = threadIdx.x; u < ntok * P; u += kThreads) {
    const int tl = u / P, i = u - tl * P;
    const double a = (double)pos[t0 + tl] * fr.f[i];
    float c, s;
    rope_cs(a, c, s);
    cs[tl][i][0] = c;
    cs[tl][i][1] = sgn * s;
  }
  __syncthreads();
  const int PV = P / VEC;             // vectors per half head
  const int heads = nq + nkv;
  const int per_tok = heads * PV;
  for (int u = threadIdx.x; u < ntok * per_tok; u += kThreads) {
    const int tl = u / per_tok;
    const int rem = u - tl * per_tok;
    const int h = rem / PV;
    const int pv = rem - h * PV;
    if (ident[tl]) continue;
    const int64_t t = t0 + tl;
    T* base = (h < nq) ? q + t * ldq + (int64_t)h * D : k + t * ldk + (int64_t)(h - nq) * D;
    T* lo = base + pv * VEC;
    T* hi = lo + P;
    float c[VEC], s[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      c[j] = cs[tl][pv * VEC + j][0];
      s[j] = cs[tl][pv * VEC + j][1];
    }
    if constexpr (VEC > 1) {
      Pack<T> a = load_pack(lo), b = load_pack(hi), oa, ob;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float x1 = to_f32(a.v[j]), x2 = to_f32(b.v[j]);
        oa.v[j] = from_f32<T>(fmaf(x1, c[j], -x2 * s[j]));
        ob.v[j] = from_f32<T>(fmaf(x2, c[j], x1 * s[j]));
      }
      store_pack(lo, oa);
      store_pack(hi, ob);
    } else {
      const float x1 = to_f32(lo[0]), x2 = to_f32(hi[0]);
      lo[0] = from_f32<T>(fmaf(x1, c[0], -x2 * s[0]));
      hi[0] = from_f32<T>(fmaf(x2, c[0], x1 * s[0]));
    }
  }
}

template <typename T>
int rope_impl(int64_t T_, int nq, int nkv, int D, void* q, int64_t ldq, void* k, int64_t ldk,
              const int64_t* pos, double theta, float sgn, hipStream_t st) {
  Freqs fr;
  for (int i = 0; i < D / 2; ++i) fr.f[i] = pow(theta, -2.0 * (double)i / (double)D);
  constexpr int VEC = Vec<T>::N;
  const bool vec = (D / 2) % VEC == 0 && ldq % VEC == 0 && ldk % VEC == 0 && aligned16(q) &&
                   aligned16(k);
  const dim3 grid((unsigned)ceil_div(T_, kTok)), block(kThreads);
  if (vec)
    rope_kernel<T, VEC><<<grid, block, 0, st>>>(T_, nq, nkv, D, static_cast<T*>(q), ldq,
                                                static_cast<T*>(k), ldk, pos, fr, sgn);
  else
    rope_kernel<T, 1><<<grid, block, 0, st>>>(T_, nq, nkv, D, static_cast<T*>(q), ldq,
                                              static_cast<T*>(k), ldk, pos, fr, sgn);
  return launch_status();
}

int rope_entry(int dtype, int64_t T, int32_t nq, int32_t nkv, int32_t D, void* q, int64_t ldq,
               void* k, int64_t ldk, const int64_t* pos, double theta, float sgn,
               void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (nq < 1 || nkv < 1 || nq % nkv != 0) return FO_ERR_SHAPE;
  if (D < 2 || D % 2 != 0 || D > kMaxHeadDim) return FO_ERR_SHAPE;
  if (!(theta > 0.0)) return FO_ERR_SHAPE;
  if ((int64_t)nq * D > INT32_MAX / 4) return FO_ERR_SHAPE;
  if (ldq < (int64_t)nq * D || ldk < (int64_t)nkv * D) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!q || !k || !pos) return FO_ERR_NULL;
  hipStream_t st = as_stream(stream);
  return dtype == FO_F32 ? rope_impl<float>(T, nq, nkv, D, q, ldq, k, ldk, pos, theta, sgn, st)
                         : rope_impl<bf16>(T, nq, nkv, D, q, ldq, k, ldk, pos, theta, sgn, st);
}

}  // namespace
}  // namespace fo

extern "C" int fo_rope_fwd(int dtype, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, void* q, int64_t ldq, void* k, int64_t ldk,
                           const int64_t* positions, double theta, void* stream) {
  return fo::rope_entry(dtype, T, n_q_heads, n_kv_heads, head_dim, q, ldq, k, ldk, positions,
                        theta, 1.0f, stream);
}

extern "C" int fo_rope_bwd(int dtype, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, void* dq, int64_t ldq, void* dk, int64_t ldk,
                           const int64_t* positions, double theta, void* stream) {
  return fo::rope_entry(dtype, T, n_q_heads, n_kv_heads, head_dim, dq, ldq, dk, ldk, positions,
                        theta, -1.0f, stream);
}
