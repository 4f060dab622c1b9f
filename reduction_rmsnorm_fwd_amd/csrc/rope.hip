// Rotary position embedding on Q and K, forward and backward, in place, for gfx950.
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构: the attention mixer
// carries RoPE; 训练配置示例 gives rotary type default with theta, and the head
// counts heads / head_groups / head_size; "LLaMA-Factory Kernels 系统" and the Liger
// section of "Kernels（自定义内核）" list it as a fused op).  Half-split pairing:
//   a[t,i] = pos[t] * theta^(-2i/D),  (x_i, x_{i+D/2}) <- R(a) (x_i, x_{i+D/2})
// The backward applies R(-a).
//
// A workgroup owns a few consecutive tokens.  It first computes cos/sin of every
// (token, pair) once into LDS: the angle is the fp64 product of the position and the
// host-computed fp64 frequency, range-reduced against 2*pi in fp64, and only the
// reduced angle (|r| <= pi) is rounded to fp32 for sincosf.  That keeps the angle
// error near 1e-7 rad at any position, where an fp32 product would be off by 1e-3 rad
// at position 16383.  The workgroup streams every head of Q and K of its tokens: a
// unit is one 16-byte vector of the low half and the matching vector of the high half
// of one head, read once and written once; the first units' loads are issued before
// the table is built, so the table's fp64 work hides under their latency.  A token at
// position 0 is the identity rotation: it is not written, so its data stays
// bit-identical, signed zeros included.
#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kMaxHeadDim = 512;
constexpr int kMaxTok = 8;       // tokens per workgroup, at most
constexpr int kThreads = 256;
constexpr int kMaxU = 4;         // (low, high) vector pairs per thread, at most

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

// VEC elements per access (16-byte vectors, or 1 for the scalar path).  A workgroup
// owns `tok` consecutive tokens (chosen by the host so that each thread has at most
// kMaxU units); every thread first issues the loads of all its units, then rotates and
// stores them, so up to 2*kMaxU 16-byte loads per thread are in flight.
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void rope_kernel(
    int64_t T_, int nq, int nkv, int D, int tok, T* q, int64_t ldq, T* k, int64_t ldk,
    const int64_t* __restrict__ pos, Freqs fr, float sgn) {
  __shared__ float cs[kMaxTok][kMaxHeadDim / 2][2];
  __shared__ int ident[kMaxTok];
  const int P = D / 2;
  const int64_t t0 = (int64_t)blockIdx.x * tok;
  const int ntok = (T_ - t0 < tok) ? (int)(T_ - t0) : tok;
  const int PV = P / VEC;  // vectors per half head
  const int per_tok = (nq + nkv) * PV;
  const int nunits = ntok * per_tok;
  for (int ub = 0; ub < nunits; ub += kThreads * kMaxU) {
    T* lo[kMaxU];
    Pack<T> a[kMaxU], b[kMaxU];
    int tlu[kMaxU], pvu[kMaxU];
#pragma unroll
    for (int m = 0; m < kMaxU; ++m) {
      const int u = ub + threadIdx.x + m * kThreads;
      lo[m] = nullptr;
      if (u < nunits) {
        const int tl = u / per_tok;
        const int rem = u - tl * per_tok;
        const int h = rem / PV;
        const int pv = rem - h * PV;
        const int64_t t = t0 + tl;
        T* base = (h < nq) ? q + t * ldq + (int64_t)h * D : k + t * ldk + (int64_t)(h - nq) * D;
        lo[m] = base + pv * VEC;
        tlu[m] = tl;
        pvu[m] = pv;
        if constexpr (VEC > 1) {
          a[m] = load_pack(lo[m]);
          b[m] = load_pack(lo[m] + P);
        } else {
          a[m].v[0] = lo[m][0];
          b[m].v[0] = lo[m][P];
        }
      }
    }
    if (ub == 0) {
      // the table is built while the first loads are in flight
      if (threadIdx.x < ntok) ident[threadIdx.x] = pos[t0 + threadIdx.x] == 0;
      for (int u = threadIdx.x; u < ntok * P; u += kThreads) {
        const int tl = u / P, i = u - tl * P;
        const double ang = (double)pos[t0 + tl] * fr.f[i];
        float c, sn;
        rope_cs(ang, c, sn);
        cs[tl][i][0] = c;
        cs[tl][i][1] = sgn * sn;
      }
      __syncthreads();
    }
#pragma unroll
    for (int m = 0; m < kMaxU; ++m) {
      if (lo[m] == nullptr || ident[tlu[m]]) continue;  // position 0: left untouched
      Pack<T> oa, ob;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float c = cs[tlu[m]][pvu[m] * VEC + j][0];
        const float sn = cs[tlu[m]][pvu[m] * VEC + j][1];
        const float x1 = to_f32(a[m].v[j]), x2 = to_f32(b[m].v[j]);
        oa.v[j] = from_f32<T>(fmaf(x1, c, -x2 * sn));
        ob.v[j] = from_f32<T>(fmaf(x2, c, x1 * sn));
      }
      if constexpr (VEC > 1) {
        store_pack(lo[m], oa);
        store_pack(lo[m] + P, ob);
      } else {
        lo[m][0] = oa.v[0];
        lo[m][P] = ob.v[0];
      }
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
  const int per_tok = (nq + nkv) * ((D / 2) / (vec ? VEC : 1));
  // tokens per workgroup: as many as fit kMaxU units per thread (at least one token;
  // a token wider than that takes several passes of the unit loop below)
  int tok = (kThreads * kMaxU) / per_tok;
  tok = tok < 1 ? 1 : (tok > kMaxTok ? kMaxTok : tok);
  const dim3 grid((unsigned)ceil_div(T_, tok)), block(kThreads);
  if (vec)
    rope_kernel<T, VEC><<<grid, block, 0, st>>>(T_, nq, nkv, D, tok, static_cast<T*>(q), ldq,
                                                static_cast<T*>(k), ldk, pos, fr, sgn);
  else
    rope_kernel<T, 1><<<grid, block, 0, st>>>(T_, nq, nkv, D, tok, static_cast<T*>(q), ldq,
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
