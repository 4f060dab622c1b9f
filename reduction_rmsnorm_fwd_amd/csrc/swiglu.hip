// SwiGLU forward and backward for gfx950, and the other MLP activations of the same
// page: gated or plain, SiLU / GeLU / ReLU ("支持的 MLP 变体": dense MLPs gated or not,
// with SiLU, GeLU or ReLU; GeLU taken as the exact x Phi(x), Phi from the complementary
// error function below).
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构: gated MLP with SiLU in the
// Transformer Block 结构 table, and mlp gated: true / activation: silu in 训练配置示例;
// fused op in "LLaMA-Factory Kernels 系统" and in the Liger section of
// "Kernels（自定义内核）"):
//   h = silu(g) u,  silu(g) = g s(g),  s(g) = 1/(1+exp(-g))
//   dg = dh u s (1 + g (1 - s)),  du = dh g s
// Purely elementwise and HBM-bound: each element of every operand is read once and
// each output written once with 16-byte vector accesses, the gate and up reads of an
// element issued together so one pass produces the output.  Rows may have their own
// strides (halves of a [T, 2F] tensor work); fully contiguous operands are walked as
// one flat row, and rows of several blocks whose last block would be partial as one
// flat space of blocks that run on into the next row.  bf16 rows off the 16-byte grid (odd F, or halves of a [T, 2F] tensor
// with odd F) still move their full vectors as 16-byte accesses at element-aligned
// addresses, the partial last vector of a row element by element.
#include <type_traits>

#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // vectors per thread per operand

__device__ __forceinline__ float sigmoid_f(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Activations of the MLP variants: SiLU, GeLU (exact: x Phi(x)), ReLU; value and
// derivative in fp32.
enum Act { kSilu = FO_ACT_SILU, kGelu = FO_ACT_GELU, kRelu = FO_ACT_RELU };

// The complementary error function (Press et al., Numerical Recipes, section 6.2, erfcc):
// erfc(|z|) = t exp(-z^2 + P(t)), t = 1/(1 + |z|/2), with P a Chebyshev-fitted polynomial
// of degree 9; fractional error below 1.2e-7 for every z; erfc(-z) = 2 - erfc(z).
__device__ __forceinline__ float erfc_poly(float t) {
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  return fmaf(p, t, -1.26551223f);
}
__device__ __forceinline__ float erfc_f(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, az, 1.0f));
  const float r = t * __expf(fmaf(-az, az, erfc_poly(t)));
  return z >= 0.f ? r : 2.0f - r;
}
// The same, with exp(-z^2) returned beside it in e2 (the normal density's exponential,
// shared with the derivative of GeLU).
__device__ __forceinline__ float erfc_e2(float z, float& e2) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, az, 1.0f));
  e2 = __expf(-az * az);
  const float r = t * e2 * __expf(erfc_poly(t));
  return z >= 0.f ? r : 2.0f - r;
}

template <int ACT>
__device__ __forceinline__ float act_f(float x) {
  if constexpr (ACT == kSilu) return x * sigmoid_f(x);
  else if constexpr (ACT == kGelu) return x * (0.5f * erfc_f(x * -0.70710678118654752f));
  else return x > 0.f ? x : 0.f;
}
template <int ACT>
__device__ __forceinline__ float act_d(float x) {
  if constexpr (ACT == kSilu) {
    const float s = sigmoid_f(x);
    return s * fmaf(x, 1.0f - s, 1.0f);
  } else if constexpr (ACT == kGelu) {
    float e2;  // exp(-x^2 / 2)
    const float phi = 0.5f * erfc_e2(x * -0.70710678118654752f, e2);
    return fmaf(x * 0.39894228040143268f, e2, phi);
  } else {
    return x > 0.f ? 1.f : 0.f;
  }
}

// Index space: rows x nvr vectors (VEC elements each), walked as one flat space.
// GATED: h = act(g) u; otherwise h = act(g) (u unused).
// Vector v of a row of nel elements.  UA (rows of any element alignment and length):
// a full vector is one 16-byte access at its element-aligned address (gfx950 serves
// global memory in unaligned mode), the partial last vector goes element by element.
template <typename T, bool UA>
__device__ __forceinline__ Pack<T> ld_v(const T* p, int64_t v, int64_t nel) {
  constexpr int VEC = Vec<T>::N;
  if (!UA || (v + 1) * VEC <= nel) return load_pack(p + v * VEC);
  Pack<T> r;
#pragma unroll
  for (int j = 0; j < VEC; ++j) r.v[j] = v * VEC + j < nel ? p[v * VEC + j] : from_f32<T>(0.f);
  return r;
}
template <typename T, bool UA>
__device__ __forceinline__ void st_v(T* p, int64_t v, int64_t nel, const Pack<T>& o) {
  constexpr int VEC = Vec<T>::N;
  if (!UA || (v + 1) * VEC <= nel) {
    store_pack(p + v * VEC, o);
  } else {
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      if (v * VEC + j < nel) p[v * VEC + j] = o.v[j];
  }
}

// The (row, vector) pairs of all rows form one flat index space, cut into blocks of
// kThreads * kUnroll consecutive pairs, so a block may run on into the next row and
// every block but the last is full whatever the row length.  Slot i of thread t takes
// pair f = block * kThreads * kUnroll + i * kThreads + t: row f / nvr (inv = 1 / nvr in
// fp64, then corrected by one where the product rounds across an integer), vector
// f - row * nvr.
__device__ __forceinline__ void flat_pair(int64_t f, int64_t nvr, double inv, int64_t& row,
                                          int64_t& v) {
  row = (int64_t)((double)f * inv);
  v = f - row * nvr;
  if (v < 0) { --row; v += nvr; }
  else if (v >= nvr) { ++row; v -= nvr; }
}
// The (row, vector) pairs of a thread's kUnroll slots, kThreads apart, and whether each
// exists.  FLAT: blocks over the flat space (rows of at least kThreads vectors step from
// the first slot, crossing at most one row boundary per step; shorter rows divide per
// slot).  Otherwise nb blocks per row, none crossing a row, as for one contiguous run:
// measured faster for rows that fill their blocks or take one (F 4864 halves: 42.0
// against 44.3 us flat), slower for rows of several blocks with a partial last one (F
// 14336 halves: forward 125.1 against 119.7 us flat, backward 215.1 against 205.1 us).
template <bool FLAT>
__device__ __forceinline__ void slot_pairs(int64_t total, int64_t nvr, double inv, int64_t nb,
                                           int64_t* row, int64_t* v, bool* ok) {
  if constexpr (FLAT) {
    const int64_t f0 = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    flat_pair(f0, nvr, inv, row[0], v[0]);
#pragma unroll
    for (int i = 1; i < kUnroll; ++i) {
      if (nvr >= kThreads) {
        row[i] = row[i - 1];
        v[i] = v[i - 1] + kThreads;
        if (v[i] >= nvr) { v[i] -= nvr; ++row[i]; }
      } else {
        flat_pair(f0 + i * kThreads, nvr, inv, row[i], v[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) ok[i] = f0 + i * kThreads < total;
  } else {
    const int64_t r = blockIdx.x / nb;
    const int64_t v0 = (blockIdx.x - r * nb) * (kThreads * kUnroll) + threadIdx.x;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      row[i] = r;
      v[i] = v0 + i * kThreads;
      ok[i] = v[i] < nvr;
    }
  }
}

// nel: elements per row (= nvr * VEC unless UA, where the last vector may be partial);
// total = rows * nvr pairs
template <typename T, int VEC, int ACT, bool GATED, bool UA = false, bool FLAT = false>
__global__ __launch_bounds__(kThreads) void swiglu_fwd_k(int64_t total, int64_t nvr, double inv,
                                                         int64_t nb, int64_t nel, const T* g,
                                                         int64_t ldg, const T* u, int64_t ldu,
                                                         T* h, int64_t ldh) {
  int64_t rw[kUnroll], vv[kUnroll];
  bool ok[kUnroll];
  slot_pairs<FLAT>(total, nvr, inv, nb, rw, vv, ok);
  if constexpr (VEC > 1) {
    Pack<T> gv[kUnroll], uv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        gv[i] = ld_v<T, UA>(g + rw[i] * ldg, vv[i], nel);
        if constexpr (GATED) uv[i] = ld_v<T, UA>(u + rw[i] * ldu, vv[i], nel);
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        Pack<T> o;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const float gf = to_f32(gv[i].v[j]);
          if constexpr (GATED) o.v[j] = from_f32<T>(act_f<ACT>(gf) * to_f32(uv[i].v[j]));
          else o.v[j] = from_f32<T>(act_f<ACT>(gf));
        }
        st_v<T, UA>(h + rw[i] * ldh, vv[i], nel, o);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        const int64_t v = vv[i];
        const float gf = to_f32(g[rw[i] * ldg + v]);
        T* hr = h + rw[i] * ldh;
        if constexpr (GATED) hr[v] = from_f32<T>(act_f<ACT>(gf) * to_f32(u[rw[i] * ldu + v]));
        else hr[v] = from_f32<T>(act_f<ACT>(gf));
      }
    }
  }
}

// GATED: dg = dh u act'(g), du = dh act(g); otherwise dg = dh act'(g) (u, du unused).
template <typename T, int VEC, int ACT, bool GATED, bool UA = false, bool FLAT = false>
__global__ __launch_bounds__(kThreads) void swiglu_bwd_k(int64_t total, int64_t nvr, double inv,
                                                         int64_t nb, int64_t nel, const T* dh,
                                                         int64_t lddh, const T* g, int64_t ldg,
                                                         const T* u, int64_t ldu, T* dg,
                                                         int64_t lddg, T* du, int64_t lddu) {
  int64_t rw[kUnroll], vv[kUnroll];
  bool ok[kUnroll];
  slot_pairs<FLAT>(total, nvr, inv, nb, rw, vv, ok);
  if constexpr (VEC > 1) {
    Pack<T> hv[kUnroll], gv[kUnroll], uv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        hv[i] = ld_v<T, UA>(dh + rw[i] * lddh, vv[i], nel);
        gv[i] = ld_v<T, UA>(g + rw[i] * ldg, vv[i], nel);
        if constexpr (GATED) uv[i] = ld_v<T, UA>(u + rw[i] * ldu, vv[i], nel);
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        const int64_t v = vv[i];
        T* dgr = dg + rw[i] * lddg;
        T* dur = GATED ? du + rw[i] * lddu : nullptr;
        Pack<T> og, ou;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const float gf = to_f32(gv[i].v[j]);
          const float hf = to_f32(hv[i].v[j]);
          if constexpr (GATED && ACT == kSilu) {
            // one sigmoid for both outputs
            const float uf = to_f32(uv[i].v[j]);
            const float s = sigmoid_f(gf);
            og.v[j] = from_f32<T>(hf * uf * s * fmaf(gf, 1.0f - s, 1.0f));
            ou.v[j] = from_f32<T>(hf * gf * s);
          } else if constexpr (GATED) {
            const float uf = to_f32(uv[i].v[j]);
            og.v[j] = from_f32<T>(hf * uf * act_d<ACT>(gf));
            ou.v[j] = from_f32<T>(hf * act_f<ACT>(gf));
          } else {
            og.v[j] = from_f32<T>(hf * act_d<ACT>(gf));
          }
        }
        st_v<T, UA>(dgr, v, nel, og);
        if constexpr (GATED) st_v<T, UA>(dur, v, nel, ou);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      if (ok[i]) {
        const int64_t v = vv[i];
        const T* gr = g + rw[i] * ldg;
        const T* dhr = dh + rw[i] * lddh;
        const T* ur = GATED ? u + rw[i] * ldu : nullptr;
        T* dgr = dg + rw[i] * lddg;
        T* dur = GATED ? du + rw[i] * lddu : nullptr;
        const float gf = to_f32(gr[v]), hf = to_f32(dhr[v]);
        if constexpr (GATED && ACT == kSilu) {
          const float uf = to_f32(ur[v]);
          const float s = sigmoid_f(gf);
          dgr[v] = from_f32<T>(hf * uf * s * fmaf(gf, 1.0f - s, 1.0f));
          dur[v] = from_f32<T>(hf * gf * s);
        } else if constexpr (GATED) {
          const float uf = to_f32(ur[v]);
          dgr[v] = from_f32<T>(hf * uf * act_d<ACT>(gf));
          dur[v] = from_f32<T>(hf * act_f<ACT>(gf));
        } else {
          dgr[v] = from_f32<T>(hf * act_d<ACT>(gf));
        }
      }
    }
  }
}

// Launch geometry: rows x vectors-per-row; one flat row when every operand is a
// single contiguous [T*F] run.
struct Geo {
  int64_t rows, nvr, nel;
  int64_t nb;    // blocks per row, or (flat) blocks over the whole (row, vector) space
  int64_t grid;  // workgroups
  bool vec;      // 16-byte vectors on the 16-byte grid
  bool ua;       // otherwise, bf16: 16-byte vectors at element-aligned addresses
  bool flat;     // rows of several blocks whose last one is partial: one flat space
};

template <typename T>
Geo plan(int64_t T_, int64_t F, int n, const void* const* ptr, const int64_t* ld) {
  constexpr int VEC = Vec<T>::N;
  bool contiguous = true, aligned = true, ld_ok = true;
  for (int i = 0; i < n; ++i) {
    contiguous = contiguous && ld[i] == F;
    aligned = aligned && aligned16(ptr[i]);
    ld_ok = ld_ok && ld[i] % VEC == 0;
  }
  bool elem = true;
  for (int i = 0; i < n; ++i) elem = elem && reinterpret_cast<uintptr_t>(ptr[i]) % sizeof(T) == 0;
  Geo g;
  const int64_t per_row = contiguous ? T_ * F : F;
  g.rows = contiguous ? 1 : T_;
  g.vec = aligned && per_row % VEC == 0 && (contiguous || ld_ok);
  // 2-byte elements one by one are bound by the access issue rate; fp32 element
  // accesses coalesce well enough to keep
  g.ua = !g.vec && sizeof(T) == 2 && elem;
  g.nel = per_row;
  g.nvr = g.vec ? per_row / VEC : g.ua ? ceil_div(per_row, (int64_t)VEC) : per_row;
  constexpr int64_t kSpan = kThreads * kUnroll;
  g.flat = g.rows > 1 && g.nvr > kSpan && g.nvr % kSpan != 0;
  g.nb = g.flat ? ceil_div(g.rows * g.nvr, kSpan) : ceil_div(g.nvr, kSpan);
  g.grid = g.flat ? g.nb : g.rows * g.nb;
  return g;
}

// GATED = false: u, du (and their strides) are ignored.
template <typename T, int ACT, bool GATED>
int fwd_impl(int64_t T_, int64_t F, const void* g, int64_t ldg, const void* u, int64_t ldu,
             void* h, int64_t ldh, hipStream_t st) {
  const void* p[3] = {g, h, u};
  const int64_t l[3] = {ldg, ldh, ldu};
  const Geo geo = plan<T>(T_, F, GATED ? 3 : 2, p, l);
  const dim3 grid((unsigned)geo.grid), block(kThreads);
  const int64_t total = geo.rows * geo.nvr;
  const double inv = 1.0 / (double)geo.nvr;
  const T* gp = static_cast<const T*>(g);
  const T* up = static_cast<const T*>(u);
  T* hp = static_cast<T*>(h);
  auto go = [&](auto flat) {
    constexpr bool FL = decltype(flat)::value;
    if (geo.vec)
      swiglu_fwd_k<T, Vec<T>::N, ACT, GATED, false, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, gp, ldg, up, ldu, hp, ldh);
    else if (geo.ua)
      swiglu_fwd_k<T, Vec<T>::N, ACT, GATED, true, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, gp, ldg, up, ldu, hp, ldh);
    else
      swiglu_fwd_k<T, 1, ACT, GATED, false, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, gp, ldg, up, ldu, hp, ldh);
  };
  if (geo.flat) go(std::true_type{});
  else go(std::false_type{});
  return launch_status();
}

template <typename T, int ACT, bool GATED>
int bwd_impl(int64_t T_, int64_t F, const void* dh, int64_t lddh, const void* g, int64_t ldg,
             const void* u, int64_t ldu, void* dg, int64_t lddg, void* du, int64_t lddu,
             hipStream_t st) {
  const void* p[5] = {dh, g, dg, u, du};
  const int64_t l[5] = {lddh, ldg, lddg, ldu, lddu};
  const Geo geo = plan<T>(T_, F, GATED ? 5 : 3, p, l);
  const dim3 grid((unsigned)geo.grid), block(kThreads);
  const int64_t total = geo.rows * geo.nvr;
  const double inv = 1.0 / (double)geo.nvr;
  const T* dhp = static_cast<const T*>(dh);
  const T* gp = static_cast<const T*>(g);
  const T* up = static_cast<const T*>(u);
  T* dgp = static_cast<T*>(dg);
  T* dup = static_cast<T*>(du);
  auto go = [&](auto flat) {
    constexpr bool FL = decltype(flat)::value;
    if (geo.vec)
      swiglu_bwd_k<T, Vec<T>::N, ACT, GATED, false, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, dhp, lddh, gp, ldg, up, ldu, dgp, lddg, dup, lddu);
    else if (geo.ua)
      swiglu_bwd_k<T, Vec<T>::N, ACT, GATED, true, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, dhp, lddh, gp, ldg, up, ldu, dgp, lddg, dup, lddu);
    else
      swiglu_bwd_k<T, 1, ACT, GATED, false, FL><<<grid, block, 0, st>>>(
          total, geo.nvr, inv, geo.nb, geo.nel, dhp, lddh, gp, ldg, up, ldu, dgp, lddg, dup, lddu);
  };
  if (geo.flat) go(std::true_type{});
  else go(std::false_type{});
  return launch_status();
}

// dtype x activation dispatch
template <bool GATED>
int fwd_dispatch(int dtype, int act, int64_t T_, int64_t F, const void* g, int64_t ldg,
                 const void* u, int64_t ldu, void* h, int64_t ldh, hipStream_t st) {
#define FO_F(TY, A) return fwd_impl<TY, A, GATED>(T_, F, g, ldg, u, ldu, h, ldh, st)
  if (dtype == FO_F32) {
    if (act == kSilu) FO_F(float, kSilu);
    if (act == kGelu) FO_F(float, kGelu);
    FO_F(float, kRelu);
  }
  if (act == kSilu) FO_F(bf16, kSilu);
  if (act == kGelu) FO_F(bf16, kGelu);
  FO_F(bf16, kRelu);
#undef FO_F
}

template <bool GATED>
int bwd_dispatch(int dtype, int act, int64_t T_, int64_t F, const void* dh, int64_t lddh,
                 const void* g, int64_t ldg, const void* u, int64_t ldu, void* dg, int64_t lddg,
                 void* du, int64_t lddu, hipStream_t st) {
#define FO_B(TY, A) \
  return bwd_impl<TY, A, GATED>(T_, F, dh, lddh, g, ldg, u, ldu, dg, lddg, du, lddu, st)
  if (dtype == FO_F32) {
    if (act == kSilu) FO_B(float, kSilu);
    if (act == kGelu) FO_B(float, kGelu);
    FO_B(float, kRelu);
  }
  if (act == kSilu) FO_B(bf16, kSilu);
  if (act == kGelu) FO_B(bf16, kGelu);
  FO_B(bf16, kRelu);
#undef FO_B
}

bool grid_fits(int64_t T_, int64_t F) {
  // rows * column blocks must fit a 1-D grid
  return T_ * ceil_div(F, kThreads * kUnroll) < (int64_t)UINT32_MAX &&
         ceil_div(T_ * F, kThreads * kUnroll) < (int64_t)UINT32_MAX;
}

}  // namespace
}  // namespace fo

using namespace fo;

static bool act_ok(int act) { return act == FO_ACT_SILU || act == FO_ACT_GELU || act == FO_ACT_RELU; }

extern "C" int fo_glu_fwd(int dtype, int act, int64_t T, int64_t F, const void* gate,
                          int64_t ldg, const void* up, int64_t ldu, void* h, int64_t ldh,
                          void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!act_ok(act)) return FO_ERR_SHAPE;
  if (T < 0 || F < 1 || !grid_fits(T, F)) return FO_ERR_SHAPE;
  if (ldg < F || ldu < F || ldh < F) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!gate || !up || !h) return FO_ERR_NULL;
  return fwd_dispatch<true>(dtype, act, T, F, gate, ldg, up, ldu, h, ldh, as_stream(stream));
}

extern "C" int fo_glu_bwd(int dtype, int act, int64_t T, int64_t F, const void* dh,
                          int64_t lddh, const void* gate, int64_t ldg, const void* up,
                          int64_t ldu, void* dgate, int64_t lddg, void* dup, int64_t lddu,
                          void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!act_ok(act)) return FO_ERR_SHAPE;
  if (T < 0 || F < 1 || !grid_fits(T, F)) return FO_ERR_SHAPE;
  if (lddh < F || ldg < F || ldu < F || lddg < F || lddu < F) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!dh || !gate || !up || !dgate || !dup) return FO_ERR_NULL;
  return bwd_dispatch<true>(dtype, act, T, F, dh, lddh, gate, ldg, up, ldu, dgate, lddg, dup,
                            lddu, as_stream(stream));
}

extern "C" int fo_swiglu_fwd(int dtype, int64_t T, int64_t F, const void* gate, int64_t ldg,
                             const void* up, int64_t ldu, void* h, int64_t ldh, void* stream) {
  return fo_glu_fwd(dtype, FO_ACT_SILU, T, F, gate, ldg, up, ldu, h, ldh, stream);
}

extern "C" int fo_swiglu_bwd(int dtype, int64_t T, int64_t F, const void* dh, int64_t lddh,
                             const void* gate, int64_t ldg, const void* up, int64_t ldu,
                             void* dgate, int64_t lddg, void* dup, int64_t lddu, void* stream) {
  return fo_glu_bwd(dtype, FO_ACT_SILU, T, F, dh, lddh, gate, ldg, up, ldu, dgate, lddg, dup,
                    lddu, stream);
}

extern "C" int fo_act_fwd(int dtype, int act, int64_t T, int64_t F, const void* x,
                          int64_t ldx, void* y, int64_t ldy, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!act_ok(act)) return FO_ERR_SHAPE;
  if (T < 0 || F < 1 || !grid_fits(T, F)) return FO_ERR_SHAPE;
  if (ldx < F || ldy < F) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!x || !y) return FO_ERR_NULL;
  return fwd_dispatch<false>(dtype, act, T, F, x, ldx, nullptr, F, y, ldy, as_stream(stream));
}

extern "C" int fo_act_bwd(int dtype, int act, int64_t T, int64_t F, const void* dy,
                          int64_t lddy, const void* x, int64_t ldx, void* dx, int64_t lddx,
                          void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (!act_ok(act)) return FO_ERR_SHAPE;
  if (T < 0 || F < 1 || !grid_fits(T, F)) return FO_ERR_SHAPE;
  if (lddy < F || ldx < F || lddx < F) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!dy || !x || !dx) return FO_ERR_NULL;
  return bwd_dispatch<false>(dtype, act, T, F, dy, lddy, x, ldx, nullptr, F, dx, lddx, nullptr, F,
                             as_stream(stream));
}
