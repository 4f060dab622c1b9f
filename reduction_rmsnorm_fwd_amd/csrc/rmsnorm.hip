// RMSNorm forward and backward for gfx950.
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构: Transformer Block 结构
// lists RMSNorm as a block normalisation; 训练配置示例 gives type rms_norm with an
// epsilon; the Liger section of "Kernels（自定义内核）" fuses it into one kernel):
//   r[t] = 1/sqrt(mean_j x[t,j]^2 + eps),  y[t,j] = x[t,j] r[t] w[j]
//   dx = r (w*dy) - r^3 x mean_j(w_j dy_j x_j),  dw[j] = sum_t dy[t,j] x[t,j] r[t]
//
// Fast path (16-byte aligned rows whose length is a multiple of the vector): the
// forward gives each row RW wave64s (one up to 8 vectors per lane, 2-16 for longer rows,
// the row sums then combined through LDS) and holds the row in registers between the
// sum of squares and the write, so x is read from HBM exactly once.  The backward gives
// each row RW waves (RW grows with d so a lane holds at most 16 elements per operand,
// up to 16 waves); every lane owns a fixed set of columns and accumulates their dw
// contribution in registers across all the rows its workgroup visits.  The waves of a
// workgroup are folded through LDS in a fixed order into one fp32 partial row per
// workgroup (a workgroup of one row group writes it from registers), at most 512
// workgroups, and a second small kernel sums the partial rows in a fixed order.  Rows that start off a 16-byte boundary or whose
// length is not a multiple of the vector take the same kernels (template flag UA):
// their full vectors are still moved as 16-byte accesses at element-aligned addresses,
// and the d % VEC elements past the last full vector go to the first lanes of the row's
// first wave, one element each.  Rows too long for the registers (beyond 131072 bf16 /
// 65536 fp32 elements forward, 16384 backward) take a workgroup-per-row path that
// reads the row twice (the second read from L2).
#include <initializer_list>
#include <type_traits>

#include "fo_common.hpp"

namespace fo {
namespace {

constexpr int kFwdWaves = 4;     // waves per workgroup, forward (rows of one wave)
constexpr int kBwdWaves = 8;     // waves per workgroup, backward (rows of <= 8 waves)
constexpr int kMaxRowWaves = 16;  // waves per row at most (one 1024-thread workgroup)
constexpr int kFwdMaxNV = 8;     // vectors per lane before a row takes more waves
constexpr size_t kMaxLds = 160 * 1024;  // LDS of one workgroup on gfx950
constexpr int kMaxPartials = 512;  // dw partial rows (workgroups of the backward)
constexpr int kGenericThreads = 256;

// ------------------------------------------------------- vectors of a row, any alignment
// A row is nvec = d / VEC full vectors, then (UA only) a tail of d % VEC elements.
// UA = false: the row (or w, b) starts on 16 bytes and d is a multiple of the vector.
// UA = true: it starts on any element and d is any length.  The full vectors are still
// moved as 16-byte accesses at their element-aligned addresses (gfx950 runs global
// memory in unaligned mode: such loads cost nothing extra, stores ~12%, measured
// against aligned ones), so every byte read or written is one of the row's.  Tail
// element k (k < d % VEC) belongs to lane k of the row's first wave, which loads,
// reduces and stores it beside its vectors, so the vectors keep the lane layout (and
// launch plan) of a row of d - d % VEC elements.
template <typename T, bool NT>
__device__ __forceinline__ Pack<T> ld_vec(const T* p, int v) {
  constexpr int VEC = Vec<T>::N;
  return NT ? load_pack(p + (int64_t)v * VEC) : load_pack_cached(p + (int64_t)v * VEC);
}
template <typename T>
__device__ __forceinline__ void st_vec(T* p, int v, const Pack<T>& o) {
  store_pack(p + (int64_t)v * Vec<T>::N, o);
}

// w g - m with the product rounded before the subtraction (no fused multiply-add), as
// the row sum that m is the mean of rounds each w g: where every w g of a row equals m
// (a one-column row) the result is exactly 0 rather than the product's rounding error.
__device__ __forceinline__ float centred(float w, float g, float m) {
#pragma clang fp contract(off)
  return w * g - m;
}

// ----------------------------------------------------------------- forward, fast
// Sum over the RW waves of a row, combined in wave order; every lane of the row gets
// the total.  With RW > 1 every wave of the workgroup must call it (two barriers).
template <int RW>
__device__ __forceinline__ float row_sum(float v, float* part) {
  v = wave_sum(v);
  if constexpr (RW > 1) {
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) part[wave] = v;
    __syncthreads();
    const int base = wave - wave % RW;
    v = 0.f;
#pragma unroll
    for (int k = 0; k < RW; ++k) v += part[base + k];
    __syncthreads();  // the slots are rewritten by the next sum
  }
  return v;
}

// threads of a forward (backward) workgroup whose rows take RW waves each
constexpr int fwd_threads(int RW) { return (RW > kFwdWaves ? RW : kFwdWaves) * kWave; }
constexpr int bwd_threads(int RW) { return (RW > kBwdWaves ? RW : kBwdWaves) * kWave; }

// A row takes RW waves (RW = 1 up to rows of kFwdMaxNV vectors per lane, more for
// longer rows); lane (wr, l) of a row holds the vectors (wr*64 + l) + i*RW*64, i < NV,
// in registers between the sums and the write, so x is read from HBM exactly once.
// LN: LayerNorm (mean subtracted before the variance, bias added); mean and centred
// variance are two sweeps over the registers.
// nvec: full vectors per row (d / VEC); UA: lanes k < d % VEC of the row's first wave
// also own tail element k.
template <typename T, int NV, int RW, bool LN, bool UA>
__global__ __launch_bounds__(fwd_threads(RW)) void rmsnorm_fwd_wave(
    int64_t T_, int nvec, int d, const T* __restrict__ x, int64_t ldx,
    const T* __restrict__ w, const T* __restrict__ b, float eps, T* y, int64_t ldy,
    float* __restrict__ mean, float* __restrict__ rstd) {
  constexpr int VEC = Vec<T>::N;
  constexpr int RG = fwd_threads(RW) / kWave / RW;  // rows per workgroup
  __shared__ float part[RW > 1 ? fwd_threads(RW) / kWave : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wr = wave % RW;
  const int64_t row = (int64_t)blockIdx.x * RG + wave / RW;
  // a one-wave row leaves at once; waves of wider rows stay for the barriers
  if (RW == 1 && row >= T_) return;
  const bool live = row < T_;
  const int vbase = wr * kWave + lane;
  const T* xr = x + (live ? row : 0) * ldx;
  const int tcol = nvec * VEC + lane;  // this lane's tail element (UA, first wave)
  const bool tl = UA && live && wr == 0 && tcol < d;
  Pack<T> xv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = vbase + i * RW * kWave;
    if (live && v < nvec) xv[i] = ld_vec<T, true>(xr, v);
    else xv[i].raw = u32x4{0, 0, 0, 0};
  }
  const float xt = tl ? to_f32(xr[tcol]) : 0.f;
  float mu = 0.f;
  if constexpr (LN) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < VEC; ++j) s += to_f32(xv[i].v[j]);
    mu = row_sum<RW>(UA ? s + xt : s, part) / (float)d;
    // re-widen for the variance sweep instead of holding fp32 copies (as below)
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(xv[i].raw));
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      if constexpr (LN) {
        const float f = to_f32(xv[i].v[j]) - mu;
        // unused slots hold 0, not mu.  (Aligned rows test per element: the same set,
        // and measured 9% faster at T 8192, d 4096 bf16 than the per-vector test.)
        const int v = vbase + i * RW * kWave;
        if (UA ? v < nvec : v * VEC + j < d) ss = fmaf(f, f, ss);
      } else {
        const float f = to_f32(xv[i].v[j]);
        ss = fmaf(f, f, ss);
      }
    }
  if (tl) ss = fmaf(xt - mu, xt - mu, ss);
  ss = row_sum<RW>(ss, part);
  if (!live) return;
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  T* yr = y + row * ldy;
  // re-widen from the packed row instead of holding fp32 copies: fewer VGPRs, more
  // waves per SIMD
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(xv[i].raw));
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = vbase + i * RW * kWave;
    if (v < nvec) {
      const Pack<T> wv = ld_vec<T, false>(w, v);
      Pack<T> o;
      if constexpr (LN) {
        const Pack<T> bv = ld_vec<T, false>(b, v);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
          o.v[j] = from_f32<T>(fmaf((to_f32(xv[i].v[j]) - mu) * r, to_f32(wv.v[j]), to_f32(bv.v[j])));
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.v[j] = from_f32<T>(to_f32(xv[i].v[j]) * r * to_f32(wv.v[j]));
      }
      st_vec<T>(yr, v, o);
    }
  }
  if (tl) {
    if constexpr (LN) yr[tcol] = from_f32<T>(fmaf((xt - mu) * r, to_f32(w[tcol]), to_f32(b[tcol])));
    else yr[tcol] = from_f32<T>(xt * r * to_f32(w[tcol]));
  }
  if (lane == 0 && wr == 0) {
    if (rstd != nullptr) rstd[row] = r;
    if constexpr (LN) {
      if (mean != nullptr) mean[row] = mu;
    }
  }
}

// Workgroup sum with a fixed combination order; every thread gets the total.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += sh[i];
  return t;
}

// -------------------------------------------------------------- forward, generic
template <typename T, bool LN>
__global__ __launch_bounds__(kGenericThreads) void rmsnorm_fwd_block(
    int64_t T_, int64_t d, const T* x, int64_t ldx, const T* __restrict__ w,
    const T* __restrict__ b, float eps, T* y, int64_t ldy, float* __restrict__ mean,
    float* __restrict__ rstd) {
  __shared__ float sh[kGenericThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ldx;
  float mu = 0.f;
  if constexpr (LN) {
    float s = 0.f;
    for (int64_t j = threadIdx.x; j < d; j += kGenericThreads) s += to_f32(xr[j]);
    mu = block_sum<kGenericThreads>(s, sh) / (float)d;
  }
  float ss = 0.f;
  for (int64_t j = threadIdx.x; j < d; j += kGenericThreads) {
    const float f = to_f32(xr[j]) - mu;
    ss = fmaf(f, f, ss);
  }
  ss = block_sum<kGenericThreads>(ss, sh);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  T* yr = y + row * ldy;
  for (int64_t j = threadIdx.x; j < d; j += kGenericThreads) {
    if constexpr (LN) yr[j] = from_f32<T>(fmaf((to_f32(xr[j]) - mu) * r, to_f32(w[j]), to_f32(b[j])));
    else yr[j] = from_f32<T>(to_f32(xr[j]) * r * to_f32(w[j]));
  }
  if (threadIdx.x == 0) {
    if (rstd != nullptr) rstd[row] = r;
    if constexpr (LN) {
      if (mean != nullptr) mean[row] = mu;
    }
  }
}

// ----------------------------------------------------------------- backward, fast
// A workgroup of kBwdWaves waves works on kBwdWaves/RW rows at a time, RW waves per
// row; lane (w, l) of a row owns the vectors (w*64 + l) + i*RW*64, i < NV, and keeps
// its columns' dw contribution in registers across all rows the workgroup visits.
// With RW > 1 the per-row dot products are combined across the RW waves through LDS
// (every wave runs the same number of row rounds, so the barriers match).  The next
// round's rows (and their saved 1/rms) are loaded before the current round is reduced,
// so a round's cross-wave barrier never leaves the memory pipe empty.  At the end the
// waves' column partials are folded through LDS in a fixed order into one fp32 partial
// row per workgroup: partial[blockIdx.x, :].
//
// LN (LayerNorm, mean and rstd saved by the forward): with g = w*dy and xc = x - mean,
//   dx = r (g - mean_j(g)) - r^3 xc mean_j(g xc),  dw += dy xc r,  db += dy,
// the db partials folded beside the dw partials (partial row of 2d floats).  g - mean(g)
// is formed first (see centred()), so a row whose centred gradient vanishes exactly
// (one column) gives dx exactly 0.
// nvec: full vectors per row (d / VEC); UA: lanes k < d % VEC of each row group's first
// wave also own tail element k, held as scalars beside the vectors.
template <typename T, int NV, int RW, bool LN, bool UA>
__global__ __launch_bounds__(bwd_threads(RW)) void rmsnorm_bwd_wave(
    int64_t T_, int nvec, int d, const T* dy, int64_t lddy, const T* x, int64_t ldx,
    const T* __restrict__ w, const float* __restrict__ mean, const float* __restrict__ rstd,
    float eps, T* dx, int64_t lddx, float* __restrict__ partial, int direct) {
  constexpr int VEC = Vec<T>::N;
  constexpr int NW = bwd_threads(RW) / kWave;  // waves per workgroup
  constexpr int RG = NW / RW;         // rows in flight per workgroup
  constexpr int NB = LN ? NV : 1;     // db accumulators (LayerNorm only)
  extern __shared__ float fold[];     // [d], or [2d] for LN
  __shared__ float xdot[NW], xss[NW];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = wave / RW, wr = wave % RW;
  const int vbase = wr * kWave + lane;
  const int tcol = nvec * VEC + lane;  // this lane's tail element (UA, first wave only)
  const bool tl = UA && wr == 0 && tcol < d;
  const float wt = tl ? to_f32(w[tcol]) : 0.f;
  float acct = 0.f, accbt = 0.f;
  Pack<T> wv[NV];
  float acc[NV][VEC], accb[NB][VEC];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = vbase + i * RW * kWave;
    if (v < nvec) wv[i] = ld_vec<T, false>(w, v);
    else wv[i].raw = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[i][j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < VEC; ++j) accb[i][j] = 0.f;
  const float inv_d = 1.0f / (float)d;
  const int64_t stride = (int64_t)gridDim.x * RG;
  const int64_t rounds = ceil_div(T_ - (int64_t)blockIdx.x * RG, stride);
  Pack<T> gv[NV], xv[NV], gn[NV], xn[NV];
  float rv = 0.f, rn = 0.f;  // the saved 1/rms (1/std) of the row (loaded with the row)
  float mv = 0.f, mn = 0.f;  // LN: the saved mean of the row
  float gt = 0.f, xt = 0.f, gtn = 0.f, xtn = 0.f;  // the tail element of dy and x (UA)
  auto load_round = [&](int64_t rd, Pack<T>* g, Pack<T>* xx, float& r, float& m, float& g1,
                        float& x1) {
    const int64_t row = (int64_t)blockIdx.x * RG + rg + rd * stride;
    const bool live = rd < rounds && row < T_;
    if (rstd != nullptr && live) r = rstd[row];
    if constexpr (LN) {
      if (live) m = mean[row];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = vbase + i * RW * kWave;
      if (live && v < nvec) {
        g[i] = ld_vec<T, true>(dy + row * lddy, v);
        xx[i] = ld_vec<T, true>(x + row * ldx, v);
      } else {
        g[i].raw = u32x4{0, 0, 0, 0};
        xx[i].raw = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (UA) {
      g1 = live && tl ? to_f32(dy[row * lddy + tcol]) : 0.f;
      x1 = live && tl ? to_f32(x[row * ldx + tcol]) : 0.f;
    }
  };
  load_round(0, gv, xv, rv, mv, gt, xt);
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t row = (int64_t)blockIdx.x * RG + rg + rd * stride;
    const bool live = row < T_;
    load_round(rd + 1, gn, xn, rn, mn, gtn, xtn);
    // RMS: dot = sum g x, ss = sum x^2;  LN: dot = sum g (x - mean), ss = sum g
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float gf = to_f32(wv[i].v[j]) * to_f32(gv[i].v[j]);
        if constexpr (LN) {
          // padding lanes hold zeros in w and dy, so gf = 0 there
          dot = fmaf(gf, to_f32(xv[i].v[j]) - mv, dot);
          ss += gf;
        } else {
          const float xf = to_f32(xv[i].v[j]);
          dot = fmaf(gf, xf, dot);
          ss = fmaf(xf, xf, ss);
        }
      }
    if constexpr (UA) {
      // lanes without a tail element hold zeros in wt, gt and xt
      const float gf = wt * gt;
      if constexpr (LN) {
        dot = fmaf(gf, xt - mv, dot);
        ss += gf;
      } else {
        dot = fmaf(gf, xt, dot);
        ss = fmaf(xt, xt, ss);
      }
    }
    dot = wave_sum(dot);
    ss = wave_sum(ss);
    // keep the operands packed across the reduction (re-widened below)
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(gv[i].raw), "+v"(xv[i].raw), "+v"(wv[i].raw));
    if constexpr (RW > 1) {
      if (lane == 0) { xdot[wave] = dot; xss[wave] = ss; }
      __syncthreads();
      dot = 0.f;
      ss = 0.f;
#pragma unroll
      for (int k = 0; k < RW; ++k) { dot += xdot[rg * RW + k]; ss += xss[rg * RW + k]; }
      __syncthreads();  // slots are rewritten next round
    }
    if (live) {
      float r, k, c = 0.f;
      if constexpr (LN) {
        r = rv;
        k = r * r * r * (dot * inv_d);
        c = ss * inv_d;
      } else {
        r = rstd != nullptr ? rv : 1.0f / sqrtf(ss * inv_d + eps);
        k = r * r * r * (dot * inv_d);
      }
      T* dxr = dx + row * lddx;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = vbase + i * RW * kWave;
        if (v < nvec) {
          Pack<T> o;
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const float gf = to_f32(gv[i].v[j]);
            if constexpr (LN) {
              const float xc = to_f32(xv[i].v[j]) - mv;
              o.v[j] = from_f32<T>(r * centred(to_f32(wv[i].v[j]), gf, c) - k * xc);
              acc[i][j] = fmaf(gf * xc, r, acc[i][j]);
              accb[i][j] += gf;
            } else {
              const float xf = to_f32(xv[i].v[j]);
              o.v[j] = from_f32<T>(r * (to_f32(wv[i].v[j]) * gf) - k * xf);
              acc[i][j] = fmaf(gf * xf, r, acc[i][j]);
            }
          }
          st_vec<T>(dxr, v, o);
        }
      }
      if (tl) {
        if constexpr (LN) {
          const float xc = xt - mv;
          dxr[tcol] = from_f32<T>(r * centred(wt, gt, c) - k * xc);
          acct = fmaf(gt * xc, r, acct);
          accbt += gt;
        } else {
          dxr[tcol] = from_f32<T>(r * (wt * gt) - k * xt);
          acct = fmaf(gt * xt, r, acct);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      gv[i] = gn[i];
      xv[i] = xn[i];
    }
    rv = rn;
    mv = mn;
    gt = gtn;
    xt = xtn;
  }
  constexpr int kCols = LN ? 2 : 1;
  float* out = partial + (int64_t)blockIdx.x * kCols * d;
  if constexpr (RG == 1) {
    if (direct != 0) {
      // one row group: every column belongs to one lane, which writes it from its
      // registers (direct 2: as 16-byte stores, the partial row being 16-byte aligned)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = vbase + i * RW * kWave;
        if (v < nvec) {
          if (!UA && direct == 2) {
#pragma unroll
            for (int j = 0; j < VEC; j += 4) {
              *reinterpret_cast<float4*>(out + v * VEC + j) =
                  make_float4(acc[i][j], acc[i][j + 1], acc[i][j + 2], acc[i][j + 3]);
              if constexpr (LN)
                *reinterpret_cast<float4*>(out + d + v * VEC + j) =
                    make_float4(accb[i][j], accb[i][j + 1], accb[i][j + 2], accb[i][j + 3]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
              out[v * VEC + j] = acc[i][j];
              if constexpr (LN) out[d + v * VEC + j] = accb[i][j];
            }
          }
        }
      }
      if (tl) {
        out[tcol] = acct;
        if constexpr (LN) out[d + tcol] = accbt;
      }
      return;
    }
  }
  // fold the row groups' column partials in order 0,1,2,... (RW waves of a group own
  // disjoint columns, so they write their slots in the same step)
  for (int s = 0; s < RG; ++s) {
    if (rg == s) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = vbase + i * RW * kWave;
        if (v < nvec) {
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            float* p = &fold[v * VEC + j];
            *p = (s == 0) ? acc[i][j] : (*p + acc[i][j]);
            if constexpr (LN) {
              float* q = &fold[d + v * VEC + j];
              *q = (s == 0) ? accb[i][j] : (*q + accb[i][j]);
            }
          }
        }
      }
      if (tl) {
        fold[tcol] = (s == 0) ? acct : (fold[tcol] + acct);
        if constexpr (LN) fold[d + tcol] = (s == 0) ? accbt : (fold[d + tcol] + accbt);
      }
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < kCols * d; j += blockDim.x) out[j] = fold[j];
}

// -------------------------------------------------------------- backward, generic
// One workgroup per row: dx, and (RMS) r[t] saved for the dw pass.  LN uses the saved
// mean and rstd.
template <typename T, bool LN>
__global__ __launch_bounds__(kGenericThreads) void rmsnorm_bwd_dx_block(
    int64_t T_, int64_t d, const T* dy, int64_t lddy, const T* x, int64_t ldx,
    const T* __restrict__ w, const float* __restrict__ mean, const float* __restrict__ rstd,
    float eps, T* dx, int64_t lddx, float* __restrict__ r_out) {
  __shared__ float sh[kGenericThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* dyr = dy + row * lddy;
  const T* xr = x + row * ldx;
  const float mu = LN ? mean[row] : 0.f;
  float dot = 0.f, ss = 0.f;
  for (int64_t j = threadIdx.x; j < d; j += kGenericThreads) {
    const float gf = to_f32(w[j]) * to_f32(dyr[j]);
    if constexpr (LN) {
      dot = fmaf(gf, to_f32(xr[j]) - mu, dot);
      ss += gf;
    } else {
      const float xf = to_f32(xr[j]);
      dot = fmaf(gf, xf, dot);
      ss = fmaf(xf, xf, ss);
    }
  }
  dot = block_sum<kGenericThreads>(dot, sh);
  float r, c = 0.f;
  if constexpr (LN) {
    r = rstd[row];
    c = block_sum<kGenericThreads>(ss, sh) / (float)d;
  } else if (rstd != nullptr) {
    r = rstd[row];
  } else {
    ss = block_sum<kGenericThreads>(ss, sh);
    r = 1.0f / sqrtf(ss / (float)d + eps);
  }
  const float k = r * r * r * (dot / (float)d);
  T* dxr = dx + row * lddx;
  // dx may alias dy: every element is read (above) by the thread that writes it, and
  // the block_sum barriers separate all reads of the dot product from these writes.
  for (int64_t j = threadIdx.x; j < d; j += kGenericThreads) {
    const float xf = to_f32(xr[j]) - mu;
    const float gw = LN ? centred(to_f32(w[j]), to_f32(dyr[j]), c) : to_f32(w[j]) * to_f32(dyr[j]);
    dxr[j] = from_f32<T>(r * gw - k * xf);
  }
  if constexpr (!LN) {
    if (threadIdx.x == 0) r_out[row] = r;
  }
}

// dw (and, LN, db) partial rows of the generic path: workgroup (g, column block) sums
// its row range; LN writes the db partial at column d + j.
template <typename T, bool LN>
__global__ __launch_bounds__(256) void rmsnorm_dw_partial_block(
    int64_t T_, int64_t d, const T* dy, int64_t lddy, const T* x, int64_t ldx,
    const float* __restrict__ mean, const float* __restrict__ r, int64_t rows_per_group,
    float* __restrict__ partial) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = blockIdx.y;
  if (j >= d) return;
  const int64_t r0 = g * rows_per_group;
  const int64_t r1 = (r0 + rows_per_group < T_) ? r0 + rows_per_group : T_;
  float acc = 0.f, accb = 0.f;
  for (int64_t t = r0; t < r1; ++t) {
    const float gf = to_f32(dy[t * lddy + j]);
    if constexpr (LN) {
      acc = fmaf(gf * (to_f32(x[t * ldx + j]) - mean[t]), r[t], acc);
      accb += gf;
    } else {
      acc = fmaf(gf * to_f32(x[t * ldx + j]), r[t], acc);
    }
  }
  if constexpr (LN) {
    partial[g * 2 * d + j] = acc;
    partial[g * 2 * d + d + j] = accb;
  } else {
    partial[g * d + j] = acc;
  }
}

// dw[j] = sum_g partial[g, j].  A workgroup covers 32 columns (one 128-byte line of a
// partial row) as 8 float4 lanes; its 32 row phases each sum a contiguous block of
// partial rows in order (up to 16 rows' loads issued before the first add), then 32
// threads add the 32 phase sums in order 0..31.  Each line is read by one workgroup
// only, and whole, so no two XCDs fetch the same line.
constexpr int kReducePhases = 32;
constexpr int kReduceCols = 32;
constexpr int kReduceUnroll = 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Columns [0, split) go to out0, columns [split, d) to out1 (LayerNorm: dw then db from
// one launch over the 2d-wide partial rows).
__global__ __launch_bounds__(256) void rmsnorm_dw_reduce(int64_t G, int64_t d, int64_t ldp,
                                                        const float* __restrict__ partial,
                                                        float* __restrict__ out0, int64_t split,
                                                        float* __restrict__ out1) {
  constexpr int Q = kReduceCols / 4;  // float4 lanes per row phase
  static_assert(Q * kReducePhases == 256, "one thread per (phase, float4 lane)");
  __shared__ float sh[kReducePhases][kReduceCols + 1];
  const int q = threadIdx.x % Q;
  const int ph = threadIdx.x / Q;
  const int64_t j = (int64_t)blockIdx.x * kReduceCols + q * 4;
  const int64_t per = (G + kReducePhases - 1) / kReducePhases;
  const int64_t g0 = ph * per;
  const int64_t g1 = (g0 + per < G) ? g0 + per : G;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (j + 3 < d && ldp % 4 == 0 && (reinterpret_cast<uintptr_t>(partial) & 15) == 0) {
    for (int64_t g = g0; g < g1; g += kReduceUnroll) {
      f32x4 v[kReduceUnroll];
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u)
        if (g + u < g1)
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(partial + (g + u) * ldp + j));
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u)
        if (g + u < g1)
#pragma unroll
          for (int c = 0; c < 4; ++c) a[c] += v[u][c];
    }
  } else {
    for (int64_t g = g0; g < g1; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j + c < d) a[c] += partial[g * ldp + j + c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) sh[ph][q * 4 + c] = a[c];
  __syncthreads();
  if (threadIdx.x < kReduceCols) {
    const int64_t jc = (int64_t)blockIdx.x * kReduceCols + threadIdx.x;
    float v[kReducePhases];
#pragma unroll
    for (int p = 0; p < kReducePhases; ++p) v[p] = sh[p][threadIdx.x];
    float t = v[0];
#pragma unroll
    for (int p = 1; p < kReducePhases; ++p) t += v[p];
    if (jc < split) out0[jc] = t;
    else if (jc < d) out1[jc - split] = t;
  }
}

__global__ void fill_f32(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------------------------ dispatch
template <typename T>
bool vector_ok(int64_t d, const void* a, int64_t lda, const void* b, int64_t ldb,
               const void* c, int64_t ldc, const void* w) {
  constexpr int VEC = Vec<T>::N;
  return d % VEC == 0 && lda % VEC == 0 && ldb % VEC == 0 && ldc % VEC == 0 &&
         aligned16(a) && aligned16(b) && aligned16(c) && aligned16(w) &&
         d / VEC <= (int64_t)kMaxRowWaves * kWave * 16;
}

// Rows of any alignment and length that still fit the registers of the wave kernels
// (UA = true there): element-aligned pointers, at most 16 full vectors per lane of
// kMaxRowWaves waves (the tail of fewer than VEC elements rides on scalar registers
// beside them).  The backward fits fewer (bwd_fits).
template <typename T>
bool unaligned_ok(int64_t d, std::initializer_list<const void*> ptrs) {
  bool ok = d / Vec<T>::N <= (int64_t)kMaxRowWaves * kWave * 16;
  for (const void* p : ptrs) ok = ok && reinterpret_cast<uintptr_t>(p) % sizeof(T) == 0;
  return ok;
}

// Launch plan of the forward: waves per row (rw, the fewest that keep a lane at
// kFwdMaxNV vectors, up to kMaxRowWaves) and vectors per lane (nv).
struct FwdPlan {
  int rw, nv;
};
inline FwdPlan fwd_plan(int64_t nvec) {
  FwdPlan p{1, 1};
  while (p.rw < kMaxRowWaves && ceil_div(nvec, (int64_t)p.rw * kWave) > kFwdMaxNV) p.rw *= 2;
  const int64_t per = ceil_div(nvec, (int64_t)p.rw * kWave);
  p.nv = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
  return p;
}

template <typename T, bool LN>
int fwd_impl(int64_t T_, int64_t d, const void* x, int64_t ldx, const void* w, const void* b,
             float eps, void* y, int64_t ldy, float* mean, float* rstd, hipStream_t st) {
  const T* xp = static_cast<const T*>(x);
  const T* wp = static_cast<const T*>(w);
  const T* bp = static_cast<const T*>(b);
  T* yp = static_cast<T*>(y);
  const bool aligned = vector_ok<T>(d, x, ldx, y, ldy, x, ldx, w) && (!LN || aligned16(b));
  if (aligned || unaligned_ok<T>(d, {x, y, w, LN ? b : x})) {
    const int nvec = (int)(d / Vec<T>::N);  // full vectors; the rest is the tail (UA)
    const FwdPlan p = fwd_plan(nvec);
    auto go = [&](auto nv_c, auto rw_c, auto ua) {
      constexpr int NV = decltype(nv_c)::value, RW = decltype(rw_c)::value;
      constexpr int NT = fwd_threads(RW);
      const dim3 grid((unsigned)ceil_div(T_, (int64_t)(NT / kWave / RW)));
      rmsnorm_fwd_wave<T, NV, RW, LN, decltype(ua)::value><<<grid, dim3(NT), 0, st>>>(
          T_, nvec, (int)d, xp, ldx, wp, bp, eps, yp, ldy, mean, rstd);
    };
    // a row of one wave takes 1, 2, 4 or kFwdMaxNV vectors per lane; a row of more
    // waves has more than kFwdMaxNV / 2 per lane, so it takes kFwdMaxNV (16 where
    // kMaxRowWaves waves still need more)
    static_assert(kFwdMaxNV == 8, "the one-wave cases below list 1, 2, 4, 8");
    auto go_rw = [&](auto ua) {
      using I = std::integral_constant<int, kFwdMaxNV>;
      using One = std::integral_constant<int, 1>;
      switch (p.rw) {
        case 1:
          switch (p.nv) {
            case 1: go(std::integral_constant<int, 1>{}, One{}, ua); break;
            case 2: go(std::integral_constant<int, 2>{}, One{}, ua); break;
            case 4: go(std::integral_constant<int, 4>{}, One{}, ua); break;
            default: go(I{}, One{}, ua); break;
          }
          break;
        case 2: go(I{}, std::integral_constant<int, 2>{}, ua); break;
        case 4: go(I{}, std::integral_constant<int, 4>{}, ua); break;
        case 8: go(I{}, std::integral_constant<int, 8>{}, ua); break;
        default:
          if (p.nv <= kFwdMaxNV) go(I{}, std::integral_constant<int, 16>{}, ua);
          else go(std::integral_constant<int, 16>{}, std::integral_constant<int, 16>{}, ua);
          break;
      }
    };
    if (aligned) go_rw(std::false_type{});
    else go_rw(std::true_type{});
  } else {
    rmsnorm_fwd_block<T, LN><<<dim3((unsigned)T_), dim3(kGenericThreads), 0, st>>>(
        T_, d, xp, ldx, wp, bp, eps, yp, ldy, mean, rstd);
  }
  return launch_status();
}

// Rows the backward wave kernel holds: at most 16 elements per operand per lane of
// kMaxRowWaves waves.
template <typename T>
bool bwd_fits(int64_t d) {
  return d / Vec<T>::N <= (int64_t)kMaxRowWaves * kWave * (16 / Vec<T>::N);
}

// Upper bound of the dw partial rows of either backward path (workspace sizing).
int64_t bwd_groups(int64_t T_) { return T_ < kMaxPartials ? T_ : kMaxPartials; }

// Launch plan of the fast backward: waves per row (rw), vectors per lane and operand
// (nv), and the workgroup count (= dw partial rows).
struct BwdPlan {
  int rw, nv;
  int64_t groups;
};

template <typename T>
BwdPlan bwd_plan(int64_t T_, int nvec) {
  // fewest waves per row that keep each lane at <= 16 elements per operand
  constexpr int kMaxNV = 16 / Vec<T>::N;
  BwdPlan p{1, 1, 0};
  while (p.rw < kMaxRowWaves && ceil_div(nvec, (int64_t)p.rw * kWave) > kMaxNV) p.rw *= 2;
  const int64_t per = ceil_div(nvec, (int64_t)p.rw * kWave);
  p.nv = per <= 1 ? 1 : per <= 2 ? 2 : kMaxNV;
  const int64_t rows_in_flight = bwd_threads(p.rw) / kWave / p.rw;
  p.groups = ceil_div(T_, rows_in_flight);
  if (p.groups > kMaxPartials) p.groups = kMaxPartials;
  return p;
}

template <typename T, int NV, int RW, bool LN, bool UA>
void launch_bwd(const BwdPlan& p, int64_t T_, int nvec, int d, const T* dy, int64_t lddy,
                const T* x, int64_t ldx, const T* w, const float* mean, const float* rstd,
                float eps, T* dx, int64_t lddx, float* partial, hipStream_t st) {
  // the LDS fold of the row groups' dw partials (none with one row group)
  constexpr int RG = bwd_threads(RW) / kWave / RW;
  const size_t fold = (size_t)(LN ? 2 : 1) * d * sizeof(float);
  // One row group (RG 1) writes its partial row from registers: as 16-byte stores
  // where the row is 16-byte aligned (direct 2); otherwise through the LDS fold, which
  // measured faster than scattered 4-byte stores, or scalar stores (direct 1) past
  // the LDS of a workgroup.
  const bool vec_out = !UA && reinterpret_cast<uintptr_t>(partial) % 16 == 0;
  const int direct = RG != 1 ? 0 : vec_out ? 2 : fold > kMaxLds ? 1 : 0;
  const size_t lds = direct ? 0 : fold;
  rmsnorm_bwd_wave<T, NV, RW, LN, UA>
      <<<dim3((unsigned)p.groups), dim3(bwd_threads(RW)), lds, st>>>(T_, nvec, d, dy, lddy, x, ldx, w, mean, rstd, eps, dx, lddx, partial, direct);
}

// LN: mean and rstd are the forward's saved statistics (required); db receives the
// bias gradient.  RMS: mean and db unused, rstd optional.
template <typename T, bool LN>
int bwd_impl(int64_t T_, int64_t d, const void* dy, int64_t lddy, const void* x,
             int64_t ldx, const void* w, const float* mean, const float* rstd, float eps,
             void* dx, int64_t lddx, float* dw, float* db, void* ws, hipStream_t st) {
  const T* dyp = static_cast<const T*>(dy);
  const T* xp = static_cast<const T*>(x);
  const T* wp = static_cast<const T*>(w);
  T* dxp = static_cast<T*>(dx);
  float* partial = static_cast<float*>(ws);
  constexpr int64_t kCols = LN ? 2 : 1;  // partial row: dw (and db) columns
  int64_t G;
  const bool fits = bwd_fits<T>(d);
  const bool aligned = fits && vector_ok<T>(d, dy, lddy, x, ldx, dx, lddx, w);
  if (aligned || (fits && unaligned_ok<T>(d, {dy, x, dx, w}))) {
    const int nvec = (int)(d / Vec<T>::N);  // full vectors; the rest is the tail (UA)
    const BwdPlan p = bwd_plan<T>(T_, nvec);
    G = p.groups;
    constexpr int kMaxNV = 16 / Vec<T>::N;
    auto go = [&](auto nv_c, auto rw_c, auto ua) {
      launch_bwd<T, decltype(nv_c)::value, decltype(rw_c)::value, LN, decltype(ua)::value>(
          p, T_, nvec, (int)d, dyp, lddy, xp, ldx, wp, mean, rstd, eps, dxp, lddx, partial, st);
    };
    auto go_nv = [&](auto rw_c, auto ua) {
      if (p.nv == 1) go(std::integral_constant<int, 1>{}, rw_c, ua);
      else if (p.nv == 2 || kMaxNV == 2) go(std::integral_constant<int, 2>{}, rw_c, ua);
      else go(std::integral_constant<int, kMaxNV>{}, rw_c, ua);
    };
    auto go_rw = [&](auto ua) {
      switch (p.rw) {
        case 1: go_nv(std::integral_constant<int, 1>{}, ua); break;
        case 2: go_nv(std::integral_constant<int, 2>{}, ua); break;
        case 4: go_nv(std::integral_constant<int, 4>{}, ua); break;
        case 8: go_nv(std::integral_constant<int, 8>{}, ua); break;
        default: go_nv(std::integral_constant<int, 16>{}, ua); break;
      }
    };
    if (aligned) go_rw(std::false_type{});
    else go_rw(std::true_type{});
  } else {
    // RMS: r[t] after the partials in the workspace; LN uses the saved rstd
    G = bwd_groups(T_);
    float* r = partial + align_up((size_t)G * (size_t)(kCols * d), 64);
    rmsnorm_bwd_dx_block<T, LN><<<dim3((unsigned)T_), dim3(kGenericThreads), 0, st>>>(
        T_, d, dyp, lddy, xp, ldx, wp, mean, rstd, eps, dxp, lddx, r);
    const int64_t rows_per_group = ceil_div(T_, G);
    G = ceil_div(T_, rows_per_group);
    rmsnorm_dw_partial_block<T, LN><<<dim3((unsigned)ceil_div(d, 256), (unsigned)G), dim3(256), 0, st>>>(
        T_, d, dyp, lddy, xp, ldx, mean, LN ? rstd : r, rows_per_group, partial);
  }
  rmsnorm_dw_reduce<<<dim3((unsigned)ceil_div(kCols * d, kReduceCols)), dim3(256), 0, st>>>(
      G, kCols * d, kCols * d, partial, dw, d, db);
  return launch_status();
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" size_t fo_rmsnorm_bwd_workspace(int64_t T, int64_t d) {
  if (T < 0 || d < 1) return 0;
  const int64_t G = T > 0 ? bwd_groups(T) : 1;
  return (align_up((size_t)G * (size_t)d, 64) + (size_t)T) * sizeof(float) + 256;
}

extern "C" int fo_rmsnorm_fwd(int dtype, int64_t T, int64_t d, const void* x, int64_t ldx,
                              const void* w, float eps, void* y, int64_t ldy, float* rstd,
                              void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || d < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (ldx < d || ldy < d) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!x || !w || !y) return FO_ERR_NULL;
  hipStream_t st = as_stream(stream);
  return dtype == FO_F32
             ? fwd_impl<float, false>(T, d, x, ldx, w, nullptr, eps, y, ldy, nullptr, rstd, st)
             : fwd_impl<bf16, false>(T, d, x, ldx, w, nullptr, eps, y, ldy, nullptr, rstd, st);
}

extern "C" int fo_rmsnorm_bwd(int dtype, int64_t T, int64_t d, const void* dy, int64_t lddy,
                              const void* x, int64_t ldx, const void* w, const float* rstd,
                              float eps, void* dx, int64_t lddx, float* dw, void* ws,
                              size_t ws_bytes, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || d < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (lddy < d || ldx < d || lddx < d) return FO_ERR_STRIDE;
  if (!dw) return FO_ERR_NULL;
  hipStream_t st = as_stream(stream);
  if (T == 0) {
    fill_f32<<<dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st>>>(dw, d, 0.f);
    return launch_status();
  }
  if (!dy || !x || !w || !dx) return FO_ERR_NULL;
  if (!ws || ws_bytes < fo_rmsnorm_bwd_workspace(T, d)) return FO_ERR_WORKSPACE;
  return dtype == FO_F32
             ? bwd_impl<float, false>(T, d, dy, lddy, x, ldx, w, nullptr, rstd, eps, dx, lddx, dw,
                                      nullptr, ws, st)
             : bwd_impl<bf16, false>(T, d, dy, lddy, x, ldx, w, nullptr, rstd, eps, dx, lddx, dw,
                                     nullptr, ws, st);
}

extern "C" int fo_layernorm_fwd(int dtype, int64_t T, int64_t d, const void* x, int64_t ldx,
                                const void* w, const void* b, float eps, void* y, int64_t ldy,
                                float* mean, float* rstd, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || d < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (ldx < d || ldy < d) return FO_ERR_STRIDE;
  if (T == 0) return FO_OK;
  if (!x || !w || !b || !y) return FO_ERR_NULL;
  hipStream_t st = as_stream(stream);
  return dtype == FO_F32 ? fwd_impl<float, true>(T, d, x, ldx, w, b, eps, y, ldy, mean, rstd, st)
                         : fwd_impl<bf16, true>(T, d, x, ldx, w, b, eps, y, ldy, mean, rstd, st);
}

extern "C" size_t fo_layernorm_bwd_workspace(int64_t T, int64_t d) {
  if (T < 0 || d < 1) return 0;
  const int64_t G = T > 0 ? bwd_groups(T) : 1;
  return align_up((size_t)G * (size_t)(2 * d), 64) * sizeof(float) + 256;
}

extern "C" int fo_layernorm_bwd(int dtype, int64_t T, int64_t d, const void* dy, int64_t lddy,
                                const void* x, int64_t ldx, const void* w, const float* mean,
                                const float* rstd, void* dx, int64_t lddx, float* dw, float* db,
                                void* ws, size_t ws_bytes, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || d < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (lddy < d || ldx < d || lddx < d) return FO_ERR_STRIDE;
  if (!dw || !db) return FO_ERR_NULL;
  hipStream_t st = as_stream(stream);
  if (T == 0) {
    fill_f32<<<dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st>>>(dw, d, 0.f);
    fill_f32<<<dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, st>>>(db, d, 0.f);
    return launch_status();
  }
  if (!dy || !x || !w || !dx || !mean || !rstd) return FO_ERR_NULL;
  if (!ws || ws_bytes < fo_layernorm_bwd_workspace(T, d)) return FO_ERR_WORKSPACE;
  return dtype == FO_F32
             ? bwd_impl<float, true>(T, d, dy, lddy, x, ldx, w, mean, rstd, 0.f, dx, lddx, dw, db,
                                     ws, st)
             : bwd_impl<bf16, true>(T, d, dy, lddy, x, ldx, w, mean, rstd, 0.f, dx, lddx, dw, db,
                                    ws, st);
}
