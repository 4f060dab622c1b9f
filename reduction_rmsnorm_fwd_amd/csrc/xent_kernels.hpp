// Cross-entropy row kernels (forward + backward in one sweep), shared by the
// cross-entropy entry point and the fused linear cross-entropy chunk loop.
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构, 损失函数体系: cross-entropy
// and a z-loss regulariser against over-confidence; the Triton kernel list of 整体框架结构
// names entropy_loss and z_loss; the Liger section of "Kernels（自定义内核）" fuses
// CrossEntropy).  For a valid row t with target y:
//   lse = log sum_j exp(z_j),  loss_t = lse - z_y + c lse^2,
//   dz_j = (dloss/N) (softmax_j (1 + 2 c lse) - [j == y])
// Invalid rows (ignore_index or a target outside [0,V)) contribute no loss and get an
// all +0.0 gradient row.  N, the number of valid rows, is counted by a first tiny
// kernel so that the row kernel can scale the gradient in the same sweep.
//
// Row kernel, register-resident form: one workgroup per row; every thread loads its
// NV 16-byte vectors of the row into registers, folding each into a running
// (max, sum of exp) pair as it arrives (online logsumexp); the pairs are merged across
// the workgroup in a fixed order; the gradient is then formed from the registers and
// written.  The row is read from HBM once, also when it starts off the 16-byte grid or
// its length is not a multiple of the vector (full vectors are still 16-byte accesses).
// Rows up to 8 vectors per thread longer than the registers hold keep the rest in LDS
// (still one read); longer rows take the streaming form, which makes the same online
// pass and then reads the row a second time for the gradient.
#pragma once

#include <type_traits>

#include "fo_common.hpp"

namespace fo {
namespace xent {
namespace {  // internal linkage: each including source file gets its own copy

struct Counters {
  long long n_valid;
  int n_bad;
  int pad;
};

__device__ __forceinline__ bool row_valid(long long y, long long V, long long ignore) {
  return y != ignore && y >= 0 && y < V;
}

template <typename T> __device__ __forceinline__ float ex(float x);
// fp32 inputs keep the accurate exponential (fp32 parity is checked at 1e-5);
// bf16 inputs use the hardware exp2 path.
template <> __device__ __forceinline__ float ex<float>(float x) { return expf(x); }
template <> __device__ __forceinline__ float ex<bf16>(float x) { return __expf(x); }

// exp(x - m) inside a row sweep, with nb = nl2e<T>(m) formed once per shift m.  bf16
// rows: 2^(x log2 e - m log2 e) as one fused multiply-add into the hardware 2^x, where
// __expf(x - m) takes a subtraction, a multiplication and the same 2^x (one VALU
// operation less per element and pass; the shift's rounding, |m| log2(e) 2^-24, stays
// far below a bf16 step).  fp32 rows keep expf(x - m).
constexpr float kLog2e = 1.4426950408889634f;
template <typename T> __device__ __forceinline__ float nl2e(float m) {
  return std::is_same<T, bf16>::value ? -m * kLog2e : m;
}
template <typename T> __device__ __forceinline__ float exs(float x, float nb);
template <> __device__ __forceinline__ float exs<float>(float x, float m) { return expf(x - m); }
template <> __device__ __forceinline__ float exs<bf16>(float x, float nb) {
  return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, nb));
}

// Count valid and bad targets of rows [0, T).  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void count_targets(int64_t T_, int64_t V,
                                                      const int64_t* __restrict__ tg,
                                                      int64_t ignore, Counters* cnt) {
  __shared__ long long sv[16], sb[16];
  long long nv = 0, nb = 0;
  for (int64_t t = threadIdx.x; t < T_; t += 1024) {
    const long long y = tg[t];
    nv += row_valid(y, V, ignore);
    nb += (y != ignore) && (y < 0 || y >= V);
  }
  nv = wave_sum_i64(nv);
  nb = wave_sum_i64(nb);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) { sv[w] = nv; sb[w] = nb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long a = 0, b = 0;
    for (int i = 0; i < 16; ++i) { a += sv[i]; b += sb[i]; }
    cnt->n_valid = a;
    cnt->n_bad = (int)b;
    cnt->pad = 0;
  }
}

// Valid rows in order: idx[j] = the j-th valid row, pos_of[t] = its j (or -1),
// tg_valid[j] = its target; also the counters.  One workgroup of 1024 threads walks T
// in blocks with a ballot/popcount prefix scan (deterministic).
__global__ __launch_bounds__(1024) void compact_targets(int64_t T_, int64_t V,
                                                        const int64_t* __restrict__ tg,
                                                        int64_t ignore, Counters* cnt,
                                                        int* __restrict__ idx,
                                                        int* __restrict__ pos_of,
                                                        int64_t* __restrict__ tg_valid) {
  __shared__ int wsum[16];
  __shared__ long long sb[16];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  long long base = 0, nb = 0;
  for (int64_t b0 = 0; b0 < T_; b0 += 1024) {
    const int64_t t = b0 + threadIdx.x;
    const long long y = t < T_ ? tg[t] : ignore;
    const bool v = t < T_ && row_valid(y, V, ignore);
    nb += (t < T_) && (y != ignore) && (y < 0 || y >= V);
    const unsigned long long bal = __ballot(v);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < 16; ++i) {
      off += (i < w) ? wsum[i] : 0;
      tot += wsum[i];
    }
    if (t < T_) {
      const int p = v ? (int)(base + off + pre) : -1;
      pos_of[t] = p;
      if (v) {
        idx[p] = (int)t;
        tg_valid[p] = y;
      }
    }
    base += tot;
    __syncthreads();  // wsum is rewritten next block
  }
  nb = wave_sum_i64(nb);
  if (lane == 0) sb[w] = nb;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long b = 0;
    for (int i = 0; i < 16; ++i) b += sb[i];
    cnt->n_valid = base;
    cnt->n_bad = (int)b;
    cnt->pad = 0;
  }
}

// Fixed-order merge of the per-wave (m, s) pairs: every thread gets the same lse.
template <int NT>
__device__ __forceinline__ float block_lse(float m, float s, float* shm, float* shs) {
  wave_lse(m, s);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) { shm[w] = m; shs[w] = s; }
  __syncthreads();
  float M = shm[0], S = shs[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) lse_merge(M, S, shm[i], shs[i]);
  return M + __logf(S);
}

// Writes one all-zero gradient row.
template <typename Tout, int VEC, int NT>
__device__ __forceinline__ void zero_row(Tout* dr, int64_t nvec) {
  if constexpr (VEC > 1) {
    Pack<Tout> z;
    z.raw = u32x4{0, 0, 0, 0};
    for (int64_t v = threadIdx.x; v < nvec; v += NT) store_pack(dr + v * VEC, z);
  } else {
    for (int64_t v = threadIdx.x; v < nvec; v += NT) dr[v] = from_f32<Tout>(0.f);
  }
}

struct RowArgs {
  int64_t T, V;
  int64_t ldz, ldd;
  int64_t ignore;
  float zc, dloss;
  const int64_t* tg;
  const Counters* cnt;
  float* row_loss;  // [T] loss_t (0 for invalid rows)
  float* row_z;     // [T] c lse^2 (0 for invalid rows)
};

// Vector v of a row of n elements.  UA (rows of any element alignment and length): a
// full vector is one 16-byte load at its element-aligned address (gfx950 serves global
// memory in unaligned mode), the last, partial vector is read element by element and
// padded with -inf, which drops out of the maximum and the sum of exponentials.
template <typename T, bool UA>
__device__ __forceinline__ Pack<T> row_vec(const T* p, int64_t v, int64_t n) {
  constexpr int VEC = Vec<T>::N;
  if (!UA || (v + 1) * VEC <= n) return load_pack(p + v * VEC);
  Pack<T> r;
#pragma unroll
  for (int j = 0; j < VEC; ++j) r.v[j] = v * VEC + j < n ? p[v * VEC + j] : from_f32<T>(-INFINITY);
  return r;
}

// Register-resident row kernel.  Requires nvec <= NT*NV and, unless UA, V % VEC == 0 and
// 16-byte aligned rows.  UA: rows of any element alignment and length (same element
// type in and out): full vectors are still 16-byte accesses, the partial last vector of
// each row goes element by element, so no access touches a neighbouring row.
template <typename Tin, typename Tout, int NV, int NT, bool UA = false>
__global__ __launch_bounds__(NT) void row_reg(RowArgs a, const Tin* z, Tout* dz) {
  constexpr int VEC = Vec<Tin>::N;
  static_assert(Vec<Tout>::N == VEC || Vec<Tout>::N == 2 * VEC, "vector widths");
  static_assert(!UA || Vec<Tout>::N == VEC, "unaligned rows: one element type");
  __shared__ float shm[NT / kWave], shs[NT / kWave];
  __shared__ float sh_zy;
  const int64_t row = blockIdx.x;
  const long long y = a.tg[row];
  const int64_t nvec = UA ? ceil_div(a.V, (int64_t)VEC) : a.V / VEC;
  if (!row_valid(y, a.V, a.ignore)) {
    if (dz != nullptr) {
      Tout* dr = dz + row * a.ldd;
      if constexpr (UA) {
        zero_row<Tout, VEC, NT>(dr, a.V / VEC);
        for (int64_t e = a.V / VEC * VEC + threadIdx.x; e < a.V; e += NT) dr[e] = from_f32<Tout>(0.f);
      } else if constexpr (Vec<Tout>::N == VEC) {
        zero_row<Tout, VEC, NT>(dr, nvec);
      } else {
        for (int64_t e = threadIdx.x; e < a.V; e += NT) dr[e] = from_f32<Tout>(0.f);
      }
    }
    if (threadIdx.x == 0) { a.row_loss[row] = 0.f; a.row_z[row] = 0.f; }
    return;
  }
  const Tin* zr = z + row * a.ldz;
  if (threadIdx.x == 0) sh_zy = to_f32(zr[y]);  // read before any gradient write
  Pack<Tin> xv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t v = threadIdx.x + (int64_t)i * NT;
    if (v < nvec) xv[i] = row_vec<Tin, UA>(zr, v, a.V);
  }
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t v = threadIdx.x + (int64_t)i * NT;
    if (v < nvec) {
      float vm = to_f32(xv[i].v[0]);
#pragma unroll
      for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, to_f32(xv[i].v[j]));
      if (vm > m) { s *= ex<Tin>(m - vm); m = vm; }
      const float nb = nl2e<Tin>(m);
#pragma unroll
      for (int j = 0; j < VEC; ++j) s += exs<Tin>(to_f32(xv[i].v[j]), nb);
    }
  }
  const float lse = block_lse<NT>(m, s, shm, shs);
  if (threadIdx.x == 0) {
    const float zt = a.zc * lse * lse;
    a.row_loss[row] = (lse - sh_zy) + zt;
    a.row_z[row] = zt;
  }
  if (dz == nullptr) return;
  const float scale = a.dloss / (float)a.cnt->n_valid;
  const float coef = scale * fmaf(2.f * a.zc, lse, 1.f);
  Tout* dr = dz + row * a.ldd;
  // Keep the row in its packed 16-byte form between the passes (re-widen it below)
  // instead of letting the compiler hold widened fp32 copies: half the registers.
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(xv[i].raw));
  const int64_t yv = y / VEC;          // the vector holding the target
  const int yj = (int)(y - yv * VEC);  // and its element
  const float nl = nl2e<Tin>(lse);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t v = threadIdx.x + (int64_t)i * NT;
    if (v < nvec) {
      float g[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) g[j] = coef * exs<Tin>(to_f32(xv[i].v[j]), nl);
      if (v == yv) {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
          if (j == yj) g[j] -= scale;
      }
      if constexpr (Vec<Tout>::N == VEC) {
        Pack<Tout> o;
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.v[j] = from_f32<Tout>(g[j]);
        if (!UA || (v + 1) * VEC <= a.V) {
          store_pack(dr + v * VEC, o);
        } else {
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            if (v * VEC + j < a.V) dr[v * VEC + j] = o.v[j];
        }
      } else {
        // fp32 in, bf16 out: VEC outputs fill half a 16-byte vector
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        union { u32x2 raw; Tout e[VEC]; } o;
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.e[j] = from_f32<Tout>(g[j]);
        __builtin_nontemporal_store(o.raw, reinterpret_cast<u32x2*>(dr + v * VEC));
      }
    }
  }
}

// Persistent prefetching row kernel (register-resident rows of NV vectors per thread,
// 1024 threads).  A workgroup per CU walks the rows blockIdx.x, +gridDim.x, ...  The
// first NL vectors of each thread's share of the NEXT row are copied into LDS by
// buffer_load ... lds while the current row is reduced and written, so the CU keeps
// reads in flight through its compute and store phases (one row per CU in registers
// leaves no room to overlap two rows otherwise).  Per row:
//   1. issue the loads of vectors NL..NV-1 (into registers)
//   2. wait for every outstanding access (this row's LDS copy, the previous row's
//      stores, step 1), barrier, read the LDS copy into registers, barrier
//   3. issue the LDS copy of the next row (an empty buffer range for an ignored or
//      missing row: no memory traffic)
//   4. online (max, sum) over the row, workgroup merge, loss, gradient, stores.
// Vector i of thread t is row vector t + i*1024 in both the LDS copy and the
// registers, so every LDS access is 16 consecutive bytes per lane.  The targets of a
// workgroup's rows are staged in LDS kTgCache at a time, so no target load sits
// between the prefetch and its use.
typedef __attribute__((address_space(3))) void* lds_vptr;
constexpr int kPfThreads = 1024;
constexpr int kTgCache = 1024;

// cache policy of a buffer load: non-temporal (the row is read once; T 8192, V 128256:
// 817 -> 782 us against plain buffer loads, V 151936 at T 4096: 519 -> 489 us)
constexpr int kNtAux = 2;

template <int N>
__device__ __forceinline__ void wait_vm_n() {
  // s_waitcnt with only vmcnt constrained (6-bit count: bits 3:0 and 15:14)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename Tin, typename Tout, int NV, int NL>
__global__ __launch_bounds__(kPfThreads) void row_pf(RowArgs a, const Tin* z, Tout* dz) {
  constexpr int NT = kPfThreads;
  constexpr int VEC = Vec<Tin>::N;
  constexpr int kFlags = 0x00020000;  // raw buffer, 32-bit data format
  static_assert(NL > 0 && NL < NV, "split");
  static_assert(Vec<Tout>::N == VEC, "same element width in and out");
  __shared__ __attribute__((aligned(16))) u32x4 stage[NL * NT];
  __shared__ long long tgc[kTgCache];
  __shared__ float shm[NT / kWave], shs[NT / kWave];
  __shared__ float sh_zy;
  const int wave = threadIdx.x / kWave;
  const int nvec = (int)(a.V / VEC);
  const int64_t G = gridDim.x;
  const int row_bytes = (int)(a.V * (int64_t)sizeof(Tin));
  // target of this workgroup's k-th row (k within the cached batch)
  auto load_targets = [&](int64_t k0) {
    __syncthreads();
    for (int t = threadIdx.x; t < kTgCache; t += NT) {
      const int64_t r = blockIdx.x + (k0 + t) * G;
      tgc[t] = r < a.T ? a.tg[r] : a.ignore;
    }
    __syncthreads();
  };
  auto live_row = [&](int64_t r, long long y) { return r < a.T && row_valid(y, a.V, a.ignore); };
  // the buffer over row r's logits, or an empty one (ignored row, past the end)
  auto row_rsrc = [&](int64_t r, bool live) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(z + (live ? r : 0) * a.ldz), (short)0,
                                             live ? row_bytes : 0, kFlags);
  };
  auto stage_row = [&](int64_t r, bool live) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(r, live);
    // lane offset in a VGPR, the vector index's offset in an SGPR
    const uint32_t voff = threadIdx.x * 16u;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(stage + i * NT + wave * kWave), 16,
                                               voff, i * NT * 16, 0, kNtAux);
  };
  // a target read from LDS is the same in every lane: keep it in scalar registers
  auto uniform = [](long long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
  };
  load_targets(0);
  stage_row(blockIdx.x, live_row(blockIdx.x, uniform(tgc[0])));
  int64_t k = 0;  // index of `row` in this workgroup's sequence
  for (int64_t row = blockIdx.x; row < a.T; row += G, ++k) {
    if (k % kTgCache == 0 && k > 0) load_targets(k);
    const long long y = uniform(tgc[k % kTgCache]);
    const bool valid = row_valid(y, a.V, a.ignore);
    // 1. the register part of the row (an empty buffer when the row is ignored)
    Pack<Tin> xv[NV];
    {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, valid);
      const uint32_t voff = threadIdx.x * 16u;
#pragma unroll
      for (int i = NL; i < NV; ++i)
        xv[i].raw = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * NT * 16, kNtAux));
    }
    // 2. all of it has landed (the LDS copy was issued one row ago)
    wait_vm_n<0>();
    __syncthreads();
    // (the lane index is made opaque once per row, so the compiler recomputes the
    // per-vector addresses and indices from it instead of holding dozens of them
    // across the loop: no spills)
    int tix = (int)threadIdx.x;
    asm volatile("" : "+v"(tix));
    if (valid) {
#pragma unroll
      for (int i = 0; i < NL; ++i) xv[i].raw = stage[i * NT + tix];
    }
    __syncthreads();
    // 3. the next row's LDS copy overlaps this row's reduction and stores
    {
      const int64_t kn = k + 1;
      const long long yn = uniform(kn % kTgCache == 0
                                       ? (row + G < a.T ? a.tg[row + G] : a.ignore)
                                       : tgc[kn % kTgCache]);
      stage_row(row + G, live_row(row + G, yn));
    }
    Tout* dr = dz != nullptr ? dz + row * a.ldd : nullptr;
    if (!valid) {
      if (dr != nullptr) zero_row<Tout, VEC, NT>(dr, nvec);
      if (threadIdx.x == 0) { a.row_loss[row] = 0.f; a.row_z[row] = 0.f; }
      continue;
    }
    // 4. as the register-resident kernel; the target logit comes from the registers of
    //    the thread that holds it
    const int yv = (int)(y / VEC);
    const int yj = (int)(y - (long long)yv * VEC);
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tix + i * NT;
      if (v < nvec) {
        if (v == yv) {
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            if (j == yj) sh_zy = to_f32(xv[i].v[j]);
        }
        float vm = to_f32(xv[i].v[0]);
#pragma unroll
        for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, to_f32(xv[i].v[j]));
        if (vm > m) { s *= ex<Tin>(m - vm); m = vm; }
        const float nb = nl2e<Tin>(m);
#pragma unroll
        for (int j = 0; j < VEC; ++j) s += exs<Tin>(to_f32(xv[i].v[j]), nb);
      }
    }
    const float lse = block_lse<NT>(m, s, shm, shs);  // (its barrier publishes sh_zy)
    if (threadIdx.x == 0) {
      const float zt = a.zc * lse * lse;
      a.row_loss[row] = (lse - sh_zy) + zt;
      a.row_z[row] = zt;
    }
    if (dr == nullptr) continue;
    const float scale = a.dloss / (float)a.cnt->n_valid;
    const float coef = scale * fmaf(2.f * a.zc, lse, 1.f);
    const float nl = nl2e<Tin>(lse);
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(xv[i].raw));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tix + i * NT;
      if (v < nvec) {
        float g[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) g[j] = coef * exs<Tin>(to_f32(xv[i].v[j]), nl);
        if (v == yv) {
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            if (j == yj) g[j] -= scale;
        }
        Pack<Tout> o;
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.v[j] = from_f32<Tout>(g[j]);
        store_pack(dr + (int64_t)v * VEC, o);
      }
    }
  }
  // the last LDS copy (an empty range unless the grid is cut short) lands before exit
  wait_vm_n<0>();
}

// Register-resident row kernel with an LDS extension, for rows of 16 + NS vectors per
// thread (1024 threads; bf16 V up to 163840 with NS 4, 196608 with NS 8): vectors
// t + i*1024 of thread t sit in registers for i < NV and in LDS for NV <= i < NV + NS,
// so the row is read from HBM once.  The LDS part is copied by buffer_load ... lds into
// the thread's own 16-byte slots (slot i*1024 + t, 16 consecutive bytes per lane) and
// read back by the same lane after its wave's loads have landed, so no barrier orders
// it.  Requires V % VEC == 0 and 16-byte aligned rows; the whole byte offset of a
// vector goes in the lane's offset register, so the buffer's range check (the row's
// bytes) returns zeros for vectors past the row, which are skipped.
template <typename Tin, typename Tout, int NV, int NS>
__global__ __launch_bounds__(1024) void row_ls(RowArgs a, const Tin* z, Tout* dz) {
  constexpr int NT = 1024;
  constexpr int VEC = Vec<Tin>::N;
  constexpr int kFlags = 0x00020000;  // raw buffer, 32-bit data format
  static_assert(Vec<Tout>::N == VEC, "same element width in and out");
  __shared__ __attribute__((aligned(16))) u32x4 ext[NS * NT];
  __shared__ float shm[NT / kWave], shs[NT / kWave];
  __shared__ float sh_zy;
  const int64_t row = blockIdx.x;
  const long long y = a.tg[row];
  const int64_t nvec = a.V / VEC;
  if (!row_valid(y, a.V, a.ignore)) {
    if (dz != nullptr) zero_row<Tout, VEC, NT>(dz + row * a.ldd, nvec);
    if (threadIdx.x == 0) { a.row_loss[row] = 0.f; a.row_z[row] = 0.f; }
    return;
  }
  const Tin* zr = z + row * a.ldz;
  if (threadIdx.x == 0) sh_zy = to_f32(zr[y]);  // read before any gradient write
  const int wave = threadIdx.x / kWave;
  {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)zr, (short)0, (int)(a.V * (int64_t)sizeof(Tin)), kFlags);
#pragma unroll
    for (int i = 0; i < NS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(ext + i * NT + wave * kWave), 16,
                                               (threadIdx.x + (uint32_t)(NV + i) * NT) * 16u, 0, 0, kNtAux);
  }
  Pack<Tin> xv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t v = threadIdx.x + (int64_t)i * NT;
    if (v < nvec) xv[i] = load_pack(zr + v * VEC);
  }
  float m = -INFINITY, s = 0.f;
  auto fold = [&](const Pack<Tin>& p) {
    float vm = to_f32(p.v[0]);
#pragma unroll
    for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, to_f32(p.v[j]));
    if (vm > m) { s *= ex<Tin>(m - vm); m = vm; }
    const float nb = nl2e<Tin>(m);
#pragma unroll
    for (int j = 0; j < VEC; ++j) s += exs<Tin>(to_f32(p.v[j]), nb);
  };
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (threadIdx.x + (int64_t)i * NT < nvec) fold(xv[i]);
  wait_vm_n<0>();  // this wave's LDS copies have landed
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (threadIdx.x + (int64_t)(NV + i) * NT < nvec) {
      Pack<Tin> p;
      p.raw = ext[i * NT + threadIdx.x];
      fold(p);
    }
  }
  const float lse = block_lse<NT>(m, s, shm, shs);
  if (threadIdx.x == 0) {
    const float zt = a.zc * lse * lse;
    a.row_loss[row] = (lse - sh_zy) + zt;
    a.row_z[row] = zt;
  }
  if (dz == nullptr) return;
  const float scale = a.dloss / (float)a.cnt->n_valid;
  const float coef = scale * fmaf(2.f * a.zc, lse, 1.f);
  Tout* dr = dz + row * a.ldd;
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(xv[i].raw));
  const int64_t yv = y / VEC;
  const int yj = (int)(y - yv * VEC);
  const float nl = nl2e<Tin>(lse);
  auto grad = [&](const Pack<Tin>& p, int64_t v) {
    float g[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) g[j] = coef * exs<Tin>(to_f32(p.v[j]), nl);
    if (v == yv) {
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        if (j == yj) g[j] -= scale;
    }
    Pack<Tout> o;
#pragma unroll
    for (int j = 0; j < VEC; ++j) o.v[j] = from_f32<Tout>(g[j]);
    store_pack(dr + v * VEC, o);
  };
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t v = threadIdx.x + (int64_t)i * NT;
    if (v < nvec) grad(xv[i], v);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int64_t v = threadIdx.x + (int64_t)(NV + i) * NT;
    if (v < nvec) {
      Pack<Tin> p;
      p.raw = ext[i * NT + threadIdx.x];
      grad(p, v);
    }
  }
}

// Streaming row kernel: any V, any alignment (VEC = 1) or aligned vectors (VEC > 1), for
// rows longer than the register-resident kernels hold.  With vectors, each thread keeps
// its first KEEP vectors of the row in registers from the first pass to the second (as
// the register-resident kernel does with the whole row) and streams the rest twice:
// the first pass (plain loads) gives (max, sum), the second, served mostly by L2 and
// the Infinity Cache, re-reads only that rest to write its gradient; loads of values read
// once (the kept vectors, the second pass) are non-temporal.  Streamed vectors
// are loaded kStreamUnroll at a time before any is used, so a wave keeps that many
// 16-byte loads in flight, and every gradient vector goes out as one 16-byte store.
constexpr int kStreamUnroll = 8;

template <typename Tin, typename Tout, int VEC, int NT, int KEEP = 0, int U = kStreamUnroll>
__global__ __launch_bounds__(NT) void row_stream(RowArgs a, const Tin* z, Tout* dz) {
  static_assert(KEEP == 0 || VEC > 1, "registers hold whole vectors");
  __shared__ float shm[NT / kWave], shs[NT / kWave];
  __shared__ float sh_zy;
  const int64_t row = blockIdx.x;
  const long long y = a.tg[row];
  if (!row_valid(y, a.V, a.ignore)) {
    if (dz != nullptr) {
      Tout* dr = dz + row * a.ldd;
      for (int64_t e = threadIdx.x; e < a.V; e += NT) dr[e] = from_f32<Tout>(0.f);
    }
    if (threadIdx.x == 0) { a.row_loss[row] = 0.f; a.row_z[row] = 0.f; }
    return;
  }
  const Tin* zr = z + row * a.ldz;
  const int64_t nvec = a.V / VEC;  // VEC divides V on this path
  if (threadIdx.x == 0) sh_zy = to_f32(zr[y]);
  float m = -INFINITY, s = 0.f;
  constexpr int KR = KEEP > 0 ? KEEP : 1;
  Pack<Tin> kept[KR];  // vectors threadIdx.x + i*NT, i < KEEP
  auto fold = [&](const Pack<Tin>& p) {
    float vm = to_f32(p.v[0]);
#pragma unroll
    for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, to_f32(p.v[j]));
    if (vm > m) { s *= ex<Tin>(m - vm); m = vm; }
    const float nb = nl2e<Tin>(m);
#pragma unroll
    for (int j = 0; j < VEC; ++j) s += exs<Tin>(to_f32(p.v[j]), nb);
  };
  const int64_t tail0 = threadIdx.x + (int64_t)KEEP * NT;  // first streamed vector
  if constexpr (VEC > 1) {
    if constexpr (KEEP > 0) {
#pragma unroll
      for (int i = 0; i < KEEP; ++i)
        if (threadIdx.x + i * NT < nvec) kept[i] = load_pack(zr + (threadIdx.x + i * NT) * VEC);
#pragma unroll
      for (int i = 0; i < KEEP; ++i)
        if (threadIdx.x + i * NT < nvec) fold(kept[i]);
    }
    for (int64_t v0 = tail0; v0 < nvec; v0 += (int64_t)U * NT) {
      Pack<Tin> p[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (v0 + u * NT < nvec) p[u] = load_pack_cached(zr + (v0 + u * NT) * VEC);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (v0 + u * NT < nvec) fold(p[u]);
    }
  } else {
    for (int64_t v = threadIdx.x; v < nvec; v += NT) {
      const float x = to_f32(zr[v]);
      if (x > m) { s *= ex<Tin>(m - x); m = x; }
      s += ex<Tin>(x - m);
    }
  }
  const float lse = block_lse<NT>(m, s, shm, shs);
  if (threadIdx.x == 0) {
    const float zt = a.zc * lse * lse;
    a.row_loss[row] = (lse - sh_zy) + zt;
    a.row_z[row] = zt;
  }
  if (dz == nullptr) return;
  // In place (dz == z): every element below is read by the thread that then
  // overwrites it, and the barrier in block_lse separates all first-pass reads.
  const float scale = a.dloss / (float)a.cnt->n_valid;
  const float coef = scale * fmaf(2.f * a.zc, lse, 1.f);
  Tout* dr = dz + row * a.ldd;
  if constexpr (VEC > 1) {
    const float nl = nl2e<Tin>(lse);
    auto grad = [&](const Pack<Tin>& p, int64_t v) {
      float g[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        g[j] = coef * exs<Tin>(to_f32(p.v[j]), nl);
        if (v * VEC + j == y) g[j] -= scale;
      }
      if constexpr (Vec<Tout>::N == VEC) {
        Pack<Tout> o;
#pragma unroll
        for (int j = 0; j < VEC; ++j) o.v[j] = from_f32<Tout>(g[j]);
        store_pack(dr + v * VEC, o);
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) dr[v * VEC + j] = from_f32<Tout>(g[j]);
      }
    };
    for (int64_t v0 = tail0; v0 < nvec; v0 += (int64_t)U * NT) {
      Pack<Tin> p[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (v0 + u * NT < nvec) p[u] = load_pack(zr + (v0 + u * NT) * VEC);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (v0 + u * NT < nvec) grad(p[u], v0 + u * NT);
    }
    if constexpr (KEEP > 0) {
#pragma unroll
      for (int i = 0; i < KEEP; ++i)
        if (threadIdx.x + i * NT < nvec) grad(kept[i], threadIdx.x + i * NT);
    }
  } else {
    for (int64_t v = threadIdx.x; v < nvec; v += NT) {
      float g = coef * ex<Tin>(to_f32(zr[v]) - lse);
      if (v == y) g -= scale;
      dr[v] = from_f32<Tout>(g);
    }
  }
}

// loss = sum_t row_loss / N, z_loss = sum_t row_z / N (fp64, fixed order); also
// publishes n_valid and the bad-target count.
// compacted: the per-row arrays hold the valid rows first; only those are summed.
__global__ __launch_bounds__(1024) void finalize(int64_t T_, const float* __restrict__ row_loss,
                                                 const float* __restrict__ row_z,
                                                 const Counters* __restrict__ cnt, float* loss,
                                                 float* z_loss, int64_t* n_valid,
                                                 int32_t* status, int compacted = 0) {
  __shared__ double s1[16], s2[16];
  double a = 0.0, b = 0.0;
  if (compacted && cnt->n_valid < T_) T_ = cnt->n_valid;
  for (int64_t t = threadIdx.x; t < T_; t += 1024) {
    a += (double)row_loss[t];
    b += (double)row_z[t];
  }
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) { s1[w] = a; s2[w] = b; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double A = 0.0, B = 0.0;
    for (int i = 0; i < 16; ++i) { A += s1[i]; B += s2[i]; }
    const long long n = cnt->n_valid;
    *loss = n > 0 ? (float)(A / (double)n) : 0.f;
    if (z_loss) *z_loss = n > 0 ? (float)(B / (double)n) : 0.f;
    if (n_valid) *n_valid = n;
    if (status) *status = cnt->n_bad;
  }
}

// Chooses and launches the row kernel for rows [0, a.T) of z/dz.
constexpr int kPfStage = 9;  // vectors per thread staged in LDS (144 KB)

template <typename Tin, typename Tout>
hipError_t launch_rows(const RowArgs& a, const Tin* z, Tout* dz, hipStream_t st,
                       int64_t n_cu) {
  constexpr int VEC = Vec<Tin>::N;
  const bool vec = a.V % VEC == 0 && a.ldz % VEC == 0 && aligned16(z) &&
                   (dz == nullptr || (a.ldd % VEC == 0 && aligned16(dz)));
  // otherwise: element-aligned rows of one element type that fit the registers
  const bool ua_ok = std::is_same<Tin, Tout>::value &&
                     reinterpret_cast<uintptr_t>(z) % sizeof(Tin) == 0 &&
                     reinterpret_cast<uintptr_t>(dz) % sizeof(Tout) == 0 &&
                     ceil_div(a.V, (int64_t)VEC) <= 16 * 1024;
  const dim3 grid((unsigned)a.T);
  if (vec) {
    const int64_t nvec = a.V / VEC;
    if (nvec <= 256 * 4) {
      const int64_t per = ceil_div(nvec, 256);
      if (per <= 1) row_reg<Tin, Tout, 1, 256><<<grid, 256, 0, st>>>(a, z, dz);
      else if (per <= 2) row_reg<Tin, Tout, 2, 256><<<grid, 256, 0, st>>>(a, z, dz);
      else row_reg<Tin, Tout, 4, 256><<<grid, 256, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    // rows of up to 3072 vectors: 8 vectors per thread in 256- or 512-thread workgroups,
    // so that 3-7 rows share a CU where 1024-thread workgroups of 2-4 vectors fit two
    // (T 8192: V 16384 135 -> 104 us, V 24000 162 -> 146 us)
    if (nvec <= 256 * 8) {
      row_reg<Tin, Tout, 8, 256><<<grid, 256, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    if (nvec <= 384 * 8) {
      row_reg<Tin, Tout, 8, 512><<<grid, 512, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    const int64_t per = ceil_div(nvec, 1024);
    switch (per) {
      case 1: case 2: case 3: case 4: row_reg<Tin, Tout, 4, 1024><<<grid, 1024, 0, st>>>(a, z, dz); break;
      // 512-thread workgroups of 16 vectors per thread (114 VGPRs): two rows per CU,
      // where 1024 threads of 8 (71 VGPRs) fit one (T 16384, V 49152: 607 -> 520 us)
      case 5: case 6: case 7: case 8: row_reg<Tin, Tout, 16, 512><<<grid, 512, 0, st>>>(a, z, dz); break;
      case 9: case 10: case 11: case 12: row_reg<Tin, Tout, 12, 1024><<<grid, 1024, 0, st>>>(a, z, dz); break;
      case 13: case 14: case 15: case 16:
        if constexpr (std::is_same<Tin, bf16>::value && std::is_same<Tout, bf16>::value) {
          // one persistent workgroup per CU, the next row prefetched into LDS
          const unsigned g = (unsigned)(a.T < n_cu ? a.T : n_cu);
          row_pf<Tin, Tout, 16, kPfStage><<<dim3(g), kPfThreads, 0, st>>>(a, z, dz);
        } else {
          row_reg<Tin, Tout, 16, 1024><<<grid, 1024, 0, st>>>(a, z, dz);
        }
        break;
      // 16 vectors per thread in registers, the rest (4 or 8) in LDS: one read of the row
      // (T 4096, V 151936: 572 -> 526 us against the streaming kernel, T 8192, V 196608:
      // 1341 -> 1309 us)
      case 17: case 18: case 19: case 20: case 21: case 22: case 23: case 24:
        if constexpr (Vec<Tout>::N == VEC) {
          if (per <= 20) row_ls<Tin, Tout, 16, 4><<<grid, 1024, 0, st>>>(a, z, dz);
          else row_ls<Tin, Tout, 16, 8><<<grid, 1024, 0, st>>>(a, z, dz);
          break;
        }
        [[fallthrough]];
      default:
        // longer rows: the first 16 vectors per thread stay in registers between the
        // passes, the rest is read twice, 4 vectors in flight per thread (V 151936 at
        // T 8192: 1389 -> 1093 us against one vector in flight and nothing kept)
        row_stream<Tin, Tout, VEC, 1024, 16, 4><<<grid, 1024, 0, st>>>(a, z, dz);
        break;
    }
  } else if (ua_ok) {
    // rows of any element alignment and length that fit the registers
    const int64_t nvec = ceil_div(a.V, (int64_t)VEC);
    if (nvec <= 256 * 4) {
      const int64_t per = ceil_div(nvec, 256);
      if (per <= 1) row_reg<Tin, Tout, 1, 256, true><<<grid, 256, 0, st>>>(a, z, dz);
      else if (per <= 2) row_reg<Tin, Tout, 2, 256, true><<<grid, 256, 0, st>>>(a, z, dz);
      else row_reg<Tin, Tout, 4, 256, true><<<grid, 256, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    if (nvec <= 256 * 8) {
      row_reg<Tin, Tout, 8, 256, true><<<grid, 256, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    if (nvec <= 384 * 8) {
      row_reg<Tin, Tout, 8, 512, true><<<grid, 512, 0, st>>>(a, z, dz);
      return hipGetLastError();
    }
    switch (ceil_div(nvec, 1024)) {
      case 1: case 2: case 3: case 4: row_reg<Tin, Tout, 4, 1024, true><<<grid, 1024, 0, st>>>(a, z, dz); break;
      case 5: case 6: case 7: case 8: row_reg<Tin, Tout, 16, 512, true><<<grid, 512, 0, st>>>(a, z, dz); break;
      case 9: case 10: case 11: case 12: row_reg<Tin, Tout, 12, 1024, true><<<grid, 1024, 0, st>>>(a, z, dz); break;
      default: row_reg<Tin, Tout, 16, 1024, true><<<grid, 1024, 0, st>>>(a, z, dz); break;
    }
  } else {
    row_stream<Tin, Tout, 1, 1024><<<grid, 1024, 0, st>>>(a, z, dz);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace xent
}  // namespace fo
