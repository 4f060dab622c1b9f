// Soft-target cross-entropy (distillation) forward+backward for gfx950.
//
// Definition ("Fast-LLM: 高效大语言模型训练框架", 三 技术架构, 损失函数体系: label-entropy
// and distillation losses beside the hard-label cross-entropy, computed by the
// framework's fused entropy-loss kernel), read as the cross-entropy of the student's
// softmax against the teacher's (temperature 1), over the rows a mask keeps:
//   q = softmax(z), p = softmax(zt) per row;  loss = (1/N) sum_t -sum_v p log q,
//   kl = (1/N) sum_t sum_v p (log p - log q),  dz = dloss (q - p) / N.
// Per row, one sweep gives both online logsumexps (m_z, s_z), (m_t, s_t) and the two
// p-weighted sums
//   A = sum_v exp(zt - m_t) z,  D = sum_v exp(zt - m_t) (zt - z)   (rescaled with m_t),
// so -sum p log q = lse_z - A/s_t, and the KL, sum p (zt - z) + lse_z - lse_t, is
// D/s_t + (m_z - m_t) + log(s_z/s_t): a sum of terms of the size of the KL itself,
// where the difference of the two cross-entropies would cancel two logsumexp-sized
// values.  A second sweep over the same values writes dz.  A workgroup per row streams
// both rows with several 16-byte loads of each in flight per thread; each thread keeps
// up to 8 vectors of each row in registers between the sweeps (rows of up to 2048
// vectors whole, in 256-thread workgroups; longer rows in 512-thread workgroups, two per
// CU), and the second sweep re-reads the rest, mostly from L2 and the Infinity Cache,
// so HBM sees each input about once and dz once (3 T V b).  Unaligned rows take the
// same streaming form, their full vectors still 16-byte accesses at element-aligned
// addresses, in register-lean plans that keep two rows per CU; only rows whose pointers
// are not element-aligned go element by element.
#include "xent_kernels.hpp"

namespace fo {
namespace {

using xent::Counters;

constexpr int kRowThreads = 1024;

// Per-thread (then per-row) state of the sweep: student (ms, ss), teacher (mt, st) and
// the teacher-weighted sums A (of z) and D (of zt - z), all relative to mt.
struct Stats {
  float ms, ss, mt, st, a, d;
};

__device__ __forceinline__ void stats_init(Stats& s) {
  s.ms = -INFINITY; s.ss = 0.f; s.mt = -INFINITY; s.st = 0.f; s.a = 0.f; s.d = 0.f;
}

__device__ __forceinline__ void stats_merge(Stats& s, const Stats& o) {
  lse_merge(s.ms, s.ss, o.ms, o.ss);
  const float m = fmaxf(s.mt, o.mt);
  if (m == -INFINITY) return;
  const float f1 = __expf(s.mt - m), f2 = __expf(o.mt - m);
  s.st = s.st * f1 + o.st * f2;
  s.a = s.a * f1 + o.a * f2;
  s.d = s.d * f1 + o.d * f2;
  s.mt = m;
}

// VEC values of the student (z) and teacher (t)
// (exponentials: accurate for fp32 rows, for bf16 rows one fused multiply-add into the
// hardware 2^x per value, as the hard-label kernels)
// PAD: some values are -inf padding (both z and t) past the end of the row; a zero
// teacher weight then contributes nothing to A and D (plain fmaf would give 0 * -inf).
template <typename T, int VEC, bool PAD = false>
__device__ __forceinline__ void stats_add(Stats& s, const float* z, const float* t) {
  float vz = z[0], vt = t[0];
#pragma unroll
  for (int j = 1; j < VEC; ++j) { vz = fmaxf(vz, z[j]); vt = fmaxf(vt, t[j]); }
  if (vz > s.ms) { s.ss *= xent::ex<T>(s.ms - vz); s.ms = vz; }
  if (vt > s.mt) {
    const float f = xent::ex<T>(s.mt - vt);
    s.st *= f; s.a *= f; s.d *= f; s.mt = vt;
  }
  const float nz = xent::nl2e<T>(s.ms), nt = xent::nl2e<T>(s.mt);
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    s.ss += xent::exs<T>(z[j], nz);
    const float e = xent::exs<T>(t[j], nt);
    s.st += e;
    if (PAD && e == 0.f) continue;
    s.a = fmaf(e, z[j], s.a);
    s.d = fmaf(e, t[j] - z[j], s.d);
  }
}

// Fixed-order workgroup merge: every thread gets the row's totals.
template <int NT>
__device__ __forceinline__ Stats block_stats(Stats s, Stats* sh) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    Stats q;
    q.ms = __shfl_xor(s.ms, o, kWave); q.ss = __shfl_xor(s.ss, o, kWave);
    q.mt = __shfl_xor(s.mt, o, kWave); q.st = __shfl_xor(s.st, o, kWave);
    q.a = __shfl_xor(s.a, o, kWave); q.d = __shfl_xor(s.d, o, kWave);
    stats_merge(s, q);
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = s;
  __syncthreads();
  Stats r = sh[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) stats_merge(r, sh[i]);
  return r;
}

struct DistillArgs {
  int64_t T, V, ldz, ldt, ldd;
  const uint8_t* mask;  // null: every row kept
  float dloss;
  const Counters* cnt;
  float* row_ce;  // [T]
  float* row_kl;  // [T]
};

// The row's loss terms from its totals (thread 0), and the logsumexps for the gradient.
__device__ __forceinline__ void row_terms(const DistillArgs& a, int64_t row, const Stats& r,
                                          float& lse_z, float& lse_t) {
  lse_z = r.ms + logf(r.ss);
  lse_t = r.mt + logf(r.st);
  if (threadIdx.x == 0) {
    a.row_ce[row] = lse_z - r.a / r.st;  // -sum p log q
    a.row_kl[row] = r.d / r.st + ((r.ms - r.mt) + logf(r.ss / r.st));
  }
}

template <typename T>
__device__ __forceinline__ void masked_row(const DistillArgs& a, int64_t row, T* dz) {
  if (dz != nullptr) {
    T* dr = dz + row * a.ldd;
    for (int64_t e = threadIdx.x; e < a.V; e += blockDim.x) dr[e] = from_f32<T>(0.f);
  }
  if (threadIdx.x == 0) { a.row_ce[row] = 0.f; a.row_kl[row] = 0.f; }
}

// Element path, for rows whose pointers are not even element-aligned: one element per
// thread and step, the second sweep re-reading both rows.  dz may alias z (each element
// is read by the thread that writes it; the merge barrier separates the first sweep's
// reads from the writes).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void soft_stream(DistillArgs a, const T* z,
                                                          const T* zt, T* dz) {
  __shared__ Stats sh[kRowThreads / kWave];
  const int64_t row = blockIdx.x;
  if (a.mask != nullptr && a.mask[row] == 0) {
    masked_row<T>(a, row, dz);
    return;
  }
  const T* zr = z + row * a.ldz;
  const T* tr = zt + row * a.ldt;
  Stats s;
  stats_init(s);
  for (int64_t v = threadIdx.x; v < a.V; v += kRowThreads) {
    const float zf = to_f32(zr[v]), tf = to_f32(tr[v]);
    stats_add<T, 1>(s, &zf, &tf);
  }
  const Stats r = block_stats<kRowThreads>(s, sh);
  float lse_z, lse_t;
  row_terms(a, row, r, lse_z, lse_t);
  if (dz == nullptr) return;
  const float scale = a.dloss / (float)a.cnt->n_valid;
  T* dr = dz + row * a.ldd;
  for (int64_t v = threadIdx.x; v < a.V; v += kRowThreads)
    dr[v] = from_f32<T>(scale * (xent::ex<T>(to_f32(zr[v]) - lse_z) -
                                 xent::ex<T>(to_f32(tr[v]) - lse_t)));
}

// Aligned rows of any length (V % VEC == 0), streamed: each thread keeps its first KS
// vectors of both rows in registers from the first sweep to the second and re-reads the
// rest (from L2 and the Infinity Cache); streamed vectors of both rows are loaded U at a
// time before any is used (2U 16-byte loads in flight per thread), and the gradient
// goes out as 16-byte vectors.  dz may alias z (each element is read by the thread that
// writes it; the merge barrier separates the first sweep's reads from the writes).
// Loads of values read once (the kept vectors, the second sweep's re-reads) carry the
// non-temporal hint; only the first sweep's streamed loads, whose lines the second sweep
// wants back, are plain (T 8192, V 16384: 214 -> 146 us; V 128256: 1269 -> 1227 us
// against plain loads throughout).
// Vector v of a row of V elements.  UA (rows of any element alignment and length): full
// vectors are still 16-byte accesses at element-aligned addresses, the partial last
// vector goes element by element, read as -inf padding past the row (a zero teacher
// weight adds nothing).  NTH: the non-temporal hint, for a value read once.  (The hint is
// a template argument: one function with both loads behind a runtime flag compiles to a
// single plain load, the two merged.)
template <typename T, bool UA, bool NTH>
__device__ __forceinline__ Pack<T> row_ld(const T* p, int64_t v, int64_t V) {
  constexpr int VEC = Vec<T>::N;
  if (!UA || (v + 1) * VEC <= V) {
    if constexpr (NTH) return load_pack(p + v * VEC);
    else return load_pack_cached(p + v * VEC);
  }
  Pack<T> r;
#pragma unroll
  for (int j = 0; j < VEC; ++j) r.v[j] = v * VEC + j < V ? p[v * VEC + j] : from_f32<T>(-INFINITY);
  return r;
}

template <typename T, int U, int KS, int NT = kRowThreads, bool UA = false>
__global__ __launch_bounds__(NT) void soft_stream_u(DistillArgs a, const T* z, const T* zt,
                                                   T* dz) {
  constexpr int VEC = Vec<T>::N;
  constexpr int KR = KS > 0 ? KS : 1;
  __shared__ Stats sh[NT / kWave];
  const int64_t row = blockIdx.x;
  if (a.mask != nullptr && a.mask[row] == 0) {
    masked_row<T>(a, row, dz);
    return;
  }
  const int64_t n = UA ? ceil_div(a.V, (int64_t)VEC) : a.V / VEC;
  const T* zr = z + row * a.ldz;
  const T* tr = zt + row * a.ldt;
  const int64_t tid = threadIdx.x;
  Pack<T> kz[KR], kt[KR];
  Stats s;
  stats_init(s);
  auto add = [&](const Pack<T>& zp, const Pack<T>& tp) {
    float zf[VEC], tf[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) { zf[j] = to_f32(zp.v[j]); tf[j] = to_f32(tp.v[j]); }
    stats_add<T, VEC, UA>(s, zf, tf);
  };
  if constexpr (KS > 0) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int64_t v = tid + (int64_t)i * NT;
      if (v < n) { kz[i] = row_ld<T, UA, true>(zr, v, a.V); kt[i] = row_ld<T, UA, true>(tr, v, a.V); }
    }
#pragma unroll
    for (int i = 0; i < KS; ++i)
      if (tid + (int64_t)i * NT < n) add(kz[i], kt[i]);
  }
  const int64_t tail0 = tid + (int64_t)KS * NT;
  for (int64_t v0 = tail0; v0 < n; v0 += (int64_t)U * NT) {
    Pack<T> zp[U], tp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * NT;
      if (v < n) { zp[u] = row_ld<T, UA, false>(zr, v, a.V); tp[u] = row_ld<T, UA, false>(tr, v, a.V); }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT < n) add(zp[u], tp[u]);
  }
  const Stats r = block_stats<NT>(s, sh);
  float lse_z, lse_t;
  row_terms(a, row, r, lse_z, lse_t);
  if (dz == nullptr) return;
  const float scale = a.dloss / (float)a.cnt->n_valid;
  const float nz = xent::nl2e<T>(lse_z), nt = xent::nl2e<T>(lse_t);
  T* dr = dz + row * a.ldd;
  auto grad = [&](const Pack<T>& zp, const Pack<T>& tp, int64_t v) {
    Pack<T> o;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      o.v[j] = from_f32<T>(scale * (xent::exs<T>(to_f32(zp.v[j]), nz) -
                                    xent::exs<T>(to_f32(tp.v[j]), nt)));
    if (!UA || (v + 1) * VEC <= a.V) {
      store_pack(dr + v * VEC, o);
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        if (v * VEC + j < a.V) dr[v * VEC + j] = o.v[j];
    }
  };
  for (int64_t v0 = tail0; v0 < n; v0 += (int64_t)U * NT) {
    Pack<T> zp[U], tp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * NT;
      if (v < n) { zp[u] = row_ld<T, UA, true>(zr, v, a.V); tp[u] = row_ld<T, UA, true>(tr, v, a.V); }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT < n) grad(zp[u], tp[u], v0 + u * NT);
  }
  if constexpr (KS > 0) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int64_t v = tid + (int64_t)i * NT;
      if (v < n) grad(kz[i], kt[i], v);
    }
  }
}

// N = rows the mask keeps (all T without a mask), into cnt.  One workgroup.
__global__ __launch_bounds__(1024) void count_mask(int64_t T_, const uint8_t* __restrict__ mask,
                                                   Counters* cnt) {
  __shared__ long long sh[16];
  long long c = 0;
  for (int64_t t = threadIdx.x; t < T_; t += 1024) c += (mask == nullptr || mask[t] != 0) ? 1 : 0;
  c = wave_sum_i64(c);
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long n = 0;
    for (int i = 0; i < 16; ++i) n += sh[i];
    cnt->n_valid = n;
    cnt->n_bad = 0;
    cnt->pad = 0;
  }
}

struct Ws {
  size_t off_cnt, off_ce, off_kl, total;
};
Ws ws_layout(int64_t T_) {
  Ws w;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  w.off_cnt = take(sizeof(Counters));
  w.off_ce = take((size_t)(T_ > 0 ? T_ : 1) * 4);
  w.off_kl = take((size_t)(T_ > 0 ? T_ : 1) * 4);
  w.total = o;
  return w;
}

template <typename T>
int distill_impl(const DistillArgs& a0, const T* z, const T* zt, T* dz, float* loss, float* kl,
                 int64_t* n_valid, char* ws, hipStream_t st) {
  const Ws w = ws_layout(a0.T);
  DistillArgs a = a0;
  Counters* cnt = reinterpret_cast<Counters*>(ws + w.off_cnt);
  a.cnt = cnt;
  a.row_ce = reinterpret_cast<float*>(ws + w.off_ce);
  a.row_kl = reinterpret_cast<float*>(ws + w.off_kl);
  count_mask<<<1, 1024, 0, st>>>(a.T, a.mask, cnt);
  if (a.T > 0) {
    constexpr int VEC = Vec<T>::N;
    const bool vec = a.V % VEC == 0 && a.ldz % VEC == 0 && a.ldt % VEC == 0 && aligned16(z) &&
                     aligned16(zt) && (dz == nullptr || (a.ldd % VEC == 0 && aligned16(dz)));
    const int64_t nvec = a.V / VEC;
    const dim3 grid((unsigned)a.T), block(kRowThreads);
    if (vec) {
      // Each thread keeps up to 8 vectors of each row in registers between the sweeps:
      // rows of up to 2048 vectors whole in 256-thread workgroups (several rows per CU),
      // longer rows in 512-thread workgroups (two per CU at 127 VGPRs) with their first
      // 4096 vectors kept and the rest streamed twice, 4 loads of each row in flight per
      // thread.  T 8192, bf16, against 1024 threads that kept nothing up to 8192 vectors:
      // V 16384 296 -> 219 us, 32000 418 -> 347, 65536 725 -> 646; 512 against 1024
      // threads keeping 8 at V 128256: 1303 -> 1268 us.
      if (nvec <= 4 * 256) soft_stream_u<T, 4, 4, 256><<<grid, dim3(256), 0, st>>>(a, z, zt, dz);
      else if (nvec <= 8 * 256) soft_stream_u<T, 4, 8, 256><<<grid, dim3(256), 0, st>>>(a, z, zt, dz);
      else soft_stream_u<T, 4, 8, 512><<<grid, dim3(512), 0, st>>>(a, z, zt, dz);
    } else if (reinterpret_cast<uintptr_t>(z) % sizeof(T) == 0 &&
               reinterpret_cast<uintptr_t>(zt) % sizeof(T) == 0 &&
               reinterpret_cast<uintptr_t>(dz) % sizeof(T) == 0) {
      // element-aligned rows of any alignment and length: the same streaming form, 16-byte
      // accesses at element-aligned addresses and the partial last vector element-wise,
      // in register-lean plans (at most 128 VGPRs, so that two 512-thread rows share a
      // CU).  T 8192, against one vector per thread and step and nothing kept: V 8199
      // 257 -> 124 us, 50257 766 -> 650, 128257 1908 -> 1694.
      const int64_t nv = ceil_div(a.V, (int64_t)VEC);
      if (nv <= 4 * 256) soft_stream_u<T, 4, 4, 256, true><<<grid, dim3(256), 0, st>>>(a, z, zt, dz);
      else if (nv <= 6 * 256) soft_stream_u<T, 4, 6, 256, true><<<grid, dim3(256), 0, st>>>(a, z, zt, dz);
      else soft_stream_u<T, 2, 8, 512, true><<<grid, dim3(512), 0, st>>>(a, z, zt, dz);
    } else {
      soft_stream<T><<<grid, block, 0, st>>>(a, z, zt, dz);
    }
  }
  xent::finalize<<<1, 1024, 0, st>>>(a.T, a.row_ce, a.row_kl, cnt, loss, kl, n_valid, nullptr);
  return launch_status();
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" size_t fo_distill_workspace(int64_t T, int64_t V) {
  if (T < 0 || V < 1) return 0;
  return ws_layout(T).total;
}

extern "C" int fo_distill_fwd_bwd(int dtype, int64_t T, int64_t V, const void* logits,
                                  int64_t ldl, const void* teacher, int64_t ldt,
                                  const uint8_t* row_mask, float dloss, void* dlogits,
                                  int64_t ldd, float* loss, float* kl, int64_t* n_valid,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (dtype != FO_F32 && dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || V < 1 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (ldl < V || ldt < V || (dlogits && ldd < V)) return FO_ERR_STRIDE;
  if (!loss) return FO_ERR_NULL;
  if (T > 0 && (!logits || !teacher)) return FO_ERR_NULL;
  if (!ws || ws_bytes < fo_distill_workspace(T, V)) return FO_ERR_WORKSPACE;
  DistillArgs a{};
  a.T = T; a.V = V; a.ldz = ldl; a.ldt = ldt; a.ldd = ldd;
  a.mask = row_mask;
  a.dloss = dloss;
  hipStream_t st = as_stream(stream);
  if (dtype == FO_F32)
    return distill_impl<float>(a, static_cast<const float*>(logits), static_cast<const float*>(teacher),
                               static_cast<float*>(dlogits), loss, kl, n_valid, static_cast<char*>(ws), st);
  return distill_impl<bf16>(a, static_cast<const bf16*>(logits), static_cast<const bf16*>(teacher),
                            static_cast<bf16*>(dlogits), loss, kl, n_valid, static_cast<char*>(ws), st);
}
