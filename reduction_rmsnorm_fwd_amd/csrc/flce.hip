// Fused linear cross-entropy (lm head + loss, forward and backward) for gfx950.
//
// Definition (the Liger section of "Kernels（自定义内核）": FusedLinearCrossEntropy fuses
// the lm-head projection with the loss so that large vocabularies fit in memory; the
// loss itself is the cross-entropy with z-loss of "Fast-LLM: 高效大语言模型训练框架",
// 三 技术架构, 损失函数体系):
//   Z = H W^T,  (loss, dZ) = cross_entropy(Z),  dH = dZ W,  dW = dZ^T H
// The full [T, V] logits never exist: tokens go through in chunks of C rows, and per
// chunk
//   1. Z_c = H_c W^T            bf16 MFMA; the epilogue never stores Z_c itself: per
//                               row and 128-column block it keeps the online-logsumexp
//                               partial (m, sum exp(z - m)), writes E = exp(z - m) in
//                               bf16 into the chunk's dZ rows, and the target's logit
//                               in fp32
//   2. CE over the chunk's rows the partials give each row's lse, hence its loss (with
//                               the target logit); one in-place pass turns E into
//                               dZ_c = (dloss/N)(E exp(m - lse)(1 + 2 c lse) - onehot)
//                               (the target column from its fp32 logit), with N
//                               counted once over all T targets up front
//   3. dH_c = dZ_c W            bf16 MFMA reading W as it is stored ([V, H]: k-major
//                               for this product), bf16 out
//   4. dW (+)= dZ_c^T H_c       bf16 MFMA reading dZ and H as stored (token-major:
//                               k-major for this product), fp32 accumulation across
//                               chunks in dW (or a workspace buffer, cast to bf16
//                               once at the end): the first chunk's product writes
//                               dW, each later one loads the dW tile into its
//                               accumulators and writes the sum back
// The workspace holds one chunk's bf16 dZ rows ([C, V]), so it grows with the chunk,
// never with T * V.
// The k-major operands go through LDS untransposed and are read with the transposing
// LDS loads of gfx950, so no operand is ever transposed in memory.
// Rows whose target is ignored (or out of range) contribute nothing, so the valid rows
// are compacted first (one scan kernel; their hidden states gathered into a workspace
// copy) and the chunks run over valid rows only; row and K extents of the last chunk
// are read on the device, so no host synchronisation is needed.  dH is scattered back
// at the end, with exact zeros in the rows of ignored tokens.
#include "gemm.hpp"
#include "xent_kernels.hpp"

namespace fo {
namespace {

constexpr int64_t kAutoChunk = 2048;

struct Layout {
  int64_t C, Vpad;
  int64_t nparts;   // logsumexp partials per logits row
  int64_t dh_smax;  // split-K slice bound of the dH product (1: no split)
  size_t off_cnt, off_loss, off_z, off_dz, off_dw, off_part, off_stats, off_idx,
      off_pos, off_tgv, off_hv, off_dhv, off_zy, total;
};

Layout layout(int64_t T, int64_t H, int64_t V, int64_t chunk, int dw_dtype) {
  Layout L;
  int64_t C = chunk > 0 ? chunk : kAutoChunk;
  if (C > T) C = T > 0 ? T : 1;
  L.C = C;
  L.Vpad = align_up((size_t)V, 64);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.off_cnt = take(256);
  L.off_loss = take((size_t)(T > 0 ? T : 1) * 4);
  L.off_z = take((size_t)(T > 0 ? T : 1) * 4);
  L.off_dz = take((size_t)C * L.Vpad * 2);
  L.off_dw = take(dw_dtype == FO_BF16 ? (size_t)V * H * 4 : 0);
  // dH of a chunk has few 256x256 tiles: split it over the vocabulary, the slice count
  // chosen on the device from the chunk's valid rows (at most 4, each >= 2048 deep:
  // as fast as 8 at the lm-head workload, with 201 -> 67 MB of partials); the partials
  // are packed, so the buffer holds the largest slices x rows product any row count
  // up to C can choose
  L.dh_smax = 1;
  if (gemm::split_plan(C, H, L.Vpad).splits > 1) {
    L.dh_smax = L.Vpad / 2048 < 4 ? L.Vpad / 2048 : 4;
    if (L.dh_smax < 1) L.dh_smax = 1;
  }
  L.off_part = take(L.dh_smax > 1
                        ? (size_t)gemm::split_rows_bound(C, H, L.Vpad, L.dh_smax) * H * 4
                        : 0);
  const size_t Tn = (size_t)(T > 0 ? T : 1);
  L.nparts = ceil_div(V, gemm::kStatsCols);
  L.off_stats = take((size_t)C * L.nparts * 8);
  L.off_idx = take(Tn * 4);
  L.off_pos = take(Tn * 4);
  L.off_tgv = take(Tn * 8);
  L.off_hv = take(Tn * H * 2);
  L.off_dhv = take(Tn * H * 2);
  L.off_zy = take(Tn * 4);
  L.total = o;
  return L;
}

__global__ void fill_f32_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

__global__ void cast_f32_bf16(const float* __restrict__ s, bf16* __restrict__ d, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = from_f32<bf16>(s[i]);
}

// Hv[j] = H[idx[j]] for the n_valid compacted rows, zero rows after them.
__global__ __launch_bounds__(256) void gather_rows(const bf16* __restrict__ Hm, int64_t H,
                                                   const int* __restrict__ idx,
                                                   const xent::Counters* __restrict__ cnt,
                                                   bf16* __restrict__ Hv) {
  const int64_t j = blockIdx.x;
  const bool live = j < cnt->n_valid;
  const bf16* src = live ? Hm + (int64_t)idx[j] * H : nullptr;
  bf16* dst = Hv + j * H;
  for (int64_t v = threadIdx.x; v < H / 8; v += 256)
    *reinterpret_cast<u32x4*>(dst + v * 8) =
        live ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + v * 8)) : u32x4{0, 0, 0, 0};
}

// dH[t] = dHv[pos_of[t]], or zeros for a row whose target was ignored or bad.
__global__ __launch_bounds__(256) void scatter_rows(const bf16* __restrict__ dHv, int64_t H,
                                                    const int* __restrict__ pos_of,
                                                    bf16* __restrict__ dH) {
  const int64_t t = blockIdx.x;
  const int p = pos_of[t];
  bf16* dst = dH + t * H;
  const bf16* src = p >= 0 ? dHv + (int64_t)p * H : nullptr;
  for (int64_t v = threadIdx.x; v < H / 8; v += 256)
    *reinterpret_cast<u32x4*>(dst + v * 8) =
        p >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + v * 8)) : u32x4{0, 0, 0, 0};
}

// Cross-entropy of one chunk from what the logits product left: per row its
// online-logsumexp partials (m_p, s_p) for each 128-column block p, its target logit zy,
// and (gradient wanted) E = exp(z - m_p) in bf16 in the row of dZ.  Merges the row's
// partials (fixed order) into lse, writes the row's loss, then rewrites the row in place
// as dZ = (dloss/N)(softmax (1 + 2 c lse) - onehot) in bf16, softmax = E exp(m_p - lse),
// the target column computed from zy; zeros go to the padding columns [V, ldd) (the K
// tail of the dH product).  Rows past the chunk's valid count are never read by the
// products and are left alone.  One 256-thread workgroup per row.
constexpr int kApplyThreads = 256;
__global__ __launch_bounds__(kApplyThreads) void ce_apply(
    const float2* __restrict__ stats, int64_t nparts, const int64_t* __restrict__ tg,
    const float* __restrict__ zy, const xent::Counters* __restrict__ cnt, int64_t rows_base,
    int64_t rows, int64_t V, float zc, float dloss, bf16* __restrict__ dZ, int64_t ldd,
    float* __restrict__ row_loss, float* __restrict__ row_z) {
  __shared__ float shm[kApplyThreads / kWave], shs[kApplyThreads / kWave];
  const int64_t row = blockIdx.x;
  int64_t eff = cnt->n_valid - rows_base;
  eff = eff < 0 ? 0 : (eff > rows ? rows : eff);
  if (row >= eff) return;
  float m = -INFINITY, s = 0.f;
  const float2* sp = stats + row * nparts;
  for (int64_t p = threadIdx.x; p < nparts; p += kApplyThreads) {
    const float2 q = sp[p];
    lse_merge(m, s, q.x, q.y);
  }
  const float lse = xent::block_lse<kApplyThreads>(m, s, shm, shs);
  const long long y = tg[row];
  const float zt_logit = zy[row];
  if (threadIdx.x == 0) {
    const float zt = zc * lse * lse;
    row_loss[row] = (lse - zt_logit) + zt;
    row_z[row] = zt;
  }
  if (dZ == nullptr) return;
  const float scale = dloss / (float)cnt->n_valid;
  const float coef = scale * fmaf(2.f * zc, lse, 1.f);
  const float gy = coef * __expf(zt_logit - lse) - scale;  // the target column
  bf16* dr = dZ + row * ldd;
  constexpr int kCols = gemm::kStatsCols;
  const int64_t V8 = V / 8 * 8;  // 8-column groups never straddle a 128-column block
  for (int64_t v = (int64_t)threadIdx.x * 8; v < V8; v += kApplyThreads * 8) {
    const float f = coef * __expf(sp[v / kCols].x - lse);
    union { u32x4 raw; bf16 e[8]; } o;
    o.raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dr + v));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float g = v + j == y ? gy : f * to_f32(o.e[j]);
      o.e[j] = from_f32<bf16>(g);
    }
    *reinterpret_cast<u32x4*>(dr + v) = o.raw;
  }
  for (int64_t v = V8 + threadIdx.x; v < V; v += kApplyThreads) {
    const float g = v == y ? gy : coef * __expf(sp[v / kCols].x - lse) * to_f32(dr[v]);
    dr[v] = from_f32<bf16>(g);
  }
  for (int64_t v = V + threadIdx.x; v < ldd; v += kApplyThreads) dr[v] = from_f32<bf16>(0.f);
}

#define FO_HIP(...)                                \
  do {                                             \
    if ((__VA_ARGS__) != hipSuccess) return FO_ERR_HIP; \
  } while (0)

int flce_impl(int64_t T, int64_t H, int64_t V, const bf16* Hm, const bf16* W,
              const int64_t* tg, int64_t ignore, float zc, float dloss, bf16* dH, void* dW,
              int dw_dtype, float* loss, float* z_loss, int64_t* n_valid, int32_t* status,
              const Layout& L, char* ws, hipStream_t st) {
  xent::Counters* cnt = reinterpret_cast<xent::Counters*>(ws + L.off_cnt);
  const long long* nv = &cnt->n_valid;
  float* row_loss = reinterpret_cast<float*>(ws + L.off_loss);
  float* row_z = reinterpret_cast<float*>(ws + L.off_z);
  float* zy = reinterpret_cast<float*>(ws + L.off_zy);
  bf16* dZ = reinterpret_cast<bf16*>(ws + L.off_dz);
  int* idx = reinterpret_cast<int*>(ws + L.off_idx);
  int* pos_of = reinterpret_cast<int*>(ws + L.off_pos);
  int64_t* tgv = reinterpret_cast<int64_t*>(ws + L.off_tgv);
  bf16* Hv = reinterpret_cast<bf16*>(ws + L.off_hv);
  bf16* dHv = reinterpret_cast<bf16*>(ws + L.off_dhv);
  float2* stats = reinterpret_cast<float2*>(ws + L.off_stats);
  float* dW32 = dw_dtype == FO_BF16 ? reinterpret_cast<float*>(ws + L.off_dw)
                                    : static_cast<float*>(dW);

  if (T > 0) {
    xent::compact_targets<<<1, 1024, 0, st>>>(T, V, tg, ignore, cnt, idx, pos_of, tgv);
    gather_rows<<<(unsigned)T, 256, 0, st>>>(Hm, H, idx, cnt, Hv);
    FO_HIP(hipGetLastError());
    const bool need_grad = dH != nullptr || dW != nullptr;
    for (int64_t c0 = 0; c0 < T; c0 += L.C) {
      const int64_t cl = (T - c0 < L.C) ? T - c0 : L.C;  // rows at most (valid rows: on device)
      // 1. logits of the chunk's valid rows: row partials, target logits and (gradient
      //    wanted) exp(z - m) in the chunk's dZ rows
      gemm::Args g;
      g.A = Hv + c0 * H; g.lda = H;
      g.B = W; g.ldb = H;
      g.C = need_grad ? dZ : nullptr; g.ldc = L.Vpad;
      g.M = cl; g.N = V; g.K = H;
      g.dev_count = nv; g.count_base = c0; g.dev_dim = 1;
      g.stats = stats; g.stats_ld = L.nparts;
      g.tgt = tgv + c0; g.zy = zy + c0;
      FO_HIP(gemm::run<gemm::kStoreExpStats>(g, gemm::kWide, st));
      // 2. loss rows, and dZ in place from the row partials
      ce_apply<<<(unsigned)cl, kApplyThreads, 0, st>>>(
          stats, L.nparts, tgv + c0, zy + c0, cnt, c0, cl, V, zc, dloss,
          need_grad ? dZ : nullptr, L.Vpad, row_loss + c0, row_z + c0);
      FO_HIP(hipGetLastError());
      // 3. dH rows of the chunk: dZ_c [cl, Vpad] times W read k-major ([V, H]; its rows
      //    past V read as zeros against dZ's zero padding columns).  Split over the
      //    vocabulary when the chunk's 256x256 tiles cannot fill the chip; the fp32
      //    partials are summed in a fixed order.
      if (dH != nullptr) {
        gemm::Args h;
        h.A = dZ; h.lda = L.Vpad;
        h.B = W; h.ldb = H; h.b_rows = V;
        h.M = cl; h.N = H; h.K = L.Vpad;
        h.dev_count = nv; h.count_base = c0; h.dev_dim = 1;
        if (L.dh_smax > 1) {
          float* part = reinterpret_cast<float*>(ws + L.off_part);
          h.C = part; h.ldc = H;
          h.split_max = L.dh_smax; h.split_compact = true;
          FO_HIP((gemm::run<gemm::kStoreF32, false, true>(h, gemm::kWide, st)));
          gemm::reduce_splits_bf16<<<2048, 256, 0, st>>>(part, L.dh_smax, cl * H, H,
                                                         dHv + c0 * H, H, nv, c0, L.Vpad,
                                                         L.dh_smax, true);
          FO_HIP(hipGetLastError());
        } else {
          h.C = dHv + c0 * H; h.ldc = H;
          FO_HIP((gemm::run<gemm::kStoreBF16, false, true>(h, gemm::kNarrow, st)));
        }
      }
      // 4. dW contribution of the chunk's rows: dZ_c^T Hv_c with both operands read
      //    k-major (token-major as stored), K = the chunk's valid rows, read on the
      //    device.  The first chunk writes dW, later ones accumulate into it.
      if (dW != nullptr) {
        gemm::Args w;
        w.A = dZ; w.lda = L.Vpad;
        w.B = Hv + c0 * H; w.ldb = H;
        w.C = dW32; w.ldc = H;
        w.M = V; w.N = H; w.K = cl;
        w.dev_count = nv; w.count_base = c0; w.dev_dim = 2;
        if (c0 == 0) FO_HIP((gemm::run<gemm::kStoreF32, true, true>(w, gemm::kWide, st)));
        else FO_HIP((gemm::run<gemm::kAccumF32, true, true>(w, gemm::kWide, st)));
      }
    }
    if (dH != nullptr) {
      scatter_rows<<<(unsigned)T, 256, 0, st>>>(dHv, H, pos_of, dH);
      FO_HIP(hipGetLastError());
    }
  } else {
    xent::count_targets<<<1, 1024, 0, st>>>(0, V, tg, ignore, cnt);
    FO_HIP(hipGetLastError());
    if (dW != nullptr) {
      fill_f32_zero<<<1024, 256, 0, st>>>(dW32, V * H);
      FO_HIP(hipGetLastError());
    }
  }
  if (dW != nullptr && dw_dtype == FO_BF16) {
    cast_f32_bf16<<<4096, 256, 0, st>>>(dW32, static_cast<bf16*>(dW), V * H);
    FO_HIP(hipGetLastError());
  }
  xent::finalize<<<1, 1024, 0, st>>>(T, row_loss, row_z, cnt, loss, z_loss, n_valid, status, 1);
  return launch_status();
}

}  // namespace
}  // namespace fo

using namespace fo;

extern "C" size_t fo_flce_workspace(int64_t T, int64_t H, int64_t V, int64_t chunk_tokens,
                                    int dweight_dtype) {
  if (T < 0 || H < 1 || V < 1 || chunk_tokens < 0) return 0;
  return layout(T, H, V, chunk_tokens, dweight_dtype).total;
}

extern "C" int fo_flce_fwd_bwd(int dtype, int64_t T, int64_t H, int64_t V, const void* hidden,
                               const void* weight, const int64_t* targets, int64_t ignore_index,
                               float z_loss_coef, float dloss, void* dhidden, void* dweight,
                               int dweight_dtype, float* loss, float* z_loss, int64_t* n_valid,
                               int32_t* status, int64_t chunk_tokens, void* ws, size_t ws_bytes,
                               void* stream) {
  if (dtype != FO_BF16) return FO_ERR_DTYPE;
  if (dweight_dtype != FO_F32 && dweight_dtype != FO_BF16) return FO_ERR_DTYPE;
  if (T < 0 || H < 1 || V < 1 || chunk_tokens < 0 || T > INT32_MAX) return FO_ERR_SHAPE;
  if (H % 8 != 0) return FO_ERR_SHAPE;
  if (!loss) return FO_ERR_NULL;
  if (T > 0 && (!hidden || !targets)) return FO_ERR_NULL;
  if (!weight) return FO_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(weight) || (dhidden && !aligned16(dhidden)))
    return FO_ERR_STRIDE;
  const Layout L = layout(T, H, V, chunk_tokens, dweight_dtype);
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return FO_ERR_WORKSPACE;
  return flce_impl(T, H, V, static_cast<const bf16*>(hidden), static_cast<const bf16*>(weight),
                   targets, ignore_index, z_loss_coef, dloss, static_cast<bf16*>(dhidden),
                   dweight, dweight_dtype, loss, z_loss, n_valid, status, L,
                   static_cast<char*>(ws), as_stream(stream));
}
