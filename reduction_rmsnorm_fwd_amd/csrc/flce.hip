// Fused linear cross-entropy (lm head + loss, forward and backward) for gfx950.
//
// Definition (the Liger section of "Kernels（自定义内核）": FusedLinearCrossEntropy fuses
// the lm-head projection with the loss so that large vocabularies fit in memory; the
// loss itself is the cross-entropy with z-loss of "Fast-LLM: 高效大语言模型训练框架",
// 三 技术架构, 损失函数体系):
//   Z = H W^T,  (loss, dZ) = cross_entropy(Z),  dH = dZ W,  dW = dZ^T H
// The full [T, V] logits never exist: tokens go through in chunks of C rows, and per
// chunk
//   1. Z_c = H_c W^T            bf16 MFMA, fp32 out, into a [C, V] fp32 buffer
//   2. row kernel on Z_c        loss rows + dZ_c (bf16), scaled by dloss/N with N
//                               counted once over all T targets up front
//   3. dH_c = dZ_c (W^T)^T      bf16 MFMA (W^T made once per call), bf16 out
//   4. dW (+)= dZ_c^T H_c       bf16 MFMA on transposed copies of dZ_c and H_c, fp32
//                               accumulation across chunks in dW (or a workspace
//                               buffer, cast to bf16 once at the end)
// Ignored rows have an all-zero dZ row, so their dH rows come out exactly zero and
// they add nothing to dW.
#include "gemm.hpp"
#include "xent_kernels.hpp"

namespace fo {
namespace {

constexpr int64_t kAutoChunk = 2048;

struct Layout {
  int64_t C, Cpad, Vpad, ldz;
  gemm::SplitPlan dh_split;  // split-K of the dH product (a full chunk)
  size_t off_cnt, off_loss, off_z, off_wt, off_zbuf, off_dz, off_dzt, off_hct, off_dw,
      off_part, total;
};

Layout layout(int64_t T, int64_t H, int64_t V, int64_t chunk, int dw_dtype) {
  Layout L;
  int64_t C = chunk > 0 ? chunk : kAutoChunk;
  if (C > T) C = T > 0 ? T : 1;
  L.C = C;
  L.Cpad = align_up((size_t)C, 8);
  L.Vpad = align_up((size_t)V, 64);
  L.ldz = L.Vpad;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.off_cnt = take(256);
  L.off_loss = take((size_t)(T > 0 ? T : 1) * 4);
  L.off_z = take((size_t)(T > 0 ? T : 1) * 4);
  L.off_wt = take((size_t)H * L.Vpad * 2);
  L.off_zbuf = take((size_t)C * L.ldz * 4);
  L.off_dz = take((size_t)C * L.Vpad * 2);
  L.off_dzt = take((size_t)V * L.Cpad * 2);
  L.off_hct = take((size_t)H * L.Cpad * 2);
  L.off_dw = take(dw_dtype == FO_BF16 ? (size_t)V * H * 4 : 0);
  L.dh_split = gemm::split_plan(C, H, L.Vpad);
  L.off_part = take(L.dh_split.splits > 1 ? (size_t)L.dh_split.splits * C * H * 4 : 0);
  L.total = o;
  return L;
}

__global__ void fill_bf16_zero(bf16* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = from_f32<bf16>(0.f);
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

#define FO_HIP(...)                                \
  do {                                             \
    if ((__VA_ARGS__) != hipSuccess) return FO_ERR_HIP; \
  } while (0)

int flce_impl(int64_t T, int64_t H, int64_t V, const bf16* Hm, const bf16* W,
              const int64_t* tg, int64_t ignore, float zc, float dloss, bf16* dH, void* dW,
              int dw_dtype, float* loss, float* z_loss, int64_t* n_valid, int32_t* status,
              const Layout& L, char* ws, hipStream_t st) {
  xent::Counters* cnt = reinterpret_cast<xent::Counters*>(ws + L.off_cnt);
  float* row_loss = reinterpret_cast<float*>(ws + L.off_loss);
  float* row_z = reinterpret_cast<float*>(ws + L.off_z);
  bf16* Wt = reinterpret_cast<bf16*>(ws + L.off_wt);
  float* Z = reinterpret_cast<float*>(ws + L.off_zbuf);
  bf16* dZ = reinterpret_cast<bf16*>(ws + L.off_dz);
  bf16* dZt = reinterpret_cast<bf16*>(ws + L.off_dzt);
  bf16* Hct = reinterpret_cast<bf16*>(ws + L.off_hct);
  float* dW32 = dw_dtype == FO_BF16 ? reinterpret_cast<float*>(ws + L.off_dw)
                                    : static_cast<float*>(dW);

  xent::count_targets<<<1, 1024, 0, st>>>(T, V, tg, ignore, cnt);
  FO_HIP(hipGetLastError());
  if (T > 0) {
    if (dH != nullptr) {
      FO_HIP(gemm::transpose(W, H, Wt, L.Vpad, V, H, L.Vpad, st));
      // columns [V, Vpad) of dZ are the zero K-padding of the dH contraction
      fill_bf16_zero<<<1024, 256, 0, st>>>(dZ, L.C * L.Vpad);
      FO_HIP(hipGetLastError());
    }
    for (int64_t c0 = 0; c0 < T; c0 += L.C) {
      const int64_t cl = (T - c0 < L.C) ? T - c0 : L.C;
      const int64_t clp = align_up((size_t)cl, 8);
      // 1. logits of the chunk
      gemm::Args g;
      g.A = Hm + c0 * H; g.lda = H;
      g.B = W; g.ldb = H;
      g.C = Z; g.ldc = L.ldz;
      g.M = cl; g.N = V; g.K = H;
      FO_HIP(gemm::run<gemm::kStoreF32>(g, gemm::kWide, st));
      // 2. loss rows and dZ
      xent::RowArgs r;
      r.T = cl; r.V = V; r.ldz = L.ldz; r.ldd = L.Vpad; r.ignore = ignore; r.zc = zc;
      r.dloss = dloss; r.tg = tg + c0; r.cnt = cnt; r.row_loss = row_loss + c0;
      r.row_z = row_z + c0;
      const bool need_grad = dH != nullptr || dW != nullptr;
      FO_HIP(xent::launch_rows<float, bf16>(r, Z, need_grad ? dZ : nullptr, st));
      // 3. dH rows of the chunk (split over the vocabulary when a chunk's 256x256 tiles
      //    cannot fill the chip; the fp32 partials are summed in a fixed order)
      if (dH != nullptr) {
        gemm::Args h;
        h.A = dZ; h.lda = L.Vpad;
        h.B = Wt; h.ldb = L.Vpad;
        h.M = cl; h.N = H; h.K = L.Vpad;
        const gemm::SplitPlan sp = gemm::split_plan(cl, H, L.Vpad);
        if (sp.splits > 1 && sp.splits <= L.dh_split.splits) {
          float* part = reinterpret_cast<float*>(ws + L.off_part);
          h.C = part; h.ldc = H;
          h.k_split = sp.k_split; h.c_split = cl * H;
          FO_HIP(gemm::run<gemm::kStoreF32>(h, gemm::kWide, st));
          gemm::reduce_splits_bf16<<<2048, 256, 0, st>>>(part, sp.splits, cl * H, H, dH + c0 * H, H);
          FO_HIP(hipGetLastError());
        } else {
          h.C = dH + c0 * H; h.ldc = H;
          FO_HIP(gemm::run<gemm::kStoreBF16>(h, gemm::kNarrow, st));
        }
      }
      // 4. dW contribution
      if (dW != nullptr) {
        FO_HIP(gemm::transpose(dZ, L.Vpad, dZt, L.Cpad, cl, V, clp, st));
        FO_HIP(gemm::transpose(Hm + c0 * H, H, Hct, L.Cpad, cl, H, clp, st));
        gemm::Args w;
        w.A = dZt; w.lda = L.Cpad;
        w.B = Hct; w.ldb = L.Cpad;
        w.C = dW32; w.ldc = H;
        w.M = V; w.N = H; w.K = clp;
        if (c0 == 0) FO_HIP(gemm::run<gemm::kStoreF32>(w, gemm::kWide, st));
        else FO_HIP(gemm::run<gemm::kAccumF32>(w, gemm::kWide, st));
      }
    }
  } else if (dW != nullptr) {
    fill_f32_zero<<<1024, 256, 0, st>>>(dW32, V * H);
    FO_HIP(hipGetLastError());
  }
  if (dW != nullptr && dw_dtype == FO_BF16) {
    cast_f32_bf16<<<4096, 256, 0, st>>>(dW32, static_cast<bf16*>(dW), V * H);
    FO_HIP(hipGetLastError());
  }
  xent::finalize<<<1, 1024, 0, st>>>(T, row_loss, row_z, cnt, loss, z_loss, n_valid, status);
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
