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
  int64_t C, Cpad, Vpad, ldz;
  gemm::SplitPlan dh_split;  // split-K of the dH product (a full chunk)
  size_t off_cnt, off_loss, off_z, off_wt, off_zbuf, off_dz, off_dzt, off_hct, off_dw,
      off_part, off_idx, off_pos, off_tgv, off_hv, off_dhv, total;
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
  const size_t Tn = (size_t)(T > 0 ? T : 1);
  L.off_idx = take(Tn * 4);
  L.off_pos = take(Tn * 4);
  L.off_tgv = take(Tn * 8);
  L.off_hv = take(Tn * H * 2);
  L.off_dhv = take(Tn * H * 2);
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
        live ? *reinterpret_cast<const u32x4*>(src + v * 8) : u32x4{0, 0, 0, 0};
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
        p >= 0 ? *reinterpret_cast<const u32x4*>(src + v * 8) : u32x4{0, 0, 0, 0};
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
  bf16* Wt = reinterpret_cast<bf16*>(ws + L.off_wt);
  float* Z = reinterpret_cast<float*>(ws + L.off_zbuf);
  bf16* dZ = reinterpret_cast<bf16*>(ws + L.off_dz);
  bf16* dZt = reinterpret_cast<bf16*>(ws + L.off_dzt);
  bf16* Hct = reinterpret_cast<bf16*>(ws + L.off_hct);
  int* idx = reinterpret_cast<int*>(ws + L.off_idx);
  int* pos_of = reinterpret_cast<int*>(ws + L.off_pos);
  int64_t* tgv = reinterpret_cast<int64_t*>(ws + L.off_tgv);
  bf16* Hv = reinterpret_cast<bf16*>(ws + L.off_hv);
  bf16* dHv = reinterpret_cast<bf16*>(ws + L.off_dhv);
  float* dW32 = dw_dtype == FO_BF16 ? reinterpret_cast<float*>(ws + L.off_dw)
                                    : static_cast<float*>(dW);

  if (T > 0) {
    xent::compact_targets<<<1, 1024, 0, st>>>(T, V, tg, ignore, cnt, idx, pos_of, tgv);
    gather_rows<<<(unsigned)T, 256, 0, st>>>(Hm, H, idx, cnt, Hv);
    FO_HIP(hipGetLastError());
    if (dH != nullptr) {
      FO_HIP(gemm::transpose(W, H, Wt, L.Vpad, V, H, L.Vpad, st));
      // columns [V, Vpad) of dZ are the zero K-padding of the dH contraction
      fill_bf16_zero<<<1024, 256, 0, st>>>(dZ, L.C * L.Vpad);
      FO_HIP(hipGetLastError());
    }
    const bool need_grad = dH != nullptr || dW != nullptr;
    for (int64_t c0 = 0; c0 < T; c0 += L.C) {
      const int64_t cl = (T - c0 < L.C) ? T - c0 : L.C;  // rows at most (valid rows: on device)
      const int64_t clp = align_up((size_t)cl, 8);
      // 1. logits of the chunk's valid rows
      gemm::Args g;
      g.A = Hv + c0 * H; g.lda = H;
      g.B = W; g.ldb = H;
      g.C = Z; g.ldc = L.ldz;
      g.M = cl; g.N = V; g.K = H;
      g.dev_count = nv; g.count_base = c0; g.dev_dim = 1;
      FO_HIP(gemm::run<gemm::kStoreF32>(g, gemm::kWide, st));
      // 2. loss rows and dZ
      xent::RowArgs r;
      r.T = cl; r.V = V; r.ldz = L.ldz; r.ldd = L.Vpad; r.ignore = ignore; r.zc = zc;
      r.dloss = dloss; r.tg = tgv + c0; r.cnt = cnt; r.row_loss = row_loss + c0;
      r.row_z = row_z + c0; r.dev_rows = nv; r.rows_base = c0;
      FO_HIP(xent::launch_rows<float, bf16>(r, Z, need_grad ? dZ : nullptr, st));
      // 3. dH rows of the chunk (split over the vocabulary when a chunk's 256x256 tiles
      //    cannot fill the chip; the fp32 partials are summed in a fixed order)
      if (dH != nullptr) {
        gemm::Args h;
        h.A = dZ; h.lda = L.Vpad;
        h.B = Wt; h.ldb = L.Vpad;
        h.M = cl; h.N = H; h.K = L.Vpad;
        h.dev_count = nv; h.count_base = c0; h.dev_dim = 1;
        const gemm::SplitPlan sp = gemm::split_plan(cl, H, L.Vpad);
        if (sp.splits > 1 && sp.splits <= L.dh_split.splits) {
          float* part = reinterpret_cast<float*>(ws + L.off_part);
          h.C = part; h.ldc = H;
          h.k_split = sp.k_split; h.c_split = cl * H;
          FO_HIP(gemm::run<gemm::kStoreF32>(h, gemm::kWide, st));
          gemm::reduce_splits_bf16<<<2048, 256, 0, st>>>(part, sp.splits, cl * H, H,
                                                         dHv + c0 * H, H, nv, c0);
          FO_HIP(hipGetLastError());
        } else {
          h.C = dHv + c0 * H; h.ldc = H;
          FO_HIP(gemm::run<gemm::kStoreBF16>(h, gemm::kNarrow, st));
        }
      }
      // 4. dW contribution: K = the chunk's valid rows, rounded up to 64 (the rows
      //    after the valid ones are zero in both transposed operands)
      if (dW != nullptr) {
        FO_HIP(gemm::transpose(dZ, L.Vpad, dZt, L.Cpad, cl, V, clp, st));
        FO_HIP(gemm::transpose(Hv + c0 * H, H, Hct, L.Cpad, cl, H, clp, st));
        gemm::Args w;
        w.A = dZt; w.lda = L.Cpad;
        w.B = Hct; w.ldb = L.Cpad;
        w.C = dW32; w.ldc = H;
        w.M = V; w.N = H; w.K = clp;
        w.dev_count = nv; w.count_base = c0; w.dev_dim = 2;
        if (c0 == 0) FO_HIP(gemm::run<gemm::kStoreF32>(w, gemm::kWide, st));
        else FO_HIP(gemm::run<gemm::kAccumF32>(w, gemm::kWide, st));
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
