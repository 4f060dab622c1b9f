// bf16 MFMA GEMM for gfx950 (fp32 accumulate), both operands K-contiguous:
//   C[m, n] (=|+=) sum_k A[m, k] * B[n, k]
// used for the three contractions of the fused linear cross-entropy.  The other
// operand layouts are produced by the LDS-tiled transpose below.
//
// Tiling: a 256-thread workgroup (4 wave64s in a 2x2 grid) owns a BM x BN tile of C;
// each wave owns (BM/2) x (BN/2) as 32x32 blocks of v_mfma_f32_32x32x16_bf16.  The K
// loop stages BK-deep slices of A and B in LDS (double-buffered, padded rows so the
// 16-byte fragment reads of the 32 rows of a block fall in different banks); the
// next slice's global loads are issued before the current slice's MFMAs, so HBM/L2
// latency hides behind the matrix math.  One barrier per slice.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[l%32][8(l/32) .. 8(l/32)+7]
// and B[8(l/32) .. +7][l%32]; it receives D[8(r/4) + 4(l/32) + r%4][l%32] in
// accumulator register r = 0..15.
//
// Launch order is XCD-aware: consecutive workgroup ids are dealt round-robin to the 8
// XCDs, so ids are remapped so that each XCD receives a contiguous range of tiles,
// walked in column groups of kGroupM tile rows; tiles that share A rows or B rows
// then run on the same XCD and share its L2.
#pragma once

#include "fo_common.hpp"

namespace fo {
namespace gemm {
namespace {  // internal linkage: each including source file gets its own copy

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum OutMode { kStoreF32 = 0, kAccumF32 = 1, kStoreBF16 = 2 };

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

struct Args {
  const bf16* A;
  const bf16* B;
  void* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
};

// Maps a linear workgroup id to (tile_m, tile_n).
__device__ __forceinline__ void tile_of(int64_t bid, int64_t nbl, int64_t tm, int64_t tn,
                                        int64_t& om, int64_t& on) {
  // XCD remap: ids x, x+8, x+16, ... (all on XCD x % 8) become one contiguous range.
  const int64_t per = nbl / kXcds;
  const int64_t rem = nbl % kXcds;
  const int64_t x = bid % kXcds, i = bid / kXcds;
  int64_t pid;
  if (x < rem) pid = x * (per + 1) + i;
  else pid = rem * (per + 1) + (x - rem) * per + i;
  // grouped order: kGroupM tile rows advance together along n
  const int64_t width = (int64_t)kGroupM * tn;
  const int64_t g = pid / width;
  const int64_t first_m = g * kGroupM;
  const int64_t gm = (tm - first_m < kGroupM) ? tm - first_m : kGroupM;
  const int64_t r = pid - g * width;
  om = first_m + r % gm;
  on = r / gm;
}

// WGM x WGN waves; wave tile (BM/WGM) x (BN/WGN) as FM x FN blocks of 32x32.
template <int BM, int BN, int BK, int WGM, int WGN, int MODE>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_nt(Args a) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int PAD = 8;
  constexpr int LDS_ROW = BK + PAD;                 // elements
  constexpr int WM = BM / WGM, WN = BN / WGN;       // wave tile
  constexpr int FM = WM / 32, FN = WN / 32;         // 32x32 blocks per wave
  constexpr int VPR = BK / 8;                       // 16-byte vectors per row slice
  constexpr int A_LD = BM * VPR / NT;               // vectors per thread per slice
  constexpr int B_LD = BN * VPR / NT;
  static_assert(BM * VPR % NT == 0 && BN * VPR % NT == 0, "tile/threads");
  static_assert(BK % 16 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDS_ROW];

  const int64_t tm_n = ceil_div(a.M, BM), tn_n = ceil_div(a.N, BN);
  int64_t tm, tn;
  tile_of(blockIdx.x, (int64_t)gridDim.x, tm_n, tn_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // global -> register staging
  u32x4 ra[A_LD], rb[B_LD];
  auto load_slice = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * 8;
      const int64_t gm = m0 + r, gk = k0 + c;
      if (gm < a.M && gk < a.K)
        ra[i] = *reinterpret_cast<const u32x4*>(a.A + gm * a.lda + gk);
      else
        ra[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * 8;
      const int64_t gn = n0 + r, gk = k0 + c;
      if (gn < a.N && gk < a.K)
        rb[i] = *reinterpret_cast<const u32x4*>(a.B + gn * a.ldb + gk);
      else
        rb[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_slice = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][r * LDS_ROW + c]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VPR, c = (idx % VPR) * 8;
      *reinterpret_cast<u32x4*>(&Bs[buf][r * LDS_ROW + c]) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int64_t nk = ceil_div(a.K, BK);
  load_slice(0);
  store_slice(0);
  __syncthreads();
  const int fr = lane & 31;         // fragment row within a 32x32 block
  const int fk = (lane >> 5) * 8;   // fragment k offset
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_slice((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &As[cur][(wm * WM + i * 32 + fr) * LDS_ROW + kk + fk]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[cur][(wn * WN + j * 32 + fr) * LDS_ROW + kk + fk]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slice(cur ^ 1);
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WN + j * 32 + fr;
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (m >= a.M) continue;
        if constexpr (MODE == kStoreF32) {
          static_cast<float*>(a.C)[m * a.ldc + n] = acc[i][j][r];
        } else if constexpr (MODE == kAccumF32) {
          float* p = static_cast<float*>(a.C) + m * a.ldc + n;
          *p = *p + acc[i][j][r];
        } else {
          static_cast<bf16*>(a.C)[m * a.ldc + n] = from_f32<bf16>(acc[i][j][r]);
        }
      }
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int MODE>
hipError_t launch_cfg(const Args& a, hipStream_t st) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles == 0) return hipSuccess;
  gemm_nt<BM, BN, BK, WGM, WGN, MODE><<<dim3((unsigned)tiles), dim3(WGM * WGN * 64), 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch(const Args& a, hipStream_t st) {
  return launch_cfg<128, 128, 64, 2, 2, MODE>(a, st);
}

// dst[c, r] = src[r, c] for r < R, c < Cn; dst[c, r] = 0 for R <= r < Rpad.
// 64x64 tiles through LDS (one padding column against bank conflicts).
__global__ __launch_bounds__(256) void transpose_bf16(const bf16* __restrict__ src, int64_t lds,
                                                      bf16* __restrict__ dst, int64_t ldd,
                                                      int64_t R, int64_t Cn, int64_t Rpad) {
  __shared__ bf16 tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cn) ? src[r * lds + c] : from_f32<bf16>(0.f);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < Cn && r < Rpad) dst[c * ldd + r] = tile[tx][i];
  }
}

inline hipError_t transpose(const bf16* src, int64_t lds, bf16* dst, int64_t ldd, int64_t R,
                            int64_t Cn, int64_t Rpad, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(Cn, 64), (unsigned)ceil_div(Rpad, 64));
  transpose_bf16<<<grid, dim3(256), 0, st>>>(src, lds, dst, ldd, R, Cn, Rpad);
  return hipGetLastError();
}

}  // namespace
}  // namespace gemm
}  // namespace fo
