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

// kStoreF32Stats: fp32 store plus, per row, the (max, sum of exp(x - max)) pair of each
// wave's WN columns (an online-logsumexp partial) at stats[row * stats_ld + col / WN].
enum OutMode { kStoreF32 = 0, kAccumF32 = 1, kStoreBF16 = 2, kStoreF32Stats = 3 };

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

struct Args {
  const bf16* A;
  const bf16* B;
  void* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  // split-K: workgroup row blockIdx.y covers K range [y*k_split, (y+1)*k_split) and
  // writes its fp32 partial at C + y*c_split (elements); k_split = 0: no split
  int64_t k_split = 0;
  int64_t c_split = 0;
  // device-side extent: when dev_count is set, the effective M (dev_dim 1) or K
  // (dev_dim 2) is clamp(*dev_count - count_base, 0, M or K), K rounded up to 64 (the
  // operands hold zeros up to that point).  The grid stays sized for the static M;
  // workgroups whose tile starts past the effective M return at once.
  const long long* dev_count = nullptr;
  int64_t count_base = 0;
  int dev_dim = 0;
  float2* stats = nullptr;  // kStoreF32Stats only
  int64_t stats_ld = 0;
};

// The K slice of this workgroup row (split-K), applied to a copy of the arguments.
__device__ __forceinline__ Args split_args(const Args& in) {
  Args a = in;
  if (in.dev_count != nullptr) {
    int64_t e = *in.dev_count - in.count_base;
    if (e < 0) e = 0;
    if (in.dev_dim == 1) {
      a.M = e < in.M ? e : in.M;
    } else {
      e = (e + 63) / 64 * 64;
      a.K = e < in.K ? e : in.K;
    }
  }
  if (in.k_split > 0) {
    const int64_t kb = (int64_t)blockIdx.y * in.k_split;
    a.A += kb;
    a.B += kb;
    a.K = (in.K - kb < in.k_split) ? in.K - kb : in.k_split;
    a.C = static_cast<float*>(in.C) + (int64_t)blockIdx.y * in.c_split;
  }
  return a;
}

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
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_nt(Args a_in) {
  const Args a = split_args(a_in);
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

  const int64_t tm_n = ceil_div(a_in.M, BM), tn_n = ceil_div(a_in.N, BN);
  int64_t tm, tn;
  tile_of(blockIdx.x, (int64_t)gridDim.x, tm_n, tn_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  if (m0 >= a.M) return;  // past a device-side row count
  if (MODE == kAccumF32 && a.K == 0) return;  // nothing to add

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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant.  Each wave moves its share of a K slice with
// buffer_load_dwordx4 ... lds (64 lanes x 16 bytes = one contiguous 1 KB run of LDS
// per instruction, no VGPR staging, no ds_write).  Buffer resources cover the tile's
// row panel, so rows past M/N and the K tail read as zero.  The LDS tile is unpadded
// and XOR-swizzled: row r keeps its 16-byte chunk c in slot c ^ ((r >> SH) & (CPR-1)),
// which spreads the 32 rows of a fragment read over distinct banks.  ST stages rotate
// through separate LDS arrays (distinct objects, so the compiler can tell the DMA
// target of slice k+1 from the slice being read); with ST = 3 one barrier per slice
// separates "slice k landed" from "slice k-1 no longer read".
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_vptr;
constexpr int kBufFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr uint32_t kOob = 0x80000000u;  // voffset that is always out of range

__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt at their maxima)
  // (n is a compile-time constant at every call site)
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8)); break;
    case 4: __builtin_amdgcn_s_waitcnt((4 & 15) | (7 << 4) | (15 << 8)); break;
    case 8: __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8)); break;
    case 16: __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | (7 << 4) | (15 << 8)); break;
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
}

// Accumulator start values: zero, or (accumulate mode) the current C tile, loaded
// straight into the accumulator registers before the K loop.  All loads are
// independent, so they are in flight together with the first K slices' DMA.
template <int MODE, int BM, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void init_tile(const Args& a, f32x16 (&acc)[FM][FN], int64_t m0,
                                          int64_t n0, int wm, int wn, int fr, int fh) {
  if constexpr (MODE != kAccumF32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  } else {
    const bool full = m0 + BM <= a.M && n0 + BN <= a.N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + fr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t mb = m0 + wm * WM + i * 32 + 8 * g + 4 * fh;
          const float* p = static_cast<const float*>(a.C) + mb * a.ldc + n;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i][j][4 * g + q] =
                (full || (mb + q < a.M && n < a.N)) ? p[q * a.ldc] : 0.f;
        }
      }
  }
}

// Row partials of an online logsumexp over this wave's WN columns (kStoreF32Stats).
// Lane (fr, fh) holds, for each of its rows, the FN values at columns j*32 + fr.  The
// row max is folded over j and over the 32 lanes of the half-wave (butterfly), then the
// sum of exp(x - max) the same way; lane fr == 0 writes the pair.
// Columns at or past N do not take part.
template <int BM, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void row_stats(const Args& a, f32x16 (&acc)[FM][FN], int64_t m0,
                                          int64_t n0, int wm, int wn, int fr, int fh) {
  const int64_t nb = n0 + wn * WN;  // first column of this wave
  const int64_t part = nb / WN;
  if (nb >= a.N) return;  // no partial slot for a wave wholly past the last column
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // the row's max over the wave's columns first (max only), then one exp per value
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (nb + j * 32 + fr < a.N) m = fmaxf(m, acc[i][j][r]);
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (nb + j * 32 + fr < a.N) s += __expf(acc[i][j][r] - m);
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o, 64);
      const int64_t row = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * fh + (r % 4);
      if (fr == 0 && row < a.M) a.stats[row * a.stats_ld + part] = make_float2(m, s);
    }
}

// Epilogue: accumulator register r of block (i, j) holds C[8(r/4) + 4 fh + r%4][fr]
// of the block.  Each group of 4 registers is 4 consecutive rows of one column, so a
// row pointer is formed once per group; whole tiles skip the bounds tests.
template <int MODE, int BM, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void store_tile(const Args& a, f32x16 (&acc)[FM][FN], int64_t m0,
                                           int64_t n0, int wm, int wn, int fr, int fh) {
  const bool full = m0 + BM <= a.M && n0 + BN <= a.N;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WN + j * 32 + fr;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t mb = m0 + wm * WM + i * 32 + 8 * g + 4 * fh;
        if constexpr (MODE == kStoreBF16) {
          bf16* p = static_cast<bf16*>(a.C) + mb * a.ldc + n;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (full || (mb + q < a.M && n < a.N)) p[q * a.ldc] = from_f32<bf16>(acc[i][j][4 * g + q]);
        } else {
          float* p = static_cast<float*>(a.C) + mb * a.ldc + n;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (full || (mb + q < a.M && n < a.N)) p[q * a.ldc] = acc[i][j][4 * g + q];
        }
      }
    }
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST, int SH, int MODE>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_nt_dma(Args a_in) {
  const Args a = split_args(a_in);
  constexpr int NW = WGM * WGN;
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per DMA instruction
  constexpr int A_PW = BM / RPI / NW;         // DMA instructions per wave per slice
  constexpr int B_PW = BN / RPI / NW;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "DMA split");
  static_assert(ST == 2 || ST == 3, "stages");
  static_assert(BK == 32 || BK == 64, "BK");

  __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * BK], sB0[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * BK], sB1[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA2[ST == 3 ? BM * BK : 8], sB2[ST == 3 ? BN * BK : 8];

  const int64_t tm_n = ceil_div(a_in.M, BM), tn_n = ceil_div(a_in.N, BN);
  int64_t tm, tn;
  tile_of(blockIdx.x, (int64_t)gridDim.x, tm_n, tn_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  if (m0 >= a.M) return;  // past a device-side row count
  if (MODE == kAccumF32 && a.K == 0) return;  // nothing to add
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t rows_a = (a.M - m0 < BM) ? a.M - m0 : BM;
  const int64_t rows_b = (a.N - n0 < BN) ? a.N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.A + m0 * a.lda), (short)0, (int)(rows_a * a.lda * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.B + n0 * a.ldb), (short)0, (int)(rows_b * a.ldb * 2), kBufFlags);

  // per-lane source row / chunk of each DMA instruction (fixed over K)
  const int rl = lane / CPR, slot = lane % CPR;
  uint32_t offa[A_PW], offb[B_PW];
  int ca[A_PW], cb[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int r = (wave * A_PW + i) * RPI + rl;
    ca[i] = slot ^ ((r >> SH) & (CPR - 1));
    offa[i] = (uint32_t)(r * a.lda * 2 + ca[i] * 16);
  }
#pragma unroll
  for (int i = 0; i < B_PW; ++i) {
    const int r = (wave * B_PW + i) * RPI + rl;
    cb[i] = slot ^ ((r >> SH) & (CPR - 1));
    offb[i] = (uint32_t)(r * a.ldb * 2 + cb[i] * 16);
  }
  // K offset of each lane's chunk inside a slice; only the slice holding the K tail
  // needs the per-lane range test (K % 8 == 0, so a chunk is wholly in or out).
  const int64_t k_full = (a.K / BK) * BK;
  auto dma = [&](bf16* dA, bf16* dB, int64_t k0) {
    const uint32_t kb = (uint32_t)(k0 * 2);
    const bool tail = k0 >= k_full;
    const int krem = (int)(a.K - k0);
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
      const uint32_t off = (!tail || ca[i] * 8 < krem) ? offa[i] + kb : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_vptr)(dA + (wave * A_PW + i) * RPI * BK), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
      const uint32_t off = (!tail || cb[i] * 8 < krem) ? offb[i] + kb : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_vptr)(dB + (wave * B_PW + i) * RPI * BK), 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
  const int fr = lane & 31;
  const int fh = lane >> 5;
  // Every fragment row this lane reads is fr plus a multiple of 32, and
  // (32 >> SH) & (CPR-1) == 0, so the swizzle term depends only on the lane: the
  // chunk of k-step kk sits at slot (2kk + fh) ^ sw of each of those rows.
  static_assert(((32 >> SH) & (CPR - 1)) == 0, "swizzle period must divide 32");
  const int sw = (fr >> SH) & (CPR - 1);
  const int a_row = (wm * WM + fr) * BK;
  const int b_row = (wn * WN + fr) * BK;
  auto compute = [&](const bf16* cA, const bf16* cB) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
      const int kof = ((kk * 2 + fh) ^ sw) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(cA + a_row + i * 32 * BK + kof);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(cB + b_row + j * 32 * BK + kof);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  constexpr int PER_WAVE = A_PW + B_PW;
  const int64_t nk = ceil_div(a.K, BK);
  // One step: wait until slice kt has landed (allowing the younger slices still in
  // flight), barrier (slice kt visible to all waves; every wave is done with slice
  // kt-1, whose stage the next DMA reuses), issue the DMA of slice kt+ST-1, compute kt.
  // The loops run whole periods of ST steps (static stage buffers, one exit) and the
  // remainder follows.
  if constexpr (ST == 2) {
    auto step = [&](bf16* cA, bf16* cB, bf16* nA, bf16* nB, int64_t kt) {
      wait_vm(0);
      __syncthreads();
      if (kt + 1 < nk) dma(nA, nB, (kt + 1) * BK);
      compute(cA, cB);
    };
    dma(sA0, sB0, 0);
    init_tile<MODE, BM, BN, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
    int64_t kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      step(sA0, sB0, sA1, sB1, kt);
      step(sA1, sB1, sA0, sB0, kt + 1);
    }
    if (kt < nk) step(sA0, sB0, sA1, sB1, kt);
  } else {
    auto step = [&](bf16* cA, bf16* cB, bf16* nA, bf16* nB, int64_t kt) {
      if (kt + 1 < nk) wait_vm(PER_WAVE); else wait_vm(0);
      __syncthreads();
      if (kt + 2 < nk) dma(nA, nB, (kt + 2) * BK);
      compute(cA, cB);
    };
    dma(sA0, sB0, 0);
    if (nk > 1) dma(sA1, sB1, BK);
    init_tile<MODE, BM, BN, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
    int64_t kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
      step(sA0, sB0, sA2, sB2, kt);
      step(sA1, sB1, sA0, sB0, kt + 1);
      step(sA2, sB2, sA1, sB1, kt + 2);
    }
    if (kt < nk) step(sA0, sB0, sA2, sB2, kt);
    if (kt + 1 < nk) step(sA1, sB1, sA0, sB0, kt + 1);
  }

  if constexpr (MODE == kStoreF32Stats) row_stats<BM, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
  store_tile<MODE == kStoreF32Stats ? kStoreF32 : MODE, BM, BN, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST, int SH, int MODE>
hipError_t launch_dma(const Args& a, hipStream_t st) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles == 0) return hipSuccess;
  const unsigned splits = a.k_split > 0 ? (unsigned)ceil_div(a.K, a.k_split) : 1u;
  gemm_nt_dma<BM, BN, BK, WGM, WGN, ST, SH, MODE>
      <<<dim3((unsigned)tiles, splits), dim3(WGM * WGN * 64), 0, st>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, int MODE>
hipError_t launch_cfg(const Args& a, hipStream_t st) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles == 0) return hipSuccess;
  const unsigned splits = a.k_split > 0 ? (unsigned)ceil_div(a.K, a.k_split) : 1u;
  gemm_nt<BM, BN, BK, WGM, WGN, MODE>
      <<<dim3((unsigned)tiles, splits), dim3(WGM * WGN * 64), 0, st>>>(a);
  return hipGetLastError();
}

// Tile choice per product.  kWide: 256x256x64, 8 waves (4x2, 64x128 per wave), two
// LDS stages (128 KB); kNarrow: 128x128x64, 4 waves, for products with too few 256^2
// tiles to fill the 256 CUs.  The direct-to-LDS kernel needs 16-byte aligned rows,
// K % 8 == 0 and 32-bit buffer offsets within a tile's row panel; otherwise the
// register-staged kernel runs (same arithmetic, same results).
enum TileShape { kWide = 0, kNarrow = 1 };

inline bool dma_ok(const Args& a, int bm, int bn) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B)) & 15) == 0;
  const int64_t lim = (int64_t)1 << 31;
  return aligned && a.K % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
         (int64_t)bm * a.lda * 2 < lim && (int64_t)bn * a.ldb * 2 < lim;
}

template <int MODE>
hipError_t run(const Args& a, TileShape shape, hipStream_t st) {
  if constexpr (MODE == kStoreF32Stats) {
    // the row partials come from the direct-to-LDS kernel's wide tile only (its waves
    // cover kStatsCols columns each)
    if (shape != kWide || !dma_ok(a, 256, 256)) return hipErrorInvalidValue;
    return launch_dma<256, 256, 64, 4, 2, 2, 1, MODE>(a, st);
  } else {
    if (shape == kWide) {
      if (dma_ok(a, 256, 256)) return launch_dma<256, 256, 64, 4, 2, 2, 1, MODE>(a, st);
      return launch_cfg<256, 256, 64, 4, 2, MODE>(a, st);
    }
    if (dma_ok(a, 128, 128)) return launch_dma<128, 128, 64, 2, 2, 2, 1, MODE>(a, st);
    return launch_cfg<128, 128, 64, 2, 2, MODE>(a, st);
  }
}

// columns per row partial of kStoreF32Stats (the wide tile's wave width)
constexpr int kStatsCols = 128;

// Split-K plan for a product whose 256x256 tiles cannot fill the chip: the number of
// K slices (a multiple of the 64-deep K step each) and the partial buffer it needs.
struct SplitPlan {
  int64_t splits, k_split;
};
inline SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ceil_div(M, 256) * ceil_div(N, 256);
  int64_t s = ceil_div(512, tiles > 0 ? tiles : 1);
  if (s > 8) s = 8;
  while (s > 1 && K / s < 2048) --s;
  if (s <= 1) return {1, 0};
  const int64_t ks = ceil_div(ceil_div(K, s), 64) * 64;
  return {ceil_div(K, ks), ks};
}

// out[m, n] = bf16(sum_s part[s, m, n]) summed in the order s = 0, 1, ...
// (dev_rows: only rows m < *dev_rows - rows_base exist.)
__global__ __launch_bounds__(256) void reduce_splits_bf16(const float* __restrict__ part,
                                                          int64_t splits, int64_t MN,
                                                          int64_t N, bf16* __restrict__ out,
                                                          int64_t ldo,
                                                          const long long* dev_rows,
                                                          int64_t rows_base) {
  int64_t len = MN;  // elements to reduce; MN stays the stride between partials
  if (dev_rows != nullptr) {
    int64_t eff = *dev_rows - rows_base;
    eff = eff < 0 ? 0 : eff;
    if (eff * N < len) len = eff * N;
  }
  for (int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x; e4 * 4 < len;
       e4 += (int64_t)gridDim.x * 256) {
    const int64_t e = e4 * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t s = 0; s < splits; ++s) {
      const float4 p = *reinterpret_cast<const float4*>(part + s * MN + e);
      v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = (e + q) / N, n = (e + q) - m * N;
      out[m * ldo + n] = from_f32<bf16>(v[q]);
    }
  }
}

// dst[c, r] = src[r, c] for r < R, c < Cn; dst[c, r] = 0 for R <= r < Rpad.
// 64x64 tiles: 16-byte loads along src rows into LDS, 16-byte stores along dst rows
// gathered from LDS columns (rows of 65 words: a column walk hits distinct banks).
// Requires 16-byte aligned src/dst rows (lds % 8 == 0, ldd % 8 == 0) and Cn % 8 == 0.
__global__ __launch_bounds__(256) void transpose_bf16_v(const bf16* __restrict__ src, int64_t lds,
                                                        bf16* __restrict__ dst, int64_t ldd,
                                                        int64_t R, int64_t Cn, int64_t Rpad) {
  __shared__ uint32_t tile[64][65];  // tile[r][c/2]: bf16 pairs of row r
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x;
  // load: 64 rows x 8 vectors; thread t -> (row t/8 + 32i, vector t%8)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = t / 8 + 32 * i, v = t % 8;
    const int64_t gr = r0 + r, gc = c0 + v * 8;
    u32x4 d = u32x4{0, 0, 0, 0};
    if (gr < R && gc < Cn) d = *reinterpret_cast<const u32x4*>(src + gr * lds + gc);
    tile[r][v * 4 + 0] = d.x;
    tile[r][v * 4 + 1] = d.y;
    tile[r][v * 4 + 2] = d.z;
    tile[r][v * 4 + 3] = d.w;
  }
  __syncthreads();
  // store: dst row c (64 of them) x 8 vectors of 8 src rows; thread t -> (c t/8 + 32i, vector t%8)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = t / 8 + 32 * i, v = t % 8;
    const int64_t gc = c0 + c, gr = r0 + v * 8;
    if (gc >= Cn || gr >= Rpad) continue;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = tile[v * 8 + 2 * q][c / 2], hi = tile[v * 8 + 2 * q + 1][c / 2];
      const uint32_t a = (c & 1) ? (lo >> 16) : (lo & 0xffffu);
      const uint32_t b = (c & 1) ? (hi >> 16) : (hi & 0xffffu);
      w[q] = a | (b << 16);
    }
    if (gr + 8 <= Rpad) {
      *reinterpret_cast<u32x4*>(dst + gc * ldd + gr) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      const bf16* e = reinterpret_cast<const bf16*>(w);
      for (int q = 0; q < 8 && gr + q < Rpad; ++q) dst[gc * ldd + gr + q] = e[q];
    }
  }
}

// Scalar form for shapes the vector form does not take.
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
  const bool vec = lds % 8 == 0 && ldd % 8 == 0 && Cn % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  if (vec) transpose_bf16_v<<<grid, dim3(256), 0, st>>>(src, lds, dst, ldd, R, Cn, Rpad);
  else transpose_bf16<<<grid, dim3(256), 0, st>>>(src, lds, dst, ldd, R, Cn, Rpad);
  return hipGetLastError();
}

}  // namespace
}  // namespace gemm
}  // namespace fo
