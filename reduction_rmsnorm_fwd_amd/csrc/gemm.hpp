// bf16 MFMA GEMM for gfx950 (fp32 accumulate):
//   C[m, n] (=|+=) sum_k A[m, k] * B[n, k]
// used for the three contractions of the fused linear cross-entropy.  Each operand is
// stored either k-contiguous (element (x, k) at p[x*ld + k]) or k-major (at
// p[k*ld + x]); the direct-to-LDS kernel reads both without a transposed copy (the
// k-major one through the transposing LDS loads of gfx950).
//
// Tiling (direct-to-LDS kernel): a 512-thread workgroup (8 wave64s in a 4x2 grid)
// owns a 256x256 tile of C; each wave owns 64x128 as 2x4 blocks of
// v_mfma_f32_32x32x16_bf16.  The K loop stages 64-deep slices of A and B in LDS
// (two stages, unpadded and XOR-swizzled), filled by buffer loads that write LDS
// directly; the next slice's loads are issued before the current slice's MFMAs, so
// HBM/L2 latency hides behind the matrix math.  One barrier per slice.  A register-
// staged kernel (padded LDS rows) serves k-contiguous operands the buffer path cannot
// address (misaligned rows).
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[l%32][8(l/32) .. 8(l/32)+7]
// and B[8(l/32) .. +7][l%32]; it receives D[8(r/4) + 4(l/32) + r%4][l%32] in
// accumulator register r = 0..15.
//
// Launch order is XCD-aware: consecutive workgroup ids are dealt round-robin to the 8
// XCDs, so ids are remapped so that each XCD receives a contiguous range of (split-K
// slice, tile) pairs, walked in column groups of kGroupM tile rows; tiles that share
// A rows or B rows then run on the same XCD and share its L2.
#pragma once

#include "fo_common.hpp"

namespace fo {
namespace gemm {
namespace {  // internal linkage: each including source file gets its own copy

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// kStoreExpStats (logits of a cross-entropy): per row and per wave's WN columns, the
// online-logsumexp partial (m, sum of exp(x - m)) at stats[row * stats_ld + col / WN];
// C (bf16, may be null: then nothing else is stored) receives exp(x - m) of that
// partial's m, in (0, 1]; and the fp32 value at the row's target column tgt[row] goes to
// zy[row].
enum OutMode { kStoreF32 = 0, kAccumF32 = 1, kStoreBF16 = 2, kStoreExpStats = 3 };

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

struct Args {
  const bf16* A;
  const bf16* B;
  void* C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  // split-K: slice y covers the K range [y*k_split, (y+1)*k_split) and writes its
  // fp32 partial at C + y*c_split (elements); k_split = 0: no split.  split_compact:
  // the partials are packed, slice y at C + y*M*ldc for the effective M (so a buffer
  // for the largest slices x rows product the device may choose is enough)
  int64_t k_split = 0;
  int64_t c_split = 0;
  bool split_compact = false;
  // device-side extent: when dev_count is set, the effective M (dev_dim 1) or K
  // (dev_dim 2) is clamp(*dev_count - count_base, 0, M or K), K rounded up to 64 (the
  // operands hold zeros up to that point).  The grid stays sized for the static M;
  // workgroups whose tile starts past the effective M return at once.
  const long long* dev_count = nullptr;
  int64_t count_base = 0;
  int dev_dim = 0;
  // split_max > 0: split-K with the slice count chosen on the device from the
  // effective M (dyn_splits, at most split_max slices); k_split unused
  int64_t split_max = 0;
  // k-major B only: B has b_rows k-rows (counted from the product's first k); the
  // rows past them read as zeros.  0: all K rows exist.
  int64_t b_rows = 0;
  float2* stats = nullptr;  // kStoreExpStats only
  int64_t stats_ld = 0;
  const int64_t* tgt = nullptr;  // kStoreExpStats: target column of each row
  float* zy = nullptr;           // kStoreExpStats: the row's value at that column
};

constexpr int64_t kCus = 256;

// Split-K slice count for an M x N product of 256x256 tiles over K: the count s <=
// smax (each slice at least 2048 deep) that minimises the workgroup waves per unit of
// K, ceil(tiles*s / kCus) / s; ties go to the smaller s (fewer partials to sum).
__host__ __device__ inline int64_t dyn_splits(int64_t M, int64_t N, int64_t K, int64_t smax) {
  const int64_t tiles = ceil_div(M, 256) * ceil_div(N, 256);
  if (tiles <= 0) return 1;
  int64_t best = 1, bw = ceil_div(tiles, kCus);
  for (int64_t s = 2; s <= smax && K / s >= 2048; ++s) {
    const int64_t w = ceil_div(tiles * s, kCus);
    if (w * best < bw * s) { best = s; bw = w; }
  }
  return best;
}

// K extent of each of s split-K slices (a multiple of the 64-deep K step).
__host__ __device__ inline int64_t split_len(int64_t K, int64_t s) {
  return ceil_div(ceil_div(K, s), 64) * 64;
}

// What this workgroup computes: the arguments with the device-side extent applied,
// the split-K slice and the output tile.  The (slice, tile) pairs of the effective
// work take the first workgroup ids (a device-side count may cut it below the grid's
// size; the workgroups past it return false at once), and are remapped so that each
// XCD (ids x, x+8, x+16, ... run on XCD x % 8) gets one contiguous range of them: a
// run of tiles of one slice, walked kGroupM tile rows at a time along n, so the
// workgroups resident on an XCD share operand panels in its L2.
template <int BM, int BN, bool AT = false, bool BT = false>
__device__ __forceinline__ bool locate(const Args& in, Args& a, int64_t& om, int64_t& on) {
  a = in;
  if (in.dev_count != nullptr) {
    int64_t e = *in.dev_count - in.count_base;
    if (e < 0) e = 0;
    if (in.dev_dim == 1) {
      a.M = e < in.M ? e : in.M;
    } else {
      // a k-contiguous operand is read in 8-deep chunks (the caller keeps zeros up to
      // the next multiple of 8); k-major operands stop at the exact row
      if (!AT || !BT) e = (e + 7) / 8 * 8;
      a.K = e < in.K ? e : in.K;
    }
  }
  if (a.b_rows <= 0 || a.b_rows > a.K) a.b_rows = a.K;
  int64_t ns = 1, ks = 0;
  if (in.split_max > 0) ks = split_len(a.K, dyn_splits(a.M, a.N, a.K, in.split_max));
  else if (in.k_split > 0) ks = in.k_split;
  if (ks > 0) ns = ceil_div(a.K, ks);
  const int64_t tm = ceil_div(a.M, BM), tn = ceil_div(a.N, BN);
  const int64_t tiles = tm * tn, total = tiles * ns;
  const int64_t bid = blockIdx.x;
  if (bid >= total) return false;
  const int64_t per = total / kXcds, rem = total % kXcds;
  const int64_t x = bid % kXcds, i = bid / kXcds;
  const int64_t pid = x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int64_t sl = pid / tiles, t = pid - sl * tiles;
  const int64_t width = (int64_t)kGroupM * tn;
  const int64_t g = t / width;
  const int64_t first_m = g * kGroupM;
  const int64_t gm = (tm - first_m < kGroupM) ? tm - first_m : kGroupM;
  const int64_t r = t - g * width;
  om = first_m + r % gm;
  on = r / gm;
  if (ks > 0) {
    const int64_t kb = sl * ks;
    a.A += AT ? kb * in.lda : kb;
    a.B += BT ? kb * in.ldb : kb;
    a.K = (a.K - kb < ks) ? a.K - kb : ks;
    a.b_rows = a.b_rows - kb < 0 ? 0 : (a.b_rows - kb < a.K ? a.b_rows - kb : a.K);
    a.C = static_cast<float*>(in.C) + sl * (in.split_compact ? a.M * in.ldc : in.c_split);
  }
  return true;
}

// WGM x WGN waves; wave tile (BM/WGM) x (BN/WGN) as FM x FN blocks of 32x32.
template <int BM, int BN, int BK, int WGM, int WGN, int MODE>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_nt(Args a_in) {
  Args a;
  int64_t tm, tn;
  if (!locate<BM, BN>(a_in, a, tm, tn)) return;
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

  const int64_t m0 = tm * BM, n0 = tn * BN;
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
// (non-temporal: read once) straight into the accumulator registers before the K loop.  All loads are
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
                (full || (mb + q < a.M && n < a.N)) ? __builtin_nontemporal_load(p + q * a.ldc) : 0.f;
        }
      }
  }
}

// All-reduce over each 32-lane half of a wave (the 32 columns of a fragment row): xor
// 1 and 2 within quads, then the half-row and row mirrors (DPP, no LDS traffic), then
// xor 16 (ds_swizzle, bit-mask mode) — two LDS-path operations instead of five.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return fmaxf(x, xor16_f(x));
}
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x + xor16_f(x);
}

// Epilogue of kStoreExpStats.  Lane (fr, fh) holds, for each of its rows, the FN values
// at columns j*32 + fr of this wave's WN.  Per row: the value at the target column goes
// to zy if that column is one of this wave's; the max over the wave's columns is reduced
// over j and over the 32 lanes of the half-wave; every value is replaced by exp(x - max)
// and their sum reduced the same way; lane fr == 0 writes (max, sum).  Columns at or
// past N do not take part (their values are not stored).
template <int BM, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void exp_stats(const Args& a, f32x16 (&acc)[FM][FN], int64_t m0,
                                          int64_t n0, int wm, int wn, int fr, int fh) {
  const int64_t nb = n0 + wn * WN;  // first column of this wave
  const int64_t part = nb / WN;
  if (nb >= a.N) return;  // no partial slot for a wave wholly past the last column
  // the wave's WM (= 64) rows: lane l loads row l's target, as a column relative to the
  // wave's first column, or -1 when it is not one of the wave's columns; most waves hold
  // no target at all and skip the lookup
  static_assert(WM == 64, "one target per lane");
  const int lane = fr + 32 * fh;
  const int64_t lrow = m0 + wm * WM + lane;
  const int64_t ly = lrow < a.M ? a.tgt[lrow] : -1;
  const int lrel = (ly >= nb && ly < nb + WN && ly < a.N) ? (int)(ly - nb) : -1;
  if (__ballot(lrel >= 0) != 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rw = i * 32 + 8 * (r / 4) + 4 * fh + (r % 4);  // row within the wave
        const int yrel = __shfl(lrel, rw, 64);
        float zv = 0.f;
        bool has = false;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (yrel == j * 32 + fr) { zv = acc[i][j][r]; has = true; }
        if (has) a.zy[m0 + wm * WM + rw] = zv;
      }
  }
  const bool all_cols = nb + WN <= a.N;  // no column of the wave is past N
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * fh + (r % 4);
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (all_cols || nb + j * 32 + fr < a.N) m = fmaxf(m, acc[i][j][r]);
      m = half_max(m);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const float e = __expf(acc[i][j][r] - m);
        acc[i][j][r] = e;
        if (all_cols || nb + j * 32 + fr < a.N) s += e;
      }
      s = half_sum(s);
      if (fr == 0 && row < a.M) a.stats[row * a.stats_ld + part] = make_float2(m, s);
    }
}

// Epilogue: accumulator register r of block (i, j) holds C[8(r/4) + 4 fh + r%4][fr]
// of the block.  Each group of 4 registers is 4 consecutive rows of one column, so a
// row pointer is formed once per group; whole tiles skip the bounds tests.  The stores
// are non-temporal: a product never reads its own output back, and every wave of tiles
// writes more than the whole L2 holds, which would otherwise evict the operand panels
// the next tiles read (12% off the logits-shaped product with an fp32 output, 4% off
// the dW-shaped one).  A 32-lane fp32 store covers one whole 128-byte line of a row;
// for bf16, blocks j and j+1 (64 columns) are first redistributed over the half-wave
// (two lane permutes of packed pairs) so that lane fr holds columns 2fr and 2fr+1 and
// one 4-byte store again covers a whole line (2-byte stores of half lines lose ~3%).
template <int MODE, int BM, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void store_tile(const Args& a, f32x16 (&acc)[FM][FN], int64_t m0,
                                           int64_t n0, int wm, int wn, int fr, int fh) {
  const bool full = m0 + BM <= a.M && n0 + BN <= a.N;
  if constexpr (MODE == kStoreBF16) {
    static_assert(FN % 2 == 0, "pairs of 32-column blocks");
    const bool pairs = ((reinterpret_cast<uintptr_t>(a.C) & 3) | (a.ldc & 1)) == 0;
    // source lanes of this lane's two columns, and the v_perm_b32 byte selector that
    // takes the block-j halves (fr < 16) or the block-(j+1) halves of the packed words
    const int srcA = (((2 * fr) & 31) + 32 * fh) * 4, srcB = (((2 * fr + 1) & 31) + 32 * fh) * 4;
    const uint32_t sel = fr < 16 ? 0x05040100u : 0x07060302u;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jp = 0; jp < FN / 2; ++jp) {
        const int64_t n = n0 + wn * WN + jp * 64 + 2 * fr;  // this lane's first column
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t mb = m0 + wm * WM + i * 32 + 8 * g + 4 * fh;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_bit_cast(unsigned short, from_f32<bf16>(acc[i][2 * jp][4 * g + q]));
            const uint32_t hi = __builtin_bit_cast(unsigned short, from_f32<bf16>(acc[i][2 * jp + 1][4 * g + q]));
            const int w = (int)(lo | (hi << 16));  // columns fr and 32 + fr of the pair
            const uint32_t wA = (uint32_t)__builtin_amdgcn_ds_bpermute(srcA, w);
            const uint32_t wB = (uint32_t)__builtin_amdgcn_ds_bpermute(srcB, w);
            const uint32_t o = __builtin_amdgcn_perm(wB, wA, sel);
            unsigned short* p = reinterpret_cast<unsigned short*>(static_cast<bf16*>(a.C) + (mb + q) * a.ldc + n);
            if (full && pairs) {
              __builtin_nontemporal_store(o, reinterpret_cast<uint32_t*>(p));
            } else if (mb + q < a.M) {
              if (n < a.N) __builtin_nontemporal_store((unsigned short)(o & 0xffffu), p);
              if (n + 1 < a.N) __builtin_nontemporal_store((unsigned short)(o >> 16), p + 1);
            }
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * WN + j * 32 + fr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t mb = m0 + wm * WM + i * 32 + 8 * g + 4 * fh;
          float* p = static_cast<float*>(a.C) + mb * a.ldc + n;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (full || (mb + q < a.M && n < a.N)) __builtin_nontemporal_store(acc[i][j][4 * g + q], p + q * a.ldc);
        }
      }
  }
}

// One operand of the direct-to-LDS kernel: an X (rows of C: m or n) by BK (k) slice
// per stage.  Two storage orders:
//  - K-contiguous (T = false): element (x, k) at p[x*ld + k].  LDS holds [X][BK]; the
//    16-byte chunk c of row r sits at slot c ^ ((r >> SH) & (CPR-1)).  A fragment
//    (8 consecutive k of one row) is one ds_read_b128.
//  - X-contiguous (T = true): element (x, k) at p[k*ld + x].  LDS holds [BK][X]; the
//    16-byte chunk c of k-row r sits at slot c ^ ((r & 3) << 2), so the four k-rows a
//    transposing read touches at once fall in four different 64-byte bank groups.  A
//    fragment is two ds_read_b64_tr_b16: in each 16-lane group, lane j points at the
//    4 x-values (4(j&3) .. +3) of k-row j>>2, and lane i receives the 4 k-values of
//    x = i, i.e. 4 consecutive k of one row of the operand, as the MFMA wants them.
// DMA: each wave issues PW buffer_load_dwordx4 ... lds per slice; lane l of an
// instruction fills LDS slot l of it, so the swizzle is applied by choosing which
// global chunk lane l loads.  Rows past the operand (and, T = false, k past K) read
// as zeros through the buffer range / an out-of-range offset.
template <int X, int BK, int NW, int SH, bool T>
struct DmaOperand {
  static constexpr int CPR = T ? X / 8 : BK / 8;  // 16-byte chunks per LDS row
  static constexpr int RPI = 64 / CPR;            // LDS rows per DMA instruction
  static constexpr int ROWS = T ? BK : X;         // LDS rows per slice
  // Waves that issue the DMA: with 8 waves, the first 4 (one per SIMD) issue all of
  // it, so the other wave of each SIMD keeps its MFMAs going while the issuing one
  // waits for the vector memory queue to take its loads (a few percent faster than
  // all 8 waves issuing at the same moment after the barrier).
  static constexpr int DW = NW >= 8 ? NW / 2 : NW;
  static constexpr int PW = ROWS / RPI / DW;      // DMA instructions per issuing wave
  static_assert(ROWS % (RPI * DW) == 0, "DMA split");
  static_assert(!T || (CPR >= 16 && BK % 16 == 0), "transposed tile shape");
  uint32_t off[PW];          // per-lane byte offset of each instruction's chunk
  __amdgpu_buffer_rsrc_t rs;  // k-contiguous: the tile's row panel
  const bf16* base;          // k-major: the tile's first column at k = 0
  int64_t ldk;               // k-major: elements per k row
  int64_t K;                 // k extent (k-major: the k rows that exist)

  __device__ __forceinline__ int row_of(int i, int wave, int lane) const {
    return (wave * PW + i) * RPI + lane / CPR;
  }
  // the global chunk lane `lane` loads in instruction i (chunk c of LDS row r sits at
  // slot c ^ swizzle(r), and lane l fills slot l % CPR)
  __device__ __forceinline__ int chunk_of(int i, int wave, int lane) const {
    const int r = row_of(i, wave, lane), slot = lane % CPR;
    if constexpr (!T) return slot ^ ((r >> SH) & (CPR - 1));
    else return slot ^ ((r & 3) << 2);
  }

  __device__ __forceinline__ void init(const bf16* p, int64_t ld, int64_t x0, int64_t xn,
                                       int64_t k_extent, int wave, int lane) {
    K = k_extent;
    if constexpr (!T) {
      const int64_t rows = (xn - x0 < X) ? xn - x0 : X;
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p + x0 * ld), (short)0,
                                             (int)(rows * ld * 2), kBufFlags);
#pragma unroll
      for (int i = 0; i < PW; ++i)
        off[i] = (uint32_t)(row_of(i, wave, lane) * ld * 2 + chunk_of(i, wave, lane) * 16);
    } else {
      base = p + x0;
      ldk = ld;
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        const int c = chunk_of(i, wave, lane);
        off[i] = x0 + c * 8 < xn ? (uint32_t)(row_of(i, wave, lane) * ld * 2 + c * 16) : kOob;
      }
    }
  }

  // slice of k0 .. k0+BK-1 into the stage at dst (ROWS x CPR chunks)
  __device__ __forceinline__ void dma(bf16* dst, int64_t k0, int wave, int lane) const {
    if (wave >= DW) return;
    if constexpr (!T) {
      const uint32_t kb = (uint32_t)k0 * 2;
      // only the slice holding the K tail needs the per-lane range test (K % 8 == 0,
      // so a chunk is wholly in or out)
      const bool tail = k0 + BK > K;
      const int krem = (int)(K - k0);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        const uint32_t o = (!tail || chunk_of(i, wave, lane) * 8 < krem) ? off[i] + kb : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(dst + (wave * PW + i) * RPI * CPR * 8),
                                                 16, o, 0, 0, 0);
      }
    } else {
      // a buffer over this slice's k rows only: rows past K read as zeros, and no
      // offset exceeds 64 rows
      const int64_t nrow = (K - k0 < BK) ? K - k0 : BK;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(base + k0 * ldk), (short)0, (int)(nrow > 0 ? nrow * ldk * 2 : 0), kBufFlags);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        // (a local copy: handing the member straight to the builtin makes this hipcc
        // drop the host launch stubs of later instantiations of the kernel)
        const uint32_t o = off[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(dst + (wave * PW + i) * RPI * CPR * 8),
                                                 16, o, 0, 0, 0);
      }
    }
  }
};

// Per-lane LDS byte offsets of the F fragments (32 rows of the operand each) of a
// wave whose first operand row is xoff; frag() adds the k step.
template <int X, int BK, int SH, int F, bool T>
struct FragReader {
  uint32_t base[F];
  __device__ __forceinline__ void init(int xoff, int lane) {
    if constexpr (!T) {
      constexpr int CPR = BK / 8;
      const int fr = lane & 31;
      // every fragment row is fr plus a multiple of 32 and (32 >> SH) & (CPR-1) == 0,
      // so the swizzle term depends only on the lane
      static_assert(((32 >> SH) & (CPR - 1)) == 0, "swizzle period must divide 32");
#pragma unroll
      for (int f = 0; f < F; ++f) base[f] = (uint32_t)((xoff + f * 32 + fr) * BK * 2);
    } else {
      const int g = lane >> 4, j = lane & 15;
      const int krow = 8 * (g >> 1) + (j >> 2);
      const int sw = (j >> 2) << 2;
      const int lco = 2 * (g & 1) + ((j & 3) >> 1);
      const int within = 8 * (j & 1);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int c0 = (xoff + f * 32) / 8;  // first chunk of the fragment's 32 columns
        base[f] = (uint32_t)(krow * X * 2 + (((c0 ^ sw) + lco) * 16) + within);
      }
    }
  }
  // fragment f, k step kk (16 deep) of the stage at src
  __device__ __forceinline__ bf16x8 frag(const bf16* src, int f, int kk, int lane) const {
    const char* b = reinterpret_cast<const char*>(src);
    if constexpr (!T) {
      constexpr int CPR = BK / 8;
      const int fr = lane & 31, fh = lane >> 5;
      const int sw = (fr >> SH) & (CPR - 1);
      const int kof = ((kk * 2 + fh) ^ sw) * 16;
      return *reinterpret_cast<const bf16x8*>(b + base[f] + kof);
    } else {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const char* p0 = b + base[f] + kk * 16 * X * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(p0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(p0 + 4 * X * 2));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

template <int BM, int BN, int BK, int WGM, int WGN, int ST, int SH, int MODE, bool AT = false,
          bool BT = false>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_nt_dma(Args a_in) {
  Args a;
  int64_t tm, tn;
  if (!locate<BM, BN, AT, BT>(a_in, a, tm, tn)) return;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(ST == 2 || ST == 3, "stages");
  static_assert(BK == 32 || BK == 64, "BK");
  using OpA = DmaOperand<BM, BK, NW, SH, AT>;
  using OpB = DmaOperand<BN, BK, NW, SH, BT>;

  __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * BK], sB0[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * BK], sB1[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA2[ST == 3 ? BM * BK : 8], sB2[ST == 3 ? BN * BK : 8];

  const int64_t m0 = tm * BM, n0 = tn * BN;
  if (MODE == kAccumF32 && a.K == 0) return;  // nothing to add
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  OpA opa;
  OpB opb;
  opa.init(a.A, a.lda, m0, a.M, a.K, wave, lane);
  opb.init(a.B, a.ldb, n0, a.N, BT ? a.b_rows : a.K, wave, lane);
  auto dma = [&](bf16* dA, bf16* dB, int64_t k0) {
    opa.dma(dA, k0, wave, lane);
    opb.dma(dB, k0, wave, lane);
  };

  f32x16 acc[FM][FN];
  const int fr = lane & 31;
  const int fh = lane >> 5;
  FragReader<BM, BK, SH, FM, AT> ra;
  FragReader<BN, BK, SH, FN, BT> rb;
  ra.init(wm * WM, lane);
  rb.init(wn * WN, lane);
  auto compute = [&](const bf16* cA, const bf16* cB) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = ra.frag(cA, i, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = rb.frag(cB, j, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  constexpr int PER_WAVE = OpA::PW + OpB::PW;
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

  if constexpr (MODE == kStoreExpStats) {
    exp_stats<BM, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
    if (a.C != nullptr) store_tile<kStoreBF16, BM, BN, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
  } else {
    store_tile<MODE, BM, BN, WM, WN, FM, FN>(a, acc, m0, n0, wm, wn, fr, fh);
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST, int SH, int MODE, bool AT = false,
          bool BT = false>
hipError_t launch_dma(const Args& a, hipStream_t st) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles == 0) return hipSuccess;
  const int64_t splits = a.split_max > 0 ? a.split_max
                       : a.k_split > 0   ? ceil_div(a.K, a.k_split)
                                         : 1;
  gemm_nt_dma<BM, BN, BK, WGM, WGN, ST, SH, MODE, AT, BT>
      <<<dim3((unsigned)(tiles * splits)), dim3(WGM * WGN * 64), 0, st>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, int MODE>
hipError_t launch_cfg(const Args& a, hipStream_t st) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles == 0) return hipSuccess;
  const int64_t splits = a.split_max > 0 ? a.split_max
                       : a.k_split > 0   ? ceil_div(a.K, a.k_split)
                                         : 1;
  gemm_nt<BM, BN, BK, WGM, WGN, MODE>
      <<<dim3((unsigned)(tiles * splits)), dim3(WGM * WGN * 64), 0, st>>>(a);
  return hipGetLastError();
}

// Tile choice per product.  kWide: 256x256x64, 8 waves (4x2, 64x128 per wave), two
// LDS stages (128 KB); kNarrow: 128x128x64, 4 waves, for products with too few 256^2
// tiles to fill the 256 CUs.  The direct-to-LDS kernel needs 16-byte aligned rows,
// K % 8 == 0 and 32-bit buffer offsets within a tile's row panel; otherwise the
// register-staged kernel runs (same arithmetic, same results).
enum TileShape { kWide = 0, kNarrow = 1 };

// Whether the direct-to-LDS kernel can read the operands: 16-byte aligned bases and
// rows, 32-bit buffer offsets within a tile's row panel (k-contiguous) and k-contiguous
// rows read in whole 8-deep chunks (K % 8 == 0); a k-major operand's rows hold at
// least the X extent rounded up to 8 (its last chunk is read whole).
template <bool AT, bool BT>
inline bool dma_ok(const Args& a, int bm, int bn) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B)) & 15) == 0;
  const int64_t lim = (int64_t)1 << 31;
  auto op_ok = [&](bool t, int64_t ld, int64_t x, int tile) {
    if (ld % 8 != 0) return false;
    if (t) return ld >= (x + 7) / 8 * 8 && 64 * ld * 2 < lim;
    return a.K % 8 == 0 && (int64_t)tile * ld * 2 < lim;
  };
  return aligned && op_ok(AT, a.lda, a.M, bm) && op_ok(BT, a.ldb, a.N, bn);
}

// Runs C (op)= A B^T.  AT / BT: A or B is stored k-major (element (x, k) at
// p[k*ld + x]); those layouts exist in the direct-to-LDS kernel only.
template <int MODE, bool AT = false, bool BT = false>
hipError_t run(const Args& a, TileShape shape, hipStream_t st) {
  if constexpr (MODE == kStoreExpStats) {
    // the row partials come from the direct-to-LDS kernel's wide tile only (its waves
    // cover kStatsCols columns each)
    if (shape != kWide || !dma_ok<AT, BT>(a, 256, 256)) return hipErrorInvalidValue;
    return launch_dma<256, 256, 64, 4, 2, 2, 1, MODE, AT, BT>(a, st);
  } else if constexpr (AT || BT) {
    if (shape == kWide) {
      if (!dma_ok<AT, BT>(a, 256, 256)) return hipErrorInvalidValue;
      return launch_dma<256, 256, 64, 4, 2, 2, 1, MODE, AT, BT>(a, st);
    }
    if (!dma_ok<AT, BT>(a, 128, 128)) return hipErrorInvalidValue;
    return launch_dma<128, 128, 64, 2, 2, 2, 1, MODE, AT, BT>(a, st);
  } else {
    if (shape == kWide) {
      if (dma_ok<false, false>(a, 256, 256)) return launch_dma<256, 256, 64, 4, 2, 2, 1, MODE>(a, st);
      return launch_cfg<256, 256, 64, 4, 2, MODE>(a, st);
    }
    if (dma_ok<false, false>(a, 128, 128)) return launch_dma<128, 128, 64, 2, 2, 2, 1, MODE>(a, st);
    return launch_cfg<128, 128, 64, 2, 2, MODE>(a, st);
  }
}

// columns per row partial of kStoreExpStats (the wide tile's wave width)
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

// Largest (slice count x rows) a product of at most M rows (N columns, K deep, at most
// smax slices, dyn_splits on the device) can choose: the rows of a packed partial
// buffer (Args::split_compact).  dyn_splits depends on M only through its 256-row tile
// count, so the largest M of each tile count is the worst case.
inline int64_t split_rows_bound(int64_t M, int64_t N, int64_t K, int64_t smax) {
  int64_t worst = 0;
  for (int64_t m = 256; m < M + 256; m += 256) {
    const int64_t rows = m < M ? m : M;
    const int64_t s = dyn_splits(rows, N, K, smax);
    if (s * rows > worst) worst = s * rows;
  }
  return worst;
}

// out[m, n] = bf16(sum_s part[s, m, n]) summed in the order s = 0, 1, ...
// (dev_rows: only rows m < *dev_rows - rows_base exist; split_max > 0: the slice count
// is dyn_splits of those rows, as the product chose it, for a K-deep product;
// compact: the partials are packed, slice s at part + s * rows * N for the rows that
// exist, as the product wrote them with Args::split_compact.)
__global__ __launch_bounds__(256) void reduce_splits_bf16(const float* __restrict__ part,
                                                          int64_t splits, int64_t MN,
                                                          int64_t N, bf16* __restrict__ out,
                                                          int64_t ldo,
                                                          const long long* dev_rows,
                                                          int64_t rows_base, int64_t K,
                                                          int64_t split_max, bool compact) {
  int64_t len = MN;  // elements to reduce; MN stays the stride between partials
  if (dev_rows != nullptr) {
    int64_t eff = *dev_rows - rows_base;
    eff = eff < 0 ? 0 : eff;
    if (eff * N < len) len = eff * N;
  }
  if (split_max > 0) splits = ceil_div(K, split_len(K, dyn_splits(len / N, N, K, split_max)));
  const int64_t stride = compact ? len : MN;
  for (int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x; e4 * 4 < len;
       e4 += (int64_t)gridDim.x * 256) {
    const int64_t e = e4 * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t s = 0; s < splits; ++s) {
      const float4 p = *reinterpret_cast<const float4*>(part + s * stride + e);
      v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = (e + q) / N, n = (e + q) - m * N;
      out[m * ldo + n] = from_f32<bf16>(v[q]);
    }
  }
}

}  // namespace
}  // namespace gemm
}  // namespace fo
