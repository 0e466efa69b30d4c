// Tile-level building blocks shared by the loss kernels and the teacher-cache
// builder: the 8-wave 256 x 256 block configuration, fp32 staging of
// accumulators through LDS, and a 256 x 256 output tile of C (+)= A B^T with
// an fp32 epilogue.
#pragma once

#include "fkl_device.h"
#include "fkl_internal.h"

namespace fkl {

constexpr int kStageLd = 132;  // fp32 LDS stride of a staged 256 x 128 half tile

// Block tiles are 256 x 256 with 8 waves (2 per SIMD), each 128 x 64.
constexpr int kNBW = 2;
constexpr int kWN = 4;
using MainCfg = TileCfg<kNBW, kWN>;
constexpr int kBlockThreads = MainCfg::kThreads;  // 512

// Accumulators of one wave of a main block tile: 8 x 4 blocks of 16 x 16.
using MainAcc = f32x4[8][2 * kNBW];

// Waves whose 64 columns fall in half `half` of the tile copy their 128 x 64
// accumulators into a 256 x 128 fp32 LDS half tile (stride kStageLd floats).
__device__ __forceinline__ void stage_half_tile(const MainAcc& acc, float* stage, int wm, int wn, int lane) {
  const int cbase = (wn & 1) * 64;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 2 * kNBW; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stage[(wm * 128 + acc_row(x, i, lane)) * kStageLd + cbase + acc_col(y, lane)] = acc[x][y][i];
}

constexpr int kStageFp32Bytes = kTile * kStageLd * 4;  // 256 x 128 fp32 half tile, padded
constexpr int kKernelLdsBytes =
    kStageFp32Bytes > MainCfg::kLdsBytes ? kStageFp32Bytes : MainCfg::kLdsBytes;

// ---------------------------------------------------------------------------
// Output tiles of C (+)= A B^T with an fp32 read-modify-write epilogue
// ---------------------------------------------------------------------------

struct GemmAccParams {
  Operand A, B;
  int32_t nk;  // contraction stages of 32
  float* C;
  int64_t ldc, m_lim, n_lim;
  int32_t beta;  // 0: C = A B^T, 1: C += A B^T
  int32_t mblocks, nblocks;
  // Split of the contraction: split s covers stages [s * kper, (s + 1) * kper)
  // and writes its own C + s * c_split (splits = 1: no split).
  int32_t splits, kper;
  int64_t c_split;
  DebugCheck dbg;  // debug build: span 0 = C (with every split), 1 = A, 2 = B
};

// Operand restricted to contraction indices [k0, k0 + klen).
template <bool TRANS>
__device__ __forceinline__ Operand k_window(const Operand& op, int64_t k0, int64_t klen) {
  Operand o = op;
  o.base = op.base + (TRANS ? k0 * op.ld : k0);
  o.k_lim = min(klen, op.k_lim - k0);
  return o;
}

// Renumber workgroup w of the contiguous range [first, first + count) so that
// the members of the range on each XCD take one contiguous block of indices.
__device__ __forceinline__ int xcd_contiguous_range(int w, int first, int count) {
  const int x = w % kXcds;
  int before = 0;
  for (int y = 0; y < x; ++y) {
    const int f = first + ((y - first) % kXcds + kXcds) % kXcds;
    before += f < first + count ? (first + count - 1 - f) / kXcds + 1 : 0;
  }
  const int fx = first + ((x - first) % kXcds + kXcds) % kXcds;
  return before + (w - fx) / kXcds;
}

// 256 x 64 output tile of C (+)= A B^T: 8 waves of 32 x 64, fp32 epilogue
// through a 256 x 64 LDS tile (stride kNarrowLd), old values loaded first.
constexpr int kNarrowN = 64;
constexpr int kNarrowLd = kNarrowN + 4;

template <bool TA, bool TB>
__device__ __forceinline__ void narrow_acc_tile(const GemmAccParams& P, const Operand& A, const Operand& B,
                                                int64_t m0, int64_t n0, int nk, float* C, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  f32x4 acc[2][4];
  zero_acc(acc);
  dcheck_operands<TA, TB>(P.dbg, 1, 2, A, B, m0, n0, kNarrowN);
  gemm_mainloop<TA, TB, 2, 1, 1>(A, B, m0, n0, nk, acc, lds);
  const int rmax = static_cast<int>(min<int64_t>(kTile, P.m_lim - m0));
  const int cmax = static_cast<int>(P.n_lim - n0);
  float* ctile = C + m0 * P.ldc + n0;
  constexpr int kPer = (kTile * kNarrowN / 4) / kBlockThreads;  // 16-byte pieces per thread
  f32x4 old[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + i * kBlockThreads;
    const int r = q >> 4;
    const int c4 = (q & 15) * 4;
    old[i] = (P.beta && r < rmax && c4 < cmax)
                 ? dload(P.dbg, 0, kDbgGemmOut,
                         reinterpret_cast<const f32x4*>(ctile + static_cast<int64_t>(r) * P.ldc + c4))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float* stage = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stage[(wave * 32 + acc_row(x, i, lane)) * kNarrowLd + acc_col(y, lane)] = acc[x][y][i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + i * kBlockThreads;
    const int r = q >> 4;
    const int c4 = (q & 15) * 4;
    if (r < rmax && c4 < cmax) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * kNarrowLd + c4);
      dstore(P.dbg, 0, kDbgGemmOut, reinterpret_cast<f32x4*>(ctile + static_cast<int64_t>(r) * P.ldc + c4),
             f32x4{old[i][0] + v[0], old[i][1] + v[1], old[i][2] + v[2], old[i][3] + v[3]});
    }
  }
  __syncthreads();
}

// One output tile of C (+)= A B^T (256 x 256, or 256 x 64 for a last column
// block of at most 64 columns); `local` is this workgroup's index among the
// problem's tiles (XCD-renumbered).
template <bool TA, bool TB>
__device__ __forceinline__ void gemm_acc_tile(const GemmAccParams& P, int local, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;
  const int wn = wave % kWN;
  const int tiles = P.mblocks * P.nblocks;
  const int split = local / tiles;
  int mbi, nbi;
  grouped_tile(local - split * tiles, P.mblocks, P.nblocks, 8, mbi, nbi);
  const int64_t m0 = static_cast<int64_t>(mbi) * kTile;
  const int64_t n0 = static_cast<int64_t>(nbi) * kTile;
  const int64_t k0 = static_cast<int64_t>(split) * P.kper * kStageK;
  const int64_t klen = static_cast<int64_t>(P.kper) * kStageK;
  const int nk = min(P.kper, P.nk - split * P.kper);
  float* C = P.C + split * P.c_split;
  if (P.n_lim - n0 <= kNarrowN) {
    // A last column block of at most 64 columns (d = 2880 leaves one): the
    // 8 waves stack along the rows (32 x 64 each) instead of computing a
    // 256-wide tile that is three quarters zero padding.
    narrow_acc_tile<TA, TB>(P, k_window<TA>(P.A, k0, klen), k_window<TB>(P.B, k0, klen), m0, n0, nk, C, lds);
    return;
  }
  MainAcc acc;
  zero_acc(acc);
  const Operand Aw = k_window<TA>(P.A, k0, klen);
  const Operand Bw = k_window<TB>(P.B, k0, klen);
  dcheck_operands<TA, TB>(P.dbg, 1, 2, Aw, Bw, m0, n0, kTile);
  gemm_mainloop<TA, TB, kNBW, kWN>(Aw, Bw, m0, n0, nk, acc, lds);
  // Epilogue through LDS: each 256 x 128 half tile is staged in fp32, then
  // 32 lanes per row move 512 contiguous bytes with 16-byte accesses. When
  // accumulating, all of a thread's old values for the half are loaded before
  // the staging, so their latency is paid once per half.
  float* stage = reinterpret_cast<float*>(lds);
  const int rmax = static_cast<int>(min<int64_t>(kTile, P.m_lim - m0));
  constexpr int kPer = (kTile * 32) / kBlockThreads;  // 16-byte pieces per thread per half
  for (int half = 0; half < 2; ++half) {
    const int64_t cbase = n0 + half * 128;
    const int cmax = static_cast<int>(min<int64_t>(128, P.n_lim - cbase));
    float* ctile = C + m0 * P.ldc + cbase;
    f32x4 old[kPer];
    if (P.beta) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int q = tid + i * kBlockThreads;
        const int r = q >> 5;
        const int c4 = (q & 31) * 4;
        old[i] = (r < rmax && c4 < cmax)
                     ? dload(P.dbg, 0, kDbgGemmOut,
                             reinterpret_cast<const f32x4*>(ctile + static_cast<int64_t>(r) * P.ldc + c4))
                     : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) old[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if ((wn >> 1) == half) stage_half_tile(acc, stage, wm, wn, lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * kBlockThreads;
      const int r = q >> 5;
      const int c4 = (q & 31) * 4;
      if (r < rmax && c4 < cmax) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * kStageLd + c4);
        dstore(P.dbg, 0, kDbgGemmOut, reinterpret_cast<f32x4*>(ctile + static_cast<int64_t>(r) * P.ldc + c4),
               f32x4{old[i][0] + v[0], old[i][1] + v[1], old[i][2] + v[2], old[i][3] + v[3]});
      }
    }
    __syncthreads();
  }
}

}  // namespace fkl
