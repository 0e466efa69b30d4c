// Device building blocks for libfkl on gfx950 (CDNA4): bf16 MFMA block tiles
// staged through LDS, with loaders for operands stored contraction-contiguous
// ("plain") or contraction-strided ("transposed").
//
// Block tile: 256 (M) x BN (N) x 64 (K) per LDS stage, 256 threads = 4 waves
// in a 2 x 2 arrangement; each wave owns 128 x BN/2 of the output as
// 4 x (BN/64) accumulators of v_mfma_f32_32x32x16_bf16 (32 x 32, fp32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;       // block rows
constexpr int kBK = 64;        // contraction depth of one LDS stage
constexpr int kLDK = kBK + 8;  // LDS row stride in bf16 elements (144 B: 16 B skew per row)
constexpr int kThreads = 256;  // four wave64s
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element (mn, k) of a GEMM operand. Plain: base[mn * ld + k] (k contiguous).
// Transposed: base[k * ld + mn] (mn contiguous). Loads outside
// [0, mn_lim) x [0, k_lim) read as zero. mn_lim and k_lim are multiples of 8
// on the contiguous side, so a 16-byte chunk is either wholly in or out.
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int64_t mn_lim;
  int64_t k_lim;
};

// R x 64 tile of a plain operand: R*8 16-byte chunks, R/32 per thread.
// Eight consecutive lanes read one 128-byte row segment. Addresses are a
// uniform 64-bit tile base plus 32-bit per-lane offsets (element units).
template <int R>
struct PlainLoader {
  static constexpr int kPer = R * 8 / kThreads;
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const Operand& op, int64_t mn0, int64_t k0, int tid) {
    const uint16_t* tile = op.base + mn0 * op.ld + k0;
    const int row = tid >> 3;
    const int kc = (tid & 7) * 8;
    const uint32_t off0 = static_cast<uint32_t>(row * op.ld + kc);
    const uint32_t step = static_cast<uint32_t>(32 * op.ld);
    const bool k_ok = k0 + kc < op.k_lim;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (k_ok && mn0 + row + 32 * i < op.mn_lim) {
        v[i] = *reinterpret_cast<const u32x4*>(tile + (off0 + i * step));
      } else {
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int base = (tid >> 3) * kLDK + (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(lds + base + i * 32 * kLDK) = v[i];
  }
};

// R x 64 tile of a transposed operand. Thread t < R owns the 8 (k) x 8 (mn)
// block (k-group t & 7, mn-group t >> 3): eight 16-byte row loads, an 8 x 8
// transpose of 16-bit lanes in registers, eight 16-byte LDS stores that land
// the tile k-contiguous like a plain one. Eight consecutive lanes cover one
// 128-byte segment of each global row and one 128-byte LDS row segment.
template <int R>
struct TransLoader {
  u32x4 v[8];

  __device__ __forceinline__ void load(const Operand& op, int64_t mn0, int64_t k0, int tid) {
    if (tid >= R) return;
    const uint16_t* tile = op.base + k0 * op.ld + mn0;
    const int kb = (tid & 7) * 8;
    const int mg = (tid >> 3) * 8;
    const uint32_t off0 = static_cast<uint32_t>(kb * op.ld + mg);
    const uint32_t step = static_cast<uint32_t>(op.ld);
    const bool mn_ok = mn0 + mg < op.mn_lim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (mn_ok && k0 + kb + i < op.k_lim) {
        v[i] = *reinterpret_cast<const u32x4*>(tile + (off0 + i * step));
      } else {
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    if (tid >= R) return;
    const int base = (tid >> 3) * 8 * kLDK + (tid & 7) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = v[2 * q][j >> 1];
        const uint32_t b = v[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(lds + base + j * kLDK) = o;
    }
  }
};

template <bool Trans, int R>
struct LoaderSel {
  using type = PlainLoader<R>;
};
template <int R>
struct LoaderSel<true, R> {
  using type = TransLoader<R>;
};

// LDS bytes of the double-buffered mainloop for a 256 x BN tile.
template <int BN>
constexpr int mainloop_lds_bytes() {
  return 2 * (kBM + BN) * kLDK * 2;
}

template <int BN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][BN / 64]) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < BN / 64; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
}

// acc += A[m0:m0+256, kbeg:kend] * B[n0:n0+BN, kbeg:kend]^T, contraction
// length a multiple of 64 (the loaders zero-fill past k_lim). Ends with a
// barrier, so the caller may reuse the LDS right away.
template <int BN, bool TA, bool TB>
__device__ __forceinline__ void gemm_mainloop(const Operand& A, const Operand& B, int64_t m0,
                                              int64_t n0, int64_t kbeg, int64_t kend,
                                              f32x16 (&acc)[4][BN / 64], uint16_t* lds) {
  constexpr int NB = BN / 64;
  constexpr int kStage = (kBM + BN) * kLDK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  typename LoaderSel<TA, kBM>::type la;
  typename LoaderSel<TB, BN>::type lb;

  const int nk = static_cast<int>((kend - kbeg) / kBK);
  if (nk <= 0) return;

  la.load(A, m0, kbeg, tid);
  lb.load(B, n0, kbeg, tid);
  la.store(lds, tid);
  lb.store(lds + kBM * kLDK, tid);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = (kt + 1) < nk;
    if (more) {
      la.load(A, m0, kbeg + (kt + 1) * kBK, tid);
      lb.load(B, n0, kbeg + (kt + 1) * kBK, tid);
    }
    const uint16_t* sa = lds + (kt & 1) * kStage;
    const uint16_t* sb = sa + kBM * kLDK;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[4];
      bf16x8 bfr[NB];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(
            sa + (wm * 128 + mb * 32 + frag_row) * kLDK + ks * 16 + frag_k);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8*>(
            sb + (wn * (BN / 2) + nb * 32 + frag_row) * kLDK + ks * 16 + frag_k);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      uint16_t* da = lds + ((kt + 1) & 1) * kStage;
      la.store(da, tid);
      lb.store(da + kBM * kLDK, tid);
    }
    __syncthreads();
  }
}

// Row / column of accumulator element i of block (mb, nb) for this lane,
// relative to the wave's 128 x BN/2 sub-tile.
__device__ __forceinline__ int acc_row(int mb, int i, int lane) {
  return mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}
__device__ __forceinline__ int acc_col(int nb, int lane) { return nb * 32 + (lane & 31); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace fkl
