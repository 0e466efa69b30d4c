// Device building blocks for libfkl on gfx950 (CDNA4): bf16 MFMA block tiles
// staged through LDS, with loaders for operands stored contraction-contiguous
// ("plain") or contraction-strided ("transposed").
//
// Block tile: 256 (M) x (WN * NBW * 32) (N), contraction in LDS stages of 32,
// 2 x WN waves; each wave owns 128 x NBW*32 of the output as 4 x NBW
// accumulators of v_mfma_f32_32x32x16_bf16 (32 x 32, fp32). The path's
// kernels use WN = 4, NBW = 2: a 256 x 256 tile on 8 waves (2 per SIMD).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element (mn, k) of a GEMM operand. Plain: base[mn * ld + k] (k contiguous).
// Transposed: base[k * ld + mn] (mn contiguous). Elements outside
// [0, mn_lim) x [0, k_lim) read as zero. The contiguous extent (k_lim for a
// plain operand, mn_lim for a transposed one) is a multiple of 8, so a
// 16-byte chunk is either wholly inside or wholly outside.
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int64_t mn_lim;
  int64_t k_lim;
};

#define FKL_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Mainloop: 256 x 256 block tile, contraction in stages of 32, a ring of four
// LDS stages filled by direct global->LDS loads (buffer_load ... lds, 16 B per
// lane), so each stage's loads are issued three stages ahead of their use and
// no registers stage the operands.
//
// LDS layout of one stage (32 KiB): operand A then operand B, 16 KiB each.
//  * plain operand: 256 rows x 32 k = 64 B per row (4 chunks of 16 B); chunk
//    c of row r is stored at physical chunk c ^ swz_plain(r).
//  * transposed operand: 32 k-rows x 256 mn = 512 B per k-row (32 chunks of
//    8 mn); chunk c of k-row r is stored at physical chunk c ^ swz_trans(r).
// The XOR swizzles keep the fragment reads (16 lanes per LDS cycle) on
// distinct banks. MFMA fragments (32 mn x 16 k per lane group) are read with
// ds_read_b128 from a plain stage and with two ds_read_b64_tr_b16 (4 x 16
// transposes within each 16-lane group) from a transposed stage.
// ---------------------------------------------------------------------------

constexpr int kStageK = 32;
constexpr int kARows = 256;                                    // A operand extent of a block tile
constexpr int kAStageBytes = kARows * kStageK * 2;             // 16 KiB
constexpr uint32_t kOob = 0x80000000u;                         // offset past every buffer

// Block tile 256 x (WN * NBW * 32): (8 / MB) x WN waves, each MB*32 x NBW*32
// of the output. The B operand's LDS extent is the tile width rounded up to
// 128 or 256 (a narrower tile keeps that layout and masks the rest).
template <int NBW, int WN = 2, int MB = 4>
struct TileCfg {
  static constexpr int kWM = kARows / (MB * 32);
  static constexpr int kWaves = kWM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTileN = WN * NBW * 32;
  static constexpr int kBExtent = kTileN <= 128 ? 128 : 256;
  static constexpr int kBStageBytes = kBExtent * kStageK * 2;
  static constexpr int kStageBytes = kAStageBytes + kBStageBytes;
  static constexpr int kStages = kStageBytes <= 24576 ? 3 : 4;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kDmaA = kAStageBytes / (kThreads * 16);  // 16-byte loads per lane per stage
  static constexpr int kDmaB = kBStageBytes / (kThreads * 16);
  static constexpr int kDmaStage = kDmaA + kDmaB;
};

__device__ __forceinline__ int swz_plain(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
__device__ __forceinline__ int swz_trans(int r) { return (r & 3) << 2; }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Wait until at most n of this wave's vector-memory operations are in flight.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

__device__ __forceinline__ void block_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Per-lane source offsets of one operand's stage loads (extent R rows of a
// plain operand or R columns of a transposed one; R / 64 loads per lane).
template <int LW>
struct StageSrc {
  const uint16_t* base;     // buffer start (wave-uniform)
  int32_t bytes;            // buffer size; offsets at or past it read as zero
  uint32_t voff[LW];        // byte offsets for stage 0 (kOob when masked for every stage)
  uint32_t kstep;           // byte advance per stage along k
  int32_t kchunk[LW];       // plain: first k of the lane's chunk (k-tail mask)
  int32_t klim;
  bool trans;
};

// Plain operand rows [mn0, mn0 + R) (only the first `used` are loaded): the
// buffer is based at row mn0 and sized to the valid rows, so rows past mn_lim
// read as zero; chunks past k_lim are masked per stage. LDS: row r at r * 64
// bytes, 16-byte chunk c at physical chunk c ^ swz_plain(r).
template <int R, int LW>
__device__ __forceinline__ StageSrc<LW> make_plain_src(const Operand& op, int64_t mn0, int wave, int lane,
                                                       int used = R) {
  StageSrc<LW> s;
  const int64_t rows = op.mn_lim - mn0 < used ? op.mn_lim - mn0 : used;
  const int64_t bytes = rows > 0 ? rows * op.ld * 2 : 0;
  s.base = op.base + mn0 * op.ld;
  s.bytes = static_cast<int32_t>(bytes);
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int r = (wave * LW + j) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_plain(r);
    s.kchunk[j] = c * 8;
    s.voff[j] = static_cast<uint32_t>((r * op.ld + c * 8) * 2);
  }
  s.kstep = kStageK * 2;
  s.klim = static_cast<int32_t>(op.k_lim);
  s.trans = false;
  return s;
}

// Transposed operand columns [mn0, mn0 + R) (only the first `used` are
// loaded): the buffer starts at column mn0 of k-row 0 and ends after k-row
// k_lim - 1, so k-rows past k_lim read as zero; columns past mn_lim are
// masked once. LDS: k-row r at r * 2R bytes, 16-byte chunk c (8 columns) at
// physical chunk c ^ swz_trans(r).
template <int R, int LW>
__device__ __forceinline__ StageSrc<LW> make_trans_src(const Operand& op, int64_t mn0, int wave, int lane,
                                                       int used = R) {
  StageSrc<LW> s;
  const int64_t bytes = op.k_lim * op.ld * 2 - mn0 * 2;
  s.base = op.base + mn0;
  s.bytes = static_cast<int32_t>(bytes > 0 ? bytes : 0);
  constexpr int kChunks = R / 8;          // 16-byte chunks per k-row
  constexpr int kRowsPerLoad = 64 / kChunks;
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int r = (wave * LW + j) * kRowsPerLoad + lane / kChunks;
    const int c = (lane % kChunks) ^ swz_trans(r);
    const bool ok = mn0 + c * 8 < op.mn_lim && c * 8 < used;
    s.voff[j] = ok ? static_cast<uint32_t>((r * op.ld + c * 8) * 2) : kOob;
    s.kchunk[j] = 0;
  }
  s.kstep = static_cast<uint32_t>(kStageK * op.ld * 2);
  s.klim = static_cast<int32_t>(op.k_lim);
  s.trans = true;
  return s;
}

// Issue one operand's loads of stage kt into its LDS region dst. When live
// is false every lane reads out of range, which fills zeros without a memory
// access: the loop issues a stage every iteration so its wait counts never
// depend on the trip count.
template <int LW>
__device__ __forceinline__ void issue_stage(const StageSrc<LW>& s, int kt, bool live, char* dst, int wave) {
  const uint32_t adv = static_cast<uint32_t>(kt) * s.kstep;
  const int k0 = kt * kStageK;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(s.base), 0, s.bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    uint32_t off = s.voff[j];
    if (!s.trans) off = (k0 + s.kchunk[j] < s.klim) ? off + adv : kOob;
    else if (off != kOob) off += adv;
    if (!live) off = kOob;
    FKL_LDS void* p = (FKL_LDS void*)(dst + (wave * LW + j) * 1024);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, p, 16, static_cast<int>(off), 0, 0, 0);
  }
}

// Fragment of 32 (mn) x 16 (k) for this lane from a plain stage region: lane
// l receives mn = mn_base + (l & 31), k = kb + 8 * (l >> 5) .. + 7.
__device__ __forceinline__ bf16x8 frag_plain(const char* region, int mn_base, int kb, int lane) {
  const int r = mn_base + (lane & 31);
  const int c = (kb >> 3) + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(region + r * (kStageK * 2) + ((c ^ swz_plain(r)) << 4));
}

// Transposed fragments are read with ds_read_b64_tr_b16 issued from inline
// assembly: the compiler's builtin for it makes every such read wait for all
// outstanding global->LDS loads, which would drain the load pipeline. Results
// are settled explicitly (Frags::settle) before the MFMAs use them.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 ds_read_tr16(const char* p) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const FKL_LDS char*)p));
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}

// Lane l receives mn = mn_base + (l & 31) and k = kb + 8 * (l >> 5) .. + 7 as
// two halves of 4 k each: lanes 4j..4j+3 of each 16-lane group point at k-row j
// (4 consecutive mn each) and lane i gets column i.
template <int R>
__device__ __forceinline__ void frag_trans_issue(const char* region, int mn_base, int kb, int lane,
                                                 u32x2& lo, u32x2& hi) {
  const int g = lane >> 4;
  const int i = lane & 15;
  const int r = kb + 8 * (g >> 1) + (i >> 2);
  const int mn = mn_base + 16 * (g & 1) + 4 * (i & 3);
  const int c = mn >> 3;
  const int half = (mn & 7) * 2;
  lo = ds_read_tr16(region + r * (2 * R) + ((c ^ swz_trans(r)) << 4) + half);
  hi = ds_read_tr16(region + (r + 4) * (2 * R) + ((c ^ swz_trans(r + 4)) << 4) + half);
}

__device__ __forceinline__ bf16x8 join_halves(u32x2 lo, u32x2 hi) {
  const u32x4 w{lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Fragments of one 16-deep contraction step for a wave: MB of A (MB * 32
// rows), NBW of B (NBW * 32 columns).
template <bool TA, bool TB, int NBW, int RB, int MB = 4>
struct Frags {
  static constexpr int kX = MB > NBW ? MB : NBW;
  bf16x8 a[MB], b[NBW];
  u32x2 ta[MB][2], tb[NBW][2];

  __device__ __forceinline__ void issue(const char* ra, const char* rb, int wm, int wn, int kb, int lane) {
#pragma unroll
    for (int x = 0; x < kX; ++x) {
      if (x < MB) {
        if constexpr (TA) frag_trans_issue<kARows>(ra, wm * MB * 32 + x * 32, kb, lane, ta[x][0], ta[x][1]);
        else a[x] = frag_plain(ra, wm * MB * 32 + x * 32, kb, lane);
      }
      if (x < NBW) {
        if constexpr (TB) frag_trans_issue<RB>(rb, wn * NBW * 32 + x * 32, kb, lane, tb[x][0], tb[x][1]);
        else b[x] = frag_plain(rb, wn * NBW * 32 + x * 32, kb, lane);
      }
    }
  }

  // Wait for the transposed reads; the asm operands make every later use of
  // these registers depend on the wait.
  __device__ __forceinline__ void settle() {
    if constexpr (TA) {
      if constexpr (MB == 4) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(ta[0][0]), "+v"(ta[0][1]), "+v"(ta[1][0]), "+v"(ta[1][1]), "+v"(ta[2][0]),
                       "+v"(ta[2][1]), "+v"(ta[3][0]), "+v"(ta[3][1]));
      } else if constexpr (MB == 2) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(ta[0][0]), "+v"(ta[0][1]), "+v"(ta[1][0]), "+v"(ta[1][1]));
      } else {
        static_assert(MB == 1, "MB must be 1, 2 or 4");
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ta[0][0]), "+v"(ta[0][1]));
      }
    }
    if constexpr (TB) {
      if constexpr (NBW == 4) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(tb[0][0]), "+v"(tb[0][1]), "+v"(tb[1][0]), "+v"(tb[1][1]), "+v"(tb[2][0]),
                       "+v"(tb[2][1]), "+v"(tb[3][0]), "+v"(tb[3][1]));
      } else if constexpr (NBW == 3) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(tb[0][0]), "+v"(tb[0][1]), "+v"(tb[1][0]), "+v"(tb[1][1]), "+v"(tb[2][0]),
                       "+v"(tb[2][1]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(tb[0][0]), "+v"(tb[0][1]), "+v"(tb[1][0]), "+v"(tb[1][1]));
      }
    }
#pragma unroll
    for (int x = 0; x < kX; ++x) {
      if constexpr (TA) if (x < MB) a[x] = join_halves(ta[x][0], ta[x][1]);
      if constexpr (TB) if (x < NBW) b[x] = join_halves(tb[x][0], tb[x][1]);
    }
  }

  __device__ __forceinline__ void mma(f32x16 (&acc)[MB][NBW]) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
  }
};

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[MB][NB]) {
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
}

// acc += A[m0 : m0+256, 0 : 32*nk] * B[n0 : n0+kTileN, 0 : 32*nk]^T over a
// ring of TileCfg<NBW, WN, MB>::kStages LDS stages ((8 / MB) x WN waves, each
// MB*32 x NBW*32 of the output; wave w sits at row block w / WN, column block
// w % WN).
//
// Schedule per stage kt (two 16-deep steps f0, f1):
//   issue f1 reads (stage kt) | f0 MFMAs | settle f1
//   wait for stage kt+1 + block barrier   (every wave has issued its reads
//                                          of stage kt)
//   issue f0 reads of stage kt+1 | DMA stage kt+S into stage kt's buffer
//   f1 MFMAs | settle f0
// so the barrier and the LDS latency of the next stage sit between two MFMA
// bursts instead of in front of an idle pipe. Plain-layout reads of stage kt
// may still be queued at the LDS when the barrier opens. The schedule relies
// on the LDS serving them before the DMA writes into that buffer, which are
// issued after the barrier and first make a round trip through the caches.
// (Waiting for those reads before the barrier cost 1.3% of the loop's
// throughput when measured.) The loop body has no branch
// (the last stage is peeled and a stage is issued every iteration, out of
// range past the end), so the compiler's wait counts hold on every path.
// Starts with a block barrier (the previous user of the LDS is done) and ends
// with one; on return no load is in flight and the LDS may be reused.
template <bool TA, bool TB, int NBW, int WN = 2, int MB = 4>
__device__ __forceinline__ void gemm_mainloop(const Operand& A, const Operand& B, int64_t m0, int64_t n0,
                                              int nk, f32x16 (&acc)[MB][NBW], char* lds) {
  using C = TileCfg<NBW, WN, MB>;
  constexpr int S = C::kStages;
  constexpr int RB = C::kBExtent;
  constexpr int LA = C::kDmaA;
  constexpr int LB = C::kDmaB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  StageSrc<LA> sa;
  StageSrc<LB> sb;
  if constexpr (TA) sa = make_trans_src<kARows, LA>(A, m0, wave, lane);
  else sa = make_plain_src<kARows, LA>(A, m0, wave, lane);
  if constexpr (TB) sb = make_trans_src<RB, LB>(B, n0, wave, lane, C::kTileN);
  else sb = make_plain_src<RB, LB>(B, n0, wave, lane, C::kTileN);

  block_barrier();
  if (nk <= 0) return;
#pragma unroll
  for (int p = 0; p < S; ++p) {
    issue_stage<LA>(sa, p, p < nk, lds + p * C::kStageBytes, wave);
    issue_stage<LB>(sb, p, p < nk, lds + p * C::kStageBytes + kAStageBytes, wave);
  }
  wait_vmcnt<(S - 1) * C::kDmaStage>();  // stage 0 landed
  block_barrier();
  Frags<TA, TB, NBW, RB, MB> f0, f1;
  f0.issue(lds, lds + kAStageBytes, wm, wn, 0, lane);
  f0.settle();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    char* cur = lds + (kt % S) * C::kStageBytes;
    const char* nxt = lds + ((kt + 1) % S) * C::kStageBytes;
    f1.issue(cur, cur + kAStageBytes, wm, wn, 16, lane);
    f0.mma(acc);
    f1.settle();
    wait_vmcnt<(S - 2) * C::kDmaStage>();  // stage kt+1 landed
    block_barrier();
    f0.issue(nxt, nxt + kAStageBytes, wm, wn, 0, lane);
    const bool live = kt + S < nk;
    issue_stage<LA>(sa, kt + S, live, cur, wave);
    issue_stage<LB>(sb, kt + S, live, cur + kAStageBytes, wave);
    f1.mma(acc);
    f0.settle();
  }
  {
    char* cur = lds + ((nk - 1) % S) * C::kStageBytes;
    f1.issue(cur, cur + kAStageBytes, wm, wn, 16, lane);
    f0.mma(acc);
    f1.settle();
    f1.mma(acc);
  }
  wait_vmcnt<0>();
  block_barrier();
}

// Workgroup placement. The dispatcher hands workgroups to the eight XCDs
// round-robin (workgroup w runs on XCD w % 8) and each XCD has its own L2.
// xcd_contiguous renumbers workgroups so that every XCD owns one contiguous
// range of tile indices; grouped_tile then rasters an R x S tile grid in
// bands of `group` rows, so the tiles resident on one XCD at the same time
// form a compact rectangle and share operand panels in that XCD's L2.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_contiguous(int w, int total) {
  const int x = w % kXcds;
  const int i = w / kXcds;
  const int base = total / kXcds;
  const int rem = total % kXcds;
  return x * base + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ void grouped_tile(int L, int R, int S, int group, int& r, int& s) {
  const int per_group = group * S;
  const int g = L / per_group;
  const int first = g * group;
  const int rows = R - first < group ? R - first : group;
  const int in = L - g * per_group;
  r = first + in % rows;
  s = in / rows;
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
