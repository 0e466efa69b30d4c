// Device building blocks for libfkl on gfx950 (CDNA4): bf16 MFMA block tiles
// staged through LDS, with loaders for operands stored contraction-contiguous
// ("plain") or contraction-strided ("transposed").
//
// Block tile: 256 (M) x (WN * NBW * 32) (N), contraction in LDS stages of 32,
// (8 / MB) x WN waves; each wave owns MB*32 x NBW*32 of the output as
// 2MB x 2NBW accumulators of v_mfma_f32_16x16x32_bf16 (16 x 16, fp32), one
// MFMA step of 32 per stage. The path's kernels use WN = 4, NBW = 2, MB = 4:
// a 256 x 256 tile on 8 waves (2 per SIMD), 128 x 64 per wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fkl_debug.h"
#include "fkl_internal.h"

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
// The XOR swizzles keep the fragment reads on distinct banks (16 lanes per
// LDS cycle for ds_read_b128, 32 for ds_read_b64_tr_b16). MFMA fragments
// (16 mn x 32 k) are read with ds_read_b128 from a plain stage and with two
// ds_read_b64_tr_b16 (4 x 16 transposes within each 16-lane group) from a
// transposed stage.
// ---------------------------------------------------------------------------

constexpr int kStageK = kContractionStep;
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
__device__ __forceinline__ int swz_trans(int r) { return ((r & 3) << 2) | (((r >> 3) & 1) << 1); }

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
// The memory a block tile's stage loads of an operand may touch (the buffer
// view its descriptor covers): rows [mn0, mn0 + used) of a plain operand,
// cut at mn_lim; for a transposed one, from column mn0 of k-row 0 to the end
// of k-row k_lim - 1.
struct OperandView {
  const uint16_t* base;
  int64_t bytes;
};

__device__ __forceinline__ OperandView plain_view(const Operand& op, int64_t mn0, int used) {
  const int64_t rows = op.mn_lim - mn0 < used ? op.mn_lim - mn0 : used;
  return OperandView{op.base + mn0 * op.ld, rows > 0 ? rows * op.ld * 2 : 0};
}

__device__ __forceinline__ OperandView trans_view(const Operand& op, int64_t mn0) {
  const int64_t bytes = op.k_lim * op.ld * 2 - mn0 * 2;
  return OperandView{op.base + mn0, bytes > 0 ? bytes : 0};
}

template <int R, int LW>
__device__ __forceinline__ StageSrc<LW> make_plain_src(const Operand& op, int64_t mn0, int wave, int lane,
                                                       int used = R) {
  StageSrc<LW> s;
  const OperandView v = plain_view(op, mn0, used);
  s.base = v.base;
  s.bytes = static_cast<int32_t>(v.bytes);
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
  const OperandView v = trans_view(op, mn0);
  s.base = v.base;
  s.bytes = static_cast<int32_t>(v.bytes);
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

// Fragment of 16 (mn) x 32 (k) for this lane from a plain stage region: lane
// l receives mn = mn_base + (l & 15), k = 8 * (l >> 4) .. + 7.
__device__ __forceinline__ bf16x8 frag_plain(const char* region, int mn_base, int lane) {
  const int r = mn_base + (lane & 15);
  const int c = lane >> 4;
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

// Lane l receives mn = mn_base + (l & 15) and k = 8 * (l >> 4) .. + 7 as two
// halves of 4 k each: in 16-lane group g, lanes 4j..4j+3 point at k-row
// 8g + j (then 8g + 4 + j), 4 consecutive mn each, and lane i gets column i.
template <int R>
__device__ __forceinline__ void frag_trans_issue(const char* region, int mn_base, int lane, u32x2& lo,
                                                 u32x2& hi) {
  const int g = lane >> 4;
  const int i = lane & 15;
  const int r = 8 * g + (i >> 2);
  const int mn = mn_base + 4 * (i & 3);
  const int c = mn >> 3;
  const int half = (mn & 7) * 2;
  lo = ds_read_tr16(region + r * (2 * R) + ((c ^ swz_trans(r)) << 4) + half);
  hi = ds_read_tr16(region + (r + 4) * (2 * R) + ((c ^ swz_trans(r + 4)) << 4) + half);
}

__device__ __forceinline__ bf16x8 join_halves(u32x2 lo, u32x2 hi) {
  const u32x4 w{lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Settle outstanding ds_read_b64_tr_b16 results: the asm operands make every
// later use of these registers depend on the wait.
template <int X>
__device__ __forceinline__ void settle_tr(u32x2 (&t)[X][2]) {
  static_assert(X == 2 || X == 4 || X == 8, "fragment count");
  if constexpr (X == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1]));
  } else if constexpr (X == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1]), "+v"(t[2][0]), "+v"(t[2][1]),
                   "+v"(t[3][0]), "+v"(t[3][1]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0][0]), "+v"(t[0][1]), "+v"(t[1][0]), "+v"(t[1][1]), "+v"(t[2][0]), "+v"(t[2][1]),
                   "+v"(t[3][0]), "+v"(t[3][1]), "+v"(t[4][0]), "+v"(t[4][1]), "+v"(t[5][0]), "+v"(t[5][1]),
                   "+v"(t[6][0]), "+v"(t[6][1]), "+v"(t[7][0]), "+v"(t[7][1]));
  }
}

// Fragments of one 32-deep stage for a wave: XA of A (16 rows each), XB of B
// (16 columns each).
template <bool TA, bool TB, int XA, int XB, int RB>
struct Frags {
  bf16x8 a[XA], b[XB];
  u32x2 ta[XA][2], tb[XB][2];

  __device__ __forceinline__ void issue(const char* ra, const char* rb, int am, int bn, int lane) {
#pragma unroll
    for (int x = 0; x < XA; ++x) {
      if constexpr (TA) frag_trans_issue<kARows>(ra, am + x * 16, lane, ta[x][0], ta[x][1]);
      else a[x] = frag_plain(ra, am + x * 16, lane);
    }
#pragma unroll
    for (int y = 0; y < XB; ++y) {
      if constexpr (TB) frag_trans_issue<RB>(rb, bn + y * 16, lane, tb[y][0], tb[y][1]);
      else b[y] = frag_plain(rb, bn + y * 16, lane);
    }
  }

  __device__ __forceinline__ void settle() {
    if constexpr (TA) {
      settle_tr(ta);
#pragma unroll
      for (int x = 0; x < XA; ++x) a[x] = join_halves(ta[x][0], ta[x][1]);
    }
    if constexpr (TB) {
      settle_tr(tb);
#pragma unroll
      for (int y = 0; y < XB; ++y) b[y] = join_halves(tb[y][0], tb[y][1]);
    }
  }

  __device__ __forceinline__ void mma(f32x4 (&acc)[XA][XB]) const {
#pragma unroll
    for (int x = 0; x < XA; ++x)
#pragma unroll
      for (int y = 0; y < XB; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
  }
};

template <int X, int Y>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[X][Y]) {
#pragma unroll
  for (int a = 0; a < X; ++a)
#pragma unroll
    for (int b = 0; b < Y; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc += A[m0 : m0+256, 0 : 32*nk] * B[n0 : n0+kTileN, 0 : 32*nk]^T over a
// ring of TileCfg<NBW, WN, MB>::kStages LDS stages ((8 / MB) x WN waves, each
// MB*32 x NBW*32 of the output as 2MB x 2NBW blocks of 16 x 16; wave w sits at
// row block w / WN, column block w % WN).
//
// Schedule per stage kt: the stage's MFMAs, a wait for stage kt+1 and one
// block barrier (every wave has read stage kt), then the fragment reads of
// stage kt+1 and the DMA of stage kt+S into stage kt's buffer. The two waves
// on a SIMD interleave, so one wave's MFMAs cover the other's LDS reads.
// (Splitting the MFMAs around the barrier measured slower.) The loop body has
// no branch (a stage is issued every iteration, out of range past the end),
// so the compiler's wait counts hold on every path. Starts with a block
// barrier (the previous user of the LDS is done) and ends with one; on return
// no load is in flight and the LDS may be reused.
template <bool TA, bool TB, int NBW, int WN = 2, int MB = 4>
__device__ __forceinline__ void gemm_mainloop(const Operand& A, const Operand& B, int64_t m0, int64_t n0,
                                              int nk, f32x4 (&acc)[2 * MB][2 * NBW], char* lds) {
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
  const int am = wm * MB * 32;
  const int bn = wn * NBW * 32;
  Frags<TA, TB, 2 * MB, 2 * NBW, RB> f;
  f.issue(lds, lds + kAStageBytes, am, bn, lane);
  f.settle();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    char* cur = lds + (kt % S) * C::kStageBytes;
    const char* nxt = lds + ((kt + 1) % S) * C::kStageBytes;
    f.mma(acc);
    wait_vmcnt<(S - 2) * C::kDmaStage>();  // stage kt+1 landed
    block_barrier();
    f.issue(nxt, nxt + kAStageBytes, am, bn, lane);
    const bool live = kt + S < nk;
    issue_stage<LA>(sa, kt + S, live, cur, wave);
    issue_stage<LB>(sb, kt + S, live, cur + kAStageBytes, wave);
    f.settle();
  }
  f.mma(acc);
  wait_vmcnt<0>();
  block_barrier();
}

// Debug build: the memory a block tile's loads of an operand can reach must
// lie inside the operand's span: for a transposed operand its whole view; for
// a plain one the view up to the last row's contraction extent (k_lim rounded
// up to a 16-byte chunk), since a window along the contraction shifts the
// view's base by k0 while every load stays below k_lim in its row.
__device__ __forceinline__ bool dcheck_operand(const DebugCheck& d, int span, const Operand& op, int64_t mn0,
                                               int used, bool trans) {
  if (trans) {
    const OperandView v = trans_view(op, mn0);
    return dcheck_range(d, span, kDbgOperand, v.base, static_cast<uint64_t>(v.bytes));
  }
  const OperandView v = plain_view(op, mn0, used);
  if (v.bytes == 0) return true;
  const int64_t rows = v.bytes / (op.ld * 2);
  const int64_t reach = ((rows - 1) * op.ld + ((op.k_lim + 7) / 8) * 8) * 2;
  return dcheck_range(d, span, kDbgOperand, v.base, static_cast<uint64_t>(reach));
}

// The same for both operands of a block tile: A from row (or column) m0, B
// from n0 with `used_b` of them.
template <bool TA, bool TB>
__device__ __forceinline__ void dcheck_operands(const DebugCheck& d, int a_span, int b_span, const Operand& A,
                                                const Operand& B, int64_t m0, int64_t n0, int used_b) {
  dcheck_operand(d, a_span, A, m0, kARows, TA);
  dcheck_operand(d, b_span, B, n0, used_b, TB);
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

// Row / column of accumulator element i of block (x, y) for this lane,
// relative to the wave's sub-tile (16 x 16 blocks: lane l holds column
// l & 15 and rows 4 (l >> 4) .. + 3).
__device__ __forceinline__ int acc_row(int x, int i, int lane) { return x * 16 + 4 * (lane >> 4) + i; }
__device__ __forceinline__ int acc_col(int y, int lane) { return y * 16 + (lane & 15); }

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
