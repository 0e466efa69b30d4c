// HIP kernels of libfkl for gfx950, and their launch sequences.
//
// Forward, per pass of rows (blog post on the page "Efficient Offline Top-K
// Logits and Fused Chunked KL Loss Enable Scalable LLM Distillation",
// section "Two systems changes": logits are formed one chunk at a time,
// folded into the running loss and dropped):
//   k_teacher_prep  softmax of the cached teacher logits over K, its
//                   negative entropy, and each row's (index, p) list sorted by
//                   vocabulary index
//   k_fwd_sweep     256-row block x a run of 256-column vocabulary tiles:
//                   MFMA logits tile -> LDS -> per-row online max / sum of
//                   exp2, and the logits at the teacher indices picked up by a
//                   per-row cursor while the tile is resident
//   k_fwd_combine   merge the vocabulary splits -> row_lse, row KL, fp64 sums
//   k_accumulate    fixed-order fp64 running loss
// Backward, per pass of rows and vocabulary slab (same section: each pass's
// logits are recomputed rather than stored):
//   k_bwd_g         logits tile again -> fp32 through LDS -> G = c (exp(s - lse)
//                   - p~) formed in fp32 by the row owners (teacher entries
//                   subtracted before rounding) -> bf16 row-major gradient
//                   block G in the workspace
//   k_bwd_grads     grad_h[chunk] (+)= G W_slab and grad_W[slab] (+)= G^T h_chunk
//                   in one launch (grad_h tiles optionally split along the
//                   vocabulary into partial sums)
//   k_reduce_grad_h grad_h[chunk] (+)= the partial sums, in split order
#include <climits>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "fkl_device.h"
#include "fkl_internal.h"
#include "fkl_tiles.h"

namespace fkl {

struct Scalars {
  double acc;       // running sum of valid-row KL (fp64, fixed order)
  int64_t n_valid;  // number of valid rows
  double wsum;      // sum over rows of mask x row weight (= n_valid without weights)
};
static_assert(sizeof(Scalars) <= kValidateCountOffset, "scalars overlap the validation count");

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_count_valid(const uint8_t* __restrict__ mask,
                                                     const float* __restrict__ weight, int64_t N,
                                                     Scalars* sc) {
  __shared__ int64_t part[256];
  __shared__ double wpart[256];
  int64_t cnt = 0;
  double ws = 0.0;
  // A row counts when it is unmasked; its weight enters the sum only when
  // positive, the rule every other kernel applies (a row whose weight is zero,
  // negative or NaN takes no part in the loss).
  for (int64_t r = threadIdx.x; r < N; r += 256) {
    const bool valid = !mask || mask[r] != 0;
    cnt += valid;
    const float w = weight ? weight[r] : 1.0f;
    ws += (valid && w > 0.f) ? static_cast<double>(w) : 0.0;
  }
  part[threadIdx.x] = cnt;
  wpart[threadIdx.x] = ws;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) {
      part[threadIdx.x] += part[threadIdx.x + s];
      wpart[threadIdx.x] += wpart[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    sc->n_valid = part[0];
    sc->wsum = wpart[0];
    sc->acc = 0.0;
  }
}

// One wave per row, four rows per workgroup: p = softmax(t_logit / T) over
// the K cached entries, the row's list of (index, weight) sorted by vocabulary
// index (ties by position, so even repeated indices fill every slot), and the
// weighted negative entropy. With a hard label y (weight a), the list holds
// the target (1 - a) p~ + a onehot(y): teacher weights are scaled by 1 - a and
// y is inserted with a, or a is added to the teacher entry at y (the list then
// ends with an empty entry at INT_MAX). Lists have L = K (+ 1 with labels)
// entries.
//
// LONG = false: each entry's rank by counting, for K up to kPrepRankMaxK.
// LONG = true: a bitonic sort of (index, position) pairs in the wave's LDS
// row, which gives the same order, for K up to 1024.
constexpr int kPrepRankMaxK = 128;
template <bool LONG>
__global__ __launch_bounds__(256) void k_teacher_prep(const int32_t* __restrict__ t_idx,
                                                      const float* __restrict__ t_logit,
                                                      const int32_t* __restrict__ label, float label_w,
                                                      int64_t r0, int32_t rows, int32_t K, int32_t L,
                                                      float invT, int32_t* __restrict__ tsort_idx,
                                                      float* __restrict__ tsort_p,
                                                      float* __restrict__ negent, DebugCheck dbg) {
  // dbg spans: 0 t_idx, 1 t_logit, 2 sorted indices, 3 sorted weights, 4 negentropies, 5 labels
  using Key = typename std::conditional<LONG, uint64_t, int32_t>::type;
  __shared__ Key skey[4][1024];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= rows) return;  // no block-wide synchronisation below
  Key* sk = &skey[wave][0];
  const int32_t* ti = t_idx + (r0 + r) * static_cast<int64_t>(K);
  const float* tl = t_logit + (r0 + r) * static_cast<int64_t>(K);
  int Kp = K;
  if constexpr (LONG) {
    Kp = 1;
    while (Kp < K) Kp <<= 1;
  }
  float mx = -INFINITY;
  for (int k = lane; k < Kp; k += 64) {
    if constexpr (LONG) {
      sk[k] = k < K ? (static_cast<uint64_t>(static_cast<uint32_t>(dload(dbg, 0, kDbgTeacherInput, ti + k))) << 32) |
                          static_cast<uint32_t>(k)
                    : ~uint64_t(0);
    } else {
      sk[k] = dload(dbg, 0, kDbgTeacherInput, ti + k);
    }
    if (k < K) mx = fmaxf(mx, dload(dbg, 1, kDbgTeacherInput, tl + k) * invT);
  }
  __builtin_amdgcn_wave_barrier();
  mx = wave_max(mx);
  float se = 0.f;
  for (int k = lane; k < K; k += 64) se += expf(dload(dbg, 1, kDbgTeacherInput, tl + k) * invT - mx);
  se = wave_sum(se);
  const float lnorm = mx + logf(se);
  auto index_at = [sk](int k) -> int32_t {
    if constexpr (LONG) return static_cast<int32_t>(sk[k] >> 32);
    else return sk[k];
  };
  const bool has_label = label != nullptr;
  const int32_t y = has_label ? dload(dbg, 5, kDbgTeacherInput, label + r0 + r) : 0;
  const float keep = has_label ? 1.0f - label_w : 1.0f;
  // where y goes: the number of teacher indices below it, and whether it is one
  int below = 0, dup = 0;
  if (has_label) {
    for (int k = lane; k < K; k += 64) {
      below += index_at(k) < y;
      dup += index_at(k) == y;
    }
    below = static_cast<int>(wave_sum(static_cast<float>(below)));
    dup = static_cast<int>(wave_sum(static_cast<float>(dup)));
  }
  const bool insert = has_label && dup == 0;
  float ne = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float lp = dload(dbg, 1, kDbgTeacherInput, tl + k) * invT - lnorm;
    ne += expf(lp) * lp;
  }
  int32_t* oi = tsort_idx + static_cast<int64_t>(r) * L;
  float* op = tsort_p + static_cast<int64_t>(r) * L;
  if constexpr (!LONG) {
    for (int k = lane; k < K; k += 64) {
      const int32_t key = sk[k];
      int rank = 0;
      for (int j = 0; j < K; ++j) {
        const int32_t o = sk[j];
        rank += (o < key) | ((o == key) & (j < k));
      }
      if (insert && key > y) ++rank;
      dstore(dbg, 2, kDbgTeacherList, oi + rank, key);
      dstore(dbg, 3, kDbgTeacherList, op + rank,
             keep * expf(dload(dbg, 1, kDbgTeacherInput, tl + k) * invT - lnorm) +
                 ((has_label && key == y) ? label_w : 0.0f));
    }
  } else {
    for (int size = 2; size <= Kp; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = lane; t < Kp / 2; t += 64) {
          const int i = 2 * t - (t & (stride - 1));
          const int j = i + stride;
          const uint64_t a = sk[i];
          const uint64_t b = sk[j];
          if (((i & size) == 0) == (a > b)) {
            sk[i] = b;
            sk[j] = a;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    for (int i = lane; i < K; i += 64) {
      const uint64_t v = sk[i];
      const int32_t key = static_cast<int32_t>(v >> 32);
      const int k = static_cast<int>(v & 0xFFFFFFFFu);
      const int rank = i + ((insert && key > y) ? 1 : 0);
      dstore(dbg, 2, kDbgTeacherList, oi + rank, key);
      dstore(dbg, 3, kDbgTeacherList, op + rank,
             keep * expf(dload(dbg, 1, kDbgTeacherInput, tl + k) * invT - lnorm) +
                 ((has_label && key == y) ? label_w : 0.0f));
    }
  }
  ne = wave_sum(ne);
  if (lane == 0) {
    dstore(dbg, 4, kDbgTeacherList, negent + r, keep * ne);
    if (insert) {
      dstore(dbg, 2, kDbgTeacherList, oi + below, y);
      dstore(dbg, 3, kDbgTeacherList, op + below, label_w);
    } else if (has_label) {
      dstore(dbg, 2, kDbgTeacherList, oi + K, static_cast<int32_t>(INT_MAX));
      dstore(dbg, 3, kDbgTeacherList, op + K, 0.0f);
    }
  }
}

// (Launch errors surface through hipGetLastError at the end of the sequence.)
static void launch_teacher_prep(const int32_t* t_idx, const float* t_logit, const int32_t* label, float label_w,
                                int64_t r0, int rows, int K, int L, float invT, int32_t* tsort_idx, float* tsort_p,
                                float* negent, const DebugCheck& dbg, hipStream_t st) {
  if (K <= kPrepRankMaxK)
    hipLaunchKernelGGL(k_teacher_prep<false>, dim3(ceil_div(rows, 4)), dim3(256), 0, st, t_idx, t_logit, label,
                       label_w, r0, rows, K, L, invT, tsort_idx, tsort_p, negent, dbg);
  else
    hipLaunchKernelGGL(k_teacher_prep<true>, dim3(ceil_div(rows, 4)), dim3(256), 0, st, t_idx, t_logit, label,
                       label_w, r0, rows, K, L, invT, tsort_idx, tsort_p, negent, dbg);
}

// One wave: lane l sums block sums l, l + 64, ... in order, then the 64
// lane sums are combined by a fixed butterfly, so the result does not depend
// on timing (the loads of all lanes are in flight together).
__global__ void k_accumulate(const double* __restrict__ block_sum, int nblocks, Scalars* sc) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64 || blockIdx.x != 0) return;
  double a = 0.0;
  for (int i = lane; i < nblocks; i += 64) a += block_sum[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) sc->acc += a;
}

__global__ void k_finalize(const Scalars* sc, float T, float* loss) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const double w = sc->wsum;
    loss[0] = w > 0.0 ? static_cast<float>(static_cast<double>(T) * T * sc->acc / w) : 0.0f;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Per-row sorted teacher cursor
// ---------------------------------------------------------------------------

// Walk over one row's teacher entries sorted by vocabulary index. A window of
// four entries sits in registers. A step shifts the window and leaves its
// last slot empty; refill(), called once per tile after the epilogue, loads
// the empty slots, so those loads have the whole next mainloop to arrive and
// the epilogue never waits for memory unless a row takes more than three
// entries in one tile (then the current entry is loaded on the spot).
constexpr int kUnloaded = INT_MAX - 1;  // slot not loaded yet (INT_MAX: past the row's end)

struct Cursor {
  const int32_t* idx;
  const float* p;
  int K, pos;  // pos: index of entry e0
  int e0, e1, e2, e3;
  float p0, p1, p2, p3;
  DebugCheck dbg;  // debug build: span 0 = the pass's sorted indices, 1 = their weights

  __device__ __forceinline__ int32_t ld_idx(int k) const { return dload(dbg, 0, kDbgTeacherList, idx + k); }
  __device__ __forceinline__ float ld_p(int k) const { return dload(dbg, 1, kDbgTeacherList, p + k); }

  __device__ __forceinline__ void load_at(int k, int& e, float& q) const {
    if (k < K) {
      e = ld_idx(k);
      q = ld_p(k);
    } else {
      e = INT_MAX;
      q = 0.f;
    }
  }

  // Position at the first entry >= target in three rounds of loads: 16
  // evenly spaced samples locate the segment, the segment is counted, then
  // the window is loaded. Every load of a round is issued unconditionally
  // (index clamped into the list, out-of-range results masked afterwards),
  // so a round costs one memory latency rather than one per load.
  __device__ __forceinline__ void init(const int32_t* i, const float* pp, int k, int target, bool on) {
    idx = i;
    p = pp;
    K = k;
    pos = k;
    e0 = e1 = e2 = e3 = INT_MAX;
    p0 = p1 = p2 = p3 = 0.f;
    if (!on) return;
    const int seg = (K + 15) / 16;
    int sample[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sample[j] = ld_idx(min(j * seg, K - 1));
    int c1 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) c1 += (j * seg < K) & (sample[j] < target);
    int start = 0;
    if (c1 > 0) {
      // the first entry >= target lies in ((c1 - 1) seg, c1 seg]
      const int lo = (c1 - 1) * seg + 1;
      const int hi = min(c1 * seg, K);
      int c2 = 0;
      for (int base = lo; base < hi; base += 8) {
        int v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ld_idx(min(base + e, K - 1));
#pragma unroll
        for (int e = 0; e < 8; ++e) c2 += (base + e < hi) & (v[e] < target);
      }
      start = lo + c2;
    }
    pos = start;
    int ev[4];
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = min(start + e, K - 1);
      ev[e] = ld_idx(kk);
      pv[e] = ld_p(kk);
    }
    e0 = start < K ? ev[0] : INT_MAX;
    p0 = start < K ? pv[0] : 0.f;
    e1 = start + 1 < K ? ev[1] : INT_MAX;
    p1 = start + 1 < K ? pv[1] : 0.f;
    e2 = start + 2 < K ? ev[2] : INT_MAX;
    p2 = start + 2 < K ? pv[2] : 0.f;
    e3 = start + 3 < K ? ev[3] : INT_MAX;
    p3 = start + 3 < K ? pv[3] : 0.f;
  }

  __device__ __forceinline__ int cur() const { return e0; }
  __device__ __forceinline__ float cp() const { return p0; }

  __device__ __forceinline__ void next() {
    e0 = e1;
    p0 = p1;
    e1 = e2;
    p1 = p2;
    e2 = e3;
    p2 = p3;
    e3 = kUnloaded;
    ++pos;
    if (e0 == kUnloaded) load_at(pos, e0, p0);
  }

  __device__ __forceinline__ void refill() {
    if (e1 == kUnloaded) load_at(pos + 1, e1, p1);
    if (e2 == kUnloaded) load_at(pos + 2, e2, p2);
    if (e3 == kUnloaded) load_at(pos + 3, e3, p3);
  }
};

// ---------------------------------------------------------------------------
// Forward sweep
// ---------------------------------------------------------------------------

struct FwdSweepParams {
  const uint16_t* h;
  const uint16_t* W;
  int64_t d, V;
  int64_t r0;
  int32_t rows, K;
  float k2;  // log2(e) / T
  const int32_t* tsort_idx;
  const float* tsort_p;
  int32_t n_vt;
  int32_t rbs, splits;  // tile grid: row blocks x vocabulary splits (splits <= n_vt)
  f32x4* partial;  // [splits][2][rbs * 256]: (offset m2 in log2 units, sum of exp2(s log2 e - m2), sum p*z)
  DebugCheck dbg;  // debug build: spans 0, 1 sorted lists, 2 partials, 3 h, 4 W
};

// Each thread owns one row (tid & 255) of the block and one 64-column quarter
// (tid >> 8) of every half tile: it keeps that quarter's online max / sum of
// exp2 and picks up the logits at the row's teacher indices inside it.
__global__ __launch_bounds__(kBlockThreads, 1) void k_fwd_sweep(FwdSweepParams P) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;
  const int wn = wave % kWN;
  int rb, split;
  grouped_tile(xcd_contiguous(blockIdx.x, P.rbs * P.splits), P.rbs, P.splits, 8, rb, split);
  // Vocabulary tiles split as evenly as possible (sizes differ by at most one).
  const int vt0 = static_cast<int>(static_cast<int64_t>(split) * P.n_vt / P.splits);
  const int vt1 = static_cast<int>(static_cast<int64_t>(split + 1) * P.n_vt / P.splits);
  const int rloc = tid & (kTile - 1);
  const int sub = tid >> 8;
  const int row = rb * kTile + rloc;  // chunk-local row whose statistics this thread keeps
  const bool row_ok = row < P.rows;

  Cursor cur;
  cur.dbg = P.dbg;
  cur.init(P.tsort_idx + static_cast<int64_t>(row) * P.K, P.tsort_p + static_cast<int64_t>(row) * P.K,
           P.K, vt0 * kTile, row_ok && vt0 < vt1);

  const Operand A{P.h, P.d, P.r0 + P.rows, P.d};
  const Operand B{P.W, P.d, P.V, P.d};
  const int nk = static_cast<int>((P.d + kStageK - 1) / kStageK);  // chunks past d read as zero
  float* stage = reinterpret_cast<float*>(lds);
  float m2 = -INFINITY, se = 0.f, gz = 0.f;

  for (int vt = vt0; vt < vt1; ++vt) {
    MainAcc acc;
    zero_acc(acc);
    dcheck_operands<false, false>(P.dbg, 3, 4, A, B, P.r0 + static_cast<int64_t>(rb) * kTile,
                                  static_cast<int64_t>(vt) * kTile, kTile);
    gemm_mainloop<false, false, kNBW, kWN>(A, B, P.r0 + static_cast<int64_t>(rb) * kTile,
                                           static_cast<int64_t>(vt) * kTile, nk, acc, lds);
    for (int half = 0; half < 2; ++half) {
      if ((wn >> 1) == half) stage_half_tile(acc, stage, wm, wn, lane);
      __syncthreads();
      const int64_t col0 = static_cast<int64_t>(vt) * kTile + half * 128;
      const int64_t cs = col0 + sub * 64;
      const int nvalid = static_cast<int>(min<int64_t>(64, P.V - cs));
      const float* sr = stage + rloc * kStageLd + sub * 64;
      if (nvalid > 0) {
        // Running sum of exp2(s * log2 e - m2) with an offset m2 that only
        // moves when the new values would exceed it by more than 2^64, so the
        // block's sum and its max come out of one pass over the LDS row.
        float mx = -INFINITY;
        float s = 0.f;
        const float off = m2 == -INFINITY ? 0.f : m2;
        if (nvalid == 64) {
          // four independent chains (columns c mod 4), summed in a fixed order
          f32x4 mx4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 64; c += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sr + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              mx4[e] = fmaxf(mx4[e], x[e]);
              s4[e] += __builtin_amdgcn_exp2f(fmaf(x[e], P.k2, -off));
            }
          }
          mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
          s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        } else {
          for (int c = 0; c < nvalid; ++c) {
            mx = fmaxf(mx, sr[c]);
            s += __builtin_amdgcn_exp2f(fmaf(sr[c], P.k2, -off));
          }
        }
        const float mb = mx * P.k2;
        if (m2 == -INFINITY || mb > m2 + 64.f) {
          // First block of this thread, or values far above the offset:
          // redo the block relative to its own max.
          s = 0.f;
          for (int c = 0; c < nvalid; ++c) s += __builtin_amdgcn_exp2f(fmaf(sr[c], P.k2, -mb));
          se = (m2 == -INFINITY) ? s : se * __builtin_amdgcn_exp2f(m2 - mb) + s;
          m2 = mb;
        } else {
          se += s;
        }
      }
      // Walk the row's sorted teacher list past this half tile, keeping the
      // entries that fall in this thread's quarter.
      const int c0 = static_cast<int>(col0);
      const int c1 = static_cast<int>(cs);
      while (cur.cur() < c0 + 128) {
        const int e = cur.cur();
        if (e >= c1 && e < c1 + 64) gz += cur.cp() * sr[e - c1];
        cur.next();
      }
      __syncthreads();
    }
    cur.refill();
  }
  const int ld = P.rbs * kTile;
  dstore(P.dbg, 2, kDbgPartial, P.partial + static_cast<int64_t>(split * 2 + sub) * ld + row, f32x4{m2, se, gz, 0.f});
}

// Sixteen lanes per row of the chunk merge the split statistics (each lane a
// strided subset of the parts, then a fixed-order reduction across the 16):
// row_lse, row_kl, and one fp64 KL sum per workgroup of kCombineRows rows.

__global__ __launch_bounds__(256) void k_fwd_combine(const f32x4* __restrict__ partial, int parts, int64_t ld,
                                                     int rows, int64_t r0,
                                                     const float* __restrict__ negent,
                                                     const uint8_t* __restrict__ mask,
                                                     const float* __restrict__ weight, float invT,
                                                     float* __restrict__ row_lse,
                                                     float* __restrict__ row_kl,
                                                     double* __restrict__ block_sum, DebugCheck dbg) {
  // dbg spans: 0 partials, 1 row_lse, 2 row_kl, 3 block sums, 4 negentropies
  __shared__ double red[kCombineRows];
  const int l16 = threadIdx.x & 15;
  const int rl = threadIdx.x >> 4;
  const int r = blockIdx.x * kCombineRows + rl;
  const bool ok = r < rows;
  float M = -INFINITY;
  if (ok)
    for (int s = l16; s < parts; s += 16)
      M = fmaxf(M, dload(dbg, 0, kDbgPartial, partial + static_cast<int64_t>(s) * ld + r)[0]);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
  float sum = 0.f, gz = 0.f;
  if (ok) {
    for (int s = l16; s < parts; s += 16) {
      const f32x4 pr = dload(dbg, 0, kDbgPartial, partial + static_cast<int64_t>(s) * ld + r);
      if (pr[1] > 0.f) sum += pr[1] * exp2f(pr[0] - M);
      gz += pr[2];
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o, 16);
    gz += __shfl_xor(gz, o, 16);
  }
  double kl_d = 0.0;
  if (ok && l16 == 0) {
    const float lse = (M + log2f(sum)) * kLn2;
    const float kl = dload(dbg, 4, kDbgTeacherList, negent + r) - gz * invT + lse;
    const bool valid = !mask || mask[r0 + r] != 0;
    const float w = valid ? (weight ? weight[r0 + r] : 1.0f) : 0.0f;
    dstore(dbg, 1, kDbgRowOut, row_lse + r0 + r, lse);
    if (row_kl) dstore(dbg, 2, kDbgRowOut, row_kl + r0 + r, w > 0.f ? kl : 0.f);
    kl_d = w > 0.f ? static_cast<double>(w) * kl : 0.0;
  }
  if (l16 == 0) red[rl] = kl_d;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kCombineRows; ++i) t += red[i];
    dstore(dbg, 3, kDbgRowOut, block_sum + blockIdx.x, t);
  }
}

// ---------------------------------------------------------------------------
// Backward: recompute the logits tile and form the bf16 gradient block
// ---------------------------------------------------------------------------

struct BwdGParams {
  const uint16_t* h;
  const uint16_t* W;
  int64_t d, V;
  int64_t r0;
  int32_t rows, K;
  float k2, T;
  const int32_t* tsort_idx;
  const float* tsort_p;
  const float* row_lse;
  const uint8_t* mask;
  const float* weight;
  const float* grad_loss;
  const Scalars* sc;
  int64_t slab0;
  int32_t slab_w;
  int64_t ld_g;  // row stride of G (vslab)
  uint16_t* G;   // G [pass rows][vslab], row-major
  int32_t n_vt;
  int32_t rbs, splits;  // splits <= n_vt
  DebugCheck dbg;       // debug build: spans 0, 1 sorted lists, 2 G, 3 h, 4 W, 5 row_lse
};

// One 256 x 256 tile of G = c_r (softmax(z/T) - p~) per step. The logits tile
// is staged in fp32 through LDS one 128-column half at a time (as in the
// forward); the thread that owns a row's 64-column quarter forms
// c_r (exp2(z log2(e)/T - lse_r log2(e)) - p_k) in fp32, subtracting p_k at the
// teacher entries it meets on the row's sorted list, and rounds once to bf16;
// the half tile then goes to the row-major gradient block G [pass rows][vslab]
// with coalesced 16-byte stores.
__global__ __launch_bounds__(kBlockThreads, 1) void k_bwd_g(BwdGParams P) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;
  const int wn = wave % kWN;
  int rb, split;
  grouped_tile(xcd_contiguous(blockIdx.x, P.rbs * P.splits), P.rbs, P.splits, 8, rb, split);
  // Vocabulary tiles split as evenly as possible (sizes differ by at most one).
  const int vt0 = static_cast<int>(static_cast<int64_t>(split) * P.n_vt / P.splits);
  const int vt1 = static_cast<int>(static_cast<int64_t>(split + 1) * P.n_vt / P.splits);
  const int rloc = tid & (kTile - 1);
  const int sub = tid >> 8;
  const int row = rb * kTile + rloc;
  const int64_t grow = P.r0 + row;

  // The row's mask, weight and lse are loaded unconditionally (from lse's
  // address where an optional array is absent) so that these loads and the
  // cursor's first round are in flight together.
  const bool row_in = row < P.rows;
  const int64_t grow_c = row_in ? grow : P.r0;
  const float* lse_p = P.row_lse + grow_c;
  const uint8_t mraw = *(P.mask ? P.mask + grow_c : reinterpret_cast<const uint8_t*>(lse_p));
  const float wraw = *(P.weight ? P.weight + grow_c : lse_p);
  const float lse_r = dload(P.dbg, 5, kDbgRowOut, lse_p);
  Cursor cur;
  cur.dbg = P.dbg;
  cur.init(P.tsort_idx + static_cast<int64_t>(row) * P.K, P.tsort_p + static_cast<int64_t>(row) * P.K,
           P.K, static_cast<int>(P.slab0) + vt0 * kTile, row_in && vt0 < vt1);
  float c = 0.f, lse2 = 0.f;
  if (row_in) {
    const double wsum = P.sc->wsum;
    const float g = P.grad_loss ? P.grad_loss[0] : 1.0f;
    const bool valid = !P.mask || mraw != 0;
    const float w = valid ? (P.weight ? wraw : 1.0f) : 0.0f;
    c = (w > 0.f && wsum > 0.0) ? static_cast<float>(static_cast<double>(g) * P.T * w / wsum) : 0.f;
    lse2 = lse_r * kLog2e;
  }

  const Operand A{P.h, P.d, P.r0 + P.rows, P.d};
  const Operand B{P.W, P.d, P.V, P.d};
  const int nk = static_cast<int>((P.d + kStageK - 1) / kStageK);
  float* stage = reinterpret_cast<float*>(lds);
  const int slab_end = static_cast<int>(P.slab0 + P.slab_w);

  for (int vt = vt0; vt < vt1; ++vt) {
    MainAcc acc;
    zero_acc(acc);
    const int vbase = static_cast<int>(P.slab0) + vt * kTile;
    dcheck_operands<false, false>(P.dbg, 3, 4, A, B, P.r0 + static_cast<int64_t>(rb) * kTile, vbase, kTile);
    gemm_mainloop<false, false, kNBW, kWN>(A, B, P.r0 + static_cast<int64_t>(rb) * kTile, vbase, nk, acc, lds);
    for (int half = 0; half < 2; ++half) {
      if ((wn >> 1) == half) stage_half_tile(acc, stage, wm, wn, lane);
      __syncthreads();
      const int c0 = vbase + half * 128;
      const int c1 = c0 + sub * 64;
      // This thread's 64 fp32 logits; its 64 bf16 results go back over the
      // first half of the same 256 bytes.
      float* sr = stage + rloc * kStageLd + sub * 64;
      bf16x8* so = reinterpret_cast<bf16x8*>(sr);
      while (cur.cur() < c1) cur.next();  // entries of the other quarter before this one
#pragma unroll
      for (int c8 = 0; c8 < 64; c8 += 8) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(sr + c8);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(sr + c8 + 4);
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_exp2f(fmaf(e < 4 ? x0[e] : x1[e - 4], P.k2, -lse2));
        if (cur.cur() < c1 + c8 + 8) {  // teacher entries among these 8 columns
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (cur.cur() == c1 + c8 + e) {
              q[e] -= cur.cp();
              cur.next();
            }
          }
        }
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(c1 + c8 + e < slab_end ? c * q[e] : 0.f);
        so[c8 / 8] = o;
      }
      while (cur.cur() < c0 + 128) cur.next();  // the rest of this half tile
      __syncthreads();
      // Coalesced copy of the 256 x 128 bf16 half tile: 16 lanes per row, each
      // 16 bytes (the row's two quarters sit 256 bytes apart in LDS).
      const char* sb = reinterpret_cast<const char*>(stage);
      uint16_t* gdst = P.G + static_cast<int64_t>(rb) * kTile * P.ld_g + vt * kTile + half * 128;
#pragma unroll
      for (int i = 0; i < (kTile * 16) / kBlockThreads; ++i) {
        const int q = tid + i * kBlockThreads;
        const int r = q >> 4;
        const int j = q & 15;
        dstore(P.dbg, 2, kDbgGBlock, reinterpret_cast<u32x4*>(gdst + static_cast<int64_t>(r) * P.ld_g + j * 8),
               *reinterpret_cast<const u32x4*>(sb + r * (kStageLd * 4) + (j < 8 ? j * 16 : 256 + (j - 8) * 16)));
      }
      __syncthreads();
    }
    cur.refill();
  }
}

// ---------------------------------------------------------------------------
// Backward contractions
// ---------------------------------------------------------------------------

// grad_h[chunk] (+)= G W_slab and grad_W[slab] (+)= G^T h_chunk in one
// launch (h_tiles counts grad_h tiles x vocabulary splits). The contraction
// whose tiles are longer is dispatched first, so the shorter tiles fill the
// launch's last round: with w_first the first w_tiles workgroups take grad_W
// tiles and the rest grad_h tiles, otherwise the other way round.
struct GradParams {
  GemmAccParams gh, gw;
  int32_t h_tiles, w_tiles;
  int32_t w_first;
};

__global__ __launch_bounds__(kBlockThreads, 1) void k_bwd_grads(GradParams P) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
  const int w = blockIdx.x;
  const int h0 = P.w_first ? P.w_tiles : 0;  // first workgroup of the grad_h range
  const int w0 = P.w_first ? 0 : P.h_tiles;  // first workgroup of the grad_W range
  if (w >= h0 && w < h0 + P.h_tiles) {
    gemm_acc_tile<false, true>(P.gh, xcd_contiguous_range(w, h0, P.h_tiles), lds);
  } else {
    gemm_acc_tile<true, true>(P.gw, xcd_contiguous_range(w, w0, P.w_tiles), lds);
  }
}

// grad_h[rows] (+)= sum over s of the split partial sums, in split order.
// dbg spans: 0 partial sums, 1 grad_h rows.
__global__ __launch_bounds__(256) void k_reduce_grad_h(const f32x4* __restrict__ part, int splits,
                                                       int64_t split_stride4, int64_t n4,
                                                       f32x4* __restrict__ out, int beta, DebugCheck dbg) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
    f32x4 a = beta ? dload(dbg, 1, kDbgReduce, out + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) {
      const f32x4 v = dload(dbg, 0, kDbgReduce, part + sp * split_stride4 + i);
      a = f32x4{a[0] + v[0], a[1] + v[1], a[2] + v[2], a[3] + v[3]};
    }
    dstore(dbg, 1, kDbgReduce, out + i, a);
  }
}

// bf16 grad_h rows from the fp32 accumulator (round to nearest even), adding
// the old bf16 values in fp32 first when accumulating.
// dbg spans: 0 the fp32 accumulator, 1 grad_h rows.
__global__ __launch_bounds__(256) void k_grad_h_to_bf16(const f32x4* __restrict__ src, int64_t n4,
                                                        uint16_t* __restrict__ dst, int accumulate, DebugCheck dbg) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
    f32x4 v = dload(dbg, 0, kDbgReduce, src + i);
    bf16x4* o = reinterpret_cast<bf16x4*>(dst) + i;
    if (accumulate) {
      const bf16x4 old = dload(dbg, 1, kDbgReduce, static_cast<const bf16x4*>(o));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += static_cast<float>(old[e]);
    }
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(v[e]);
    dstore(dbg, 1, kDbgReduce, o, r);
  }
}

// ---------------------------------------------------------------------------
// Teacher-cache validation: one wave per row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_validate(const int32_t* __restrict__ t_idx,
                                                  const float* __restrict__ t_logit, int64_t N,
                                                  int64_t V, int32_t K, int32_t* bad_rows) {
  __shared__ int32_t sidx[4][1024];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t r = blockIdx.x * 4LL + wave;
  const bool active = r < N;
  int bad = 0;
  if (active) {
    for (int k = lane; k < K; k += 64) {
      const int32_t v = t_idx[r * K + k];
      sidx[wave][k] = v;
      const float x = t_logit[r * K + k];
      bad |= (v < 0) | (v >= V) | !isfinite(x);
    }
  }
  __syncthreads();
  if (active) {
    for (int k = lane; k < K; k += 64) {
      const int32_t key = sidx[wave][k];
      for (int j = 0; j < k; ++j) bad |= (sidx[wave][j] == key);
    }
    const unsigned long long any = __ballot(bad);
    if (lane == 0 && any) atomicAdd(bad_rows, 1);
  }
}

// Loss-term validation: one thread per row; a row is bad when its hard label
// lies outside [0, V) or its weight is not finite.
__global__ __launch_bounds__(256) void k_validate_terms(const float* __restrict__ weight,
                                                        const int32_t* __restrict__ label, int64_t N,
                                                        int64_t V, int32_t* bad_rows) {
  const int64_t r = blockIdx.x * 256LL + threadIdx.x;
  bool bad = false;
  if (r < N) {
    if (label) bad |= label[r] < 0 || label[r] >= V;
    if (weight) bad |= !isfinite(weight[r]);
  }
  const unsigned long long any = __ballot(bad);
  const int n = __popcll(any);
  if ((threadIdx.x & 63) == 0 && n > 0) atomicAdd(bad_rows, n);
}

__global__ void k_set_int(int32_t* p, int32_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = v;
}

// ---------------------------------------------------------------------------
// Launch sequences
// ---------------------------------------------------------------------------

static inline int splits_for(int64_t rbs, int64_t tiles) {
  int64_t s = ceil_div(kTargetBlocks, rbs);
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

// Extents of the workspace regions and caller buffers of one call, for the
// debug build's checks (sizes as the plan lays them out).
struct CallSpans {
  uint32_t* word;
  HostSpan t_idx, t_logit, label, list_idx, list_p, negent, h, W;
};

static CallSpans call_spans(const Plan& p, char* ws, const uint16_t* h, const uint16_t* W, const int32_t* t_idx,
                            const float* t_logit, const int32_t* label) {
  const uint64_t list = static_cast<uint64_t>(p.list_rows) * (p.K + 1) * 4;
  return CallSpans{reinterpret_cast<uint32_t*>(ws + p.off_scalars + kDebugWordOffset),
                   {t_idx, static_cast<uint64_t>(p.N) * p.K * 4},
                   {t_logit, static_cast<uint64_t>(p.N) * p.K * 4},
                   {label, label ? static_cast<uint64_t>(p.N) * 4 : 0},
                   {ws + p.off_tidx, list},
                   {ws + p.off_tp, list},
                   {ws + p.off_negent, static_cast<uint64_t>(p.list_rows) * 4},
                   {h, static_cast<uint64_t>(p.N) * p.d * 2},
                   {W, static_cast<uint64_t>(p.V) * p.d * 2}};
}

static DebugCheck prep_check(const CallSpans& c) {
  return make_debug_check(c.word, {c.t_idx, c.t_logit, c.list_idx, c.list_p, c.negent, c.label});
}

hipError_t launch_forward(const Plan& p, const FwdArgs& a, hipStream_t st) {
  Scalars* sc = reinterpret_cast<Scalars*>(a.ws + p.off_scalars);
  float* negent = reinterpret_cast<float*>(a.ws + p.off_negent);
  int32_t* tidx = reinterpret_cast<int32_t*>(a.ws + p.off_tidx);
  float* tp = reinterpret_cast<float*>(a.ws + p.off_tp);
  f32x4* partial = reinterpret_cast<f32x4*>(a.ws + p.off_partial);
  double* bsum = reinterpret_cast<double*>(a.ws + p.off_blocksum);
  const float invT = 1.0f / p.T;
  const float k2 = kLog2e / p.T;
  const int32_t L = p.K + (a.label ? 1 : 0);  // teacher list entries per row
  const CallSpans cs = call_spans(p, a.ws, a.h, a.W, a.t_idx, a.t_logit, a.label);
  const HostSpan partial_span{partial, static_cast<uint64_t>(kTargetBlocks + p.chunk_alloc / kTile) * 2 * kTile * 16};
  const HostSpan bsum_span{bsum, static_cast<uint64_t>(p.chunk_alloc / kCombineRows) * 8};
  const DebugCheck combine_dbg = make_debug_check(
      cs.word, {partial_span, {a.row_lse, static_cast<uint64_t>(p.N) * 4},
                {a.row_kl, a.row_kl ? static_cast<uint64_t>(p.N) * 4 : 0}, bsum_span, cs.negent});

  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(256), 0, st, a.mask, a.weight, p.N, sc);
  for (int64_t c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int rows = static_cast<int>(p.N - c0 < p.chunk ? p.N - c0 : p.chunk);
    const int rbs = static_cast<int>(ceil_div(rows, kTile));
    {
      TraceScope ts(st, "teacher_prep", 0.0, 16.0 * rows * p.K);
      launch_teacher_prep(a.t_idx, a.t_logit, a.label, a.label_weight, c0, rows, p.K, L, invT, tidx, tp, negent,
                          prep_check(cs), st);
    }
    const int splits = splits_for(rbs, p.n_vt);
    FwdSweepParams fp{a.h, a.W, p.d, p.V, c0, rows, L, k2, tidx, tp,
                      static_cast<int32_t>(p.n_vt), rbs, splits, partial,
                      make_debug_check(cs.word, {cs.list_idx, cs.list_p, partial_span, cs.h, cs.W})};
    {
      const double dd = static_cast<double>(p.d);
      TraceScope ts(st, "fwd_sweep", 2.0 * rows * static_cast<double>(p.V) * dd,
                    2.0 * rows * dd + 2.0 * p.V * dd + 8.0 * rows * p.K + 16.0 * splits * rows);
      hipLaunchKernelGGL(k_fwd_sweep, dim3(rbs * splits), dim3(kBlockThreads), 0, st, fp);
    }
    const int cblocks = static_cast<int>(ceil_div(rows, kCombineRows));
    {
      TraceScope ts(st, "fwd_combine", 0.0, 16.0 * splits * rows + 16.0 * rows);
      hipLaunchKernelGGL(k_fwd_combine, dim3(cblocks), dim3(256), 0, st, partial, 2 * splits,
                         static_cast<int64_t>(rbs) * kTile, rows, c0, negent, a.mask, a.weight, invT, a.row_lse,
                         a.row_kl, bsum, combine_dbg);
    }
    hipLaunchKernelGGL(k_accumulate, dim3(1), dim3(64), 0, st, bsum, cblocks, sc);
  }
  hipLaunchKernelGGL(k_finalize, dim3(1), dim3(64), 0, st, sc, p.T, a.loss);
  return hipGetLastError();
}

hipError_t launch_backward(const Plan& p, const BwdArgs& a, hipStream_t st) {
  Scalars* sc = reinterpret_cast<Scalars*>(a.ws + p.off_scalars);
  float* negent = reinterpret_cast<float*>(a.ws + p.off_negent);
  int32_t* tidx = reinterpret_cast<int32_t*>(a.ws + p.off_tidx);
  float* tp = reinterpret_cast<float*>(a.ws + p.off_tp);
  uint16_t* G = reinterpret_cast<uint16_t*>(a.ws + p.off_G);
  const float invT = 1.0f / p.T;
  const float k2 = kLog2e / p.T;
  const int32_t L = p.K + (a.label ? 1 : 0);  // teacher list entries per row

  const bool want_w = !(p.flags & FKL_SKIP_GRAD_W);
  const bool want_h = !(p.flags & FKL_SKIP_GRAD_H);
  const bool acc_w = (p.flags & FKL_ACCUMULATE_GRAD_W) != 0;
  const bool acc_h = (p.flags & FKL_ACCUMULATE_GRAD_H) != 0;
  const bool h_bf16 = (p.flags & FKL_GRAD_H_BF16) != 0;
  // fp32 destination of grad_h while the slabs of a chunk are summed: the
  // caller's grad_h, or the workspace accumulator when grad_h is bf16
  float* gh32 = reinterpret_cast<float*>(a.ws + p.off_gh32);
  const CallSpans cs = call_spans(p, a.ws, a.h, a.W, a.t_idx, a.t_logit, a.label);
  const HostSpan g_span{G, debug_g_bytes(static_cast<uint64_t>(p.bchunk_alloc) * p.vslab * 2)};
  const HostSpan ghp_span{a.ws + p.off_ghp, static_cast<uint64_t>(p.ghp_rows) * p.d * 4};
  const HostSpan gh32_span{gh32, h_bf16 ? static_cast<uint64_t>(p.bchunk_alloc) * p.d * 4 : 0};

  if (!want_w && !want_h) return hipGetLastError();
  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(256), 0, st, a.mask, a.weight, p.N, sc);
  if (p.N == 0) {
    if (want_w && !acc_w) hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, st, a.grad_W, p.V * p.d);
    return hipGetLastError();
  }
  const int64_t n_slabs = ceil_div(p.V, p.vslab);
  int64_t chunk_index = 0;
  for (int64_t c0 = 0; c0 < p.N; c0 += p.bchunk, ++chunk_index) {
    const int rows = static_cast<int>(p.N - c0 < p.bchunk ? p.N - c0 : p.bchunk);
    const int rbs = static_cast<int>(ceil_div(rows, kTile));
    {
      TraceScope ts(st, "teacher_prep", 0.0, 16.0 * rows * p.K);
      launch_teacher_prep(a.t_idx, a.t_logit, a.label, a.label_weight, c0, rows, p.K, L, invT, tidx, tp, negent,
                          prep_check(cs), st);
    }
    const double dd = static_cast<double>(p.d);
    // this pass's grad_h rows (fp32 or bf16 in the caller's buffer)
    // (grad_h is NULL when it is skipped: no kernel then writes it)
    const HostSpan gh_rows = want_h ? HostSpan{static_cast<char*>(a.grad_h) + c0 * p.d * (h_bf16 ? 2 : 4),
                                               static_cast<uint64_t>(rows) * p.d * (h_bf16 ? 2 : 4)}
                                    : HostSpan{nullptr, 0};
    for (int64_t s = 0; s < n_slabs; ++s) {
      const int64_t slab0 = s * p.vslab;
      const int slab_w = static_cast<int>(p.V - slab0 < p.vslab ? p.V - slab0 : p.vslab);
      const int nvt = static_cast<int>(ceil_div(slab_w, kTile));
      const int splits = splits_for(rbs, nvt);
      BwdGParams gp{a.h, a.W, p.d, p.V, c0, rows, L, k2, p.T, tidx, tp, a.row_lse, a.mask, a.weight,
                    a.grad_loss, sc, slab0, slab_w, p.vslab, G, nvt, rbs, splits,
                    make_debug_check(cs.word, {cs.list_idx, cs.list_p, g_span, cs.h, cs.W,
                                               {a.row_lse, static_cast<uint64_t>(p.N) * 4}})};
      {
        TraceScope ts(st, "bwd_g", 2.0 * rows * slab_w * dd,
                      2.0 * rows * dd + 2.0 * slab_w * dd + 2.0 * rows * slab_w + 8.0 * rows * p.K);
        hipLaunchKernelGGL(k_bwd_g, dim3(rbs * splits), dim3(kBlockThreads), 0, st, gp);
      }

      // grad_h[c0 : c0 + rows] (+)= G[:, :slab_w] @ W[slab0 : slab0 + slab_w] and
      // grad_W[slab0 : slab0 + slab_w] (+)= G[:rows, :slab_w]^T @ h[c0 : c0 + rows], one launch.
      GradParams gp2;
      GemmAccParams& hp = gp2.gh;
      const int64_t rows_written = static_cast<int64_t>(rbs) * kTile;  // G rows this pass wrote
      int hsplits = want_h ? grad_h_splits(rows, slab_w, p.d) : 1;
      if (hsplits > 1 && hsplits * rows_written > p.ghp_rows)
        hsplits = static_cast<int>(p.ghp_rows / rows_written);
      if (hsplits < 1) hsplits = 1;
      hp.A = Operand{G, p.vslab, rows_written, slab_w};
      hp.B = Operand{a.W + slab0 * p.d, p.d, p.d, slab_w};
      hp.nk = static_cast<int32_t>(ceil_div(slab_w, kStageK));
      hp.ldc = p.d;
      hp.m_lim = rows;
      hp.n_lim = p.d;
      hp.mblocks = rbs;
      hp.nblocks = static_cast<int32_t>(ceil_div(p.d, kTile));
      hp.splits = hsplits;
      hp.kper = static_cast<int32_t>(ceil_div(hp.nk, hsplits));
      if (hsplits > 1) {  // partial sums, reduced into grad_h after the launch
        hp.C = reinterpret_cast<float*>(a.ws + p.off_ghp);
        hp.beta = 0;
        hp.c_split = rows_written * p.d;
      } else {
        hp.C = h_bf16 ? gh32 : static_cast<float*>(a.grad_h) + c0 * p.d;
        hp.beta = s > 0 || (acc_h && !h_bf16);
        hp.c_split = 0;
      }
      hp.dbg = make_debug_check(cs.word, {hsplits > 1 ? ghp_span : (h_bf16 ? gh32_span : gh_rows), g_span, cs.W});
      GemmAccParams& wp = gp2.gw;
      wp.A = Operand{G, p.vslab, slab_w, rows_written};
      wp.B = Operand{a.h + c0 * p.d, p.d, p.d, rows};
      wp.nk = static_cast<int32_t>(ceil_div(rows, kStageK));
      wp.C = a.grad_W + slab0 * p.d;
      wp.ldc = p.d;
      wp.m_lim = slab_w;
      wp.n_lim = p.d;
      wp.beta = chunk_index > 0 || acc_w;
      wp.mblocks = nvt;
      wp.nblocks = static_cast<int32_t>(ceil_div(p.d, kTile));
      wp.splits = 1;
      wp.kper = wp.nk;
      wp.c_split = 0;
      wp.dbg = make_debug_check(cs.word, {want_w ? HostSpan{a.grad_W + slab0 * p.d, static_cast<uint64_t>(slab_w) * p.d * 4}
                                                 : HostSpan{nullptr, 0},
                                          g_span, cs.h});
      gp2.h_tiles = want_h ? hp.mblocks * hp.nblocks * hsplits : 0;
      gp2.w_tiles = want_w ? wp.mblocks * wp.nblocks : 0;
      // longer tiles first: grad_h tiles contract over kper stages of the
      // slab, grad_W tiles over the pass's rows
      gp2.w_first = wp.nk > hp.kper ? 1 : 0;
      {
        const double hw = (want_h ? 1.0 : 0.0) + (want_w ? 1.0 : 0.0);
        TraceScope ts(st, "bwd_grads", 2.0 * hw * rows * slab_w * dd,
                      2.0 * rows * slab_w + 2.0 * slab_w * dd + 2.0 * rows * dd +
                          (want_h ? (hp.beta ? 8.0 : 4.0) * rows * dd : 0.0) +
                          (want_w ? (wp.beta ? 8.0 : 4.0) * slab_w * dd : 0.0));
        hipLaunchKernelGGL(k_bwd_grads, dim3(gp2.h_tiles + gp2.w_tiles), dim3(kBlockThreads), 0, st, gp2);
      }
      if (hsplits > 1) {
        const int64_t n4 = static_cast<int64_t>(rows) * p.d / 4;
        const int64_t rgrid = ceil_div(n4, 256) < 2048 ? ceil_div(n4, 256) : 2048;
        TraceScope ts(st, "grad_h_reduce", 0.0, 4.0 * rows * p.d * (hsplits + (s > 0 ? 2 : 1)));
        hipLaunchKernelGGL(k_reduce_grad_h, dim3(static_cast<unsigned>(rgrid)),
                           dim3(256), 0, st, reinterpret_cast<const f32x4*>(a.ws + p.off_ghp), hsplits,
                           rows_written * p.d / 4, n4,
                           reinterpret_cast<f32x4*>(h_bf16 ? gh32 : static_cast<float*>(a.grad_h) + c0 * p.d),
                           static_cast<int>(s > 0 || (acc_h && !h_bf16)),
                           make_debug_check(cs.word, {ghp_span, h_bf16 ? gh32_span : gh_rows}));
      }
    }
    if (want_h && h_bf16) {
      const int64_t n4 = static_cast<int64_t>(rows) * p.d / 4;
      const int64_t cgrid = ceil_div(n4, 256) < 2048 ? ceil_div(n4, 256) : 2048;
      TraceScope ts(st, "grad_h_to_bf16", 0.0, (acc_h ? 8.0 : 6.0) * rows * p.d);
      hipLaunchKernelGGL(k_grad_h_to_bf16, dim3(static_cast<unsigned>(cgrid)), dim3(256), 0, st,
                         reinterpret_cast<const f32x4*>(gh32), n4,
                         static_cast<uint16_t*>(a.grad_h) + c0 * p.d, static_cast<int>(acc_h),
                         make_debug_check(cs.word, {gh32_span, gh_rows}));
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free forward
// ---------------------------------------------------------------------------

// The workspace of fkl_forward_static, for callers that cannot allocate. Every
// GPU the library runs on holds its own copy until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device is handed to the
// kernels.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(hipStream_t stream, char** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_debug_clear(uint32_t* word, hipStream_t st) {
  hipLaunchKernelGGL(k_set_int, dim3(1), dim3(64), 0, st, reinterpret_cast<int32_t*>(word), 0);
  return hipGetLastError();
}

hipError_t launch_validate(int64_t N, int64_t V, int32_t K, const int32_t* t_idx, const float* t_logit,
                           int32_t* bad_rows, hipStream_t st) {
  hipLaunchKernelGGL(k_set_int, dim3(1), dim3(64), 0, st, bad_rows, 0);
  if (N > 0)
    hipLaunchKernelGGL(k_validate, dim3(ceil_div(N, 4)), dim3(256), 0, st, t_idx, t_logit, N, V, K,
                       bad_rows);
  return hipGetLastError();
}

hipError_t launch_validate_terms(int64_t N, int64_t V, const float* weight, const int32_t* label,
                                 int32_t* bad_rows, bool clear, hipStream_t st) {
  if (clear) hipLaunchKernelGGL(k_set_int, dim3(1), dim3(64), 0, st, bad_rows, 0);
  if (N > 0 && (weight || label))
    hipLaunchKernelGGL(k_validate_terms, dim3(ceil_div(N, 256)), dim3(256), 0, st, weight, label, N, V,
                       bad_rows);
  return hipGetLastError();
}

}  // namespace fkl
