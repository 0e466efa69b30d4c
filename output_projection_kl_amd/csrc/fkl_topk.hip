// Offline teacher-cache builder: per row of h, the K largest logits of
// h W^T with their vocabulary indices (blog post on the page "Efficient
// Offline Top-K Logits and Fused Chunked KL Loss Enable Scalable LLM
// Distillation", section "Two systems changes": the teacher's top-100
// logits per position are cached once, offline, and nothing else of its
// distribution is kept).
//
// Keys make every element distinct: key = (order-preserving bits of z) << 32
// | (0xFFFFFFFF - index), so larger keys are larger logits and, for equal
// logits, lower indices. Selection by 12-bit radix digits of the key from the
// top, keeping only the keys that share the digits chosen so far, until the
// digit bin at the K-th key is taken whole.
//
// Fused route (default), per pass of rows; no [rows x V] block is formed:
//   k_topk_logits  the logits of the sampled vocabulary tiles (every stride-th
//                  full tile, gathered once into a compact copy of W by
//                  k_gather_tiles) for the pass's rows
//   k_topk_thresh  one workgroup per row: the row's j-th largest sampled key,
//                  chosen so that about cap / 2 of the row's keys are expected
//                  at or above it
//   k_topk_sweep   256-row block x a run of the other vocabulary tiles: MFMA
//                  logits tile -> LDS -> the keys at or above the row's
//                  threshold appended to the row's candidate list
//   k_topk_pick    one workgroup per row: the top K among the candidates and
//                  the sampled keys at or above the threshold; exact whenever
//                  at least K keys reached the threshold and none was dropped
//                  (a row with fewer than K, or more than cap, flags the pass)
//   k_topk_logits + k_topk_select (materialised route) redo a flagged pass;
//                  they return at once when the flag is clear
//
// Materialised route (FKL_TOPK_MATERIALIZE, FKL_TOPK_DIRECT, and the redo),
// per block of rows:
//   k_topk_logits  256 x 256 MFMA tiles of z = h_chunk W^T (fp32 accumulation)
//                  written to an fp32 logits block in the workspace
//   k_topk_select  one workgroup per row: exact radix selection of the K
//                  largest keys, then a bitonic sort in LDS. Each row is read
//                  once in the usual case: a threshold key is taken from a
//                  sample of the row (runs of contiguous logits spread over
//                  it) such that a bounded number of keys, at least K and at
//                  most half the LDS buffer, is expected at or above it; one
//                  pass collects those keys into LDS, and the selection runs
//                  there. A threshold that keeps fewer than K keys or more than
//                  the buffer holds is moved and the row read again; after
//                  three tries (or with FKL_TOPK_DIRECT) the row is selected
//                  directly: a histogram pass over the row, a pass that takes
//                  the keys above the boundary bin and copies the bin to LDS,
//                  the rest in LDS (or over the row when the bin does not fit).
// Every route selects the same K keys: the logits come from the same MFMA
// tile code with the same contraction order.
#include <climits>

#include "fkl_device.h"
#include "fkl_internal.h"
#include "fkl_tiles.h"

namespace fkl {

// run_if: NULL, or a flag that makes the whole launch return at once when 0.
__global__ __launch_bounds__(kBlockThreads, 1) void k_topk_logits(GemmAccParams P, const uint32_t* run_if) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
  if (run_if && *run_if == 0) return;
  const int tiles = P.mblocks * P.nblocks;
  gemm_acc_tile<false, false>(P, xcd_contiguous(blockIdx.x, tiles), lds);
}

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t topk_key(float v, int i) {
  return (static_cast<uint64_t>(ordered_bits(v)) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - i);
}

constexpr int kSelThreads = 256;
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr int kMaxK = 1024;
constexpr int kCand = 4096;  // LDS candidate keys
constexpr int kSampleRuns = 64;  // threshold sample: runs of contiguous logits
constexpr int kSampleRun = 32;
constexpr int kSample = kSampleRuns * kSampleRun;
static_assert(kSample == kSelThreads * 8, "each thread samples 8 logits");
static_assert(kSample <= kCand, "the sample is held in the candidate buffer");

struct SelectState {
  uint64_t prefix;  // chosen digits, most significant first
  int pbits;        // number of chosen bits
  uint32_t need;    // keys still to take among those matching prefix
};

// One digit (DB bits) of the selection over n keys given by key_at(i):
// histogram of the next digit among keys matching the prefix, then the digit
// holding the need-th largest key. Returns the number of keys in that digit's
// bin. hist holds 1 << DB counters.
template <int DB = kDigitBits, class KeyAt>
__device__ uint32_t select_digit(KeyAt key_at, int n, SelectState& st, uint32_t* hist, uint32_t* wave_tot,
                                 uint32_t* s_vals) {
  const int tid = threadIdx.x;
  const int w = 64 - st.pbits < DB ? 64 - st.pbits : DB;
  const int nb = 1 << w;
  const int shift = 64 - st.pbits - w;
  for (int b = tid; b < nb; b += kSelThreads) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kSelThreads) {
    const uint64_t key = key_at(i);
    if (st.pbits == 0 || (key >> (64 - st.pbits)) == st.prefix)
      atomicAdd(&hist[static_cast<uint32_t>(key >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int b0 = tid * per;
  const int b1 = b0 + per < nb ? b0 + per : nb;
  uint32_t mine = 0;
  for (int b = b0; b < b1; ++b) mine += hist[b];
  // Keys in the bins of all later threads: a suffix sum within the wave, then
  // the totals of the later waves.
  const int lane = tid & 63;
  const int wv = tid >> 6;
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(incl), o, 64));
    if (lane + o < 64) incl += y;
  }
  if (lane == 0) wave_tot[wv] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
  for (int w2 = wv + 1; w2 < kSelThreads / 64; ++w2) above += wave_tot[w2];
  if (above < st.need && above + mine >= st.need) {
    for (int b = b1 - 1; b >= b0; --b) {
      const uint32_t c = hist[b];
      if (above + c >= st.need) {
        s_vals[0] = static_cast<uint32_t>(b);
        s_vals[1] = above;
        s_vals[2] = c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
  st.need -= s_vals[1];
  st.prefix = (st.prefix << w) | s_vals[0];
  st.pbits += w;
  const uint32_t in_bin = s_vals[2];
  __syncthreads();  // every thread has read s_vals
  return in_bin;
}

// Digits until the bin at the K-th key is taken whole (at the latest when all
// 64 bits are fixed: keys are distinct), or until max_bits are fixed: then the
// keys whose top bits are at least the prefix are the need largest and the
// rest of the last bin.
template <int DB = kDigitBits, class KeyAt>
__device__ void select_rest(KeyAt key_at, int n, SelectState& st, uint32_t* hist, uint32_t* wave_tot,
                            uint32_t* s_vals, int max_bits = 64) {
  while (st.pbits < max_bits) {
    if (select_digit<DB>(key_at, n, st, hist, wave_tot, s_vals) == st.need) break;
  }
}

// Direct selection over the row: the first digit from a histogram pass, then a
// pass that takes the keys above the boundary bin and copies the bin to cand[];
// the remaining digits in LDS, or over the row when the bin does not fit.
// The K keys go to keys[] in no particular order. *s_fill and *s_cand are 0.
__device__ void select_row(const float* row, int V, int K, uint64_t* keys, uint64_t* cand, uint32_t* hist,
                           uint32_t* wave_tot, uint32_t* s_vals, uint32_t* s_fill, uint32_t* s_cand) {
  const int tid = threadIdx.x;
  auto row_key = [row](int i) { return topk_key(row[i], i); };
  SelectState st{0, 0, static_cast<uint32_t>(K)};
  const uint32_t in_bin = select_digit(row_key, V, st, hist, wave_tot, s_vals);
  // Pass 2 over the row: keys above the boundary bin are taken now; the
  // boundary bin goes to LDS (or everything of the bin when it is taken whole).
  const uint64_t d0 = st.prefix;
  const bool whole = in_bin == st.need;
  for (int i = tid; i < V; i += kSelThreads) {
    const uint64_t key = row_key(i);
    const uint64_t top = key >> (64 - kDigitBits);
    if (top > d0 || (whole && top == d0)) {
      const uint32_t slot = atomicAdd(s_fill, 1u);
      if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
    } else if (top == d0) {
      const uint32_t c = atomicAdd(s_cand, 1u);
      if (c < static_cast<uint32_t>(kCand)) cand[c] = key;
    }
  }
  __syncthreads();
  if (!whole) {
    const uint32_t nc = *s_cand;
    if (nc <= static_cast<uint32_t>(kCand)) {
      const uint64_t* cp = cand;
      auto cand_key = [cp](int i) { return cp[i]; };
      select_rest(cand_key, static_cast<int>(nc), st, hist, wave_tot, s_vals);
      for (uint32_t i = tid; i < nc; i += kSelThreads) {
        const uint64_t key = cand[i];
        if ((key >> (64 - st.pbits)) >= st.prefix) {
          const uint32_t slot = atomicAdd(s_fill, 1u);
          if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
        }
      }
    } else {
      // Boundary bin too large for LDS: finish over the row itself.
      select_rest(row_key, V, st, hist, wave_tot, s_vals);
      for (int i = tid; i < V; i += kSelThreads) {
        const uint64_t key = row_key(i);
        if ((key >> (64 - kDigitBits)) == d0 && (key >> (64 - st.pbits)) >= st.prefix) {
          const uint32_t slot = atomicAdd(s_fill, 1u);
          if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
        }
      }
    }
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v)), mask, 64));
  const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v >> 32)), mask, 64));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Bitonic sort of the Kp keys (K selected, the rest 0), descending, and the
// row's output: the K logits and their indices. Up to 128 keys are sorted by
// the first wave alone in registers (two keys per lane, element e = 2 lane +
// j; partners more than one element apart are exchanged with shuffles), with
// zeros past Kp, which sort last (no key is 0): no block barrier. Longer
// lists are sorted by the whole workgroup through LDS. Called after a block
// barrier that makes keys[] complete; the kernel ends after it.
// (dbg spans 4 and 5: t_idx and t_logit.)
__device__ void sort_and_write(uint64_t* keys, int K, int Kp, int64_t out_row, int32_t* __restrict__ t_idx,
                               float* __restrict__ t_logit, const DebugCheck& dbg) {
  const int tid = threadIdx.x;
  const int64_t out = out_row * static_cast<int64_t>(K);
  if (Kp <= 128) {
    if (tid >= 64) return;
    const int lane = tid;
    uint64_t v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = 2 * lane + j < Kp ? keys[2 * lane + j] : 0;
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        if (stride == 1) {
          // partners 2 lane and 2 lane + 1: the lower element keeps the
          // larger key where the block of `size` sorts descending
          const bool desc = ((2 * lane) & size) == 0;
          const uint64_t hi = v[0] > v[1] ? v[0] : v[1];
          const uint64_t lo = v[0] > v[1] ? v[1] : v[0];
          v[0] = desc ? hi : lo;
          v[1] = desc ? lo : hi;
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int e = 2 * lane + j;
            const int partner = e ^ stride;
            const uint64_t other = shfl_xor_u64(v[j], stride >> 1);
            const int lower = e < partner ? e : partner;
            const bool keep_max = (e == lower) == ((lower & size) == 0);
            v[j] = keep_max ? (v[j] > other ? v[j] : other) : (v[j] > other ? other : v[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = 2 * lane + j;
      if (k < K) {
        dstore(dbg, 5, kDbgTopkOut, t_logit + out + k, from_ordered_bits(static_cast<uint32_t>(v[j] >> 32)));
        dstore(dbg, 4, kDbgTopkOut, t_idx + out + k, static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(v[j])));
      }
    }
    return;
  }
  for (int size = 2; size <= Kp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < Kp; i += kSelThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = keys[i];
          const uint64_t b = keys[j];
          const bool desc = (i & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            keys[i] = b;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int k = tid; k < K; k += kSelThreads) {
    const uint64_t key = keys[k];
    dstore(dbg, 5, kDbgTopkOut, t_logit + out + k, from_ordered_bits(static_cast<uint32_t>(key >> 32)));
    dstore(dbg, 4, kDbgTopkOut, t_idx + out + k, static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key)));
  }
}

__global__ __launch_bounds__(kSelThreads) void k_topk_select(const float* __restrict__ logits, int64_t ld,
                                                             int V, int K, int Kp, int64_t r0, int direct,
                                                             const uint32_t* run_if,
                                                             int32_t* __restrict__ t_idx,
                                                             float* __restrict__ t_logit, DebugCheck dbg) {
  // dbg spans: 0 the logits block, 4 t_idx, 5 t_logit
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t keys[kMaxK];
  __shared__ uint64_t cand[kCand];
  __shared__ uint32_t wave_tot[kSelThreads / 64];
  __shared__ uint32_t s_vals[3];
  __shared__ uint32_t s_fill, s_cand;
  const int tid = threadIdx.x;
  if (run_if && *run_if == 0) return;
  const float* row = logits + static_cast<int64_t>(blockIdx.x) * ld;
  if (!dcheck_range(dbg, 0, kDbgTopkWork, row, static_cast<uint64_t>((V + 3) & ~3) * 4)) return;

  for (int i = tid; i < Kp; i += kSelThreads) keys[i] = 0;
  if (tid == 0) {
    s_fill = 0;
    s_cand = 0;
  }
  __syncthreads();
  const uint64_t* cp = cand;
  auto cand_key = [cp](int i) { return cp[i]; };

  bool done = false;
  if (!direct) {
    // Sampled threshold: the j-th largest key of the sample, so that about
    // j * V / kSample keys of the row are at or above it. j starts at
    // max(16, 3K * kSample / V) (16 sampled keys keep the count within a few
    // tens of percent of its expectation), capped so that the expected count
    // stays within half the buffer. A count outside [K, kCand] moves j in
    // proportion towards the target and reads the row again; after three
    // tries the row is selected whole. Rows that fit the buffer take every key.
    const int64_t target = 3 * K < kCand / 2 ? 3 * K : kCand / 2;
    const int64_t j_cap = static_cast<int64_t>(kCand / 2) * kSample / V;
    int64_t j = (target * kSample + V / 2) / V;
    if (j < 16) j = 16;
    if (j > j_cap) j = j_cap;
    if (j < 1) j = 1;
    for (int attempt = 0; attempt < 3 && !done; ++attempt) {
      uint64_t thr = 0;
      if (V > kCand) {
        const int run = tid >> 2;
        const int i0 = static_cast<int>((static_cast<int64_t>(run) * V / kSampleRuns) & ~int64_t(3)) + (tid & 3) * 8;
        const f32x4 a = *reinterpret_cast<const f32x4*>(row + i0);
        const f32x4 b = *reinterpret_cast<const f32x4*>(row + i0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cand[tid * 8 + e] = topk_key(a[e], i0 + e);
          cand[tid * 8 + 4 + e] = topk_key(b[e], i0 + 4 + e);
        }
        __syncthreads();
        SelectState ss{0, 0, static_cast<uint32_t>(j)};
        select_rest(cand_key, kSample, ss, hist, wave_tot, s_vals);
        thr = ss.pbits >= 64 ? ss.prefix : ss.prefix << (64 - ss.pbits);
      }
      if (tid == 0) s_cand = 0;
      __syncthreads();  // the sample is read and the count cleared
      // One pass over the row: keys at or above the threshold go to cand[].
      // A lane looks at 32 logits per step; a wave whose lanes see none whose
      // ordered bits reach the threshold's moves on, otherwise it counts its
      // keys at or above the threshold, reserves room with one LDS atomic and
      // writes them.
      {
        const int v4 = (V + 3) & ~3;
        const uint32_t thr_hi = static_cast<uint32_t>(thr >> 32);
        const int lane = tid & 63;
        constexpr int kU = 8;
        for (int i0 = tid * 4; i0 < v4; i0 += kSelThreads * 4 * kU) {
          f32x4 x[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kSelThreads * 4;
            x[u] = i < v4 ? *reinterpret_cast<const f32x4*>(row + i) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
          bool near = false;
#pragma unroll
          for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) near |= ordered_bits(x[u][e]) >= thr_hi;
          if (__ballot(near) == 0) continue;
          uint32_t c = 0;
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kSelThreads * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) c += (i + e < V && topk_key(x[u][e], i + e) >= thr) ? 1u : 0u;
          }
          // exclusive prefix of c over the wave's lanes, from the bit planes
          // of c (c <= 32)
          uint32_t pre = 0, tot = 0;
#pragma unroll
          for (int bit = 0; bit < 6; ++bit) {
            const uint64_t m = __ballot((c >> bit) & 1u);
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
            pre += below << bit;
            tot += static_cast<uint32_t>(__popcll(m)) << bit;
          }
          const int leader = __ffsll(static_cast<unsigned long long>(__ballot(true))) - 1;
          uint32_t base = 0;
          if (lane == leader) base = atomicAdd(&s_cand, tot);
          uint32_t pos = __builtin_amdgcn_readfirstlane(base) + pre;
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kSelThreads * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint64_t key = topk_key(x[u][e], i + e);
              if (i + e < V && key >= thr) {
                if (pos < static_cast<uint32_t>(kCand)) cand[pos] = key;
                ++pos;
              }
            }
          }
        }
      }
      __syncthreads();
      const uint32_t n_cand = s_cand;
      __syncthreads();  // every thread has read s_cand
      if (n_cand >= static_cast<uint32_t>(K) && n_cand <= static_cast<uint32_t>(kCand)) {
        SelectState st{0, 0, static_cast<uint32_t>(K)};
        select_rest(cand_key, static_cast<int>(n_cand), st, hist, wave_tot, s_vals);
        for (uint32_t i = tid; i < n_cand; i += kSelThreads) {
          const uint64_t key = cand[i];
          if ((key >> (64 - st.pbits)) >= st.prefix) {
            const uint32_t slot = atomicAdd(&s_fill, 1u);
            if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
          }
        }
        done = true;
      } else {
        // n_cand >= j > 0: scale j towards the target count
        int64_t jn = j * target / static_cast<int64_t>(n_cand);
        if (jn < 1) jn = 1;
        if (jn > kSample) jn = kSample;
        if (jn == j) break;
        j = jn;
      }
    }
  }
  if (!done) {
    if (tid == 0) s_cand = 0;
    select_row(row, V, K, keys, cand, hist, wave_tot, s_vals, &s_fill, &s_cand);
  }
  __syncthreads();
  sort_and_write(keys, K, Kp, r0 + blockIdx.x, t_idx, t_logit, dbg);
}

// ---------------------------------------------------------------------------
// Fused route
// ---------------------------------------------------------------------------

// Compact copy of the sampled tiles of W: tile s of the copy is rows
// [s * stride * 256, + 256) of W (every sampled tile is a full tile). One
// 16-byte chunk per thread and step.
// (dbg spans: 0 the compact copy, 1 W.)
__global__ __launch_bounds__(256) void k_gather_tiles(const uint16_t* __restrict__ W, int64_t d, int stride,
                                                      int n_sample, uint16_t* __restrict__ Ws, DebugCheck dbg) {
  const int64_t per_row = d / 8;
  const int64_t total = static_cast<int64_t>(n_sample) * kTile * per_row;
  for (int64_t q = blockIdx.x * 256LL + threadIdx.x; q < total; q += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = q / per_row;  // row of the copy
    const int64_t c = q - r * per_row;
    const int64_t src = (r / kTile) * stride * kTile + (r % kTile);
    dstore(dbg, 0, kDbgTopkWork, reinterpret_cast<u32x4*>(Ws + r * d) + c,
           dload(dbg, 1, kDbgOperand, reinterpret_cast<const u32x4*>(W + src * d) + c));
  }
}

// Vocabulary index of column i of the sample (sampled tile i / 256).
__device__ __forceinline__ int sample_col(int i, int stride) { return (i >> 8) * stride * kTile + (i & 255); }

constexpr int kMaxSample = kTopkMaxSampleTiles * kTile;
constexpr int kFusedDigitBits = 8;   // radix digits of the fused route's selections
constexpr int kThreshBits = 24;      // the threshold is fixed to its top 24 bits

// The threshold's two digits: 12 bits each fix the top 24 bits of the
// logit's ordered bits. The first digit (sign, exponent and three mantissa
// bits) spreads the sampled keys over enough bins that the histogram's LDS
// atomics rarely meet on one address.
constexpr int kThreshDigit = 12;
constexpr int kThreshBins = 1 << kThreshDigit;
constexpr int kThreshLoads = kMaxSample / (4 * kSelThreads);  // 16-byte sample loads per thread
static_assert(kThreshDigit * 2 == kThreshBits, "two digits fix the threshold's bits");
static_assert(kThreshBins % (4 * kSelThreads) == 0, "each thread clears whole 16-byte groups of bins");

struct BinPick {
  uint32_t bin;    // the digit's bin holding the need-th largest key
  uint32_t above;  // keys in higher bins
  uint32_t count;  // keys in the bin
};

// One digit of the threshold over the workgroup's sampled keys (each thread's
// in registers: ob[q][e] where live[q]): a histogram of bits [shift, shift +
// 12) among the keys whose bits from hi_shift up equal hi (every key when
// !match), then the bin holding the need-th largest of them. need >= 1 and
// at most the number of keys counted.
template <int Q>
__device__ BinPick thresh_digit(const uint32_t (&ob)[Q][4], const bool (&live)[Q], int shift, bool match,
                                int hi_shift, uint32_t hi, uint32_t need, uint32_t* hist, uint32_t* wave_tot,
                                uint32_t* s_vals) {
  const int tid = threadIdx.x;
  for (int b = tid * 4; b < kThreshBins; b += kSelThreads * 4) *reinterpret_cast<u32x4*>(hist + b) = u32x4{0, 0, 0, 0};
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (live[q] && (!match || (ob[q][e] >> hi_shift) == hi))
        atomicAdd(&hist[(ob[q][e] >> shift) & (kThreshBins - 1)], 1u);
    }
  }
  __syncthreads();
  // thread t owns bins [16 t, 16 t + 16); keys in later threads' bins are larger
  constexpr int kPer = kThreshBins / kSelThreads;
  const int b0 = tid * kPer;
  uint32_t c[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int v = 0; v < kPer / 4; ++v) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(hist + b0 + 4 * v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[4 * v + e] = x[e];
      mine += x[e];
    }
  }
  const int lane = tid & 63;
  const int wv = tid >> 6;
  uint32_t incl = mine;  // this thread's keys and those of the later lanes of its wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(incl), o, 64));
    if (lane + o < 64) incl += y;
  }
  if (lane == 0) wave_tot[wv] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
  for (int w2 = wv + 1; w2 < kSelThreads / 64; ++w2) above += wave_tot[w2];
  if (above < need && above + mine >= need) {
#pragma unroll
    for (int b = kPer - 1; b >= 0; --b) {
      if (above + c[b] >= need) {
        s_vals[0] = static_cast<uint32_t>(b0 + b);
        s_vals[1] = above;
        s_vals[2] = c[b];
        break;
      }
      above += c[b];
    }
  }
  __syncthreads();
  const BinPick r{s_vals[0], s_vals[1], s_vals[2]};
  __syncthreads();  // every thread has read s_vals and wave_tot
  return r;
}

// One workgroup per row of the pass: thr[row] = a key at or below the row's
// j-th largest sampled key: the lower bound of the bin of 24-bit prefixes
// that holds it (of its 12-bit bin when that bin is taken whole); 0 when
// j = 0 (every key is a candidate). Any threshold gives the exact top K as
// long as at least K of the row's keys reach it and none is dropped (the pick
// checks both), so aiming at the j-th key need not be exact. The row's
// sampled keys at or above the threshold go to its extra candidate slice
// (xcap slots; the sweep skips the sampled tiles), their number to xcnt[row].
// Workgroup 0 also clears the pass's redo flag (the previous pass's redo has
// read it: launches are in stream order).
__global__ __launch_bounds__(kSelThreads) void k_topk_thresh(const float* __restrict__ sample, int S, int stride,
                                                             int j, uint64_t* __restrict__ thr,
                                                             uint32_t* __restrict__ xcnt,
                                                             uint64_t* __restrict__ xcand, int xcap,
                                                             uint32_t* flag, DebugCheck dbg) {
  // dbg spans: 0 the sample's logits, 1 extra slices, 2 thresholds, 3 extra-slice counts
  __shared__ __align__(16) uint32_t hist[kThreshBins];
  __shared__ uint32_t wave_tot[kSelThreads / 64];
  __shared__ uint32_t s_vals[3];
  __shared__ uint32_t s_hits;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  if (row == 0 && tid == 0) *flag = 0;
  if (tid == 0) s_hits = 0;
  const float* zr = sample + static_cast<int64_t>(row) * S;
  if (!dcheck_range(dbg, 0, kDbgTopkWork, zr, static_cast<uint64_t>(S) * 4)) return;
  // sampled logit i = 4 f + e, f = tid + 256 q: the ordered bits in registers
  uint32_t ob[kThreshLoads][4];
  bool live[kThreshLoads];
#pragma unroll
  for (int q = 0; q < kThreshLoads; ++q) {
    const int f = tid + kSelThreads * q;
    live[q] = 4 * f < S;
    const f32x4 v = live[q] ? *reinterpret_cast<const f32x4*>(zr + 4 * f) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[q][e] = ordered_bits(v[e]);
  }
  uint32_t t32 = 0;
  if (j > 0) {
    const BinPick d1 = thresh_digit(ob, live, 32 - kThreshDigit, false, 32, 0u, static_cast<uint32_t>(j), hist,
                                    wave_tot, s_vals);
    t32 = d1.bin << (32 - kThreshDigit);
    const uint32_t need = static_cast<uint32_t>(j) - d1.above;
    if (d1.count != need) {
      const BinPick d2 = thresh_digit(ob, live, 32 - 2 * kThreshDigit, true, 32 - kThreshDigit, d1.bin, need,
                                      hist, wave_tot, s_vals);
      t32 |= d2.bin << (32 - 2 * kThreshDigit);
    }
  }
  const uint64_t t = static_cast<uint64_t>(t32) << 32;
  __syncthreads();  // s_hits is zero before any wave counts into it (j = 0 runs no digit)
  // the keys at or above the threshold go straight to the row's extra slice
  // (in no particular order; the first xcap of them), counted in s_hits
  uint64_t* xrow = xcand + static_cast<int64_t>(row) * xcap;
  const int lane = tid & 63;
#pragma unroll
  for (int q = 0; q < kThreshLoads; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (tid + kSelThreads * q) + e;
      const bool take = live[q] && ob[q][e] >= t32;
      const uint64_t m = __ballot(take);
      if (m == 0) continue;
      const uint64_t key =
          (static_cast<uint64_t>(ob[q][e]) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - sample_col(i, stride));
      const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&s_hits, static_cast<uint32_t>(__popcll(m)));
      base = static_cast<uint32_t>(__shfl(static_cast<int>(base), leader, 64));
      if (take && base + below < static_cast<uint32_t>(xcap)) dstore(dbg, 1, kDbgTopkWork, xrow + base + below, key);
    }
  }
  __syncthreads();
  const uint32_t nh = s_hits;
  if (tid == 0) {
    dstore(dbg, 2, kDbgTopkWork, thr + row, t);
    dstore(dbg, 3, kDbgTopkWork, xcnt + row, nh);
  }
}

struct TopkSweepParams {
  const uint16_t* h;  // the pass's first row
  const uint16_t* W;
  int64_t d, V;
  int32_t rows;
  int32_t n_vt;      // vocabulary tiles
  int32_t stride, n_sample;
  int32_t rbs, splits;
  const uint64_t* thr;
  uint32_t* cnt;     // [rows][2 * splits]: keys each slice found (may exceed slice_cap)
  uint64_t* cand;    // [rows][2 * splits][slice_cap]
  int32_t slice_cap;
  DebugCheck dbg;    // debug build: spans 0 thresholds, 1 candidate slices, 2 counts, 3 h, 4 W
};

// The u-th vocabulary tile that is not sampled (sampled: t % stride == 0 for
// t < n_sample * stride).
__device__ __forceinline__ int unsampled_tile(int u, int stride, int n_sample) {
  const int in_groups = n_sample * (stride - 1);
  if (u >= in_groups) return u + n_sample;
  return (u / (stride - 1)) * stride + 1 + u % (stride - 1);
}

// Each thread owns one row (tid & 255) of the block and one 64-column quarter
// (tid >> 8) of every half tile: it compares its 64 keys with the row's
// threshold (the logit's ordered bits first, the full key only where they
// reach the threshold's) and stores those at or above it in its own slice of
// the row's candidate list (slice 2 * split + quarter), counting them in a
// register, so no two threads ever write the same slot and no atomic is
// needed. The count (which may exceed the slice) is stored at the end.
__global__ __launch_bounds__(kBlockThreads, 1) void k_topk_sweep(TopkSweepParams P) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;
  const int wn = wave % kWN;
  int rb, split;
  grouped_tile(xcd_contiguous(blockIdx.x, P.rbs * P.splits), P.rbs, P.splits, 8, rb, split);
  const int n_u = P.n_vt - P.n_sample;
  const int u0 = static_cast<int>(static_cast<int64_t>(split) * n_u / P.splits);
  const int u1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_u / P.splits);
  const int rloc = tid & (kTile - 1);
  const int sub = tid >> 8;
  const int row = rb * kTile + rloc;
  const bool row_ok = row < P.rows;
  const uint64_t thr = row_ok ? dload(P.dbg, 0, kDbgTopkWork, P.thr + row) : ~uint64_t(0);
  const uint32_t thr_hi = static_cast<uint32_t>(thr >> 32);
  const int slices = 2 * P.splits;
  const int slice = 2 * split + sub;
  uint64_t* mine = P.cand + (static_cast<int64_t>(row_ok ? row : 0) * slices + slice) * P.slice_cap;
  const bool mine_ok = dcheck_range(P.dbg, 1, kDbgTopkWork, mine, static_cast<uint64_t>(P.slice_cap) * 8);
  uint32_t found = 0;
  const Operand A{P.h, P.d, P.rows, P.d};
  const Operand B{P.W, P.d, P.V, P.d};
  const int nk = static_cast<int>((P.d + kStageK - 1) / kStageK);
  float* stage = reinterpret_cast<float*>(lds);
  for (int u = u0; u < u1; ++u) {
    const int vt = unsampled_tile(u, P.stride, P.n_sample);
    MainAcc acc;
    zero_acc(acc);
    dcheck_operands<false, false>(P.dbg, 3, 4, A, B, static_cast<int64_t>(rb) * kTile,
                                  static_cast<int64_t>(vt) * kTile, kTile);
    gemm_mainloop<false, false, kNBW, kWN>(A, B, static_cast<int64_t>(rb) * kTile, static_cast<int64_t>(vt) * kTile,
                                           nk, acc, lds);
    for (int half = 0; half < 2; ++half) {
      if ((wn >> 1) == half) stage_half_tile(acc, stage, wm, wn, lane);
      __syncthreads();
      const int cs = vt * kTile + half * 128 + sub * 64;
      const int nvalid = row_ok ? static_cast<int>(min<int64_t>(64, P.V - cs)) : 0;
      const float* sr = stage + rloc * kStageLd + sub * 64;
      for (int e0 = 0; e0 < nvalid; e0 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(sr + e0);
        const uint32_t o0 = ordered_bits(x[0]), o1 = ordered_bits(x[1]);
        const uint32_t o2 = ordered_bits(x[2]), o3 = ordered_bits(x[3]);
        if (max(max(o0, o1), max(o2, o3)) < thr_hi) continue;  // the usual case
        const uint32_t ob[4] = {o0, o1, o2, o3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t key = (static_cast<uint64_t>(ob[e]) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - (cs + e0 + e));
          if (e0 + e < nvalid && key >= thr) {
            if (found < static_cast<uint32_t>(P.slice_cap) && mine_ok) mine[found] = key;
            ++found;
          }
        }
      }
      __syncthreads();
    }
  }
  if (row_ok) dstore(P.dbg, 2, kDbgTopkWork, P.cnt + static_cast<int64_t>(row) * slices + slice, found);
}

// One workgroup per row: the top K among the row's candidates (its 2 * splits
// slices from the sweep and the extra slice of sampled keys from the
// threshold). When fewer than K keys reached the threshold, or a slice
// overflowed (keys were dropped), the row cannot be answered here: the pass's
// redo flag is set and nothing is written.
constexpr int kMaxSlices = 2 * kTargetBlocks;
static_assert(kMaxSlices % kSelThreads == 0, "each thread owns the same number of slice offsets");
constexpr int kPickBatch = 6;  // slot loads issued before any is used
// Two instantiations differ only in LDS room: CandCap candidates gathered
// into LDS (a row with more is selected in place, over its slots) and KeysCap
// output keys (at least Kp). For K <= 128 about 1024 candidates are targeted:
// 1536 slots and 128 keys take 16 KiB, so that eight rows' workgroups share a
// CU; larger K takes 3072 and 1024 (36 KiB, four per CU).
constexpr int kPickCandSmall = 1536;
constexpr int kPickKeysSmall = 128;
constexpr int kPickCandLarge = 3072;

template <int CandCap, int KeysCap>
__global__ __launch_bounds__(kSelThreads) void k_topk_pick(const uint32_t* __restrict__ xcnt,
                                                           const uint64_t* __restrict__ xcand, int xcap,
                                                           const uint32_t* __restrict__ cnt,
                                                           const uint64_t* __restrict__ cand_g, int slices,
                                                           int slice_cap, int K, int Kp, int64_t r0,
                                                           uint32_t* flag, int32_t* __restrict__ t_idx,
                                                           float* __restrict__ t_logit, DebugCheck dbg) {
  // dbg spans: 0 extra-slice counts, 1 extra slices, 2 slice counts, 3 candidate slices, 4 t_idx, 5 t_logit
  __shared__ uint32_t hist[1 << kFusedDigitBits];
  static_assert(KeysCap <= kMaxK && (KeysCap <= 128 || KeysCap == kMaxK), "the block sort needs room for Kp");
  __shared__ uint64_t keys[KeysCap];
  __shared__ uint64_t cand[CandCap];
  __shared__ uint32_t s_cnt[kMaxSlices];
  __shared__ uint32_t s_off[kMaxSlices];
  __shared__ uint32_t wave_tot[kSelThreads / 64];
  __shared__ uint64_t s_and[kSelThreads / 64], s_or[kSelThreads / 64];
  __shared__ uint32_t s_vals[3];
  __shared__ uint32_t s_fill, s_over;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const uint32_t* crow = cnt + static_cast<int64_t>(row) * slices;
  const uint64_t* cg = cand_g + static_cast<int64_t>(row) * slices * slice_cap;
  const uint64_t* xg = xcand + static_cast<int64_t>(row) * xcap;
  if (!dcheck_range(dbg, 1, kDbgTopkWork, xg, static_cast<uint64_t>(xcap) * 8) ||
      !dcheck_range(dbg, 2, kDbgTopkWork, crow, static_cast<uint64_t>(slices) * 4) ||
      !dcheck_range(dbg, 3, kDbgTopkWork, cg, static_cast<uint64_t>(slices) * slice_cap * 8))
    return;
  const uint32_t nx = dload(dbg, 0, kDbgTopkWork, xcnt + row);
  for (int i = tid; i < Kp; i += kSelThreads) keys[i] = 0;
  if (tid == 0) {
    s_fill = 0;
    s_over = 0;
  }
  uint32_t n_part = 0;
  bool over = false;
  for (int s = tid; s < slices; s += kSelThreads) {
    const uint32_t c = crow[s];
    s_cnt[s] = c;
    over |= c > static_cast<uint32_t>(slice_cap);
    n_part += c;
  }
  for (int o = 32; o > 0; o >>= 1) n_part += static_cast<uint32_t>(__shfl_xor(static_cast<int>(n_part), o, 64));
  if ((tid & 63) == 0) wave_tot[tid >> 6] = n_part;
  __syncthreads();
  if (over || (tid == 0 && nx > static_cast<uint32_t>(xcap))) s_over = 1;
  __syncthreads();
  uint32_t n = nx;
  for (int w = 0; w < kSelThreads / 64; ++w) n += wave_tot[w];
  const bool overflow = s_over != 0;
  __syncthreads();  // wave_tot is reused by the selection
  if (overflow || n < static_cast<uint32_t>(K)) {
    if (tid == 0) *flag = 1;
    return;
  }
  // every used slot of every slice, in slot order; unused slots read as 0
  const int list = slices * slice_cap;
  SelectState st{0, 0, static_cast<uint32_t>(K)};
  if (n <= static_cast<uint32_t>(CandCap)) {
    // Candidate t of the sweep's slices goes to cand[t]: an exclusive prefix
    // sum of the slice counts (thread t owns slices kOffPer t ..) places each
    // slice's used slots, so only those are loaded, in one batch per thread
    // for the usual count, and no atomics are needed.
    constexpr int kOffPer = kMaxSlices / kSelThreads;
    uint32_t c[kOffPer];
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < kOffPer; ++e) {
      const int sl = tid * kOffPer + e;
      c[e] = sl < slices ? s_cnt[sl] : 0u;
      mine += c[e];
    }
    const int lane = tid & 63;
    const int wv = tid >> 6;
    uint32_t incl = mine;  // this thread's slices and those of the earlier lanes of its wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), o, 64));
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    uint32_t before = incl - mine;
    for (int w2 = 0; w2 < wv; ++w2) before += wave_tot[w2];
#pragma unroll
    for (int e = 0; e < kOffPer; ++e) {
      const int sl = tid * kOffPer + e;
      if (sl < slices) s_off[sl] = before;
      before += c[e];
    }
    __syncthreads();
    const uint32_t np = n - nx;  // candidates in the sweep's slices
    for (uint32_t t0 = 0; t0 < np; t0 += kSelThreads * kPickBatch) {
      int64_t slot[kPickBatch];
#pragma unroll
      for (int b = 0; b < kPickBatch; ++b) {
        const uint32_t t = t0 + b * kSelThreads + tid;
        slot[b] = -1;
        if (t < np) {
          // the last slice whose first candidate is at or before t (it is
          // not empty: the next slice starts after t)
          int lo = 0, hi = slices - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= t) lo = mid;
            else hi = mid - 1;
          }
          slot[b] = static_cast<int64_t>(lo) * slice_cap + (t - s_off[lo]);
        }
      }
      uint64_t k[kPickBatch];
#pragma unroll
      for (int b = 0; b < kPickBatch; ++b) k[b] = slot[b] >= 0 ? cg[slot[b]] : 0;
#pragma unroll
      for (int b = 0; b < kPickBatch; ++b) {
        const uint32_t t = t0 + b * kSelThreads + tid;
        if (t < np) cand[t] = k[b];
      }
    }
    for (uint32_t t = tid; t < nx; t += kSelThreads) cand[np + t] = xg[t];
    __syncthreads();
    // The candidates all lie at or above the threshold, so their leading bits
    // (the logit's sign, exponent and first mantissa bits) are mostly shared:
    // the digits every candidate has in common are fixed up front instead of
    // being selected one histogram at a time over a single crowded bin.
    uint64_t all_and = ~uint64_t(0), all_or = 0;
    for (uint32_t i = tid; i < n; i += kSelThreads) {
      all_and &= cand[i];
      all_or |= cand[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      all_and &= shfl_xor_u64(all_and, o);
      all_or |= shfl_xor_u64(all_or, o);
    }
    if ((tid & 63) == 0) {
      s_and[tid >> 6] = all_and;
      s_or[tid >> 6] = all_or;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      all_and &= s_and[w];
      all_or |= s_or[w];
    }
    const uint64_t differ = all_and ^ all_or;
    // length of the common prefix (keys are distinct, so it is shorter than
    // 64 bits whenever n > 1); the next digit starts at the first bit that
    // differs
    const int common = differ == 0 ? 64 : __clzll(static_cast<long long>(differ));
    if (common > 0) {
      st.pbits = common;
      st.prefix = common >= 64 ? all_and : all_and >> (64 - common);
    }
    const uint64_t* cp = cand;
    auto cand_key = [cp](int i) { return cp[i]; };
    select_rest<kFusedDigitBits>(cand_key, static_cast<int>(n), st, hist, wave_tot, s_vals);
    for (uint32_t i = tid; i < n; i += kSelThreads) {
      const uint64_t key = cand[i];
      if ((key >> (64 - st.pbits)) >= st.prefix) {
        const uint32_t slot = atomicAdd(&s_fill, 1u);
        if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
      }
    }
  } else {
    // More candidates than LDS holds (large K): select in place over every
    // slot of every slice and the extra slice; unused slots count as 0 (at
    // least K keys are larger, so they never reach the top K).
    const uint32_t* sc = s_cnt;
    auto key_at = [cg, sc, slice_cap, list, xg, nx](int i) -> uint64_t {
      if (i < list) {
        const int sl = i / slice_cap;
        return static_cast<uint32_t>(i - sl * slice_cap) < sc[sl] ? cg[i] : 0;
      }
      return static_cast<uint32_t>(i - list) < nx ? xg[i - list] : 0;
    };
    const int total = list + static_cast<int>(nx);
    select_rest<kFusedDigitBits>(key_at, total, st, hist, wave_tot, s_vals);
    for (int i = tid; i < total; i += kSelThreads) {
      const uint64_t key = key_at(i);
      if (key != 0 && (key >> (64 - st.pbits)) >= st.prefix) {
        const uint32_t slot = atomicAdd(&s_fill, 1u);
        if (slot < static_cast<uint32_t>(K)) keys[slot] = key;
      }
    }
  }
  __syncthreads();
  sort_and_write(keys, K, Kp, r0 + row, t_idx, t_logit, dbg);
}

// ---------------------------------------------------------------------------
// Launch sequence
// ---------------------------------------------------------------------------

// The materialised route for rows [c0, c0 + rows), in blocks of block_rows rows
// (run_if: NULL, or the redo flag the kernels test before doing anything).
// Extents for the debug build's checks: the call's control word and buffers.
struct TopkSpans {
  uint32_t* word;
  HostSpan h, W, t_idx, t_logit, z;
};

static void launch_materialised(const TopkPlan& p, const uint16_t* h, const uint16_t* W, int32_t* t_idx,
                                float* t_logit, float* z, int64_t c0, int64_t rows, int64_t block_rows, int Kp,
                                const uint32_t* run_if, const TopkSpans& sp, hipStream_t st) {
  for (int64_t b0 = c0; b0 < c0 + rows; b0 += block_rows) {
    const int brows = static_cast<int>(c0 + rows - b0 < block_rows ? c0 + rows - b0 : block_rows);
    GemmAccParams g;
    g.A = Operand{h + b0 * p.d, p.d, brows, p.d};
    g.B = Operand{W, p.d, p.V, p.d};
    g.nk = static_cast<int32_t>(ceil_div(p.d, kStageK));
    g.C = z;
    g.ldc = p.ld;
    g.m_lim = brows;
    g.n_lim = p.V;
    g.beta = 0;
    g.mblocks = static_cast<int32_t>(ceil_div(brows, kTile));
    g.nblocks = static_cast<int32_t>(ceil_div(p.V, kTile));
    g.splits = 1;
    g.kper = g.nk;
    g.c_split = 0;
    g.dbg = make_debug_check(sp.word, {sp.z, sp.h, sp.W});
    {
      TraceScope ts(st, "topk_logits", 2.0 * brows * static_cast<double>(p.V) * p.d,
                    2.0 * brows * p.d + 2.0 * p.V * p.d + 4.0 * brows * p.V);
      hipLaunchKernelGGL(k_topk_logits, dim3(g.mblocks * g.nblocks), dim3(kBlockThreads), 0, st, g, run_if);
    }
    {
      TraceScope ts(st, "topk_select", 0.0, 2.0 * 4.0 * brows * p.V + 8.0 * brows * p.K);
      hipLaunchKernelGGL(k_topk_select, dim3(brows), dim3(kSelThreads), 0, st, z, p.ld, static_cast<int>(p.V), p.K,
                         Kp, b0, static_cast<int>((p.flags & FKL_TOPK_DIRECT) != 0), run_if, t_idx, t_logit,
                         make_debug_check(sp.word, {sp.z, {}, {}, {}, sp.t_idx, sp.t_logit}));
    }
  }
}

hipError_t launch_topk(const TopkPlan& p, const uint16_t* h, const uint16_t* W, int32_t* t_idx, float* t_logit,
                       char* ws, hipStream_t st) {
  int Kp = 1;
  while (Kp < p.K) Kp <<= 1;
  float* z = reinterpret_cast<float*>(ws + p.off_region);
  const uint64_t out_bytes = static_cast<uint64_t>(p.N) * p.K * 4;
  const TopkSpans sp{reinterpret_cast<uint32_t*>(ws + p.off_flag + kDebugWordOffset),
                     {h, static_cast<uint64_t>(p.N) * p.d * 2},
                     {W, static_cast<uint64_t>(p.V) * p.d * 2},
                     {t_idx, out_bytes},
                     {t_logit, out_bytes},
                     {z, static_cast<uint64_t>(round_up(p.fused ? p.redo_rows : p.fb_rows, kTile)) * p.ld * 4}};
  if (!p.fused) {
    for (int64_t c0 = 0; c0 < p.N; c0 += p.chunk) {
      const int64_t rows = p.N - c0 < p.chunk ? p.N - c0 : p.chunk;
      launch_materialised(p, h, W, t_idx, t_logit, z, c0, rows, p.fb_rows, Kp, nullptr, sp, st);
    }
    return hipGetLastError();
  }
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws + p.off_flag);
  uint16_t* Ws = reinterpret_cast<uint16_t*>(ws + p.off_ws);
  float* sample = reinterpret_cast<float*>(ws + p.off_sample);
  uint64_t* thr = reinterpret_cast<uint64_t*>(ws + p.off_thr);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + p.off_cnt);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + p.off_cand);
  uint32_t* xcnt = reinterpret_cast<uint32_t*>(ws + p.off_xcnt);
  uint64_t* xcand = reinterpret_cast<uint64_t*>(ws + p.off_xcand);
  const int S = p.n_sample * kTile;
  const int n_vt = static_cast<int>(ceil_div(p.V, kTile));
  const uint64_t chunk_alloc = static_cast<uint64_t>(round_up(p.chunk, kTile));
  const HostSpan ws_span{Ws, static_cast<uint64_t>(S) * p.d * 2};
  const HostSpan sample_span{sample, chunk_alloc * S * 4};
  const HostSpan thr_span{thr, chunk_alloc * 8};
  const HostSpan cnt_span{cnt, p.off_cand - p.off_cnt};
  const HostSpan cand_span{cand, p.off_xcnt - p.off_cand};
  const HostSpan xcnt_span{xcnt, chunk_alloc * 4};
  const HostSpan xcand_span{xcand, chunk_alloc * p.xcap * 8};
  if (p.n_sample > 0) {
    const int64_t q = static_cast<int64_t>(S) * (p.d / 8);
    const int64_t grid = ceil_div(q, 256) < 4096 ? ceil_div(q, 256) : 4096;
    TraceScope ts(st, "topk_gather", 0.0, 4.0 * S * p.d);
    hipLaunchKernelGGL(k_gather_tiles, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, W, p.d, p.stride,
                       p.n_sample, Ws, make_debug_check(sp.word, {ws_span, sp.W}));
  }
  for (int64_t c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int rows = static_cast<int>(p.N - c0 < p.chunk ? p.N - c0 : p.chunk);
    const int rbs = static_cast<int>(ceil_div(rows, kTile));
    if (p.n_sample > 0) {
      GemmAccParams g;
      g.A = Operand{h + c0 * p.d, p.d, rows, p.d};
      g.B = Operand{Ws, p.d, S, p.d};
      g.nk = static_cast<int32_t>(ceil_div(p.d, kStageK));
      g.C = sample;
      g.ldc = S;
      g.m_lim = rows;
      g.n_lim = S;
      g.beta = 0;
      g.mblocks = rbs;
      g.nblocks = p.n_sample;
      g.splits = 1;
      g.kper = g.nk;
      g.c_split = 0;
      g.dbg = make_debug_check(sp.word, {sample_span, sp.h, ws_span});
      TraceScope ts(st, "topk_sample", 2.0 * rows * static_cast<double>(S) * p.d,
                    2.0 * rows * p.d + 2.0 * S * p.d + 4.0 * rows * S);
      hipLaunchKernelGGL(k_topk_logits, dim3(g.mblocks * g.nblocks), dim3(kBlockThreads), 0, st, g,
                         static_cast<const uint32_t*>(nullptr));
    }
    {
      TraceScope ts(st, "topk_thresh", 0.0, 4.0 * rows * S + 8.0 * rows);
      hipLaunchKernelGGL(k_topk_thresh, dim3(rows), dim3(kSelThreads), 0, st, sample, S, p.stride, p.j, thr, xcnt,
                         xcand, p.xcap, flag,
                         make_debug_check(sp.word, {sample_span, xcand_span, thr_span, xcnt_span}));
    }
    const int splits = topk_splits(p, rows);
    const int slice_cap = topk_slice_cap(p, splits);
    {
      TopkSweepParams swp{h + c0 * p.d, W, p.d, p.V, rows, n_vt, p.stride, p.n_sample, rbs, splits, thr, cnt,
                          cand, slice_cap, make_debug_check(sp.word, {thr_span, cand_span, cnt_span, sp.h, sp.W})};
      const double cols = static_cast<double>(p.V) - S;
      TraceScope ts(st, "topk_sweep", 2.0 * rows * cols * p.d, 2.0 * rows * p.d + 2.0 * cols * p.d);
      // launched even when every tile is sampled: its workgroups then store zero counts
      hipLaunchKernelGGL(k_topk_sweep, dim3(rbs * splits), dim3(kBlockThreads), 0, st, swp);
    }
    {
      TraceScope ts(st, "topk_pick", 0.0, 4.0 * rows * S + 8.0 * rows * p.K);
      auto* pick = Kp <= kPickKeysSmall ? k_topk_pick<kPickCandSmall, kPickKeysSmall>
                                        : k_topk_pick<kPickCandLarge, kMaxK>;
      hipLaunchKernelGGL(pick, dim3(rows), dim3(kSelThreads), 0, st, xcnt, xcand, p.xcap, cnt, cand, 2 * splits,
                         slice_cap, p.K, Kp, c0, flag, t_idx, t_logit,
                         make_debug_check(sp.word, {xcnt_span, xcand_span, cnt_span, cand_span, sp.t_idx, sp.t_logit}));
    }
    // redo of the pass by the materialised route, only if a row flagged it
    launch_materialised(p, h, W, t_idx, t_logit, z, c0, rows, p.redo_rows, Kp, flag, sp, st);
  }
  return hipGetLastError();
}

}  // namespace fkl
