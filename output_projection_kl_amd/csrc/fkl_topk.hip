// Offline teacher-cache builder: per row of h, the K largest logits of
// h W^T with their vocabulary indices (blog post on the page "Efficient
// Offline Top-K Logits and Fused Chunked KL Loss Enable Scalable LLM
// Distillation", section "Two systems changes": the teacher's top-100
// logits per position are cached once, offline, and nothing else of its
// distribution is kept).
//
// Per chunk of rows:
//   k_topk_logits  256 x 256 MFMA tiles of z = h_chunk W^T (fp32 accumulation)
//                  written to an fp32 logits block in the workspace
//   k_topk_select  one workgroup per row: exact radix selection of the K
//                  largest keys, then a bitonic sort in LDS
//
// Keys make every element distinct: key = (order-preserving bits of z) << 32
// | (0xFFFFFFFF - index), so larger keys are larger logits and, for equal
// logits, lower indices. Selection by 12-bit radix digits of the key from the
// top, keeping only the keys that share the digits chosen so far, until the
// digit bin at the K-th key is taken whole.
//
// Each row is read once in the usual case: a threshold key is taken from a
// sample of the row (runs of contiguous logits spread over it) such that a
// bounded number of keys, at least K and at most half the LDS buffer, is
// expected at or above it; one pass collects those keys into LDS, and the
// selection runs there. A threshold that keeps fewer than K keys or more than
// the buffer holds is moved and the row read again; after three tries the row
// is selected directly: a histogram pass over the row, a pass that takes the
// keys above the boundary bin and copies the bin to LDS, the rest in LDS (or
// over the row when the bin does not fit). Both routes select the same K keys.
#include <climits>

#include "fkl_device.h"
#include "fkl_internal.h"
#include "fkl_tiles.h"

namespace fkl {

__global__ __launch_bounds__(kBlockThreads, 1) void k_topk_logits(GemmAccParams P) {
  __shared__ __align__(16) char lds[kKernelLdsBytes];
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

// One digit of the selection over n keys given by key_at(i): histogram of the
// next digit among keys matching the prefix, then the digit holding the
// need-th largest key. Returns the number of keys in that digit's bin.
template <class KeyAt>
__device__ uint32_t select_digit(KeyAt key_at, int n, SelectState& st, uint32_t* hist, uint32_t* wave_tot,
                                 uint32_t* s_vals) {
  const int tid = threadIdx.x;
  const int w = 64 - st.pbits < kDigitBits ? 64 - st.pbits : kDigitBits;
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
// 64 bits are fixed: keys are distinct).
template <class KeyAt>
__device__ void select_rest(KeyAt key_at, int n, SelectState& st, uint32_t* hist, uint32_t* wave_tot,
                            uint32_t* s_vals) {
  while (st.pbits < 64) {
    if (select_digit(key_at, n, st, hist, wave_tot, s_vals) == st.need) break;
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

__global__ __launch_bounds__(kSelThreads) void k_topk_select(const float* __restrict__ logits, int64_t ld,
                                                             int V, int K, int Kp, int64_t r0, int direct,
                                                             int32_t* __restrict__ t_idx,
                                                             float* __restrict__ t_logit) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t keys[kMaxK];
  __shared__ uint64_t cand[kCand];
  __shared__ uint32_t wave_tot[kSelThreads / 64];
  __shared__ uint32_t s_vals[3];
  __shared__ uint32_t s_fill, s_cand;
  const int tid = threadIdx.x;
  const float* row = logits + static_cast<int64_t>(blockIdx.x) * ld;

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
  // Bitonic sort of Kp keys, descending.
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
  const int64_t out = (r0 + blockIdx.x) * static_cast<int64_t>(K);
  for (int k = tid; k < K; k += kSelThreads) {
    const uint64_t key = keys[k];
    t_logit[out + k] = from_ordered_bits(static_cast<uint32_t>(key >> 32));
    t_idx[out + k] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
  }
}

hipError_t launch_topk(const TopkPlan& p, const uint16_t* h, const uint16_t* W, int32_t* t_idx, float* t_logit,
                       char* ws, hipStream_t st) {
  float* z = reinterpret_cast<float*>(ws);
  int Kp = 1;
  while (Kp < p.K) Kp <<= 1;
  for (int64_t c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int rows = static_cast<int>(p.N - c0 < p.chunk ? p.N - c0 : p.chunk);
    GemmAccParams g;
    g.A = Operand{h + c0 * p.d, p.d, rows, p.d};
    g.B = Operand{W, p.d, p.V, p.d};
    g.nk = static_cast<int32_t>(ceil_div(p.d, kStageK));
    g.C = z;
    g.ldc = p.ld;
    g.m_lim = rows;
    g.n_lim = p.V;
    g.beta = 0;
    g.mblocks = static_cast<int32_t>(ceil_div(rows, kTile));
    g.nblocks = static_cast<int32_t>(ceil_div(p.V, kTile));
    g.splits = 1;
    g.kper = g.nk;
    g.c_split = 0;
    {
      TraceScope ts(st, "topk_logits", 2.0 * rows * static_cast<double>(p.V) * p.d,
                    2.0 * rows * p.d + 2.0 * p.V * p.d + 4.0 * rows * p.V);
      hipLaunchKernelGGL(k_topk_logits, dim3(g.mblocks * g.nblocks), dim3(kBlockThreads), 0, st, g);
    }
    {
      TraceScope ts(st, "topk_select", 0.0, 2.0 * 4.0 * rows * p.V + 8.0 * rows * p.K);
      hipLaunchKernelGGL(k_topk_select, dim3(rows), dim3(kSelThreads), 0, st, z, p.ld, static_cast<int>(p.V),
                         p.K, Kp, c0, static_cast<int>((p.flags & FKL_TOPK_DIRECT) != 0), t_idx, t_logit);
    }
  }
  return hipGetLastError();
}

}  // namespace fkl
