// Host-only check of libfkl's C-ABI layer (csrc/fkl_api.cpp), built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer, no GPU and no HIP
// runtime. The kernel launchers and the three HIP runtime calls the layer
// makes are replaced by stubs: a launcher stub checks the plan it is handed
// (every workspace region inside the caller's workspace, 256-byte aligned and
// disjoint where the kernels need it; every operand view the kernels address
// through a 32-bit buffer descriptor under 2 GiB; the forward's split
// partials and the backward's grad_h partial sums inside their regions), and
// a HIP stub aborts if it is ever reached. main() drives every entry point
// over edge shapes and a seeded random sweep; any sanitizer report, failed
// check or unexpected status ends the program with a non-zero exit code.
#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fkl.h"
#include "fkl_internal.h"

namespace {

int g_fail = 0;
long g_launches = 0;

#define CHECK(cond)                                                                 \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);       \
      ++g_fail;                                                                     \
    }                                                                               \
  } while (0)

constexpr int64_t kMaxView = (int64_t(1) << 31) - 1;

bool al256(size_t x) { return (x & 255) == 0; }

// Vocabulary splits of the forward and backward logits launches (the
// launcher's rule: enough workgroups for every CU, no more than the tiles).
int64_t splits_for(int64_t rbs, int64_t tiles) {
  int64_t s = fkl::ceil_div(fkl::kTargetBlocks, rbs);
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  return s;
}

void check_shared(const fkl::Plan& p) {
  CHECK(p.off_scalars == 0);
  CHECK(p.off_negent >= 256 && al256(p.off_negent));
  // the lists serve the longer of the forward and backward passes
  CHECK(p.list_rows >= p.chunk_alloc && p.list_rows >= p.bchunk_alloc);
  CHECK(al256(p.off_tidx) && p.off_tidx >= p.off_negent + static_cast<size_t>(p.list_rows) * 4);
  CHECK(al256(p.off_tp) && p.off_tp >= p.off_tidx + static_cast<size_t>(p.list_rows) * (p.K + 1) * 4);
  // the forward's passes are at least as long as the backward's; they differ
  // only where the forward's floor raised its rows
  CHECK(p.bchunk >= 1 && p.chunk >= p.bchunk);
  if (p.chunk != p.bchunk) CHECK(p.chunk <= fkl::kFwdPassRows && p.chunk <= p.N);
  CHECK(p.chunk_alloc % fkl::kTile == 0 && p.chunk_alloc >= p.chunk && p.chunk_alloc - p.chunk < fkl::kTile);
  CHECK(p.bchunk_alloc % fkl::kTile == 0 && p.bchunk_alloc >= p.bchunk);
  CHECK(p.vslab % fkl::kTile == 0 && p.vslab >= fkl::kTile && p.vslab <= fkl::round_up(p.V, fkl::kTile));
  CHECK(p.n_vt == fkl::ceil_div(p.V, fkl::kTile));
  // operand views addressed through 32-bit buffer descriptors
  CHECK(p.list_rows * p.d * 2 <= kMaxView);
  CHECK(p.vslab * p.d * 2 <= kMaxView);
  CHECK(p.bchunk_alloc * p.vslab * 2 <= kMaxView);
}

void check_forward(const fkl::Plan& p, size_t ws_bytes) {
  check_shared(p);
  CHECK(p.fwd_bytes <= ws_bytes);
  const size_t tp_end = p.off_tp + static_cast<size_t>(p.list_rows) * (p.K + 1) * 4;
  CHECK(p.off_partial >= tp_end && al256(p.off_partial));
  const int64_t rbs_max = p.chunk_alloc / fkl::kTile;
  CHECK(p.off_blocksum >=
        p.off_partial + static_cast<size_t>(fkl::kTargetBlocks + rbs_max) * 2 * fkl::kTile * 16);
  CHECK(p.fwd_bytes >= p.off_blocksum + static_cast<size_t>(p.chunk_alloc / fkl::kCombineRows) * 8);
  // full passes are alike; the last one may be shorter
  for (int64_t c0 : {int64_t(0), (fkl::ceil_div(p.N, p.chunk) - 1) * p.chunk}) {
    if (p.N <= 0) break;
    const int64_t rows = p.N - c0 < p.chunk ? p.N - c0 : p.chunk;
    const int64_t rbs = fkl::ceil_div(rows, fkl::kTile);
    const int64_t splits = splits_for(rbs, p.n_vt);
    // partial[(split * 2 + sub) * ld + row], ld = rbs * 256
    const int64_t last = ((splits - 1) * 2 + 1) * rbs * fkl::kTile + rbs * fkl::kTile - 1;
    CHECK(p.off_partial + static_cast<size_t>(last + 1) * 16 <= p.off_blocksum);
    CHECK(static_cast<size_t>(fkl::ceil_div(rows, fkl::kCombineRows)) * 8 + p.off_blocksum <= p.fwd_bytes);
  }
}

void check_backward(const fkl::Plan& p, size_t ws_bytes) {
  check_shared(p);
  CHECK(p.bwd_bytes <= ws_bytes);
  const size_t tp_end = p.off_tp + static_cast<size_t>(p.list_rows) * (p.K + 1) * 4;
  CHECK(p.off_G >= tp_end && al256(p.off_G));
  CHECK(p.off_ghp >= p.off_G + static_cast<size_t>(p.bchunk_alloc) * p.vslab * 2 && al256(p.off_ghp));
  CHECK(p.off_gh32 >= p.off_ghp + static_cast<size_t>(p.ghp_rows) * p.d * 4 && al256(p.off_gh32));
  const bool bf16_h = (p.flags & FKL_GRAD_H_BF16) && !(p.flags & FKL_SKIP_GRAD_H);
  CHECK(p.bwd_bytes >= p.off_gh32 + (bf16_h ? static_cast<size_t>(p.bchunk_alloc) * p.d * 4 : 0));
  const int64_t n_slabs = fkl::ceil_div(p.V, p.vslab);
  for (int64_t c0 : {int64_t(0), (fkl::ceil_div(p.N, p.bchunk) - 1) * p.bchunk}) {
    if (p.N <= 0) break;
    const int64_t rows = p.N - c0 < p.bchunk ? p.N - c0 : p.bchunk;
    const int64_t rows_written = fkl::ceil_div(rows, fkl::kTile) * fkl::kTile;
    CHECK(rows_written <= p.bchunk_alloc);
    for (int64_t s : {int64_t(0), n_slabs - 1}) {
      const int64_t slab_w = p.V - s * p.vslab < p.vslab ? p.V - s * p.vslab : p.vslab;
      CHECK(slab_w >= 1 && slab_w <= p.vslab);
      // the launcher caps a grad_h split to the partial-sum rows the plan holds
      int hs = (p.flags & FKL_SKIP_GRAD_H) ? 1 : fkl::grad_h_splits(rows, slab_w, p.d);
      if (hs > 1 && hs * rows_written > p.ghp_rows) hs = static_cast<int>(p.ghp_rows / rows_written);
      if (hs < 1) hs = 1;
      if (hs > 1) CHECK(hs * rows_written <= p.ghp_rows);
    }
  }
}

}  // namespace

// ---- stubs of the kernel launchers (csrc/fkl_kernels.hip, csrc/fkl_topk.hip) ----
namespace fkl {

size_t g_ws_bytes = 0;  // workspace size of the call under test

hipError_t launch_forward(const Plan& p, const FwdArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.h && a.W && a.t_idx && a.t_logit && a.loss && a.row_lse && a.ws);
  check_forward(p, g_ws_bytes);
  return hipSuccess;
}

hipError_t launch_backward(const Plan& p, const BwdArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.ws != nullptr);
  check_backward(p, g_ws_bytes);
  return hipSuccess;
}

hipError_t launch_topk(const TopkPlan& p, const uint16_t* h, const uint16_t* W, int32_t* ti, float* tl, char* ws,
                       hipStream_t) {
  ++g_launches;
  CHECK(h && W && ti && tl && ws);
  CHECK(p.chunk >= 1 && p.ld % kTile == 0 && p.ld >= p.V);
  CHECK(p.fb_rows >= 1 && p.fb_rows <= p.chunk);
  CHECK(p.redo_rows >= p.fb_rows && p.redo_rows <= p.chunk && (!p.fused ? p.redo_rows == p.fb_rows : true));
  CHECK(p.bytes <= g_ws_bytes);
  // the materialised route's logits block (also the fused route's redo)
  CHECK(al256(p.off_region) && p.off_region + static_cast<size_t>(round_up(p.fb_rows, kTile)) * p.ld * 4 <= p.bytes);
  CHECK(p.off_region + static_cast<size_t>(round_up(p.redo_rows, kTile)) * p.ld * 4 <= p.bytes);
  CHECK(p.off_flag + 4 <= p.off_ws && p.off_ws <= p.off_region);
  if (p.fused) {
    const int64_t S = static_cast<int64_t>(p.n_sample) * kTile;
    const size_t ca = static_cast<size_t>(round_up(p.chunk, kTile));
    CHECK(p.n_sample >= 0 && p.n_sample <= kTopkMaxSampleTiles);
    CHECK(p.stride >= kTopkMinStride);
    // every sampled tile is a full vocabulary tile
    if (p.n_sample > 0) CHECK(static_cast<int64_t>(p.n_sample - 1) * p.stride < p.V / kTile);
    CHECK(p.j >= 0 && (p.j == 0 || p.j < S));
    CHECK(p.target >= 1024 && p.target > p.K);
    // unless the target reached V (or j = 0): j >= 16, and fewer than K keys
    // at the threshold (j sampled keys among the K largest, about
    // Poisson(K S / V) of them) has probability <= kTopkMissTail, by a term
    // sum of its own here
    if (p.j > 0 && p.target < p.V) {
      CHECK(p.j >= 16);
      const double mu = double(p.K) * S / p.V;
      double tail = 0.0, term = std::exp(-mu);
      for (int64_t k = 0; k < p.j + 2000; ++k) {
        if (k >= p.j) tail += term;
        term *= mu / double(k + 1);
      }
      CHECK(tail <= kTopkMissTail * 1.000001);
    }
    CHECK(p.off_ws + static_cast<size_t>(S) * p.d * 2 <= p.off_region);
    CHECK(p.off_sample == p.off_region && p.off_sample + ca * S * 4 <= p.off_thr && al256(p.off_thr));
    CHECK(p.off_thr + ca * 8 <= p.off_cnt && al256(p.off_cnt));
    // every pass (full ones and the last) fits its count and slice regions
    for (int64_t c0 : {int64_t(0), (ceil_div(p.N, p.chunk) - 1) * p.chunk}) {
      if (p.N <= 0) break;
      const int64_t rows = p.N - c0 < p.chunk ? p.N - c0 : p.chunk;
      const int sp = topk_splits(p, rows);
      const int cap = topk_slice_cap(p, sp);
      CHECK(sp >= 1 && cap >= 16);
      CHECK(p.off_cnt + static_cast<size_t>(rows) * 2 * sp * 4 <= p.off_cand && al256(p.off_cand));
      CHECK(p.off_cand + static_cast<size_t>(rows) * 2 * sp * cap * 8 <= p.off_xcnt);
      // slice offsets are formed in 64-bit; counts and slots in 32-bit
      CHECK(static_cast<int64_t>(2 * sp) * cap < (int64_t(1) << 31));
      CHECK(2 * sp <= 2 * kTargetBlocks);
    }
    CHECK(al256(p.off_xcnt) && p.off_xcnt + ca * 4 <= p.off_xcand && al256(p.off_xcand));
    // the extra slice holds all S sampled keys, or at least 2j of them
    CHECK(p.xcap >= 0 && p.xcap <= S && (p.j == 0 ? p.xcap == S : p.xcap >= std::min<int64_t>(S, 2 * p.j)));
    CHECK(p.off_xcand + ca * p.xcap * 8 <= p.bytes);
    // sweep tiles: the unsampled ones, each addressed in 32-bit tile units
    CHECK(ceil_div(p.V, kTile) - p.n_sample >= 0);
  }
  // both builder operands are plain: each view covers one 256-row block
  CHECK(kTile * p.d * 2 <= kMaxView);
  CHECK(p.chunk <= INT32_MAX);
  return hipSuccess;
}

hipError_t static_scratch(hipStream_t, char** ptr) {
  *ptr = reinterpret_cast<char*>(uintptr_t(0x40000000));
  g_ws_bytes = kStaticScratchBytes;
  return hipSuccess;
}

hipError_t launch_validate(int64_t, int64_t, int32_t, const int32_t*, const float*, int32_t* bad, hipStream_t) {
  ++g_launches;
  CHECK(bad != nullptr);
  return hipSuccess;
}

hipError_t launch_validate_terms(int64_t, int64_t, const float*, const int32_t*, int32_t* bad, bool, hipStream_t) {
  ++g_launches;
  CHECK(bad != nullptr);
  return hipSuccess;
}

}  // namespace fkl

// ---- HIP runtime stubs: the layer reaches them only under FKL_VALIDATE=1 ----
extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  std::fprintf(stderr, "unexpected hipMemcpyAsync\n");
  std::abort();
}
hipError_t hipStreamSynchronize(hipStream_t) {
  std::fprintf(stderr, "unexpected hipStreamSynchronize\n");
  std::abort();
}
}

namespace {

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}
int64_t pick(const std::vector<int64_t>& v) { return v[next() % v.size()]; }

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

// One shape through every entry point: sizing, the plan, the error paths that
// must return before any launch, and (when the shape is valid) the launches.
void drive(const fkl_shape& s) {
  size_t fb = 0, bb = 0;
  const fkl_status st = fkl_workspace_size(&s, &fb, &bb);
  fkl_plan pl;
  const fkl_status st2 = fkl_plan_info(&s, &pl);
  CHECK(st == st2);
  if (st != FKL_OK) {
    CHECK(st == FKL_EINVAL || st == FKL_EUNSUPPORTED);
    CHECK(fkl_last_error()[0] != '\0');
    return;
  }
  CHECK(pl.fwd_bytes == fb && pl.bwd_bytes == bb);
  CHECK(pl.slabs * pl.vslab >= s.V && (pl.slabs - 1) * pl.vslab < s.V);
  if (s.N > 0) CHECK(pl.fwd_passes * pl.fwd_rows >= s.N && (pl.fwd_passes - 1) * pl.fwd_rows < s.N);
  fkl::Plan p;
  CHECK(fkl::make_plan(&s, &p) == FKL_OK);
  check_shared(p);
  void* h = fake(0x100000);
  void* W = fake(0x200000);
  const int32_t* ti = static_cast<const int32_t*>(fake(0x300000));
  const float* tl = static_cast<const float*>(fake(0x400000));
  float* out = static_cast<float*>(fake(0x500000));
  void* ws = fake(0x600000);
  const long before = g_launches;
  // errors that must come back before any launch
  CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, nullptr, nullptr, out, nullptr, ws, fb, nullptr) == FKL_EINVAL);
  CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, nullptr, out, out, nullptr, fake(0x600010), fb, nullptr) ==
        FKL_EWORKSPACE);
  if (fb > 0)
    CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, nullptr, out, out, nullptr, ws, fb - 1, nullptr) ==
          FKL_EWORKSPACE);
  if (s.N > 0) {
    CHECK(fkl_forward(&s, fake(0x100008), W, ti, tl, nullptr, nullptr, out, out, nullptr, ws, fb, nullptr) ==
          FKL_EINVAL);
    CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, nullptr, out, nullptr, nullptr, ws, fb, nullptr) == FKL_EINVAL);
  }
  if (!(s.flags & FKL_SKIP_GRAD_W))
    CHECK(fkl_backward(&s, h, W, ti, tl, nullptr, nullptr, out, nullptr, out, nullptr, ws, bb, nullptr) ==
          FKL_EINVAL);
  if (bb > 0)
    CHECK(fkl_backward(&s, h, W, ti, tl, nullptr, nullptr, out, nullptr, out, out, ws, bb - 1, nullptr) ==
          FKL_EWORKSPACE);
  fkl_terms bad_terms{nullptr, nullptr, 2.0f};
  CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, &bad_terms, out, out, nullptr, ws, fb, nullptr) == FKL_EINVAL);
  CHECK(g_launches == before);
  // valid calls reach the (stub) launchers with the plan checked there
  fkl::g_ws_bytes = fb;
  CHECK(fkl_forward(&s, h, W, ti, tl, nullptr, nullptr, out, out, out, ws, fb, nullptr) == FKL_OK);
  // the allocation-free forward: the static scratch, or FKL_EWORKSPACE when the plan needs more
  // (with the default slab it falls back to the backward's pass rows)
  size_t static_bytes = fb;
  if (fb > fkl::kStaticScratchBytes && s.vslab == 0) {
    fkl::Plan q;
    CHECK(fkl::make_plan(&s, &q, fkl::kPassRows) == FKL_OK);
    CHECK(q.fwd_bytes <= fb && q.bchunk == p.bchunk);
    check_shared(q);
    static_bytes = q.fwd_bytes;
  }
  const fkl_status sst = fkl_forward_static(&s, h, W, ti, tl, nullptr, nullptr, out, out, out, nullptr);
  CHECK(sst == (static_bytes <= fkl::kStaticScratchBytes ? FKL_OK : FKL_EWORKSPACE));
  CHECK(fkl_forward_static(&s, h, W, ti, tl, nullptr, nullptr, nullptr, out, out, nullptr) == FKL_EINVAL);
  fkl::g_ws_bytes = bb;
  CHECK(fkl_backward(&s, h, W, ti, tl, nullptr, nullptr, out, nullptr, out, out, ws, bb, nullptr) == FKL_OK);
  fkl_terms terms{out, static_cast<const int32_t*>(fake(0x700000)), 0.25f};
  CHECK(fkl_backward(&s, h, W, ti, tl, static_cast<const uint8_t*>(fake(0x800000)), &terms, out, out, out, out,
                     ws, bb, nullptr) == FKL_OK);
  int32_t* bad = static_cast<int32_t*>(fake(0x900000));
  CHECK(fkl_validate_teacher(&s, ti, tl, bad, nullptr) == FKL_OK);
  CHECK(fkl_validate_terms(&s, &terms, bad, nullptr) == FKL_OK);
}

void drive_topk(const fkl_topk_shape& s) {
  size_t b = 0;
  const fkl_status st = fkl_topk_workspace_size(&s, &b);
  if (st != FKL_OK) {
    CHECK(st == FKL_EINVAL || st == FKL_EUNSUPPORTED);
    return;
  }
  fkl::TopkPlan p;
  CHECK(fkl::make_topk_plan(&s, &p) == FKL_OK);
  CHECK(p.bytes == b);
  void* h = fake(0x100000);
  void* W = fake(0x200000);
  int32_t* ti = static_cast<int32_t*>(fake(0x300000));
  float* tl = static_cast<float*>(fake(0x400000));
  void* ws = fake(0x600000);
  if (s.N > 0) {
    CHECK(fkl_topk(&s, h, W, ti, tl, ws, b - 1, nullptr) == FKL_EWORKSPACE);
    CHECK(fkl_topk(&s, nullptr, W, ti, tl, ws, b, nullptr) == FKL_EINVAL);
  }
  fkl::g_ws_bytes = b;
  CHECK(fkl_topk(&s, h, W, ti, tl, ws, b, nullptr) == FKL_OK);
}

}  // namespace

int main() {
  unsetenv("FKL_VALIDATE");
  const std::vector<int64_t> Ns = {0, 1, 2, 255, 256, 257, 1000, 4095, 4096, 8191, 8192, 8193, 32768, 65536,
                                   262144, 1000003, (int64_t(1) << 31) - 1, int64_t(1) << 31, -1};
  const std::vector<int64_t> ds = {8, 16, 64, 136, 264, 2880, 3072, 4096, 65536, 65544, 0, 7, 12};
  const std::vector<int64_t> Vs = {1, 2, 100, 255, 256, 257, 4096, 5000, 128256, 201088, 1000000,
                                   (int64_t(1) << 31) - 1025, (int64_t(1) << 31) - 1024, 0};
  const std::vector<int64_t> Ks = {1, 7, 16, 100, 128, 129, 300, 700, 1024, 1025, 0};
  const std::vector<int64_t> chunks = {0, 1, 64, 100, 256, 1000, 1024, 4096, 8192, 65536,
                                       (int64_t(1) << 31) - 1, -5};
  const std::vector<int64_t> slabs = {0, 1, 256, 768, 1024, 2048, 8192, 65536, 1 << 20, (int64_t(1) << 31) - 1,
                                      -1};
  const std::vector<float> Ts = {1.0f, 2.0f, 0.5f, 0.0f, -1.0f, NAN, INFINITY};
  // edge grid over the named sizes (flags from every combination of the five bits)
  long shapes = 0;
  for (int64_t N : {int64_t(0), int64_t(1), int64_t(257), int64_t(8192), int64_t(32768), int64_t(262144)})
    for (int64_t d : {int64_t(8), int64_t(2880), int64_t(65536)})
      for (int64_t V : {int64_t(1), int64_t(257), int64_t(201088)})
        for (int64_t K : {int64_t(1), int64_t(100), int64_t(1024)})
          for (int64_t c : {int64_t(0), int64_t(1024), int64_t(4096)})
            for (int64_t vs : {int64_t(0), int64_t(256), int64_t(65536)}) {
              fkl_shape s{N, d, V, static_cast<int32_t>(K), 1.0f, static_cast<int32_t>(c),
                          static_cast<int32_t>(vs), static_cast<uint32_t>(shapes % 32)};
              drive(s);
              ++shapes;
            }
  // seeded random sweep over the wider lists, including invalid values
  for (int i = 0; i < 40000; ++i) {
    fkl_shape s{pick(Ns), pick(ds), pick(Vs), static_cast<int32_t>(pick(Ks)), Ts[next() % Ts.size()],
                static_cast<int32_t>(pick(chunks)), static_cast<int32_t>(pick(slabs)),
                static_cast<uint32_t>(next() % 40)};
    drive(s);
    ++shapes;
  }
  for (int i = 0; i < 20000; ++i) {
    fkl_topk_shape t{pick(Ns), pick(ds), pick(Vs), static_cast<int32_t>(pick(Ks)),
                     static_cast<int32_t>(pick(chunks)), static_cast<uint32_t>(next() % 5)};
    drive_topk(t);
  }
  // the allocation-free forward's fallback: 16384-row teacher lists of K = 300
  // exceed its scratch, 8192-row ones fit
  {
    const fkl_shape s{16384, 64, 5000, 300, 1.0f, 0, 0, 0};
    size_t fb = 0;
    CHECK(fkl_workspace_size(&s, &fb, nullptr) == FKL_OK && fb > fkl::kStaticScratchBytes);
    const long before = g_launches;
    drive(s);
    float* out = static_cast<float*>(fake(0x500000));
    CHECK(fkl_forward_static(&s, fake(0x100000), fake(0x200000), static_cast<const int32_t*>(fake(0x300000)),
                             static_cast<const float*>(fake(0x400000)), nullptr, nullptr, out, out, nullptr,
                             nullptr) == FKL_OK);
    CHECK(g_launches > before);
    ++shapes;
  }
  // NULL shapes and pointers
  CHECK(fkl_workspace_size(nullptr, nullptr, nullptr) == FKL_EINVAL);
  CHECK(fkl_plan_info(nullptr, nullptr) == FKL_EINVAL);
  CHECK(fkl_topk_workspace_size(nullptr, nullptr) == FKL_EINVAL);
  for (int c = -1; c < 8; ++c) CHECK(fkl_status_string(static_cast<fkl_status>(c)) != nullptr);
  std::printf("shapes %ld launches %ld failures %d\n", shapes, g_launches, g_fail);
  if (g_fail) return 1;
  std::printf("OK\n");
  return 0;
}
