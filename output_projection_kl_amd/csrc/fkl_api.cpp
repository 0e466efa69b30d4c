// C ABI of libfkl: argument checks (pure host code, no HIP call), workspace
// planning, and dispatch of the kernel sequences in fkl_kernels.hip.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "fkl.h"
#include "fkl_internal.h"

static_assert(fkl::kStaticScratchBytes == FKL_STATIC_SCRATCH_BYTES, "static scratch size differs from the header");

namespace {

thread_local std::string g_last_error;

fkl_status fail(fkl_status st, const char* msg) {
  g_last_error = msg;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Optional loss terms: NULL means none; checks what the host can check.
fkl_status read_terms(const fkl_terms* t, const float** weight, const int32_t** label, float* label_w) {
  *weight = t ? t->row_weight : nullptr;
  *label = t ? t->label : nullptr;
  *label_w = (t && t->label) ? t->label_weight : 0.0f;
  if (t && !(t->label_weight >= 0.0f && t->label_weight <= 1.0f))
    return fail(FKL_EINVAL, "label_weight must be in [0, 1]");
  if ((*weight && !aligned(*weight, 4)) || (*label && !aligned(*label, 4)))
    return fail(FKL_EINVAL, "row_weight and label must be 4-byte aligned");
  return FKL_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// With FKL_VALIDATE=1 in the environment, fkl_forward and fkl_backward first
// check the teacher lists on the device (the checks of fkl_validate_teacher)
// and refuse bad ones with FKL_EINDEX. This waits for `stream` on the host: a
// debugging aid, not for graph capture.
fkl_status validate_if_asked(const fkl::Plan& p, const int32_t* t_idx, const float* t_logit,
                             const float* weight, const int32_t* label, char* ws, hipStream_t stream) {
  const char* v = std::getenv("FKL_VALIDATE");
  if (!v || std::strcmp(v, "1") != 0 || p.N == 0) return FKL_OK;
  int32_t* bad = reinterpret_cast<int32_t*>(ws + p.off_scalars + fkl::kValidateCountOffset);
  hipError_t e = fkl::launch_validate(p.N, p.V, p.K, t_idx, t_logit, bad, stream);
  if (e == hipSuccess) e = fkl::launch_validate_terms(p.N, p.V, weight, label, bad, false, stream);
  int32_t host_bad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&host_bad, bad, sizeof(host_bad), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    g_last_error = std::string("teacher validation failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  if (host_bad > 0) {
    g_last_error = std::to_string(host_bad) +
                   " rows rejected: a teacher index outside [0, V) or repeated within the row, a"
                   " non-finite teacher logit, a hard label outside [0, V) or a non-finite weight";
    return FKL_EINDEX;
  }
  return FKL_OK;
}

}  // namespace

namespace fkl {

int grad_h_splits(int64_t rows, int64_t slab_w, int64_t d) {
  if (rows <= 0 || slab_w <= 0) return 1;
  const int64_t nb = ceil_div(d, kTile);
  const int64_t h_tiles = ceil_div(rows, kTile) * nb;
  const int64_t nk_h = ceil_div(slab_w, kContractionStep);
  const int64_t w_tiles = ceil_div(slab_w, kTile) * nb;
  const int64_t nk_w = ceil_div(rows, kContractionStep);
  const int64_t per_cu = ceil_div(h_tiles * nk_h + w_tiles * nk_w, kTargetBlocks);
  int64_t sp = ceil_div(nk_h, per_cu > 0 ? per_cu : 1);
  if (sp < 1) sp = 1;
  if (sp > kMaxGradHSplits) sp = kMaxGradHSplits;
  return static_cast<int>(sp);
}

fkl_status make_plan(const fkl_shape* s, Plan* p, int64_t fwd_floor_rows) {
  if (!s) return fail(FKL_EINVAL, "shape is NULL");
  if (s->N < 0) return fail(FKL_EINVAL, "N must be >= 0");
  if (s->N > (int64_t(1) << 31) - 1) return fail(FKL_EUNSUPPORTED, "N must be < 2^31");
  if (s->d < 8 || s->d % 8 != 0) return fail(FKL_EINVAL, "d must be a positive multiple of 8");
  if (s->d > 65536) return fail(FKL_EUNSUPPORTED, "d must be <= 65536");
  if (s->V < 1) return fail(FKL_EINVAL, "V must be >= 1");
  if (s->V > (int64_t(1) << 31) - 1024) return fail(FKL_EUNSUPPORTED, "V must be < 2^31 - 1024");
  if (s->K < 1) return fail(FKL_EINVAL, "K must be >= 1");
  if (s->K > 1024) return fail(FKL_EUNSUPPORTED, "K must be <= 1024");
  if (s->K > s->V) return fail(FKL_EINVAL, "K must be <= V");
  if (!(s->T > 0.0f) || !std::isfinite(s->T)) return fail(FKL_EINVAL, "T must be finite and > 0");
  if (s->chunk < 0) return fail(FKL_EINVAL, "chunk must be >= 0");
  if (s->vslab < 0) return fail(FKL_EINVAL, "vslab must be >= 0");
  if (s->flags & ~FKL_FLAGS_ALL) return fail(FKL_EINVAL, "unknown bits in flags");

  p->N = s->N;
  p->d = s->d;
  p->V = s->V;
  p->K = s->K;
  p->T = s->T;
  int64_t chunk = s->chunk ? s->chunk : kDefaultChunk;
  if (s->N > 0 && chunk > s->N) chunk = s->N;
  // Passes: no [rows x V] block is ever formed, so a forward pass costs only
  // its teacher lists and split statistics (15 MiB at 16384 rows, K = 100) and a
  // backward pass its gradient block (rows x vslab). With the default slab
  // the forward takes passes of at least min(N, fwd_floor_rows) rows and the
  // backward of at least min(N, kPassRows) (more rows share each W stream; a
  // narrower slab keeps the gradient block's size); an explicit vslab keeps
  // the caller's chunk in both directions.
  // The kernels address each operand view (an h chunk, a W slab, the
  // gradient block) through a buffer descriptor with a 32-bit byte size; a
  // raised floor stays under that limit.
  const int64_t kMaxView = (int64_t(1) << 31) - 1;
  const int64_t view_rows = kMaxView / (2 * s->d) / kTile * kTile;
  int64_t bchunk = chunk;
  if (s->vslab == 0 && s->N > 0) {
    chunk = std::max(chunk, std::min<int64_t>({s->N, fwd_floor_rows, view_rows}));
    bchunk = std::max(bchunk, std::min<int64_t>({s->N, kPassRows, view_rows}));
  }
  p->chunk = chunk;
  p->chunk_alloc = round_up(chunk, kTile);
  p->bchunk = bchunk;
  p->bchunk_alloc = round_up(bchunk, kTile);
  // the teacher lists serve the larger of the two directions' passes
  p->list_rows = std::max(p->chunk_alloc, p->bchunk_alloc);
  if (p->list_rows * s->d * 2 > kMaxView)
    return fail(FKL_EUNSUPPORTED, "chunk x d too large: a chunk of h must stay under 2 GiB");
  const int64_t slab_cap = std::min(kMaxView / (2 * s->d), kMaxView / (2 * p->bchunk_alloc)) / kTile * kTile;
  int64_t vslab = s->vslab ? s->vslab : std::min<int64_t>(kDefaultSlabElems / p->bchunk_alloc, slab_cap);
  vslab = round_up(vslab < kTile ? kTile : vslab, kTile);
  const int64_t v_all = round_up(s->V, kTile);
  if (vslab > v_all) vslab = v_all;
  if (vslab > slab_cap)
    return fail(FKL_EUNSUPPORTED, "vslab too large: a W slab and the gradient block must stay under 2 GiB");
  p->vslab = vslab;
  p->n_vt = ceil_div(s->V, kTile);
  const int64_t rbs = p->chunk_alloc / kTile;

  size_t off = 0;
  p->off_scalars = off;
  off += 256;
  p->off_negent = off;
  off = align256(off + static_cast<size_t>(p->list_rows) * 4);
  p->off_tidx = off;
  // teacher lists hold K entries, or K + 1 with hard labels (rows of the
  // larger of the forward and backward passes)
  off = align256(off + static_cast<size_t>(p->list_rows) * (p->K + 1) * 4);
  p->off_tp = off;
  off = align256(off + static_cast<size_t>(p->list_rows) * (p->K + 1) * 4);
  const size_t shared_end = off;
  // forward: split partials (two per row per workgroup) for up to (256 + rbs)
  // workgroups' rows, then one fp64 KL sum per kCombineRows rows
  p->off_partial = off;
  off = align256(off + static_cast<size_t>(kTargetBlocks + rbs) * 2 * kTile * 16);
  p->off_blocksum = off;
  off = align256(off + static_cast<size_t>(p->chunk_alloc / kCombineRows) * 8);
  p->fwd_bytes = off;
  // backward: the bf16 gradient block of bchunk_alloc x vslab, then grad_h
  // partial sums when a full pass needs a vocabulary split (sized for a full
  // pass; a shorter last pass takes at most as many partial rows)
  p->off_G = shared_end;
  off = align256(shared_end + static_cast<size_t>(p->bchunk_alloc) * p->vslab * 2);
  int splits = 1;
  if (!(s->flags & FKL_SKIP_GRAD_H)) {
    for (int64_t slab_w : {p->vslab, s->V - (ceil_div(s->V, p->vslab) - 1) * p->vslab}) {
      const int sp = grad_h_splits(bchunk, slab_w, s->d);
      if (sp > splits) splits = sp;
    }
  }
  p->ghp_rows = splits > 1 ? splits * p->bchunk_alloc : 0;
  p->off_ghp = off;
  off = align256(off + static_cast<size_t>(p->ghp_rows) * s->d * 4);
  p->flags = s->flags;
  p->off_gh32 = off;
  if ((s->flags & FKL_GRAD_H_BF16) && !(s->flags & FKL_SKIP_GRAD_H))
    off = align256(off + static_cast<size_t>(p->bchunk_alloc) * s->d * 4);
  p->bwd_bytes = off;
  return FKL_OK;
}

// P(X >= j) for X ~ Poisson(mu), summed from the pmf at j (log space).
double poisson_tail(double mu, int64_t j) {
  if (j <= 0) return 1.0;
  double term = std::exp(-mu + static_cast<double>(j) * std::log(mu) - std::lgamma(static_cast<double>(j) + 1.0));
  double sum = 0.0;
  for (int64_t k = j; k < j + 100000; ++k) {
    sum += term;
    term *= mu / static_cast<double>(k + 1);
    if (term <= sum * 1e-17) break;
  }
  return sum;
}

fkl_status make_topk_plan(const fkl_topk_shape* s, TopkPlan* p) {
  if (!s) return fail(FKL_EINVAL, "shape is NULL");
  if (s->N < 0) return fail(FKL_EINVAL, "N must be >= 0");
  if (s->N > (int64_t(1) << 31) - 1) return fail(FKL_EUNSUPPORTED, "N must be < 2^31");
  if (s->d < 8 || s->d % 8 != 0) return fail(FKL_EINVAL, "d must be a positive multiple of 8");
  if (s->d > 65536) return fail(FKL_EUNSUPPORTED, "d must be <= 65536");
  if (s->V < 1) return fail(FKL_EINVAL, "V must be >= 1");
  if (s->V > (int64_t(1) << 31) - 1024) return fail(FKL_EUNSUPPORTED, "V must be < 2^31 - 1024");
  if (s->K < 1) return fail(FKL_EINVAL, "K must be >= 1");
  if (s->K > 1024) return fail(FKL_EUNSUPPORTED, "K must be <= 1024");
  if (s->K > s->V) return fail(FKL_EINVAL, "K must be <= V");
  if (s->chunk < 0) return fail(FKL_EINVAL, "chunk must be >= 0");
  if (s->flags & ~static_cast<uint32_t>(FKL_TOPK_DIRECT | FKL_TOPK_MATERIALIZE))
    return fail(FKL_EINVAL, "unknown fkl_topk_shape flag");
  p->N = s->N;
  p->d = s->d;
  p->V = s->V;
  p->K = s->K;
  p->flags = s->flags;
  p->ld = round_up(s->V, kTile);
  p->fused = !(s->flags & (FKL_TOPK_DIRECT | FKL_TOPK_MATERIALIZE));
  // materialised block: 512 MiB of fp32 logits by default
  int64_t block_rows = kTopkDefaultBlockElems / p->ld / kTile * kTile;
  if (block_rows < kTile) block_rows = kTile;
  // sample: every stride-th full tile, at most kTopkMaxSampleTiles of them
  const int64_t n_full = s->V / kTile;
  const int64_t stride = std::max<int64_t>(kTopkMinStride, ceil_div(n_full, kTopkMaxSampleTiles));
  p->stride = static_cast<int32_t>(stride);
  p->n_sample = p->fused ? static_cast<int32_t>(ceil_div(n_full, stride)) : 0;
  // threshold: aimed at the j-th largest sampled key, j = ceil(target S / V),
  // so that about `target` keys of the row are expected at or above it (j = 0:
  // the sample is too small to aim, every key is a candidate). A row has
  // fewer than K keys at or above it only when j of its sampled keys lie
  // among its K largest; their number is about Poisson(K S / V) distributed,
  // so the target is the smallest count (at least 1024, and at least 16 V / S
  // so that j >= 16) whose j leaves that tail below kTopkMissTail per row.
  // (The other way out, more keys than the candidate slices hold, needs about
  // four times the target, which j >= 16 makes at least as improbable.)
  const int64_t S = static_cast<int64_t>(p->n_sample) * kTile;
  int64_t target = std::max<int64_t>({1024, s->K + 1, S > 0 ? ceil_div(16 * s->V, S) : 0});
  if (S > 0) {
    const double mu = static_cast<double>(s->K) * static_cast<double>(S) / static_cast<double>(s->V);
    while (target < s->V && poisson_tail(mu, ceil_div(target * S, s->V)) > kTopkMissTail)
      target += std::max<int64_t>(16, target / 64);
  }
  p->target = static_cast<int32_t>(std::min<int64_t>(target, std::max<int64_t>(s->V, 1024)));
  int64_t j = S > 0 ? ceil_div(static_cast<int64_t>(p->target) * S, s->V) : 0;
  if (j >= S) j = 0;
  p->j = static_cast<int32_t>(j);
  // about j sampled keys reach the threshold, more only when the 24-bit prefix
  // bin at the j-th key is crowded; a row with more than xcap is redone
  p->xcap = static_cast<int32_t>(j > 0 ? std::min<int64_t>(S, 2 * j + 256) : S);
  // per-row candidate slots of a full pass of R rows: 2 * splits slices
  auto slots_per_row = [p](int64_t R) {
    const int sp = topk_splits(*p, R);
    return static_cast<int64_t>(2 * sp) * topk_slice_cap(*p, sp);
  };
  int64_t chunk = s->chunk;
  if (chunk == 0) {
    if (p->fused) {
      const int64_t per_row = slots_per_row(kTopkFusedRows) * 8;
      const int64_t by_cand = kTopkCandBytes / per_row / kTile * kTile;
      chunk = std::min<int64_t>(kTopkFusedRows, std::max<int64_t>(kTile, by_cand));
    } else {
      chunk = block_rows;
    }
  }
  if (s->N > 0 && chunk > s->N) chunk = s->N;
  p->chunk = chunk;
  p->fb_rows = std::min(chunk, block_rows);
  size_t off = 0;
  p->off_flag = off;
  off += 256;
  p->off_ws = off;
  off = align256(off + static_cast<size_t>(S) * s->d * 2);
  p->off_region = off;
  const size_t chunk_alloc = static_cast<size_t>(round_up(chunk, kTile));
  size_t fused_bytes = 0;
  if (p->fused) {
    // candidate slices: the larger of a full pass and the last, shorter one
    // (fewer rows take more splits, hence more, smaller slices)
    int64_t slots = 0, slices = 0;
    for (int64_t R : {chunk, (s->N > 0 ? s->N - (ceil_div(s->N, chunk) - 1) * chunk : chunk)}) {
      const int sp = topk_splits(*p, R);
      slots = std::max(slots, round_up(R, kTile) * 2 * sp * topk_slice_cap(*p, sp));
      slices = std::max(slices, round_up(R, kTile) * 2 * sp);
    }
    p->off_sample = off;
    size_t o = align256(off + chunk_alloc * S * 4);
    p->off_thr = o;
    o = align256(o + chunk_alloc * 8);
    p->off_cnt = o;
    o = align256(o + static_cast<size_t>(slices) * 4);
    p->off_cand = o;
    o = align256(o + static_cast<size_t>(slots) * 8);
    // the extra slice of each row: its sampled keys at or above the threshold
    p->off_xcnt = o;
    o = align256(o + chunk_alloc * 4);
    p->off_xcand = o;
    o = align256(o + chunk_alloc * p->xcap * 8);
    fused_bytes = o - off;
  } else {
    p->off_sample = p->off_thr = p->off_cnt = p->off_cand = p->off_xcnt = p->off_xcand = off;
  }
  const size_t block_bytes = align256(static_cast<size_t>(round_up(p->fb_rows, kTile)) * p->ld * 4);
  p->bytes = off + std::max(fused_bytes, block_bytes);
  // the redo's blocks may fill the whole region: fewer launches when no row
  // is flagged (each then returns at once)
  p->redo_rows = p->fb_rows;
  if (p->fused) {
    const int64_t fit = static_cast<int64_t>(std::max(fused_bytes, block_bytes) / (static_cast<size_t>(p->ld) * 4)) /
                        kTile * kTile;
    if (fit > p->redo_rows) p->redo_rows = std::min(fit, chunk);
  }
  return FKL_OK;
}

}  // namespace fkl

extern "C" {

fkl_status fkl_workspace_size(const fkl_shape* shape, size_t* fwd_bytes, size_t* bwd_bytes) {
  fkl::Plan p;
  const fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (fwd_bytes) *fwd_bytes = p.fwd_bytes;
  if (bwd_bytes) *bwd_bytes = p.bwd_bytes;
  return FKL_OK;
}

}  // extern "C"

namespace {

// Checks shared by fkl_forward and fkl_forward_static (everything but the
// workspace), in the order the header documents; no HIP call.
fkl_status check_forward_args(const fkl::Plan& p, const void* h, const void* W, const int32_t* t_idx,
                              const float* t_logit, const fkl_terms* terms, const float* loss,
                              const float* row_lse, const float* row_kl, const float** weight,
                              const int32_t** label, float* label_w) {
  if (!loss) return fail(FKL_EINVAL, "loss is NULL");
  fkl_status st = read_terms(terms, weight, label, label_w);
  if (st != FKL_OK) return st;
  if (!aligned(loss, 4)) return fail(FKL_EINVAL, "loss must be 4-byte aligned");
  if (p.N > 0) {
    if (!h || !W || !t_idx || !t_logit || !row_lse)
      return fail(FKL_EINVAL, "h, W, t_idx, t_logit and row_lse must not be NULL");
    if (!aligned(h, 16) || !aligned(W, 16)) return fail(FKL_EINVAL, "h and W must be 16-byte aligned");
    if (!aligned(t_idx, 4) || !aligned(t_logit, 4) || !aligned(row_lse, 4) ||
        (row_kl && !aligned(row_kl, 4)))
      return fail(FKL_EINVAL, "t_idx, t_logit, row_lse and row_kl must be 4-byte aligned");
  }
  return FKL_OK;
}

// Debug build (FKL_DEBUG): the call's violation word is cleared before its
// first launch; after its last, the host waits for the stream and reports the
// access classes whose bounds checks fired. The release build does neither.
static_assert(fkl::kDebugWordOffset >= fkl::kValidateCountOffset + 4 && fkl::kDebugWordOffset + 4 <= 256,
              "the debug word shares the 256-byte control block with the scalars and the validation count");

fkl_status debug_begin(uint32_t* word, hipStream_t stream) {
#ifdef FKL_DEBUG
  const hipError_t e = fkl::launch_debug_clear(word, stream);
  if (e != hipSuccess) {
    g_last_error = std::string("debug word clear failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
#else
  (void)word, (void)stream;
#endif
  return FKL_OK;
}

fkl_status debug_end(uint32_t* word, hipStream_t stream) {
#ifdef FKL_DEBUG
  static const char* const kNames[fkl::kDebugBits] = {
      "teacher input rows", "sorted teacher lists", "forward split partials", "row outputs",
      "MFMA operand views", "gradient block",       "contraction outputs",    "grad_h reduction",
      "builder workspace",  "builder outputs"};
  uint32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    g_last_error = std::string("debug word read failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  if (host != 0) {
    std::string msg = "device bounds check failed (accesses skipped):";
    for (int b = 0; b < fkl::kDebugBits; ++b)
      if (host & (1u << b)) msg += std::string(" ") + kNames[b] + ";";
    g_last_error = msg;
    return FKL_EDEVICE;
  }
#else
  (void)word, (void)stream;
#endif
  return FKL_OK;
}

fkl_status run_forward(const fkl::Plan& p, const void* h, const void* W, const int32_t* t_idx,
                       const float* t_logit, const uint8_t* row_mask, const float* weight, const int32_t* label,
                       float label_w, float* loss, float* row_lse, float* row_kl, char* ws, hipStream_t stream) {
  fkl_status st = validate_if_asked(p, t_idx, t_logit, weight, label, ws, stream);
  if (st != FKL_OK) return st;
  uint32_t* dword = reinterpret_cast<uint32_t*>(ws + p.off_scalars + fkl::kDebugWordOffset);
  st = debug_begin(dword, stream);
  if (st != FKL_OK) return st;
  fkl::FwdArgs a{static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), t_idx, t_logit, row_mask,
                 weight, label, label_w, loss, row_lse, row_kl, ws};
  const hipError_t e = fkl::launch_forward(p, a, stream);
  if (e != hipSuccess) {
    g_last_error = std::string("forward launch failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return debug_end(dword, stream);
}

}  // namespace

extern "C" {

fkl_status fkl_forward(const fkl_shape* shape, const void* h, const void* W, const int32_t* t_idx,
                       const float* t_logit, const uint8_t* row_mask, const fkl_terms* terms, float* loss,
                       float* row_lse,
                       float* row_kl, void* workspace, size_t workspace_bytes, void* stream) {
  fkl::Plan p;
  fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  const float* weight;
  const int32_t* label;
  float label_w;
  st = check_forward_args(p, h, W, t_idx, t_logit, terms, loss, row_lse, row_kl, &weight, &label, &label_w);
  if (st != FKL_OK) return st;
  if (!workspace) return fail(FKL_EWORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FKL_EWORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.fwd_bytes) return fail(FKL_EWORKSPACE, "workspace is smaller than fkl_workspace_size()");
  return run_forward(p, h, W, t_idx, t_logit, row_mask, weight, label, label_w, loss, row_lse, row_kl,
                     static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

fkl_status fkl_forward_static(const fkl_shape* shape, const void* h, const void* W, const int32_t* t_idx,
                              const float* t_logit, const uint8_t* row_mask, const fkl_terms* terms, float* loss,
                              float* row_lse, float* row_kl, void* stream) {
  fkl::Plan p;
  fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  // A forward pass's rows do not change its results: where the default
  // slab's longer forward passes need more than the scratch, take passes of
  // the backward's rows (smaller teacher lists).
  if (p.fwd_bytes > fkl::kStaticScratchBytes && shape->vslab == 0) {
    fkl::Plan q;
    if (fkl::make_plan(shape, &q, fkl::kPassRows) == FKL_OK && q.fwd_bytes < p.fwd_bytes) p = q;
  }
  const float* weight;
  const int32_t* label;
  float label_w;
  st = check_forward_args(p, h, W, t_idx, t_logit, terms, loss, row_lse, row_kl, &weight, &label, &label_w);
  if (st != FKL_OK) return st;
  if (p.fwd_bytes > fkl::kStaticScratchBytes) {
    g_last_error = "the shape's forward workspace (" + std::to_string(p.fwd_bytes) +
                   " bytes) exceeds the static scratch of " + std::to_string(fkl::kStaticScratchBytes) +
                   " bytes; use fkl_forward with a workspace, or fewer rows per pass";
    return FKL_EWORKSPACE;
  }
  char* ws = nullptr;
  const hipError_t e = fkl::static_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e == hipErrorInvalidDevice) return fail(FKL_EINVAL, "stream must belong to the current device");
  if (e != hipSuccess) {
    g_last_error = std::string("static scratch lookup failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return run_forward(p, h, W, t_idx, t_logit, row_mask, weight, label, label_w, loss, row_lse, row_kl, ws,
                     static_cast<hipStream_t>(stream));
}

fkl_status fkl_backward(const fkl_shape* shape, const void* h, const void* W, const int32_t* t_idx,
                        const float* t_logit, const uint8_t* row_mask, const fkl_terms* terms,
                        const float* row_lse,
                        const float* grad_loss, void* grad_h, float* grad_W, void* workspace,
                        size_t workspace_bytes, void* stream) {
  fkl::Plan p;
  fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  const bool want_w = !(p.flags & FKL_SKIP_GRAD_W);
  const bool want_h = !(p.flags & FKL_SKIP_GRAD_H);
  const float* weight;
  const int32_t* label;
  float label_w;
  st = read_terms(terms, &weight, &label, &label_w);
  if (st != FKL_OK) return st;
  if (want_w && !grad_W) return fail(FKL_EINVAL, "grad_W is NULL");
  if (want_w && !aligned(grad_W, 16)) return fail(FKL_EINVAL, "grad_W must be 16-byte aligned");
  if (grad_loss && !aligned(grad_loss, 4)) return fail(FKL_EINVAL, "grad_loss must be 4-byte aligned");
  if (p.N > 0) {
    if (!h || !W || !t_idx || !t_logit || !row_lse)
      return fail(FKL_EINVAL, "h, W, t_idx, t_logit and row_lse must not be NULL");
    if (want_h && !grad_h) return fail(FKL_EINVAL, "grad_h is NULL");
    if (!aligned(h, 16) || !aligned(W, 16)) return fail(FKL_EINVAL, "h and W must be 16-byte aligned");
    if (want_h && !aligned(grad_h, 16)) return fail(FKL_EINVAL, "grad_h must be 16-byte aligned");
    if (!aligned(t_idx, 4) || !aligned(t_logit, 4) || !aligned(row_lse, 4))
      return fail(FKL_EINVAL, "t_idx, t_logit and row_lse must be 4-byte aligned");
  }
  if (!workspace) return fail(FKL_EWORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FKL_EWORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.bwd_bytes) return fail(FKL_EWORKSPACE, "workspace is smaller than fkl_workspace_size()");
  if (!want_w && !want_h) return FKL_OK;  // nothing asked for
  st = validate_if_asked(p, t_idx, t_logit, weight, label, static_cast<char*>(workspace),
                         static_cast<hipStream_t>(stream));
  if (st != FKL_OK) return st;
  uint32_t* dword =
      reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + p.off_scalars + fkl::kDebugWordOffset);
  st = debug_begin(dword, static_cast<hipStream_t>(stream));
  if (st != FKL_OK) return st;
  fkl::BwdArgs a{static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), t_idx, t_logit, row_mask,
                 weight, label, label_w, row_lse, grad_loss, grad_h, grad_W, static_cast<char*>(workspace)};
  const hipError_t e = fkl::launch_backward(p, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("backward launch failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return debug_end(dword, static_cast<hipStream_t>(stream));
}

fkl_status fkl_validate_teacher(const fkl_shape* shape, const int32_t* t_idx, const float* t_logit,
                                int32_t* bad_rows, void* stream) {
  fkl::Plan p;
  fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (!bad_rows || !aligned(bad_rows, 4)) return fail(FKL_EINVAL, "bad_rows must be a 4-byte aligned pointer");
  if (p.N > 0 && (!t_idx || !t_logit)) return fail(FKL_EINVAL, "t_idx and t_logit must not be NULL");
  if (p.N > 0 && (!aligned(t_idx, 4) || !aligned(t_logit, 4)))
    return fail(FKL_EINVAL, "t_idx and t_logit must be 4-byte aligned");
  const hipError_t e =
      fkl::launch_validate(p.N, p.V, p.K, t_idx, t_logit, bad_rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("validate launch failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return FKL_OK;
}

fkl_status fkl_validate_terms(const fkl_shape* shape, const fkl_terms* terms, int32_t* bad_rows, void* stream) {
  fkl::Plan p;
  fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (!bad_rows || !aligned(bad_rows, 4)) return fail(FKL_EINVAL, "bad_rows must be a 4-byte aligned pointer");
  const float* weight;
  const int32_t* label;
  float label_w;
  st = read_terms(terms, &weight, &label, &label_w);
  if (st != FKL_OK) return st;
  const hipError_t e =
      fkl::launch_validate_terms(p.N, p.V, weight, label, bad_rows, true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("validate launch failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return FKL_OK;
}

fkl_status fkl_plan_info(const fkl_shape* shape, fkl_plan* plan) {
  fkl::Plan p;
  const fkl_status st = fkl::make_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (!plan) return fail(FKL_EINVAL, "plan is NULL");
  plan->fwd_rows = p.chunk;
  plan->bwd_rows = p.bchunk;
  plan->vslab = p.vslab;
  plan->fwd_passes = p.N > 0 ? fkl::ceil_div(p.N, p.chunk) : 0;
  plan->bwd_passes = p.N > 0 ? fkl::ceil_div(p.N, p.bchunk) : 0;
  plan->slabs = fkl::ceil_div(p.V, p.vslab);
  plan->fwd_bytes = p.fwd_bytes;
  plan->bwd_bytes = p.bwd_bytes;
  return FKL_OK;
}

fkl_status fkl_topk_workspace_size(const fkl_topk_shape* shape, size_t* bytes) {
  fkl::TopkPlan p;
  const fkl_status st = fkl::make_topk_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (bytes) *bytes = p.bytes;
  return FKL_OK;
}

fkl_status fkl_topk(const fkl_topk_shape* shape, const void* h, const void* W, int32_t* t_idx, float* t_logit,
                    void* workspace, size_t workspace_bytes, void* stream) {
  fkl::TopkPlan p;
  const fkl_status st = fkl::make_topk_plan(shape, &p);
  if (st != FKL_OK) return st;
  if (p.N == 0) return FKL_OK;
  if (!h || !W || !t_idx || !t_logit) return fail(FKL_EINVAL, "h, W, t_idx and t_logit must not be NULL");
  if (!aligned(h, 16) || !aligned(W, 16)) return fail(FKL_EINVAL, "h and W must be 16-byte aligned");
  if (!aligned(t_idx, 4) || !aligned(t_logit, 4)) return fail(FKL_EINVAL, "t_idx and t_logit must be 4-byte aligned");
  if (!workspace) return fail(FKL_EWORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FKL_EWORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.bytes) return fail(FKL_EWORKSPACE, "workspace is smaller than fkl_topk_workspace_size()");
  uint32_t* dword = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + p.off_flag + fkl::kDebugWordOffset);
  const fkl_status ds = debug_begin(dword, static_cast<hipStream_t>(stream));
  if (ds != FKL_OK) return ds;
  const hipError_t e = fkl::launch_topk(p, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), t_idx,
                                        t_logit, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("top-k launch failed: ") + hipGetErrorString(e);
    return FKL_EDEVICE;
  }
  return debug_end(dword, static_cast<hipStream_t>(stream));
}

const char* fkl_status_string(fkl_status status) {
  switch (status) {
    case FKL_OK: return "ok";
    case FKL_EINVAL: return "invalid argument";
    case FKL_EWORKSPACE: return "workspace missing or too small";
    case FKL_EINDEX: return "bad teacher index";
    case FKL_EDEVICE: return "device error";
    case FKL_EUNSUPPORTED: return "unsupported shape";
  }
  return "unknown status";
}

const char* fkl_last_error(void) { return g_last_error.c_str(); }

int fkl_version(void) { return 200; }

}  // extern "C"
