// Host-side plan and kernel launchers shared by the C-ABI layer and the
// kernel translation unit. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fkl.h"

namespace fkl {

constexpr int kTile = 256;          // rows and vocabulary columns of one logits tile
constexpr int kContractionStep = 32;  // contraction depth of one LDS stage of the MFMA mainloop
constexpr int kTargetBlocks = 256;  // workgroups a launch aims for (one per CU on MI355X)
constexpr int kDefaultChunk = 4096;
constexpr int kPassRows = 8192;      // backward pass rows floor with the default slab
constexpr int kFwdPassRows = 16384;  // forward pass rows floor with the default slab
constexpr int64_t kDefaultSlabElems = int64_t(64) << 20;  // gradient block of ~64 Mi bf16 (128 MiB)

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// Everything derived from the shape; computed on the host only.
struct Plan {
  int64_t N, d, V;
  int32_t K;
  float T;
  int64_t chunk;        // rows per pass (<= N rounded up to 256 when N is small)
  int64_t chunk_alloc;  // chunk rounded up to 256
  int64_t bchunk;       // rows per backward pass (>= chunk)
  int64_t bchunk_alloc; // bchunk rounded up to 256
  int64_t list_rows;    // rows of the teacher lists and negentropies: max(chunk_alloc, bchunk_alloc)
  int64_t vslab;        // vocabulary columns per backward pass, multiple of 256
  int64_t n_vt;         // ceil(V / 256): logits tiles along the vocabulary
  // workspace offsets (bytes)
  size_t off_scalars, off_negent, off_tidx, off_tp, off_partial, off_blocksum, fwd_bytes;
  size_t off_G, bwd_bytes;
  // grad_h split along the vocabulary: partial sums for up to ghp_rows
  // (= splits x rows) rows of d fp32 each, reduced in a fixed order
  int64_t ghp_rows;
  size_t off_ghp;
  uint32_t flags;  // FKL_* backward options
  size_t off_gh32;  // fp32 [chunk_alloc][d] grad_h accumulator when grad_h is bf16
};

constexpr int kCombineRows = 16;  // rows per workgroup of the forward's split merge

// Byte offset, in the workspace's 256-byte scalars block, of the int32 bad-row
// count that FKL_VALIDATE=1 uses (the block's loss accumulators sit below it).
constexpr size_t kValidateCountOffset = 128;

constexpr int kMaxGradHSplits = 8;

// Debug build (FKL_DEBUG): classes of checked device accesses, the bits of a
// call's violation word, which sits at this offset in a 256-byte control block
// of the workspace (the loss's scalars block, the builder's flag block).
enum DebugBit : uint32_t {
  kDbgTeacherInput = 1u << 0,  // t_idx / t_logit / label rows read by the teacher prep
  kDbgTeacherList = 1u << 1,   // per-pass sorted teacher lists and negentropies
  kDbgPartial = 1u << 2,       // forward split partials
  kDbgRowOut = 1u << 3,        // row_lse / row_kl / per-block KL sums, row inputs of the backward
  kDbgOperand = 1u << 4,       // MFMA operand views (h, W, the gradient block, compact W)
  kDbgGBlock = 1u << 5,        // the bf16 gradient block G
  kDbgGemmOut = 1u << 6,       // fp32 outputs of the contractions (grad_h, grad_W, partial sums, logits)
  kDbgReduce = 1u << 7,        // grad_h reductions and the bf16 conversion
  kDbgTopkWork = 1u << 8,      // builder workspace: thresholds, candidate slices and counts
  kDbgTopkOut = 1u << 9,       // builder outputs t_idx / t_logit
};
constexpr int kDebugBits = 10;
constexpr size_t kDebugWordOffset = 192;

// Vocabulary splits for the grad_h tiles of one backward launch (rows of the
// chunk, slab_w columns of the slab) so that no grad_h tile is much longer than
// the launch's average work per CU; 1 when the launch is balanced without.
int grad_h_splits(int64_t rows, int64_t slab_w, int64_t d);

// fwd_floor_rows: the forward's pass rows floor with the default slab
// (kFwdPassRows; the allocation-free forward lowers it to kPassRows when its
// scratch cannot hold the longer passes' teacher lists).
fkl_status make_plan(const fkl_shape* s, Plan* p, int64_t fwd_floor_rows = kFwdPassRows);

// Per-call device pointers of the forward pass.
struct FwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int32_t* t_idx;
  const float* t_logit;
  const uint8_t* mask;
  const float* weight;   // per-row weights or NULL
  const int32_t* label;  // hard labels or NULL
  float label_weight;
  float* loss;
  float* row_lse;
  float* row_kl;
  char* ws;
};

struct BwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int32_t* t_idx;
  const float* t_logit;
  const uint8_t* mask;
  const float* weight;
  const int32_t* label;
  float label_weight;
  const float* row_lse;
  const float* grad_loss;
  void* grad_h;  // fp32, or bf16 with FKL_GRAD_H_BF16
  float* grad_W;
  char* ws;
};

// Event-based kernel timing (enabled by fkl_trace_enable). A scope records a
// start event on construction and a stop event on destruction, on `stream`.
class TraceScope {
 public:
  TraceScope(hipStream_t stream, const char* name, double flops, double bytes);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  hipStream_t stream_;
  uint64_t id_;  // 0: not traced
};

// Teacher-cache builder (fkl_topk). Two routes:
//  * fused (default): per pass of `chunk` rows, the logits of a sample of
//    whole vocabulary tiles give each row a threshold key; one sweep over the
//    other tiles keeps the keys at or above it (candidates, at most `cap` per
//    row); the top K is selected among them. A pass in which some row kept
//    fewer than K keys or more than `cap` is redone by the materialised route.
//  * materialised: the logits of fb_rows rows at a time are formed in an fp32
//    block and each row's top K is selected there.
struct TopkPlan {
  int64_t N, d, V;
  int32_t K;
  int64_t chunk;    // rows per pass
  int64_t fb_rows;  // rows per materialised logits block (<= chunk)
  int64_t redo_rows;  // rows per block of the fused route's guarded redo (>= fb_rows, <= chunk): as
                      // many as the pass's fused buffers, which the redo's block replaces, make room for
  int64_t ld;       // row stride of the logits block (V rounded up to 256)
  uint32_t flags;   // FKL_TOPK_* options
  bool fused;       // the fused route runs (otherwise every pass is materialised)
  int32_t stride;   // sampled tiles: the full vocabulary tiles t with t % stride == 0
  int32_t n_sample; // number of sampled tiles
  int32_t target;   // candidates per row the threshold aims at
  int32_t j;        // the threshold is aimed at a row's j-th largest sampled key (0: every key)
  int32_t xcap;     // slots of a row's extra slice (its sampled keys at or above the threshold)
  // workspace offsets (bytes); the fused buffers and the logits block share
  // the region at off_region (a pass's fused buffers are dead before its
  // materialised redo starts)
  size_t off_flag, off_ws, off_region, off_sample, off_thr, off_cnt, off_cand, off_xcnt, off_xcand;
  size_t bytes;
};

constexpr int64_t kTopkDefaultBlockElems = int64_t(128) << 20;  // default logits block (512 MiB)
constexpr int64_t kTopkFusedRows = 16384;                        // default rows per fused pass
constexpr int64_t kTopkCandBytes = int64_t(1) << 30;             // bound on a pass's candidate slices
constexpr int kTopkMaxSampleTiles = 16;
constexpr double kTopkMissTail = 1e-12;  // per-row probability of too few keys at the threshold
constexpr int kTopkMinStride = 16;

// Vocabulary splits of a fused pass's sweep over `rows` rows (as many
// workgroups as fit in one round on the CUs, at most one per unsampled
// tile), and the slots of
// each of a row's 2 * splits candidate slices: room for four times the
// slice's share of the target, plus 16 (candidates may cluster in parts of
// the vocabulary).
inline int topk_splits(const TopkPlan& p, int64_t rows) {
  const int64_t rbs = (rows + kTile - 1) / kTile;
  int64_t s = kTargetBlocks / rbs;  // rbs x splits stays within one round of workgroups
  const int64_t n_u = (p.V + kTile - 1) / kTile - p.n_sample;
  if (s > n_u) s = n_u;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}
inline int topk_slice_cap(const TopkPlan& p, int splits) {
  return static_cast<int>((2 * static_cast<int64_t>(p.target) + 2 * splits - 1) / (2 * splits)) * 2 + 16;
}

fkl_status make_topk_plan(const fkl_topk_shape* s, TopkPlan* p);
// P(X >= j) for X ~ Poisson(mu) (host; the builder's target uses it).
double poisson_tail(double mu, int64_t j);

hipError_t launch_forward(const Plan& p, const FwdArgs& a, hipStream_t stream);

// Static scratch of the allocation-free forward (fkl_forward_static): its
// size, and the device address of the calling device's copy. The lookup runs
// once per device, with that device current; `stream` must belong to the
// current device (hipErrorInvalidDevice otherwise).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch(hipStream_t stream, char** ptr);
hipError_t launch_topk(const TopkPlan& p, const uint16_t* h, const uint16_t* W, int32_t* t_idx, float* t_logit,
                       char* ws, hipStream_t stream);
hipError_t launch_backward(const Plan& p, const BwdArgs& a, hipStream_t stream);
hipError_t launch_validate(int64_t N, int64_t V, int32_t K, const int32_t* t_idx,
                           const float* t_logit, int32_t* bad_rows, hipStream_t stream);
// Zero the debug build's violation word of a call (one small kernel).
hipError_t launch_debug_clear(uint32_t* word, hipStream_t stream);
// Rows whose label is outside [0, V) or whose weight is not finite are added
// to *bad_rows (cleared first when `clear`).
hipError_t launch_validate_terms(int64_t N, int64_t V, const float* weight, const int32_t* label,
                                 int32_t* bad_rows, bool clear, hipStream_t stream);

}  // namespace fkl
