/*
 * libfkl: fused output projection + sparse top-K KL divergence, forward and
 * backward with recomputation, for AMD Instinct MI355X (gfx950).
 *
 * What is computed. The method fuses the student's output projection into
 * the distillation loss: it walks the token positions one chunk at a time,
 * forms that chunk's logits from the hidden states and the head weight,
 * folds them into a running loss against the teacher's cached top-K
 * (index, logit) pairs, and drops them; backward forms each chunk's logits
 * again instead of storing them (blog post on the page "Efficient Offline
 * Top-K Logits and Fused Chunked KL Loss Enable Scalable LLM Distillation",
 * section "Two systems changes"). The pages print no formula; the library
 * implements these readings of the prose:
 *
 *   s[r,v]  = (h[r,:] . W[v,:]) / T                        (all rows)
 *   lse[r]  = log sum_v exp(s[r,v])                        -> row_lse
 *   p[r,k]  = softmax_k(t_logit[r,k] / T)   over the K cached entries
 *   KL[r]   = sum_k p[r,k] (log p[r,k] - s[r, t_idx[r,k]] + lse[r])
 *             (forward KL teacher || student; 0 on masked rows) -> row_kl
 *   loss    = T^2 / n * sum_{r valid} KL[r]      (n valid rows; 0 if n = 0)
 *   G[r,v]  = g * (T/n) * mask[r] * (exp(s[r,v] - lse[r]) - p~[r,v])
 *   grad_h  = G W        grad_W = G^T h
 *
 * where p~ is p scattered onto the vocabulary at t_idx (zero elsewhere) and
 * g the upstream gradient of the loss.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE memory owned by the caller. The library
 *     allocates and frees nothing and keeps no state between calls.
 *   - Row-major, contiguous. h: bf16 [N, d]; W: bf16 [V, d]; t_idx: int32
 *     [N, K]; t_logit: fp32 [N, K]; row_mask: uint8 [N] (nonzero = valid) or
 *     NULL (all valid); fp32 outputs.
 *   - h, W, grad_h and grad_W must be 16-byte aligned; every other array
 *     4-byte aligned.
 *   - d must be a multiple of 8; 1 <= K <= min(V, 1024); T > 0 and finite.
 *   - Teacher indices must lie in [0, V) and be distinct within each row;
 *     t_logit finite. Checked by fkl_validate_teacher, and by fkl_forward and
 *     fkl_backward themselves when the environment sets FKL_VALIDATE=1: they
 *     then return FKL_EINDEX for bad lists (a debugging aid that waits for
 *     the stream on the host). Bad lists never make the kernels access memory
 *     out of bounds; the loss and gradients are then undefined.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream)
 *     and is complete when the stream is. No call synchronises the host
 *     (except under FKL_VALIDATE=1).
 *   - Argument errors are reported before any device work is enqueued; such
 *     calls never touch the device, so they are safe without a GPU.
 *   - The same workspace must not be used by two calls in flight at once.
 *   - The debug build (libfkl_debug.so, compiled with FKL_DEBUG) has the same
 *     interface and results. Its kernels also check every global store, list
 *     read and operand view against the extents the host planned, skipping
 *     any access outside them. Each call then waits for its stream and
 *     returns FKL_EDEVICE naming the access classes that fired. The release
 *     build does no such checks.
 */
#ifndef FKL_H
#define FKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FKL_OK = 0,
  FKL_EINVAL = 1,       /* bad shape, NULL or misaligned pointer */
  FKL_EWORKSPACE = 2,   /* workspace NULL or smaller than fkl_workspace_size() */
  FKL_EINDEX = 3,       /* bad teacher lists or loss terms (FKL_VALIDATE=1) */
  FKL_EDEVICE = 4,      /* a HIP call failed, or (debug build) a bounds check fired; see fkl_last_error() */
  FKL_EUNSUPPORTED = 5  /* shape outside what this build supports */
} fkl_status;

typedef struct {
  int64_t N;     /* token positions (rows); N >= 0 */
  int64_t d;     /* hidden size; multiple of 8, 8 <= d <= 65536 */
  int64_t V;     /* vocabulary size; V >= 1 */
  int32_t K;     /* cached teacher entries per row */
  float T;       /* temperature */
  int32_t chunk; /* rows per pass; 0 = 4096. With vslab = 0 forward passes
                    are at least min(N, 16384) rows and backward passes at
                    least min(N, 8192) (either floor lowered where an h pass
                    would reach 2 GiB): no [rows x V] block is ever formed,
                    so a pass costs only its teacher lists forward and the
                    gradient block (whose size vslab fixes) backward. With
                    an explicit vslab both directions take passes of chunk
                    rows. Results do not depend on it. */
  int32_t vslab; /* vocabulary columns per backward pass; 0 = chosen so that
                    a pass's gradient block holds about 64 Mi elements.
                    Rounded up to a multiple of 256. Results do not depend
                    on it beyond fp32 summation order of grad_h. */
  uint32_t flags; /* backward options, FKL_* below (0 = defaults); ignored by
                     fkl_forward */
} fkl_shape;

/*
 * Backward options, for use inside a training step (the loss is meant as a
 * drop-in replacement for the KL term of a distillation loop: page "Making
 * knowledge distillation cheap enough to run in production").
 *   FKL_ACCUMULATE_GRAD_W  grad_W += this call's gradient (micro-batch
 *                          accumulation) instead of grad_W = ...
 *   FKL_ACCUMULATE_GRAD_H  grad_h += this call's gradient
 *   FKL_SKIP_GRAD_W        grad_W is not computed (frozen head); may be NULL
 *   FKL_SKIP_GRAD_H        grad_h is not computed; may be NULL
 *   FKL_GRAD_H_BF16        grad_h is bf16 [N, d]: accumulated in fp32 in the
 *                          workspace over the vocabulary and rounded once
 *                          (round to nearest even); with FKL_ACCUMULATE_GRAD_H
 *                          the old bf16 value is added in fp32 first
 */
#define FKL_ACCUMULATE_GRAD_W 0x1u
#define FKL_ACCUMULATE_GRAD_H 0x2u
#define FKL_SKIP_GRAD_W 0x4u
#define FKL_SKIP_GRAD_H 0x8u
#define FKL_GRAD_H_BF16 0x10u
#define FKL_FLAGS_ALL 0x1fu

/*
 * Optional loss terms (pass NULL for the plain loss). The pages name a
 * "choice of loss function" for the distillation loss without defining
 * variants; these are the ones the fused structure carries at no extra
 * contraction work:
 *   row_weight   fp32 [N] per-token weights (finite), multiplied by the row
 *                mask; NULL means 1. A row whose weight is not positive
 *                (zero, negative or NaN) takes no part, as if masked. The
 *                loss is the weighted mean T^2 sum_r w_r l_r / sum_r w_r over
 *                the rows with w_r > 0 (0 when there are none).
 *   label        int32 [N] hard labels y_r in [0, V) (precondition, checked
 *                by fkl_validate_terms and under FKL_VALIDATE=1; a label
 *                outside the range never makes a kernel access memory out of
 *                bounds, the loss is then undefined); NULL means no label
 *                term.
 *   label_weight a in [0, 1]: per row l_r = (1 - a) KL(p_r || q_r) +
 *                a CE(y_r, q_r), both at the loss temperature (q = softmax(z/T)).
 * row_kl then reports l_r (0 where w_r <= 0 or the row is masked).
 */
typedef struct {
  const float* row_weight;
  const int32_t* label;
  float label_weight;
} fkl_terms;

/*
 * Workspace bytes needed by fkl_forward and fkl_backward for this shape.
 *
 * Defined by: the blog post, section "Two systems changes" (only one chunk
 * of positions is ever in flight, so the extra memory is bounded by a
 * chunk's working set) and section "Scaling to long context lengths" (peak
 * memory of the fused loss grows with the sequence only through its inputs
 * and outputs). Here no [chunk x V] block exists at all: a forward pass
 * needs its teacher lists and split statistics, a backward pass the bf16
 * gradient block of one vocabulary slab.
 *
 * Arguments: shape (host pointer, read only); fwd_bytes, bwd_bytes (host
 * pointers, either may be NULL) receive the byte counts. One workspace of
 * max(fwd_bytes, bwd_bytes) serves both calls. Pure host code: no HIP call.
 * Sizes: with R the pass rows and S the slab (fkl_plan_info), forward
 * O(R * (K + 64)), backward O(R * (S + K)), plus O(R * d) fp32 when a pass's
 * grad_h is split along the vocabulary (few rows per pass) or returned in
 * bf16; N enters only below one pass, V only through one slab.
 * Errors: FKL_EINVAL for a NULL or malformed shape; FKL_EUNSUPPORTED when an
 * h pass (R x d bf16), W slab (S x d bf16) or gradient block (R x S bf16)
 * would exceed 2 GiB (the default slab is capped to stay below).
 */
fkl_status fkl_workspace_size(const fkl_shape* shape, size_t* fwd_bytes, size_t* bwd_bytes);

/*
 * How a shape is run (host only): rows per forward and backward pass,
 * vocabulary columns per backward slab, the pass and slab counts, and the
 * workspace sizes of fkl_workspace_size. Results never depend on these;
 * they describe the memory and launch plan (blog post, section "Two systems
 * changes": the loss walks the positions one chunk at a time).
 * Errors: those of fkl_workspace_size; FKL_EINVAL if plan is NULL.
 */
typedef struct {
  int64_t fwd_rows;   /* rows per forward pass */
  int64_t bwd_rows;   /* rows per backward pass */
  int64_t vslab;      /* vocabulary columns per backward slab */
  int64_t fwd_passes; /* ceil(N / fwd_rows) (0 when N = 0) */
  int64_t bwd_passes; /* ceil(N / bwd_rows) (0 when N = 0) */
  int64_t slabs;      /* ceil(V / vslab) */
  size_t fwd_bytes;   /* workspace bytes of fkl_forward */
  size_t bwd_bytes;   /* workspace bytes of fkl_backward */
} fkl_plan;

fkl_status fkl_plan_info(const fkl_shape* shape, fkl_plan* plan);

/*
 * Forward pass of the fused loss.
 *
 * Defined by: the blog post, section "Two systems changes": the output
 * projection is fused into the loss, so the call takes the hidden states
 * and the head weight rather than logits; it walks the positions one chunk
 * at a time, projects the chunk to logits, folds them into the running loss
 * against the cached sparse top-K teacher and drops them. The loss is the
 * KL term of a distillation step ("drop-in replacement for the KL term":
 * page "Making knowledge distillation cheap enough to run in production").
 *
 * Inputs (device): h bf16 [N, d], W bf16 [V, d], t_idx int32 [N, K],
 * t_logit fp32 [N, K], row_mask uint8 [N] or NULL, terms (host struct
 * pointing at device arrays) or NULL.
 * Outputs (device, caller-allocated, overwritten): loss fp32 [1]; row_lse
 * fp32 [N], logsumexp over the vocabulary of s = z/T for every row including
 * masked ones; row_kl fp32 [N] (the per-row loss term, 0 on rows that take
 * no part) or NULL.
 * workspace: device, 256-byte aligned, at least fwd_bytes of
 * fkl_workspace_size; stream: hipStream_t (NULL = default stream).
 * Errors: argument errors (NULL, misaligned, bad shape, short workspace)
 * return before any device work; FKL_EDEVICE if a launch fails;
 * FKL_EINDEX under FKL_VALIDATE=1 for bad teacher lists or loss terms.
 * Deterministic: the same inputs give bitwise the same outputs.
 */
fkl_status fkl_forward(const fkl_shape* shape, const void* h, const void* W,
                       const int32_t* t_idx, const float* t_logit, const uint8_t* row_mask,
                       const fkl_terms* terms, float* loss, float* row_lse, float* row_kl,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation and kernels as fkl_forward,
 * with the workspace taken from a static device array of the library,
 * FKL_STATIC_SCRATCH_BYTES (32 MiB) on every GPU the library runs on, held
 * until the process ends. Allocates nothing. The results are fkl_forward's
 * bit for bit, except that with vslab = 0, where fkl_forward's passes of at
 * least min(N, 16384) rows would need more than the scratch (fwd_bytes of
 * fkl_workspace_size), passes of at least min(N, 8192) rows are taken
 * instead, which changes only the fp32 summation order.
 *
 * Arguments and outputs as fkl_forward. The stream must belong to the
 * current device (the scratch used is that device's copy).
 * Errors: as fkl_forward; FKL_EWORKSPACE when the forward workspace of the
 * passes taken still exceeds FKL_STATIC_SCRATCH_BYTES (fewer rows per pass,
 * chunk with an explicit vslab, lower it); FKL_EINVAL when the stream
 * belongs to another device.
 * Concurrency: all calls on one GPU share its scratch, so calls that overlap
 * on one GPU (several streams or threads) race and must be serialised by the
 * caller. Nothing in the scratch needs to start at zero: every call writes
 * each region before reading it.
 */
#define FKL_STATIC_SCRATCH_BYTES (32u << 20)

fkl_status fkl_forward_static(const fkl_shape* shape, const void* h, const void* W,
                              const int32_t* t_idx, const float* t_logit, const uint8_t* row_mask,
                              const fkl_terms* terms, float* loss, float* row_lse, float* row_kl,
                              void* stream);

/*
 * Backward pass of the fused loss, with recomputation.
 *
 * Defined by: the blog post, section "Two systems changes": backward forms
 * each chunk's logits again instead of storing them (the projection is done
 * twice), and yields the gradients of the hidden states and of the head
 * that the training step needs (page "Making knowledge distillation cheap
 * enough to run in production": a drop-in replacement for the KL term).
 * With G = dloss/dz (the closed form in this file's header), grad_h = G W
 * and grad_W = G^T h.
 *
 * Inputs (device): as fkl_forward, plus row_lse fp32 [N] from the forward of
 * the same inputs and grad_loss fp32 [1] holding the upstream gradient g
 * (NULL: g = 1).
 * Outputs (device, caller-allocated): grad_h fp32 [N, d] (bf16 with
 * FKL_GRAD_H_BF16) and grad_W fp32 [V, d], overwritten or accumulated into
 * as shape->flags says; either may be NULL when skipped. Rows that take no
 * part in the loss get exactly zero grad_h rows (unchanged when
 * accumulating).
 * workspace: device, 256-byte aligned, at least bwd_bytes of
 * fkl_workspace_size; stream as fkl_forward.
 * Errors: as fkl_forward. Deterministic: no floating-point atomics.
 */
fkl_status fkl_backward(const fkl_shape* shape, const void* h, const void* W,
                        const int32_t* t_idx, const float* t_logit, const uint8_t* row_mask,
                        const fkl_terms* terms, const float* row_lse, const float* grad_loss,
                        void* grad_h, float* grad_W,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Checks the teacher cache on the device: every index in [0, V), no index
 * repeated within a row, every logit finite. Writes the number of offending
 * rows to bad_rows (device int32 [1]). The cache is the method's offline
 * top-K store (section "Two systems changes" of the blog post).
 */
fkl_status fkl_validate_teacher(const fkl_shape* shape, const int32_t* t_idx,
                                const float* t_logit, int32_t* bad_rows, void* stream);

/*
 * Checks the optional loss terms on the device: every hard label in [0, V)
 * and every row weight finite. Writes the number of offending rows to
 * bad_rows (device int32 [1]). terms may be NULL (nothing to check: 0).
 * Errors: FKL_EINVAL for a bad shape, a NULL or misaligned bad_rows, or a
 * label_weight outside [0, 1]; FKL_EDEVICE if the launch fails.
 */
fkl_status fkl_validate_terms(const fkl_shape* shape, const fkl_terms* terms, int32_t* bad_rows,
                              void* stream);

/*
 * Offline teacher-cache builder: the step before the fused loss. The blog
 * post (section "Two systems changes") caches each position's top-100
 * teacher logits once, offline, and keeps nothing else of the teacher's
 * distribution; this computes such a cache on the GPU.
 *
 * For every row r of h [N,d] (bf16, row-major) and a teacher head
 * W [V,d] (bf16, row-major), the K largest logits z[r,v] = sum_j h[r,j] W[v,j]
 * (bf16 products, fp32 accumulation) with their indices:
 *   t_idx   int32 [N,K]  vocabulary indices, row-major
 *   t_logit fp32  [N,K]  the logits, in descending order; equal logits are
 *                        ordered by the lower index first, and the K-th place
 *                        goes to the lowest indices among equal logits.
 * The output is in the layout fkl_forward / fkl_backward read.
 *
 * Default (fused) route, per pass of `chunk` rows (0: 16384, fewer for
 * large K): the logits of a sample of whole vocabulary tiles (every 16th or
 * more sparse, at most 16 tiles) give each row a threshold key aimed at about
 * T of its logits, T >= 1024 chosen so that a row keeps fewer than K only
 * with probability below 1e-12; one sweep over the other tiles keeps only the
 * keys at or above it (no [rows x V] block is formed), and the top K is
 * selected exactly among them. A row for which fewer than K keys reached the
 * threshold, or more than its candidate slots hold, makes the pass be redone
 * by the materialised route, so the result never depends on the sample.
 * Materialised route (FKL_TOPK_MATERIALIZE, FKL_TOPK_DIRECT): the logits of
 * up to chunk rows at a time (0: enough rows for a 512 MiB fp32 block, at
 * least 256) are formed in the workspace and each row's top K is selected
 * there: normally from a threshold taken from a sample of the row (a
 * threshold that keeps fewer than K logits or too many is moved and the row
 * read again, three tries), with FKL_TOPK_DIRECT over the whole row. Every
 * route returns the same result. Constraints: d a multiple of 8
 * (<= 65536), 1 <= K <= min(V, 1024); h and W 16-byte aligned; the workspace
 * 256-byte aligned. Argument errors return before any HIP call.
 */
typedef struct {
  int64_t N, d, V;
  int32_t K;
  int32_t chunk;   /* rows per pass; 0 = default */
  uint32_t flags;  /* FKL_TOPK_* below; 0 = default */
} fkl_topk_shape;

#define FKL_TOPK_DIRECT 0x1u      /* materialised route, each row selected over the whole row */
#define FKL_TOPK_MATERIALIZE 0x2u /* materialised route, rows selected from a sampled threshold */

/*
 * Workspace bytes of fkl_topk for this shape (host only; bytes may be NULL).
 * The default fused pass of 16384 rows over a 128256-entry vocabulary needs
 * about 857 MiB (the sample's logits and the candidate slices); a smaller
 * chunk needs proportionally less. The materialised routes need one logits
 * block (512 MiB by default, chunk x V rounded up x 4 bytes otherwise).
 * Errors: FKL_EINVAL for a NULL or malformed shape or an unknown flag;
 * FKL_EUNSUPPORTED for K > 1024, d > 65536 or N, V beyond 32-bit indexing.
 */
fkl_status fkl_topk_workspace_size(const fkl_topk_shape* shape, size_t* bytes);

/*
 * Builds the cache described above: h, W device inputs; t_idx, t_logit
 * device outputs (overwritten); workspace device, at least
 * fkl_topk_workspace_size bytes. Nothing is enqueued when N = 0.
 * Errors: those of fkl_topk_workspace_size; FKL_EINVAL for NULL or
 * misaligned arrays; FKL_EWORKSPACE for a NULL, misaligned or short
 * workspace; FKL_EDEVICE if a launch fails. Deterministic: the output does
 * not depend on the route, the chunk or timing.
 */
fkl_status fkl_topk(const fkl_topk_shape* shape, const void* h, const void* W,
                    int32_t* t_idx, float* t_logit,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing. While enabled (a process-wide switch), every launch of the
 * path's main kernels is bracketed by a pair of hipEvents recorded on the
 * call's own stream, tagged with the kernel name and the launch's
 * algorithmic work: FLOPs of its contractions (2 per multiply-add of the
 * logits, grad_h or grad_W products) and the bytes it must move at least
 * (its operands read once, its outputs written once). Costs a few
 * microseconds per launch; off by default.
 */
typedef struct {
  char name[32];     /* kernel name, e.g. "fwd_sweep" */
  int64_t launches;  /* launches recorded since the last read */
  double total_ms;   /* summed event-measured durations */
  double min_ms;
  double max_ms;
  double flops;      /* summed algorithmic FLOPs */
  double bytes;      /* summed algorithmic bytes */
} fkl_kernel_stat;

fkl_status fkl_trace_enable(int on);

/*
 * Waits for the recorded events, aggregates them per kernel name into
 * stats[0 .. min(capacity, kinds)), sets *count to the number of kernel
 * names seen, and clears the record. Host-synchronising. Thread-safe: a
 * launch still being enqueued on another thread is left for a later read,
 * so each launch is reported exactly once.
 */
fkl_status fkl_trace_read(fkl_kernel_stat* stats, int capacity, int* count);

/* Static description of a status code. */
const char* fkl_status_string(fkl_status status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* fkl_last_error(void);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH (0.2.0: the plan
 * query, loss-term validation, the allocation-free forward and the fused
 * top-K builder). */
int fkl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FKL_H */
