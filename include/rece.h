/* rece.h - RECE / SCE reduced cross-entropy loss, forward and backward, on one
 * AMD Instinct MI355X (gfx950).  C ABI of librece.
 *
 * What is computed (RECE page, "RECE: Reduced Cross-Entropy Loss for
 * Large-Catalogue Sequential Recommenders", Section 3, Algorithm 1 and the
 * method paragraph before it):
 *   for every round rho = 0..r-1 (independent random vectors B_rho):
 *     bucket of each position x_i and item y_j = argmax over the n_b random
 *       vectors b of the signed scalar product b.v (ties: lowest index);
 *     positions and items are stably sorted by bucket and cut into n_c equal
 *       chunks (chunk c holds sorted slots p with c*N/n_c <= p < (c+1)*N/n_c);
 *     a position in X-chunk c is scored against the items of chunks
 *       c-n_ec .. c+n_ec (modulo n_c, or clipped to [0, n_c)), its own positive
 *       excluded, and keeps the k largest logits (order: logit descending, item
 *       id ascending);
 *   the kept pairs of all rounds form a set (the page's minus-ln(count) rule
 *   makes a pair kept in several rounds count once);
 *   loss_i = logsumexp({x_i.y_pos_i} u {x_i.y_j : j kept}) - x_i.y_pos_i,
 *   loss = mean over the s positions.
 * The backward pass returns d loss / d X and d loss / d Y with the selection held
 * fixed (Eq. 4 of the same page restricted to the kept set).
 *
 * Selection decisions (bucket argmax, top-k membership) are taken on the float64
 * value of each scalar product summed in coordinate order; the kernels compute
 * float32 matrix-core products with a proven error bound and recompute in
 * float64 only where the bound cannot decide.  Loss and gradients are float32.
 *
 * SCE variant (SCE page, "Scalable Cross-Entropy Loss for Sequential
 * Recommendations with Large Item Catalogs", abstract: softmax over a subset
 * found by maximum inner product search): n_b projection buckets; bucket b
 * takes the b_x positions and b_y items with the largest scores b.v, scores its
 * positions against its items, and every position keeps the k largest logits
 * over the union of the buckets that took it.
 *
 * Conventions for every entry point:
 *   - device pointers are caller-owned, contiguous, row-major and at least
 *     16-byte aligned; the library never allocates device memory (its one
 *     static scratch array aside, see rece_forward_static);
 *   - `stream` is a hipStream_t (NULL = the default stream); every call that
 *     takes a stream only enqueues work on it and returns without waiting,
 *     except rece_check, which waits for the stream;
 *   - every call returns a rece_status; no C++ exception crosses the ABI;
 *     rece_last_error() gives a thread-local message for the last failure.
 */
#ifndef RECE_H_
#define RECE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RECE_OK = 0,
  RECE_ERR_INVALID_ARGUMENT = 1,   /* bad config value, NULL or misaligned pointer */
  RECE_ERR_UNSUPPORTED = 2,        /* valid but not built (e.g. d outside {32,64,128,256}) */
  RECE_ERR_WORKSPACE_TOO_SMALL = 3,
  RECE_ERR_HIP = 4,                /* a HIP runtime call failed; see rece_last_error() */
  RECE_ERR_DEVICE_CHECK = 5,       /* a device-side check failed (read by rece_check) */
  RECE_ERR_INTERNAL = 6
} rece_status;

typedef enum { RECE_F32 = 0, RECE_BF16 = 1 } rece_dtype;
typedef enum { RECE_VARIANT_RECE = 0, RECE_VARIANT_SCE = 1 } rece_variant;

/* flags */
#define RECE_FLAG_VALIDATE_IDS 1u  /* device check that 0 <= pos[i] < C (error word) */
#define RECE_FLAG_IGNORE_NEGATIVE_POS 4u  /* padding mask: positions with pos[i] < 0 are padding.
                                            They stay rows of X (bucketed, sorted and chunked
                                            like the others) but have loss 0, no gradient, and
                                            the mean is over the other positions (0 if none). */
#define RECE_FLAG_BF16_GRADS 8u    /* rece_backward writes dX and dY as bf16 (round to
                                      nearest even) instead of float32 */
#define RECE_FLAG_KEEP_STAGES 2u   /* accepted, no effect: the kept lists are always kept
                                      (the backward pass reads them) */

/* Loss configuration.  RECE page, Algorithm 1 (input line: positions, items, n_b,
 * n_c) and the method paragraph of Section 3 (rounds r, neighbouring chunks n_ec,
 * the duplicate rule); k, the negatives kept per position, is this library's
 * top-k of the window (the paragraph's "logits with the largest absolute
 * gradient").  SCE page, abstract, for the bucket variant (b_x, b_y). */
typedef struct {
  int64_t s;        /* positions (batch x sequence length collapsed), >= 1 */
  int64_t C;        /* catalogue size, >= 2 */
  int32_t d;        /* embedding dimension: 32, 64, 128 or 256 */
  int32_t n_b;      /* random vectors (buckets) per round, 1..4096 */
  int32_t n_c;      /* RECE chunks, 1..min(s, C); ignored by SCE */
  int32_t n_ec;     /* RECE neighbouring chunks on each side of a window, 0..2^20
                       (1: chunks c-1, c, c+1 as in Algorithm 1); ignored by SCE */
  int32_t k;        /* negatives kept per position (RECE: per round), 0..C-1 */
  int32_t rounds;   /* RECE rounds r, 1..8; SCE: must be 1 */
  int32_t b_x;      /* SCE: positions per bucket, 1..s; RECE: 0 */
  int32_t b_y;      /* SCE: items per bucket, 1..C; RECE: 0 */
  int32_t dtype;    /* rece_dtype of X, Y and B (float32 or bfloat16 bits) */
  int32_t variant;  /* rece_variant */
  int32_t window_wrap; /* RECE: 1 = chunk indices taken modulo n_c (cyclic window),
                          0 = clipped to [0, n_c) (edge chunks see fewer items);
                          ignored by SCE */
  uint32_t flags;   /* RECE_FLAG_* */
} rece_config;

typedef struct rece_plan_s* rece_plan_t;

/* Validate `cfg` and build a host-side plan (no GPU work, no device memory).
 * The plan fixes the workspace layout and the launch shapes of Algorithm 1's
 * steps for this configuration (RECE page, Section 3).  Returns
 * RECE_ERR_INVALID_ARGUMENT for values outside the ranges above and
 * RECE_ERR_UNSUPPORTED for valid values this build does not handle (d, sizes
 * beyond int32 indexing); on error *out is NULL.  A plan may be used from
 * several threads (profiling aside, see rece_profile_enable); concurrent calls
 * need their own scratch and saved buffers.  At its first forward or backward
 * call a plan creates one extra HIP stream (default priority) and a few events
 * on the current device, and uses that device from then on: the item-side steps
 * of the forward, the position-side steps and chunk kernels of rounds after the
 * first, and the dY chain of the backward run there, ordered with `stream` by
 * events, so every result is complete in `stream` order when the call's work
 * is.  Calls that use this stream take a per-plan lock while they enqueue.
 * rece_plan_destroy releases the stream and events (the caller makes sure no
 * call is still running on the device). */
rece_status rece_plan(const rece_config* cfg, rece_plan_t* out);
rece_status rece_plan_destroy(rece_plan_t plan);

/* Plan sizing by the RECE page's rule (Section 3, the sentences on the optimal
 * number of random vectors and on memory complexity), host only:
 *   n_b* = sqrt(4 alpha_bc (1 + 2 n_ec) min(C, s))   (s = batch x sequence length,
 *          alpha_bc = n_b / n_c), rounded to the nearest integer, at least 1;
 *   n_c  = n_b* / alpha_bc, rounded, at least 1;
 *   model_elems = 2 r sqrt(alpha_bc (1 + 2 n_ec) min(C, s)) max(C, s), the page's
 *          peak-memory model (elements of the method's intermediate arrays);
 *   full_ratio  = sqrt(min(C, s)) / (2 r sqrt(alpha_bc (1 + 2 n_ec))), the page's
 *          ratio of full cross-entropy's memory to that model.
 * Any output pointer may be NULL.  Errors: s, C < 1, n_ec < 0, alpha_bc <= 0 or
 * rounds < 1 -> RECE_ERR_INVALID_ARGUMENT. */
rece_status rece_auto_size(int64_t s, int64_t C, int32_t n_ec, double alpha_bc, int32_t rounds, int32_t* n_b,
                           int32_t* n_c, double* model_elems, double* full_ratio);

/* Bytes of the two caller-provided device buffers (owned by the caller):
 *   scratch: temporaries of one call (sorted copies, histograms, the
 *            backward's sorted pairs); may be reused freely between calls;
 *   saved:   written by rece_forward, read by rece_backward / rece_export /
 *            rece_check; must stay untouched in between.
 * Neither holds an [s, C] logit block (RECE page, Section 3: the full logit
 * tensor is what the method avoids). */
rece_status rece_workspace_bytes(rece_plan_t plan, size_t* scratch_bytes, size_t* saved_bytes);

/* Forward pass: RECE page, Section 3, Algorithm 1 (every line, repeated over the
 * rounds, with the duplicate rule of the method paragraph); SCE page, abstract,
 * for the bucket variant.
 *   X    [s][d]  dtype      hidden states, one row per position
 *   Y    [C][d]  dtype      item embeddings
 *   pos  [s]     int32      positive item id of each position, 0 <= pos < C
 *   B    RECE: [rounds][d][n_b] dtype, column b of slice rho is random vector b
 *        of round rho (Algorithm 1's randn line, drawn by the caller);
 *        SCE: [d][n_b]
 *   loss [1]     float32    out: mean loss (Algorithm 1, last line)
 *   loss_pp [s]  float32    out: per-position loss, or NULL
 * Uses (overwrites) scratch and saved.  Errors: NULL or misaligned pointers ->
 * RECE_ERR_INVALID_ARGUMENT, a failed launch -> RECE_ERR_HIP; ids outside [0, C)
 * are clamped and, with RECE_FLAG_VALIDATE_IDS, reported by rece_check. */
rece_status rece_forward(rece_plan_t plan, void* stream, const void* X, const void* Y,
                         const int32_t* pos, const void* B, void* scratch, void* saved,
                         float* loss, float* loss_pp);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): rece_forward with its
 * scratch memory taken from a static device array of the library
 * (RECE_STATIC_SCRATCH_BYTES per GPU, held from the library's first use of that
 * GPU until the process ends) instead of a caller buffer.  The caller still
 * passes the inputs and the outputs (saved, loss, loss_pp; saved feeds
 * rece_backward as usual).  Every launch goes on `stream`: no second stream or
 * event is created, and no device memory is allocated or freed.  A plan whose
 * forward pass needs more scratch than the array holds is rejected with
 * RECE_ERR_WORKSPACE_TOO_SMALL.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (the forward pass clears what it needs
 * cleared): calls that overlap on one GPU race and must be serialised by the
 * caller (one stream, or events).  Results equal rece_forward's. */
#define RECE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
rece_status rece_forward_static(rece_plan_t plan, void* stream, const void* X, const void* Y,
                                const int32_t* pos, const void* B, void* saved, float* loss,
                                float* loss_pp);

/* Backward pass of the last rece_forward that wrote `saved` (same X, Y, pos):
 * RECE page, Section 3, Eq. 4 (softmax minus the one-hot of the positive)
 * restricted to {positive} u the kept set, chained through logit = x . y, with
 * the selection held fixed.
 *   dloss    [1] float32   upstream gradient of the mean loss (ignored if dloss_pp)
 *   dloss_pp [s] float32   upstream gradient of each per-position loss, or NULL
 *   dX [s][d], dY [C][d] float32 (bf16 with RECE_FLAG_BF16_GRADS)   out: overwritten
 *                                  with the gradients (rows of items that no position
 *                                  scored are zero; padding positions' rows are zero
 *                                  under RECE_FLAG_IGNORE_NEGATIVE_POS).
 * Deterministic: no float atomics; two calls give identical bits.  Errors as
 * for rece_forward. */
rece_status rece_backward(rece_plan_t plan, void* stream, const void* X, const void* Y,
                          const int32_t* pos, const float* dloss, const float* dloss_pp,
                          void* scratch, const void* saved, void* dX, void* dY);

/* Exact full cross-entropy over the whole catalogue, the dense loss the reduced
 * ones approximate: RECE page, Section 3, Eq. 3 (loss_i = log sum_j exp(x_i . y_j)
 * - x_i . y_pos(i), mean over positions) and Eq. 4 (its gradient, softmax minus
 * the one-hot of the positive).  Every logit is formed on the matrix cores and
 * consumed on chip; nothing of size s x C is ever stored.  Three sweeps over the
 * s x C logits: log-sum-exp (forward), then dX and dY (backward).
 *   s, C, d, dtype  as in rece_config (d in {32, 64, 128, 256}; dtype RECE_F32 or
 *                   RECE_BF16 for X and Y; float32 accumulation)
 *   X [s][d], Y [C][d], pos [s] (0 <= pos < C, not checked)
 *   workspace       caller-owned device buffer of rece_full_ce_workspace_bytes(s)
 *                   bytes; the forward call leaves each position's log-sum-exp in
 *                   it for the backward call (same X, Y, pos), untouched between
 *   loss [1], loss_pp [s] (or NULL)       forward outputs, float32
 *   dloss [1] / dloss_pp [s] (or NULL)    upstream gradient of the mean loss / of
 *                                         each per-position loss (dloss_pp wins)
 *   dX [s][d], dY [C][d] float32          backward outputs, overwritten
 * Deterministic (no atomics).  Errors: NULL pointers, bad sizes or a workspace
 * smaller than required -> RECE_ERR_INVALID_ARGUMENT / RECE_ERR_WORKSPACE_TOO_SMALL;
 * unsupported d, dtype or sizes -> RECE_ERR_UNSUPPORTED; a failed launch ->
 * RECE_ERR_HIP.  Host work only for the size query. */
rece_status rece_full_ce_workspace_bytes(int64_t s, size_t* bytes);
rece_status rece_full_ce_forward(void* stream, int64_t s, int64_t C, int32_t d, int32_t dtype, const void* X,
                                 const void* Y, const int32_t* pos, void* workspace, size_t workspace_bytes,
                                 float* loss, float* loss_pp);
rece_status rece_full_ce_backward(void* stream, int64_t s, int64_t C, int32_t d, int32_t dtype, const void* X,
                                  const void* Y, const int32_t* pos, void* workspace, size_t workspace_bytes,
                                  const float* dloss, const float* dloss_pp, float* dX, float* dY);

/* Intermediate results kept in `saved` (the steps of Algorithm 1, RECE page,
 * Section 3), copied asynchronously into the caller's `dst`. */
typedef enum {
  RECE_STAGE_BUCKET_X = 0,   /* int32 [s]  bucket of each position (round `round`) */
  RECE_STAGE_BUCKET_Y = 1,   /* int32 [C]  bucket of each item */
  RECE_STAGE_PERM_X = 2,     /* int32 [s]  sorted slot -> position */
  RECE_STAGE_PERM_Y = 3,     /* int32 [C]  sorted slot -> item */
  RECE_STAGE_THRESH_ID = 4,  /* int32 [s]  id of the k-th kept negative; -1 all kept; -2 none */
  RECE_STAGE_THRESH_LOGIT = 5, /* float64 [s] its logit (float64, coordinate-order sum) */
  RECE_STAGE_NEG_IDS = 6,    /* int32 [s][k] kept negatives of round `round`, unordered, -1 padded */
  RECE_STAGE_LSE = 7,        /* float32 [s] log-sum-exp over positive + kept set (round ignored) */
  RECE_STAGE_COUNTERS = 8,   /* uint32 [8] device counters: [0] error bits, [1] argmax rows
                                decided in float64, [2] top-k rows needing float64 values,
                                [3] logits recomputed in float64, [4] buffer overflows,
                                [5] rows whose top-k candidates went through the exact
                                pass (hundreds of ties near the k-th logit), [6] candidate
                                entries appended to the selection lists, [7] SCE: bucket
                                columns whose selection took a finer histogram level */
  RECE_STAGE_SCE_ROWS = 9,   /* SCE: int32 [n_b][b_x] positions taken by each bucket (a set per
                                bucket, in the library's order) */
  RECE_STAGE_SCE_ITEMS = 10, /* SCE: int32 [n_b][b_y] items taken by each bucket (a set per bucket) */
  RECE_STAGE_UNION_IDS = 11  /* int32 [s][rounds*k] per position the union over rounds of the kept
                                negatives, each id once (round order, then list order), -1 padded
                                (round ignored; SCE: rounds = 1) */
} rece_stage;
/* Stages that a plan does not keep (BUCKET_* and PERM_* for SCE, SCE_* for RECE)
 * have 0 bytes; rece_export rejects them.  For SCE, THRESH_*, NEG_IDS and LSE
 * describe the final per-position set (round 0). */

rece_status rece_export(rece_plan_t plan, void* stream, const void* saved, int stage, int round,
                        void* dst);
/* Bytes rece_export writes for (stage); 0 if the stage is not kept by this plan. */
rece_status rece_export_bytes(rece_plan_t plan, int stage, size_t* bytes);

/* Waits for `stream`, then reads the device error word in `saved`:
 * RECE_ERR_DEVICE_CHECK if an id was out of range (with VALIDATE_IDS) or a
 * selection buffer overflowed; RECE_OK otherwise. */
rece_status rece_check(rece_plan_t plan, void* stream, const void* saved);

/* Kernel timing.  rece_profile_enable(plan, mask) with mask != 0 clears earlier
 * records and, from then on, brackets the kernel launches of every phase p with
 * bit p set in mask (mask = -1: all phases) with HIP events recorded on the
 * stream each launch runs on; mask = 0 stops recording.  rece_profile_read
 * waits for the recorded events and returns the total milliseconds and the
 * number of bracketed launches of one phase.  Profiling state is the one mutable
 * part of a plan: do not profile one plan from two threads at once. */
typedef enum {
  RECE_PHASE_PROJECT = 0,   /* bucketing (projection + argmax) */
  RECE_PHASE_SORT = 1,      /* counting sorts (buckets) and sorted copies */
  RECE_PHASE_SELECT = 2,    /* chunk logits + top-k */
  RECE_PHASE_LOSS = 3,      /* round dedup, positive logit, log-sum-exp, mean */
  RECE_PHASE_BWD_DX = 4,    /* backward, dX */
  RECE_PHASE_BWD_DY = 5,    /* backward, dY from the pairs sorted by item */
  RECE_PHASE_BWD_SORT = 6,  /* backward, sort of the (item, position) pairs */
  RECE_PHASE_OTHER = 7,     /* small set-up kernels */
  RECE_NUM_PHASES = 8
} rece_phase;
rece_status rece_profile_enable(rece_plan_t plan, int mask);
rece_status rece_profile_read(rece_plan_t plan, int phase, double* total_ms, int64_t* launches);

const char* rece_status_string(rece_status status);
const char* rece_last_error(void);
const char* rece_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RECE_H_ */
