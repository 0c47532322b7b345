/*
 * lite_attn.h - C ABI of an MI355X (gfx950) implementation of LiteAttention's hot path:
 * tiled self-attention with an embedded QK-Skip test and a persistent skip mask that
 * carries across denoising steps.
 *
 * Method: "LiteAttention: Temporal Sparse Attention for Diffusion Transformers"
 * (page 1, sections "Core Concept", "Architecture Overview"; page 2, abstract).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors q, k, v and out have logical shape [B][H][N][D] with element strides
 *   (stride_b, stride_h, stride_n) and a contiguous last dimension; all four share the
 *   strides given in lite_attn_config. They are device pointers owned by the caller.
 * - The skip mask is a caller-owned device array of uint32 words, shape [B][H][Tq][W] with
 *   Tq = ceil(N / tile_q), Tk = ceil(N / tile_k), W = ceil(Tk / 32). Key tile j of query
 *   tile i of head (b, h) is bit (j % 32) of word mask[b][h][i][j / 32]; a set bit means
 *   "skip". Bits at positions >= Tk of a row's last word are reserved: they must be zero and
 *   are never read or changed. Keep one mask per attention call site (per layer, per
 *   guidance branch) and pass it to every denoising step of a generation.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream). All device work
 *   is enqueued asynchronously on it; nothing here synchronises with the host. Errors that
 *   happen during kernel execution surface at the caller's next synchronisation.
 * - Return values are lite_attn_status codes. No C++ exception crosses this interface.
 *   The message for the most recent failing call on the calling thread is available from
 *   lite_attn_last_error().
 * - A handle holds only the validated configuration; it owns no device memory. Steps on the
 *   same handle may run concurrently on different streams when their out and mask buffers
 *   differ.
 * - bf16 steps run as persistent launches: a grid of as many workgroups as the device holds
 *   at once takes query tiles from a tile queue, a pair of uint32 in the library's static
 *   device memory. Launches that share a queue must not overlap, so queues are handed out
 *   this way:
 *   - an eager step uses the queue of its (device, stream) pair: each of up to 64 streams per
 *     device is given one on first use and keeps it (steps on one stream run in order);
 *   - a step captured into a HIP graph is given a queue of its own (up to 4032 captured steps
 *     per device over the life of the process), so a graph may be replayed on any stream,
 *     concurrently with other steps that use other masks;
 *   - without a queue (more than 64 streams, more captured steps than queues, the per-thread
 *     default stream, or a stream of a device other than the current one) a step launches
 *     one workgroup per query tile instead, with the same results.
 *   Each launch leaves its queue at zero when it ends. A stream must not be destroyed while
 *   its steps are still running (its handle value could then be reused by a new stream while
 *   the queue is in use). lite_attn_last_launch() reports how the last step was launched.
 */
#ifndef LITE_ATTN_H
#define LITE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LITE_ATTN_ABI_VERSION 2

typedef enum lite_attn_status {
  LITE_ATTN_OK = 0,
  LITE_ATTN_ERR_INVALID_ARG = 1,  /* bad pointer, alignment, size, NaN/positive budget ... */
  LITE_ATTN_ERR_UNSUPPORTED = 2,  /* valid request, but no kernel is built for it */
  LITE_ATTN_ERR_HIP = 3,          /* a HIP runtime call failed (launch, device query) */
  LITE_ATTN_ERR_NO_MEMORY = 4     /* host allocation of the handle failed */
} lite_attn_status;

typedef enum lite_attn_dtype {
  LITE_ATTN_BF16 = 0,  /* q, k, v, out are bfloat16; MFMA in bf16 with fp32 accumulation */
  LITE_ATTN_FP32 = 1   /* q, k, v, out are float32; MFMA in fp32 */
} lite_attn_dtype;

typedef enum lite_attn_order {
  /* Key tiles of a query tile are visited in ascending index order at every step. */
  LITE_ATTN_ORDER_ASC = 0,
  /* Ascending on even steps, descending on odd steps. The QK-Skip test compares a tile with
   * the maximum over tiles visited before it, so alternating the direction lets tiles on both
   * sides of a query's high-score region be flagged. */
  LITE_ATTN_ORDER_ALT = 1
} lite_attn_order;

typedef enum lite_attn_option {
  /* In-step skip. A tile that the QK-Skip test flags while it is visited is also left out of
   * this step's own output (its exponentials and PV product are not computed), instead of
   * only from the next step on. The flags, and so the mask after the step, are unchanged (a
   * flagged tile lies below the running maximum, so leaving it out does not move that
   * maximum); the output becomes softmax attention over the tiles still clear in the mask
   * after the step. The left-out softmax mass of a row is at most (left-out columns) times
   * exp(log_eps_t). LiteAttention, page 1 "Architecture Overview": the skip logic sits inside
   * the FlashAttention softmax pipeline. */
  LITE_ATTN_OPT_IN_STEP_SKIP = 1u
} lite_attn_option;

typedef struct lite_attn_config {
  int32_t abi_version;   /* must be LITE_ATTN_ABI_VERSION */
  int32_t batch;         /* B >= 0 */
  int32_t heads;         /* H >= 0 */
  int32_t seq_len;       /* N >= 0; tokens per head (queries and keys: self-attention) */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t tile_q;        /* query rows per tile: 64 or 128 */
  int32_t tile_k;        /* keys per tile: 64 */
  int32_t dtype;         /* lite_attn_dtype; in and out share it */
  float softmax_scale;   /* > 0; a value <= 0 selects 1/sqrt(head_dim) */
  int32_t order;         /* lite_attn_order */
  int32_t dense_prefix;  /* tokens [0, dense_prefix) keep dense attention: a tile whose rows
                            or columns touch them is never flagged. 0 = off; <= seq_len */
  int64_t stride_b;      /* element strides shared by q, k, v, out; all three zero selects */
  int64_t stride_h;      /* the contiguous layout [B][H][N][D]. Each must be a multiple of */
  int64_t stride_n;      /* 8 elements (16 bytes); head_dim <= stride_n < 2^24.            */
  uint32_t options;      /* OR of lite_attn_option flags; 0 = the plain method */
  uint32_t reserved;     /* must be 0 */
} lite_attn_config;

typedef struct lite_attn_s* lite_attn_t;

/* Validate `cfg` and create a handle (host memory only; no device call).
 * LiteAttention, page 1 "Architecture Overview": the Skip-Mask bitmask and QK-Skip.
 * Returns INVALID_ARG for NULL arguments, a wrong abi_version, negative sizes, strides that
 * are not multiples of 8 elements, strides under which two (b, h, n) rows of out would overlap
 * (out is written through the shared strides), dense_prefix outside [0, seq_len], unknown
 * option bits or a nonzero reserved field; UNSUPPORTED for a
 * head_dim / tile / dtype combination without a kernel, for Tk > 2048 (N > 131072 with
 * 64-key tiles), and, for bf16, when one head's rows span 2^31 bytes or more
 * ((N - 1) * stride_n * 2 + head_dim * 2). On failure *out is set to NULL. */
int lite_attn_create(const lite_attn_config* cfg, lite_attn_t* out);

/* Release a handle. NULL is accepted. Returns OK. */
int lite_attn_destroy(lite_attn_t handle);

/* Bytes of the skip mask for this handle: B * H * Tq * W * 4 (0 for a NULL handle). */
size_t lite_attn_mask_bytes(lite_attn_t handle);

/* Mask geometry (Tq, Tk, W) of this handle. Any output pointer may be NULL. */
int lite_attn_mask_geometry(lite_attn_t handle, int32_t* tiles_q, int32_t* tiles_k,
                            int32_t* words_per_row);

/* One denoising step of attention over all (b, h), using and updating the skip mask.
 *
 * LiteAttention, page 1 "Core Concept" (tiles flagged when their local maximum QK score is
 * far below the cumulative maximum; the mask carries across steps) and "Architecture
 * Overview" (bitmask, QK-Skip, per-step error budgets, skip logic inside the FlashAttention
 * softmax pipeline, persistent propagation); page 2 abstract (decisions made early and
 * propagated forward).
 *
 * For every query tile i of every head, key tiles whose mask bit is set are skipped: their
 * K/V are not loaded and no score is computed. The remaining tiles are visited in this
 * step's order (see lite_attn_order; `step` selects the parity) and out receives exact
 * softmax attention over them (scale = softmax_scale), rows with no visited tile receive 0.
 * Each visited tile j is tested: with mt[r] its scaled row maxima and m[r] the running row
 * maxima over tiles visited before it, the tile is flagged when mt[r] - m[r] < log_eps_t for
 * every valid row r of the tile and the tile is not exempt (dense_prefix). Flagged bits are
 * OR-ed into `mask` when the query tile finishes (they take effect from the next step, or,
 * with LITE_ATTN_OPT_IN_STEP_SKIP, already leave this step's output); no bit is ever cleared
 * by this call.
 *
 * q, k, v: read-only device tensors (see conventions); out: device tensor written for every
 * valid row, must not alias q, k or v; mask: device words read and updated in place.
 * log_eps_t: the step's error budget in natural-log units, in [-inf, 0]; -inf flags nothing.
 * step: the denoising step index (>= 0), used only for the traversal parity.
 * Pointers must be 16-byte aligned (mask: 4-byte). Returns INVALID_ARG for NULL or misaligned
 * pointers, out aliasing an input, NaN or positive log_eps_t, negative step; HIP when the
 * launch fails. A configuration with B*H*N == 0 returns OK without launching anything. */
int lite_attn_step(lite_attn_t handle, const void* q, const void* k, const void* v, void* out,
                   uint32_t* mask, float log_eps_t, int32_t step, void* stream);

/* lite_attn_step with divergence-triggered refresh of mask rows. LiteAttention, page 1
 * "Core Concept" (the mask is updated only when the attention pattern diverges significantly)
 * and "Architecture Overview" (decisions carry forward unless the attention distribution
 * shifts significantly).
 *
 * tile_stats: caller-owned device float array [B][H][Tq] (same tile order as the mask), one
 * reference per query tile; NaN means "no reference" (fill it with NaN when a generation
 * starts, together with lite_attn_reset_mask). After the tile loop each query tile computes
 * its statistic: the mean over its valid rows of the largest scaled score over the key tiles it
 * computed (the running row maximum). If the reference is NaN, the statistic becomes the
 * reference and the mask row is updated as in lite_attn_step. Otherwise, if the statistic has
 * moved by more than refresh_delta from the reference (or the move is NaN), the reference is set
 * to NaN and the row's mask bits are all cleared, so the next step computes the row densely and
 * flags afresh; else the row is updated as usual and the reference kept. A row maximum falls
 * when attention moves into skipped tiles, which the mask alone cannot notice. With this call
 * bits can clear; refresh_delta = +inf never clears (the mask evolves as with lite_attn_step).
 * The output of the step is that of lite_attn_step (the refresh acts on the mask only).
 * Returns what lite_attn_step returns, and INVALID_ARG for a NULL or misaligned tile_stats or a
 * negative or NaN refresh_delta. */
int lite_attn_step_refresh(lite_attn_t handle, const void* q, const void* k, const void* v,
                           void* out, uint32_t* mask, float* tile_stats, float refresh_delta,
                           float log_eps_t, int32_t step, void* stream);

/* Bytes of device workspace that lite_attn_step_scheduled needs: about 6 * B * H * Tq, in
 * 256-byte units (0 for a NULL handle). */
size_t lite_attn_workspace_bytes(lite_attn_t handle);

/* lite_attn_step with a schedule from the tiles' visit counts (heavy first, short last): same
 * arguments, same results (bit for bit), plus a caller-owned device `workspace` of
 * lite_attn_workspace_bytes(handle) bytes, 256-byte aligned, that the call overwrites (it holds
 * nothing between calls). A first kernel reads the
 * mask and counts, per query tile, the key tiles it will visit (its skip-list length). Query
 * tiles that visit at least half of all key tiles and at least four times the mean (dense
 * prefix rows in a sparse step, for example) are scheduled first. The shortest tiles go last,
 * in the step's traversal order: the non-heavy tiles whose list is shorter than a cut, the
 * largest cut that leaves at most min(16 * compute units, non-heavy tiles / 4) of them. The
 * other tiles run in between, head by head, heads in decreasing order of their work (with more
 * than 1024 heads, in natural order), each head's tiles in the direction of the step's key
 * traversal, which keeps neighbouring query tiles together. The attention kernel then runs its
 * workgroups in that order, so that long work starts early and the step ends on short tiles. LiteAttention, page 1 "Architecture Overview": the skip list used at high sparsity;
 * here its list lengths drive the schedule. Calls that share a workspace must be ordered on
 * one stream. Returns what lite_attn_step returns, and INVALID_ARG for a NULL or misaligned
 * workspace. */
int lite_attn_step_scheduled(lite_attn_t handle, const void* q, const void* k, const void* v,
                             void* out, uint32_t* mask, float log_eps_t, int32_t step,
                             void* workspace, void* stream);

/* lite_attn_step_scheduled without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments as lite_attn_step_scheduled less `workspace`, same results bit
 * for bit. The workspace is a 1 MiB array in the library's static device memory, one per
 * device, held until the process ends; this call allocates nothing. It holds the schedule of
 * up to about 174,000 query tiles (B * H * ceil(N / tile_q)); larger problems return
 * UNSUPPORTED (lite_attn_workspace_bytes(handle) > 1 MiB) without any device call. The array's
 * address is looked up on the first call on each device, with that device current. Every call
 * on a device shares the one array and leaves its contents behind (nothing in it needs to
 * start at zero): calls that overlap on one device race, so order them, for example on one
 * stream. `stream` must belong to the current device (INVALID_ARG otherwise). Returns what
 * lite_attn_step_scheduled returns, and HIP when the array's address cannot be taken. */
int lite_attn_step_scheduled_static(lite_attn_t handle, const void* q, const void* k,
                                    const void* v, void* out, uint32_t* mask, float log_eps_t,
                                    int32_t step, void* stream);

/* Clear every word of `mask` (a new generation starts dense). LiteAttention, page 1
 * "Architecture Overview": decisions persist until the attention distribution shifts; this
 * is the explicit way to drop them. Uses a fill kernel (no memset node), so it may be
 * recorded into a HIP graph. Returns INVALID_ARG for a NULL handle or mask. */
int lite_attn_reset_mask(lite_attn_t handle, uint32_t* mask, void* stream);

/* Count skipped tiles per head: counts[b * H + h] = number of set bits (reserved bits
 * excluded) in mask[b][h]. `counts` is a device array of B*H uint32 words written on `stream`.
 * The skipped-tile fraction of the step that uses this mask is sum(counts) / (B*H*Tq*Tk).
 * Returns INVALID_ARG for NULL pointers. */
int lite_attn_mask_popcount(lite_attn_t handle, const uint32_t* mask, uint32_t* counts,
                            void* stream);

/* Largest absolute difference between two outputs of this handle: *result (a device float
 * written on `stream`) = max over every valid element (b, h, n, d < head_dim) of |a - b|, each
 * difference taken in float32 after widening bf16 exactly; NaN when any difference is NaN, 0
 * when B*H*N == 0. a and b are read through the handle's strides and dtype, like out; the
 * memory between rows is not read. This is the output error that the per-step budgets of
 * lite_attn_calibrate bound. LiteAttention, page 1 "Architecture Overview" (accumulated-error
 * calibration). Pointers 16-byte aligned (result: 4-byte). Returns INVALID_ARG for NULL or
 * misaligned pointers, HIP when a launch fails. */
int lite_attn_output_max_abs_diff(lite_attn_t handle, const void* a, const void* b,
                                  float* result, void* stream);

/* Bytes of device workspace that lite_attn_calibrate needs: four outputs under the handle's
 * strides, two masks and one result word, each part rounded up to 256 bytes (0 for a NULL
 * handle). */
size_t lite_attn_calibrate_workspace_bytes(lite_attn_t handle);

/* Choose the per-step error budgets log_eps_t from per-step output-error limits.
 * LiteAttention, page 1 "Architecture Overview": each denoising step gets its own error budget
 * from accumulated-error calibration, early steps tolerating less error.
 *
 * The flags of step t first change the output of step t+1. So, for t < steps - 1, log_eps[t]
 * receives the loosest of `candidates` (largest first) whose flags, OR-ed into the mask carried
 * from steps 0..t-1, keep the error of step t+1's output against dense attention within
 * error_budgets[t + 1]; -inf (flag nothing) when none does. The last step's flags change no
 * output: it keeps the previous step's choice (-inf when steps == 1). The error is
 * lite_attn_output_max_abs_diff of the step's output against that of the same step with an
 * empty mask, and errors[t] receives the error of step t under the chosen schedule (step 0's is
 * 0: its mask is empty). The mask starts empty and accumulates every flag since step 0, as in a
 * generation. Each step runs as lite_attn_step with this handle (its order, dense prefix and
 * options), step index t.
 *
 * q, k, v: host arrays of `steps` device pointers, step t's inputs (each as for
 * lite_attn_step). error_budgets: host array of `steps` limits (not NaN; error_budgets[0] is
 * not used). candidates: host array of n_candidates values in [-inf, 0] (duplicates are
 * dropped; may be NULL when n_candidates == 0, and then every step gets -inf). log_eps, errors:
 * host arrays of `steps` floats, written. workspace: lite_attn_calibrate_workspace_bytes(handle)
 * bytes of device memory, 256-byte aligned, overwritten (it may be NULL when B*H*N == 0).
 * The call runs on `stream` and waits for it after every error it measures, so it blocks the
 * host and the stream must not be capturing (INVALID_ARG). It runs about
 * steps * (2 + 2 * tried candidates) attention steps. Returns INVALID_ARG for NULL or misaligned
 * arguments, negative steps or n_candidates, a NaN budget, a NaN or positive candidate;
 * otherwise what the steps and reductions return. */
int lite_attn_calibrate(lite_attn_t handle, const void* const* q, const void* const* k,
                        const void* const* v, int32_t steps, const float* error_budgets,
                        const float* candidates, int32_t n_candidates, float* log_eps,
                        float* errors, void* workspace, void* stream);

/* Static English name of a status code. */
const char* lite_attn_status_string(int status);

/* Message describing the most recent failure on the calling thread ("" if none). */
const char* lite_attn_last_error(void);

/* How the calling thread's most recent step call launched its attention kernel (diagnostics):
 * *workgroups receives the grid size and *queue the tile queue it used, -1 when it took one
 * workgroup per query tile without a queue (see the conventions above). Before any launch on
 * the thread: 0 and -1. Either pointer may be NULL. Always returns OK. */
int lite_attn_last_launch(int32_t* workgroups, int32_t* queue);

#ifdef __cplusplus
}
#endif

#endif /* LITE_ATTN_H */
