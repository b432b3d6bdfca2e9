/*
 * libflce: fused LM-head linear + cross-entropy (per-token log-prob, log-sum-exp
 * and optional entropy) for AMD gfx950, forward and backward, without ever
 * materialising the [M, V] logits.
 *
 * The operation (Liger-Kernel commit "native Blackwell tensor-parallel fused
 * scaled linear cross-entropy", section "Summary": the classifier GEMM fused with
 * NLL/LSE and optional entropy; SkyRL PR 2141 "perf(megatron): autotune fused
 * LM-head Triton kernels", sections "Summary"/"Overview": per-token log-probs,
 * optional entropy via compute_entropy, LSE seeded from the true row maximum):
 *
 *   z[m, v]    = scale * sum_k X[m, k] * W[v, k]        bf16 inputs, fp32 accumulation
 *   lse[m]     = log sum_v exp z[m, v]
 *   logprob[m] = z[m, t[m]] - lse[m]
 *   entropy[m] = -sum_v p[m, v] log p[m, v],  p = softmax(z[m, :])
 *
 * A row m is valid iff t[m] != ignore_index and 0 <= t[m] < V.  Invalid rows get
 * logprob = 0 and entropy = 0 (lse is still written) and contribute nothing to
 * the gradients.
 *
 * M = 0 (an empty batch) is accepted everywhere: workspace sizes are 0, the forward
 * calls return FLCE_OK without touching any pointer, and the backward writes dW = 0
 * (the only output with elements).  H and V must be positive.
 *
 * Backward, for a loss L with dL/dlogprob = grad_logprob and dL/dentropy =
 * grad_entropy (Liger-Kernel PR 1294 "Triton MoE improvements and chunked GRPO
 * improvements", "Kernel design notes": logits tiles are recomputed to form
 * grad_logits in the input dtype, then the two grad GEMMs):
 *
 *   dz[m, v] = a[m] (1[v = t[m]] - p[m, v]) + b[m] p[m, v] (E[m] - z[m, v])
 *   a = grad_logprob * valid, b = grad_entropy * valid, E = lse - entropy
 *   dX = scale * dz W,  dW = scale * dz^T X            (bf16 results)
 *
 * Layouts: every matrix is row-major and contiguous.  X is [M, H] bf16, W is
 * [V, H] bf16 (the nn.Linear weight layout, logits = X W^T), targets is [M]
 * int64.  All pointers are device pointers except the size_t outputs of
 * flce_workspace_query.
 *
 * Ownership and ordering: the caller owns every buffer (inputs, outputs and the
 * workspace).  The library never allocates or frees device memory and never
 * synchronises: a call validates its arguments on the host, enqueues kernels on
 * `stream` and returns; results are valid in stream order.  Inputs are never
 * written.  Outputs are overwritten, not accumulated.  Workspace contents are not
 * preserved between calls; forward -> backward state travels only through the
 * caller-held lse and entropy outputs.  Calls on different streams may run
 * concurrently if they use different workspaces and outputs.
 *
 * Errors: return codes only; nothing aborts.  All argument checks happen on the
 * host before any HIP call, so a rejected call enqueues nothing.  After
 * FLCE_ERR_HIP some kernels of the call may already have been enqueued.
 * flce_last_error_message() gives a thread-local description of the last failure.
 */
#ifndef LIBFLCE_FLCE_H
#define LIBFLCE_FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *`; NULL = default stream */

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_VALUE = 1,       /* NULL pointer, size <= 0, bad flag, non-finite scale */
  FLCE_ERR_UNSUPPORTED = 2,         /* H % 8 != 0, pointer not 16-byte aligned, size too large */
  FLCE_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below what the call needs */
  FLCE_ERR_HIP = 4                  /* a HIP launch failed; see flce_last_error_message() */
} flce_status_t;

/*
 * Workspace bytes needed by flce_forward (*fwd_bytes) and the preferred size for
 * flce_backward (*bwd_bytes) for this problem shape.  One buffer of
 * max(*fwd_bytes, *bwd_bytes) serves both.  Either output pointer may be NULL.
 * Sizes accepted by every call: 0 <= M <= 2^30 (M = 0 is an empty batch),
 * 8 <= H <= 2^20 with H % 8 == 0, 1 <= V <= 2^30.  Negative M, or H or V <= 0:
 * FLCE_ERR_INVALID_VALUE; larger sizes, or H not a multiple of 8:
 * FLCE_ERR_UNSUPPORTED.  A dispatch covers at most 2^32 - 1 work-items, so very
 * large problems run in more token waves (and narrower chunks) than the workspace
 * alone would need; *fwd_bytes is the size of the tallest such forward wave.  The
 * one-launch calls (flce_forward_partials and its shard form, flce_forward_merge)
 * return FLCE_ERR_UNSUPPORTED for a batch taller than one launch can take.
 */
flce_status_t flce_workspace_query(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                   size_t* fwd_bytes, size_t* bwd_bytes);

/*
 * Backward workspace.  The backward runs in token waves and vocabulary chunks whose
 * sizes it derives from the workspace it is given (the token-wave scheduling of the
 * Liger-Kernel commit "native Blackwell tensor-parallel fused scaled linear
 * cross-entropy", sections "Summary", "Implementation / Backward" and "Correctness":
 * dW stored by the first wave and added to by later ones; Liger-Kernel PR 1294,
 * "Kernel design notes": d-logits in the input dtype in a reusable buffer).  The
 * workspace holds the bf16 d-logits of one wave over one chunk; an fp32 dX
 * accumulator for one wave's rows when a wave takes more than one chunk; when
 * there is more than one wave, an fp32 dW accumulator of V x H; and 256 bytes of
 * counters with which the d-logit and dW kernels hand out their last tiles.  The preferred size
 * (*bwd_bytes of flce_workspace_query) is one wave of every row with up to 4 GiB of
 * d-logits per chunk (every column at once when they fit).  With less, the call
 * takes the schedule that fits and moves the fewest extra bytes: narrower chunks, or
 * waves of 256 to 16384 rows.  Schedules whose steps (one wave over one chunk) are at
 * most 8e12 FLOP (6 x rows x H x chunk) may also run pipelined when two d-logit
 * buffers fit: one launch per step computes the step's dW and dX together with the
 * next step's d-logits; the same fewest-extra-bytes rule, which counts launches,
 * picks between the kinds.  The minimum is the smallest of: one wave with 256-column
 * chunks (d-logits + fp32 dX accumulator of M rows), one wave with every column
 * (d-logits only), 256-row waves with 256-column chunks or with every column (+ the
 * fp32 dW accumulator): once M > 256 it is at most 4 V H + 1024 H + 131328 bytes (each
 * part rounded up to 256 bytes), whatever M.  Results of different schedules differ
 * only by fp32 summation order (dX across chunks, dW across waves); every schedule is
 * deterministic, and a pipelined schedule gives the same bits as three launches per
 * step with the same waves and chunks.
 */
flce_status_t flce_backward_workspace_min(int64_t M, int64_t H, int64_t V, size_t* bytes);

/* Chunk width (vocabulary columns) flce_backward would use with this workspace;
 * FLCE_ERR_WORKSPACE_TOO_SMALL below the minimum. */
flce_status_t flce_backward_chunk_cols(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                       int64_t* chunk_cols);

/* The whole schedule flce_backward would run with this workspace: token rows per wave,
 * chunk width, and whether it runs pipelined (1: one launch per step, the dW and dX
 * tiles of one step with the d-logit tiles of the next, over two d-logit buffers) or
 * as three launches per step (0).  Any output may be NULL; FLCE_ERR_WORKSPACE_TOO_SMALL
 * below the minimum. */
flce_status_t flce_backward_schedule(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                     int64_t* rows, int64_t* chunk_cols, int* pipelined);

/* Token rows per wave flce_backward would use with this workspace (a multiple of 256;
 * M rounded up to 256 means one wave); FLCE_ERR_WORKSPACE_TOO_SMALL below the minimum. */
flce_status_t flce_backward_wave_rows(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                      int64_t* rows);

/*
 * Smallest workspace flce_forward accepts, and the wave height it uses with a given
 * workspace.  The forward walks the tokens in waves (the token-wave scheduling of
 * the Liger-Kernel commit "native Blackwell tensor-parallel fused scaled linear
 * cross-entropy", sections "Summary" and "Correctness": 4K waves, two-wave tails):
 * a wave is a multiple of 256 rows whose per-tile partials (12 bytes per row per
 * 256 vocabulary columns with entropy, 8 without), target logits (4 bytes per row)
 * and 256 bytes of tile-queue counters fit in the workspace.  The size
 * from flce_workspace_query takes all rows in one wave; the minimum takes 256.
 * Results are bitwise identical for every wave height: a row's tiles and merge do
 * not depend on the wave it falls in.
 */
flce_status_t flce_forward_workspace_min(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                         size_t* bytes);

/* Rows per token wave flce_forward would use with this workspace (a multiple of 256,
 * at most M rounded up to 256); FLCE_ERR_WORKSPACE_TOO_SMALL below the minimum. */
flce_status_t flce_forward_wave_rows(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                     size_t workspace_bytes, int64_t* rows);

/*
 * Forward.  Writes logprob[M], lse[M] and, if compute_entropy == 1, entropy[M]
 * (all fp32).  entropy may be NULL only when compute_entropy == 0.
 * scale is the temperature factor applied to the fp32 accumulator (1/T).
 * workspace: device memory of at least flce_forward_workspace_min bytes (the
 * *fwd_bytes of flce_workspace_query runs every row in one wave), 256-byte aligned.
 */
flce_status_t flce_forward(const void* X, const void* W, const int64_t* targets,
                           int64_t M, int64_t H, int64_t V, int64_t ignore_index, float scale,
                           int compute_entropy, float* logprob, float* lse, float* entropy,
                           void* workspace, size_t workspace_bytes, struct ihipStream_t* stream);

/*
 * flce_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace: the partials go to a static device scratch array of the library, 32 MiB
 * (FLCE_NOALLOC_SCRATCH_BYTES) on each GPU it runs on, held until the process ends,
 * and the token waves are sized to it.  The call allocates and frees nothing; it
 * uses the scratch of the current device, so `stream` must belong to that device.
 * Results are bitwise identical to flce_forward's.  Every value of the scratch a call
 * reads is written earlier in that call, so nothing needs clearing, but the scratch
 * is shared: calls that overlap on one GPU (different streams, or threads) race and
 * must be serialised by the caller.  A vocabulary whose partials of one 256-row wave
 * (12 bytes per 256 columns with entropy, 8 without, per row) exceed the scratch,
 * V above about 2.8M with entropy, is rejected with FLCE_ERR_UNSUPPORTED.  The first
 * call on a device looks the scratch's address up (hipGetSymbolAddress); a failure
 * there is FLCE_ERR_HIP.  Other arguments and errors as flce_forward.
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
flce_status_t flce_forward_noalloc(const void* X, const void* W, const int64_t* targets,
                                   int64_t M, int64_t H, int64_t V, int64_t ignore_index,
                                   float scale, int compute_entropy, float* logprob, float* lse,
                                   float* entropy, struct ihipStream_t* stream);

/*
 * The two halves of flce_forward, for callers that exchange or inspect the
 * per-tile statistics (a vocabulary-sharded caller gathers them across shards
 * before merging).  flce_forward_partials runs the fused GEMM + online-softmax
 * kernel over all rows in one wave (the workspace must hold *fwd_bytes of
 * flce_workspace_query) and leaves in the workspace, for every row m and
 * 256-column vocabulary tile j (j < ceil(V / 256), Mpad = 256 * ceil(M / 256)),
 * at float offsets
 *   j * Mpad + m                       max_v z[m, v] over the tile
 *   (n_vt + j) * Mpad + m              sum_v exp(z[m, v] - max)
 *   (2 n_vt + j) * Mpad + m            sum_v exp(z[m, v] - max) (z[m, v] - max)  (entropy only)
 * and after the 2 (or 3) partial arrays (each rounded up to 256 bytes) the
 * target logit z[m, t[m]] of every valid row (Mpad floats, rounded up to 256 bytes),
 * then the 256 bytes of counters with which the tile kernel hands out its last tiles.  flce_forward_merge turns them into
 * logprob, lse and entropy; its arguments must match the partials call.
 */
flce_status_t flce_forward_partials(const void* X, const void* W, const int64_t* targets,
                                    int64_t M, int64_t H, int64_t V, int64_t ignore_index,
                                    float scale, int compute_entropy, void* workspace,
                                    size_t workspace_bytes, struct ihipStream_t* stream);

flce_status_t flce_forward_merge(const int64_t* targets, int64_t M, int64_t H, int64_t V,
                                 int64_t ignore_index, int compute_entropy, float* logprob,
                                 float* lse, float* entropy, const void* workspace,
                                 size_t workspace_bytes, struct ihipStream_t* stream);

/*
 * Backward.  Recomputes the logits, forms dz and writes dX [M, H] and dW [V, H]
 * in bf16.  lse comes from flce_forward; entropy (from flce_forward with
 * compute_entropy == 1) is required iff grad_entropy != NULL.  grad_logprob and
 * grad_entropy are fp32 [M]; NULL means zero (both NULL writes zero gradients).
 * workspace: at least flce_backward_workspace_min bytes, 256-byte aligned.
 */
flce_status_t flce_backward(const void* X, const void* W, const int64_t* targets,
                            int64_t M, int64_t H, int64_t V, int64_t ignore_index, float scale,
                            const float* lse, const float* entropy,
                            const float* grad_logprob, const float* grad_entropy,
                            void* dX, void* dW,
                            void* workspace, size_t workspace_bytes, struct ihipStream_t* stream);

/*
 * Vocabulary shards (the tensor-parallel split of Liger-Kernel "native Blackwell
 * tensor-parallel fused scaled linear cross-entropy", sections "Summary" and
 * "Implementation": each rank holds a contiguous block of W's rows; SkyRL PR 2141,
 * review of the TP-aware adapter: the rank only shifts vocabulary ids).  A shard is
 * W rows [v_offset, v_offset + V_shard) of a vocabulary of V_total ids; targets stay
 * global ids.  The three calls below are what one rank runs; the exchange between
 * ranks (an all-gather of the partials, a sum of the dX partials) belongs to the
 * caller's communication library.
 *
 * flce_forward_partials_shard: as flce_forward_partials for W_shard [V_shard, H]
 * (the workspace layout is that of flce_forward_partials with V = V_shard; its
 * size is *fwd_bytes of flce_workspace_query(M, H, V_shard, ...)).  The target
 * logit of row m is written only if this shard owns t[m].  v_offset must be in
 * [0, 2^30 - V_shard].
 */
flce_status_t flce_forward_partials_shard(const void* X, const void* W_shard,
                                          const int64_t* targets, int64_t M, int64_t H,
                                          int64_t V_shard, int64_t v_offset,
                                          int64_t ignore_index, float scale, int compute_entropy,
                                          void* workspace, size_t workspace_bytes,
                                          struct ihipStream_t* stream);

/*
 * Merge of the gathered partials of n_shards shards (1 <= n_shards <= 64) into
 * logprob, lse and entropy over the whole vocabulary.  shard_offsets is a HOST
 * array of n_shards + 1 ids: shard r covers [shard_offsets[r], shard_offsets[r + 1]),
 * shard_offsets[0] = 0 and the sequence strictly increases (V_total =
 * shard_offsets[n_shards]).  Shard r's partials, exactly as
 * flce_forward_partials_shard left them, start at byte r * shard_stride_bytes of
 * `gathered` (device memory of n_shards * shard_stride_bytes bytes, 256-byte
 * aligned; the stride is a multiple of 256 and at least every shard's forward
 * workspace size).  Validity uses V_total; the target logit comes from the owning
 * shard.  Results match flce_forward on the whole vocabulary up to fp32 summation
 * order.
 */
flce_status_t flce_forward_merge_shards(const int64_t* targets, int64_t M, int64_t n_shards,
                                        const int64_t* shard_offsets, int64_t ignore_index,
                                        int compute_entropy, float* logprob, float* lse,
                                        float* entropy, const void* gathered,
                                        size_t shard_stride_bytes, struct ihipStream_t* stream);

/* Workspace bytes for flce_backward_shard: the minimum and the preferred size, as
 * for flce_backward but without a dX accumulator (dX_partial is the caller's fp32
 * buffer): d-logits of one wave over one chunk, plus the fp32 dW_shard accumulator
 * when the rows run in more than one wave.  Either output may be NULL. */
flce_status_t flce_backward_shard_workspace_query(int64_t M, int64_t H, int64_t V_shard,
                                                  size_t* min_bytes, size_t* preferred_bytes);

/*
 * Backward of one shard, given the global lse (and entropy) from the merge:
 * writes dW_shard [V_shard, H] bf16 (the shard's rows of dW) and this shard's
 * term of dX, dz_shard W_shard * scale, in fp32 to dX_partial [M, H]: overwritten
 * if accumulate == 0, added to if accumulate == 1 (one GPU can sum several shards
 * in a fixed order this way; across ranks the terms are summed by an all-reduce).
 * dX = sum over shards of dX_partial.  A row is valid iff t[m] != ignore_index and
 * 0 <= t[m] < V_total.  workspace: at least the minimum of
 * flce_backward_shard_workspace_query, 256-byte aligned.
 */
flce_status_t flce_backward_shard(const void* X, const void* W_shard, const int64_t* targets,
                                  int64_t M, int64_t H, int64_t V_shard, int64_t v_offset,
                                  int64_t V_total, int64_t ignore_index, float scale,
                                  const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy,
                                  float* dX_partial, int accumulate, void* dW_shard,
                                  void* workspace, size_t workspace_bytes,
                                  struct ihipStream_t* stream);

/*
 * Scalar cross-entropy reductions over the valid rows of a forward's logprob
 * (the token-level NLL of Liger-Kernel "native Blackwell tensor-parallel fused
 * scaled linear cross-entropy", section "Summary", reduced outside the per-token
 * kernels as SkyRL PR 2141, section "Summary", keeps it).  Writes three fp64
 * values to the device array out: the sum of -logprob[m] over valid rows, the
 * number of valid rows, and their mean (NaN when no row is valid).  One
 * workgroup with a fixed summation order: the result is bitwise repeatable.
 * Validity as in flce_forward (t != ignore_index and 0 <= t < V).
 */
flce_status_t flce_nll_reduce(const float* logprob, const int64_t* targets, int64_t M,
                              int64_t V, int64_t ignore_index, double* out,
                              struct ihipStream_t* stream);

/*
 * dL/dlogprob for L = the mean NLL: grad_logprob[m] = -1/n on valid rows and 0
 * elsewhere, n read on the device from reduced[1] (the out array of
 * flce_nll_reduce), so no host synchronisation is needed; all zeros when n = 0.
 * The result is the grad_logprob argument of flce_backward.
 */
flce_status_t flce_nll_mean_grad(const int64_t* targets, int64_t M, int64_t V,
                                 int64_t ignore_index, const double* reduced,
                                 float* grad_logprob, struct ihipStream_t* stream);

/*
 * Clipped policy-gradient loss on a forward's per-token log-probs, aggregated as a
 * token mean (Liger-Kernel PR 1294, section "Chunked Triton GRPO loss": the loss on
 * top of the fused linear log-probs, settings "Setup" (loss type dapo, clip range
 * eps 0.2/0.2, num_items_in_batch) and per-token outputs "Correctness"; the page
 * gives no formulas, this is the plain clipped-surrogate reading).  Per token m,
 * valid as in flce_forward, in fp64:
 *   r = exp(logprob[m] - old_logprob[m])          (old_logprob NULL: r = 1)
 *   c = min(max(r, 1 - eps_low), 1 + eps_high)
 *   per_token_loss[m] = -min(r A[m], c A[m])      (0 on invalid rows, as fp32)
 *   is_clipped[m]     = c A[m] < r A[m]           (optional output, NULL to skip)
 * and four fp64 values to the device array out: the sum of the per-token loss over
 * valid rows, the number of valid rows, the number of clipped rows, and the loss
 * sum / N with N = denominator if > 0 (the caller's normaliser, e.g. the number of
 * items in the batch), else the number of valid rows; NaN when N is 0.  One
 * workgroup with a fixed summation order: bitwise repeatable.  eps_low and
 * eps_high must be finite and >= 0, denominator finite; all arrays on the device.
 */
flce_status_t flce_policy_loss_reduce(const float* logprob, const float* old_logprob,
                                      const float* advantages, const int64_t* targets,
                                      int64_t M, int64_t V, int64_t ignore_index,
                                      double eps_low, double eps_high, double denominator,
                                      float* per_token_loss, uint8_t* is_clipped, double* out,
                                      struct ihipStream_t* stream);

/*
 * dL/dlogprob of the loss of flce_policy_loss_reduce (same inputs):
 * grad_logprob[m] = -r A[m] / N on valid rows whose minimum takes the unclipped
 * term, 0 on clipped and invalid rows, all zeros when N is 0.  With denominator <= 0,
 * N is read on the device from reduced[1] (the out array of
 * flce_policy_loss_reduce), so no host synchronisation is needed; reduced may be
 * NULL when denominator > 0.  The result is the grad_logprob argument of
 * flce_backward.
 */
flce_status_t flce_policy_loss_grad(const float* logprob, const float* old_logprob,
                                    const float* advantages, const int64_t* targets, int64_t M,
                                    int64_t V, int64_t ignore_index, double eps_low,
                                    double eps_high, double denominator, const double* reduced,
                                    float* grad_logprob, struct ihipStream_t* stream);

/* Static description of a status code. */
const char* flce_status_string(flce_status_t status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* flce_last_error_message(void);

/* Library version as "major.minor.patch". */
const char* flce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFLCE_FLCE_H */
