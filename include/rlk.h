/*
 * rlk.h -- C ABI of the batch-invariant selected-token log-probability
 * library for MI355X (gfx950).  Library: invariant_logprob_amd/librlk.so.
 *
 * What is computed.  For token row i with logits x_i (length V) and target
 * t_i:
 *     lse_i  = log(sum_j exp(x_ij))
 *     logp_i = x_i[t_i] - lse_i
 * and for the backward, with upstream gradient g_i of logp_i:
 *     dlogits_ij = g_i * ([j == t_i] - exp(x_ij - lse_i)).
 * The pages name this operator -- the selected logprob ("logp /
 * batch_invariant_logp") and its fusion with the lm_head projection
 * ("linear_logp") -- in the operator chain of page "docs(ws1):
 * batch-invariance contract RFC", section "First-Divergence Localization",
 * and the dense vs indexed selected-logprob paths of page "[RFC]
 * Batch-Invariant RL Kernel Suite for Train-Inference Consistency", section
 * "Scope"; they do not write the formula, so the textbook definition above is
 * used.  Inputs are bf16, every intermediate and every output is fp32 (page
 * "[WS1 Test] #154 dtype pin + #152 KV path + #153 bwd invariance + #150
 * chain gate", section "Workstream 1 - #154 dtype coverage", scope table:
 * BF16 inputs with FP32 accumulation).
 *
 * Batch invariance.  Each active row's fp32 outputs are bit-identical
 * whatever the number of rows N, the row's position, the content of the
 * other rows, padding rows, varlen packing, or how the rows are split across
 * calls (page "[RFC] ...", maintainer reply, relation I: bitwise, atol = rtol
 * = 0; page "docs(ws1): ...", transform classes T1-T6).  Every reduction has
 * a schedule fixed by V (and H) alone: fixed vocabulary chunks, a fixed
 * wavefront shuffle tree and LDS combine, partials merged in ascending chunk
 * order, and no atomics (page "[WS1 Test] ...", section "Workstream 3 -
 * #153", scope items 2 and 4).  Kernel choice never depends on N.
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers on the current HIP device.
 *    bf16 tensors are passed as raw 16-bit patterns (const void*).
 *  - Row-major layouts with an explicit leading dimension in elements.
 *    bf16 operands need ld % 8 == 0 and a 16-byte aligned base; fp32
 *    gradients need ld_g % 4 == 0 and a 16-byte aligned base.  Otherwise
 *    RLK_ERR_UNSUPPORTED: the column-to-lane map must not depend on
 *    alignment, so misaligned heads are never peeled.
 *  - targets: int64 [N].  mask: uint8 [N], nonzero = active token, NULL =
 *    every row active.  The mask is the sole authority on which rows count
 *    (page "docs(ws1): ...", section "InvarianceFixture": the action mask
 *    defines the active token set).  An inactive row's logits, hidden row
 *    and target are never read for its own outputs; its outputs are +0.0.
 *    An ACTIVE row whose target lies outside [0, V) gets NaN outputs (logp,
 *    and every dlogits entry of that row); nothing is read out of bounds.
 *  - Calls are asynchronous on `stream`; the library never allocates, frees
 *    or synchronises, holds no mutable state, and is reentrant.  The caller
 *    owns every buffer.  Outputs are fully overwritten (no accumulation).
 *  - N == 0 is a no-op returning RLK_OK.  Arguments are validated before any
 *    launch; on error nothing is launched.
 *  - Supported sizes (beyond them RLK_ERR_UNSUPPORTED, before any launch):
 *    N <= 2^31 - 1 and V <= 2^28 everywhere (the row kernels loop over rows
 *    beyond their grid, so any such N is launched, memory permitting);
 *    N * ld < 2^62 for every [N, ld] matrix.  Fused entry points: H <= 2^22
 *    - 8, ld_h, ld_w < 2^22, and ceil(N / 256) * ceil(V / 256) < 2^23 (one
 *    workgroup per 256 x 256 tile, and a launch holds fewer than 2^32
 *    work-items: at V = 151936 that is N up to about 3.6 million rows).
 *    Parameter gradients: N <= 2^22 - 16 and ceil(H / 256) * (ceil(N / 256)
 *    + min(V, 16384) / 256) within the same 2^23-tile launch bound.
 *  - There is no fallback path: the kernels exist for gfx950 only.
 */
#ifndef RLK_H
#define RLK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rlk_status {
  RLK_OK = 0,
  RLK_ERR_INVALID_ARG = 1, /* null required pointer, negative or zero size,
                              ld < V (or < H), workspace too small,
                              lse missing in the backward */
  RLK_ERR_UNSUPPORTED = 2, /* alignment / leading-dimension rule violated,
                              or a size beyond the supported range (see
                              "Supported sizes" above) */
  RLK_ERR_LAUNCH = 3       /* the HIP runtime reported an error at launch */
};

/*
 * Selected-token logprob from materialised logits.
 *   logits : bf16 [N, ld], row-major, ld >= V, ld % 8 == 0, 16-B aligned.
 *   targets: int64 [N].  mask: uint8 [N] or NULL.
 *   logp   : fp32 [N] (required).  lse: fp32 [N] or NULL.
 * One workgroup per row streams its V logits once from HBM; the row's
 * reduction schedule depends on V only.
 */
int rlk_logp_selected(const void* logits, int64_t ld, const int64_t* targets,
                      const uint8_t* mask, int64_t N, int64_t V, float* logp,
                      float* lse, hipStream_t stream);

/*
 * Selected-token logprob and the row's entropy H_i = -sum_j p_ij log p_ij
 * (p = softmax of the row), from one pass over the logits: the entropy's
 * weighted sum sum_j p_ij x_ij rides in the same per-lane state as the
 * log-sum-exp, so H_i = lse_i - sum_j p_ij x_ij with the same fixed reduction
 * schedule (hence the same batch invariance).  A statistic of the dense
 * path: page "[RFC] ...", section "Scope" contrasts dense and indexed
 * selected-logprob paths.
 *   Arguments as rlk_logp_selected; entropy: fp32 [N], required.  Inactive
 *   rows get entropy +0.0.  logp and lse are computed by the same operations
 *   in the same order as in rlk_logp_selected, so they are bit-identical to
 *   its outputs.
 */
int rlk_logp_entropy(const void* logits, int64_t ld, const int64_t* targets,
                     const uint8_t* mask, int64_t N, int64_t V, float* logp,
                     float* lse, float* entropy, hipStream_t stream);

/*
 * Dense log-softmax rows: out[i, j] = x_ij - lse_i, fp32 [N, ld_out]
 * (ld_out >= V, ld_out % 4 == 0, 16-B aligned; columns >= V not written;
 * a span that overlaps the logits' is RLK_ERR_INVALID_ARG),
 * with lse the forward's output for these rows (every log-probability of the
 * row: the dense path of page "[RFC] ...", section "Scope").  Inactive rows
 * are written as +0.0 and their logits are not read.  Elementwise, so each
 * element depends on its own row only.
 */
int rlk_log_softmax(const void* logits, int64_t ld, const uint8_t* mask,
                    const float* lse, int64_t N, int64_t V, float* out,
                    int64_t ld_out, hipStream_t stream);

/*
 * Bytes of device workspace rlk_linear_logp needs for (N, V, H): one
 * (max, sum) fp32 pair per row and 256-wide vocabulary chunk, plus one fp32
 * target logit per row, rounded up to 256 bytes.
 */
size_t rlk_linear_logp_workspace_size(int64_t N, int64_t V, int64_t H);

/*
 * Fused lm_head projection + selected logprob (the pages' "linear_logp"):
 * z_i = W . h_i computed with bf16 MFMA and fp32 accumulation in a fixed K
 * order, never rounded to bf16, reduced by an online log-sum-exp per
 * 256-wide vocabulary chunk; chunk partials are merged per row in ascending
 * chunk order.  A batch of at most 128 rows runs the same per-row instruction
 * sequence in a smaller launch (the same bits as inside a large batch).
 *   hidden : bf16 [N, ld_h], ld_h >= H, ld_h % 8 == 0, 16-B aligned.
 *   weight : bf16 [V, ld_w] (nn.Linear layout, H contiguous), ld_w >= H,
 *            ld_w % 8 == 0, 16-B aligned.  H % 8 == 0.
 *   logp   : fp32 [N] (required).  lse: fp32 [N] or NULL.
 *   workspace: device memory of at least
 *            rlk_linear_logp_workspace_size(N, V, H) bytes, 16-B aligned;
 *            its contents on entry are ignored and on return undefined.
 */
int rlk_linear_logp(const void* hidden, int64_t ld_h, const void* weight,
                    int64_t ld_w, const int64_t* targets, const uint8_t* mask,
                    int64_t N, int64_t V, int64_t H, float* logp, float* lse,
                    void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * rlk_linear_logp for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It takes no workspace: the chunk partials live in a library-owned device
 * array of 32 MiB (one per GPU, held until the process ends), so it
 * allocates nothing and calls no allocating routine.  Arguments, outputs,
 * kernels and results are those of rlk_linear_logp (the outputs are
 * bit-identical to its outputs for the same inputs).
 *   Limit: rlk_linear_logp_workspace_size(N, V, H) <= 32 MiB, otherwise
 *   RLK_ERR_UNSUPPORTED before any launch (up to 7055 rows at V = 151936,
 *   8363 rows at V = 128256).
 *   The array serves the current HIP device (the caller makes the stream's
 *   device current) and is shared by every call on that GPU: two calls that
 *   overlap in time on one GPU (other streams, other host threads) race on
 *   it; calls ordered on one stream are safe.  Nothing in it needs clearing
 *   between calls.  RLK_ERR_LAUNCH if its device address cannot be found.
 */
int rlk_linear_logp_noalloc(const void* hidden, int64_t ld_h,
                            const void* weight, int64_t ld_w,
                            const int64_t* targets, const uint8_t* mask,
                            int64_t N, int64_t V, int64_t H, float* logp,
                            float* lse, hipStream_t stream);

/*
 * Backward of the selected logprob with respect to the logits:
 *   grad_logits[i, j] = grad_logp[i] * ([j == t_i] - exp(x_ij - lse_i)),
 * fp32 [N, ld_g] (ld_g >= V, ld_g % 4 == 0, 16-B aligned); columns >= V are
 * not written.  Inactive rows are written as +0.0.  No reduction is
 * involved, so each element depends only on its own row (page "[WS1 Test]
 * ...", section "Workstream 3 - #153": gradient batch invariance).
 *   Logits mode : `logits` non-NULL (bf16 [N, ld]); hidden/weight ignored.
 *                 A grad_logits span that overlaps the logits' is
 *                 RLK_ERR_INVALID_ARG.
 *   Fused mode  : `logits` NULL; x_i = W . h_i is recomputed with exactly
 *                 the tiles and K order rlk_linear_logp uses (hidden
 *                 [N, ld_h], weight [V, ld_w], H as there); a batch of
 *                 at most 128 rows runs the same per-row instruction
 *                 sequence in a smaller launch (the same bits).
 *   lse        : fp32 [N], required -- the forward's output for these rows.
 *   grad_logp  : fp32 [N], required (the upstream gradient g).
 */
int rlk_logp_backward(const void* logits, int64_t ld, const void* hidden,
                      int64_t ld_h, const void* weight, int64_t ld_w,
                      int64_t H, const int64_t* targets, const uint8_t* mask,
                      const float* lse, const float* grad_logp, int64_t N,
                      int64_t V, float* grad_logits, int64_t ld_g,
                      hipStream_t stream);

/*
 * The fused forward of rlk_linear_logp that also keeps its fp32 logits, for
 * callers that trade N x V x 4 bytes of device memory for a backward without
 * the second projection (the pages' "linear_logp" with its backward, as in
 * rlk_logp_backward's fused mode; page "[WS1 Test] ...", section
 * "Workstream 3 - #153").  logp, lse and the workspace are exactly as in
 * rlk_linear_logp, and logp and lse are bit-identical to its outputs.
 *   logits : fp32 [N, ld_z] (ld_z >= V, ld_z % 4 == 0, 16-B aligned), caller
 *            owned: z_ij = W_j . h_i for every row i < N, masked or not (the
 *            projection does not read the mask), columns j < V; columns
 *            >= V are not written.  Each value is bit-identical to the
 *            logit the fused backward recomputes for that element.
 */
int rlk_linear_logp_with_logits(const void* hidden, int64_t ld_h,
                                const void* weight, int64_t ld_w,
                                const int64_t* targets, const uint8_t* mask,
                                int64_t N, int64_t V, int64_t H, float* logp,
                                float* lse, float* logits, int64_t ld_z,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Backward of the selected logprob from fp32 logits (normally those
 * rlk_linear_logp_with_logits kept):
 *   grad_logits[i, j] = grad_logp[i] * ([j == t_i] - exp(x_ij - lse_i)),
 * with the per-element arithmetic of rlk_logp_backward's fused mode, so
 * that for the same logits and lse the two outputs are bit-identical.
 *   logits      : fp32 [N, ld] (ld >= V, ld % 4 == 0, 16-B aligned); rows
 *                 hold ld elements; inactive rows are not read.
 *   grad_logits : fp32 [N, ld_g], same constraints; columns >= V are not
 *                 written; inactive rows are written as +0.0.  It may be
 *                 `logits` itself with ld_g == ld (in place); any other
 *                 overlap of the two is RLK_ERR_INVALID_ARG.
 *   lse, grad_logp, targets, mask: as in rlk_logp_backward.  An active row
 *                 with a target outside [0, V) gets NaN in every entry.
 */
int rlk_logp_backward_f32(const float* logits, int64_t ld,
                          const int64_t* targets, const uint8_t* mask,
                          const float* lse, const float* grad_logp, int64_t N,
                          int64_t V, float* grad_logits, int64_t ld_g,
                          hipStream_t stream);

/*
 * Bytes of device workspace rlk_linear_logp_param_grads needs for (N, V, H):
 * one vocabulary chunk of the logits gradient as two bf16 arrays (its bf16
 * rounding and the rounding's remainder), each [N, C] with C = min(16384, V
 * rounded up to 256), then a bf16 [N, H] copy of hidden with the inactive
 * rows zeroed (used when a mask is given, so that an inactive row's
 * contents, whatever they are, add nothing to grad_weight), each part
 * rounded up to 256 bytes.
 */
size_t rlk_linear_logp_param_grads_workspace_size(int64_t N, int64_t V,
                                                  int64_t H);

/*
 * Parameter gradients of the fused path: with D the gradient of
 * sum_i g_i logp_i with respect to the logits z = W . h_i (rlk_logp_backward,
 * fused mode),
 *     grad_hidden = D . W   fp32 [N, ld_gh]      (nullable)
 *     grad_weight = D^T . h fp32 [V, ld_gw]      (nullable; not both NULL)
 * (page "[WS1 Test] ...", section "Workstream 3 - #153": gradients keep the
 * invariance contract; parameter gradients are compared over the same
 * complete sample set).  D is never held whole: the vocabulary is walked in
 * fixed chunks of 16384 entries; per chunk the logits are recomputed with
 * exactly the forward's tiles and K order and D is formed in fp32 as in
 * rlk_logp_backward.  The products run on bf16 MFMA with fp32 accumulation
 * (bf16 inputs, fp32 accumulation: page "[WS1 Test] ...", section
 * "Workstream 1 - #154", scope table), so D enters as two bf16 operands,
 * D_hi = bf16(D) and D_lo = bf16(D - D_hi), whose sum holds D to a relative
 * 2^-16; each product is two passes over its K (D_hi, then D_lo) into the
 * same fp32 accumulators.  W, hidden and D are contracted over their rows by
 * reading them through transposing LDS loads, so nothing is transposed in
 * memory.
 *   grad_hidden: chunk partial products are added in ascending chunk order,
 *     so each row depends on its own token only and is bit-identical for any
 *     batch composition.  Inactive rows are +0.0.
 *   grad_weight: a sum over all active tokens in ascending row order,
 *     deterministic for a given batch (not batch-invariant by nature).
 *     An active row with an invalid target makes it NaN.
 *   hidden, weight, targets, mask, lse (the forward's), grad_logp, H: as in
 *   rlk_logp_backward's fused mode.  ld_gh >= H and ld_gw >= H, both % 4 ==
 *   0 with 16-B aligned bases.  N must stay below 2^22 - 16.
 *   workspace: >= rlk_linear_logp_param_grads_workspace_size(N, V, H) bytes,
 *   16-B aligned; contents on entry ignored, on return undefined.
 *   N == 0: grad_weight (if given) is set to zero; nothing else is read.
 */
int rlk_linear_logp_param_grads(const void* hidden, int64_t ld_h,
                                const void* weight, int64_t ld_w,
                                const int64_t* targets, const uint8_t* mask,
                                const float* lse, const float* grad_logp,
                                int64_t N, int64_t V, int64_t H,
                                float* grad_hidden, int64_t ld_gh,
                                float* grad_weight, int64_t ld_gw,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * rlk_linear_logp_param_grads from the fp32 logits the forward kept
 * (rlk_linear_logp_with_logits): each vocabulary chunk's logits gradient is
 * formed from `logits` [N, ld_z] (ld_z >= V, ld_z % 4 == 0, 16-B aligned;
 * inactive rows are not read) instead of being recomputed, with the same
 * arithmetic, so grad_hidden and grad_weight are bit-identical to
 * rlk_linear_logp_param_grads' for logits that function would recompute.
 * hidden is still read (grad_weight = D^T . hidden).  Every other argument,
 * the workspace and the error codes are as there; logits NULL with N > 0 is
 * RLK_ERR_INVALID_ARG.
 */
int rlk_linear_logp_param_grads_from_logits(const float* logits, int64_t ld_z,
                                            const void* hidden, int64_t ld_h,
                                            const void* weight, int64_t ld_w,
                                            const int64_t* targets,
                                            const uint8_t* mask, const float* lse,
                                            const float* grad_logp, int64_t N,
                                            int64_t V, int64_t H,
                                            float* grad_hidden, int64_t ld_gh,
                                            float* grad_weight, int64_t ld_gw,
                                            void* workspace,
                                            size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * Per-token loss terms consuming the selected logprob (the chain's last
 * entry, grpo_loss / ratio_kl, as per-token outputs so that each token's
 * values cannot depend on the batch: page "docs(ws1): ...", section
 * "First-Divergence Localization").  The pages give no formula; the textbook
 * GRPO / PPO terms are used, per token i:
 *   ratio = exp(logp - logp_old)
 *   surr  = -min(ratio A, clip(ratio, 1 - eps_lo, 1 + eps_hi) A)
 *   kl    = exp(ref - logp) - (ref - logp) - 1          (k3 estimator)
 *   loss  = surr + beta kl
 *   grad  = d loss / d logp   (the clipped branch, where min() picks it,
 *                              contributes 0; feed it to rlk_logp_backward)
 *   logp, logp_old, advantages: fp32 [N], required.  logp_ref: fp32 [N] or
 *   NULL (then kl = 0 and beta is unused).  mask: uint8 [N] or NULL.
 *   eps_lo in [0, 1), eps_hi >= 0, beta >= 0.
 *   ratio, loss, kl, grad_logp: fp32 [N] outputs, each nullable (at least
 *   one required).  Masked tokens get +0.0 in every output.
 */
int rlk_token_losses(const float* logp, const float* logp_old,
                     const float* logp_ref, const float* advantages,
                     const uint8_t* mask, int64_t N, float eps_lo, float eps_hi,
                     float beta, float* ratio, float* loss, float* kl,
                     float* grad_logp, hipStream_t stream);

/*
 * Static string naming a status code ("RLK_OK", ...); "unknown" otherwise.
 * A gate report states the reason when the requested backend did not run
 * (page "[WS1 Test] ...", section "Workstream 4 - #150", gate report
 * contents: requested / actual backend, fallback reason); this is the name
 * such a report carries for a failed call.  Never allocates; thread-safe.
 */
const char* rlk_status_string(int status);

/*
 * Static string describing this build: library version, target
 * architecture, source revision and the schedule constants that fix every
 * reduction order (row threads and vectors per step, tile shape, K stage,
 * chunk sizes).  It is the "actual backend" a gate report records beside the
 * requested one (same page and section as rlk_status_string), and
 * invariance records carry it, since bits are only promised stable within
 * one build (the pages' relation I compares a kernel with itself).  Never
 * allocates; thread-safe; the string lives as long as the library.
 */
const char* rlk_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H */
