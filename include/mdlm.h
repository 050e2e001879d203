/*
 * mdlm.h -- C ABI of the masked-diffusion loss library for AMD MI355X (gfx950).
 *
 * The library computes the training objective of masked-diffusion language
 * models on one GPU, in three calls that a trainer makes each step:
 *
 *   mdlm_corrupt                 per-document noise level t, then per-token
 *                                corruption (absorbing mask or uniform ids);
 *   mdlm_compact_masked          ascending list of scored rows with their
 *                                targets and 1/p weights;
 *   mdlm_fused_head_ce_fwd_bwd   frozen LM head + cross-entropy over the full
 *                                vocabulary, weighted and summed to a scalar
 *                                loss, plus the gradient with respect to the
 *                                hidden states, without writing logits to
 *                                memory.
 *
 * Loss variants replace the first two calls: mdlm_compact_rows (every-token
 * causal rows, an eligibility mask, other weightings) and the corrective
 * mixture's mdlm_corrupt_mixture + mdlm_compact_corrective;
 * mdlm_fused_head_ce_fwd_bwd_dw adds the head's own gradient.
 *
 * The method is defined on these pages:
 *   - LLaDA-8B-MDLM-LoRA model card, "Training" table, "Objective" row:
 *     one t ~ U(0,1) for each sequence, masking probability
 *     p = (1 - 1e-3) t + 1e-3, and the CE of each masked token scaled by
 *     1/p; "LoRA" row: embeddings and output layer frozen.
 *   - diffusiongemma-26B-A4B-it-ALWAYS-THINK, "Finetuning notes": corrupted
 *     canvas positions take uniformly drawn vocabulary ids, each example
 *     with its own rate t ~ U(eps, 1) (no mask token); the logit softcap
 *     acts once.
 *   - Native diffusion language-model training (Axolotl docs): model table
 *     (aligned vs shifted logits, CE weighted by the inverse noise level),
 *     "Attention backends" (cumulative document offsets), "Packed training"
 *     (documents isolated, padding excluded from loss), "Adapters, merging
 *     and inference" (CE over the whole vocabulary taken from the hidden
 *     states through a bare linear head, no logits tensor stored).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or retains device memory; scratch space is passed
 *     in as `workspace`.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream).  Outputs are valid once the stream
 *     reaches the call.  No call synchronises with the host.
 *   - Calls only launch kernels (no memset, no allocation), so a sequence of
 *     them may be captured in a HIP graph; a replay reuses the host arguments
 *     (seed, sizes, weights) given at capture, and the device data as it is
 *     at replay.
 *   - Host-side argument checks run first.  If one fails the call returns a
 *     non-zero status, enqueues nothing and records a message readable
 *     through mdlm_last_error().  Launch failures return MDLM_EHIP.
 *   - Output buffers must not overlap the inputs or one another (mdlm_corrupt,
 *     for one, uses xt's memory for its own bookkeeping before it writes the
 *     tokens there).
 *   - Device-resident data is not inspected on the host.  Preconditions on it
 *     (cu_seqlens nondecreasing from 0 to n_tokens, token and target ids in
 *     range) are the caller's responsibility; violating them gives
 *     unspecified results but never out-of-bounds writes to outputs.
 *   - Calls hold no global mutable state apart from a thread-local error
 *     string, and may be made concurrently from several host threads on
 *     different streams.  Calls on one stream that share a workspace must not
 *     overlap (they do not on one stream).
 */
#ifndef MDLM_H
#define MDLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MDLM_OK = 0,
  MDLM_EINVAL = 1,       /* bad argument (null pointer, size, range, enum) */
  MDLM_EUNSUPPORTED = 2, /* valid but unsupported shape or dtype           */
  MDLM_EWORKSPACE = 3,   /* workspace missing or smaller than required     */
  MDLM_EHIP = 4          /* a HIP runtime call or kernel launch failed     */
};

/* Noise processes. */
enum { MDLM_NOISE_ABSORB = 0, MDLM_NOISE_UNIFORM = 1 };

/* Logit alignment.  ALIGNED: the hidden state at position g predicts token g
 * (Nemotron-Labs-Diffusion).  SHIFTED: the hidden state at g-1 predicts
 * token g (Dream); a document's first token has no predecessor inside its
 * document and is never scored. */
enum { MDLM_ALIGNED = 0, MDLM_SHIFTED = 1 };

/* Element types of `hidden`, `W` and `d_hidden`. */
enum { MDLM_F32 = 0, MDLM_BF16 = 1 };

/*
 * mdlm_corrupt -- draw per-document noise levels and corrupt the tokens.
 *
 * Defined by: LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row
 * (absorbing, p = (1 - eps) t + eps with eps = 1e-3); diffusiongemma card,
 * "Finetuning notes" (uniform ids at rate t ~ U(eps, 1)); Axolotl docs,
 * "Start with Nemotron 3B" (mask id) and "Packed training" (isolation).
 *
 * Random numbers come from Philox4x32-10 (Salmon et al., SC'11) keyed by
 * (seed mod 2^32, seed >> 32).  For document b, word 0 of the call at counter
 * (b, 0, 0, 0) gives t_b = (word >> 8) * 2^-24, then in fp64
 * p_b = eps + (1 - eps) * t_b.  For token g (absolute index into x0), word
 * (g & 3) of the call at counter (lo32(g >> 2), hi32(g >> 2), 0, 1) decides:
 * corrupted iff (word >> 8) < ceil(p_b * 2^24), i.e. u < p_b for the 24-bit
 * uniform u.  A corrupted token becomes mask_id (ABSORB) or
 * (word2 * rand_vocab) >> 32 with word2 = word (g & 3) at counter
 * (lo32(g >> 2), hi32(g >> 2), 0, 2) (UNIFORM); a replacement equal to the
 * clean token still counts as corrupted.
 *
 *   x0          [n_tokens] int32, clean tokens of the packed stream.
 *   n_tokens    >= 0.
 *   cu_seqlens  [n_docs + 1] int32, cumulative document offsets, cu[0] = 0,
 *               cu[n_docs] = n_tokens, nondecreasing (empty documents
 *               allowed).  n_tokens must fit in int32 (< 2^31).
 *   n_docs      >= 1 (or 0 with n_tokens = 0).
 *   seed        64-bit Philox key.  Same seed -> same draw, bit for bit.
 *   eps         in (0, 1].  eps = 1 corrupts every token.
 *   noise       MDLM_NOISE_ABSORB or MDLM_NOISE_UNIFORM.
 *   mask_id     replacement id under ABSORB (ignored under UNIFORM).
 *   rand_vocab  >= 1; UNIFORM replacement ids lie in [0, rand_vocab).
 *   xt          [n_tokens] int32 out, corrupted tokens.
 *   corrupted   [n_tokens] uint8 out, 1 where corrupted else 0.
 *   p_doc       [n_docs] double out, p_b.
 *   doc_counts  [n_docs] int32 out, number of corrupted tokens per document.
 *   stream      hipStream_t or NULL.
 * Returns MDLM_OK, MDLM_EINVAL or MDLM_EHIP.
 */
int mdlm_corrupt(const int32_t* x0, int64_t n_tokens,
                 const int32_t* cu_seqlens, int32_t n_docs,
                 uint64_t seed, double eps,
                 int32_t noise, int32_t mask_id, int32_t rand_vocab,
                 int32_t* xt, uint8_t* corrupted, double* p_doc,
                 int32_t* doc_counts, void* stream);

/* Codes written by mdlm_corrupt_mixture into `corrupted`. */
enum { MDLM_CODE_CLEAN = 0, MDLM_CODE_MASKED = 1, MDLM_CODE_REPLACED = 2 };

/*
 * mdlm_corrupt_mixture -- corruption of the corrective mixture: absorbing
 * corruption in which a share of the corrupted tokens takes a uniform-random
 * id instead of the mask token.
 *
 * Defined by: LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row,
 * which names the corrective options (mixture_prob, noise_token_wt,
 * clean_token_wt; all 0 for the MDLM objective) without a formula.  The
 * reading implemented: each token is corrupted exactly as by mdlm_corrupt
 * with MDLM_NOISE_ABSORB (same p_b, same Bernoulli words); a corrupted token
 * g is replaced iff (word3 >> 8) < ceil(mixture_prob * 2^24), with word3 =
 * word (g & 3) at counter (lo32(g >> 2), hi32(g >> 2), 0, 3), and then takes
 * the id mdlm_corrupt's UNIFORM mode would give it; otherwise it becomes
 * mask_id.  mixture_prob = 0 gives mdlm_corrupt's ABSORB output exactly;
 * mixture_prob = 1 gives its UNIFORM tokens (codes 2 in place of 1).
 *
 *   mixture_prob  in [0, 1], the share of corrupted tokens replaced.
 *   corrupted     [n_tokens] uint8 out: MDLM_CODE_CLEAN, MDLM_CODE_MASKED or
 *                 MDLM_CODE_REPLACED.
 *   doc_counts    [n_docs] int32 out, corrupted tokens of either kind.
 *   rand_vocab    >= 1; replacement ids lie in [0, rand_vocab).
 *   other arguments as for mdlm_corrupt.
 * Returns MDLM_OK, MDLM_EINVAL or MDLM_EHIP.
 */
int mdlm_corrupt_mixture(const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                         int32_t n_docs, uint64_t seed, double eps, double mixture_prob,
                         int32_t mask_id, int32_t rand_vocab, int32_t* xt,
                         uint8_t* corrupted, double* p_doc, int32_t* doc_counts,
                         void* stream);

/*
 * Workspace bytes that mdlm_corrupt_compact needs for n_tokens tokens:
 * mdlm_compact_workspace_bytes(n_tokens) and one byte per token (the mask,
 * kept there when the caller passes no `corrupted`), each rounded up to 256.
 * Returns 0 for n_tokens <= 0.
 */
size_t mdlm_corrupt_compact_workspace_bytes(int64_t n_tokens);

/*
 * mdlm_corrupt_compact -- mdlm_corrupt followed by mdlm_compact_masked
 * (inverse-p weights) in one call: the same xt, corrupted, p_doc,
 * doc_counts, row_idx, tgt, w and n_rows, bit for bit.
 *
 * Defined by: as for mdlm_corrupt and mdlm_compact_masked (LLaDA-8B-MDLM-
 * LoRA card, Training table, "Objective" row; diffusiongemma card,
 * "Finetuning notes"; Axolotl docs, model table and "Packed training").
 *
 * The corruption pass also counts each 4096-token tile's corrupted tokens
 * (the compaction's tiles), so the compaction skips its own count pass over
 * the mask: one read of the mask (1 byte per token) and one launch fewer than
 * the two calls.
 *
 *   x0, n_tokens, cu_seqlens, n_docs, seed, eps, noise, mask_id, rand_vocab:
 *               as for mdlm_corrupt.
 *   align       MDLM_ALIGNED or MDLM_SHIFTED, as for mdlm_compact_masked.
 *   xt          [n_tokens] int32 out.
 *   corrupted   [n_tokens] uint8 out, or NULL (the mask is then not written).
 *   p_doc       [n_docs] double out.
 *   doc_counts  [n_docs] int32 out.
 *   row_idx, tgt, w   [n_tokens] out (first *n_rows valid).
 *   n_rows      [1] int32 out (device scalar).
 *   workspace   >= mdlm_corrupt_compact_workspace_bytes(n_tokens) bytes of
 *               device memory, 8-byte aligned; contents on entry are ignored.
 * Calls sharing a workspace must not overlap.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EUNSUPPORTED, MDLM_EWORKSPACE or MDLM_EHIP.
 */
int mdlm_corrupt_compact(const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                         int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                         int32_t mask_id, int32_t rand_vocab, int32_t align, int32_t* xt,
                         uint8_t* corrupted, double* p_doc, int32_t* doc_counts,
                         int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Row weightings of mdlm_compact_rows. */
enum {
  MDLM_WEIGHT_INV_P = 0,                 /* scale / (p_doc[b] * n_tokens)        */
  MDLM_WEIGHT_MEAN = 1,                  /* scale / M, M = rows listed           */
  MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED = 2   /* scale * min(1/(1-p_b), clip) / (n_b B) */
};

/*
 * Workspace bytes that mdlm_compact_masked needs for n_tokens tokens: three
 * 32-bit words per 4096-token tile (its count and its first and last
 * document) plus one per group of 1024 tiles (the group's total).  Returns 0
 * only for n_tokens <= 0.
 */
size_t mdlm_compact_workspace_bytes(int64_t n_tokens);

/*
 * mdlm_compact_masked -- list the scored rows in ascending token order.
 *
 * Defined by: LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row (CE
 * on masked tokens divided by p); Axolotl docs, model table (aligned vs
 * shifted logits) and "Batching" (logits only where a label is scored).
 *
 * For every corrupted token g of document b (ascending g):
 *   ALIGNED: row g, target x0[g];
 *   SHIFTED: row g - 1, target x0[g], except g = cu_seqlens[b] (skipped);
 * with weight w = (float)(1.0 / (p_doc[b] * (double)n_tokens)), so that
 * sum_j w_j CE_j is the 1/p-weighted CE over the call's total token count.
 *
 *   corrupted   [n_tokens] uint8 (as written by mdlm_corrupt).
 *   x0          [n_tokens] int32 clean tokens.
 *   cu_seqlens  [n_docs + 1] int32, as for mdlm_corrupt.
 *   p_doc       [n_docs] double, as written by mdlm_corrupt.
 *   align       MDLM_ALIGNED or MDLM_SHIFTED.
 *   row_idx     [n_tokens] int32 out (capacity n_tokens; first *n_rows valid).
 *   tgt         [n_tokens] int32 out.
 *   w           [n_tokens] float out.
 *   n_rows      [1] int32 out (device scalar).
 *   workspace   >= mdlm_compact_workspace_bytes(n_tokens) bytes of device
 *               memory, 4-byte aligned; contents on entry are ignored.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EWORKSPACE or MDLM_EHIP.
 */
int mdlm_compact_masked(const uint8_t* corrupted, const int32_t* x0,
                        int64_t n_tokens, const int32_t* cu_seqlens,
                        int32_t n_docs, const double* p_doc, int32_t align,
                        int32_t* row_idx, int32_t* tgt, float* w,
                        int32_t* n_rows, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Workspace bytes that mdlm_compact_rows needs: those of
 * mdlm_compact_workspace_bytes plus, for MDLM_WEIGHT_MEAN and
 * MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED, one 32-bit word per document (its
 * weight) and, for the latter, one more word per document and one more.
 * Returns 0 for n_tokens <= 0 or an invalid n_docs or weighting.
 */
size_t mdlm_compact_rows_workspace_bytes(int64_t n_tokens, int32_t n_docs,
                                         int32_t weighting);

/*
 * mdlm_compact_rows -- the scored-row list of mdlm_compact_masked, generalised
 * to the loss variants: every token (causal next-token CE), an eligibility
 * mask, and other weightings.
 *
 * Defined by: diffusiongemma card, "Finetuning notes" (total = diffusion CE +
 * encoder_loss_weight * encoder AR CE, the AR term the left-to-right
 * next-token CE of the uncorrupted sequence; each example draws its rate
 * t ~ U(eps, 1));
 * Axolotl docs, objective options (inv_one_minus_t time weighting with
 * example_mean reduction, 1/(1-t) capped by rhine_weight_clip) and "Packed
 * training" (tokens outside the loss are excluded).
 *
 * Token g of document b is scored when corrupted[g] != 0 (every token if
 * corrupted is NULL), eligible[g] != 0 (every token if eligible is NULL)
 * and, with MDLM_SHIFTED, g != cu_seqlens[b].  Rows and targets are as for
 * mdlm_compact_masked, in ascending g.  With M the number of rows, n_b the
 * rows of document b and B the number of documents with n_b > 0, each row of
 * document b has weight, evaluated in fp64 and rounded once to fp32:
 *   MDLM_WEIGHT_INV_P                 scale / (p_doc[b] * n_tokens)
 *   MDLM_WEIGHT_MEAN                  scale / M
 *   MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED  a = 1 / (1 - p_doc[b]); a = min(a, clip);
 *                                     scale * a / (n_b * B)
 * (corrupted = NULL, MDLM_SHIFTED, MDLM_WEIGHT_MEAN and scale = lambda give
 * the rows of lambda times the causal next-token CE; under uniform noise
 * p_doc[b] is the example's rate t.)
 *
 *   corrupted   [n_tokens] uint8 or NULL.
 *   eligible    [n_tokens] uint8 or NULL.
 *   x0, n_tokens, cu_seqlens, n_docs, align, row_idx, tgt, w, n_rows:
 *               as for mdlm_compact_masked.
 *   p_doc       [n_docs] double; may be NULL for MDLM_WEIGHT_MEAN.
 *   weighting   an MDLM_WEIGHT_* value.
 *   weight_scale  finite.
 *   weight_clip   > 0 (+inf: no cap); read by the clipped mode only.
 *   workspace   >= mdlm_compact_rows_workspace_bytes(n_tokens, n_docs,
 *               weighting) bytes of device memory, 4-byte aligned.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EWORKSPACE or MDLM_EHIP.
 */
int mdlm_compact_rows(const uint8_t* corrupted, const uint8_t* eligible,
                      const int32_t* x0, int64_t n_tokens,
                      const int32_t* cu_seqlens, int32_t n_docs,
                      const double* p_doc, int32_t align, int32_t weighting,
                      double weight_scale, double weight_clip,
                      int32_t* row_idx, int32_t* tgt, float* w,
                      int32_t* n_rows, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * mdlm_compact_masked_noalloc -- mdlm_compact_masked for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same rows, targets, weights and
 * row count, bit for bit, with no workspace argument.
 *
 * Its scratch space is an array inside the library, one copy per device,
 * sized for streams of at most 2^28 tokens (786,688 bytes, held until the
 * process ends); longer streams return MDLM_EUNSUPPORTED (use
 * mdlm_compact_masked with a workspace).  The call allocates nothing and
 * calls no allocating routine.  Every call on a device shares that device's
 * array, so calls that overlap on one device (on different streams or from
 * different threads) race and must not be issued; calls on one stream are
 * ordered and safe.
 *
 * Arguments as for mdlm_compact_masked, without workspace and
 * workspace_bytes.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EUNSUPPORTED or MDLM_EHIP.
 */
int mdlm_compact_masked_noalloc(const uint8_t* corrupted, const int32_t* x0,
                                int64_t n_tokens, const int32_t* cu_seqlens,
                                int32_t n_docs, const double* p_doc, int32_t align,
                                int32_t* row_idx, int32_t* tgt, float* w,
                                int32_t* n_rows, void* stream);

/*
 * mdlm_compact_corrective -- the scored-row list of the corrective mixture,
 * from the codes mdlm_corrupt_mixture writes.
 *
 * Defined by: LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row
 * (noise_token_wt and clean_token_wt, both 0 for the MDLM objective, named
 * without a formula).  The reading implemented: every listed position
 * predicts its clean token; a masked token (code 1) of document b has the
 * weight 1 / (p_doc[b] * n_tokens) of mdlm_compact_masked, a replaced token
 * (code 2) noise_token_wt / (p_doc[b] * n_tokens), and any other token
 * clean_token_wt / n_tokens, each evaluated in fp64 and rounded once to
 * fp32.  Listed are the tokens with a nonzero code and, when clean_token_wt
 * is not 0, every token; rows, targets, alignment and order as for
 * mdlm_compact_masked.  With both weights 0 the rows are those of
 * mdlm_compact_masked over (codes != 0), replaced tokens at weight 0.
 *
 *   codes       [n_tokens] uint8, as written by mdlm_corrupt_mixture.
 *   noise_token_wt, clean_token_wt   finite.
 *   workspace   >= mdlm_compact_workspace_bytes(n_tokens) bytes of device
 *               memory, 4-byte aligned; contents on entry are ignored.
 *   other arguments as for mdlm_compact_masked.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EWORKSPACE or MDLM_EHIP.
 */
int mdlm_compact_corrective(const uint8_t* codes, const int32_t* x0,
                            int64_t n_tokens, const int32_t* cu_seqlens,
                            int32_t n_docs, const double* p_doc, int32_t align,
                            double noise_token_wt, double clean_token_wt,
                            int32_t* row_idx, int32_t* tgt, float* w,
                            int32_t* n_rows, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Workspace bytes that mdlm_fused_head_ce_fwd_bwd needs for up to max_rows
 * scored rows of hidden size H against a vocabulary of V.  This is the size
 * the library prefers: with bf16 it holds a bf16 value per scored row and
 * vocabulary entry, so the forward pass keeps the softmax there and the
 * gradient needs no second pass over the logits.  Any size down to
 * mdlm_head_ce_workspace_min_bytes is accepted (the gradient then recomputes
 * the logits in vocabulary chunks that fit); a smaller one is rejected.
 * Returns 0 for invalid sizes.
 */
size_t mdlm_head_ce_workspace_bytes(int64_t max_rows, int32_t H, int32_t V,
                                    int32_t dtype);
size_t mdlm_head_ce_workspace_min_bytes(int64_t max_rows, int32_t H, int32_t V,
                                        int32_t dtype);

/*
 * mdlm_fused_head_ce_fwd_bwd -- weighted full-vocabulary cross-entropy of
 * the scored rows through a frozen linear head, and its gradient.
 *
 * Defined by: Axolotl docs, "Adapters, merging and inference" (CE over the
 * whole vocabulary taken from the hidden states, no logits tensor stored;
 * bare linear head); LLaDA-8B-MDLM-LoRA card, Training table (the CE of
 * each masked token scaled by 1/p; output layer frozen, so no weight
 * gradient); diffusiongemma card, "Finetuning notes" (softcap applied once).
 *
 * For j < *n_rows, with h = hidden[row_idx[j]] and z = W h (no bias):
 *   zhat  = softcap > 0 ? softcap * tanh(z / softcap) : z
 *   CE_j  = logsumexp(zhat) - zhat[tgt[j]]
 *   loss  = sum_j w[j] * CE_j
 *   d_hidden[row_idx[j]] = w[j] * ((softmax(zhat) - onehot(tgt[j])) * zhat') W
 * where zhat' = 1 - (zhat / softcap)^2 (1 without a cap); every other row of
 * d_hidden is set to exactly zero.  The upstream gradient is taken as 1.
 * row_idx entries must be distinct (as mdlm_compact_masked produces).
 *
 * BF16: inputs bf16, products accumulated in fp32, d_hidden written as bf16.
 * The second product takes its per-logit factor rounded to bf16: with the
 * preferred workspace, the softmax relative to the row's target logit
 * (times zhat'), the row's scale and the target's term then applied in fp32;
 * with a smaller workspace, the gradient w (softmax - onehot) zhat' itself.
 * F32: everything in fp32.
 *
 *   hidden      [n_tokens, H] row-major, element type `dtype`.
 *   W           [V, H] row-major, element type `dtype`.
 *   dtype       MDLM_BF16 or MDLM_F32.
 *   n_tokens    rows of hidden / d_hidden, >= 0.
 *   H           > 0, a multiple of 64 (else MDLM_EUNSUPPORTED).
 *   V           > 0.  With MDLM_BF16, hidden and W must each be smaller
 *               than 4 GiB (n_tokens * H * 2 and V * H * 2 bytes; else
 *               MDLM_EUNSUPPORTED).
 *   row_idx, tgt, w   as written by mdlm_compact_masked (tgt in [0, V)).
 *   n_rows      [1] int32 device scalar, 0 <= *n_rows <= max_rows.
 *   max_rows    host bound on *n_rows, 0 <= max_rows <= n_tokens; sizes
 *               the launch (no host read of *n_rows is ever made).
 *   softcap     0 = none, else > 0 and finite.
 *   loss        [1] float out.
 *   row_ce      [max_rows] float out, CE_j, or NULL.
 *   d_hidden    [n_tokens, H] out, element type `dtype`, 16-byte aligned,
 *               or NULL for a forward-only call.
 *   workspace   device memory, 256-byte aligned, of workspace_bytes >=
 *               mdlm_head_ce_workspace_min_bytes(max_rows, H, V, dtype).
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EUNSUPPORTED, MDLM_EWORKSPACE or
 * MDLM_EHIP.
 */
int mdlm_fused_head_ce_fwd_bwd(const void* hidden, const void* W, int32_t dtype,
                               int64_t n_tokens, int32_t H, int32_t V,
                               const int32_t* row_idx, const int32_t* tgt,
                               const float* w, const int32_t* n_rows,
                               int64_t max_rows, float softcap, float* loss,
                               float* row_ce, void* d_hidden, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of mdlm_fused_head_ce_fwd_bwd_dw: those of the bf16
 * mdlm_head_ce_workspace_bytes / _min_bytes plus room for the gathered
 * scored rows (max_rows * H bf16).  Returns 0 for invalid sizes.
 */
size_t mdlm_head_ce_dw_workspace_bytes(int64_t max_rows, int32_t H, int32_t V);
size_t mdlm_head_ce_dw_workspace_min_bytes(int64_t max_rows, int32_t H, int32_t V);

/*
 * mdlm_fused_head_ce_fwd_bwd_dw -- mdlm_fused_head_ce_fwd_bwd for a head that
 * is trained: the same loss, row_ce and d_hidden, plus the gradient of the
 * loss with respect to W.
 *
 * Defined by: Axolotl docs, "Adapters, merging and inference" (the plain
 * linear head whose gradient this is); LLaDA-8B-MDLM-LoRA card, Training
 * table (the frozen-head case, where no such gradient is formed).
 *
 *   dW[v] = sum_j w[j] * (softmax(zhat_j)[v] - [v == tgt[j]]) * zhat'_jv * h_j
 * (the per-logit gradient rounded to bf16, times the bf16 hidden rows;
 * products accumulated in fp32).
 *
 *   hidden, W   bf16 only (the element type is implied).
 *   d_hidden    [n_tokens, H] bf16 out, 16-byte aligned, or NULL (only dW
 *               is wanted).
 *   dW          [V, H] float out, 16-byte aligned; overwritten (zero when no
 *               row is scored).
 *   workspace   >= mdlm_head_ce_dw_workspace_min_bytes(max_rows, H, V).
 *   other arguments as for mdlm_fused_head_ce_fwd_bwd.
 * Returns MDLM_OK, MDLM_EINVAL, MDLM_EUNSUPPORTED, MDLM_EWORKSPACE or
 * MDLM_EHIP.
 */
int mdlm_fused_head_ce_fwd_bwd_dw(const void* hidden, const void* W,
                                  int64_t n_tokens, int32_t H, int32_t V,
                                  const int32_t* row_idx, const int32_t* tgt,
                                  const float* w, const int32_t* n_rows,
                                  int64_t max_rows, float softcap, float* loss,
                                  float* row_ce, void* d_hidden, float* dW,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * mdlm_scale -- y = g * x elementwise, with g a device scalar: the upstream
 * gradient of the loss applied to d_hidden, for a trainer in which the loss
 * is one term of what it differentiates (an autograd backward).
 *
 * Defined by: LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row (the
 * loss the trainer backpropagates through); by the chain rule
 * d(g * loss)/d hidden = g * d_hidden, and mdlm_fused_head_ce_fwd_bwd forms
 * d_hidden for an upstream gradient of 1.
 *
 *   x, y       n entries of element type `dtype`, each 16-byte aligned; y may
 *              be x (in place).  bf16: the fp32 product rounded once to bf16.
 *   dtype      MDLM_BF16 or MDLM_F32.
 *   n          >= 0 entries.
 *   scale      [1] float device scalar g (read on the device; no host read).
 * Returns MDLM_OK, MDLM_EINVAL or MDLM_EHIP.
 */
int mdlm_scale(const void* x, void* y, int32_t dtype, int64_t n, const float* scale,
               void* stream);

/* Violation bits of the device-side precondition checks. */
enum {
  MDLM_CHECK_OFFSETS = 1,    /* cu_seqlens not 0 = cu[0] <= ... <= cu[n_docs] = n_tokens */
  MDLM_CHECK_ROW_COUNT = 2,  /* *n_rows outside [0, max_rows]                           */
  MDLM_CHECK_ROW_INDEX = 4,  /* a listed row index outside [0, n_tokens)                */
  MDLM_CHECK_TARGET = 8,     /* a listed target outside [0, V)                          */
  MDLM_CHECK_WEIGHT = 16,    /* a listed weight that is not finite                      */
  MDLM_CHECK_PROB = 32       /* a p_doc entry outside (0, 1]                            */
};

/*
 * Device-side precondition checks.  The entry points above never read
 * device data on the host, so the preconditions on device-resident inputs
 * are the caller's; these calls check them.  Each is asynchronous on
 * `stream`, only reads its inputs, and ORs the MDLM_CHECK_* bits of what it
 * finds into the device word *status (which the caller clears beforehand:
 * several checks may accumulate into one word).
 *
 * Motivated by: Axolotl docs, "Packed training" (the default overflow policy
 * raises on an oversized example rather than training on it) and the note
 * after the model table (a configuration the trainer cannot train natively
 * is refused).
 *
 *   mdlm_check_offsets  cu_seqlens [n_docs + 1] against n_tokens.
 *   mdlm_check_probs    p_doc [n_docs] in (0, 1].
 *   mdlm_check_rows     *n_rows in [0, max_rows]; for j < *n_rows (clamped
 *                       to [0, max_rows]): row_idx[j] in [0, n_tokens),
 *                       tgt[j] in [0, V) and w[j] finite (tgt and w may be
 *                       NULL: not checked).  Distinctness of the row indices
 *                       is not checked.
 *   status              [1] int32 device word, 4-byte aligned.
 * Return MDLM_OK, MDLM_EINVAL (bad host arguments; nothing enqueued) or
 * MDLM_EHIP.
 */
int mdlm_check_offsets(const int32_t* cu_seqlens, int32_t n_docs, int64_t n_tokens,
                       int32_t* status, void* stream);
int mdlm_check_probs(const double* p_doc, int32_t n_docs, int32_t* status, void* stream);
int mdlm_check_rows(const int32_t* row_idx, const int32_t* tgt, const float* w,
                    const int32_t* n_rows, int64_t max_rows, int64_t n_tokens, int32_t V,
                    int32_t* status, void* stream);

/*
 * Checking mode.  With checking on, every entry point first checks its own
 * device inputs (as the calls above do: corruption its offsets; compaction
 * its offsets and noise levels; the fused head its row list), waits for the result on its stream, and returns MDLM_EINVAL with a
 * message naming what is wrong -- enqueueing none of its own work -- if a
 * check fails.  This trades the calls' asynchrony for the checks: a call in
 * checking mode synchronises its stream, cannot be captured in a graph (it
 * returns MDLM_EINVAL under stream capture), and calls on several threads
 * take turns for the check.  Off by default; the environment variable
 * MDLM_CHECK set to anything but "0" (read at the first call) turns it on.
 * Returns the previous setting (0 or 1).
 */
int mdlm_set_checking(int enable);

/* Message describing the last failure on the calling thread ("" if none).
 * Valid until the next library call on that thread. */
const char* mdlm_last_error(void);

/* Library ABI version, (major << 16) | minor. */
int mdlm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MDLM_H */
