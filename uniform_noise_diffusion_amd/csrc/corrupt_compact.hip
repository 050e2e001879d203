// Corruption and the inverse-p scored-row list in one call.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (one
// t ~ U(0,1) for each sequence, masking probability p = (1 - 1e-3) t + 1e-3,
// the CE of each masked token scaled by 1/p); diffusiongemma card,
// "Finetuning notes" (uniformly drawn ids, each example with its own rate);
// Axolotl diffusion docs, model table (aligned vs shifted logits) and
// "Packed training" (documents stay isolated).  The outputs are exactly
// those of corruption followed by compaction with inverse-p weights, because
// they are computed by the same kernels.
//
// The separate calls read the corruption mask twice after writing it: the
// compaction's count pass reads it to size each 4096-token tile's share of
// the list, and its scatter pass reads it again with the tokens.  Here the
// corruption kernel, whose block is exactly one such tile and which already
// counts the corrupted tokens with ballots, writes each tile's count into the
// compaction's workspace; with shifted rows the per-document pass that the
// compaction runs anyway (each tile's first and last document) takes a
// corrupted first token of a document out of its tile's count.  Then the
// compaction runs without its count pass: the scan of the counts and the
// scatter.  Traffic: the corruption's 9 bytes per token, then the mask (1)
// and the tokens (4) again and 12 per scored row -- about 20 bytes per token
// at half the tokens scored, one byte per token less than the two calls.
//
// (A single pass with a decoupled look-back across tiles -- each tile
// publishing its count and summing its predecessors' -- moves only 15 bytes
// per token, but measured 1.4x slower than the two calls on this GPU: each
// block's chain of dependent loads and its waits on its predecessors left it
// latency-bound.)
#include "mdlm_internal.h"

#include <math.h>

#include <algorithm>

namespace mdlm {
namespace {

constexpr int64_t kAlign = 256;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

size_t corrupt_compact_workspace_bytes(int64_t n_tokens) {
  if (n_tokens <= 0) return 0;
  // the compaction's workspace (its tile counts first), then room for the
  // mask when the caller does not want it written
  return (size_t)(round_up((int64_t)compact_workspace_bytes(n_tokens, 0, MDLM_WEIGHT_INV_P),
                           kAlign) +
                  round_up(n_tokens, kAlign));
}

hipError_t launch_corrupt_compact(const int32_t* x0, int64_t n, const int32_t* cu,
                                  int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                                  int32_t mask_id, int32_t rand_vocab, int32_t align,
                                  int32_t* xt, uint8_t* corrupted, double* p_doc,
                                  int32_t* doc_counts, int32_t* row_idx, int32_t* tgt,
                                  float* w, int32_t* n_rows, void* workspace,
                                  hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  // the compaction's workspace starts with one count per tile
  int32_t* tile_counts = n > 0 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  uint8_t* mask = corrupted;
  if (!mask && n > 0)
    mask = reinterpret_cast<uint8_t*>(
        ws + round_up((int64_t)compact_workspace_bytes(n, 0, MDLM_WEIGHT_INV_P), kAlign));
  hipError_t e = launch_corrupt(x0, n, cu, n_docs, seed, eps, noise, mask_id, rand_vocab, xt,
                                mask, p_doc, doc_counts, stream, 0.0, tile_counts);
  if (e != hipSuccess) return e;
  return launch_compact(mask, nullptr, x0, n, cu, n_docs, p_doc, align, MDLM_WEIGHT_INV_P, 1.0,
                        INFINITY, row_idx, tgt, w, n_rows, workspace, stream, true);
}

}  // namespace mdlm
