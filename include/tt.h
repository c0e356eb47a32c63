/*
 * tt.h -- C ABI of libtt.so: the TwoTower denoiser block-attention step, the
 * confidence unmask that follows it, and the block-commit cache append, on
 * AMD Instinct MI355X (gfx950).
 *
 * Method sources (page title, section):
 *   "Nemotron-Labs-TwoTower: Diffusion Language Modeling with Pretrained
 *    Autoregressive Context" (paperfeed.app review), "The idea: freeze the
 *    reader, train the writer" and "Training and sampling";
 *   "NVIDIA's Dual-Tower Diffusion Language Model Explained" (kongchang.com),
 *    "The 'Sky Bridges' Between Layers" and "Generating Text in Parallel Like
 *    Solving a Sudoku".
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  All tensors are contiguous,
 *     row-major, last index fastest.
 *   - Calls validate their arguments on the host, enqueue kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and return without waiting.
 *     Results are valid once the stream has reached that point.
 *   - Return value: TT_OK (0) or a negative tt_status.  On error nothing has
 *     been enqueued and tt_last_error() holds a message for this thread.
 *   - Values the host cannot see (ctx_lens[], page ids) are bounds-clamped on
 *     the device so that bad values never fault; results are then
 *     unspecified.  tt_kv_append skips a sequence whose target slots are not
 *     all backed by valid pages.
 *   - Calls are stateless apart from a per-thread error string (and the
 *     static array of tt_unmask_noalloc); concurrent calls on different
 *     streams must not share a workspace.
 *   - Results are bitwise reproducible for the same inputs and shapes (fixed
 *     reduction orders, no atomics on data).  The calls allocate nothing and
 *     enqueue only kernel launches, so they can be captured in a HIP graph
 *     and replayed; the first call on each device also sets a kernel
 *     attribute, so make one call before capturing.
 *
 * Choices of this ABI that callers must honour (the pages fix none of them):
 *   - Cached VALUES are feature-major inside a page, v_pages [P, H_kv, D,
 *     page_size], while cached keys are token-major, k_pages [P, H_kv,
 *     page_size, D].  A writer of the value pool other than tt_kv_append
 *     must use this layout: it gives P.V its matrix-core operands as
 *     contiguous 16-byte runs.
 *   - page_size is a power of two (16..4096), not any multiple of 16, so
 *     that token -> (page, offset) is a shift and a mask on the device.
 *   - The workspace-size queries return a tt_status and report the size
 *     through an out-parameter, so that a bad shape is an error, not 0.
 *   - tt_attn_desc carries num_pages, the pool size, so that page ids can be
 *     bounds-clamped on the device.
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TT_ABI_VERSION 1

typedef enum tt_status {
  TT_OK = 0,
  TT_ERR_NULL = -1,        /* a required pointer is NULL                        */
  TT_ERR_SHAPE = -2,       /* a size is out of range or sizes are inconsistent  */
  TT_ERR_DTYPE = -3,       /* unknown element type                              */
  TT_ERR_UNSUPPORTED = -4, /* valid request this build does not implement       */
  TT_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required        */
  TT_ERR_NO_DEVICE = -6,   /* no usable HIP device                              */
  TT_ERR_LAUNCH = -7       /* the HIP runtime rejected a launch                 */
} tt_status;

typedef enum tt_dtype {
  TT_BF16 = 0, /* bfloat16: MFMA path, head_dim 64 or 128                       */
  TT_F32 = 1   /* float32: small-problem path, head_dim 1..256                  */
} tt_dtype;

/*
 * Shape of one block-attention layer.
 *
 *   batch              B >= 0 sequences (B = 0 is a no-op), B <= 2048
 *   block              S, tokens per noisy block, 1..64 (the pages use 16)
 *   heads_q, heads_kv  H_q, H_kv >= 1, H_q % H_kv == 0; query head h reads
 *                      KV head h / (H_q / H_kv) (contiguous GQA groups)
 *   head_dim           D
 *   page_size          tokens per cache page, a power of two in 16..4096
 *   max_pages_per_seq  row stride of page_table (>= 1)
 *   num_pages          P, pages in the pool (page ids must be < P)
 *   max_ctx_len        host-side upper bound on every ctx_lens[b], at most
 *                      max_pages_per_seq * page_size; sizes the launch
 *   scale              softmax scale; <= 0 selects 1/sqrt(D)
 *   dtype              tt_dtype of q, k_blk, v_blk, k_pages, v_pages, out
 */
typedef struct tt_attn_desc {
  int32_t batch;
  int32_t block;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t max_ctx_len;
  float scale;
  int32_t dtype;
} tt_attn_desc;

/* Workspace bytes tt_block_attn needs for this shape on the current device
 * (0 is possible).  Returns a tt_status; *bytes is set on TT_OK. */
int tt_block_attn_workspace_bytes(const tt_attn_desc *desc, size_t *bytes);

/*
 * Denoiser block attention for one layer ("The idea: freeze the reader,
 * train the writer", paperfeed review; "The 'Sky Bridges' Between Layers",
 * kongchang explainer).  For every sequence b, query head h and block slot t:
 *
 *   O[b,t,h,:] = softmax_j( scale * q[b,t,h,:] . Kcat_j ) @ Vcat
 *
 * where Kcat/Vcat concatenate the context tower's cached keys/values of the
 * L_b = ctx_lens[b] committed tokens (gathered through page_table) with the
 * S keys/values of the block itself.  No mask: the block is bidirectional
 * inside, and causality across blocks comes from what the cache holds.
 *
 *   q          [B, S, H_q, D]
 *   k_blk      [B, S, H_kv, D]        the block's own keys
 *   v_blk      [B, S, H_kv, D]        the block's own values
 *   k_pages    [P, H_kv, page_size, D]   cached keys, token-major per page
 *   v_pages    [P, H_kv, D, page_size]   cached values, feature-major per page
 *   page_table int32 [B, max_pages_per_seq]; entry j of row b is the page of
 *              logical tokens [j*page_size, (j+1)*page_size); only the first
 *              ceil(L_b / page_size) entries of a row are read
 *   ctx_lens   int32 [B], 0 <= L_b <= max_ctx_len
 *   out        [B, S, H_q, D]; bf16 results are rounded to nearest even
 *   workspace  device scratch of tt_block_attn_workspace_bytes() bytes
 *              (may be NULL if that is 0); no initial contents required
 *
 * bf16 path: Q.K^T and P.V on bf16 MFMA with fp32 accumulation, fp32 online
 * softmax, probabilities rounded to bf16 for P.V.  f32 path: fp32 throughout.
 * k_pages, v_pages and page_table may be NULL only when max_ctx_len == 0.
 */
int tt_block_attn(const tt_attn_desc *desc, const void *q, const void *k_blk,
                  const void *v_blk, const void *k_pages, const void *v_pages,
                  const int32_t *page_table, const int32_t *ctx_lens, void *out,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Causal chunk ingest by the context tower ("The idea: freeze the reader,
 * train the writer", paperfeed review: the frozen context tower runs
 * causally over clean tokens and ingests a committed block as one clean
 * forward chunk, updating its caches).  Same arguments, layouts, workspace
 * (tt_block_attn_workspace_bytes) and precision as tt_block_attn, with one
 * difference: chunk position t attends over the L_b committed tokens and
 * chunk tokens 0..t only,
 *
 *   O[b,t,h,:] = softmax_j( scale * q[b,t,h,:] . Kcat_j ) @ Vcat,
 *   Kcat = [K_ctx(b, 0..L_b-1) ; k_blk(b, 0..t)],  Vcat likewise.
 *
 * Follow it with tt_kv_append of the same chunk to grow the caches.
 */
int tt_chunk_attn(const tt_attn_desc *desc, const void *q, const void *k_blk,
                  const void *v_blk, const void *k_pages, const void *v_pages,
                  const int32_t *page_table, const int32_t *ctx_lens, void *out,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Block commit: the context cache ingests a resolved block ("The idea: freeze
 * the reader, train the writer", paperfeed review: once a block is resolved
 * it is committed and the context tower's caches are updated).  For every
 * sequence b with L_b = ctx_lens[b], writes k_blk[b,t]/v_blk[b,t] (t < S) to
 * logical positions L_b + t of the paged pool (keys token-major, values
 * feature-major, bit-exact copies) and sets ctx_lens[b] = L_b + S.
 *
 * The caller provides the pages: page_table must map every position up to
 * L_b + S - 1.  A sequence whose target positions exceed
 * max_pages_per_seq * page_size or map to an invalid page id is left
 * untouched (no write, ctx_lens[b] unchanged).  desc->max_ctx_len is not used
 * here; the caller raises it by S for later tt_block_attn calls.
 */
int tt_kv_append(const tt_attn_desc *desc, const void *k_blk, const void *v_blk,
                 void *k_pages, void *v_pages, const int32_t *page_table,
                 int32_t *ctx_lens, void *stream);

/* tt_unmask flags */
#define TT_UNMASK_UPDATE_MASK 1u /* clear mask[b,t] where commit_out[b,t] = 1 */

/* Workspace bytes tt_unmask needs (0 is possible).  Returns a tt_status. */
int tt_unmask_workspace_bytes(int32_t batch, int32_t block, int32_t vocab, size_t *bytes);

/*
 * Confidence unmask ("Training and sampling", paperfeed review; "Generating
 * Text in Parallel Like Solving a Sudoku", kongchang explainer): predict
 * every masked slot in parallel and commit the confident ones; committed
 * slots stay fixed.  Count form of the commit rule.  For every row
 * r = b*S + t of logits:
 *
 *   ids_out[r]  = smallest v with logits[r,v] == max_v logits[r,v]
 *   conf[r]     = 1 / sum_v exp(logits[r,v] - max)   (max-softmax probability)
 *
 * and per sequence b the k_eff = clamp(k_b, 0, #masked_b) masked slots with
 * the highest conf are committed (equal conf: lower slot first), where
 * k_b = k_commit[b], or ceil(#masked_b / remaining_steps) when k_commit is
 * NULL.  commit_out[r] = 1 exactly on those slots.
 *
 *   logits     float32 [B*S, V]; finite values or -inf, at least one finite
 *              value per row
 *   mask       uint8 [B, S], nonzero = masked; read-only unless flags has
 *              TT_UNMASK_UPDATE_MASK (then cleared where committed)
 *   k_commit   int32 [B] or NULL
 *   remaining_steps  >= 1 when k_commit is NULL, else ignored
 *   batch, block, vocab  B >= 0, 1 <= S <= 64, V >= 1
 *   ids_out    int32 [B, S]
 *   commit_out uint8 [B, S]
 *   conf_out   float32 [B, S] or NULL
 */
int tt_unmask(const float *logits, uint8_t *mask, const int32_t *k_commit,
              int32_t remaining_steps, int32_t batch, int32_t block, int32_t vocab,
              int32_t *ids_out, uint8_t *commit_out, float *conf_out, uint32_t flags,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * tt_unmask for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument.  Arguments, results and errors as tt_unmask.  The row partials
 * live in a static device array of TT_UNMASK_NOALLOC_MAX_BYTES (1 MiB) that
 * every device the library runs on holds until the process ends.  Every
 * shape tt_unmask accepts fits (its tt_unmask_workspace_bytes is at most
 * 16 x max(batch * block, 1023) bytes); a larger need would fail with
 * TT_ERR_WORKSPACE before any device work.  The array needs no
 * initial contents, but every call on a device shares it: calls that may
 * overlap on one device (unordered streams) race; calls ordered on one
 * stream do not.  The first call on each device looks up the array's
 * address; make one call there before capturing a graph.
 */
#define TT_UNMASK_NOALLOC_MAX_BYTES (1u << 20)
int tt_unmask_noalloc(const float *logits, uint8_t *mask, const int32_t *k_commit,
                      int32_t remaining_steps, int32_t batch, int32_t block, int32_t vocab,
                      int32_t *ids_out, uint8_t *commit_out, float *conf_out, uint32_t flags,
                      void *stream);

/*
 * Threshold form of the commit rule, the one the pages' sampler uses
 * ("Training and sampling", paperfeed review: every prediction whose
 * confidence is above gamma = 0.8 is committed and the count per step
 * adapts; "Generating Text in Parallel Like Solving a Sudoku", kongchang
 * explainer: commit the positions whose confidence exceeds the threshold,
 * re-mask the rest).  ids_out and conf are as in tt_unmask.  Per sequence b,
 * every masked slot with conf > gamma is committed; when no masked slot
 * clears gamma, the single most confident masked slot is (lower slot on
 * equal conf), so every step makes progress.  A sequence with nothing masked
 * commits nothing.  Driving this call until every mask is clear is the
 * adaptive-step loop: sequences resolve their block at different steps.
 *
 *   logits, mask, batch, block, vocab, ids_out, commit_out, conf_out, flags,
 *   workspace   as in tt_unmask (same workspace size)
 *   gamma       confidence threshold (finite)
 *   nsteps      int32 [B] or NULL: incremented for every sequence that had at
 *               least one masked slot on entry (steps used so far)
 *
 * The comparison conf > gamma is taken on the fp32 confidence.
 */
int tt_unmask_threshold(const float *logits, uint8_t *mask, float gamma, int32_t batch,
                        int32_t block, int32_t vocab, int32_t *ids_out, uint8_t *commit_out,
                        float *conf_out, int32_t *nsteps, uint32_t flags, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * LM head fused with the confidence unmask.  The denoiser predicts every
 * masked slot through the model's output head ("Training and sampling",
 * paperfeed review; "Generating Text in Parallel Like Solving a Sudoku",
 * kongchang explainer); the head is read as a bias-free linear map:
 *
 *   logits[r, v] = sum_h hidden[r, h] * weight[v, h]     (r = b*S + t)
 *
 * and the result is exactly tt_unmask (count form) on those logits, except
 * that the logits are never written to memory: the head's matrix product
 * (bf16 inputs, fp32 accumulation, on the matrix cores) reduces each tile of
 * logits on the spot to the per-row maximum, its lowest index and the sum
 * of exp(logit - max).  ids_out / commit_out / conf_out, mask, k_commit,
 * remaining_steps and flags are as in tt_unmask.
 *
 *   hidden      bf16 [B*S, H], 16-byte aligned (the final hidden state)
 *   weight      bf16 [V, H], 16-byte aligned (one vocabulary row after another)
 *   batch, block, vocab  as in tt_unmask
 *   hidden_size H: a multiple of 32 in [32, 65536]
 *
 * Differences from tt_unmask on the same logits come only from the fp32
 * rounding of the logits (accumulation order): ids may differ where the two
 * largest logits of a row are that close, commits where confidences are.
 * Workspace: tt_lmhead_unmask_workspace_bytes (16-byte aligned, caller-owned,
 * needed for batch > 0).  It holds one 16-byte partial per row and 256-entry
 * vocabulary tile and a copy of the hidden state rearranged for the matrix
 * cores (about B*S*H*2 bytes, rows rounded up to 256); its contents on entry
 * do not matter.  Errors as tt_unmask;
 * TT_ERR_SHAPE for H.
 */
int tt_lmhead_unmask_workspace_bytes(int32_t batch, int32_t block, int32_t vocab,
                                     int32_t hidden_size, size_t *bytes);
int tt_lmhead_unmask(const void *hidden, const void *weight, uint8_t *mask,
                     const int32_t *k_commit, int32_t remaining_steps, int32_t batch,
                     int32_t block, int32_t vocab, int32_t hidden_size, int32_t *ids_out,
                     uint8_t *commit_out, float *conf_out, uint32_t flags, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * The same fused head followed by the threshold form of the commit rule
 * (tt_unmask_threshold's gamma, nsteps and rule); arguments as in
 * tt_lmhead_unmask and tt_unmask_threshold, same workspace size as
 * tt_lmhead_unmask.
 */
int tt_lmhead_unmask_threshold(const void *hidden, const void *weight, uint8_t *mask,
                               float gamma, int32_t batch, int32_t block, int32_t vocab,
                               int32_t hidden_size, int32_t *ids_out, uint8_t *commit_out,
                               float *conf_out, int32_t *nsteps, uint32_t flags, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *tt_status_str(int status);

/* Detailed message of the last failed call on this thread ("" if none). */
const char *tt_last_error(void);

/* TT_ABI_VERSION of the loaded library. */
int tt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
