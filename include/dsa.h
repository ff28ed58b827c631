/*
 * dsa.h -- C ABI of libdsa.so, the MI355X (gfx950) DeepSeek Sparse Attention
 * (DSA) hot path: lightning indexer -> top-k selector -> sparse MQA/MLA
 * attention.
 *
 * The method.  The ivugangingo.com article on DeepSeek-V3.2 (section "Sparse
 * attention with almost linear long-context costs") splits attention into a
 * lightning indexer -- a few low-precision heads scoring every (query, key)
 * pair -- and a fine-grained selector that keeps the top-k key positions per
 * query; the main attention path then runs MQA/MLA on that sparse set only.
 * The r.nikiv.dev summary ("DeepSeek-V3.2: Pushing the Frontier of Open Large
 * Language Models", section "How DSA Works") adds that the indexer is FP8 and
 * that k = 2048.  The pages give no indexer formula; this library computes
 *     score(t, s) = sum_j w[t, j] * ReLU(q[t, j, :] . k[s, :])
 * with q, k FP8 e4m3fn (OCP) bytes times per-token fp32 scales, fp32 w and
 * fp32 accumulation, over causal pairs s <= pos(t).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are caller-owned device memory, row-major and contiguous.
 *   The library never allocates, frees or synchronises; it keeps no state
 *   besides a thread-local error string.
 * - Every pointer to device memory must be 16-byte aligned (NULL only where
 *   an argument is documented as nullable).
 * - Sequences are packed: sequence b owns query rows
 *   [q_offsets[b], q_offsets[b+1]) and key/KV rows
 *   [kv_offsets[b], kv_offsets[b+1]).  Query row r of sequence b sits at
 *   position pos(r) = q_pos0[b] + (r - q_offsets[b]) and sees the keys at
 *   positions 0..pos(r) of its own sequence (causal, itself included).
 *   Required: q_pos0[b] + q_len_b <= kv_len_b.  The offset arrays live on the
 *   device, so the library cannot check them before launching; kernels clamp
 *   every index they derive from them to the host-given totals and maxima, so
 *   inconsistent offsets give wrong results but never an out-of-bounds access.
 * - FP8 is stored as OCP e4m3fn bytes (uint8_t), bf16 as raw uint16_t bit
 *   patterns, indices as int32 positions within the sequence.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   Validation runs on the host before anything is enqueued: on a non-OK
 *   status nothing was launched and dsa_last_error() describes the problem.
 *   Faults inside kernels surface at the caller's next synchronisation.
 * - Debug builds (libdsa_debug.so, compiled with DSA_DEBUG): every call also
 *   synchronises its stream, copies the offset arrays (and a paged cache's
 *   block table) to the host and checks them -- offsets from 0 to the totals,
 *   no sequence longer than the maxima, q_pos0[b] + q_len_b <= kv_len_b,
 *   table entries of used blocks inside the cache -- returning
 *   DSA_ERR_INVALID_ARGUMENT before any launch when they are inconsistent.
 *   dsa_version() then ends in " debug".
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or inconsistent dims */
  DSA_ERR_UNSUPPORTED = 2,      /* valid request outside the shapes this build supports */
  DSA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than dsa_workspace_bytes() */
  DSA_ERR_HIP = 4               /* a HIP runtime call failed (message in dsa_last_error) */
} dsa_status;

/* Problem description.  A host struct; the three arrays it points to are on
 * the device.  Scalar totals and maxima are host-known and size the grids. */
typedef struct dsa_problem {
  int32_t batch;          /* B >= 1 sequences                                       */
  int32_t idx_heads;      /* H_I: indexer heads, 1..128                              */
  int32_t idx_dim;        /* d_I: indexer head width, one of 32, 64, 128             */
  int32_t heads;          /* H: attention query heads sharing one KV row, 1..128     */
  int32_t d_latent;       /* value width (latent part of the KV row)                 */
  int32_t d_rope;         /* rotary part of the KV row (keys only)                   */
  int32_t topk;           /* k: selected positions per query, 1..4096                */
  float softmax_scale;    /* attention logit scale, finite and > 0                   */
  int64_t total_q;        /* packed query rows over all sequences                    */
  int64_t total_kv;       /* packed key / KV rows over all sequences                 */
  int64_t max_q_len;      /* >= every q_len_b                                        */
  int64_t max_kv_len;     /* >= every kv_len_b                                       */
  const int32_t *q_offsets;  /* device [B+1]: 0 = q_offsets[0] <= ... <= q_offsets[B] = total_q   */
  const int32_t *kv_offsets; /* device [B+1]: 0 = kv_offsets[0] <= ... <= kv_offsets[B] = total_kv */
  const int32_t *q_pos0;     /* device [B]: position of each sequence's first query row           */
} dsa_problem;

/* Workspace selectors for dsa_workspace_bytes(). */
enum { DSA_WS_TOPK = 0, DSA_WS_ATTN = 1, DSA_WS_FORWARD = 2, DSA_WS_INDEXER_BWD = 3,
       DSA_WS_FORWARD_FUSED = 4, DSA_WS_ATTN_PREFILL = 5 };

/*
 * Stage 1, lightning indexer (r.nikiv.dev summary, "How DSA Works"; the
 * ivugangingo.com article, "Sparse attention with almost linear long-context
 * costs").  Writes
 *   scores[r * ld_scores + s] = q_scale[r] * k_scale[s'] *
 *       sum_{j < H_I} w[r*H_I + j] * max(0, sum_{d < d_I} q8[r,j,d] * k8[s',d])
 * for every query row r and every position s <= pos(r), where s' is the
 * packed key row kv_offsets[b] + s and q8/k8 are the decoded e4m3fn values.
 * Entries with s > pos(r) are left untouched.  The scales must be >= 0 (they
 * are applied outside the ReLU; a zero scale gives zero scores).
 * Arithmetic: every e4m3 x e4m3 product is exact in fp32 and the dot products
 * and the head sum accumulate in fp32.  Batches with more than two query rows
 * per sequence take the prefill kernel, which evaluates the head sum as
 *   sum_j (w_j/2) |x_j|  +  Qe . k8,     Qe[d] = sum_j (w_j/2) q8[r,j,d]
 * (ReLU(x) = (x + |x|)/2) with Qe carried as three e4m3 pieces: that term
 * errs by up to about 2^-12 * max_d |Qe[d]| * sum_d |k8[s',d]| (times the
 * scales).  A score that is exactly 0 (every dot product <= 0) can therefore
 * come out as a tiny value of either sign, and the prefill and decode (at
 * most two query rows per sequence) kernels can return slightly different
 * scores, and so a different selection at a near-tie, for the same pair.
 *   q_fp8   [total_q, H_I, d_I] uint8   q_scale [total_q] float
 *   w       [total_q, H_I] float        k_fp8   [total_kv, d_I] uint8
 *   k_scale [total_kv] float            scores  [total_q, ld_scores] float
 * ld_scores >= max_kv_len, a multiple of 4.
 */
dsa_status dsa_indexer_scores(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale,
                              float *scores, int64_t ld_scores, void *stream);

/*
 * Stage 2, fine-grained top-k selector (same passages).  For each query row r
 * with n = pos(r) + 1 candidates, writes the m = min(k, n) positions with the
 * largest scores[r, 0..n-1], in ascending position order, then k - m entries
 * of -1.  Order: larger score first; equal scores (with -0.0 == +0.0) go to
 * the lower position.  Scores must not be NaN.
 *   scores [total_q, ld_scores] float (read on 0..pos(r) only)
 *   topk_idx [total_q, k] int32
 * workspace / workspace_bytes: at least dsa_workspace_bytes(p, DSA_WS_TOPK)
 * bytes of 16-byte aligned device memory (may be NULL when that is 0).  It is
 * zero for batches of more than 512 rows or contexts under 32768; smaller
 * batches of long rows cut each row into segments (at most 32, and few
 * enough that all of them run at once), one workgroup each, whose candidate
 * lists (5632 slots of 8 bytes per segment) live there.
 * Contents need no initialisation and are not preserved.
 */
dsa_status dsa_topk(const dsa_problem *p, const float *scores, int64_t ld_scores,
                    int32_t *topk_idx, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stage 3, sparse MQA/MLA attention over the selected rows (ivugangingo.com
 * article, "Sparse attention with almost linear long-context costs"; stage
 * order as in skillmd.com "Deepseek V3.2 Frontier", "Implementation").  With
 * D = d_latent + d_rope and, for query row r of sequence b, the valid entries
 * i of topk_idx[r] (those in [0, kv_len_b); -1 marks padding):
 *   logit[h, i] = softmax_scale * sum_{d < D} q[r, h, d] * kv[kv_offsets[b] + idx_i, d]
 *   out[r, h, :] = sum_i softmax_i(logit[h, :]) * kv[kv_offsets[b] + idx_i, 0:d_latent]
 *   lse[r, h]    = log(sum_i exp(logit[h, i]))     (natural log)
 * All heads of a token share one gather of its rows.  A row with no valid
 * index gets out = 0 and lse = -inf.  bf16 inputs, fp32 softmax and
 * accumulation, bf16 output rounded to nearest even.
 *   q [total_q, H, D] bf16     kv [total_kv, D] bf16     topk_idx [total_q, k] int32
 *   out [total_q, H, d_latent] bf16                      lse [total_q, H] float (nullable)
 * Supported: (d_latent, d_rope) = (512, 64) with H in {32, 64, 128} and
 * max_kv_len <= 3728270 (the MFMA path; a sequence's rows are addressed with
 * 32-bit byte offsets), or any D <= 1024 with H <= 128 (a plain small-shape
 * path, which also serves other head counts of the 576-wide shape).
 * workspace: at least dsa_workspace_bytes(p, DSA_WS_ATTN) bytes.  It is zero
 * for large batches; batches of fewer than 128 tokens split each token's
 * selected rows over several workgroups and need room for the partial
 * results (nsplit * total_q * H * 1048 bytes).
 */
dsa_status dsa_sparse_attn(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                           const int32_t *topk_idx, uint16_t *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stage 3 in prefill mode: per-head keys and values.  The threadnavigator.com
 * thread on DeepSeek-V3.2 (first tweet) notes separate attention modes for
 * disaggregated prefill and decode; this library reads them as MLA's two
 * forms of one attention.  dsa_sparse_attn is the decode form (one shared
 * latent + rope row per key); here every head has its own key -- a 128-wide
 * part (decompressed from the latent by the caller) followed by the 64-wide
 * rotary key all heads share -- and its own 128-wide value.  For query row r
 * of sequence b, with sel(r) the distinct entries of topk_idx[r] in
 * [0, kv_len_b) and s' = kv_offsets[b] + s:
 *   logit[h, s] = softmax_scale * (q[r, h, 0:128] . k_nope[s', h, :] +
 *                                  q[r, h, 128:192] . k_rope[s', :])
 *   out[r, h, :] = sum_{s in sel(r)} softmax_s(logit[h, :]) * v[s', h, :]
 *   lse[r, h]    = log(sum_{s in sel(r)} exp(logit[h, s]))     (natural log)
 * The selection acts as a mask: unlike dsa_sparse_attn, a position listed
 * twice counts once.  A row with nothing selected gets out = 0, lse = -inf.
 *   q [total_q, H, 192] bf16           k_nope [total_kv, H, 128] bf16
 *   k_rope [total_kv, 64] bf16         v [total_kv, H, 128] bf16
 *   topk_idx [total_q, k] int32        out [total_q, H, 128] bf16
 *   lse [total_q, H] float (nullable)
 * Requires heads in 1..128, d_rope = 64 and max_kv_len <= 131072; d_latent
 * is not used (the per-head widths are fixed).  The work runs over dense
 * 64-key tiles with the selection applied as a bit mask (tiles that no row of
 * a 256-row query block selected are skipped), so its cost follows the
 * selected span rather than k: the form for short prefills, where most of a
 * row's causal keys are selected.  bf16 MFMA, fp32 softmax and accumulation,
 * bf16 output rounded to nearest even.
 * workspace: at least dsa_workspace_bytes(p, DSA_WS_ATTN_PREFILL) bytes,
 * 16-byte aligned (mostly the row masks, about total_q * max_kv_len / 8
 * bytes); its contents need no initialisation.
 */
dsa_status dsa_sparse_attn_prefill(const dsa_problem *p, const uint16_t *q, const uint16_t *k_nope,
                                   const uint16_t *k_rope, const uint16_t *v,
                                   const int32_t *topk_idx, uint16_t *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * The three stages in order (indexer -> top-k -> attention) on one stream:
 * the pipeline of r.nikiv.dev's DeepSeek-V3.2 summary, "How DSA Works" (the
 * indexer scores every causal key, the 2048 best are kept, attention runs on
 * those only) and of the ivugangingo.com article, "Sparse attention with
 * almost linear long-context costs".
 * Arguments as in the stage calls; the results equal the three calls'.  The
 * scores matrix lives at the start of the workspace (ld_scores = max_kv_len
 * rounded up to a multiple of 64); topk_idx_out (nullable) receives the
 * selected positions when given, otherwise they also live in the workspace.
 * workspace: at least dsa_workspace_bytes(p, DSA_WS_FORWARD) bytes.
 */
dsa_status dsa_forward(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                       const float *w, const uint8_t *k_fp8, const float *k_scale,
                       const uint16_t *q, const uint16_t *kv, uint16_t *out, float *lse,
                       int32_t *topk_idx_out, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Paged caches (a serving layout: the FP8 indexer-key cache and the latent KV
 * cache of the decode setting are kept in fixed-size blocks, as the vLLM and
 * SGLang backends the ivugangingo.com article names in "Sparse attention with
 * almost linear long-context costs" do; the pages give no layout, so this one
 * is this library's).  Key position s of sequence b lives in physical block
 * block_table[b * max_blocks + s / block_size], at slot s % block_size:
 *   k_cache  [num_blocks, block_size, d_I] uint8     (e4m3fn)
 *   ks_cache [num_blocks, block_size] float          (per-row key scale)
 *   kv_cache [num_blocks, block_size, d_latent + d_rope] bf16
 * The problem's kv_offsets still give each sequence's length (kv_len_b =
 * kv_offsets[b+1] - kv_offsets[b]); rows are found through the table only.
 * Requirements: block_size a power of two >= 64; max_blocks * block_size >=
 * max_kv_len; num_blocks * block_size < 2^31.  Table entries are clamped to
 * [0, num_blocks), so a bad table gives wrong results but no out-of-bounds
 * access.  The table is a device array of batch * max_blocks int32.
 */
typedef struct dsa_paged_kv {
  const int32_t *block_table; /* device [batch, max_blocks]                        */
  int32_t block_size;         /* key rows per block, a power of two >= 64          */
  int32_t max_blocks;         /* row stride of block_table                         */
  int64_t num_blocks;         /* physical blocks in each cache                     */
} dsa_paged_kv;

/* dsa_indexer_scores over paged key caches: the same scores, with key
 * position s of sequence b read from k_cache / ks_cache through the table. */
dsa_status dsa_indexer_scores_paged(const dsa_problem *p, const dsa_paged_kv *pg,
                                    const uint8_t *q_fp8, const float *q_scale, const float *w,
                                    const uint8_t *k_cache, const float *ks_cache, float *scores,
                                    int64_t ld_scores, void *stream);

/* dsa_sparse_attn over a paged latent KV cache (selected positions are
 * translated through the table).  Workspace as for dsa_sparse_attn. */
dsa_status dsa_sparse_attn_paged(const dsa_problem *p, const dsa_paged_kv *pg, const uint16_t *q,
                                 const uint16_t *kv_cache, const int32_t *topk_idx, uint16_t *out,
                                 float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* dsa_forward over paged caches.  Workspace as for dsa_forward. */
dsa_status dsa_forward_paged(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                             const float *q_scale, const float *w, const uint8_t *k_cache,
                             const float *ks_cache, const uint16_t *q, const uint16_t *kv_cache,
                             uint16_t *out, float *lse, int32_t *topk_idx_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * dsa_forward with the indexer and the selector fused, for decode-shaped
 * problems: at most two query rows per sequence, rows of at most 262144 keys
 * (others: DSA_ERR_UNSUPPORTED).  The indexer's scores serve only the top-k
 * selection (r.nikiv.dev summary, "How DSA Works"), so instead of a scores
 * matrix each 1024-key chunk of a row leaves its keys grouped by their
 * leading 12 bits (an eighth-of-an-octave bin of the score) with a table of
 * its bins; the selection adds up the tables, finds the bin holding the k-th
 * largest score exactly, reads only the keys at or above that bin, and
 * resolves that bin and its ties (lowest position first) among them.  The
 * indices, outputs and lse are bit-identical to dsa_forward's.  No scores
 * are kept.  pg: NULL for packed caches, else the paged caches as for
 * dsa_forward_paged (k_fp8, k_scale and kv are then the caches).
 * workspace: at least dsa_workspace_bytes(p, DSA_WS_FORWARD_FUSED) bytes
 * (about 8 KB per (query row, 1024 keys of max_kv_len), plus the indices and
 * the attention's share).
 * On MI355X this form is slower than dsa_forward for the 64-sequence decode
 * batch: binning inside the bandwidth-bound decode indexer lengthens it by
 * more than the cheaper selection saves.
 */
dsa_status dsa_forward_fused(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                             const float *q_scale, const float *w, const uint8_t *k_fp8,
                             const float *k_scale, const uint16_t *q, const uint16_t *kv,
                             uint16_t *out, float *lse, int32_t *topk_idx_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Indexer alignment loss (training).  The ivugangingo.com article, section
 * "DeepSeek sparse attention pre-training continues": the indexer is trained
 * with a Kullback-Leibler loss towards the main attention's distribution,
 * over all causal keys during the dense warm-up and over the selected keys in
 * the sparse stage, where that loss is the indexer's only gradient source.
 * The pages give no formula; this library computes, for query row r with key
 * set K_r (dense: positions 0..pos(r); sparse: the valid entries of
 * topk_idx[r], as in dsa_sparse_attn):
 *   logit[h, s] = softmax_scale * q[r, h, :] . kv[kv_offsets[b] + s, :]   (as in stage 3)
 *   p_s  = (1/H) sum_h exp(logit[h, s] - lse[r, h])     attention target over K_r
 *   q_s  = exp(I_s) / sum_{s' in K_r} exp(I_s')         I_s = scores[r * ld_scores + s]
 *   loss[r] = sum_{s in K_r} p_s (ln p_s - ln q_s)      (terms with p_s = 0 are 0)
 *   d loss[r] / d I_s = q_s - p_s
 * lse must be the attention's natural-log log-sum-exp over the same K_r (the
 * lse output of dsa_sparse_attn / dsa_forward for the sparse form; of the
 * dense causal attention for the warm-up form): each head's softmax then
 * sums to one, and 1/H normalises the head sum.  The attention side is a
 * fixed target; no gradient flows into q or kv.
 *   q [total_q, H, D] bf16, kv [total_kv, D] bf16, lse [total_q, H] float
 *   scores [total_q, ld_scores] float (read at the positions of K_r only)
 *   topk_idx [total_q, k] int32, or NULL for the dense warm-up form
 *   loss [total_q] float
 *   grad: sparse, [total_q, ld_grad] with entry i of row r the derivative for
 *         topk_idx[r, i] (0 where that entry is skipped; entries i >= k are
 *         not written), ld_grad >= k; dense, [total_q, ld_grad] by position,
 *         positions 0..pos(r) written, the rest untouched, ld_grad >=
 *         max_kv_len.
 * dsa_forward keeps its scores at the start of its workspace with
 * ld_scores = max_kv_len rounded up to a multiple of 64, so a training step
 * may pass that pointer (with topk_idx_out and lse from the same call).
 * Shapes as for dsa_sparse_attn; fp32 arithmetic on bf16 products (MFMA for
 * the (512, 64) shape).  The dense form costs O(pos) per row.
 */
dsa_status dsa_indexer_align_loss(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                                  const float *lse, const float *scores, int64_t ld_scores,
                                  const int32_t *topk_idx, float *loss, float *grad,
                                  int64_t ld_grad, void *stream);

/*
 * Backward of the lightning indexer (training): carries a gradient on the
 * scores -- the alignment loss's grad above -- back to the indexer's inputs
 * (the ivugangingo.com article, "DeepSeek sparse attention pre-training
 * continues": the indexer is what that loss trains).  With q~ = q_scale * q8
 * and k~ = k_scale * k8 the dequantised values, z[j, s] = q~[r, j] . k~[s],
 * and G[r, s] the given gradient over row r's keys K_r (dense: positions
 * 0..pos(r); sparse: the valid entries of topk_idx[r], a key listed twice
 * counting twice, in any order):
 *   dw[r, j]     = sum_{s in K_r} G[r, s] * ReLU(z[j, s])
 *   dq[r, j, :]  = sum_{s in K_r} G[r, s] * w[r, j] * [z[j, s] > 0] * k~[s, :]
 *   dk[b, s, :] += sum_{r of b} sum_j G[r, s] * w[r, j] * [z[j, s] > 0] * q~[r, j, :]
 * (the ReLU's derivative at 0 is taken as 0, so a row or key whose scale is
 * 0 -- scales are >= 0 as for dsa_indexer_scores -- has z = 0 and passes no
 * gradient through the mask).  dq and dw are gradients with
 * respect to the dequantised q~ and w and are overwritten; dk, with respect
 * to k~, is ADDED to (a key is shared by many rows and, in a chunked
 * prefill, by several calls), in an order that varies from run to run, so
 * the caller zeroes it once per step.
 *   q_fp8, q_scale, w, k_fp8, k_scale as for dsa_indexer_scores
 *   topk_idx [total_q, k] int32, or NULL for the dense form
 *   grad: sparse [total_q, ld_grad] aligned with topk_idx (ld_grad >= k);
 *         dense [total_q, ld_grad] by position (ld_grad >= max_kv_len)
 *   dq [total_q, H_I, d_I] float   dw [total_q, H_I] float   dk [total_kv, d_I] float
 * The (H_I, d_I) = (64, 128) shape runs on MFMA: the mask is decided on the
 * fp32 dot product of the exact e4m3 values and the products use bf16
 * operands with the gradient split into two bf16 terms (about 2^-17
 * relative), fp32 accumulation.  Other shapes take a plain fp32 path.
 *   workspace / workspace_bytes: optional.  NULL: dk is added to with fp32
 *         atomics (dk must then be ordinary device memory, hipMalloc).  In
 *         the sparse form on the (64, 128) shape a workspace of at least
 *         dsa_workspace_bytes(p, DSA_WS_INDEXER_BWD) bytes (16-byte aligned;
 *         about total_q * k * 516 bytes) selects the faster two-pass form:
 *         each (row, key) contribution is stored there and a second kernel
 *         sums them per key, 64 keys per workgroup, and adds the sums to dk
 *         (about one atomic per dk element per 4096 rows instead of one per
 *         row that selected the key).  Its contents need no initialisation
 *         and are overwritten.  Other forms ignore it.  Too small:
 *         DSA_ERR_WORKSPACE.  dk must be ordinary device memory either way.
 * Calls that overlap on one stream's timeline and add into the same dk rows
 * must be ordered by the caller (the two-pass form reads and writes dk).
 */
dsa_status dsa_indexer_backward(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                                const float *w, const uint8_t *k_fp8, const float *k_scale,
                                const int32_t *topk_idx, const float *grad, int64_t ld_grad,
                                float *dq, float *dw, float *dk, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid it).  The workspace dsa_forward
 * would take is a fixed device array of DSA_NOALLOC_SCRATCH_BYTES inside the
 * library instead: one per GPU, created when the library's code is first
 * loaded on that GPU and held until the process ends.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Arguments and results as for dsa_forward, on the current device (stream
 * must belong to it).  Problems whose dsa_workspace_bytes(p, DSA_WS_FORWARD)
 * exceeds DSA_NOALLOC_SCRATCH_BYTES are refused with DSA_ERR_UNSUPPORTED
 * before anything is enqueued (the decode batch of 64 sequences at 128K
 * context and prefills of a few thousand tokens fit).  Every call on a GPU
 * shares that GPU's array, whose contents need no initialisation and are
 * left as the last call wrote them: calls that overlap in time on one GPU
 * (different streams or host threads without ordering between them) race
 * on it and give wrong results.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
dsa_status dsa_forward_noalloc(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                               const float *w, const uint8_t *k_fp8, const float *k_scale,
                               const uint16_t *q, const uint16_t *kv, uint16_t *out, float *lse,
                               int32_t *topk_idx_out, void *stream);

/* Bytes of device workspace the given entry point needs for problem p
 * (which = DSA_WS_TOPK, DSA_WS_ATTN, DSA_WS_FORWARD, DSA_WS_FORWARD_FUSED, or
 * DSA_WS_INDEXER_BWD for the two-pass form of dsa_indexer_backward); 0 if
 * none.  Returns
 * (size_t)-1 for an invalid problem (see dsa_last_error).  The paged entry
 * points need the same amounts. */
size_t dsa_workspace_bytes(const dsa_problem *p, int which);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *dsa_last_error(void);

/* Library version string, e.g. "dsa 0.1.0 gfx950". */
const char *dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
