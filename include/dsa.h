/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD MI355X (gfx950).
 *
 * The path has three steps, each a hand-written HIP kernel family, and a step
 * before them that produces the operands of a new token (step 0 below):
 *   1. lightning-indexer scores   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]),  s <= t
 *      (DeepSeek-V3.2-Exp paper as translated on the m.163.com page, section 1
 *      "Architecture", Eq. 1 and the prose around it: few indexer heads, ReLU,
 *      FP8 arithmetic);
 *   2. fine-grained top-k selection of the k highest-scoring positions per query
 *      (same paper, section 1 text after Eq. 1, and section 2.1 "sparse training
 *      stage": S_t and k = 2048);
 *   3. sparse MLA attention in MQA mode over the selected latent entries, every
 *      entry shared by all query heads (same paper, section 1 Eq. 2 and
 *      "Instantiate DSA under MLA"; Appendix A, Fig. 4).  Key = the whole
 *      qk_dim-wide entry (latent + rope part), value = its first v_dim columns.
 *      The page "DeepSeek-V3.2开源技术报告" (nsmao.com, "DSA principle") gives the
 *      cache widths: 128 per token for the indexer key, 512 for the latent.
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors are
 *     dense, row-major, 16-byte aligned.  The library allocates nothing: scratch
 *     comes from the caller's workspace.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the device.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     status other than DSA_OK nothing was enqueued, except DSA_E_HIP, which
 *     reports a failed launch (earlier launches of the same call may have run).
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Thread-safe and re-entrant: no global mutable state except the per-thread
 *     text behind dsa_last_error() and the per-device index-domain flag (a
 *     debugging aid, see dsa_check_index_domain).
 *   - No C++ exception crosses this interface.
 *
 * Row model: a call processes R query rows.  Row r belongs to sequence
 * row_seq[r] (in [0, B)) and sits at position t = row_pos[r] (in [0, max_pos]) of
 * that sequence; its candidates are the positions 0..t (inclusive).  Caches are
 * per sequence with capacity N = max_ctx entries.  Rows whose row_seq or row_pos
 * is out of range are not processed (their outputs are left unspecified) and
 * cause no out-of-bounds access.
 *
 * Supported dimension sets (anything else returns DSA_E_UNSUPPORTED):
 *   - production: H_I = 64, d_I = 128, fp8 e4m3fn indexer operands with fp32
 *     scales; H = 128, D_k = 576, D_v = 512, bf16 attention operands; topk = 2048.
 *   - fp32: idx_dtype = attn_dtype = DSA_F32 with H_I <= 64, d_I <= 128,
 *     H <= 128, D_v <= D_k <= 576, topk <= 2048 (correctness configuration; plain
 *     fp32 vector kernels).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_API_VERSION 2

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_E_INVALID = 1,     /* null pointer, negative or inconsistent size */
  DSA_E_UNSUPPORTED = 2, /* dimension / dtype combination with no kernel */
  DSA_E_WORKSPACE = 3,   /* workspace missing or smaller than required */
  DSA_E_HIP = 4          /* a HIP runtime call or launch failed */
} dsa_status;

typedef enum dsa_dtype {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3FN = 2 /* OCP 8-bit E4M3, finite-only ("fn"), bias 7, max 448 */
} dsa_dtype;

/* Query rows of one call.  The two arrays live in device memory; every other
 * field is a host value. */
typedef struct dsa_rows {
  int32_t num_rows;       /* R >= 0 */
  int32_t num_seqs;       /* B >= 1 */
  int32_t max_ctx;        /* N >= 1: cache capacity per sequence, in entries */
  int32_t max_pos;        /* host upper bound of row_pos[*]: 0 <= max_pos < N */
  const int32_t* row_seq; /* device [R] */
  const int32_t* row_pos; /* device [R] */
} dsa_rows;

typedef struct dsa_dims {
  int32_t n_idx_heads; /* H_I: indexer heads */
  int32_t idx_dim;     /* d_I: indexer query/key width */
  int32_t n_heads;     /* H: attention query heads (all share each latent entry) */
  int32_t qk_dim;      /* D_k: latent entry width (latent + rope) */
  int32_t v_dim;       /* D_v: value width = leading columns of the entry */
  int32_t topk;        /* k: positions selected per row */
  dsa_dtype idx_dtype; /* DSA_FP8_E4M3FN or DSA_F32 */
  dsa_dtype attn_dtype;/* DSA_BF16 or DSA_F32 */
} dsa_dims;

/* ---------------------------------------------------------------------------
 * Step 1: indexer scores.
 *   q_idx   [R, H_I, d_I]  fp8 codes (uint8) or fp32, per idx_dtype
 *   q_scale [R, H_I]  fp32 > 0, dequantisation scale of each q vector (fp8 only;
 *                     ignored and may be NULL for fp32)
 *   w       [R, H_I]  fp32 head weights (any sign)
 *   k_idx   [B, N, d_I] fp8 codes or fp32
 *   k_scale [B, N]    fp32 > 0 (fp8 only; may be NULL for fp32)
 *   scores  [R, ld_scores] fp32 output, ld_scores >= max_pos + 1
 * For row r with t = row_pos[r], b = row_seq[r] and every s in [0, t]:
 *   scores[r*ld + s] = sum_j w[r,j] * max(0, (q_scale[r,j] q_idx[r,j,:]) . (k_scale[b,s] k_idx[b,s,:]))
 * with the 128-term fp8 dots formed by the gfx950 fp8 MFMA: exact products,
 * summed in 16 groups of 8 (bytes [8m, 8m + 8) of both vectors) in which each
 * product is cut toward zero to a multiple of 2^-13 of the group's largest
 * |product|, the group sums then added with fp32 rounding; so a dot is off by at
 * most 7 * 2^-13 per unit of each group's largest |product| plus fp32 rounding
 * (measured against exact sums).  The epilogue (scales, ReLU, weighted head sum)
 * is fp32.  Entries s > t are not candidates: the call may write -inf to some of them and leaves the rest
 * untouched.  Positive scales are required (they are folded through the ReLU).
 * ------------------------------------------------------------------------- */
dsa_status dsa_indexer_scores(const dsa_rows* rows, const dsa_dims* dims,
                              const void* q_idx, const float* q_scale, const float* w,
                              const void* k_idx, const float* k_scale,
                              float* scores, int64_t ld_scores, void* stream);

/* ---------------------------------------------------------------------------
 * Step 2: top-k selection.
 *   scores  [R, ld_scores] fp32 (only s <= row_pos[r] is read)
 *   indices [R, topk] int32 output
 * Row r selects exactly n = min(topk, t+1) positions: those with the largest
 * scores, equal scores taken from the lowest position first (-0.0 equals +0.0).
 * indices[r, 0..n) hold them in ascending order, indices[r, n..topk) hold -1.
 * Supports topk in [1, 4096] and rows of up to 131072 candidates: max_pos + 1 >
 * 131072 returns DSA_E_UNSUPPORTED before anything is enqueued.  Scores must not be
 * NaN (a NaN row gives an unspecified but in-range selection).  Calls with fewer
 * than 128 rows whose max_pos + 1 exceeds 32768 split each row over several
 * blocks and need a workspace of dsa_topk_workspace_size bytes (candidates and
 * per-row counts, cleared by the call itself); otherwise the size is 0 and
 * workspace may be NULL.
 * ------------------------------------------------------------------------- */
size_t dsa_topk_workspace_size(const dsa_rows* rows, int32_t topk);

dsa_status dsa_topk(const dsa_rows* rows, int32_t topk, const float* scores,
                    int64_t ld_scores, int32_t* indices, void* workspace, size_t ws_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------
 * Step 3: sparse MLA attention (MQA mode).
 *   q       [R, H, D_k]  bf16 or fp32 per attn_dtype
 *   latent  [B, N, D_k]  bf16 or fp32
 *   indices [R, topk] int32: positions to attend; entries outside [0, t] are
 *           padding (causal rule of the selection: S_t holds preceding positions).
 *           An entry past t also sets the device's index-domain flag, which
 *           dsa_check_index_domain reports; -1 and other negatives are plain padding.
 *   out     [R, H, D_v]  bf16 or fp32 output
 *   lse     [R, H] fp32 output (natural log of the softmax denominator), or NULL
 * For each row r and head h over the listed positions S:
 *   z[s] = softmax_scale * q[r,h,:] . latent[b,s,:]
 *   out[r,h,:] = sum_s softmax(z)[s] * latent[b,s,0:D_v],  lse[r,h] = log sum_s e^z[s]
 * A listed position counts once per occurrence.  A row with no valid position
 * gets out = 0 and lse = -inf.  bf16 path: bf16 products, fp32 accumulation and
 * softmax, softmax weights rounded to bf16 for the value product, out rounded to
 * nearest-even bf16.  When few rows cannot fill the GPU, a row's positions are
 * split into S slices; the workspace then holds each slice's normalised output
 * (bf16) and its lse (fp32), merged as out = sum_i e^(lse_i - LSE) out_i in fp32
 * (see dsa_sparse_mla_attn_workspace_size; 0 bytes when no row is split).
 * A contiguous bf16 latent cache is addressed with 32-bit byte offsets per
 * sequence: max_ctx * D_k * 2 must stay below 4 GiB (else DSA_E_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
size_t dsa_sparse_mla_attn_workspace_size(const dsa_rows* rows, const dsa_dims* dims);

dsa_status dsa_sparse_mla_attn(const dsa_rows* rows, const dsa_dims* dims,
                               const void* q, const void* latent, const int32_t* indices,
                               float softmax_scale, void* out, float* lse,
                               void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Whole path: the scoring, selection and sparse-attention steps of the DSA
 * workflow ("DeepSeek-V3.2开源技术报告", "DSA principle": after the query and key
 * projection, the indexer scores the preceding tokens, the top-k are selected,
 * and sparse attention runs over them), i.e. step 1 -> step 2 -> step 3 for all
 * R rows, processed in chunks of
 * chunk_rows rows (0 = all rows at once) so the score workspace stays bounded.
 * Inputs are those of the three steps; outputs out/lse as in step 3, plus the
 * selected positions in indices_out [R, topk] when it is not NULL.  The workspace
 * must be at least dsa_forward_workspace_size(rows, dims, chunk_rows) bytes.
 * The limits of steps 2 and 3 apply (max_pos + 1 <= 131072; contiguous latent
 * below 4 GiB per sequence); they are checked before anything is enqueued.
 * ------------------------------------------------------------------------- */
size_t dsa_forward_workspace_size(const dsa_rows* rows, const dsa_dims* dims, int32_t chunk_rows);

dsa_status dsa_forward(const dsa_rows* rows, const dsa_dims* dims,
                       const void* q_idx, const float* q_scale, const float* w,
                       const void* k_idx, const float* k_scale,
                       const void* q, const void* latent, float softmax_scale,
                       void* out, float* lse, int32_t* indices_out,
                       int32_t chunk_rows, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_forward without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, computation, kernels and results as dsa_forward;
 * the scratch is a fixed 64 MiB device array inside the library (one per GPU,
 * held until the process ends), so nothing is allocated.  A call whose
 * dsa_forward_workspace_size exceeds 64 MiB returns DSA_E_WORKSPACE before
 * anything is enqueued (decode batches fit: 32 rows at 32K context use 38 MB;
 * prefill needs small chunk_rows).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams or threads) race
 * and must be serialised by the caller.  The array's previous contents are never
 * read (no part of it needs to start at zero).
 * ------------------------------------------------------------------------- */
dsa_status dsa_forward_noalloc(const dsa_rows* rows, const dsa_dims* dims,
                               const void* q_idx, const float* q_scale, const float* w,
                               const void* k_idx, const float* k_scale,
                               const void* q, const void* latent, float softmax_scale,
                               void* out, float* lse, int32_t* indices_out,
                               int32_t chunk_rows, void* stream);

/* ---------------------------------------------------------------------------
 * Step 0: projections of new tokens with fp8 quantisation and cache append.
 * The first step of the DSA workflow, before indexer scoring ("DeepSeek-V3.2开源技术
 * 报告", "DSA principle": query and key projection; DeepSeek-V3.2-Exp paper,
 * section 1, text around Eq. 1: q[t,j] and w[t,j] are derived from the query token
 * h_t, k[s] from the token h_s).  Production dims only (H_I = 64, d_I = 128,
 * D_k = 576, idx_dtype fp8, attn_dtype bf16; the other dims fields are ignored).
 *   h      [R, d_model] bf16: row r is the token at position row_pos[r] of sequence
 *          row_seq[r]
 *   w_q    [H_I*d_I, d_model] bf16, head j = rows j*d_I .. j*d_I + d_I - 1
 *   w_k    [d_I, d_model] bf16;  w_c [D_k, d_model] bf16;  w_w [H_I, d_model] bf16
 * With y = W h[r] (exact bf16 products, fp32 accumulation) the call writes
 *   q_idx  [R, H_I, d_I] e4m3fn codes and q_scale [R, H_I] fp32
 *   w      [R, H_I] fp32
 *   k_idx  [B, N, d_I] codes and k_scale [B, N]: the row (row_seq[r], row_pos[r])
 *   latent [B, N, D_k] bf16 (round to nearest even): the row (row_seq[r], row_pos[r])
 * Each 128-wide vector (one per (token, head) for q, one per token for k) is
 * quantised with scale = 2^e, e the smallest integer with max|y| <= 448 * 2^e
 * (scale 1 when max|y| = 0), and code = e4m3fn round-to-nearest-even of y / scale,
 * the format dsa_indexer_scores reads.  Rows whose row_seq or row_pos is out of
 * range still get q_idx, q_scale and w but write no cache row; two rows naming the
 * same cache row leave one of them (unspecified which).  Every other cache row is
 * left untouched.  d_model must be a positive multiple of 64 (at most 65536).
 * RoPE is not applied.  Few rows split the contraction over blocks; the workspace
 * then holds the fp32 partial sums (dsa_project_append_workspace_size; 0 bytes
 * when nothing is split).
 * ------------------------------------------------------------------------- */
size_t dsa_project_append_workspace_size(const dsa_rows* rows, int32_t d_model);

dsa_status dsa_project_append(const dsa_rows* rows, const dsa_dims* dims, int32_t d_model,
                              const void* h, const void* w_q, const void* w_k, const void* w_c,
                              const void* w_w, void* q_idx, float* q_scale, float* w,
                              void* k_idx, float* k_scale, void* latent, void* workspace,
                              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Paged ("dynamic") caches.  The serving path keeps its KV caches dynamic
 * ("DeepSeek-V3.2开源技术报告", "DSA principle": optimised kernels with a dynamic KV
 * cache); here that is a pool of fixed-size pages seen through a block table.
 * Entry s of sequence b is entry s % P of pool page block_table[b * pages_per_seq
 * + s / P], for the indexer-key pool, its scale pool and the latent pool alike
 * (one table for all three).  The _paged calls compute exactly what their
 * contiguous forms compute on the caches these views describe; workspace sizes
 * are those of the contiguous forms.
 *   - Production dims only; page_size a power of two in [64, 65536];
 *     rows->max_ctx must equal pages_per_seq * page_size; each pool < 4 GiB.
 *   - Pools: k_pool [num_pages, P, d_I] fp8 codes, k_scale_pool [num_pages, P] fp32,
 *     latent_pool [num_pages, P, D_k] bf16.
 *   - block_table entries outside [0, num_pages) are read as page 0 (the result is
 *     unspecified; nothing outside the pools is accessed).
 * ------------------------------------------------------------------------- */
typedef struct dsa_pages {
  int32_t page_size;          /* P: entries per page */
  int32_t pages_per_seq;      /* columns of block_table */
  int32_t num_pages;          /* pages in each pool */
  const int32_t* block_table; /* device [B, pages_per_seq] */
} dsa_pages;

dsa_status dsa_indexer_scores_paged(const dsa_rows* rows, const dsa_dims* dims,
                                    const dsa_pages* pages, const void* q_idx,
                                    const float* q_scale, const float* w, const void* k_pool,
                                    const float* k_scale_pool, float* scores, int64_t ld_scores,
                                    void* stream);

dsa_status dsa_sparse_mla_attn_paged(const dsa_rows* rows, const dsa_dims* dims,
                                     const dsa_pages* pages, const void* q,
                                     const void* latent_pool, const int32_t* indices,
                                     float softmax_scale, void* out, float* lse, void* workspace,
                                     size_t ws_bytes, void* stream);

dsa_status dsa_forward_paged(const dsa_rows* rows, const dsa_dims* dims, const dsa_pages* pages,
                             const void* q_idx, const float* q_scale, const float* w,
                             const void* k_pool, const float* k_scale_pool, const void* q,
                             const void* latent_pool, float softmax_scale, void* out, float* lse,
                             int32_t* indices_out, int32_t chunk_rows, void* workspace,
                             size_t ws_bytes, void* stream);

/* Step 0 into paged caches: the appended indexer key, its scale and the latent
 * entry of row r go to logical entry (row_seq[r], row_pos[r]) of the pools. */
dsa_status dsa_project_append_paged(const dsa_rows* rows, const dsa_dims* dims,
                                    const dsa_pages* pages, int32_t d_model, const void* h,
                                    const void* w_q, const void* w_k, const void* w_c,
                                    const void* w_w, void* q_idx, float* q_scale, float* w,
                                    void* k_pool, float* k_scale_pool, void* latent_pool,
                                    void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Indexer training loss of the sparse stage (DeepSeek-V3.2-Exp paper, section 2.1,
 * "sparse training stage": the indexer output is aligned with the main attention
 * distribution over the selected set S_t only, by a KL divergence; the indexer's
 * inputs are detached from the main model).  Production dims only.
 *
 * dsa_indexer_loss, for each row r with S = {indices[r, i] in [0, t]}:
 *   u_i   = sum_h exp(softmax_scale q[r,h,:] . latent[b,s_i,:] - lse[r,h])   (target)
 *   p_i   = u_i / sum_i u_i       (the heads' attention weights summed, L1-normalised)
 *   loss[r]        = sum_i p_i (log p_i - log softmax_S(scores[r, s_i]))
 *   dscores[r, i]  = softmax_S(scores[r, s_i]) - p_i   (0 at padding entries)
 * lse is the attention call's lse output for the same indices; scores the indexer
 * scores [R, ld_scores].  fp32 throughout; the target recomputes the q.c products on
 * the bf16 MFMA.  The workspace holds u (dsa_indexer_loss_workspace_size bytes).
 *
 * dsa_indexer_backward, with d = (q_scale q_idx[r,j,:]) . (k_scale k_idx[b,s,:]) and
 * m = [d > 0], for every selected entry s_i of row r and every head j:
 *   dw[r,j]      += dscores[r,i] * max(d, 0)
 *   dq[r,j,:]    += dscores[r,i] * w[r,j] * m * (k_scale k_idx[b,s_i,:])
 *   dk[b,s_i,:]  += dscores[r,i] * w[r,j] * m * (q_scale q_idx[r,j,:])
 * i.e. the gradients of sum_i dscores[r,i] I[r,s_i] with respect to w and the
 * dequantised indexer queries and keys.  dq [R, H_I, d_I], dw [R, H_I] and
 * dk [B, N, d_I] are fp32 and ACCUMULATED (the caller zeroes them).  The dots are
 * the forward's (the fp8 MFMA's dots, see dsa_indexer_scores).  The two products
 * run on the bf16 MFMA with fp32 accumulation: the fp8 codes are bf16 values
 * exactly, and each fp32 coefficient enters as three bf16 parts that sum to it (to
 * within 2^-25 of it).  Contiguous caches only.
 *
 * Every sum is formed in an order fixed by the call's shape, so the outputs are the
 * same bits from run to run: dq and dw from per-chunk sums added in chunk order;
 * dk of a key selected once in the call by its one writer; dk of a key selected
 * more than once (rows of one sequence sharing keys, or an index list that repeats
 * a position) as an exact 64-bit fixed-point sum, added into dk once.  The
 * fixed-point step is 2^-s for the largest s with (largest selection count) x
 * (bound on one contribution) < 2^62; the bound is max |dscores| over the call
 * times the largest over rows of max_d sum_j |w[r,j]| |q_scale q_idx[r,j,d]|, so
 * each contribution is rounded to within 2^-(s+1) and no sum overflows.
 *
 * Workspace (dsa_indexer_backward_workspace_size(rows, dims, shared_keys)): the
 * selection counts of the B (max_pos + 1) keys, the per-chunk sums of dq and dw,
 * and room for shared_keys fixed-point accumulators (1 KiB each); shared_keys = -1
 * gives room for the most the call's shape allows, min(B (max_pos + 1), R k / 2).
 * The call takes any ws_bytes from the size for shared_keys = 0 up, and uses what
 * is left for accumulators.  Keys selected more than once beyond those
 * accumulators, and all of them when the bound is not finite (inf or NaN inputs),
 * are added into dk with fp32 atomics, whose order and last bits vary.  A call in
 * which no key is selected twice (one row per sequence, as at decode) needs no
 * accumulators: shared_keys = 0 keeps it deterministic.  Below that size:
 * DSA_E_WORKSPACE.
 * max_pos + 1 <= 131072 and num_seqs * (max_pos + 1) < 2^31, else DSA_E_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
size_t dsa_indexer_loss_workspace_size(const dsa_rows* rows, const dsa_dims* dims);

dsa_status dsa_indexer_loss(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                            const void* latent, const int32_t* indices, const float* lse,
                            float softmax_scale, const float* scores, int64_t ld_scores,
                            float* loss, float* dscores, void* workspace, size_t ws_bytes,
                            void* stream);

/* Dense warm-up loss of the indexer (DeepSeek-V3.2-Exp paper, section 2.1, "dense
 * warm-up stage": with the main attention dense, the indexer is trained with the
 * KL divergence to the heads' attention weights summed and L1-normalised over all
 * preceding positions).  Production dims only.  For each row r at position t:
 *   lse[h]  = log sum_{s<=t} exp(softmax_scale q[r,h,:] . latent[b,s,:])
 *   u_s     = sum_h exp(softmax_scale q[r,h,:] . latent[b,s,:] - lse[h]),  p = u / sum_s u_s
 *   loss[r]         = sum_{s<=t} p_s (log p_s - log softmax_{s<=t}(scores[r,s]))
 *   dscores[r, s]   = softmax_{s<=t}(scores[r,s]) - p_s for s <= t, 0 for t < s < ld_scores
 * scores and dscores are [R, ld_scores] fp32; every causal position is read, so the
 * cost is that of dense attention (two passes of q.c on the bf16 MFMA, in chunks of
 * 1024 positions; fp32 softmax sums).  The workspace holds the target and the
 * per-chunk partial sums (dsa_indexer_loss_dense_workspace_size bytes).  Rows whose
 * sequence or position is out of range (including t > max_pos) get loss 0 and a
 * zero dscores row, and read nothing past the workspace.
 */
size_t dsa_indexer_loss_dense_workspace_size(const dsa_rows* rows, const dsa_dims* dims);

dsa_status dsa_indexer_loss_dense(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                                  const void* latent, float softmax_scale, const float* scores,
                                  int64_t ld_scores, float* loss, float* dscores, void* workspace,
                                  size_t ws_bytes, void* stream);

/* Backward of the dense warm-up loss into the indexer: dsa_indexer_backward's
 * products with every causal position s <= t as an entry and dscores [R, ld_dscores]
 * indexed by position (the dscores of dsa_indexer_loss_dense):
 *   dw[r,j] += dscores[r,s] max(d, 0),  dq[r,j,:] += dscores[r,s] w[r,j] m k_s,
 *   dk[b,s,:] += dscores[r,s] w[r,j] m q_j          for all s <= t(r)
 * Same formats, accumulation (caller-zeroed), summation order, workspace rules and
 * arithmetic as dsa_indexer_backward, with t + 1 entries per row in place of k
 * (shared_keys = -1 here means min(B (max_pos + 1), R (max_pos + 1) / 2)).
 * Contiguous caches; production dims. */
size_t dsa_indexer_backward_dense_workspace_size(const dsa_rows* rows, const dsa_dims* dims,
                                                 int64_t shared_keys);

dsa_status dsa_indexer_backward_dense(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                                      const float* q_scale, const float* w, const void* k_idx,
                                      const float* k_scale, const float* dscores,
                                      int64_t ld_dscores, float* dq, float* dw, float* dk,
                                      void* workspace, size_t ws_bytes, void* stream);

size_t dsa_indexer_backward_workspace_size(const dsa_rows* rows, const dsa_dims* dims,
                                           int64_t shared_keys);

dsa_status dsa_indexer_backward(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                                const float* q_scale, const float* w, const void* k_idx,
                                const float* k_scale, const int32_t* indices,
                                const float* dscores, float* dq, float* dw, float* dk,
                                void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Masked MHA mode for short prefill (DeepSeek-V3.2-Exp paper, section 3: short-
 * sequence prefill runs a masked MHA mode that simulates DSA; Appendix A, Fig. 4:
 * MLA's MHA mode).  Each head decompresses its own key and value from the latent:
 *   k[h,s] = [w_uk[h] latent[b,s,0:512] ; latent[b,s,512:576]],  v[h,s] = w_uv[h] latent[b,s,0:512]
 * and row r attends per head over its selected positions S (indices[r,:] in [0, t]):
 *   out[r,h,:] = sum_{s in S} softmax_s(softmax_scale q[r,h,:] . k[h,s]) v[h,s],
 *   lse[r,h] = log sum_{s in S} e^(softmax_scale q[r,h,:] . k[h,s])
 * This equals w_uv[h] times the MQA-mode output (dsa_sparse_mla_attn) for the
 * absorbed query [w_uk[h]^T q[r,h,0:128] ; q[r,h,128:192]].
 *   q     [R, H, 192] bf16 (128 nope + 64 rope dims per head)
 *   w_uk  [H, 128, 512] bf16, w_uv [H, 128, 512] bf16
 *   out   [R, H, 128] bf16; lse [R, H] fp32 or NULL
 * Production dims; max_pos + 1 <= 16384.  Rows may belong to any sequences in any
 * order: a tile of 128 consecutive rows makes one pass over the keys per distinct
 * sequence among its rows, so rows grouped by sequence cost least.  Rows whose
 * sequence or position is out of range are not written.  The workspace holds the
 * decompressed keys and values of positions [0, max_pos] and the selection mask
 * (dsa_mha_prefill_workspace_size).  bf16 MFMA with fp32 accumulation and softmax;
 * decompressed keys and values and the softmax weights are rounded to bf16.
 * ------------------------------------------------------------------------- */
size_t dsa_mha_prefill_workspace_size(const dsa_rows* rows, const dsa_dims* dims);

dsa_status dsa_mha_prefill(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                           const void* latent, const void* w_uk, const void* w_uv,
                           const int32_t* indices, float softmax_scale, void* out, float* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/* Index-domain check (a debugging aid for callers that build index lists
 * themselves).  Sets *seen to 1 if an attention kernel on the calling thread's
 * current device met an index entry past its row's position t since the last
 * check (such entries are padding in the result), else 0, and clears the flag.
 * Synchronises the device first.  Returns DSA_E_HIP if a runtime call fails. */
dsa_status dsa_check_index_domain(int32_t* seen);

/* Status text, and the detail of the last failure on the calling thread. */
const char* dsa_status_string(dsa_status status);
const char* dsa_last_error(void);
int32_t dsa_api_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
