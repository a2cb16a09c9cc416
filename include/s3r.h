/*
 * s3r.h - C ABI of libs3r.so: the decode hot path of Self-Sparse Speculative
 * Rollouts (S3R) on AMD Instinct MI355X (gfx950).
 *
 * S3R drafts a block of gamma tokens with the policy itself, reading a sparse
 * budget of its own KV history, then verifies the gamma + 1 block queries with
 * full attention over the complete KV cache and keeps or corrects the drafts by
 * exact speculative sampling, so the emitted tokens follow the dense policy
 * (abstract of "S^3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative
 * Decoding"; wispaper.ai, "S3R drafts sparsely and verifies densely").
 *
 * Conventions shared by every call
 *   - Every pointer is a device pointer unless stated otherwise. Buffers are
 *     owned by the caller, contiguous, row-major in the stated shape. The KV
 *     caches, queries and logits must be 16-byte aligned (INVALID_VALUE
 *     otherwise): the kernels read them with 16-byte vector loads.
 *   - The library allocates nothing and keeps no mutable global state; calls
 *     are reentrant. Calls sharing one workspace must be ordered on one stream.
 *   - Calls are asynchronous: they only enqueue kernels on `stream` (a
 *     hipStream_t, NULL for the default stream). Outputs are valid once the
 *     stream reaches that point; inputs must stay alive until then.
 *   - Everything the host can check is checked before any launch. On failure
 *     the call returns a status, launches nothing and leaves outputs untouched.
 *     A launch failure reported by the runtime returns S3R_ERROR_HIP.
 *   - Device-resident values (context lengths, page ids, token ids) cannot be
 *     checked without a host sync. Their preconditions are stated per call;
 *     kernels clamp page and block indices so that out-of-range values never
 *     reach memory outside the buffers described here, but the results are then
 *     unspecified.
 *
 * Paged KV cache layout (one layer), page size P = 16 tokens:
 *   k_cache[num_blocks][num_kv_heads][P][head_dim]
 *   v_cache[num_blocks][num_kv_heads][head_dim][P]   (V is page-transposed)
 *   page_table[num_seqs][max_pages_per_seq]  logical page -> physical block
 *   Token t of sequence b is slot t % P of block page_table[b][t / P].
 *   ctx_lens[num_seqs] is the committed length L_b: positions 0 .. L_b - 1
 *   hold history; the pending token sits at position L_b.
 *   The attention kernels read whole pages: the slots of a page past the last
 *   position a call attends are read and given weight zero. Those slots must
 *   hold finite values (a zero weight times a NaN or an infinity is not zero),
 *   e.g. a block pool cleared once when it is allocated; s3r_check_step_inputs
 *   reports a step whose pages break this (S3R_CHECK_SLOT).
 */
#ifndef S3R_H_
#define S3R_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  S3R_SUCCESS = 0,
  S3R_ERROR_INVALID_VALUE = 1,         /* NULL pointer, bad size or inconsistent shape  */
  S3R_ERROR_NOT_SUPPORTED = 2,         /* valid but outside what the kernels implement */
  S3R_ERROR_INSUFFICIENT_WORKSPACE = 3,
  S3R_ERROR_HIP = 4                    /* the HIP runtime reported an error            */
} s3r_status;

typedef enum { S3R_F32 = 0, S3R_BF16 = 1 } s3r_dtype;

/* The paged KV cache of one layer. All pointers are device pointers. */
typedef struct {
  void* k_cache;               /* [num_blocks][num_kv_heads][16][head_dim], dtype  */
  void* v_cache;               /* [num_blocks][num_kv_heads][head_dim][16], dtype  */
  const int32_t* page_table;   /* [num_seqs][max_pages_per_seq]                    */
  const int32_t* ctx_lens;     /* [num_seqs] committed lengths L_b                 */
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t page_size;           /* must be 16                                       */
  int32_t head_dim;            /* 64 or 128                                        */
  int32_t max_pages_per_seq;
  int32_t dtype;               /* s3r_dtype of k_cache, v_cache, queries, outputs */
} s3r_paged_kv;

/* Text of a status code (static storage, never NULL). */
const char* s3r_status_string(s3r_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t s3r_version(void);

/*
 * s3r_append_kv - write new K/V rows into the paged cache (plumbing of the
 * step: draft step j writes its row at L_b + j - 1; the verify block writes its
 * gamma + 1 rows at L_b .. L_b + gamma, replacing the draft rows, since
 * verification recomputes the block's states with full attention; rebasdaily.com,
 * "真正难搬的，还是那叠完整笔记").
 *
 * k_rows, v_rows: [num_seqs][num_rows][num_kv_heads][head_dim], kv->dtype.
 * Row r of sequence b goes to position ctx_lens[b] + offset + r.
 * Precondition (device data): that position < max_pages_per_seq * 16 and the
 * page's block id is in [0, num_blocks); rows that break it are skipped.
 * Errors: INVALID_VALUE for NULL pointers, num_seqs/num_rows < 1, offset < 0,
 * inconsistent kv fields; NOT_SUPPORTED for page_size != 16 or head_dim not in
 * {64, 128}.
 */
s3r_status s3r_append_kv(const s3r_paged_kv* kv, int32_t num_seqs, int32_t offset, int32_t num_rows,
                         const void* k_rows, const void* v_rows, void* stream);

/*
 * s3r_dense_verify_attn - dense verification attention of the gamma + 1 block
 * queries over the complete paged KV history (abstract; wispaper.ai, "Dense
 * verification still pays the full KV-cache bill"), plus the attention-score
 * summary that picks the next draft's history (rit.work, "Как разреженный
 * черновик сохраняет ответы плотной модели").
 *
 * q:   [num_seqs][block_len][num_q_heads][head_dim], kv->dtype. Query i of
 *      sequence b sits at position L_b + i and attends every t <= L_b + i; its
 *      own K/V rows must already be in the cache (s3r_append_kv).
 * GQA: query head h reads kv head h / (num_q_heads / num_kv_heads).
 * softmax_scale: multiplies q.k (1/sqrt(head_dim) for standard attention).
 * out: [num_seqs][block_len][num_q_heads][head_dim], kv->dtype (bf16 rounded to
 *      nearest even).
 * page_scores (nullable): float [num_seqs][max_pages_per_seq]; entry p is the
 *      sum over the block's queries, all query heads and the tokens of page p of
 *      the softmax weights, for p < ceil((L_b + block_len) / 16), and 0 beyond.
 * Precondition (device data): L_b >= 0 and L_b + block_len <= 16 * max_pages_per_seq.
 * workspace: device memory of s3r_dense_verify_workspace_size bytes (split
 *      partials, the per-kv-head page masses, and the per-page log-sum-exps that
 *      two column tiles or long histories stage there); no initialisation needed.
 * Errors: INVALID_VALUE (NULLs, sizes < 1, num_q_heads not a multiple of
 * num_kv_heads, softmax_scale not finite and > 0); NOT_SUPPORTED (page_size != 16,
 * head_dim not in {64, 128}, block_len * group > 32); INSUFFICIENT_WORKSPACE
 * (workspace_bytes below s3r_dense_verify_workspace_size).
 */
s3r_status s3r_dense_verify_attn(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t block_len, const void* q, float softmax_scale, void* out,
                                 float* page_scores, void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_dense_verify_attn_ragged - s3r_dense_verify_attn where each sequence has
 * its own draft horizon gamma_b <= block_len - 1: sequence b's block is its first
 * gamma_b + 1 queries (positions L_b .. L_b + gamma_b). The pages observe that
 * acceptance falls at later draft positions and leave a shorter, adaptive draft
 * horizon to future work (wispaper.ai, "Acceptance falls at later draft
 * positions"); with a horizon per sequence the block is ragged.
 *
 * horizons: int32 [num_seqs], device; values are clamped to 0 .. block_len - 1.
 * q, out keep the [num_seqs][block_len][num_q_heads][head_dim] layout: rows
 * i > gamma_b are not read as queries and are written as zeros; page_scores sum
 * the softmax weights of the block's queries i <= gamma_b only.
 * Other arguments, preconditions, errors and the workspace size as
 * s3r_dense_verify_attn; INVALID_VALUE when horizons is NULL.
 */
s3r_status s3r_dense_verify_attn_ragged(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t block_len, const void* q, const int32_t* horizons,
                                        float softmax_scale, void* out, float* page_scores, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * s3r_dense_verify_attn_head_scores - s3r_dense_verify_attn with page scores
 * kept per kv head, for a page selection per kv head (context selection is left
 * as future work by the pages, wispaper.ai, "What to watch before adopting
 * S3R"): entry [b][h][p] sums the softmax weights over the block's queries, the
 * query heads of kv head h and the tokens of page p; summed over h they give
 * s3r_dense_verify_attn's page_scores. Select per kv head with
 * s3r_select_budget over num_seqs * num_kv_heads rows (ctx_lens repeated per kv
 * head) and draft with s3r_sparse_draft_attn_head_sel.
 *
 * head_page_scores: float [num_seqs][num_kv_heads][max_pages_per_seq], 0 at and
 * beyond ceil((L_b + block_len) / 16). Other arguments, preconditions, errors
 * and the workspace size as s3r_dense_verify_attn; INVALID_VALUE when
 * head_page_scores is NULL.
 */
s3r_status s3r_dense_verify_attn_head_scores(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t block_len, const void* q, float softmax_scale, void* out,
                                             float* head_page_scores, void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * s3r_dense_verify_attn_append - s3r_dense_verify_attn that first writes the
 * block's own K/V rows into the cache, as the verification pass produces them
 * when it recomputes the block's states with full attention (rebasdaily.com,
 * "真正难搬的，还是那叠完整笔记"); one launch instead of s3r_append_kv followed by
 * s3r_dense_verify_attn, with the same results. (On MI355X the two launches are
 * measured faster: the fused stores run while the kernel streams KV.)
 *
 * k_block, v_block: [num_seqs][block_len][num_kv_heads][head_dim], kv->dtype;
 * row i of sequence b goes to position L_b + i (these rows replace whatever the
 * cache held there, e.g. draft rows). Rows whose page id is out of range are
 * skipped. Other arguments, preconditions and errors as s3r_dense_verify_attn;
 * also INVALID_VALUE when k_block or v_block is NULL. The workspace size is
 * s3r_dense_verify_workspace_size's.
 */
s3r_status s3r_dense_verify_attn_append(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t block_len, const void* q, const void* k_block, const void* v_block,
                                        float softmax_scale, void* out, float* page_scores, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Workspace bytes s3r_dense_verify_attn needs for these shapes (0 on bad shapes). */
size_t s3r_dense_verify_workspace_size(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t block_len);

/*
 * s3r_select_budget - score-selected budget of history pages for the next
 * draft (rit.work, "Как разреженный черновик ..."; wispaper.ai, "Where the
 * speedup claim holds"; the budget ratio s of wispaper.ai, "Throughput gains
 * with comparable task performance").
 *
 * Candidates of sequence b are its full pages p < n_full = floor(L_b / 16) of
 * the committed length ctx_lens (host the new length after s3r_spec_accept).
 * n_sel = 0 if n_full == 0, else min(n_full, max(1, ceil(budget * n_full - 1e-9)))
 * in double precision. The n_sel pages with the largest page_scores are kept,
 * ties going to the lower page index, and written in ascending page order.
 *
 * page_scores: float [num_seqs][max_pages_per_seq] (non-negative).
 * sel_pages:   int32 [num_seqs][max_sel]; entries past n_sel are set to -1.
 * num_sel:     int32 [num_seqs].
 * max_sel must hold the largest selection any row can make: max_sel >=
 * n_sel(max_pages_per_seq) by the rule above (n_sel grows with n_full), checked
 * on the host, so every row's n_sel pages are written.
 * Errors: INVALID_VALUE (NULLs, sizes < 1, budget not in (0, 1], max_sel below
 * n_sel(max_pages_per_seq)); NOT_SUPPORTED (page_size != 16,
 * max_pages_per_seq > 32768, the candidate keys staged in LDS).
 * No workspace is needed; the arguments are kept for a stable ABI.
 */
s3r_status s3r_select_budget(const float* page_scores, const int32_t* ctx_lens, int32_t num_seqs,
                             int32_t max_pages_per_seq, int32_t page_size, double budget, int32_t* sel_pages,
                             int32_t* num_sel, int32_t max_sel, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * s3r_select_budget_rows - s3r_select_budget with a budget per row (sequence,
 * or (sequence, kv head) with page sets per kv head): row b keeps n_sel =
 * min(n_full, max(1, ceil(s_b * n_full - 1e-9))) pages (0 if n_full == 0) with
 * s_b = min(budgets[b], max_budget), by the same double-precision rule as
 * s3r_select_budget, so a budget of 0.1 keeps 100 of 1000 pages through either
 * call. The pages name adaptive sparse budgets as future work, and note that a
 * larger budget's cost eventually outweighs its acceptance gain (wispaper.ai,
 * "What to watch before adopting S3R" and "Where the speedup claim holds").
 *
 * budgets:    double [num_seqs], device. Values are not checked on the host: a
 *             NaN or non-positive budget keeps one page, a budget above
 *             max_budget is lowered to it.
 * max_budget: host double in (0, 1], the largest budget any row takes.
 * max_sel must be >= n_sel(max_pages_per_seq) at max_budget (checked on the
 * host), so every row's selection is written whole.
 * Other arguments, preconditions and errors as s3r_select_budget; also
 * INVALID_VALUE when budgets is NULL or max_budget is not in (0, 1].
 */
s3r_status s3r_select_budget_rows(const float* page_scores, const int32_t* ctx_lens, int32_t num_seqs,
                                  int32_t max_pages_per_seq, int32_t page_size, const double* budgets,
                                  double max_budget, int32_t* sel_pages, int32_t* num_sel, int32_t max_sel,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_attn - sparse self-draft attention of draft step j
 * (1-based): the same policy proposes tokens while reading only part of its KV
 * history (abstract; wispaper.ai, "S3R drafts sparsely and verifies densely";
 * rebasdaily.com, "草稿可以稀疏，交卷必须完整").
 *
 * q:   [num_seqs][num_q_heads][head_dim], kv->dtype: the query of the token at
 *      position pi = L_b + j - 1, whose K/V row is already in the cache.
 * The attended keys are the pages sel_pages[b][0 .. num_sel[b]) (full pages)
 * plus the tail 16 * floor(L_b / 16) <= t <= pi; the softmax is taken over that
 * set.
 * out: [num_seqs][num_q_heads][head_dim], kv->dtype.
 * Preconditions (device data): selected pages are distinct and < floor(L_b/16);
 * num_sel[b] <= max_sel (larger values are clamped to max_sel).
 * Errors: INVALID_VALUE (NULLs, sizes < 1, draft_step < 1, bad scale);
 * NOT_SUPPORTED (page_size != 16, head_dim not in {64, 128}, group size not in
 * {1, 2, 4, 8}).
 * No workspace is needed; the arguments are kept for a stable ABI.
 */
s3r_status s3r_sparse_draft_attn(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t draft_step, const void* q, float softmax_scale,
                                 const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_attn_head_sel - s3r_sparse_draft_attn with a page set per kv
 * head: the query heads of kv head h attend sel_pages[b][h][0 .. num_sel[b][h])
 * plus the tail.
 *
 * sel_pages: int32 [num_seqs][num_kv_heads][max_sel]; num_sel: int32
 * [num_seqs][num_kv_heads] (all kv heads of a sequence select the same number
 * when they come from one s3r_select_budget call). Other arguments,
 * preconditions and errors as s3r_sparse_draft_attn.
 */
s3r_status s3r_sparse_draft_attn_head_sel(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t draft_step, const void* q, float softmax_scale,
                                          const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_attn_append - s3r_sparse_draft_attn that first writes the
 * draft token's own K/V row (the one its forward pass produced) at position
 * pi = L_b + j - 1; one launch instead of s3r_append_kv followed by
 * s3r_sparse_draft_attn, with the same results. (On MI355X the two launches are
 * measured faster: the fused stores run while the kernel streams KV.)
 *
 * k_row, v_row: [num_seqs][num_kv_heads][head_dim], kv->dtype. A row whose page
 * id is out of range is skipped. Other arguments, preconditions and errors as
 * s3r_sparse_draft_attn; also INVALID_VALUE when k_row or v_row is NULL.
 */
s3r_status s3r_sparse_draft_attn_append(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t draft_step, const void* q, const void* k_row, const void* v_row,
                                        float softmax_scale, const int32_t* sel_pages, const int32_t* num_sel,
                                        int32_t max_sel, void* out, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * s3r_sparse_draft_attn_rows - sparse self-draft attention of draft step j that
 * takes the K/V rows of the in-flight draft tokens (positions L_b .. L_b + j - 1)
 * from the caller's draft-row buffers instead of the cache. The attended set and
 * the result are those of s3r_sparse_draft_attn after those rows were appended
 * (abstract; wispaper.ai, "S3R drafts sparsely and verifies densely"); the draft
 * steps of a block then need no append launches, and the verify block's append
 * (which writes the same positions) is the only write to the cache.
 *
 * k_rows, v_rows: kv->dtype, 16-byte aligned; row r (the K/V of the token at
 *      position L_b + r) of sequence b and kv head h is the head_dim elements
 *      starting at element r * row_stride + b * seq_stride + h * head_dim. Only
 *      rows 0 .. j-1 are read. A [rows][num_seqs][num_kv_heads][head_dim] buffer
 *      has row_stride = num_seqs * num_kv_heads * head_dim and seq_stride =
 *      num_kv_heads * head_dim; a [num_seqs][rows][num_kv_heads][head_dim] one
 *      has row_stride = num_kv_heads * head_dim and seq_stride = rows *
 *      num_kv_heads * head_dim (one sequence's rows adjacent).
 * row_stride, seq_stride: in elements, >= 0, multiples of 16 bytes.
 * The cache is read only below L_b (selected full pages, and the partial last
 * page up to L_b - 1) and is not written.
 * page_set_per_kv_head: 0 - sel_pages [num_seqs][max_sel], num_sel [num_seqs];
 *      1 - one page set per kv head as in s3r_sparse_draft_attn_head_sel.
 * Other arguments, preconditions and errors as s3r_sparse_draft_attn; also
 * INVALID_VALUE when k_rows or v_rows is NULL or misaligned, a stride is
 * negative or not a multiple of 16 bytes, or page_set_per_kv_head is not 0 or 1.
 * No workspace is needed.
 */
s3r_status s3r_sparse_draft_attn_rows(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t draft_step, const void* q, const void* k_rows, const void* v_rows,
                                      int64_t row_stride, int64_t seq_stride, float softmax_scale,
                                      const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                      int32_t page_set_per_kv_head, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_attn_ragged - s3r_sparse_draft_attn_rows where each sequence
 * has its own draft horizon gamma_b (wispaper.ai, "Acceptance falls at later
 * draft positions": a shorter horizon where late drafts are rarely kept): a
 * sequence with draft_step > horizons[b] is skipped, and its out rows are left as
 * they were.
 *
 * horizons: int32 [num_seqs], device. Other arguments, preconditions and errors
 * as s3r_sparse_draft_attn_rows; INVALID_VALUE when horizons is NULL.
 */
s3r_status s3r_sparse_draft_attn_ragged(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t draft_step, const void* q, const void* k_rows, const void* v_rows,
                                        int64_t row_stride, int64_t seq_stride, float softmax_scale,
                                        const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                        int32_t page_set_per_kv_head, const int32_t* horizons, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_spec_accept - exact speculative sampling of one drafted block per
 * sequence: draft token d_j is kept with probability min(1, p_j(d_j) / q_j(d_j));
 * at the first rejection one token is drawn from max(0, p_j - q_j) normalised
 * and the block ends (rebasdaily.com, "草稿可以稀疏，交卷必须完整"; rit.work,
 * "Как разреженный черновик ..."). If every draft is kept, one bonus token is
 * drawn from p_gamma.
 *
 * p_i = softmax(target_logits[b][i] / temperature), q_j likewise from draft_logits.
 * Logits are finite or -inf; a -inf logit (a token masked out, e.g. by top-k or
 * top-p filtering upstream) has probability 0. Every row needs at least one
 * finite logit.
 * target_logits: [num_seqs][gamma + 1][vocab], logits_dtype.
 * draft_logits:  [num_seqs][gamma][vocab], logits_dtype.
 * draft_tokens:  int32 [num_seqs][gamma], each in [0, vocab).
 * u_accept:      float [num_seqs][gamma], uniforms in [0, 1): d_j is kept iff
 *                u * q_j(d_j) < p_j(d_j) (double precision), the test
 *                u < p_j(d_j) / q_j(d_j) where q_j(d_j) > 0; a draft its own
 *                row masks (q_j(d_j) = 0) is kept iff p_j(d_j) > 0.
 * u_sample:      float [num_seqs], uniform in [0, 1) for the one final draw:
 *                the smallest x with sum_{y <= x} r_y > u * sum(r), in vocabulary
 *                order (r the residual, or p_gamma for the bonus); if rounding
 *                leaves none, the largest x with r_x > 0. A residual with zero
 *                total falls back to p_j.
 * Outputs: num_accepted int32 [num_seqs]; out_tokens int32 [num_seqs][gamma + 1]
 *          (the kept drafts, then the corrected or bonus token, then -1);
 *          ctx_lens_inout (nullable) int32 [num_seqs] += num_accepted + 1.
 * Sums over the vocabulary and the final ratio test are in double precision.
 * Errors: INVALID_VALUE (NULLs, num_seqs/gamma/vocab < 1, temperature not
 * finite and > 0, bad dtype); INSUFFICIENT_WORKSPACE.
 */
s3r_status s3r_spec_accept(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                           const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                           const float* u_accept, const float* u_sample, float temperature,
                           int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens_inout, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * s3r_spec_accept_no_alloc - s3r_spec_accept for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It takes no workspace: the library keeps one static
 * device workspace of 4 MiB per GPU (a file-scope device array, held until the
 * process ends), found on the first call on each device. It allocates nothing and
 * calls no allocating routine.
 *
 * The workspace is shared by every call on a GPU: calls that overlap on one GPU
 * (on different streams, or from several host threads) race and give undefined
 * results; order them on one stream. Nothing in it needs clearing between calls.
 * The stream must belong to the current device.
 * Arguments, outputs and results are those of s3r_spec_accept.
 * Errors: those of s3r_spec_accept; INSUFFICIENT_WORKSPACE when the shapes need
 * more than 4 MiB (s3r_spec_accept_workspace_size bytes > 4194304; about 820 B per
 * sequence at gamma 4 and a 151,936-token vocabulary); HIP when the workspace's
 * address cannot be found on the current device.
 */
s3r_status s3r_spec_accept_no_alloc(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                                    const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                                    float temperature, int32_t* num_accepted, int32_t* out_tokens,
                                    int32_t* ctx_lens_inout, void* stream);

/*
 * s3r_spec_accept_ragged - s3r_spec_accept where each sequence has its own draft
 * horizon gamma_b (wispaper.ai, "Acceptance falls at later draft positions"):
 * sequence b tests only its drafts 0 .. gamma_b - 1, and when all of them are
 * kept the bonus token is drawn from p_{gamma_b}; gamma_b = 0 is one plain draw
 * from p_0. The block of every sequence is then exact speculative sampling with
 * gamma_b drafts.
 *
 * horizons: int32 [num_seqs], device; values are clamped to 0 .. gamma. Logit
 * rows, draft tokens and uniforms past a sequence's horizon are not read (target
 * rows i > gamma_b, draft rows j >= gamma_b). The layouts stay those of gamma.
 * out_tokens: the kept drafts, the corrected or bonus token, then -1 up to gamma + 1.
 * Other arguments, errors and the workspace size as s3r_spec_accept;
 * INVALID_VALUE when horizons is NULL.
 */
s3r_status s3r_spec_accept_ragged(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                                  const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                                  const float* u_accept, const float* u_sample, const int32_t* horizons,
                                  float temperature, int32_t* num_accepted, int32_t* out_tokens,
                                  int32_t* ctx_lens_inout, void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_check_step_inputs - checks the device-resident inputs of a decode step
 * that the other calls cannot check without a host sync, for debug runs: the
 * attention kernels clamp out-of-range values so that no access leaves the
 * buffers, but their results are then unspecified. This call reports them.
 * (Not a step of the method; it validates the preconditions stated above.)
 *
 * One pass per sequence b writes errors[b] (int32 [num_seqs], device, written
 * for every sequence, 0 when all is well) as an OR of:
 *   S3R_CHECK_LEN        ctx_lens[b] < 0 or ctx_lens[b] + block_len > 16 * max_pages_per_seq
 *   S3R_CHECK_PAGE       a page-table entry the step uses (logical pages below
 *                        ceil((L_b + block_len) / 16)) is outside [0, num_blocks)
 *   S3R_CHECK_NUM_SEL    a num_sel value outside [0, max_sel]
 *   S3R_CHECK_SEL_RANGE  a selected page outside [0, floor(L_b / 16))
 *   S3R_CHECK_SEL_DUP    a page selected twice in one selection row
 *   S3R_CHECK_TOKEN      a draft token outside [0, vocab)
 *   S3R_CHECK_SLOT       an infinity or NaN in K or V at a position >= L_b of the
 *                        pages holding L_b .. L_b + block_len - 1: slots the step
 *                        reads with zero weight, which must hold finite values
 *                        (the layout note above)
 * block_len: the step's block, gamma + 1 (the positions L_b .. L_b + gamma it
 * writes and reads). sel_pages / num_sel (both or neither): the selection the
 * drafts will read, one row per sequence, or one per (sequence, kv head) with
 * page_set_per_kv_head = 1. draft_tokens (nullable): int32 [num_seqs][gamma]
 * with vocab the vocabulary size. Selection and token checks are skipped when
 * their arrays are NULL. Every read stays inside the buffers described; the
 * values are compared, never used as addresses.
 * Errors: INVALID_VALUE (NULL errors, sizes < 1, sel_pages without num_sel or
 * the reverse, a flag other than 0/1, block_len beyond the page table);
 * NOT_SUPPORTED (max_pages_per_seq above 524288).
 */
#define S3R_CHECK_LEN 1
#define S3R_CHECK_PAGE 2
#define S3R_CHECK_NUM_SEL 4
#define S3R_CHECK_SEL_RANGE 8
#define S3R_CHECK_SEL_DUP 16
#define S3R_CHECK_TOKEN 32
#define S3R_CHECK_SLOT 64
s3r_status s3r_check_step_inputs(const s3r_paged_kv* kv, int32_t num_seqs, int32_t block_len,
                                 const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                 int32_t page_set_per_kv_head, const int32_t* draft_tokens, int32_t gamma,
                                 int32_t vocab, int32_t* errors, void* stream);

/*
 * s3r_pack_pages / s3r_unpack_pages - whole-page moves between the paged cache
 * and a contiguous staging buffer, the data movement of offloading a paused
 * request's history to host memory and restoring it. Dense verification needs
 * the complete history, so a request paused under memory pressure keeps its
 * pages (moved out and back) rather than recomputing them (rebasdaily.com,
 * "真正难搬的，还是那叠完整笔记"; wispaper.ai, "Dense verification still pays the
 * full KV-cache bill" and its scheduler, which limits these moves).
 *
 * blocks: int32 [num_pages], device: physical block ids. Page i of the staging
 * buffer is the K tiles of block blocks[i] (all kv heads, [num_kv_heads][16]
 * [head_dim] as stored) followed by its V tiles ([num_kv_heads][head_dim][16]),
 * s3r_page_bytes(kv) bytes per page. pack copies blocks -> staging, unpack
 * copies staging -> blocks (the page table is the caller's). Both are exact byte
 * copies. staging: device memory, 16-byte aligned, num_pages * s3r_page_bytes(kv)
 * bytes. Block ids outside [0, num_blocks) are skipped: that page's staging slot
 * (pack) or block (unpack) is left as it was.
 * Errors: INVALID_VALUE (NULLs, num_pages < 1, misaligned staging, a bad kv).
 */
size_t s3r_page_bytes(const s3r_paged_kv* kv);
s3r_status s3r_pack_pages(const s3r_paged_kv* kv, const int32_t* blocks, int32_t num_pages, void* staging,
                          void* stream);
s3r_status s3r_unpack_pages(const s3r_paged_kv* kv, const int32_t* blocks, int32_t num_pages, const void* staging,
                            void* stream);

/* Workspace bytes of the selection and the sparse draft calls: 0 for every
 * shape (they need none; their workspace arguments may be NULL with 0 bytes).
 * Given so that every op has a *_workspace_size call. */
size_t s3r_select_budget_workspace_size(int32_t num_seqs, int32_t max_pages_per_seq);
size_t s3r_sparse_draft_workspace_size(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads);

/* Workspace bytes s3r_spec_accept needs for these shapes (0 on bad shapes). */
size_t s3r_spec_accept_workspace_size(int32_t num_seqs, int32_t gamma, int32_t vocab);

#ifdef __cplusplus
}
#endif

#endif /* S3R_H_ */
