// C ABI of libs3r.so (declared in include/s3r.h): host-side validation, workspace
// planning and dispatch to the HIP kernels. Nothing here allocates device memory.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/s3r.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxVerifyRows = 32;     // block_len * group: two 16-column MFMA tiles
constexpr int kMaxSelectPages = 32768; // candidate keys staged in LDS (4 bytes each, 128 KB of gfx950's 160 KB)
constexpr size_t kMaxLds = 65536;

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

// Pages a budget keeps out of n_full full pages: 0 without a full page, else
// ceil(budget * n_full - 1e-9) in double, clamped to [1, n_full]. The select
// kernel takes the same rule per row; this host copy sizes max_sel.
int64_t pages_kept(double budget, int64_t n_full) {
  if (n_full <= 0) return 0;
  const double x = ceil(budget * static_cast<double>(n_full) - 1e-9);
  return static_cast<int64_t>(fmin(fmax(x, 1.0), static_cast<double>(n_full)));
}

// Kernels read caches, queries and logits with 16-byte vector loads.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

s3r_status check_kv(const s3r_paged_kv* kv) {
  if (kv == nullptr || kv->k_cache == nullptr || kv->v_cache == nullptr || kv->page_table == nullptr ||
      kv->ctx_lens == nullptr)
    return S3R_ERROR_INVALID_VALUE;
  if (kv->num_blocks < 1 || kv->num_kv_heads < 1 || kv->page_size < 1 || kv->head_dim < 1 ||
      kv->max_pages_per_seq < 1)
    return S3R_ERROR_INVALID_VALUE;
  if (kv->dtype != S3R_F32 && kv->dtype != S3R_BF16) return S3R_ERROR_INVALID_VALUE;
  if (!aligned16(kv->k_cache) || !aligned16(kv->v_cache)) return S3R_ERROR_INVALID_VALUE;
  if (kv->page_size != s3r::kPageSize) return S3R_ERROR_NOT_SUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return S3R_ERROR_NOT_SUPPORTED;
  return S3R_SUCCESS;
}

s3r::KvView view_of(const s3r_paged_kv* kv) {
  s3r::KvView v{};
  v.k = kv->k_cache;
  v.v = kv->v_cache;
  v.table = kv->page_table;
  v.lens = kv->ctx_lens;
  v.num_blocks = kv->num_blocks;
  v.hkv = kv->num_kv_heads;
  v.head_dim = kv->head_dim;
  v.maxp = kv->max_pages_per_seq;
  v.bf16 = kv->dtype == S3R_BF16 ? 1 : 0;
  return v;
}

s3r_status from_hip(hipError_t e) { return e == hipSuccess ? S3R_SUCCESS : S3R_ERROR_HIP; }

s3r_status check_verify_shapes(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads, int32_t block_len) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (num_seqs < 1 || num_q_heads < 1 || block_len < 1) return S3R_ERROR_INVALID_VALUE;
  if (num_q_heads % kv->num_kv_heads != 0) return S3R_ERROR_INVALID_VALUE;
  if (static_cast<int64_t>(block_len) > static_cast<int64_t>(kv->max_pages_per_seq) * kv->page_size)
    return S3R_ERROR_INVALID_VALUE;
  if (static_cast<int64_t>(block_len) * (num_q_heads / kv->num_kv_heads) > kMaxVerifyRows)
    return S3R_ERROR_NOT_SUPPORTED;
  return S3R_SUCCESS;
}

}  // namespace

extern "C" {

const char* s3r_status_string(s3r_status status) {
  switch (status) {
    case S3R_SUCCESS: return "success";
    case S3R_ERROR_INVALID_VALUE: return "invalid value";
    case S3R_ERROR_NOT_SUPPORTED: return "not supported";
    case S3R_ERROR_INSUFFICIENT_WORKSPACE: return "insufficient workspace";
    case S3R_ERROR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t s3r_version(void) { return 300; }  // 0.3.0: double per-row budgets under a host maximum, max_sel checked

s3r_status s3r_append_kv(const s3r_paged_kv* kv, int32_t num_seqs, int32_t offset, int32_t num_rows,
                         const void* k_rows, const void* v_rows, void* stream) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (num_seqs < 1 || num_rows < 1 || offset < 0 || k_rows == nullptr || v_rows == nullptr)
    return S3R_ERROR_INVALID_VALUE;
  // the grid pads the sequences to a multiple of the 8 XCDs
  if ((static_cast<int64_t>(num_seqs) + 7) / 8 * 8 * num_rows > INT32_MAX) return S3R_ERROR_NOT_SUPPORTED;
  return from_hip(s3r::launch_append(view_of(kv), num_seqs, offset, num_rows, k_rows, v_rows,
                                     static_cast<hipStream_t>(stream)));
}

size_t s3r_dense_verify_workspace_size(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t block_len) {
  if (check_verify_shapes(kv, num_seqs, num_q_heads, block_len) != S3R_SUCCESS) return 0;
  return s3r::plan_verify(view_of(kv), num_seqs, num_q_heads, block_len).bytes;
}

}  // extern "C"

namespace {

s3r_status verify_impl(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads, int32_t block_len,
                       const void* q, const void* k_block, const void* v_block, float softmax_scale, void* out,
                       float* page_scores, void* workspace, size_t workspace_bytes, void* stream,
                       float* head_page_scores = nullptr, const int32_t* horizons = nullptr) {
  s3r_status st = check_verify_shapes(kv, num_seqs, num_q_heads, block_len);
  if (st != S3R_SUCCESS) return st;
  if (q == nullptr || out == nullptr || !finite_pos(softmax_scale) || !aligned16(q)) return S3R_ERROR_INVALID_VALUE;
  const s3r::KvView v = view_of(kv);
  const s3r::VerifyPlan plan = s3r::plan_verify(v, num_seqs, num_q_heads, block_len);
  if (workspace_bytes < plan.bytes || (plan.bytes > 0 && workspace == nullptr))
    return S3R_ERROR_INSUFFICIENT_WORKSPACE;
  if (s3r::verify_combine_lds_bytes(kv->num_kv_heads, plan.M, plan.max_splits) > kMaxLds)
    return S3R_ERROR_NOT_SUPPORTED;
  if (static_cast<int64_t>(num_seqs) * kv->num_kv_heads * plan.max_splits > INT32_MAX)
    return S3R_ERROR_NOT_SUPPORTED;
  return from_hip(s3r::launch_verify(v, plan, q, softmax_scale, out, page_scores, workspace,
                                     static_cast<hipStream_t>(stream), k_block, v_block, head_page_scores,
                                     horizons));
}

s3r_status draft_impl(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads, int32_t draft_step,
                      const void* q, const void* k_row, const void* v_row, float softmax_scale,
                      const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel, void* out, void* stream,
                      bool sel_per_head = false, const void* k_rows = nullptr, const void* v_rows = nullptr,
                      int64_t row_stride = 0, int64_t seq_stride = 0, const int32_t* horizons = nullptr) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (num_seqs < 1 || num_q_heads < 1 || draft_step < 1 || max_sel < 1) return S3R_ERROR_INVALID_VALUE;
  if (num_q_heads % kv->num_kv_heads != 0) return S3R_ERROR_INVALID_VALUE;
  if (static_cast<int64_t>(draft_step) > static_cast<int64_t>(kv->max_pages_per_seq) * kv->page_size)
    return S3R_ERROR_INVALID_VALUE;
  if (q == nullptr || out == nullptr || sel_pages == nullptr || num_sel == nullptr || !finite_pos(softmax_scale) ||
      !aligned16(q))
    return S3R_ERROR_INVALID_VALUE;
  const int g = num_q_heads / kv->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return S3R_ERROR_NOT_SUPPORTED;
  if (static_cast<int64_t>(num_seqs) * kv->num_kv_heads > INT32_MAX) return S3R_ERROR_NOT_SUPPORTED;
  if ((k_rows != nullptr) != (v_rows != nullptr)) return S3R_ERROR_INVALID_VALUE;
  if (k_rows != nullptr) {
    if (k_row != nullptr || !aligned16(k_rows) || !aligned16(v_rows)) return S3R_ERROR_INVALID_VALUE;
    // strides in elements: every row start must stay 16-byte aligned
    const int64_t elem = kv->dtype == S3R_BF16 ? 2 : 4;
    if (row_stride < 0 || seq_stride < 0 || (row_stride * elem) % 16 != 0 || (seq_stride * elem) % 16 != 0)
      return S3R_ERROR_INVALID_VALUE;
  }
  return from_hip(s3r::launch_draft(view_of(kv), num_seqs, num_q_heads, draft_step, q, softmax_scale, sel_pages,
                                    num_sel, max_sel, out, static_cast<hipStream_t>(stream), k_row, v_row,
                                    sel_per_head, k_rows, v_rows, row_stride, seq_stride, horizons));
}

s3r_status check_accept_args(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                             const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                             const float* u_accept, const float* u_sample, float temperature,
                             const int32_t* num_accepted, const int32_t* out_tokens) {
  if (num_seqs < 1 || gamma < 1 || vocab < 1) return S3R_ERROR_INVALID_VALUE;
  if (logits_dtype != S3R_F32 && logits_dtype != S3R_BF16) return S3R_ERROR_INVALID_VALUE;
  if (target_logits == nullptr || draft_logits == nullptr || draft_tokens == nullptr || u_accept == nullptr ||
      u_sample == nullptr || num_accepted == nullptr || out_tokens == nullptr)
    return S3R_ERROR_INVALID_VALUE;
  if (!finite_pos(temperature)) return S3R_ERROR_INVALID_VALUE;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return S3R_ERROR_INVALID_VALUE;
  if (static_cast<int64_t>(num_seqs) * s3r::plan_accept(num_seqs, gamma, vocab).rows > INT32_MAX)
    return S3R_ERROR_NOT_SUPPORTED;
  return S3R_SUCCESS;
}

s3r_status accept_impl(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                       const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const float* u_accept, const float* u_sample, const int32_t* horizons, float temperature,
                       int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens_inout, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const s3r_status st = check_accept_args(num_seqs, gamma, vocab, logits_dtype, target_logits, draft_logits,
                                          draft_tokens, u_accept, u_sample, temperature, num_accepted, out_tokens);
  if (st != S3R_SUCCESS) return st;
  const s3r::AcceptPlan plan = s3r::plan_accept(num_seqs, gamma, vocab);
  if (workspace_bytes < plan.bytes || workspace == nullptr) return S3R_ERROR_INSUFFICIENT_WORKSPACE;
  return from_hip(s3r::launch_accept(plan, logits_dtype == S3R_BF16 ? 1 : 0, target_logits, draft_logits,
                                     draft_tokens, u_accept, u_sample, temperature, num_accepted, out_tokens,
                                     ctx_lens_inout, workspace, static_cast<hipStream_t>(stream), horizons));
}


}  // namespace

extern "C" {

s3r_status s3r_dense_verify_attn(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t block_len, const void* q, float softmax_scale, void* out,
                                 float* page_scores, void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(kv, num_seqs, num_q_heads, block_len, q, nullptr, nullptr, softmax_scale, out, page_scores,
                     workspace, workspace_bytes, stream);
}

s3r_status s3r_dense_verify_attn_ragged(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t block_len, const void* q, const int32_t* horizons,
                                        float softmax_scale, void* out, float* page_scores, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (horizons == nullptr) return S3R_ERROR_INVALID_VALUE;
  return verify_impl(kv, num_seqs, num_q_heads, block_len, q, nullptr, nullptr, softmax_scale, out, page_scores,
                     workspace, workspace_bytes, stream, nullptr, horizons);
}

s3r_status s3r_dense_verify_attn_head_scores(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t block_len, const void* q, float softmax_scale, void* out,
                                             float* head_page_scores, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (head_page_scores == nullptr) return S3R_ERROR_INVALID_VALUE;
  return verify_impl(kv, num_seqs, num_q_heads, block_len, q, nullptr, nullptr, softmax_scale, out, nullptr,
                     workspace, workspace_bytes, stream, head_page_scores);
}

s3r_status s3r_dense_verify_attn_append(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t block_len, const void* q, const void* k_block, const void* v_block,
                                        float softmax_scale, void* out, float* page_scores, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (k_block == nullptr || v_block == nullptr) return S3R_ERROR_INVALID_VALUE;
  return verify_impl(kv, num_seqs, num_q_heads, block_len, q, k_block, v_block, softmax_scale, out, page_scores,
                     workspace, workspace_bytes, stream);
}

s3r_status s3r_select_budget(const float* page_scores, const int32_t* ctx_lens, int32_t num_seqs,
                             int32_t max_pages_per_seq, int32_t page_size, double budget, int32_t* sel_pages,
                             int32_t* num_sel, int32_t max_sel, void* workspace, size_t workspace_bytes,
                             void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (page_scores == nullptr || ctx_lens == nullptr || sel_pages == nullptr || num_sel == nullptr)
    return S3R_ERROR_INVALID_VALUE;
  if (num_seqs < 1 || max_pages_per_seq < 1 || page_size < 1 || max_sel < 1) return S3R_ERROR_INVALID_VALUE;
  if (!(isfinite(budget) && budget > 0.0 && budget <= 1.0)) return S3R_ERROR_INVALID_VALUE;
  if (page_size != s3r::kPageSize) return S3R_ERROR_NOT_SUPPORTED;
  if (max_pages_per_seq > kMaxSelectPages) return S3R_ERROR_NOT_SUPPORTED;
  // every row's selection must fit: n_sel grows with n_full <= max_pages_per_seq
  if (max_sel < pages_kept(budget, max_pages_per_seq)) return S3R_ERROR_INVALID_VALUE;
  return from_hip(s3r::launch_select(page_scores, ctx_lens, num_seqs, max_pages_per_seq, budget, sel_pages,
                                     num_sel, max_sel, static_cast<hipStream_t>(stream)));
}

s3r_status s3r_select_budget_rows(const float* page_scores, const int32_t* ctx_lens, int32_t num_seqs,
                                  int32_t max_pages_per_seq, int32_t page_size, const double* budgets,
                                  double max_budget, int32_t* sel_pages, int32_t* num_sel, int32_t max_sel,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (page_scores == nullptr || ctx_lens == nullptr || budgets == nullptr || sel_pages == nullptr ||
      num_sel == nullptr)
    return S3R_ERROR_INVALID_VALUE;
  if (num_seqs < 1 || max_pages_per_seq < 1 || page_size < 1 || max_sel < 1) return S3R_ERROR_INVALID_VALUE;
  if (!(isfinite(max_budget) && max_budget > 0.0 && max_budget <= 1.0)) return S3R_ERROR_INVALID_VALUE;
  if (page_size != s3r::kPageSize) return S3R_ERROR_NOT_SUPPORTED;
  if (max_pages_per_seq > kMaxSelectPages) return S3R_ERROR_NOT_SUPPORTED;
  if (max_sel < pages_kept(max_budget, max_pages_per_seq)) return S3R_ERROR_INVALID_VALUE;
  return from_hip(s3r::launch_select(page_scores, ctx_lens, num_seqs, max_pages_per_seq, max_budget, sel_pages,
                                     num_sel, max_sel, static_cast<hipStream_t>(stream), budgets));
}

s3r_status s3r_sparse_draft_attn(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t draft_step, const void* q, float softmax_scale,
                                 const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return draft_impl(kv, num_seqs, num_q_heads, draft_step, q, nullptr, nullptr, softmax_scale, sel_pages, num_sel,
                    max_sel, out, stream);
}

s3r_status s3r_sparse_draft_attn_head_sel(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t draft_step, const void* q, float softmax_scale,
                                          const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return draft_impl(kv, num_seqs, num_q_heads, draft_step, q, nullptr, nullptr, softmax_scale, sel_pages, num_sel,
                    max_sel, out, stream, true);
}

s3r_status s3r_sparse_draft_attn_append(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t draft_step, const void* q, const void* k_row, const void* v_row,
                                        float softmax_scale, const int32_t* sel_pages, const int32_t* num_sel,
                                        int32_t max_sel, void* out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k_row == nullptr || v_row == nullptr) return S3R_ERROR_INVALID_VALUE;
  return draft_impl(kv, num_seqs, num_q_heads, draft_step, q, k_row, v_row, softmax_scale, sel_pages, num_sel,
                    max_sel, out, stream);
}

s3r_status s3r_sparse_draft_attn_rows(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t draft_step, const void* q, const void* k_rows, const void* v_rows,
                                      int64_t row_stride, int64_t seq_stride, float softmax_scale,
                                      const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                      int32_t page_set_per_kv_head, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k_rows == nullptr || v_rows == nullptr) return S3R_ERROR_INVALID_VALUE;
  if (page_set_per_kv_head != 0 && page_set_per_kv_head != 1) return S3R_ERROR_INVALID_VALUE;
  return draft_impl(kv, num_seqs, num_q_heads, draft_step, q, nullptr, nullptr, softmax_scale, sel_pages, num_sel,
                    max_sel, out, stream, page_set_per_kv_head == 1, k_rows, v_rows, row_stride, seq_stride);
}

s3r_status s3r_sparse_draft_attn_ragged(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t draft_step, const void* q, const void* k_rows, const void* v_rows,
                                        int64_t row_stride, int64_t seq_stride, float softmax_scale,
                                        const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                        int32_t page_set_per_kv_head, const int32_t* horizons, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k_rows == nullptr || v_rows == nullptr || horizons == nullptr) return S3R_ERROR_INVALID_VALUE;
  if (page_set_per_kv_head != 0 && page_set_per_kv_head != 1) return S3R_ERROR_INVALID_VALUE;
  return draft_impl(kv, num_seqs, num_q_heads, draft_step, q, nullptr, nullptr, softmax_scale, sel_pages, num_sel,
                    max_sel, out, stream, page_set_per_kv_head == 1, k_rows, v_rows, row_stride, seq_stride,
                    horizons);
}

s3r_status s3r_check_step_inputs(const s3r_paged_kv* kv, int32_t num_seqs, int32_t block_len,
                                 const int32_t* sel_pages, const int32_t* num_sel, int32_t max_sel,
                                 int32_t page_set_per_kv_head, const int32_t* draft_tokens, int32_t gamma,
                                 int32_t vocab, int32_t* errors, void* stream) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (num_seqs < 1 || block_len < 1 || errors == nullptr) return S3R_ERROR_INVALID_VALUE;
  if (static_cast<int64_t>(block_len) > static_cast<int64_t>(kv->max_pages_per_seq) * kv->page_size)
    return S3R_ERROR_INVALID_VALUE;
  if ((sel_pages == nullptr) != (num_sel == nullptr)) return S3R_ERROR_INVALID_VALUE;
  if (sel_pages != nullptr && (max_sel < 1 || (page_set_per_kv_head != 0 && page_set_per_kv_head != 1)))
    return S3R_ERROR_INVALID_VALUE;
  if (draft_tokens != nullptr && (gamma < 1 || vocab < 1)) return S3R_ERROR_INVALID_VALUE;
  if (s3r::check_lds_bytes(kv->max_pages_per_seq) > kMaxLds) return S3R_ERROR_NOT_SUPPORTED;
  const int sel_rows = page_set_per_kv_head == 1 ? kv->num_kv_heads : 1;
  return from_hip(s3r::launch_check(view_of(kv), num_seqs, block_len, sel_pages, num_sel, max_sel, sel_rows,
                                    draft_tokens, gamma, vocab, errors, static_cast<hipStream_t>(stream)));
}

size_t s3r_page_bytes(const s3r_paged_kv* kv) {
  if (check_kv(kv) != S3R_SUCCESS) return 0;
  return 2 * s3r::page_run_bytes(view_of(kv));
}

s3r_status s3r_pack_pages(const s3r_paged_kv* kv, const int32_t* blocks, int32_t num_pages, void* staging,
                          void* stream) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (blocks == nullptr || staging == nullptr || num_pages < 1 || !aligned16(staging)) return S3R_ERROR_INVALID_VALUE;
  if (num_pages > (INT32_MAX >> 1)) return S3R_ERROR_NOT_SUPPORTED;
  return from_hip(s3r::launch_page_copy(view_of(kv), blocks, num_pages, staging, true,
                                        static_cast<hipStream_t>(stream)));
}

s3r_status s3r_unpack_pages(const s3r_paged_kv* kv, const int32_t* blocks, int32_t num_pages, const void* staging,
                            void* stream) {
  s3r_status st = check_kv(kv);
  if (st != S3R_SUCCESS) return st;
  if (blocks == nullptr || staging == nullptr || num_pages < 1 || !aligned16(staging)) return S3R_ERROR_INVALID_VALUE;
  if (num_pages > (INT32_MAX >> 1)) return S3R_ERROR_NOT_SUPPORTED;
  return from_hip(s3r::launch_page_copy(view_of(kv), blocks, num_pages, const_cast<void*>(staging), false,
                                        static_cast<hipStream_t>(stream)));
}

size_t s3r_select_budget_workspace_size(int32_t num_seqs, int32_t max_pages_per_seq) {
  (void)num_seqs;
  (void)max_pages_per_seq;
  return 0;
}

size_t s3r_sparse_draft_workspace_size(const s3r_paged_kv* kv, int32_t num_seqs, int32_t num_q_heads) {
  (void)kv;
  (void)num_seqs;
  (void)num_q_heads;
  return 0;
}

size_t s3r_spec_accept_workspace_size(int32_t num_seqs, int32_t gamma, int32_t vocab) {
  if (num_seqs < 1 || gamma < 1 || vocab < 1) return 0;
  return s3r::plan_accept(num_seqs, gamma, vocab).bytes;
}

s3r_status s3r_spec_accept(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                           const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                           const float* u_accept, const float* u_sample, float temperature,
                           int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens_inout, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return accept_impl(num_seqs, gamma, vocab, logits_dtype, target_logits, draft_logits, draft_tokens, u_accept,
                     u_sample, nullptr, temperature, num_accepted, out_tokens, ctx_lens_inout, workspace,
                     workspace_bytes, stream);
}

s3r_status s3r_spec_accept_no_alloc(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                                    const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                                    float temperature, int32_t* num_accepted, int32_t* out_tokens,
                                    int32_t* ctx_lens_inout, void* stream) {
  const s3r_status st = check_accept_args(num_seqs, gamma, vocab, logits_dtype, target_logits, draft_logits,
                                          draft_tokens, u_accept, u_sample, temperature, num_accepted, out_tokens);
  if (st != S3R_SUCCESS) return st;
  if (s3r::plan_accept(num_seqs, gamma, vocab).bytes > s3r::kStaticAcceptScratchBytes)
    return S3R_ERROR_INSUFFICIENT_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = s3r::static_accept_scratch(&ws);
  if (e != hipSuccess) return S3R_ERROR_HIP;
  return accept_impl(num_seqs, gamma, vocab, logits_dtype, target_logits, draft_logits, draft_tokens, u_accept,
                     u_sample, nullptr, temperature, num_accepted, out_tokens, ctx_lens_inout, ws,
                     s3r::kStaticAcceptScratchBytes, stream);
}

s3r_status s3r_spec_accept_ragged(int32_t num_seqs, int32_t gamma, int32_t vocab, int32_t logits_dtype,
                                  const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                                  const float* u_accept, const float* u_sample, const int32_t* horizons,
                                  float temperature, int32_t* num_accepted, int32_t* out_tokens,
                                  int32_t* ctx_lens_inout, void* workspace, size_t workspace_bytes, void* stream) {
  if (horizons == nullptr) return S3R_ERROR_INVALID_VALUE;
  return accept_impl(num_seqs, gamma, vocab, logits_dtype, target_logits, draft_logits, draft_tokens, u_accept,
                     u_sample, horizons, temperature, num_accepted, out_tokens, ctx_lens_inout, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"
