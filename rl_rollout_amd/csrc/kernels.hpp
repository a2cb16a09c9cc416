// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s3r {

constexpr int kPageSize = 16;  // tokens per KV page

struct KvView {
  void* k;
  void* v;
  const int32_t* table;
  const int32_t* lens;
  int num_blocks, hkv, head_dim, maxp;
  int bf16;  // 1: bf16 storage, 0: fp32
};

// ---- dense verify --------------------------------------------------------
struct VerifyPlan {
  int num_seqs, hq, G1, g, M;   // M = G1 * g query rows per kv head
  int pps;                      // pages per split (<= 256)
  int depth;                    // pages in flight per wave
  int max_splits;               // ceil(maxp / pps)
  bool unit;                    // whole-unit mode: one workgroup per (sequence, kv head)
  bool gstage;                  // whole-unit mode with the per-page staging in the workspace
  int lse_stride;               // whole-unit mode: LDS stride of the per-page staging
  int gchunks;                  // global staging: chunks of 512 pages per unit
  bool lpt;                     // whole-unit mode: longest sequences first
  size_t off_part_o, off_part_ml, off_lse, off_gstage, bytes;
};
size_t verify_combine_lds_bytes(int hkv, int M, int max_splits);
VerifyPlan plan_verify(const KvView& kv, int num_seqs, int hq, int G1);
// k_new / v_new (nullable): the block's rows [B][G1][hkv][D], written into the
// cache at L_b .. L_b + G1 - 1 by the kernel itself before it attends.
// head_scores (nullable): per-kv-head page scores [B][hkv][maxp] instead of the
// shared `scores` (give one or the other).
// horizons (nullable): [B] draft horizon gamma_b of each sequence; block query i of
// sequence b exists for i <= gamma_b, later ones see no key (zero output, no page mass).
hipError_t launch_verify(const KvView& kv, const VerifyPlan& plan, const void* q, float scale, void* out,
                         float* scores, void* workspace, hipStream_t stream, const void* k_new = nullptr,
                         const void* v_new = nullptr, float* head_scores = nullptr,
                         const int32_t* horizons = nullptr);

// ---- sparse draft ----------------------------------------------------------
// k_new / v_new (nullable): this draft token's row [B][hkv][D], written at
// L_b + step - 1 by the kernel itself before it attends.
// sel_per_head: sel is [B][hkv][max_sel] and nsel [B][hkv] (a page set per kv head).
// k_rows / v_rows (nullable, not with k_new): the rows of draft steps 1 .. step
// (positions L_b .. L_b + step - 1), row r of sequence b and kv head h at element
// r * row_stride + b * seq_stride + h * head_dim, read instead of the cache at those
// positions; the cache is read only below L_b and is not written.
hipError_t launch_draft(const KvView& kv, int num_seqs, int hq, int step, const void* q, float scale,
                        const int32_t* sel, const int32_t* nsel, int max_sel, void* out, hipStream_t stream,
                        const void* k_new = nullptr, const void* v_new = nullptr, bool sel_per_head = false,
                        const void* k_rows = nullptr, const void* v_rows = nullptr, long long row_stride = 0,
                        long long seq_stride = 0, const int32_t* horizons = nullptr);

// ---- budget selection --------------------------------------------------
// budgets (nullable): double [num_seqs] budget per row (capped at `budget`), used instead of it.
hipError_t launch_select(const float* scores, const int32_t* lens, int num_seqs, int maxp, double budget,
                         int32_t* sel, int32_t* nsel, int max_sel, hipStream_t stream,
                         const double* budgets = nullptr);

// ---- KV append -------------------------------------------------------------
hipError_t launch_append(const KvView& kv, int num_seqs, int offset, int rows, const void* k_rows,
                         const void* v_rows, hipStream_t stream);

// ---- speculative accept ----------------------------------------------------
struct AcceptPlan {
  int num_seqs, gamma, vocab, rows;   // rows = 2 * gamma + 1 logit rows per sequence
  int nch, clen;                      // row-statistics chunks
  int unroll;                         // row-statistics loads in flight per thread (4, 8 or 16)
  int nch2, clen2;                    // residual chunks
  int cpw;                            // residual chunks per workgroup
  size_t off_st_m, off_st_s, off_dstat, off_dec, off_rsum, off_rlast, bytes;
};
AcceptPlan plan_accept(int num_seqs, int gamma, int vocab);
// The allocation-free accept's workspace: a file-scope device array of this size,
// one per GPU; static_accept_scratch gives its address on the current device.
constexpr size_t kStaticAcceptScratchBytes = size_t(4) << 20;
hipError_t static_accept_scratch(void** ptr);
// horizons (nullable): [B] draft horizon gamma_b (clamped to 0 .. gamma); sequence b
// tests its first gamma_b drafts and takes the bonus from target row gamma_b.
hipError_t launch_accept(const AcceptPlan& plan, int bf16, const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                         float temperature, int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens,
                         void* workspace, hipStream_t stream, const int32_t* horizons = nullptr);

// ---- device-input checks ----------------------------------------------------
// Bits of the per-sequence error word (the same values as S3R_CHECK_* in s3r.h).
constexpr int kCheckLen = 1, kCheckPage = 2, kCheckNumSel = 4, kCheckSelRange = 8, kCheckSelDup = 16,
              kCheckToken = 32, kCheckSlot = 64;
// One workgroup per sequence: errors[b] = the bits of sequence b's problems.
// span: positions the step reaches past L_b (block length); sel / nsel
// (nullable): sel_rows selection rows per sequence; tokens (nullable): [B][gamma].
size_t check_lds_bytes(int maxp);
hipError_t launch_check(const KvView& kv, int num_seqs, int span, const int32_t* sel, const int32_t* nsel,
                        int max_sel, int sel_rows, const int32_t* tokens, int gamma, int vocab, int32_t* errors,
                        hipStream_t stream);

// ---- whole-page moves (offload / restore) ----------------------------------
// Bytes of one page's K run (and of its V run): hkv * 16 * head_dim elements.
size_t page_run_bytes(const KvView& kv);
// pack: staging[i] = (K run, V run) of block blocks[i]; unpack: the reverse.
hipError_t launch_page_copy(const KvView& kv, const int32_t* blocks, int n, void* staging, bool pack,
                            hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace s3r
