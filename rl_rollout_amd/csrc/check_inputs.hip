// Validation of the device-resident inputs of a decode step: the values the host
// cannot check without a sync (committed lengths, page-table entries, selections,
// draft tokens, and the finite values the cache must hold in the slots a step
// reads but gives zero weight). The attention kernels clamp such values so that they never
// address memory outside their buffers, but the results are then unspecified;
// this pass reports them instead, as bits per sequence, for debug runs.
//
// One workgroup per sequence; every read is inside the buffers the call
// describes (the entries themselves are only compared, never dereferenced).
// Duplicate selected pages are found with a bitmap of the sequence's pages in
// LDS (one bit per page, set with LDS atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kChkThreads = 256;

struct CheckArgs {
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* nsel;
  const int32_t* tokens;
  int32_t* errors;
  int num_blocks, maxp, span, max_sel, sel_rows, gamma, vocab, words;
  int hkv, head_dim, bf16;
};

// A bf16 or fp32 element of the cache that is an infinity or a NaN (all exponent bits set).
__device__ __forceinline__ bool nonfinite(const void* base, size_t i, int bf16) {
  if (bf16) return (static_cast<const uint16_t*>(base)[i] & 0x7F80u) == 0x7F80u;
  return (__float_as_uint(static_cast<const float*>(base)[i]) & 0x7F800000u) == 0x7F800000u;
}

__global__ __launch_bounds__(kChkThreads) void check_kernel(CheckArgs a) {
  extern __shared__ uint32_t seen[];  // [words]: one bit per page of the sequence
  __shared__ int s_err;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_err = 0;
  int err = 0;
  const int L_raw = a.lens[b];
  const bool len_ok = L_raw >= 0 && static_cast<long long>(L_raw) + a.span <= static_cast<long long>(a.maxp) * kPage;
  if (!len_ok) err |= kCheckLen;
  // pages the step reads or writes: 0 .. ceil((L + span) / 16) - 1, at the clamped
  // length when the length itself is out of range
  const int L = min(max(L_raw, 0), a.maxp * kPage - a.span);
  const int used = (L + a.span + kPage - 1) / kPage;
  const int32_t* row = a.table + static_cast<size_t>(b) * a.maxp;
  for (int p = threadIdx.x; p < used; p += kChkThreads) {
    const int blk = row[p];
    if (blk < 0 || blk >= a.num_blocks) err |= kCheckPage;
  }
  // The pages holding positions L .. L + span - 1 are read whole: the drafts give
  // zero weight to their slots at and after L (or after the draft position), the
  // verify to those after L + span - 1. Zero times an infinity or a NaN is not
  // zero, so every K and V value at a position >= L in those pages must be finite.
  for (int pp = L >> 4; pp <= (L + a.span - 1) >> 4; ++pp) {
    const int blk = row[pp];
    if (blk < 0 || blk >= a.num_blocks) continue;  // reported as kCheckPage
    const int per_head = kPage * a.head_dim;
    for (int i = threadIdx.x; i < a.hkv * per_head; i += kChkThreads) {
      const int kvh = i / per_head;
      const int s = (i / a.head_dim) % kPage;
      const int d = i % a.head_dim;
      if (pp * kPage + s < L) continue;
      const size_t head = (static_cast<size_t>(blk) * a.hkv + kvh) * per_head;
      if (nonfinite(a.k, head + static_cast<size_t>(s) * a.head_dim + d, a.bf16) ||
          nonfinite(a.v, head + static_cast<size_t>(d) * kPage + s, a.bf16))
        err |= kCheckSlot;
    }
  }
  if (a.sel != nullptr) {
    const int n_full = L >> 4;
    for (int r = 0; r < a.sel_rows; ++r) {
      for (int w = threadIdx.x; w < a.words; w += kChkThreads) seen[w] = 0u;
      __syncthreads();
      const size_t srow = static_cast<size_t>(b) * a.sel_rows + r;
      const int ns_raw = a.nsel[srow];
      if (ns_raw < 0 || ns_raw > a.max_sel) err |= kCheckNumSel;
      const int ns = min(max(ns_raw, 0), a.max_sel);
      for (int e = threadIdx.x; e < ns; e += kChkThreads) {
        const int page = a.sel[srow * a.max_sel + e];
        if (page < 0 || page >= n_full) {
          err |= kCheckSelRange;
        } else {
          const uint32_t bit = 1u << (page & 31);
          if (atomicOr(&seen[page >> 5], bit) & bit) err |= kCheckSelDup;
        }
      }
      __syncthreads();
    }
  }
  if (a.tokens != nullptr) {
    for (int j = threadIdx.x; j < a.gamma; j += kChkThreads) {
      const int t = a.tokens[static_cast<size_t>(b) * a.gamma + j];
      if (t < 0 || t >= a.vocab) err |= kCheckToken;
    }
  }
  __syncthreads();
  if (err != 0) atomicOr(&s_err, err);
  __syncthreads();
  if (threadIdx.x == 0) a.errors[b] = s_err;
}

}  // namespace

size_t check_lds_bytes(int maxp) { return static_cast<size_t>((maxp + 31) / 32) * sizeof(uint32_t); }

hipError_t launch_check(const KvView& kv, int num_seqs, int span, const int32_t* sel, const int32_t* nsel,
                        int max_sel, int sel_rows, const int32_t* tokens, int gamma, int vocab, int32_t* errors,
                        hipStream_t stream) {
  CheckArgs a{};
  a.k = kv.k;
  a.v = kv.v;
  a.hkv = kv.hkv;
  a.head_dim = kv.head_dim;
  a.bf16 = kv.bf16;
  a.table = kv.table;
  a.lens = kv.lens;
  a.sel = sel;
  a.nsel = nsel;
  a.tokens = tokens;
  a.errors = errors;
  a.num_blocks = kv.num_blocks;
  a.maxp = kv.maxp;
  a.span = span;
  a.max_sel = max_sel;
  a.sel_rows = sel_rows;
  a.gamma = gamma;
  a.vocab = vocab;
  a.words = (kv.maxp + 31) / 32;
  hipLaunchKernelGGL(check_kernel, dim3(num_seqs), dim3(kChkThreads), check_lds_bytes(kv.maxp), stream, a);
  return hipGetLastError();
}

}  // namespace s3r
