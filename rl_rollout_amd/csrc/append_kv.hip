// Writes new K/V rows into the paged cache at ctx_lens[b] + offset + r: the draft
// rows of each draft step, then the verify block's rows, which verification
// recomputes with full attention (rebasdaily.com, "真正难搬的，还是那叠完整笔记").
// K rows land contiguously in their page slot; V rows are scattered into the
// page-transposed V slab (one element per dim, stride 16).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

// One workgroup per new row (sequence b, row r); each thread moves 16 bytes of K
// and of V per pass. The thread's first 16-byte chunks of the row and the
// sequence's length are loaded together, then the page-table entry, then the
// stores: two memory round trips before the first store.
//
// Workgroup r * seqs_pad + b takes row r of sequence b, with seqs_pad a multiple
// of the 8 XCDs: the dispatcher deals workgroups to the XCDs round-robin, so all
// rows of a sequence run on one XCD. Their V elements of one dim share a 32-byte
// sector of the page-transposed slab; written from one XCD they merge in its L2
// before going to HBM, instead of one partial write-back per row.
constexpr int kAppendThreads = 128;  // one pass over a row of 8 kv heads x 128 dims in bf16
constexpr int kXcds = 8;

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(KvView kv, int offset, int rows, int num_seqs,
                                                                int seqs_pad, const T* __restrict__ k_rows,
                                                                const T* __restrict__ v_rows) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk; divides head_dim (64 or 128)
  const int r = blockIdx.x / seqs_pad;
  const int b = blockIdx.x - r * seqs_pad;
  if (b >= num_seqs) return;
  const int D = kv.head_dim;
  const int n = kv.hkv * D;  // elements of one row, a multiple of EPC
  const size_t src = (static_cast<size_t>(b) * rows + r) * n;
  const int i0 = threadIdx.x * EPC;
  // first chunk, at an index clamped into the row (threads past the row store nothing)
  const int ic = min(i0, n - EPC);
  u32x4_t kq = *reinterpret_cast<const u32x4_t*>(k_rows + src + ic);
  u32x4_t vq = *reinterpret_cast<const u32x4_t*>(v_rows + src + ic);
  int len = kv.lens[b];
  // the three values are needed here: the loads go out together, not sunk past
  // the checks below
  asm volatile("" : "+v"(kq), "+v"(vq), "+s"(len));
  const long long t = static_cast<long long>(len) + offset + r;
  if (t < 0 || t >= static_cast<long long>(kv.maxp) * kPage) return;
  const int page = static_cast<int>(t >> 4);
  const int slot = static_cast<int>(t & 15);
  const int blk = kv.table[static_cast<size_t>(b) * kv.maxp + page];
  if (blk < 0 || blk >= kv.num_blocks) return;
  T* kc = static_cast<T*>(kv.k);
  T* vc = static_cast<T*>(kv.v);
  // K: the chunk is contiguous in the row's page slot; V: one element per dim of
  // the page-transposed slab (stride 16 elements)
  auto put = [&](int i, const u32x4_t& kk, const u32x4_t& vv) {
    const int h = i / D;
    const int d = i - h * D;
    const size_t pg = (static_cast<size_t>(blk) * kv.hkv + h) * (kPage * D);
    *reinterpret_cast<u32x4_t*>(kc + pg + static_cast<size_t>(slot) * D + d) = kk;
    T vals[EPC];
    __builtin_memcpy(vals, &vv, 16);
#pragma unroll
    for (int e = 0; e < EPC; ++e) vc[pg + static_cast<size_t>(d + e) * kPage + slot] = vals[e];
  };
  if (i0 < n) put(i0, kq, vq);
  for (int i = i0 + kAppendThreads * EPC; i < n; i += kAppendThreads * EPC) {
    put(i, *reinterpret_cast<const u32x4_t*>(k_rows + src + i), *reinterpret_cast<const u32x4_t*>(v_rows + src + i));
  }
}

}  // namespace

hipError_t launch_append(const KvView& kv, int num_seqs, int offset, int rows, const void* k_rows,
                         const void* v_rows, hipStream_t stream) {
  const int seqs_pad = (num_seqs + kXcds - 1) / kXcds * kXcds;
  const dim3 grid(static_cast<unsigned>(seqs_pad) * rows);
  if (kv.bf16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, stream, kv, offset, rows, num_seqs,
                       seqs_pad, static_cast<const uint16_t*>(k_rows), static_cast<const uint16_t*>(v_rows));
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(kAppendThreads), 0, stream, kv, offset, rows, num_seqs,
                       seqs_pad, static_cast<const float*>(k_rows), static_cast<const float*>(v_rows));
  return hipGetLastError();
}

}  // namespace s3r
