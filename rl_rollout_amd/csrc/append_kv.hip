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

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(KvView kv, int offset, int rows, const T* __restrict__ k_rows,
                                                     const T* __restrict__ v_rows) {
  const int b = blockIdx.x / rows;
  const int r = blockIdx.x - b * rows;
  const int D = kv.head_dim;
  const long long t = static_cast<long long>(kv.lens[b]) + offset + r;
  if (t < 0 || t >= static_cast<long long>(kv.maxp) * kPage) return;
  const int page = static_cast<int>(t >> 4);
  const int slot = static_cast<int>(t & 15);
  const int blk = kv.table[static_cast<size_t>(b) * kv.maxp + page];
  if (blk < 0 || blk >= kv.num_blocks) return;
  T* kc = static_cast<T*>(kv.k);
  T* vc = static_cast<T*>(kv.v);
  const size_t src = (static_cast<size_t>(b) * rows + r) * kv.hkv * D;
  for (int idx = threadIdx.x; idx < kv.hkv * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    const size_t pg = (static_cast<size_t>(blk) * kv.hkv + h) * (kPage * D);
    kc[pg + static_cast<size_t>(slot) * D + d] = k_rows[src + idx];
    vc[pg + static_cast<size_t>(d) * kPage + slot] = v_rows[src + idx];
  }
}

}  // namespace

hipError_t launch_append(const KvView& kv, int num_seqs, int offset, int rows, const void* k_rows,
                         const void* v_rows, hipStream_t stream) {
  if (kv.bf16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(num_seqs * rows), dim3(256), 0, stream, kv, offset, rows,
                       static_cast<const uint16_t*>(k_rows), static_cast<const uint16_t*>(v_rows));
  else
    hipLaunchKernelGGL(append_kernel<float>, dim3(num_seqs * rows), dim3(256), 0, stream, kv, offset, rows,
                       static_cast<const float*>(k_rows), static_cast<const float*>(v_rows));
  return hipGetLastError();
}

}  // namespace s3r
