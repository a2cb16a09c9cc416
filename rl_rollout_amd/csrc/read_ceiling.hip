// Streaming-read ceiling of the GPU, the practical roof for the HBM-bound
// kernels: one pass over a 4.25 GiB buffer (about the bytes of one 16K-context
// verify call) with 16-byte loads, for several workgroup counts, load depths and
// cache policies. Each workgroup reads one contiguous share; the loads of a round
// are unconditional (clamped addresses) so that all of them are in flight before
// the first is consumed. Prints one line per configuration and a JSON summary.
// Built by rl_rollout_amd.build into rl_rollout_amd/read_ceiling; run with
// `python bench.py --read-ceiling`.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U, bool kNonTemporal>
__global__ __launch_bounds__(256) void read_pass(const u32x4_t* __restrict__ p, size_t n16, size_t per_wg,
                                                 uint32_t* out) {
  const size_t b0 = static_cast<size_t>(blockIdx.x) * per_wg;
  const size_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
  uint32_t acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + static_cast<size_t>(u) * 256;
      const size_t jj = j < b1 ? j : b1 - 1;
      v[u] = kNonTemporal ? __builtin_nontemporal_load(p + jj) : p[jj];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + static_cast<size_t>(u) * 256 < b1) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // a use of the loaded values, practically never taken
}

template <int U, bool kNonTemporal>
double run(const u32x4_t* p, size_t n16, int wgs, uint32_t* out, const char* name) {
  const size_t per_wg = (n16 + wgs - 1) / wgs;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 0.0;
  hipLaunchKernelGGL((read_pass<U, kNonTemporal>), dim3(wgs), dim3(256), 0, 0, p, n16, per_wg, out);
  if (hipDeviceSynchronize() != hipSuccess) return 0.0;
  float best = 1e30f, total = 0.f;
  for (int r = 0; r < 5; ++r) {
    hipEventRecord(a);
    hipLaunchKernelGGL((read_pass<U, kNonTemporal>), dim3(wgs), dim3(256), 0, 0, p, n16, per_wg, out);
    hipEventRecord(b);
    hipEventSynchronize(b);
    float ms = 0.f;
    hipEventElapsedTime(&ms, a, b);
    best = ms < best ? ms : best;
    total += ms;
  }
  hipEventDestroy(a);
  hipEventDestroy(b);
  const double bytes = static_cast<double>(n16) * 16.0;
  const double gbps = bytes / (best * 1e-3) / 1e9;
  printf("%-18s workgroups %6d  best %7.1f us  %6.0f GB/s  mean %6.0f GB/s\n", name, wgs, best * 1e3, gbps,
         bytes / (total / 5 * 1e-3) / 1e9);
  fflush(stdout);
  return gbps;
}

}  // namespace

int main() {
  const size_t bytes = static_cast<size_t>(4352) << 20;
  const size_t n16 = bytes / 16;
  u32x4_t* p = nullptr;
  uint32_t* out = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || hipMalloc(&out, 64) != hipSuccess) {
    fprintf(stderr, "read_ceiling: allocation failed\n");
    return 1;
  }
  if (hipMemset(p, 1, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 1;
  double best = 0.0, at512 = 0.0;
  for (int wgs : {512, 1024, 2048, 4096, 16384}) {
    const double a = run<4, true>(p, n16, wgs, out, "nontemporal, 4");
    const double b = run<8, true>(p, n16, wgs, out, "nontemporal, 8");
    const double c = run<8, false>(p, n16, wgs, out, "cached, 8");
    const double m = a > b ? (a > c ? a : c) : (b > c ? b : c);
    best = m > best ? m : best;
    if (wgs == 512) at512 = m;
  }
  printf("{\"read_ceiling_gbps\": %.0f, \"at_512_workgroups_gbps\": %.0f, \"bytes\": %zu}\n", best, at512, bytes);
  hipFree(p);
  hipFree(out);
  return 0;
}
