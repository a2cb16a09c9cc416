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

// The verify's access pattern without its arithmetic: one 4-wave workgroup per
// (sequence, kv head) unit, waves taking the unit's pages round-robin, each page
// a 4 KB K tile ([16][128] bf16, 16-byte loads) and a 4 KB V^T tile ([128][16],
// 8-byte loads) of a block taken from a random permutation (or in order), DEPTH
// pages in flight per wave, NWV waves per workgroup.
template <int DEPTH, int NWV>
__global__ __launch_bounds__(NWV * 64) void paged_pass(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                  const int32_t* __restrict__ table, int pages, int hkv,
                                                  uint32_t* out) {
  const int unit = blockIdx.x;
  const int seq = unit / hkv, h = unit % hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int n_it = (pages - wave + NWV - 1) / NWV;
  uint32_t acc = 0;
  for (int it0 = 0; it0 < n_it; it0 += DEPTH) {
    u32x4_t kf[DEPTH][4];
    uint32_t vf[DEPTH][8][2];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int it = it0 + d < n_it ? it0 + d : n_it - 1;
      const int page = wave + NWV * it;
      const size_t blk = static_cast<size_t>(table[static_cast<size_t>(seq) * pages + page]);
      const uint8_t* kp = k + ((blk * hkv + h) * 16 + r16) * 256 + grp * 16;
      const uint8_t* vp = v + (blk * hkv + h) * 4096 + r16 * 32 + grp * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[d][kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + kk * 64));
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vp + dd * 512));
        vf[d][dd][0] = t.x;
        vf[d][dd][1] = t.y;
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (it0 + d < n_it) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc ^= kf[d][kk].x ^ kf[d][kk].w;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) acc ^= vf[d][dd][0] ^ vf[d][dd][1];
      }
    }
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

template <int DEPTH, int NWV = 4>
double run_paged(const uint8_t* k, const uint8_t* v, const int32_t* table, int seqs, int pages, int hkv,
                 uint32_t* out) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 0.0;
  hipLaunchKernelGGL((paged_pass<DEPTH, NWV>), dim3(seqs * hkv), dim3(NWV * 64), 0, 0, k, v, table, pages, hkv,
                     out);
  if (hipDeviceSynchronize() != hipSuccess) return 0.0;
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    hipEventRecord(a);
    hipLaunchKernelGGL((paged_pass<DEPTH, NWV>), dim3(seqs * hkv), dim3(NWV * 64), 0, 0, k, v, table, pages, hkv,
                       out);
    hipEventRecord(b);
    hipEventSynchronize(b);
    float ms = 0.f;
    hipEventElapsedTime(&ms, a, b);
    best = ms < best ? ms : best;
  }
  hipEventDestroy(a);
  hipEventDestroy(b);
  const double bytes = static_cast<double>(seqs) * pages * hkv * 8192.0;
  const double gbps = bytes / (best * 1e-3) / 1e9;
  printf("paged, depth %d, %2d waves  units %4d  pages %5d  best %7.1f us  %6.0f GB/s\n", DEPTH, NWV, seqs * hkv,
         pages, best * 1e3, gbps);
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
  hipFree(p);
  // the verify's pattern: 64 sequences x 8 kv heads, 1029 pages each (16K tokens
  // plus the block), blocks in a random permutation (a fixed linear congruential
  // shuffle, so runs are comparable)
  const int seqs = 64, hkv = 8, pages = 1029, nb = seqs * pages;
  const size_t tile = static_cast<size_t>(nb) * hkv * 4096;
  uint8_t *k = nullptr, *v = nullptr;
  int32_t* table = nullptr;
  if (hipMalloc(&k, tile) != hipSuccess || hipMalloc(&v, tile) != hipSuccess ||
      hipMalloc(&table, sizeof(int32_t) * nb) != hipSuccess) {
    fprintf(stderr, "read_ceiling: allocation failed\n");
    return 1;
  }
  hipMemset(k, 1, tile);
  hipMemset(v, 1, tile);
  int32_t* perm = new int32_t[nb];
  for (int i = 0; i < nb; ++i) perm[i] = i;
  uint64_t x = 0x2545f4914f6cdd1dull;
  for (int i = nb - 1; i > 0; --i) {
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    const int j = static_cast<int>((x >> 33) % static_cast<uint64_t>(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  // blocks in order first (each sequence's pages in consecutive blocks), then permuted
  int32_t* ident = new int32_t[nb];
  for (int i = 0; i < nb; ++i) ident[i] = i;
  hipMemcpy(table, ident, sizeof(int32_t) * nb, hipMemcpyHostToDevice);
  delete[] ident;
  printf("blocks in order:\n");
  run_paged<1>(k, v, table, seqs, pages, hkv, out);
  run_paged<2>(k, v, table, seqs, pages, hkv, out);
  printf("blocks in a random permutation:\n");
  hipMemcpy(table, perm, sizeof(int32_t) * nb, hipMemcpyHostToDevice);
  delete[] perm;
  run_paged<1, 8>(k, v, table, seqs, pages, hkv, out);
  run_paged<2, 8>(k, v, table, seqs, pages, hkv, out);
  run_paged<1, 16>(k, v, table, seqs, pages, hkv, out);
  const double p1 = run_paged<1>(k, v, table, seqs, pages, hkv, out);
  const double p2 = run_paged<2>(k, v, table, seqs, pages, hkv, out);
  const double p3 = run_paged<3>(k, v, table, seqs, pages, hkv, out);
  const double paged = p1 > p2 ? (p1 > p3 ? p1 : p3) : (p2 > p3 ? p2 : p3);
  // the sparse draft's shape on the same pages: 52 selected pages per unit (5 % of
  // 1029), 218 MB per launch
  const double d1 = run_paged<1>(k, v, table, seqs, 52, hkv, out);
  const double d2 = run_paged<2>(k, v, table, seqs, 52, hkv, out);
  const double draft = d1 > d2 ? d1 : d2;
  // the same bytes with each unit's pages cut into two or four workgroups (1024 or
  // 2048 workgroups of 26 or 13 pages): what a draft split across workgroups could reach
  printf("the draft's bytes cut into more workgroups:\n");
  run_paged<1>(k, v, table, seqs * 2, 26, hkv, out);
  run_paged<2>(k, v, table, seqs * 2, 26, hkv, out);
  run_paged<1>(k, v, table, seqs * 4, 13, hkv, out);
  run_paged<2>(k, v, table, seqs * 4, 13, hkv, out);
  printf("{\"read_ceiling_gbps\": %.0f, \"at_512_workgroups_gbps\": %.0f, \"paged_verify_pattern_gbps\": %.0f, "
         "\"paged_draft_pattern_gbps\": %.0f, \"bytes\": %zu}\n", best, at512, paged, draft, bytes);
  hipFree(k);
  hipFree(v);
  hipFree(table);
  hipFree(out);
  return 0;
}
