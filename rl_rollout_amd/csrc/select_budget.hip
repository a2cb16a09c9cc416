// Score-selected budget of history pages for the next draft: the n_sel full
// pages with the largest summed softmax scores, ties to the lower page index,
// written in ascending page order (rit.work, "Как разреженный черновик
// сохраняет ответы плотной модели"; wispaper.ai, "Where the speedup claim holds"
// asks for a cheap selection).
//
// One workgroup per sequence. The scores are mapped to order-preserving 32-bit
// keys in LDS; a 4-pass, 8-bit radix select finds the n_sel-th largest key
// exactly (histograms in LDS, the digit found by a wave-wide suffix scan), then
// one ordered pass with wave ballots compacts the pages above the threshold plus
// the first pages equal to it. Integer work only after the key mapping, so the
// result is bit-exact and deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of x over the workgroup in thread order; returns the
// prefix and writes the workgroup total to *total (uniform). Two barriers.
__device__ __forceinline__ int block_exclusive_sum(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = wave_tot[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + incl - x;
}

// budgets (nullable): one budget per row, used instead of `budget`; `budget` is
// then the largest budget a row may take (a larger one is lowered to it, so no row
// selects more than the max_sel the host checked against it).
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ lens, int maxp,
                                                             double budget, const double* __restrict__ budgets,
                                                             int32_t* __restrict__ sel,
                                                             int32_t* __restrict__ nsel, int max_sel) {
  extern __shared__ uint32_t keys[];  // [maxp]
  __shared__ int hist[256];
  __shared__ int wave_tot[kSelWaves];
  __shared__ int s_digit, s_rem;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = max(0, lens[b]);
  const int n_full = min(L >> 4, maxp);
  int k = 0;
  if (n_full > 0) {
    double s = budget;
    if (budgets != nullptr) {
      s = budgets[b];
      if (s > budget) s = budget;  // a NaN stays NaN
    }
    // fmax/fmin return the non-NaN operand: a NaN budget keeps one page
    const double x = ceil(s * static_cast<double>(n_full) - 1e-9);
    k = static_cast<int>(fmin(fmax(x, 1.0), static_cast<double>(n_full)));
  }

  for (int p = tid; p < n_full; p += kSelThreads) keys[p] = order_key(scores[static_cast<size_t>(b) * maxp + p]);
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int rem = k;  // how many of the keys matching `prefix` are still to be taken
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int p = tid; p < n_full; p += kSelThreads) {
        const uint32_t key = keys[p];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < kWave) {
        // wave 0: lane l owns digits 4l .. 4l + 3; suffix sums from the top digit
        int c[4], own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[4 * lane + j];
          own += c[j];
        }
        int above = 0;  // count in digits owned by higher lanes
        int incl = own;
        for (int off = 1; off < kWave; off <<= 1) {
          const int v = __shfl_down(incl, off);
          if (lane + off < kWave) incl += v;
        }
        above = incl - own;
        // within the lane, from digit 4l+3 down to 4l
        int acc = above;
        int found = -1, found_rem = 0;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (found < 0 && acc + c[j] >= rem) {
            found = 4 * lane + j;
            found_rem = rem - acc;
          }
          acc += c[j];
        }
        // the chosen digit is the largest digit whose suffix count reaches rem:
        // exactly one lane finds it with acc_before < rem <= acc_before + c
        if (found >= 0 && above < rem) {
          s_digit = found;
          s_rem = found_rem;
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      mask |= 255u << shift;
      rem = s_rem;
      __syncthreads();
    }
  }
  const uint32_t thr = prefix;
  const int take_eq = rem;

  // Ordered compaction: thread t owns the contiguous pages [t * per, (t + 1) * per)
  // and counts the keys above the threshold and equal to it; one scan of the equal
  // counts fixes which equal keys are taken (the first take_eq in page order), one
  // scan of the taken counts gives each thread its output position, and every
  // thread then writes its pages in order.
  const int per = (n_full + kSelThreads - 1) / kSelThreads;
  const int p0 = min(tid * per, n_full);
  const int p1 = min(p0 + per, n_full);
  int n_gt = 0, n_eq = 0;
  if (k > 0) {
    for (int p = p0; p < p1; ++p) {
      const uint32_t key = keys[p];
      n_gt += key > thr;
      n_eq += key == thr;
    }
  }
  int eq_tot = 0, take_tot = 0;
  const int eq_before = block_exclusive_sum(n_eq, wave_tot, &eq_tot);
  const int eq_take = min(max(take_eq - eq_before, 0), n_eq);  // this thread's equal keys that are taken
  int pos = block_exclusive_sum(n_gt + eq_take, wave_tot, &take_tot);
  if (k > 0) {
    int eq_left = eq_take;
    for (int p = p0; p < p1 && pos < max_sel; ++p) {
      const uint32_t key = keys[p];
      const bool take = key > thr || (key == thr && eq_left > 0);
      eq_left -= (key == thr);
      if (take) sel[static_cast<size_t>(b) * max_sel + pos++] = p;
    }
  }
  const int written = take_tot;
  for (int j = min(written, max_sel) + tid; j < max_sel; j += kSelThreads) sel[static_cast<size_t>(b) * max_sel + j] = -1;
  if (tid == 0) nsel[b] = k;
  (void)lane;
}

}  // namespace

hipError_t launch_select(const float* scores, const int32_t* lens, int num_seqs, int maxp, double budget,
                         int32_t* sel, int32_t* nsel, int max_sel, hipStream_t stream, const double* budgets) {
  const size_t smem = static_cast<size_t>(maxp) * 4;
  hipLaunchKernelGGL(select_kernel, dim3(num_seqs), dim3(kSelThreads), smem, stream, scores, lens, maxp, budget,
                     budgets, sel, nsel, max_sel);
  return hipGetLastError();
}

}  // namespace s3r
