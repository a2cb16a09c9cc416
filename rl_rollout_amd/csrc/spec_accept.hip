// Exact speculative sampling of one drafted block per sequence (rebasdaily.com,
// "草稿可以稀疏，交卷必须完整"; rit.work, "Как разреженный черновик сохраняет
// ответы плотной модели"): draft token d_j is kept with probability
// min(1, p_j(d_j) / q_j(d_j)); at the first rejection one token is drawn from
// max(0, p_j - q_j) normalised, or, if every draft is kept, from p_gamma.
//
// Three kernels, all reading the logits with 16-byte vector loads:
//   accept_rowstats  grid (sequence x logit row, vocab chunk): per chunk the
//                    logit max and the double-precision sum of exp((l - max)/T).
//                    This is the one full pass over the 2*gamma+1 rows and the
//                    HBM-bound part.
//   accept_residual  grid (sequence, vocab chunk): every workgroup merges its
//                    sequence's row statistics, replays the accept tests in
//                    double precision (cheap, redundant per chunk, no extra
//                    launch), then sums the residual (or bonus) mass of its chunk
//                    in double precision and records the last index with mass.
//   accept_pick      grid (sequence): prefix over chunk sums, finds the chunk
//                    holding u * R, rescans only that chunk with a workgroup scan
//                    to get the smallest index whose cumulative mass exceeds
//                    u * R, writes tokens and commits ctx_lens += a + 1.
// Probabilities at the tested and sampled tokens use double-precision exp of
// (l - max) / T over the double-precision normaliser; the row sums use the
// hardware exp2 in fp32 per element and double accumulation.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kAccThreads = 256;
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;

struct AcceptArgs {
  const void* tl;
  const void* dl;
  const int32_t* dtok;
  const float* ua;
  const float* us;
  int32_t* nacc;
  int32_t* out;
  int32_t* ctx;
  float* st_m;      // [B][rows][nch]
  double* st_s;     // [B][rows][nch]
  double* rsum;     // [B][nch2]
  int32_t* rlast;   // [B][nch2]
  int32_t* dec;     // [B][2]: accepted count, mode
  int B, gamma, V, rows, nch, clen, nch2, clen2;
  float c_hi, c_lo; // log2(e) / T split into float head + tail (exponent scale)
  double c_d;       // log2(e) / T
  double inv_t;     // 1 / T
};

// 2^((v - m) * log2(e) / T) with the scale carried in two floats, so the fp32
// exponent has no systematic error from rounding log2(e) / T.
__device__ __forceinline__ float exp_scaled(float d, float c_hi, float c_lo) {
  return fast_exp2(fmaf(d, c_hi, d * c_lo));
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const AcceptArgs& a, int b, int r) {
  const int G1 = a.gamma + 1;
  if (r < G1) return static_cast<const T*>(a.tl) + (static_cast<size_t>(b) * G1 + r) * a.V;
  return static_cast<const T*>(a.dl) + (static_cast<size_t>(b) * a.gamma + (r - G1)) * a.V;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int x) {
  if constexpr (std::is_same<T, bf16_t>::value)
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[x]);
  else
    return reinterpret_cast<const float*>(p)[x];
}

// Load 8 consecutive logits starting at x (x multiple of 8, row 16-byte aligned).
template <typename T>
__device__ __forceinline__ void ld8(const T* p, int x, float (&v)[8]) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const uint4 u = ld_stream16(reinterpret_cast<const uint16_t*>(p) + x);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4 a0 = ld_stream16f(reinterpret_cast<const float*>(p) + x);
    const float4 a1 = ld_stream16f(reinterpret_cast<const float*>(p) + x + 4);
    v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
    v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
  }
}

__device__ __forceinline__ double block_sum_f64(double x, double* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum_f64(x);
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kAccThreads / kWave; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------- row statistics
template <typename T>
__global__ __launch_bounds__(kAccThreads) void accept_rowstats(AcceptArgs a) {
  __shared__ float sm_m[kAccThreads / kWave];
  __shared__ double sm_s[kAccThreads / kWave];
  const int row = blockIdx.x;
  const int chunk = blockIdx.y;
  const int b = row / a.rows;
  const int r = row - b * a.rows;
  const T* p = row_ptr<T>(a, b, r);
  const int x0 = chunk * a.clen;
  const int x1 = min(a.V, x0 + a.clen);
  float m = -INFINITY;
  double s = 0.0;
  const bool vec = (a.V % 8) == 0;
  if (vec) {
    for (int x = x0 + threadIdx.x * 8; x < x1; x += kAccThreads * 8) {
      float v[8];
      ld8<T>(p, x, v);
      float m8 = v[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) m8 = fmaxf(m8, v[j]);
      if (m8 > m) {
        if (m != -INFINITY) s *= exp2((static_cast<double>(m) - static_cast<double>(m8)) * a.c_d);
        m = m8;
      }
      float e = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) e += exp_scaled(v[j] - m, a.c_hi, a.c_lo);
      s += static_cast<double>(e);
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kAccThreads) {
      const float v = ld<T>(p, x);
      if (v > m) {
        if (m != -INFINITY) s *= exp2((static_cast<double>(m) - static_cast<double>(v)) * a.c_d);
        m = v;
      }
      s += static_cast<double>(exp_scaled(v - m, a.c_hi, a.c_lo));
    }
  }
  // workgroup merge
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float wm = wave_max(m);
  double ws = (m == -INFINITY) ? 0.0 : s * exp2((static_cast<double>(m) - static_cast<double>(wm)) * a.c_d);
  ws = wave_sum_f64(ws);
  if (lane == 0) {
    sm_m[wave] = wm;
    sm_s[wave] = ws;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = -INFINITY;
    for (int w = 0; w < kAccThreads / kWave; ++w) mm = fmaxf(mm, sm_m[w]);
    double ss = 0.0;
    for (int w = 0; w < kAccThreads / kWave; ++w)
      if (sm_m[w] != -INFINITY)
        ss += sm_s[w] * exp2((static_cast<double>(sm_m[w]) - static_cast<double>(mm)) * a.c_d);
    const size_t o = static_cast<size_t>(row) * a.nch + chunk;
    a.st_m[o] = mm;
    a.st_s[o] = ss;
  }
}

// Row statistics of sequence b merged over chunks: max logit and the normaliser
// Z = sum exp((l - max) / T).
__device__ void merge_rows(const AcceptArgs& a, int b, float* Ms, double* Zs) {
  for (int r = threadIdx.x; r < a.rows; r += kAccThreads) {
    const size_t o = (static_cast<size_t>(b) * a.rows + r) * a.nch;
    float mm = -INFINITY;
    for (int c = 0; c < a.nch; ++c) mm = fmaxf(mm, a.st_m[o + c]);
    double z = 0.0;
    for (int c = 0; c < a.nch; ++c) {
      const float mc = a.st_m[o + c];
      if (mc != -INFINITY) z += a.st_s[o + c] * exp2((static_cast<double>(mc) - static_cast<double>(mm)) * a.c_d);
    }
    Ms[r] = mm;
    Zs[r] = z;
  }
}

__device__ __forceinline__ double prob_at(double logit, float M, double Z, double inv_t) {
  return exp((logit - static_cast<double>(M)) * inv_t) / Z;
}

// Residual (or bonus) mass at token x.
template <typename T>
__device__ __forceinline__ double resid_at(const T* pt, const T* pd, int x, int mode, float Mt, double Zt, float Md,
                                           double Zd, double inv_t) {
  const double p = prob_at(static_cast<double>(ld<T>(pt, x)), Mt, Zt, inv_t);
  if (mode == kModeBonus) return p;
  const double q = prob_at(static_cast<double>(ld<T>(pd, x)), Md, Zd, inv_t);
  return fmax(0.0, p - q);
}

// Accept tests of sequence b (one thread). Returns the accepted count.
template <typename T>
__device__ int decide(const AcceptArgs& a, int b, const float* Ms, const double* Zs) {
  const int G1 = a.gamma + 1;
  int acc = 0;
  for (int j = 0; j < a.gamma; ++j) {
    int x = a.dtok[static_cast<size_t>(b) * a.gamma + j];
    x = min(max(x, 0), a.V - 1);
    const double p = prob_at(static_cast<double>(ld<T>(row_ptr<T>(a, b, j), x)), Ms[j], Zs[j], a.inv_t);
    const double q = prob_at(static_cast<double>(ld<T>(row_ptr<T>(a, b, G1 + j), x)), Ms[G1 + j], Zs[G1 + j], a.inv_t);
    const double u = static_cast<double>(a.ua[static_cast<size_t>(b) * a.gamma + j]);
    if (q == 0.0 || u < p / q) {
      ++acc;
    } else {
      break;
    }
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kAccThreads) void accept_residual(AcceptArgs a) {
  extern __shared__ unsigned char smem_raw[];
  double* Zs = reinterpret_cast<double*>(smem_raw);
  float* Ms = reinterpret_cast<float*>(Zs + a.rows);
  __shared__ double scratch[kAccThreads / kWave];
  __shared__ int s_a;
  __shared__ int s_last[kAccThreads / kWave];
  const int b = blockIdx.x;
  const int chunk = blockIdx.y;
  merge_rows(a, b, Ms, Zs);
  __syncthreads();
  if (threadIdx.x == 0) s_a = decide<T>(a, b, Ms, Zs);
  __syncthreads();
  const int acc = s_a;
  const int mode = acc < a.gamma ? kModeResidual : kModeBonus;
  const int G1 = a.gamma + 1;
  const T* pt = row_ptr<T>(a, b, acc);                         // target row of the decision
  const T* pd = row_ptr<T>(a, b, G1 + min(acc, a.gamma - 1));  // matching draft row (unused for bonus)
  const float Mt = Ms[acc];
  const double Zt = Zs[acc];
  const float Md = Ms[G1 + min(acc, a.gamma - 1)];
  const double Zd = Zs[G1 + min(acc, a.gamma - 1)];

  const int x0 = chunk * a.clen2;
  const int x1 = min(a.V, x0 + a.clen2);
  double s = 0.0;
  int last = -1;
  for (int x = x0 + threadIdx.x; x < x1; x += kAccThreads) {
    const double r = resid_at<T>(pt, pd, x, mode, Mt, Zt, Md, Zd, a.inv_t);
    s += r;
    if (r > 0.0) last = x;
  }
  const double tot = block_sum_f64(s, scratch);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wl = wave_max_i(last);
  if (lane == 0) s_last[wave] = wl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int l = -1;
    for (int w = 0; w < kAccThreads / kWave; ++w) l = max(l, s_last[w]);
    a.rsum[static_cast<size_t>(b) * a.nch2 + chunk] = tot;
    a.rlast[static_cast<size_t>(b) * a.nch2 + chunk] = l;
    if (chunk == 0) {
      a.dec[2 * b] = acc;
      a.dec[2 * b + 1] = mode;
      a.nacc[b] = acc;
    }
  }
  if (chunk == 0) {
    for (int j = threadIdx.x; j < acc; j += kAccThreads)
      a.out[static_cast<size_t>(b) * G1 + j] = a.dtok[static_cast<size_t>(b) * a.gamma + j];
  }
}

// Inclusive workgroup scan (thread order) of doubles; returns the inclusive value.
__device__ __forceinline__ double block_scan_incl_f64(double x, double* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) scratch[wave] = x;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += scratch[w];
  __syncthreads();
  return before + x;
}

// Smallest index in [x0, x1) whose running mass (starting at `base`) exceeds thr,
// scanning contiguous per-thread segments; -1 if none. `mass(x)` gives r_x.
template <typename F>
__device__ int find_crossing(int x0, int x1, double base, double thr, F mass, double* scratch, int* s_tok) {
  const int n = x1 - x0;
  const int seg = (n + kAccThreads - 1) / kAccThreads;
  const int s0 = x0 + min(n, static_cast<int>(threadIdx.x) * seg);
  const int s1 = x0 + min(n, (static_cast<int>(threadIdx.x) + 1) * seg);
  double ss = 0.0;
  for (int x = s0; x < s1; ++x) ss += mass(x);
  const double incl = block_scan_incl_f64(ss, scratch);
  if (threadIdx.x == 0) *s_tok = 0x7fffffff;
  __syncthreads();
  double cum = base + (incl - ss);
  if (base + incl > thr) {
    for (int x = s0; x < s1; ++x) {
      const double r = mass(x);
      cum += r;
      if (cum > thr && r > 0.0) {
        atomicMin(s_tok, x);
        break;
      }
    }
  }
  __syncthreads();
  const int t = *s_tok;
  __syncthreads();
  return t == 0x7fffffff ? -1 : t;
}

template <typename T>
__global__ __launch_bounds__(kAccThreads) void accept_pick(AcceptArgs a) {
  extern __shared__ unsigned char smem_raw[];
  double* Zs = reinterpret_cast<double*>(smem_raw);
  float* Ms = reinterpret_cast<float*>(Zs + a.rows);
  __shared__ double scratch[kAccThreads / kWave];
  __shared__ int s_tok;
  __shared__ int s_chunk;
  __shared__ double s_base, s_thr;
  const int b = blockIdx.x;
  const int G1 = a.gamma + 1;
  merge_rows(a, b, Ms, Zs);
  const int acc = a.dec[2 * b];
  int mode = a.dec[2 * b + 1];
  const double u = static_cast<double>(a.us[b]);
  if (threadIdx.x == 0) {
    const double* rs = a.rsum + static_cast<size_t>(b) * a.nch2;
    double R = 0.0;
    for (int c = 0; c < a.nch2; ++c) R += rs[c];
    const double thr = u * R;
    double run = 0.0;
    int cstar = -1;
    double base = 0.0;
    if (R > 0.0) {
      for (int c = 0; c < a.nch2; ++c) {
        if (run + rs[c] > thr) {
          cstar = c;
          base = run;
          break;
        }
        run += rs[c];
      }
    }
    s_chunk = (R > 0.0) ? cstar : -2;  // -2: residual with zero mass
    s_base = base;
    s_thr = thr;
  }
  __syncthreads();
  const T* pt = row_ptr<T>(a, b, acc);
  const T* pd = row_ptr<T>(a, b, G1 + min(acc, a.gamma - 1));
  const float Mt = Ms[acc];
  const double Zt = Zs[acc];
  const float Md = Ms[G1 + min(acc, a.gamma - 1)];
  const double Zd = Zs[G1 + min(acc, a.gamma - 1)];
  const double inv_t = a.inv_t;
  int token = -1;
  const int cstar = s_chunk;
  if (cstar >= 0) {
    const int x0 = cstar * a.clen2;
    const int x1 = min(a.V, x0 + a.clen2);
    auto mass = [&](int x) { return resid_at<T>(pt, pd, x, mode, Mt, Zt, Md, Zd, inv_t); };
    token = find_crossing(x0, x1, s_base, s_thr, mass, scratch, &s_tok);
    if (token < 0) token = a.rlast[static_cast<size_t>(b) * a.nch2 + cstar];
  } else if (cstar == -1) {
    // rounding left no crossing: largest index with mass
    int l = -1;
    for (int c = 0; c < a.nch2; ++c) l = max(l, a.rlast[static_cast<size_t>(b) * a.nch2 + c]);
    token = l;
  } else {
    // zero residual mass: draw from p of the decision row over the whole vocabulary
    mode = kModeBonus;
    auto mass = [&](int x) { return resid_at<T>(pt, pd, x, kModeBonus, Mt, Zt, Md, Zd, inv_t); };
    double part = 0.0;
    for (int x = threadIdx.x; x < a.V; x += kAccThreads) part += mass(x);
    const double W = block_sum_f64(part, scratch);
    token = find_crossing(0, a.V, 0.0, u * W, mass, scratch, &s_tok);
    if (token < 0) token = a.V - 1;
  }
  if (threadIdx.x == 0) {
    a.out[static_cast<size_t>(b) * G1 + acc] = token;
    for (int j = acc + 1; j < G1; ++j) a.out[static_cast<size_t>(b) * G1 + j] = -1;
    if (a.ctx != nullptr) a.ctx[b] += acc + 1;
  }
  (void)mode;
}

template <typename T>
hipError_t launch_typed(const AcceptArgs& a, hipStream_t stream) {
  const size_t smem = static_cast<size_t>(a.rows) * (8 + 4) + 16;
  hipLaunchKernelGGL(accept_rowstats<T>, dim3(a.B * a.rows, a.nch), dim3(kAccThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_residual<T>, dim3(a.B, a.nch2), dim3(kAccThreads), smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_pick<T>, dim3(a.B), dim3(kAccThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

AcceptPlan plan_accept(int num_seqs, int gamma, int vocab) {
  AcceptPlan pl{};
  pl.num_seqs = num_seqs;
  pl.gamma = gamma;
  pl.vocab = vocab;
  pl.rows = 2 * gamma + 1;
  pl.clen = 8192;
  pl.nch = (vocab + pl.clen - 1) / pl.clen;
  pl.clen2 = 4096;
  pl.nch2 = (vocab + pl.clen2 - 1) / pl.clen2;
  const size_t B = num_seqs;
  size_t off = 0;
  pl.off_st_m = off;
  off = align_up(off + B * pl.rows * pl.nch * 4, 256);
  pl.off_st_s = off;
  off = align_up(off + B * pl.rows * pl.nch * 8, 256);
  pl.off_rsum = off;
  off = align_up(off + B * pl.nch2 * 8, 256);
  pl.off_rlast = off;
  off = align_up(off + B * pl.nch2 * 4, 256);
  pl.off_dec = off;
  off = align_up(off + B * 2 * 4, 256);
  pl.bytes = off;
  return pl;
}

hipError_t launch_accept(const AcceptPlan& pl, int bf16, const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                         float temperature, int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens,
                         void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  AcceptArgs a{};
  a.tl = target_logits;
  a.dl = draft_logits;
  a.dtok = draft_tokens;
  a.ua = u_accept;
  a.us = u_sample;
  a.nacc = num_accepted;
  a.out = out_tokens;
  a.ctx = ctx_lens;
  a.st_m = reinterpret_cast<float*>(ws + pl.off_st_m);
  a.st_s = reinterpret_cast<double*>(ws + pl.off_st_s);
  a.rsum = reinterpret_cast<double*>(ws + pl.off_rsum);
  a.rlast = reinterpret_cast<int32_t*>(ws + pl.off_rlast);
  a.dec = reinterpret_cast<int32_t*>(ws + pl.off_dec);
  a.B = pl.num_seqs;
  a.gamma = pl.gamma;
  a.V = pl.vocab;
  a.rows = pl.rows;
  a.nch = pl.nch;
  a.clen = pl.clen;
  a.nch2 = pl.nch2;
  a.clen2 = pl.clen2;
  a.c_d = 1.4426950408889634074 / static_cast<double>(temperature);
  a.c_hi = static_cast<float>(a.c_d);
  a.c_lo = static_cast<float>(a.c_d - static_cast<double>(a.c_hi));
  a.inv_t = 1.0 / static_cast<double>(temperature);
  return bf16 ? launch_typed<bf16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace s3r
