// Exact speculative sampling of one drafted block per sequence (rebasdaily.com,
// "草稿可以稀疏，交卷必须完整"; rit.work, "Как разреженный черновик сохраняет
// ответы плотной модели"): draft token d_j is kept with probability
// min(1, p_j(d_j) / q_j(d_j)); at the first rejection one token is drawn from
// max(0, p_j - q_j) normalised, or, if every draft is kept, from p_gamma.
//
// Three kernels:
//   accept_rowstats  grid (sequence x logit row, vocab chunk of 64K): per chunk
//                    the logit max and the sum of exp((l - max) / T), with eight
//                    16-byte non-temporal loads in flight per thread. This is the
//                    one full pass over the 2 gamma + 1 rows and the HBM-bound part.
//   accept_residual  grid (sequence, group of cpw vocab chunks of 4K): each
//                    workgroup first takes the sequence's accept decision (merges
//                    the chunk statistics of its rows, replays the accept tests in
//                    double precision; the group holding chunk 0 writes the
//                    accepted count, the kept drafts and the statistics of the
//                    final draw's rows), then, for each chunk of its group, sums
//                    the residual (or bonus) mass in double and finds the chunk's
//                    last index with mass, loading the next chunk while it sums
//                    this one; it reads only the one or two rows the final draw
//                    uses. cpw grows with the batch so that the workgroups fit the
//                    chip about once and the decision is replayed that often.
//   accept_pick      grid (sequence): scans the chunk masses, rescans only the
//                    chunk holding u * R with a workgroup prefix sum to find the
//                    smallest index whose cumulative mass exceeds u * R, writes the
//                    token and commits ctx_lens += a + 1.
// Precision: the accept test p/q < u uses double-precision exp of (l - max) / T
// over double normalisers. Per-element masses use the hardware exp2 in fp32 with
// the exponent scale log2(e)/T carried as a float pair (no systematic error from
// rounding the scale; about 1 ulp per term, which averages out in the sums) and
// are summed in double.
#include <float.h>
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kAccThreads = 256;
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;
constexpr int kResChunk = 4096;  // residual chunk: two rounds of 8 tokens per thread
constexpr int kPickSeg = kResChunk / kAccThreads;  // tokens per thread in the final chunk rescan
constexpr int kMaxCpw = 8;       // residual chunks per workgroup, at most
static_assert(kResChunk % (kAccThreads * 8) == 0, "a residual chunk is whole rounds of 8 tokens per thread");

struct AcceptArgs {
  const void* tl;
  const void* dl;
  const int32_t* dtok;
  const float* ua;
  const float* us;
  int32_t* nacc;
  int32_t* out;
  int32_t* ctx;
  float* st_m;      // [B][rows][nch]  chunk max
  double* st_s;     // [B][rows][nch]  chunk sum of exp((l - max) / T)
  double* dstat;    // [B][4]          M_target, Z_target, M_draft, Z_draft of the final draw's rows
  int32_t* dec;     // [B][2]          accepted count, mode
  double* rsum;     // [B][nch2]       residual mass per chunk
  int32_t* rlast;   // [B][nch2]       last index with mass per chunk (-1: none)
  const int32_t* horizons;  // optional [B]: sequence b tests only its first horizons[b] drafts
  int B, gamma, V, rows, nch, clen, nch2, clen2;
  int cpw;          // residual chunks per workgroup (1 .. kMaxCpw)
  float c_hi, c_lo; // log2(e) / T split into float head + tail
  double c_d;       // log2(e) / T
  double inv_t;     // 1 / T
};

// 2^((v - m) * log2(e) / T) in fp32 with the scale carried in two floats. The
// host rounds c_hi down and keeps c_lo at least FLT_MIN, so both are positive: a
// masked logit (d = -inf) gives -inf + -inf and no mass, never inf - inf.
__device__ __forceinline__ float exp_scaled(float d, float c_hi, float c_lo) {
  return fast_exp2(fmaf(d, c_hi, d * c_lo));
}

// Draft horizon gamma_b of sequence b (gamma without per-sequence horizons).
__device__ __forceinline__ int horizon_of(const AcceptArgs& a, int b) {
  return a.horizons != nullptr ? min(max(a.horizons[b], 0), a.gamma) : a.gamma;
}

// Whether row r of sequence b is read under horizon gb: target rows 0 .. gb and
// draft rows 0 .. gb - 1.
__device__ __forceinline__ bool row_in_horizon(const AcceptArgs& a, int r, int gb) {
  const int G1 = a.gamma + 1;
  return r < G1 ? r <= gb : r - G1 < gb;
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

// 8 consecutive logits at x (x multiple of 8, rows 16-byte aligned), streamed:
// the raw bits (issued now) and their conversion to float (where they are used).
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  uint4 u;
};
template <>
struct Raw8<float> {
  float4 a, b;
};
template <typename T>
__device__ __forceinline__ Raw8<T> ld8_raw(const T* p, int x) {
  Raw8<T> r;
  if constexpr (std::is_same<T, bf16_t>::value) {
    r.u = ld_stream16(reinterpret_cast<const uint16_t*>(p) + x);
  } else {
    r.a = ld_stream16f(reinterpret_cast<const float*>(p) + x);
    r.b = ld_stream16f(reinterpret_cast<const float*>(p) + x + 4);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void cvt8(const Raw8<T>& r, float (&v)[8]) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
}

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

// ---------------------------------------------------------------- row statistics
// U: 16-byte loads issued together per thread before their values are absorbed
// (the whole chunk is a few such rounds, so U sets how many memory latencies the
// workgroup waits in sequence).
template <typename T, int U>
__global__ __launch_bounds__(kAccThreads) void accept_rowstats(AcceptArgs a) {
  __shared__ float sm_m[kAccThreads / kWave];
  __shared__ double sm_s[kAccThreads / kWave];
  const int row = blockIdx.x;
  const int chunk = blockIdx.y;
  const int b = row / a.rows;
  const int r = row - b * a.rows;
  // rows past the sequence's horizon are never read (uniform over the workgroup)
  if (a.horizons != nullptr && !row_in_horizon(a, r, horizon_of(a, b))) return;
  const T* p = row_ptr<T>(a, b, r);
  const int x0 = chunk * a.clen;
  const int x1 = min(a.V, x0 + a.clen);
  float m = -INFINITY;
  double s = 0.0;
  // m <- max(m, values); s rescaled to the new max, plus the values' mass. A
  // group of masked (-inf) logits has no mass; skipping it also keeps
  // -inf - (-inf) out of the sum while m is still -inf.
  auto absorb = [&](const float* v, int n) {
    float mv = v[0];
    for (int j = 1; j < n; ++j) mv = fmaxf(mv, v[j]);
    if (mv == -INFINITY) return;
    if (mv > m) {
      if (m != -INFINITY) s *= exp2((static_cast<double>(m) - static_cast<double>(mv)) * a.c_d);
      m = mv;
    }
    float e = 0.f;
    for (int j = 0; j < n; ++j) e += exp_scaled(v[j] - m, a.c_hi, a.c_lo);
    s += static_cast<double>(e);
  };
  if ((a.V % 8) == 0) {
    // The U loads of a round are unconditional (addresses past the chunk are
    // clamped to its last group of 8 and their values ignored), so they are all
    // in flight before the first is waited for; a guarded load would end the
    // basic block and make the compiler wait for it on the spot.
    // The wave keeps one reference m for all its lanes: each round first takes
    // the wave's maximum of the loaded values and moves m only when that exceeds
    // it by more than kRowSlack (log2 units, after the 1/T scale), in one uniform
    // branch, so the double-precision rescale of the sums is rare and never
    // divergent; the weights against a stale reference stay below 2^kRowSlack.
    constexpr float kRowSlack = 8.f;
    const int last = x1 - 8;
    for (int xb = x0 + threadIdx.x * 8; xb < x1; xb += kAccThreads * 8 * U) {
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) ld8<T>(p, min(xb + u * kAccThreads * 8, last), v[u]);
      float mv = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (xb + u * kAccThreads * 8 < x1) {
#pragma unroll
          for (int j = 0; j < 8; ++j) mv = fmaxf(mv, v[u][j]);
        }
      }
      mv = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_max(mv))));
      // uniform; true from -inf to a finite maximum, false while everything is -inf
      if ((mv - m) * a.c_hi > kRowSlack) {
        if (m != -INFINITY) s *= exp2((static_cast<double>(m) - static_cast<double>(mv)) * a.c_d);
        m = mv;
      }
      if (m == -INFINITY) continue;  // every value the wave has seen is masked: no mass yet
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (xb + u * kAccThreads * 8 < x1) {
          float e = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) e += exp_scaled(v[u][j] - m, a.c_hi, a.c_lo);
          s += static_cast<double>(e);
        }
      }
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kAccThreads) {
      const float v = ld<T>(p, x);
      absorb(&v, 1);
    }
  }
  // workgroup merge
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float wm = wave_max(m);
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

__device__ __forceinline__ double prob_at(double logit, float M, double Z, double inv_t) {
  return exp((logit - static_cast<double>(M)) * inv_t) / Z;
}

// ---------------------------------------------------------------- decision
// The accept decision of sequence b. Wave 0 merges the chunk statistics of the
// sequence's rows into the row max and normaliser, then runs every test at once
// in double precision (lane j evaluates draft j); the accepted count is the
// position of the first failing test. Every workgroup that needs the decision
// computes it (they all reach the same result from the same inputs); the one
// with `publish` set also writes the count, the kept drafts and the statistics
// of the final draw's rows. All threads of the workgroup call this: it holds
// two barriers. Returns the accepted count.
template <typename T>
__device__ int decide(const AcceptArgs& a, int b, bool publish, float* Ms, double* Zs, int* s_acc) {
  const int lane = threadIdx.x & 63;
  const bool w0 = threadIdx.x < kWave;
  const int G1 = a.gamma + 1;
  const int gb = horizon_of(a, b);
  if (w0) {
    for (int r = lane; r < a.rows; r += kWave) {
      if (!row_in_horizon(a, r, gb)) {  // no statistics were taken; never used
        Ms[r] = 0.f;
        Zs[r] = 1.0;
        continue;
      }
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
  __syncthreads();
  if (w0) {
    int acc = gb;
    for (int j0 = 0; j0 < gb && acc == gb; j0 += kWave) {
      const int j = j0 + lane;
      bool ok = true;
      if (j < gb) {
        int x = a.dtok[static_cast<size_t>(b) * a.gamma + j];
        x = min(max(x, 0), a.V - 1);
        const double p = prob_at(static_cast<double>(ld<T>(row_ptr<T>(a, b, j), x)), Ms[j], Zs[j], a.inv_t);
        const double q =
            prob_at(static_cast<double>(ld<T>(row_ptr<T>(a, b, G1 + j), x)), Ms[G1 + j], Zs[G1 + j], a.inv_t);
        const double u = static_cast<double>(a.ua[static_cast<size_t>(b) * a.gamma + j]);
        // keep iff u q < p: with q = 0 (the draft row masks its own token) the
        // draft is kept exactly when the target gives it mass
        ok = (u * q < p);
      }
      const unsigned long long fail = __ballot(!ok);
      if (fail) acc = j0 + __ffsll(static_cast<long long>(fail)) - 1;
    }
    if (lane == 0) {
      *s_acc = acc;
      if (publish) {
        const int dr = G1 + min(acc, a.gamma - 1);  // draft row of the residual (unused for the bonus)
        a.dec[2 * b] = acc;
        a.dec[2 * b + 1] = acc < gb ? kModeResidual : kModeBonus;
        a.dstat[4 * b + 0] = static_cast<double>(Ms[acc]);
        a.dstat[4 * b + 1] = Zs[acc];
        a.dstat[4 * b + 2] = static_cast<double>(Ms[dr]);
        a.dstat[4 * b + 3] = Zs[dr];
        a.nacc[b] = acc;
      }
    }
    if (publish)
      for (int j = lane; j < acc; j += kWave)
        a.out[static_cast<size_t>(b) * G1 + j] = a.dtok[static_cast<size_t>(b) * a.gamma + j];
  }
  __syncthreads();
  return *s_acc;
}

// Rows of the final draw: its mass at token x is max(0, p - q) after a
// rejection, or p for the bonus.
struct DrawRows {
  float Mt, Md;
  double inv_Zt, inv_Zd;
  int mode;
};

__device__ __forceinline__ DrawRows draw_rows(const AcceptArgs& a, int b) {
  DrawRows d;
  d.mode = a.dec[2 * b + 1];
  d.Mt = static_cast<float>(a.dstat[4 * b + 0]);
  d.inv_Zt = 1.0 / a.dstat[4 * b + 1];
  d.Md = static_cast<float>(a.dstat[4 * b + 2]);
  d.inv_Zd = 1.0 / a.dstat[4 * b + 3];
  return d;
}

__device__ __forceinline__ double draw_mass(const AcceptArgs& a, const DrawRows& d, float lt, float ldr) {
  const double p = static_cast<double>(exp_scaled(lt - d.Mt, a.c_hi, a.c_lo)) * d.inv_Zt;
  if (d.mode == kModeBonus) return p;
  const double q = static_cast<double>(exp_scaled(ldr - d.Md, a.c_hi, a.c_lo)) * d.inv_Zd;
  return fmax(0.0, p - q);
}

// Residual (or bonus) mass of the vocab chunks g0 .. g1 - 1 of the final draw.
// Each workgroup first takes the sequence's accept decision itself (the group
// holding chunk 0 publishes it).
template <typename T>
__global__ __launch_bounds__(kAccThreads) void accept_residual(AcceptArgs a) {
  extern __shared__ unsigned char smem_raw[];
  double* Zs = reinterpret_cast<double*>(smem_raw);
  float* Ms = reinterpret_cast<float*>(Zs + a.rows);
  __shared__ double wsum[kAccThreads / kWave][kMaxCpw];
  __shared__ int s_last[kAccThreads / kWave][kMaxCpw];
  __shared__ int s_acc;
  const int b = blockIdx.x;
  const int g0 = blockIdx.y * a.cpw;
  const int g1 = min(a.nch2, g0 + a.cpw);
  const int G1 = a.gamma + 1;
  const int acc = decide<T>(a, b, g0 == 0, Ms, Zs, &s_acc);
  DrawRows d;
  {
    const int dr = G1 + min(acc, a.gamma - 1);
    d.mode = acc < horizon_of(a, b) ? kModeResidual : kModeBonus;
    d.Mt = Ms[acc];
    d.inv_Zt = 1.0 / Zs[acc];
    d.Md = Ms[dr];
    d.inv_Zd = 1.0 / Zs[dr];
  }
  const T* pt = row_ptr<T>(a, b, acc);
  const T* pd = row_ptr<T>(a, b, G1 + min(acc, a.gamma - 1));
  const bool two = d.mode == kModeResidual;  // uniform: the draft row is read too
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // one chunk's sums, wave-reduced into the LDS slots of chunk c
  auto finish_chunk = [&](int c, double sc, int lc) {
    sc = wave_sum_f64(sc);
    lc = wave_max_i(lc);
    if (lane == 0) {
      wsum[wave][c - g0] = sc;
      s_last[wave][c - g0] = lc;
    }
  };
  if ((a.V % 8) == 0) {
    // Chunk c: tokens c kResChunk + k kAccThreads 8 + 8 t .. + 7 for round k < 2 of
    // thread t. The loads of chunk c + 1 (clamped into the row, so unconditional)
    // are issued before chunk c is summed.
    constexpr int kRounds = kResChunk / (kAccThreads * 8);
    const int last8 = a.V - 8;
    Raw8<T> rt[2][kRounds], rd[2][kRounds];
    auto issue = [&](int c, Raw8<T>(&t)[kRounds], Raw8<T>(&dr)[kRounds]) {
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int x = min(c * kResChunk + k * kAccThreads * 8 + static_cast<int>(threadIdx.x) * 8, last8);
        t[k] = ld8_raw<T>(pt, x);
        if (two) dr[k] = ld8_raw<T>(pd, x);
      }
    };
    auto sum_chunk = [&](int c, const Raw8<T>(&t)[kRounds], const Raw8<T>(&dr)[kRounds]) {
      const int x1 = min(a.V, (c + 1) * kResChunk);
      double sc = 0.0;
      int lc = -1;
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int x = c * kResChunk + k * kAccThreads * 8 + static_cast<int>(threadIdx.x) * 8;
        if (x < x1) {
          float vt[8], vd[8];
          cvt8<T>(t[k], vt);
          if (two) {
            cvt8<T>(dr[k], vd);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) vd[j] = 0.f;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double r = draw_mass(a, d, vt[j], vd[j]);
            sc += r;
            if (r > 0.0) lc = x + j;
          }
        }
      }
      finish_chunk(c, sc, lc);
    };
    issue(g0, rt[0], rd[0]);
    for (int c = g0; c < g1; c += 2) {
      issue(min(c + 1, g1 - 1), rt[1], rd[1]);
      sum_chunk(c, rt[0], rd[0]);
      if (c + 1 < g1) {
        issue(min(c + 2, g1 - 1), rt[0], rd[0]);
        sum_chunk(c + 1, rt[1], rd[1]);
      }
    }
  } else {
    for (int c = g0; c < g1; ++c) {
      const int x1 = min(a.V, (c + 1) * kResChunk);
      double sc = 0.0;
      int lc = -1;
      for (int x = c * kResChunk + threadIdx.x; x < x1; x += kAccThreads) {
        const double r = draw_mass(a, d, ld<T>(pt, x), two ? ld<T>(pd, x) : 0.f);
        sc += r;
        if (r > 0.0) lc = x;
      }
      finish_chunk(c, sc, lc);
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < g1 - g0) {
    const int j = threadIdx.x;
    double t = 0.0;
    int l = -1;
    for (int w = 0; w < kAccThreads / kWave; ++w) {
      t += wsum[w][j];
      l = max(l, s_last[w][j]);
    }
    a.rsum[static_cast<size_t>(b) * a.nch2 + g0 + j] = t;
    a.rlast[static_cast<size_t>(b) * a.nch2 + g0 + j] = l;
  }
}

// Inclusive workgroup scan (thread order) of doubles; returns the inclusive value.
__device__ __forceinline__ double block_scan_incl_f64(double x, double* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return before + x;
}

// Smallest index in [x0, x1) with positive mass whose running mass (from `base`)
// exceeds thr, scanning contiguous per-thread segments; -1 if none.
template <typename F>
__device__ int find_crossing(int x0, int x1, double base, double thr, F mass, double* wsum, int* s_tok) {
  const int n = x1 - x0;
  const int seg = (n + kAccThreads - 1) / kAccThreads;
  const int s0 = x0 + min(n, static_cast<int>(threadIdx.x) * seg);
  const int s1 = x0 + min(n, (static_cast<int>(threadIdx.x) + 1) * seg);
  double ss = 0.0;
  for (int x = s0; x < s1; ++x) ss += mass(x);
  const double incl = block_scan_incl_f64(ss, wsum);
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
  __shared__ double wsum[kAccThreads / kWave];
  __shared__ int s_tok;
  __shared__ int s_chunk;
  __shared__ double s_base, s_thr;
  const int b = blockIdx.x;
  const int G1 = a.gamma + 1;
  const int acc = a.dec[2 * b];
  const DrawRows d = draw_rows(a, b);
  const double u = static_cast<double>(a.us[b]);
  const double* rs = a.rsum + static_cast<size_t>(b) * a.nch2;
  if (threadIdx.x < kWave) {
    // one wave: total mass, then an inclusive prefix of the chunk masses in chunk
    // order, 64 chunks at a time, to find the chunk where u * R is crossed
    const int lane = threadIdx.x;
    double R = 0.0;
    for (int c0 = 0; c0 < a.nch2; c0 += kWave) R += wave_sum_f64(c0 + lane < a.nch2 ? rs[c0 + lane] : 0.0);
    const double thr = u * R;
    double run = 0.0;
    int cstar = -1;
    double base = 0.0;
    if (R > 0.0) {
      for (int c0 = 0; c0 < a.nch2 && cstar < 0; c0 += kWave) {
        const double own = (c0 + lane < a.nch2) ? rs[c0 + lane] : 0.0;
        double x = own;
        for (int off = 1; off < kWave; off <<= 1) {
          const double y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        const unsigned long long hit = __ballot(c0 + lane < a.nch2 && run + x > thr);
        if (hit) {
          const int f = __ffsll(static_cast<long long>(hit)) - 1;
          cstar = c0 + f;
          base = run + __shfl(x - own, f);
        }
        run += __shfl(x, kWave - 1);
      }
    }
    if (lane == 0) {
      s_chunk = (R > 0.0) ? cstar : -2;  // -2: no mass at all
      s_base = base;
      s_thr = thr;
    }
  }
  __syncthreads();
  const T* pt = row_ptr<T>(a, b, acc);
  const T* pd = row_ptr<T>(a, b, G1 + min(acc, a.gamma - 1));
  int token = -1;
  const int cstar = s_chunk;
  if (cstar >= 0 && (a.V % 8) == 0 && a.clen2 == kPickSeg * kAccThreads) {
    // each thread owns kPickSeg consecutive tokens of the chunk, loaded once
    const int x0 = cstar * a.clen2;
    const int s0 = x0 + threadIdx.x * kPickSeg;
    double r[kPickSeg];
    double ss = 0.0;
#pragma unroll
    for (int h = 0; h < kPickSeg; h += 8) {
      float vt[8], vd[8];
      const bool in = s0 + h < a.V;
      if (in) {
        ld8<T>(pt, s0 + h, vt);
        if (d.mode == kModeResidual) ld8<T>(pd, s0 + h, vd);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        r[h + j] = in ? draw_mass(a, d, vt[j], d.mode == kModeResidual ? vd[j] : 0.f) : 0.0;
        ss += r[h + j];
      }
    }
    const double incl = block_scan_incl_f64(ss, wsum);
    if (threadIdx.x == 0) s_tok = 0x7fffffff;
    __syncthreads();
    double cum = s_base + (incl - ss);
    if (s_base + incl > s_thr) {
      int hit = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kPickSeg; ++j) {
        cum += r[j];
        if (hit == 0x7fffffff && cum > s_thr && r[j] > 0.0) hit = s0 + j;
      }
      if (hit != 0x7fffffff) atomicMin(&s_tok, hit);
    }
    __syncthreads();
    token = s_tok == 0x7fffffff ? a.rlast[static_cast<size_t>(b) * a.nch2 + cstar] : s_tok;
  } else if (cstar >= 0) {
    const int x0 = cstar * a.clen2;
    const int x1 = min(a.V, x0 + a.clen2);
    auto mass = [&](int x) {
      return draw_mass(a, d, ld<T>(pt, x), d.mode == kModeResidual ? ld<T>(pd, x) : 0.f);
    };
    token = find_crossing(x0, x1, s_base, s_thr, mass, wsum, &s_tok);
    if (token < 0) token = a.rlast[static_cast<size_t>(b) * a.nch2 + cstar];
  } else if (cstar == -1) {
    // rounding left no crossing: the largest index with mass
    int l = -1;
    for (int c = 0; c < a.nch2; ++c) l = max(l, a.rlast[static_cast<size_t>(b) * a.nch2 + c]);
    token = l;
  } else {
    // the residual has no mass (possible only through rounding): draw from p of
    // the same row over the whole vocabulary
    DrawRows dp = d;
    dp.mode = kModeBonus;
    auto mass = [&](int x) { return draw_mass(a, dp, ld<T>(pt, x), 0.f); };
    double part = 0.0;
    for (int x = threadIdx.x; x < a.V; x += kAccThreads) part += mass(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    part = wave_sum_f64(part);
    if (lane == 0) wsum[wave] = part;
    __syncthreads();
    double W = 0.0;
    for (int w = 0; w < kAccThreads / kWave; ++w) W += wsum[w];
    __syncthreads();
    token = find_crossing(0, a.V, 0.0, u * W, mass, wsum, &s_tok);
    if (token < 0) token = a.V - 1;
  }
  if (threadIdx.x == 0) {
    a.out[static_cast<size_t>(b) * G1 + acc] = token;
    for (int j = acc + 1; j < G1; ++j) a.out[static_cast<size_t>(b) * G1 + j] = -1;
    if (a.ctx != nullptr) a.ctx[b] += acc + 1;
  }
}

template <typename T>
hipError_t launch_typed(const AcceptArgs& a, const AcceptPlan& pl, hipStream_t stream) {
  const dim3 g1(a.B * a.rows, a.nch);
  if (pl.unroll >= 16)
    hipLaunchKernelGGL((accept_rowstats<T, 16>), g1, dim3(kAccThreads), 0, stream, a);
  else if (pl.unroll >= 8)
    hipLaunchKernelGGL((accept_rowstats<T, 8>), g1, dim3(kAccThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((accept_rowstats<T, 4>), g1, dim3(kAccThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t smem = static_cast<size_t>(a.rows) * (8 + 4) + 16;
  hipLaunchKernelGGL(accept_residual<T>, dim3(a.B, (a.nch2 + a.cpw - 1) / a.cpw), dim3(kAccThreads), smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_pick<T>, dim3(a.B), dim3(kAccThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Workspace of the allocation-free entry point: one copy per GPU, for the life of
// the process. Host code never passes this name to a kernel (on the host it is
// only a stand-in for the symbol); it takes the device address that
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[kStaticAcceptScratchBytes];

hipError_t static_accept_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // no C++ exception leaves the library: a failing lock becomes an error status
  try {
    std::lock_guard<std::mutex> lock(mu);
    if (per_device[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      per_device[dev] = p;
    }
    *ptr = per_device[dev];
  } catch (...) {
    return hipErrorUnknown;
  }
  return hipSuccess;
}

AcceptPlan plan_accept(int num_seqs, int gamma, int vocab) {
  AcceptPlan pl{};
  pl.num_seqs = num_seqs;
  pl.gamma = gamma;
  pl.vocab = vocab;
  pl.rows = 2 * gamma + 1;
  pl.clen = 65536;  // measured: fewer, longer row-statistics workgroups stream faster
  if (const char* e = getenv("S3R_ACCEPT_CHUNK")) {
    const int v = atoi(e);
    if (v >= 2048 && v % 2048 == 0) pl.clen = v;
  }
  pl.nch = (vocab + pl.clen - 1) / pl.clen;
  pl.unroll = 8;  // measured on MI355X: 8 beats 4 (and 16) once the loads are unconditional
  if (const char* e = getenv("S3R_ACCEPT_UNROLL")) {
    const int v = atoi(e);
    if (v == 4 || v == 8 || v == 16) pl.unroll = v;
  }
  pl.clen2 = kResChunk;
  pl.nch2 = (vocab + pl.clen2 - 1) / pl.clen2;
  // Residual chunks per workgroup: enough that the residual workgroups fit the
  // chip about once (eight per CU), so the decision each of them replays costs one
  // round of latency rather than several.
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const long long groups = static_cast<long long>(num_seqs) * pl.nch2;
  const long long resident = 8LL * cus;
  pl.cpw = static_cast<int>(std::min<long long>(kMaxCpw, std::max<long long>(1, (groups + resident - 1) / resident)));
  if (const char* e = getenv("S3R_ACCEPT_CPW")) {
    const int v = atoi(e);
    if (v >= 1 && v <= kMaxCpw) pl.cpw = v;
  }
  const size_t B = num_seqs;
  size_t off = 0;
  pl.off_st_m = off;
  off = align_up(off + B * pl.rows * pl.nch * 4, 256);
  pl.off_st_s = off;
  off = align_up(off + B * pl.rows * pl.nch * 8, 256);
  pl.off_dstat = off;
  off = align_up(off + B * 4 * 8, 256);
  pl.off_dec = off;
  off = align_up(off + B * 2 * 4, 256);
  pl.off_rsum = off;
  off = align_up(off + B * pl.nch2 * 8, 256);
  pl.off_rlast = off;
  off = align_up(off + B * pl.nch2 * 4, 256);
  pl.bytes = off;
  return pl;
}

hipError_t launch_accept(const AcceptPlan& pl, int bf16, const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                         float temperature, int32_t* num_accepted, int32_t* out_tokens, int32_t* ctx_lens,
                         void* workspace, hipStream_t stream, const int32_t* horizons) {
  char* ws = static_cast<char*>(workspace);
  AcceptArgs a{};
  a.horizons = horizons;
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
  a.dstat = reinterpret_cast<double*>(ws + pl.off_dstat);
  a.dec = reinterpret_cast<int32_t*>(ws + pl.off_dec);
  a.rsum = reinterpret_cast<double*>(ws + pl.off_rsum);
  a.rlast = reinterpret_cast<int32_t*>(ws + pl.off_rlast);
  a.B = pl.num_seqs;
  a.gamma = pl.gamma;
  a.V = pl.vocab;
  a.rows = pl.rows;
  a.nch = pl.nch;
  a.clen = pl.clen;
  a.nch2 = pl.nch2;
  a.clen2 = pl.clen2;
  a.cpw = pl.cpw;
  a.c_d = 1.4426950408889634074 / static_cast<double>(temperature);
  // c_hi: the largest float not above c_d; c_lo: the rest, at least FLT_MIN (so
  // -inf logits stay -inf in exp_scaled; FLT_MIN changes no product of a logit)
  a.c_hi = static_cast<float>(a.c_d);
  if (static_cast<double>(a.c_hi) > a.c_d) a.c_hi = nextafterf(a.c_hi, 0.f);
  a.c_lo = fmaxf(static_cast<float>(a.c_d - static_cast<double>(a.c_hi)), FLT_MIN);
  a.inv_t = 1.0 / static_cast<double>(temperature);
  return bf16 ? launch_typed<bf16_t>(a, pl, stream) : launch_typed<float>(a, pl, stream);
}

}  // namespace s3r
