// Dense verify attention for the gamma + 1 block queries over the whole paged KV
// history, with per-page softmax mass for the next draft's page selection.
//
// What is computed: for sequence b, block query i (position L_b + i) and query
// head h, softmax over every key t <= L_b + i of scale * q.k, applied to V
// (abstract; wispaper.ai, "Dense verification still pays the full KV-cache bill").
// page_scores[b][p] sums those softmax weights over i, h and the tokens of page p
// (rit.work, "Как разреженный черновик сохраняет ответы плотной модели").
//
// Mapping on gfx950. One work unit is (sequence, kv head): its M = G1 * g query
// rows (all block positions of all query heads sharing the kv head) ride as the
// N columns of MFMA tiles, so every K/V page is read from HBM exactly once for the
// whole block. Per 16-token page and 16-column tile:
//   S^T = K Q^T    A = K page rows (lane: key l%16, 8 dims), B = Q^T from registers
//                  bf16: D/32 x mfma_f32_16x16x32_bf16;  fp32: D/4 x mfma_f32_16x16x4f32
//   O^T += V^T P^T A = V^T rows (the cache stores V page-transposed, so a lane's
//                  four keys of one dim are contiguous), B = P^T, which is exactly
//                  the accumulator layout of S^T (lane: 4 keys of column l%16)
//                  bf16: D/16 x mfma_f32_16x16x16bf16_1k;  fp32: D/4 x mfma_f32_16x16x4f32
// Both operands stream straight from HBM into VGPRs with 16-byte (K) and 8-byte
// (V) loads; no LDS staging is needed because no operand needs a transpose. A
// work unit's pages are cut into splits of about `pps` pages, one workgroup of
// four waves per split, waves interleaved page by page; the four waves merge in
// LDS and write one (m, l, o) partial per split. verify_combine merges splits in
// a fixed order (deterministic) and finalises the page scores, which the main
// kernel emits as a per-page log-sum-exp so no second pass over K is needed.
#include <stdlib.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kVerifyWaves = 4;
constexpr int kVerifyThreads = kVerifyWaves * kWave;

struct VerifyArgs {
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* lens;
  const void* q;
  void* out;
  float* scores;
  float* part_o;   // [B*hkv][max_splits][M][D]
  float* part_ml;  // [B*hkv][max_splits][M][2]  (max in log2 units, sum)
  float* lse;      // [B][maxp][hkv][M]           (per-page log2-sum-exp)
  int num_blocks, hkv, hq, g, maxp, G1, M, max_splits, pps;
  float scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int maxp, int G1) { return max(0, min(L, maxp * kPage - G1)); }

template <typename T>
struct Frag;

// bf16: K fragment = 8 dims (16 B) per 32-dim chunk, V fragment = 4 keys (8 B).
template <>
struct Frag<bf16_t> {
  using K = uint4;
  using V = uint2;
  template <int D>
  static constexpr int kChunks() { return D / 32; }
};
// fp32: K fragment = 4 dims (16 B) per 16-dim chunk, V fragment = 4 keys (16 B).
template <>
struct Frag<float> {
  using K = float4;
  using V = float4;
  template <int D>
  static constexpr int kChunks() { return D / 16; }
};

template <typename T, int D, int NT>
__global__ __launch_bounds__(kVerifyThreads) void verify_main(VerifyArgs a) {
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  using KF = typename Frag<T>::K;
  using VF = typename Frag<T>::V;
  constexpr int KC = Frag<T>::template kChunks<D>();
  constexpr int DT = D / 16;  // 16-dim output tiles

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int unit = blockIdx.x / a.max_splits;
  const int split = blockIdx.x % a.max_splits;
  const int b = unit / a.hkv;
  const int kvh = unit % a.hkv;

  const int L = clamp_len(a.lens[b], a.maxp, a.G1);
  const int n_pages = (L + a.G1 + kPage - 1) / kPage;
  const int n_splits = (n_pages + a.pps - 1) / a.pps;
  if (split >= n_splits) return;  // uniform over the workgroup
  const int p_begin = static_cast<int>(static_cast<long long>(split) * n_pages / n_splits);
  const int p_end = static_cast<int>(static_cast<long long>(split + 1) * n_pages / n_splits);

  const T* __restrict__ kc = static_cast<const T*>(a.k);
  const T* __restrict__ vc = static_cast<const T*>(a.v);
  const int32_t* __restrict__ trow = a.table + static_cast<size_t>(b) * a.maxp;

  // Query fragments (B operand of S^T = K Q^T) and the causal limit per column.
  KF qf[NT][KC];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + r16;
    if (c < a.M) {
      const int i = c / a.g;
      const int hh = c - i * a.g;
      lim[nt] = L + i;
      const T* qp = static_cast<const T*>(a.q) +
                    ((static_cast<size_t>(b) * a.G1 + i) * a.hq + kvh * a.g + hh) * D;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        if constexpr (kBf16)
          qf[nt][kk] = *reinterpret_cast<const uint4*>(qp + kk * 32 + grp * 8);
        else
          qf[nt][kk] = *reinterpret_cast<const float4*>(qp + kk * 16 + grp * 4);
      }
    } else {
      lim[nt] = -1;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qf[nt][kk] = KF{};
    }
  }

  float m_run[NT], l_run[NT];
  f32x4_t oacc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) oacc[nt][dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto page_base = [&](int p) -> size_t {
    int blk = trow[p];
    blk = min(max(blk, 0), a.num_blocks - 1);
    return (static_cast<size_t>(blk) * a.hkv + kvh) * (kPage * D);
  };
  auto load_page = [&](size_t base, KF (&kf)[KC], VF (&vf)[DT]) {
    const T* kp = kc + base + r16 * D;
    const T* vp = vc + base + r16 * kPage + grp * 4;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      if constexpr (kBf16)
        kf[kk] = *reinterpret_cast<const uint4*>(kp + kk * 32 + grp * 8);
      else
        kf[kk] = *reinterpret_cast<const float4*>(kp + kk * 16 + grp * 4);
    }
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) vf[dd] = *reinterpret_cast<const VF*>(vp + dd * 16 * kPage);
  };

  KF kf_cur[KC], kf_nxt[KC];
  VF vf_cur[DT], vf_nxt[DT];
  int p = p_begin + wave;
  if (p < p_end) load_page(page_base(p), kf_nxt, vf_nxt);

  for (; p < p_end; p += kVerifyWaves) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) kf_cur[kk] = kf_nxt[kk];
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) vf_cur[dd] = vf_nxt[dd];
    if (p + kVerifyWaves < p_end) load_page(page_base(p + kVerifyWaves), kf_nxt, vf_nxt);

    const int t0 = p * kPage + grp * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        if constexpr (kBf16) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf_cur[kk]),
                                                      __builtin_bit_cast(bf16x8_t, qf[nt][kk]), s, 0, 0, 0);
        } else {
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf_cur[kk].x, qf[nt][kk].x, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf_cur[kk].y, qf[nt][kk].y, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf_cur[kk].z, qf[nt][kk].z, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf_cur[kk].w, qf[nt][kk].w, s, 0, 0, 0);
        }
      }
      // lane holds S^T[key t0 + i][column nt*16 + r16], i = 0..3
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (t0 + i <= lim[nt]) ? s[i] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = cross_row_max(mx);
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[nt] - m_use);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sv[i] - m_use);
      const float psum = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      l_run[nt] = l_run[nt] * alpha + psum;
      m_run[nt] = m_new;
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) oacc[nt][dd] *= alpha;

      if (a.lse != nullptr) {
        const float ps = cross_row_sum(psum);
        const int c = nt * 16 + r16;
        if (grp == 0 && c < a.M) {
          const float v = (ps > 0.f) ? m_use + fast_log2(ps) : -INFINITY;
          a.lse[((static_cast<size_t>(b) * a.maxp + p) * a.hkv + kvh) * a.M + c] = v;
        }
      }

      if constexpr (kBf16) {
        const uint32_t lo = pack_bf16x2(pr[0], pr[1]);
        const uint32_t hi = pack_bf16x2(pr[2], pr[3]);
        const i16x4_t pb = __builtin_bit_cast(i16x4_t, make_uint2(lo, hi));
#pragma unroll
        for (int dd = 0; dd < DT; ++dd)
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, vf_cur[dd]), pb,
                                                                   oacc[nt][dd], 0, 0, 0);
      } else {
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) {
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf_cur[dd].x, pr[0], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf_cur[dd].y, pr[1], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf_cur[dd].z, pr[2], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf_cur[dd].w, pr[3], oacc[nt][dd], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_run[nt] = cross_row_sum(l_run[nt]);

  // Merge the four waves of the split in LDS; wave 0 writes the partial.
  __shared__ f32x4_t red_o[kVerifyWaves - 1][NT][DT][kWave];
  __shared__ float red_m[kVerifyWaves - 1][NT][16];
  __shared__ float red_l[kVerifyWaves - 1][NT][16];
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) red_o[wave - 1][nt][dd][lane] = oacc[nt][dd];
      if (grp == 0) {
        red_m[wave - 1][nt][r16] = m_run[nt];
        red_l[wave - 1][nt][r16] = l_run[nt];
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;

  const size_t sbase = static_cast<size_t>(unit) * a.max_splits + split;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + r16;
    float mw[kVerifyWaves], lw[kVerifyWaves], wt[kVerifyWaves];
    mw[0] = m_run[nt];
    lw[0] = l_run[nt];
#pragma unroll
    for (int w = 1; w < kVerifyWaves; ++w) {
      mw[w] = red_m[w - 1][nt][r16];
      lw[w] = red_l[w - 1][nt][r16];
    }
    float mstar = mw[0];
#pragma unroll
    for (int w = 1; w < kVerifyWaves; ++w) mstar = fmaxf(mstar, mw[w]);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) {
      wt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - mstar);
      lsum += wt[w] * lw[w];
    }
    if (c < a.M) {
      float* po = a.part_o + (sbase * a.M + c) * D + grp * 4;
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) {
        f32x4_t o = oacc[nt][dd] * wt[0];
#pragma unroll
        for (int w = 1; w < kVerifyWaves; ++w) o += red_o[w - 1][nt][dd][lane] * wt[w];
        *reinterpret_cast<f32x4_t*>(po + dd * 16) = o;
      }
      if (grp == 0) {
        a.part_ml[(sbase * a.M + c) * 2 + 0] = mstar;
        a.part_ml[(sbase * a.M + c) * 2 + 1] = lsum;
      }
    }
  }
}

// One workgroup per (sequence, kv head): merges the splits of its unit into the
// output rows, and finalises page scores for a 1/hkv slice of the sequence's
// pages (which needs the merged row statistics of every kv head of the sequence,
// recomputed here from the split partials).
template <typename T, int D>
__global__ __launch_bounds__(256) void verify_combine(VerifyArgs a) {
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  extern __shared__ float smem[];
  const int unit = blockIdx.x;
  const int b = unit / a.hkv;
  const int kvh = unit % a.hkv;
  const int L = clamp_len(a.lens[b], a.maxp, a.G1);
  const int n_pages = (L + a.G1 + kPage - 1) / kPage;
  const int n_splits = (n_pages + a.pps - 1) / a.pps;
  const int M = a.M;
  float* lse2 = smem;                 // [hkv][M] row log2-sum-exp
  float* wts = smem + a.hkv * M;      // [max_splits][M] split weights of this unit

  for (int idx = threadIdx.x; idx < a.hkv * M; idx += blockDim.x) {
    const int kv2 = idx / M;
    const int c = idx - kv2 * M;
    const float* ml = a.part_ml + (static_cast<size_t>(b * a.hkv + kv2) * a.max_splits * M + c) * 2;
    float mx = -INFINITY;
    for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ml[static_cast<size_t>(s) * M * 2]);
    float l = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float ms = ml[static_cast<size_t>(s) * M * 2];
      if (ms != -INFINITY) l += ml[static_cast<size_t>(s) * M * 2 + 1] * fast_exp2(ms - mx);
    }
    lse2[idx] = (l > 0.f) ? mx + log2f(l) : -INFINITY;
    if (kv2 == kvh) {
      for (int s = 0; s < n_splits; ++s) {
        const float ms = ml[static_cast<size_t>(s) * M * 2];
        wts[s * M + c] = (ms != -INFINITY && l > 0.f) ? fast_exp2(ms - mx) / l : 0.f;
      }
    }
  }
  __syncthreads();

  const float* po = a.part_o + static_cast<size_t>(unit) * a.max_splits * M * D;
  for (int idx = threadIdx.x; idx < M * D; idx += blockDim.x) {
    const int c = idx / D;
    const int d = idx - c * D;
    float o = 0.f;
    for (int s = 0; s < n_splits; ++s) o += wts[s * M + c] * po[(static_cast<size_t>(s) * M + c) * D + d];
    const int i = c / a.g;
    const int hh = c - i * a.g;
    const size_t oi = ((static_cast<size_t>(b) * a.G1 + i) * a.hq + kvh * a.g + hh) * D + d;
    if constexpr (kBf16)
      static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(o);
    else
      static_cast<float*>(a.out)[oi] = o;
  }

  if (a.scores != nullptr) {
    const int chunk = (a.maxp + a.hkv - 1) / a.hkv;
    const int p0 = kvh * chunk;
    const int p1 = min(a.maxp, p0 + chunk);
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
      float s = 0.f;
      if (p < n_pages) {
        const float* lp = a.lse + (static_cast<size_t>(b) * a.maxp + p) * a.hkv * M;
        for (int j = 0; j < a.hkv * M; ++j) {
          const float x = lp[j];
          if (x != -INFINITY) s += fast_exp2(x - lse2[j]);
        }
      }
      a.scores[static_cast<size_t>(b) * a.maxp + p] = s;
    }
  }
}

template <typename T, int D, int NT>
hipError_t launch_typed(const VerifyArgs& args, int num_units, hipStream_t stream) {
  const size_t smem = (static_cast<size_t>(args.hkv) * args.M + static_cast<size_t>(args.max_splits) * args.M) * 4;
  hipLaunchKernelGGL((verify_main<T, D, NT>), dim3(num_units * args.max_splits), dim3(kVerifyThreads), 0, stream,
                     args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_combine<T, D>), dim3(num_units), dim3(256), smem, stream, args);
  return hipGetLastError();
}

}  // namespace

VerifyPlan plan_verify(const KvView& kv, int num_seqs, int hq, int G1) {
  VerifyPlan pl{};
  pl.num_seqs = num_seqs;
  pl.hq = hq;
  pl.G1 = G1;
  pl.g = hq / kv.hkv;
  pl.M = G1 * pl.g;
  int pps = 128;
  if (const char* e = getenv("S3R_VERIFY_PAGES_PER_SPLIT")) {
    const int v = atoi(e);
    if (v >= 1) pps = v;
  }
  pl.pps = pps;
  pl.max_splits = (kv.maxp + pps - 1) / pps;
  const size_t units = static_cast<size_t>(num_seqs) * kv.hkv;
  size_t off = 0;
  pl.off_part_o = off;
  off = align_up(off + units * pl.max_splits * pl.M * kv.head_dim * 4, 256);
  pl.off_part_ml = off;
  off = align_up(off + units * pl.max_splits * pl.M * 2 * 4, 256);
  pl.off_lse = off;
  off = align_up(off + static_cast<size_t>(num_seqs) * kv.maxp * kv.hkv * pl.M * 4, 256);
  pl.bytes = off;
  return pl;
}

hipError_t launch_verify(const KvView& kv, const VerifyPlan& pl, const void* q, float scale, void* out,
                         float* scores, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  VerifyArgs a{};
  a.k = kv.k;
  a.v = kv.v;
  a.table = kv.table;
  a.lens = kv.lens;
  a.q = q;
  a.out = out;
  a.scores = scores;
  a.part_o = reinterpret_cast<float*>(ws + pl.off_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + pl.off_part_ml);
  a.lse = scores ? reinterpret_cast<float*>(ws + pl.off_lse) : nullptr;
  a.num_blocks = kv.num_blocks;
  a.hkv = kv.hkv;
  a.hq = pl.hq;
  a.g = pl.g;
  a.maxp = kv.maxp;
  a.G1 = pl.G1;
  a.M = pl.M;
  a.max_splits = pl.max_splits;
  a.pps = pl.pps;
  a.scale_log2 = scale * kLog2e;
  const int units = pl.num_seqs * kv.hkv;
  const bool two = pl.M > 16;
  if (kv.bf16) {
    if (kv.head_dim == 128)
      return two ? launch_typed<bf16_t, 128, 2>(a, units, stream) : launch_typed<bf16_t, 128, 1>(a, units, stream);
    return two ? launch_typed<bf16_t, 64, 2>(a, units, stream) : launch_typed<bf16_t, 64, 1>(a, units, stream);
  }
  if (kv.head_dim == 128)
    return two ? launch_typed<float, 128, 2>(a, units, stream) : launch_typed<float, 128, 1>(a, units, stream);
  return two ? launch_typed<float, 64, 2>(a, units, stream) : launch_typed<float, 64, 1>(a, units, stream);
}

}  // namespace s3r
