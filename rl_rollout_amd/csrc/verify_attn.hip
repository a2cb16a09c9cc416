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
// Both operands stream from HBM straight into VGPRs with non-temporal 16-byte (K)
// and 8-byte (V) loads through a register ring (DEPTH pages in flight per wave);
// no operand needs a transpose, so nothing is staged in LDS.
//
// A unit's pages are cut into balanced splits of at most `pps` pages, one
// workgroup of four waves per split, waves interleaved page by page; the four
// waves merge in LDS and write one (m, l, o) partial plus a log-sum-exp per page
// and row (an aligned 1 KB row per split and column, so the write-out is whole
// cache lines). verify_combine then merges the splits of each unit in split order into
// the output rows, and sums each page's softmax mass over the sequence's rows into
// page_scores; every thread there issues all of its loads at once, so the second
// kernel costs a few memory latencies. Every reduction has a fixed order, so the
// results are deterministic.
#include <stdlib.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

constexpr int kVerifyWaves = 4;
constexpr int kVerifyThreads = kVerifyWaves * kWave;
constexpr int kMaxPagesPerSplit = 256;  // a wave then holds at most 64 pages: one block id per lane
constexpr int kLseRow = kMaxPagesPerSplit + 4;  // LDS row stride of the split staging (2-way bank spread)
constexpr int kUnitBlkRegs = 8;         // whole-unit mode: block ids held in 8 lane registers, 2048 pages
constexpr size_t kUnitLdsPerWorkgroup = 80 * 1024;  // two whole-unit workgroups per CU (160 KB of LDS)
constexpr float kRescaleSlack = 8.f;    // log2 units: weights against a stale max stay below 256
constexpr int kChunk = 512;             // global staging: pages per chunk staged in LDS
constexpr int kChunkStride = kChunk + 4;  // LDS row stride: 16-byte rows, 16 columns in distinct banks

struct VerifyArgs {
  void* k;
  void* v;
  const int32_t* table;
  const int32_t* lens;
  const void* q;
  void* out;
  float* scores;
  const void* k_new;  // optional block rows [B][G1][hkv][D] written into the cache before attending
  const void* v_new;
  float* part_o;      // [B*hkv][max_splits][M][D]
  float* part_ml;     // [B*hkv][max_splits][M][2]  (max in log2 units, sum)
  float* lse;         // [B][max_splits][hkv][M][256] per-page log2-sum-exp, one 1 KB row per split and column
  float* unit_scores; // whole-unit mode: [B][hkv][maxp] page mass of one kv head's rows
  float* gstage;      // whole-unit mode, global staging: [units][gchunks][kChunk][MP] per-page log-sum-exps (MP = M up to 4)
  float* head_scores; // split mode, per-kv-head scores requested: [B][hkv][maxp] output
  const int32_t* horizons;  // optional [B]: sequence b's block is its first horizons[b] + 1 queries
  int head_out;       // whole-unit mode: unit_scores is the caller's per-kv-head output (zero-fill the tail)
  int num_blocks, hkv, hq, g, maxp, G1, M, max_splits, pps;
  int lse_stride;     // whole-unit mode: LDS row stride of the per-page log-sum-exp staging (odd)
  int gchunks;        // whole-unit mode, global staging: chunks of kChunk pages per unit (ceil(maxp / kChunk))
  int num_seqs;
  int lpt;            // whole-unit mode: take units longest first
  int num_seqs_x_chunks;  // combine grid: page-score groups come first
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

// Longest-first order for whole-unit mode when the units outnumber the
// workgroups the chip runs at once: the dispatcher starts workgroups in index
// order, so workgroup i takes the sequence of rank i / hkv in (pages descending,
// index ascending). Every workgroup ranks the num_seqs lengths itself from LDS
// (num_seqs^2 / 256 compares per thread; the host enables this for at most
// kLptMaxSeqs sequences), which costs less than a separate ordering launch.
constexpr int kLptMaxSeqs = 1024;

__device__ int lpt_unit(const VerifyArgs& a, int wg) {
  __shared__ int s_pages[kLptMaxSeqs];
  __shared__ int s_seq;
  const int B = a.num_seqs;
  for (int j = threadIdx.x; j < B; j += kVerifyThreads)
    s_pages[j] = (clamp_len(a.lens[j], a.maxp, a.G1) + a.G1 + kPage - 1) / kPage;
  __syncthreads();
  const int want = wg / a.hkv;
  for (int j = threadIdx.x; j < B; j += kVerifyThreads) {
    const int nj = s_pages[j];
    int rank = 0;
    for (int i = 0; i < B; ++i) {
      const int ni = s_pages[i];
      rank += (ni > nj) || (ni == nj && i < j);
    }
    if (rank == want) s_seq = j;
  }
  __syncthreads();
  return s_seq * a.hkv + wg % a.hkv;
}

// kUnit = false: one workgroup per split of a (sequence, kv head) unit; partials
// and per-page log-sum-exp rows go to the workspace for verify_combine.
// kUnit = true: one workgroup per whole unit; it writes the final output rows and
// the unit's per-page mass directly. The per-page log-sum-exps stay in LDS
// (kGStage = false, one column tile), or (kGStage = true, when they do not fit:
// two column tiles or long histories) are staged in LDS a chunk of kChunk pages at
// a time and written to the workspace in one burst when the chunk is complete
// (stores interleaved with the page stream cost far more than their bytes). The
// chunks are aligned so that the last one ends at the unit's last page (up to
// three pages short); that chunk never leaves LDS. After the page loop, once the
// column normalisers are known, the workgroup reads the written chunks back and
// the last one from LDS.
template <typename T, int D, int NT, int DEPTH, bool kUnit, bool kGStage = false>
__global__ __launch_bounds__(kVerifyThreads) __attribute__((amdgpu_waves_per_eu(2))) void verify_main(VerifyArgs a) {
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  using KF = typename Frag<T>::K;
  using VF = typename Frag<T>::V;
  constexpr int KC = Frag<T>::template kChunks<D>();
  constexpr int DT = D / 16;       // 16-dim output tiles
  constexpr int NS = DEPTH + 1;    // register ring slots: DEPTH pages in flight while one is consumed
  constexpr int R = kUnit ? kUnitBlkRegs : 1;  // lane registers of block ids per wave
  static_assert(!kUnit || NT == 1 || kGStage, "whole-unit mode stages two column tiles in the workspace");
  static_assert(!kGStage || kUnit, "global staging is a whole-unit mode");

  const int lane = threadIdx.x & (kWave - 1);
  // wave index made visibly uniform so the page loop runs on scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const int split = kUnit ? 0 : static_cast<int>(blockIdx.x) % a.max_splits;
  int unit = kUnit ? static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x) / a.max_splits;
  if constexpr (kUnit) {
    if (a.lpt) unit = lpt_unit(a, unit);
  }
  const int b = unit / a.hkv;
  const int kvh = unit % a.hkv;

  // Query fragments (B operand of S^T = K Q^T); column c = nt * 16 + l % 16 is
  // block query c / g of query head kvh * g + c % g. Issued before the length
  // load so both round trips overlap.
  // With two column tiles the fragments are parked in LDS after this load and
  // re-read per page, which frees 32 VGPRs and keeps two waves per SIMD.
  constexpr bool kQInLds = NT > 1;
  KF qf[NT][KC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + r16;
    if (c < a.M) {
      const int i = c / a.g;
      const int hh = c - i * a.g;
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
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qf[nt][kk] = KF{};
    }
  }

  const int L = clamp_len(a.lens[b], a.maxp, a.G1);
  const int n_pages = (L + a.G1 + kPage - 1) / kPage;
  // LDS pool: the parked query fragments and the split staging live during the
  // page loop; the wave-merge buffer reuses the same bytes after it. Whole-unit
  // mode merges in the dynamic region instead, after the page scores have read
  // the per-page staging there, so its static LDS stays small and the staging of
  // more rows or pages fits two workgroups per CU.
  constexpr size_t kQBytes = kQInLds ? sizeof(KF) * NT * KC * kWave : 0;
  constexpr size_t kStageBytes = kUnit ? 0 : sizeof(float) * NT * 16 * kLseRow;
  constexpr size_t kRedBytes = sizeof(f32x4_t) * (kVerifyWaves - 1) * NT * DT * kWave;
  constexpr size_t kLoopBytes = kQBytes + kStageBytes;
  constexpr size_t kPoolBytes = kUnit ? (kLoopBytes > 16 ? kLoopBytes : 16)
                                      : (kLoopBytes > kRedBytes ? kLoopBytes : kRedBytes);
  __shared__ __attribute__((aligned(16))) unsigned char pool[kPoolBytes];
  // whole-unit mode: [M][lse_stride] per-page staging, then the wave-merge buffer
  extern __shared__ __attribute__((aligned(16))) float lse_dyn[];
  auto q_lds = reinterpret_cast<KF (*)[KC][kWave]>(pool);                  // [NT][KC][64]
  auto lse_stage = reinterpret_cast<float (*)[kLseRow]>(pool + kQBytes);    // [NT * 16][kLseRow]
  auto red_o = reinterpret_cast<f32x4_t (*)[NT][DT][kWave]>(kUnit ? reinterpret_cast<unsigned char*>(lse_dyn)
                                                                  : pool);  // [3][NT][DT][64]
  int p_begin = 0, p_end = n_pages;
  if constexpr (!kUnit) {
    const int n_splits = (n_pages + a.pps - 1) / a.pps;
    if (split >= n_splits) return;  // uniform over the workgroup
    p_begin = static_cast<int>(static_cast<long long>(split) * n_pages / n_splits);
    p_end = static_cast<int>(static_cast<long long>(split + 1) * n_pages / n_splits);
  }

  // This wave's pages are first + 4 * it, it < n_it (<= 64 R). Lane l of
  // register r holds the physical block of iteration l + 64 r; the loop reads it
  // with readlane.
  const int first = p_begin + wave;
  const int n_it = first < p_end ? (p_end - first + kVerifyWaves - 1) / kVerifyWaves : 0;
  int my_blk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    my_blk[r] = 0;
    const int idx = lane + kWave * r;
    if (idx < n_it) {
      const int blk = a.table[static_cast<size_t>(b) * a.maxp + first + kVerifyWaves * idx];
      my_blk[r] = min(max(blk, 0), a.num_blocks - 1);
    }
  }
  // Every register is read with readlane and the choice is made on the scalar
  // results, so the compiler cannot turn it into an indexed (scratch) access.
  auto block_of = [&](int it) {
    const int ln = it & (kWave - 1);
    int blk = __builtin_amdgcn_readlane(my_blk[0], ln);
#pragma unroll
    for (int r = 1; r < R; ++r) {
      const int x = __builtin_amdgcn_readlane(my_blk[r], ln);
      blk = (it >= kWave * r) ? x : blk;
    }
    return blk;
  };
  const bool want_lse = kUnit ? (a.unit_scores != nullptr) : (a.lse != nullptr);
  if constexpr (kQInLds) {
    if (wave == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) q_lds[nt][kk][lane] = qf[nt][kk];
    }
    __syncthreads();
  }

  // causal limit per column: key t is visible to column c (block query c / g) iff t <= L + c / g;
  // columns past the tile or past the sequence's block see no key (zero output, no page mass)
  const int G1b = a.horizons != nullptr ? min(max(a.horizons[b], 0), a.G1 - 1) + 1 : a.G1;
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + r16;
    lim[nt] = (c < a.M && c / a.g < G1b) ? L + c / a.g : -1;
  }

  // Fused append: the block's rows at L .. L + G1 - 1 of this kv head, each
  // written by the workgroup whose pages hold it (the only one that reads it).
  // Each page is written by the wave that later reads it (wave (page - p_begin) %
  // 4), before its own page loop: no barrier, and the other waves start
  // streaming at once; one wave's accesses to one address stay in program order.
  if (a.k_new != nullptr) {
    const size_t src = (static_cast<size_t>(b) * a.G1 * a.hkv + kvh) * D;  // row 0 of this kv head
    for (int page = max(L >> 4, p_begin); page < p_end && page * kPage < L + a.G1; ++page) {
      if ((page - p_begin) % kVerifyWaves != wave) continue;
      const int blk = a.table[static_cast<size_t>(b) * a.maxp + page];
      if (blk < 0 || blk >= a.num_blocks) continue;
      put_rows_in_page<T, D>(a.k, a.v, a.hkv, kvh, blk, page, L, a.G1, static_cast<const T*>(a.k_new) + src,
                             static_cast<const T*>(a.v_new) + src, static_cast<size_t>(a.hkv) * D, lane, kWave);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    asm volatile("" ::: "memory");
  }

  const T* __restrict__ kc = static_cast<const T*>(a.k);
  const T* __restrict__ vc = static_cast<const T*>(a.v);

  // Per-page log2-sum-exp of each column, staged in LDS (so the loop itself
  // issues no global stores, which would make the compiler's load waits
  // conservative): split mode writes it out after the loop as one aligned block
  // per split; whole-unit mode keeps it for the page scores at the end.
  // Global staging: page q of the unit has the virtual index q + goff, chunk
  // (q + goff) / kChunk and slot (q + goff) % kChunk. goff (a multiple of the wave
  // count, so chunk boundaries fall between loop iterations) shifts the chunks so
  // that the last one, kfin, is full up to three pages and stays in LDS; chunk 0
  // holds the first kChunk - goff pages.
  const int goff = ((kChunk - n_pages % kChunk) % kChunk) & ~(kVerifyWaves - 1);
  const int kfin = (n_pages - 1 + goff) / kChunk;
  auto lse_slot = [&](int c, int q) -> float& {
    if constexpr (kGStage)
      return lse_dyn[c * kChunkStride + ((q + goff) & (kChunk - 1))];
    else if constexpr (kUnit)
      return lse_dyn[c * a.lse_stride + q];
    else
      return lse_stage[c][q];
  };
  // Chunk k < kfin (its slots from goff on for k = 0, all of them after) leaves LDS
  // as one burst of whole 16-byte vectors, page-major ([slot][MP], MP = M rounded
  // up to 4, the rows past M zero) so that the read-back takes a page's rows in a
  // few 16-byte loads; called by the whole workgroup between two barriers.
  const int MP = (a.M + 3) & ~3;
  auto flush_chunk = [&](int k) {
    const int s0 = k == 0 ? goff : 0;
    const int q4 = MP >> 2;
    float* dst = a.gstage + (static_cast<size_t>(unit) * a.gchunks + k) * kChunk * MP;
    for (int i = s0 * q4 + threadIdx.x; i < kChunk * q4; i += kVerifyThreads) {
      const int j = i / q4;
      const int c = (i - j * q4) * 4;
      float4 v;
      v.x = lse_dyn[c * kChunkStride + j];
      v.y = c + 1 < a.M ? lse_dyn[(c + 1) * kChunkStride + j] : 0.f;
      v.z = c + 2 < a.M ? lse_dyn[(c + 2) * kChunkStride + j] : 0.f;
      v.w = c + 3 < a.M ? lse_dyn[(c + 3) * kChunkStride + j] : 0.f;
      st_stream16f(dst + static_cast<size_t>(j) * MP + c, v);
    }
  };
  // Global staging keeps a second chunk on chip: chunk kfin - 1 goes to registers
  // instead of LDS (and is never written out). A wave takes 128 iterations of it;
  // register t of tile nt holds its iterations 4t .. 4t + 3, iteration 4t + g in
  // lane group g (every group holds the column values after cross_row_sum). The
  // group being filled builds up in stash_acc and is pushed in front every fourth
  // iteration, so after the chunk stash[nt][kStash - 1 - t] holds group t and no
  // register is indexed at run time.
  // Only where the 32 registers per tile fit without spilling (bf16 KV, and one
  // page in flight with two tiles); elsewhere every chunk but the last is written.
  constexpr bool kUseStash = kGStage && kBf16 && (NT == 1 || DEPTH == 1);
  static_assert(kChunk % (4 * kVerifyWaves) == 0 && kWave == 64, "a stash register holds 4 iterations, one per 16-lane group");
  constexpr int kStash = kUseStash ? kChunk / (4 * kVerifyWaves) : 1;
  float stash[NT][kStash];
  float stash_acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    stash_acc[nt] = -INFINITY;
#pragma unroll
    for (int t = 0; t < kStash; ++t) stash[nt][t] = -INFINITY;
  }
  const int kreg = kUseStash ? kfin - 1 : -1;  // the stashed chunk (none below 0)

  float m_run[NT], l_run[NT];
  f32x4_t oacc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) oacc[nt][dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto load_k = [&](int it, KF (&kf)[KC]) {
    const int blk = block_of(it);
    const T* kp = kc + (static_cast<size_t>(blk) * a.hkv + kvh) * (kPage * D) + r16 * D;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      if constexpr (kBf16)
        kf[kk] = ld_stream16(kp + kk * 32 + grp * 8);
      else
        kf[kk] = ld_stream16f(kp + kk * 16 + grp * 4);
    }
  };
  auto load_v = [&](int it, VF (&vf)[DT]) {
    const int blk = block_of(it);
    const T* vp = vc + (static_cast<size_t>(blk) * a.hkv + kvh) * (kPage * D) + r16 * kPage + grp * 4;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      if constexpr (kBf16)
        vf[dd] = ld_stream8(vp + dd * 16 * kPage);
      else
        vf[dd] = ld_stream16f(vp + dd * 16 * kPage);
    }
  };

  // One page: S^T and the online softmax for every column tile, then `mid`, then
  // O^T += V^T P^T for every tile.
  auto consume = [&](int p, const KF (&kf)[KC], const VF (&vf)[DT], auto&& mid) {
    const int t0 = p * kPage + grp * 4;
    // keeps the per-page LDS reads of the parked query fragments inside the loop
    if constexpr (kQInLds) asm volatile("" ::: "memory");
    float pr[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const KF qk = kQInLds ? q_lds[nt][kk][lane] : qf[nt][kk];
        if constexpr (kBf16) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]),
                                                      __builtin_bit_cast(bf16x8_t, qk), s, 0, 0, 0);
        } else {
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kk].x, qk.x, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kk].y, qk.y, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kk].z, qk.z, s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kk].w, qk.w, s, 0, 0, 0);
        }
      }
      // lane holds S^T[key t0 + i][column nt*16 + r16], i = 0..3
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (t0 + i <= lim[nt]) ? s[i] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = cross_row_max(mx);
      // Lazy rescale: the reference max m_run of a column only moves when the
      // page's max exceeds it by more than kRescaleSlack (log2 units), and then for
      // the whole wave at once (a uniform branch), so the accumulator tiles are
      // rescaled on a few pages per wave instead of every page. Weights taken
      // against a stale reference stay below 2^kRescaleSlack; the result is the
      // same up to rounding because l and O always share one reference.
      if (__builtin_amdgcn_ballot_w64(mx > m_run[nt] + kRescaleSlack)) {
        const float m_new = fmaxf(m_run[nt], mx);
        const float alpha = fast_exp2(m_run[nt] - ((m_new == -INFINITY) ? 0.f : m_new));
        l_run[nt] *= alpha;
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) oacc[nt][dd] *= alpha;
        m_run[nt] = m_new;
      }
      const float m_use = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[nt][i] = fast_exp2(sv[i] - m_use);
      const float psum = (pr[nt][0] + pr[nt][1]) + (pr[nt][2] + pr[nt][3]);
      l_run[nt] += psum;

      if (want_lse) {
        const float ps = cross_row_sum(psum);
        const float lse = (ps > 0.f) ? m_use + fast_log2(ps) : -INFINITY;
        bool to_lds = true;
        if constexpr (kUseStash) {
          // the page's virtual index, rounded down to its iteration's (uniform)
          const int vi = ((p + goff) >> 2) << 2;
          if (vi / kChunk == kreg) {
            stash_acc[nt] = (grp == ((vi >> 2) & 3)) ? lse : stash_acc[nt];
            to_lds = false;
          }
        }
        if (to_lds && grp == 0 && (!kUnit || nt * 16 + r16 < a.M)) lse_slot(nt * 16 + r16, p - p_begin) = lse;
      }
    }
    mid();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (kBf16) {
        const uint32_t lo = pack_bf16x2(pr[nt][0], pr[nt][1]);
        const uint32_t hi = pack_bf16x2(pr[nt][2], pr[nt][3]);
        const i16x4_t pb = __builtin_bit_cast(i16x4_t, make_uint2(lo, hi));
#pragma unroll
        for (int dd = 0; dd < DT; ++dd)
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, vf[dd]), pb,
                                                                   oacc[nt][dd], 0, 0, 0);
      } else {
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) {
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dd].x, pr[nt][0], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dd].y, pr[nt][1], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dd].z, pr[nt][2], oacc[nt][dd], 0, 0, 0);
          oacc[nt][dd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[dd].w, pr[nt][3], oacc[nt][dd], 0, 0, 0);
        }
      }
    }
  };

  // Ring of NS register slots; iteration it uses slot it % NS and the loads for
  // it + DEPTH are issued while page it is consumed. The prologue loads are
  // unconditional (clamped to the last page) and the steady-state loop issues its
  // prefetch unconditionally, so the compiler's waits before each page cover only
  // that page's loads and DEPTH pages stay in flight. With two column tiles
  // (kStagger) the next page's V is issued only after this page's S^T, when this
  // page's K slot is dead, which keeps 16 fewer VGPRs live at the peak.
  constexpr bool kStagger = NT > 1;
  KF kf[NS][KC];
  VF vf[NS][DT];
  auto step = [&](int it, int s_cur, int s_next, bool prefetch) {
    const int p = first + kVerifyWaves * it;
    if (kStagger) {
      if (prefetch) load_k(it + DEPTH, kf[s_next]);
      consume(p, kf[s_cur], vf[s_cur], [&] {
        if (prefetch) load_v(it + DEPTH, vf[s_next]);
      });
    } else {
      if (prefetch) {
        load_k(it + DEPTH, kf[s_next]);
        load_v(it + DEPTH, vf[s_next]);
      }
      consume(p, kf[s_cur], vf[s_cur], [] {});
    }
    if constexpr (kGStage) {
      // Chunk k ends with this iteration's pages when (it + 1) * 4 + goff = (k + 1)
      // kChunk; every wave has that iteration. It leaves LDS unless it is the last,
      // or the stashed one, which never was in LDS.
      const int vend = (it + 1) * kVerifyWaves + goff;
      if (want_lse && vend % kChunk == 0 && (it + 1) * kVerifyWaves < n_pages && vend / kChunk - 1 != kreg) {
        __syncthreads();
        flush_chunk(vend / kChunk - 1);
        __syncthreads();
      }
      if constexpr (kUseStash) {
        // a stashed group is complete after its fourth iteration
        const int vi = it * kVerifyWaves + goff;
        if (want_lse && vi / kChunk == kreg && ((vi >> 2) & 3) == 3) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int t = kStash - 1; t > 0; --t) stash[nt][t] = stash[nt][t - 1];
            stash[nt][0] = stash_acc[nt];
          }
        }
      }
    }
  };
  if (n_it > 0) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      load_k(min(s, n_it - 1), kf[s]);
      load_v(min(s, n_it - 1), vf[s]);
    }
    int it = 0;
    for (; it + NS - 1 + DEPTH < n_it; it += NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s) step(it + s, s, (s + DEPTH) % NS, true);
    }
#pragma unroll
    for (int s = 0; s < NS + DEPTH; ++s) {
      if (it + s < n_it) step(it + s, s % NS, (s + DEPTH) % NS, it + s + DEPTH < n_it);
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_run[nt] = cross_row_sum(l_run[nt]);

  __shared__ float red_m[kVerifyWaves - 1][NT][16];
  __shared__ float red_l[kVerifyWaves - 1][NT][16];
  __shared__ float col_lse[NT * 16];  // whole-unit mode: log2-sum-exp of each column
  // Merge weights of one column over the four waves (wave 0's own m and l in
  // registers, the others' from red_m / red_l): the column's reference max, its
  // sum and each wave's weight.
  auto merge_weights = [&](int nt, float (&wt)[kVerifyWaves], float& lsum) {
    float mw[kVerifyWaves], lw[kVerifyWaves];
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
    lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) {
      wt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - mstar);
      lsum += wt[w] * lw[w];
    }
    return mstar;
  };

  if constexpr (kUnit) {
    // Whole-unit mode: column statistics first, then the page scores from the
    // staging, then the output merge in the staging's bytes.
    if (wave > 0 && grp == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        red_m[wave - 1][nt][r16] = m_run[nt];
        red_l[wave - 1][nt][r16] = l_run[nt];
      }
    }
    __syncthreads();
    if (wave == 0 && grp == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float wt[kVerifyWaves], lsum;
        const float mstar = merge_weights(nt, wt, lsum);
        col_lse[nt * 16 + r16] = (lsum > 0.f) ? mstar + fast_log2(lsum) : -INFINITY;
      }
    }
    if (want_lse) {
      // The unit's share of each page score: softmax mass of the page summed over
      // this kv head's M rows, in column order.
      if constexpr (kGStage) {
        // Every chunk's stores are complete (acknowledged by the L2 this CU reads
        // through) before any wave of the workgroup reads them back; the lines
        // were never read before on this CU, so its L1 holds no stale copy.
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
      float* dst = a.unit_scores + static_cast<size_t>(unit) * a.maxp;
      for (int p = threadIdx.x; p < n_pages; p += kVerifyThreads) {
        float sum = 0.f;
        if constexpr (kGStage) {
          const int v = p + goff;
          if (v / kChunk == kreg) continue;  // in its wave's stash: written below
          if (v / kChunk == kfin) {  // the last chunk, still in LDS
            for (int c = 0; c < a.M; ++c) {
              const float x = lse_dyn[c * kChunkStride + (v & (kChunk - 1))];
              sum += (x == -INFINITY) ? 0.f : fast_exp2(x - col_lse[c]);
            }
          } else {
            // page p's MP rows are contiguous: all loaded together as 16-byte vectors
            // (groups past MP clamped to the last, and not summed)
            const float* src = a.gstage + ((static_cast<size_t>(unit) * a.gchunks + v / kChunk) * kChunk +
                                           (v & (kChunk - 1))) * MP;
            float4 x[NT * 4];
#pragma unroll
            for (int c4 = 0; c4 < NT * 4; ++c4)
              x[c4] = *reinterpret_cast<const float4*>(src + min(c4 * 4, MP - 4));
#pragma unroll
            for (int c4 = 0; c4 < NT * 4; ++c4) {
              const float xs[4] = {x[c4].x, x[c4].y, x[c4].z, x[c4].w};
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int c = c4 * 4 + t;
                if (c < a.M) sum += (xs[t] == -INFINITY) ? 0.f : fast_exp2(xs[t] - col_lse[c]);
              }
            }
          }
        } else {
          for (int c = 0; c < a.M; ++c) {
            const float x = lse_dyn[c * a.lse_stride + p];
            sum += (x == -INFINITY) ? 0.f : fast_exp2(x - col_lse[c]);
          }
        }
        st_stream4f(dst + p, sum);
      }
      if constexpr (kUseStash) {
        // The stashed chunk: each wave sums its own pages, the two tiles' columns
        // in each lane, then the 16 lanes of each group (one page per group).
        if (kreg >= 0) {
#pragma unroll
          for (int t = 0; t < kStash; ++t) {
            float e = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const int c = nt * 16 + r16;
              const float x = stash[nt][kStash - 1 - t];
              if (c < a.M && x != -INFINITY) e += fast_exp2(x - col_lse[c]);
            }
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) e += __shfl_xor(e, m);
            const int q = kreg * kChunk + 4 * (4 * t + grp) + wave - goff;
            if (r16 == 0 && q >= 0 && q < n_pages) st_stream4f(dst + q, e);
          }
        }
      }
      if (a.head_out)
        for (int p = n_pages + threadIdx.x; p < a.maxp; p += kVerifyThreads) dst[p] = 0.f;
    }
    __syncthreads();  // the staging has been read: the merge buffer takes its bytes
    if (wave > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dd = 0; dd < DT; ++dd) red_o[wave - 1][nt][dd][lane] = oacc[nt][dd];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = nt * 16 + r16;
        if (c < a.M) {
          float wt[kVerifyWaves], lsum;
          merge_weights(nt, wt, lsum);
          // final row: normalise and write the output directly
          const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
          const int i = c / a.g;
          const int hh = c - i * a.g;
          const size_t ob = ((static_cast<size_t>(b) * a.G1 + i) * a.hq + kvh * a.g + hh) * D + grp * 4;
#pragma unroll
          for (int dd = 0; dd < DT; ++dd) {
            f32x4_t o = oacc[nt][dd] * wt[0];
#pragma unroll
            for (int w = 1; w < kVerifyWaves; ++w) o += red_o[w - 1][nt][dd][lane] * wt[w];
            o *= inv;
            if constexpr (kBf16) {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ob + dd * 16) =
                  make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(a.out) + ob + dd * 16) =
                  make_float4(o[0], o[1], o[2], o[3]);
            }
          }
        }
      }
    }
  } else {
    // Split mode first writes out the staged per-page log-sum-exps; then the four
    // waves merge in LDS (in the pool, once every wave is past the loop and the
    // staging has been read) and wave 0 writes the split's partial.
    if constexpr (kLoopBytes > 0) __syncthreads();
    if (want_lse) {
      // The split's M rows of 256 entries are one contiguous, aligned block: whole
      // 16-byte vectors and whole cache lines (entries past the split's pages are
      // never read).
      float* dst = a.lse + ((static_cast<size_t>(b) * a.max_splits + split) * a.hkv + kvh) * a.M * kMaxPagesPerSplit;
      for (int i = threadIdx.x; i < a.M * (kMaxPagesPerSplit / 4); i += kVerifyThreads) {
        const int c = i / (kMaxPagesPerSplit / 4);
        const int q4 = i % (kMaxPagesPerSplit / 4);
        st_stream16f(dst + c * kMaxPagesPerSplit + q4 * 4, *reinterpret_cast<const float4*>(&lse_slot(c, q4 * 4)));
      }
    }
    __syncthreads();
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
    if (wave == 0) {
      const size_t sbase = static_cast<size_t>(unit) * a.max_splits + split;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = nt * 16 + r16;
        float wt[kVerifyWaves], lsum;
        const float mstar = merge_weights(nt, wt, lsum);
        if (c < a.M) {
          float* po = a.part_o + (sbase * a.M + c) * D + grp * 4;
#pragma unroll
          for (int dd = 0; dd < DT; ++dd) {
            f32x4_t o = oacc[nt][dd] * wt[0];
#pragma unroll
            for (int w = 1; w < kVerifyWaves; ++w) o += red_o[w - 1][nt][dd][lane] * wt[w];
            st_stream16f(po + dd * 16, make_float4(o[0], o[1], o[2], o[3]));
          }
          if (grp == 0) {
            st_stream4f(a.part_ml + (sbase * a.M + c) * 2 + 0, mstar);
            st_stream4f(a.part_ml + (sbase * a.M + c) * 2 + 1, lsum);
          }
        }
      }
    }
  }
}

// Whole-unit mode, second kernel: page_scores[b][p] = sum over kv heads, in kv
// head order, of the units' page masses; 0 at and beyond ceil((L_b + G1) / P).
__global__ __launch_bounds__(256) void verify_unit_scores(const float* __restrict__ unit_scores,
                                                          const int32_t* __restrict__ lens, float* scores, int hkv,
                                                          int maxp, int G1) {
  const int b = blockIdx.y;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= maxp) return;
  const int L = clamp_len(lens[b], maxp, G1);
  const int n_pages = (L + G1 + kPage - 1) / kPage;
  float s = 0.f;
  if (p < n_pages) {
    const float* src = unit_scores + static_cast<size_t>(b) * hkv * maxp + p;
    for (int h = 0; h < hkv; ++h) s += src[static_cast<size_t>(h) * maxp];
  }
  scores[static_cast<size_t>(b) * maxp + p] = s;
}

// Second kernel. Workgroups [0, B * n_chunks) finalise page scores: one chunk of
// 64 pages of one sequence, lanes over pages and the four waves over that
// sequence's hkv * M rows (row log-sum-exps first merged from the split
// partials); workgroups [B * n_chunks, + B * hkv) merge one unit's split partials
// into its output rows.
constexpr int kCombineThreads = 256;
constexpr int kCombineRowBatch = 32;  // page log-sum-exps loaded together per thread
constexpr int kCombineSplitBatch = 8; // split statistics or partials loaded together
constexpr int kCombineOutBatch = 2;   // runs of four outputs one thread merges at a time

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void verify_combine(VerifyArgs a, int n_chunks) {
  extern __shared__ float smem[];
  const int M = a.M;
  const int rows = a.hkv * M;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool scores_part = blockIdx.x < static_cast<unsigned>(a.num_seqs_x_chunks);
  const int b = scores_part ? blockIdx.x / n_chunks : (blockIdx.x - a.num_seqs_x_chunks) / a.hkv;
  const int L = clamp_len(a.lens[b], a.maxp, a.G1);
  const int n_pages = (L + a.G1 + kPage - 1) / kPage;
  const int n_splits = (n_pages + a.pps - 1) / a.pps;

  // log2-sum-exp of a row over its splits, and (for outputs) each split's weight.
  // The statistics of kCombineSplitBatch splits are loaded together (one memory
  // latency per batch instead of one per split); the sums run in split order.
  auto split_ml = [&](const float* ml, int s) {
    return s < n_splits ? *reinterpret_cast<const float2*>(ml + static_cast<size_t>(s) * M * 2)
                        : make_float2(-INFINITY, 0.f);
  };
  auto row_stats = [&](int unit, int c, float& mx, float& l) {
    const float* ml = a.part_ml + (static_cast<size_t>(unit) * a.max_splits * M + c) * 2;
    float2 v[kCombineSplitBatch];
#pragma unroll
    for (int j = 0; j < kCombineSplitBatch; ++j) v[j] = split_ml(ml, j);
    mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCombineSplitBatch; ++j) mx = fmaxf(mx, v[j].x);
    for (int s0 = kCombineSplitBatch; s0 < n_splits; s0 += kCombineSplitBatch) {
      float2 w[kCombineSplitBatch];
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j) w[j] = split_ml(ml, s0 + j);
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j) mx = fmaxf(mx, w[j].x);
    }
    l = 0.f;
#pragma unroll
    for (int j = 0; j < kCombineSplitBatch; ++j)
      if (v[j].x != -INFINITY) l += v[j].y * fast_exp2(v[j].x - mx);
    for (int s0 = kCombineSplitBatch; s0 < n_splits; s0 += kCombineSplitBatch) {
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j) v[j] = split_ml(ml, s0 + j);
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j)
        if (v[j].x != -INFINITY) l += v[j].y * fast_exp2(v[j].x - mx);
    }
  };

  if (scores_part) {
    if (a.scores == nullptr && a.head_scores == nullptr) return;
    const int chunk = blockIdx.x - b * n_chunks;
    float* lse2 = smem;               // [rows]
    float* part = smem + rows;        // [4][64]
    for (int r = tid; r < rows; r += kCombineThreads) {
      float mx, l;
      row_stats(b * a.hkv + r / M, r % M, mx, l);
      lse2[r] = (l > 0.f) ? mx + log2f(l) : -INFINITY;
    }
    __syncthreads();
    const int p = chunk * 64 + lane;
    if (a.head_scores != nullptr) {
      // per kv head: page p's mass over that head's M rows, one head per wave at a time
      for (int kvh = wave; kvh < a.hkv; kvh += 4) {
        float s = 0.f;
        if (p < n_pages) {
          const int sp = ((p + 1) * n_splits + n_pages - 1) / n_pages - 1;
          const int q = p - static_cast<int>(static_cast<long long>(sp) * n_pages / n_splits);
          const float* lb = a.lse + ((static_cast<size_t>(b) * a.max_splits + sp) * rows + kvh * M) *
                                        kMaxPagesPerSplit + q;
          for (int c0 = 0; c0 < M; c0 += kCombineSplitBatch) {
            float x[kCombineSplitBatch];
#pragma unroll
            for (int j = 0; j < kCombineSplitBatch; ++j)
              x[j] = (c0 + j < M) ? lb[static_cast<size_t>(c0 + j) * kMaxPagesPerSplit] : -INFINITY;
#pragma unroll
            for (int j = 0; j < kCombineSplitBatch; ++j)
              s += (x[j] == -INFINITY) ? 0.f : fast_exp2(x[j] - lse2[kvh * M + min(c0 + j, M - 1)]);
          }
        }
        if (p < a.maxp) a.head_scores[(static_cast<size_t>(b) * a.hkv + kvh) * a.maxp + p] = (p < n_pages) ? s : 0.f;
      }
      return;
    }
    float s = 0.f;
    if (p < n_pages) {
      // split of page p under the balanced cut p_begin(s) = floor(s * n_pages / n_splits)
      const int sp = ((p + 1) * n_splits + n_pages - 1) / n_pages - 1;
      const int q = p - static_cast<int>(static_cast<long long>(sp) * n_pages / n_splits);
      const float* lb = a.lse + (static_cast<size_t>(b) * a.max_splits + sp) * rows * kMaxPagesPerSplit + q;
      for (int r0 = wave * kCombineRowBatch; r0 < rows; r0 += 4 * kCombineRowBatch) {
        float x[kCombineRowBatch];
#pragma unroll
        for (int j = 0; j < kCombineRowBatch; ++j)
          x[j] = (r0 + j < rows) ? lb[static_cast<size_t>(r0 + j) * kMaxPagesPerSplit] : -INFINITY;
#pragma unroll
        for (int j = 0; j < kCombineRowBatch; ++j)
          s += (x[j] == -INFINITY) ? 0.f : fast_exp2(x[j] - lse2[min(r0 + j, rows - 1)]);
      }
    }
    part[wave * 64 + lane] = s;
    __syncthreads();
    if (wave == 0 && p < a.maxp)
      a.scores[static_cast<size_t>(b) * a.maxp + p] =
          (p < n_pages) ? (part[lane] + part[64 + lane]) + (part[128 + lane] + part[192 + lane]) : 0.f;
    return;
  }

  const int kvh = (blockIdx.x - a.num_seqs_x_chunks) - b * a.hkv;
  const int unit = b * a.hkv + kvh;
  float* wts = smem;  // [n_splits][M]
  for (int c = tid; c < M; c += kCombineThreads) {
    float mx, l;
    row_stats(unit, c, mx, l);
    const float* ml = a.part_ml + (static_cast<size_t>(unit) * a.max_splits * M + c) * 2;
    for (int s0 = 0; s0 < n_splits; s0 += kCombineSplitBatch) {
      float2 v[kCombineSplitBatch];
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j) v[j] = split_ml(ml, s0 + j);
#pragma unroll
      for (int j = 0; j < kCombineSplitBatch; ++j)
        if (s0 + j < n_splits) wts[(s0 + j) * M + c] = (v[j].x != -INFINITY && l > 0.f) ? fast_exp2(v[j].x - mx) / l : 0.f;
    }
  }
  __syncthreads();
  // Each thread merges kCombineOutBatch runs of four consecutive outputs (one
  // 16-byte load per split and run), each output summed over its splits in split
  // order; the partials of kCombineSplitBatch splits are loaded together.
  const float* po = a.part_o + static_cast<size_t>(unit) * a.max_splits * M * D;
  const int n_out = M * D;  // a multiple of 4: D is 64 or 128
  for (int i0 = tid * 4; i0 < n_out; i0 += kCombineThreads * 4 * kCombineOutBatch) {
    float4 o[kCombineOutBatch];
#pragma unroll
    for (int u = 0; u < kCombineOutBatch; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < n_splits; s0 += kCombineSplitBatch) {
      float4 x[kCombineOutBatch][kCombineSplitBatch];
#pragma unroll
      for (int u = 0; u < kCombineOutBatch; ++u) {
        const int idx = i0 + u * kCombineThreads * 4;
#pragma unroll
        for (int j = 0; j < kCombineSplitBatch; ++j)
          x[u][j] = (idx < n_out && s0 + j < n_splits)
                        ? *reinterpret_cast<const float4*>(po + static_cast<size_t>(s0 + j) * n_out + idx)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kCombineOutBatch; ++u) {
        const int idx = i0 + u * kCombineThreads * 4;
        const int c = min(idx / D, M - 1);
#pragma unroll
        for (int j = 0; j < kCombineSplitBatch; ++j) {
          if (idx < n_out && s0 + j < n_splits) {
            const float w = wts[min(s0 + j, n_splits - 1) * M + c];
            o[u].x += w * x[u][j].x;
            o[u].y += w * x[u][j].y;
            o[u].z += w * x[u][j].z;
            o[u].w += w * x[u][j].w;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineOutBatch; ++u) {
      const int idx = i0 + u * kCombineThreads * 4;
      if (idx >= n_out) break;
      const int c = idx / D;
      const int d = idx - c * D;
      const int i = c / a.g;
      const int hh = c - i * a.g;
      const size_t oi = ((static_cast<size_t>(b) * a.G1 + i) * a.hq + kvh * a.g + hh) * D + d;
      const float ov[4] = {o[u].x, o[u].y, o[u].z, o[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (std::is_same<T, bf16_t>::value)
          static_cast<uint16_t*>(a.out)[oi + e] = f32_to_bf16(ov[e]);
        else
          static_cast<float*>(a.out)[oi + e] = ov[e];
      }
    }
  }
}

// Static LDS of the whole-unit kernel: the wave merge statistics, the column
// log-sum-exps, the longest-first ranking and the pool's minimum.
constexpr size_t kUnitStaticLds = sizeof(float) * 2 * (kVerifyWaves - 1) * 16 + sizeof(float) * 16 +
                                  sizeof(int) * (kLptMaxSeqs + 1) + 16;
// Dynamic LDS the whole-unit merge of the output accumulators needs (NT tiles).
constexpr size_t unit_merge_bytes(int D, int NT = 1) {
  return sizeof(float) * 4 * (kVerifyWaves - 1) * NT * (D / 16) * kWave;
}

template <typename T, int D, int NT, bool kUnit, bool kGStage = false>
hipError_t launch_main(const VerifyArgs& args, int depth, dim3 grid, size_t smem, hipStream_t stream) {
  if constexpr (kGStage) {  // global staging: one or two pages in flight
    if (depth >= 2)
      hipLaunchKernelGGL((verify_main<T, D, NT, 2, true, true>), grid, dim3(kVerifyThreads), smem, stream, args);
    else
      hipLaunchKernelGGL((verify_main<T, D, NT, 1, true, true>), grid, dim3(kVerifyThreads), smem, stream, args);
  } else {
    if (depth >= 3)
      hipLaunchKernelGGL((verify_main<T, D, NT, 3, kUnit>), grid, dim3(kVerifyThreads), smem, stream, args);
    else if (depth == 2)
      hipLaunchKernelGGL((verify_main<T, D, NT, 2, kUnit>), grid, dim3(kVerifyThreads), smem, stream, args);
    else
      hipLaunchKernelGGL((verify_main<T, D, NT, 1, kUnit>), grid, dim3(kVerifyThreads), smem, stream, args);
  }
  return hipGetLastError();
}

// The unit page masses of whole-unit mode, summed over kv heads into page_scores.
hipError_t launch_unit_scores(const VerifyArgs& args, int num_seqs, hipStream_t stream) {
  if (args.scores == nullptr || args.head_out) return hipSuccess;
  hipLaunchKernelGGL(verify_unit_scores, dim3((args.maxp + 255) / 256, num_seqs), dim3(256), 0, stream,
                     args.unit_scores, args.lens, args.scores, args.hkv, args.maxp, args.G1);
  return hipGetLastError();
}

template <typename T, int D, int NT>
hipError_t launch_typed(VerifyArgs args, const VerifyPlan& pl, int num_units, hipStream_t stream) {
  const int num_seqs = num_units / args.hkv;
  if (pl.unit && pl.gstage) {
    // a chunk of per-page staging in LDS, then the wave merge in the same bytes
    const size_t stage = args.unit_scores ? static_cast<size_t>(args.M) * kChunkStride * sizeof(float) : 0;
    const size_t smem = stage > unit_merge_bytes(D, NT) ? stage : unit_merge_bytes(D, NT);
    hipError_t e = launch_main<T, D, NT, true, true>(args, pl.depth, dim3(num_units), smem, stream);
    return e != hipSuccess ? e : launch_unit_scores(args, num_seqs, stream);
  }
  if constexpr (NT == 1) {
    if (pl.unit) {
      // the per-page staging (with scores), and the wave-merge buffer after it
      const size_t stage = args.unit_scores ? static_cast<size_t>(args.M) * args.lse_stride * sizeof(float) : 0;
      const size_t smem = stage > unit_merge_bytes(D) ? stage : unit_merge_bytes(D);
      hipError_t e = launch_main<T, D, 1, true>(args, pl.depth, dim3(num_units), smem, stream);
      return e != hipSuccess ? e : launch_unit_scores(args, num_seqs, stream);
    }
  }
  hipError_t e = launch_main<T, D, NT, false>(args, pl.depth, dim3(num_units * args.max_splits), 0, stream);
  if (e != hipSuccess) return e;
  const int n_chunks = (args.maxp + 63) / 64;
  args.num_seqs_x_chunks = num_seqs * n_chunks;
  const size_t smem = verify_combine_lds_bytes(args.hkv, args.M, args.max_splits);
  hipLaunchKernelGGL((verify_combine<T, D>), dim3(args.num_seqs_x_chunks + num_units), dim3(kCombineThreads), smem,
                     stream, args, n_chunks);
  return hipGetLastError();
}

}  // namespace

size_t verify_combine_lds_bytes(int hkv, int M, int max_splits) {
  const size_t scores = static_cast<size_t>(hkv) * M + 4 * 64;
  const size_t outputs = static_cast<size_t>(max_splits) * M;
  return (scores > outputs ? scores : outputs) * 4;
}

VerifyPlan plan_verify(const KvView& kv, int num_seqs, int hq, int G1) {
  VerifyPlan pl{};
  pl.num_seqs = num_seqs;
  pl.hq = hq;
  pl.G1 = G1;
  pl.g = hq / kv.hkv;
  pl.M = G1 * pl.g;
  // Tuning knobs (environment overrides for measurement sweeps): pages per split
  // (1 .. 256, so each of the four waves holds at most 64 pages) and pages in
  // flight per wave (1 .. 3).
  int pps = kMaxPagesPerSplit;
  if (const char* e = getenv("S3R_VERIFY_PAGES_PER_SPLIT")) {
    const int v = atoi(e);
    if (v >= 1) pps = v;
  }
  pl.pps = pps > kMaxPagesPerSplit ? kMaxPagesPerSplit : pps;
  // measured on MI355X: two pages in flight per wave with one column tile (three
  // gain nothing), one with two column tiles (about 1 % faster than two, and three
  // spill); fp32 pages are twice the registers, so one
  int depth = (kv.bf16 && pl.M <= 16) ? 2 : 1;
  if (const char* e = getenv("S3R_VERIFY_DEPTH")) {
    const int v = atoi(e);
    if (v >= 1 && v <= 3) depth = v;
  }
  pl.depth = depth;
  const bool depth_forced = getenv("S3R_VERIFY_DEPTH") != nullptr;
  pl.max_splits = (kv.maxp + pl.pps - 1) / pl.pps;
  const size_t units = static_cast<size_t>(num_seqs) * kv.hkv;
  size_t off = 0;
  pl.off_part_o = off;
  off = align_up(off + units * pl.max_splits * pl.M * kv.head_dim * 4, 256);
  pl.off_part_ml = off;
  off = align_up(off + units * pl.max_splits * pl.M * 2 * 4, 256);
  pl.off_lse = off;  // whole-unit mode keeps its [B][hkv][maxp] page masses here
  off = align_up(off + units * pl.max_splits * pl.M * kMaxPagesPerSplit * 4, 256);
  // whole-unit mode with global staging: chunks of kChunk pages of the M rows
  pl.gchunks = (kv.maxp + kChunk - 1) / kChunk;
  pl.off_gstage = off;
  off = align_up(off + units * pl.gchunks * kChunk * ((pl.M + 3) & ~3) * 4, 256);
  pl.bytes = off;

  // Whole-unit mode (one workgroup per (sequence, kv head), no split partials)
  // when one column tile holds the rows, the block ids fit the lane registers and
  // the per-page staging M x maxp fits LDS next to the merge buffers, leaving room
  // for two workgroups per CU. Split mode otherwise, or when forced.
  pl.lse_stride = kv.maxp | 1;  // odd stride: the 16 columns of one page fall in distinct banks
  const size_t unit_lds = static_cast<size_t>(pl.M) * pl.lse_stride * sizeof(float);
  int max_lds = 65536;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0) max_lds = v;
  }
  const size_t per_wg_cap = max_lds < kUnitLdsPerWorkgroup ? static_cast<size_t>(max_lds) : kUnitLdsPerWorkgroup;
  const size_t unit_dyn = unit_lds > unit_merge_bytes(kv.head_dim) ? unit_lds : unit_merge_bytes(kv.head_dim);
  const bool blk_fit = kv.maxp <= kVerifyWaves * kWave * kUnitBlkRegs;
  pl.unit = pl.M <= 16 && blk_fit && unit_dyn + kUnitStaticLds <= per_wg_cap;
  pl.gstage = false;
  int cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  // Whole-unit mode with the per-page staging in the workspace, when it does not
  // fit LDS (two column tiles, or a long history) and there are at least as many
  // units as CUs (with fewer, splits keep the chip busy).
  if (!pl.unit && blk_fit && units >= static_cast<size_t>(cus)) {
    pl.unit = true;
    pl.gstage = true;
  }
  if (const char* e = getenv("S3R_VERIFY_MODE")) {
    if (e[0] == 's') pl.unit = pl.gstage = false;
    if (e[0] == 'g' && blk_fit) pl.unit = pl.gstage = true;
  }
  // measured on MI355X (8B-like 24K workload, two column tiles): one page in
  // flight per wave, 2277 us against 2328 us with two
  if (pl.gstage && !depth_forced) pl.depth = (kv.bf16 && pl.M <= 16) ? 2 : 1;
  // Longest-first order pays when the units take more than one wave of
  // workgroups (two whole-unit workgroups per CU); with one wave every unit
  // starts at once and the ranking would only add latency.
  pl.lpt = pl.unit && num_seqs <= kLptMaxSeqs && units > static_cast<size_t>(2 * cus);
  if (const char* e = getenv("S3R_VERIFY_ORDER")) pl.lpt = pl.unit && num_seqs <= kLptMaxSeqs && e[0] == 'l';
  if (getenv("S3R_VERIFY_PAGES_PER_SPLIT") != nullptr) pl.unit = pl.gstage = false;
  return pl;
}

hipError_t launch_verify(const KvView& kv, const VerifyPlan& pl, const void* q, float scale, void* out,
                         float* scores, void* workspace, hipStream_t stream, const void* k_new, const void* v_new,
                         float* head_scores, const int32_t* horizons) {
  char* ws = static_cast<char*>(workspace);
  const int units = pl.num_seqs * kv.hkv;
  VerifyArgs a{};
  a.k = kv.k;
  a.v = kv.v;
  a.table = kv.table;
  a.lens = kv.lens;
  a.q = q;
  a.out = out;
  a.scores = scores;
  a.k_new = k_new;
  a.v_new = v_new;
  a.part_o = reinterpret_cast<float*>(ws + pl.off_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + pl.off_part_ml);
  const bool any_scores = scores != nullptr || head_scores != nullptr;
  a.lse = (any_scores && !pl.unit) ? reinterpret_cast<float*>(ws + pl.off_lse) : nullptr;
  a.unit_scores = nullptr;
  if (pl.unit && head_scores != nullptr) {
    a.unit_scores = head_scores;  // the units' page masses are the per-kv-head scores
    a.head_out = 1;
  } else if (pl.unit && scores != nullptr) {
    a.unit_scores = reinterpret_cast<float*>(ws + pl.off_lse);
  }
  a.head_scores = pl.unit ? nullptr : head_scores;
  if (head_scores != nullptr) a.scores = nullptr;
  a.horizons = horizons;
  a.lse_stride = pl.lse_stride;
  a.gstage = reinterpret_cast<float*>(ws + pl.off_gstage);
  a.gchunks = pl.gchunks;
  a.num_seqs = pl.num_seqs;
  a.lpt = pl.lpt ? 1 : 0;
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
  const bool two = pl.M > 16;
  if (kv.bf16) {
    if (kv.head_dim == 128)
      return two ? launch_typed<bf16_t, 128, 2>(a, pl, units, stream)
                 : launch_typed<bf16_t, 128, 1>(a, pl, units, stream);
    return two ? launch_typed<bf16_t, 64, 2>(a, pl, units, stream)
               : launch_typed<bf16_t, 64, 1>(a, pl, units, stream);
  }
  if (kv.head_dim == 128)
    return two ? launch_typed<float, 128, 2>(a, pl, units, stream)
               : launch_typed<float, 128, 1>(a, pl, units, stream);
  return two ? launch_typed<float, 64, 2>(a, pl, units, stream)
             : launch_typed<float, 64, 1>(a, pl, units, stream);
}

}  // namespace s3r
