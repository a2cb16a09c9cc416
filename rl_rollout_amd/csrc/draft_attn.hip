// Sparse self-draft attention: one query per sequence and query head (the token
// at position pi = L_b + j - 1 of draft step j) over the score-selected full
// pages of the history plus the always-read tail page(s)
// (abstract; wispaper.ai, "S3R drafts sparsely and verifies densely";
// rebasdaily.com, "草稿可以稀疏，交卷必须完整").
//
// The work is HBM-bound at 2 (g = 2) to 4 (g = 4) flop per byte, far under the
// VALU ridge, so it stays on the vector ALUs; there is no dense contraction to
// give to MFMA. One workgroup owns one (sequence, kv head) and its g query
// heads; its NW waves take the gathered page list round-robin, each page a
// 4 KB K slab and a 4 KB page-transposed V slab (bf16), both read with 16-byte
// loads that cover 1 KB of contiguous memory per wave instruction:
//   QK: lane (key l%16, 16-byte chunk group l/16) dots its 8 (bf16) or 4 (fp32)
//       dims with each query head (v_dot2_f32_bf16 for bf16), then the four
//       chunk groups are summed across rows.
//   softmax: per-head online max / rescale over the 16 keys of a page (DPP row
//       reductions), with keys past pi masked on the tail pages.
//   PV: the page's 16 weights per head pass through a small wave-private LDS
//       slot; lane l then owns one dim per 1 KB slice of the V slab and half
//       (bf16) or a quarter (fp32) of the page's keys, combined at the end.
// The waves merge their (m, l, o) in LDS and the workgroup writes the output:
// no split partials and no second kernel.
#include <stdlib.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {
namespace {

struct DraftArgs {
  void* k;
  void* v;
  const void* k_new;  // optional row [B][hkv][D] of this draft token, written at L + step - 1 first
  const void* v_new;
  const int32_t* table;
  const int32_t* lens;
  const void* q;
  void* out;
  const int32_t* sel;
  const int32_t* nsel;
  // Draft-row mode (k_rows != nullptr): the keys and values of the in-flight draft
  // tokens (positions L .. L + step - 1) are read from these buffers; row r of
  // sequence b, kv head h starts at element r * row_stride + b * seq_stride + h * D.
  // The cache is read only below position L and is not written.
  const void* k_rows;
  const void* v_rows;
  long long row_stride, seq_stride;
  // Draft-row mode, optional [B]: the draft horizon gamma_b of each sequence; a
  // sequence with step > gamma_b is skipped (its output rows are not written)
  const int32_t* horizons;
  int max_sel, num_blocks, hkv, hq, maxp, step;
  int num_seqs;
  int lpt;           // take units longest first
  int sel_per_head;  // sel [B][hkv][max_sel], nsel [B][hkv]
  float scale_log2;
};

// Longest-first order when the units outnumber the workgroups the chip runs at
// once: workgroup i takes the sequence of rank i / hkv in (pages attended
// descending, index ascending), each workgroup ranking the num_seqs sequences
// itself from LDS (the host enables this for at most kDraftLptMaxSeqs).
constexpr int kDraftLptMaxSeqs = 1024;
constexpr int kDraftLptAutoSeqs = 128;  // default use: at most this many sequences

template <bool kHorizon>
__device__ int draft_lpt_unit(const DraftArgs& a, int wg, int nthreads) {
  __shared__ __attribute__((aligned(16))) int s_ent[kDraftLptMaxSeqs];
  __shared__ int s_seq;
  static_assert(kDraftLptMaxSeqs % 4 == 0, "the ranking reads the entries four at a time");
  const int B = a.num_seqs;
  const int B4 = (B + 3) & ~3;
  for (int j = threadIdx.x; j < B4; j += nthreads) {
    int e = -1;  // padding past B: below every entry (all >= 0), so never counted
    if (j < B) {
      const int L = max(0, min(a.lens[j], a.maxp * kPage - a.step));
      const int n_full = L >> 4;
      // with a page set per kv head every head of a sequence selects the same number
      e = max(0, min(a.nsel[a.sel_per_head ? j * a.hkv : j], a.max_sel)) + ((L + a.step - 1) >> 4) - n_full + 1;
      if constexpr (kHorizon) {
        if (a.step > a.horizons[j]) e = 0;  // skipped: ranked last
      }
    }
    s_ent[j] = e;
  }
  __syncthreads();
  // rank of j = #{i : n_i > n_j} + #{i < j : n_i == n_j}; the entries are read as
  // 16-byte broadcasts, several in flight, so the scan is not one LDS round trip
  // per entry
  const int want = wg / a.hkv;
  for (int j = threadIdx.x; j < B; j += nthreads) {
    const int nj = s_ent[j];
    int rank = 0;
#pragma unroll 8
    for (int i = 0; i < B4; i += 4) {
      const int4 v = *reinterpret_cast<const int4*>(&s_ent[i]);
      rank += static_cast<int>(v.x > nj) + static_cast<int>((v.x == nj) & (i < j));
      rank += static_cast<int>(v.y > nj) + static_cast<int>((v.y == nj) & (i + 1 < j));
      rank += static_cast<int>(v.z > nj) + static_cast<int>((v.z == nj) & (i + 2 < j));
      rank += static_cast<int>(v.w > nj) + static_cast<int>((v.w == nj) & (i + 3 < j));
    }
    if (rank == want) s_seq = j;
  }
  __syncthreads();
  return s_seq * a.hkv + wg % a.hkv;
}

// The register budget asks for two workgroups per CU: with eight waves per
// workgroup that is four waves per SIMD (at most 128 VGPRs).
// kHorizon (draft-row mode only): a.horizons holds a draft horizon per sequence.
template <typename T, int D, int G, int NW, int DEPTH, bool kRows, bool kHorizon = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 2))) void draft_kernel(DraftArgs a) {
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  constexpr int kElem = kBf16 ? 2 : 4;
  constexpr int EPC = 16 / kElem;          // elements per 16-byte chunk
  constexpr int KCH = D * kElem / 64;      // K chunks per lane per page
  constexpr int RB = kPage * kElem;        // bytes of one V^T row (16 keys of one dim)
  constexpr int LPR = RB / 16;             // lanes per V^T row
  constexpr int VCH = D * RB / 1024;       // 1 KB slices of the V^T slab
  constexpr int DPS = 1024 / RB;           // dims per 1 KB slice
  constexpr int NS = DEPTH + 1;            // register ring slots

  const int lane = threadIdx.x & 63;
  // wave index made visibly uniform so the entry loop runs on scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  int unit = blockIdx.x;
  if (a.lpt) unit = draft_lpt_unit<kHorizon>(a, unit, NW * kWave);
  const int b = unit / a.hkv;
  const int kvh = unit - b * a.hkv;

  // the page list of this sequence, or of this (sequence, kv head) with a set per kv head
  const size_t sel_row = a.sel_per_head ? static_cast<size_t>(b) * a.hkv + kvh : static_cast<size_t>(b);
  // Entry e of the gathered list (selected pages, then the tail pages) belongs to
  // wave e % NW at iteration e / NW, and lane `it` of a wave resolves the page and
  // block of its iteration `it`.
  // The lengths and the selection entries of the first 64 iterations are loaded
  // first and together (the entries before the count is known, at indices clamped
  // into the selection row); the page-table entries of those iterations and the
  // query chunks then go out together, so from kernel start to the first KV byte
  // the chain is lengths and selection, page table and queries, KV.
  const int e_first = wave + NW * lane;
  int sel_first = a.sel[sel_row * a.max_sel + min(e_first, a.max_sel - 1)];
  int len_raw = a.lens[b];
  int nsel_raw = a.nsel[sel_row];
  // the values are needed here, so the compiler issues the loads together instead
  // of sinking the selection load behind the counts it is used under
  if constexpr (kHorizon) {
    int horizon = a.horizons[b];
    asm volatile("" : "+v"(sel_first), "+s"(len_raw), "+s"(nsel_raw), "+s"(horizon));
    if (a.step > horizon) return;  // uniform: this sequence drafts fewer tokens
  } else {
    asm volatile("" : "+v"(sel_first), "+s"(len_raw), "+s"(nsel_raw));
  }
  const int L = max(0, min(len_raw, a.maxp * kPage - a.step));
  const int pi = L + a.step - 1;
  const int n_full = L >> 4;
  const int ns = max(0, min(nsel_raw, a.max_sel));
  // last cache position attended, and the tail pages that hold cache keys: up to
  // pi, or, in draft-row mode, up to L - 1 (only a partial last page)
  const int last_cache = kRows ? L - 1 : pi;
  const int n_tail = kRows ? ((L & 15) ? 1 : 0) : (pi >> 4) - n_full + 1;
  const int n_ent = ns + n_tail;
  // (page, block) of entry base + e_first, or (0, 0) past the list; the block id
  // is returned as read (clamped where it is used, so nothing waits for it here)
  auto resolve = [&](int base) __attribute__((always_inline)) {
    const int e = base + e_first;
    int2 pb = make_int2(0, 0);
    if (e < n_ent) {
      int page = e >= ns ? n_full + (e - ns) : base == 0 ? sel_first : a.sel[sel_row * a.max_sel + e];
      page = min(max(page, 0), a.maxp - 1);
      pb = make_int2(page, a.table[static_cast<size_t>(b) * a.maxp + page]);
    }
    return pb;
  };
  const int2 first_pb = resolve(0);

  // Draft-row mode: the in-flight rows (the first 16 here, in the same round trip
  // as the queries) are staged in LDS in the page layout, K rows [16][D] and V
  // transposed [D][16]; rows past the step repeat the last one and are masked.
  constexpr int CPR = D * kElem / 16;  // 16-byte chunks per row
  __shared__ uint4 rows_k[kRows ? kPage * CPR : 1];
  __shared__ T rows_v[kRows ? D * kPage : 1];
  // chunk c of the 16 rows from row g0: K chunk as is, V chunk transposed
  auto stage_chunk = [&](int g0, int c) {
    const size_t base = static_cast<size_t>(b) * a.seq_stride + static_cast<size_t>(kvh) * D;
    const T* kr = static_cast<const T*>(a.k_rows) + base;
    const T* vr = static_cast<const T*>(a.v_rows) + base;
    const int r = c / CPR;
    const int ch = c - r * CPR;
    const size_t src = static_cast<size_t>(min(g0 + r, a.step - 1)) * a.row_stride + ch * EPC;
    rows_k[c] = *reinterpret_cast<const uint4*>(kr + src);
    const uint4 v4 = *reinterpret_cast<const uint4*>(vr + src);
    T e[EPC];
    __builtin_memcpy(e, &v4, 16);
#pragma unroll
    for (int x = 0; x < EPC; ++x) rows_v[(ch * EPC + x) * kPage + r] = e[x];
  };

  // Query chunks of the g heads, matching the lane's K chunks (4k + grp), parked
  // in LDS and re-read per page: registers go to pages in flight instead. One
  // unrolled loop stages them and (draft-row mode) the first 16 rows, so all
  // their loads are issued before the first wait.
  __shared__ uint4 q_lds[G][KCH][kWave];
  constexpr int kQChunks = G * KCH * kWave;
  constexpr int kQRounds = (kQChunks + NW * kWave - 1) / (NW * kWave);
  constexpr int kRowRounds = kRows ? (kPage * CPR + NW * kWave - 1) / (NW * kWave) : 0;
  constexpr int kRounds = kQRounds > kRowRounds ? kQRounds : kRowRounds;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = static_cast<int>(threadIdx.x) + r * NW * kWave;
    if (r < kQRounds && (kQChunks % (NW * kWave) == 0 || i < kQChunks)) {
      const int h = i / (KCH * kWave);
      const int k = (i / kWave) % KCH;
      const int ln = i % kWave;
      const T* qp = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.hq + kvh * G + h) * D;
      q_lds[h][k][ln] = *reinterpret_cast<const uint4*>(qp + (4 * k + (ln >> 4)) * EPC);
    }
    if constexpr (kRows) {
      if (r < kRowRounds && ((kPage * CPR) % (NW * kWave) == 0 || i < kPage * CPR)) stage_chunk(0, i);
    }
  }

  // Fused append of this draft token's row (position pi): written by the one wave
  // that reads its page, the last entry n_ent - 1 (wave (n_ent - 1) % NW), before
  // that wave's page loop. No barrier: the other waves start streaming at once,
  // and one wave's accesses to one address stay in program order.
  if (a.k_new != nullptr && n_ent > 0 && wave == (n_ent - 1) % NW) {
    const int blk = a.table[static_cast<size_t>(b) * a.maxp + (pi >> 4)];
    if (blk >= 0 && blk < a.num_blocks) {
      const size_t src = (static_cast<size_t>(b) * a.hkv + kvh) * D;
      put_rows_in_page<T, D>(a.k, a.v, a.hkv, kvh, blk, pi >> 4, pi, 1, static_cast<const T*>(a.k_new) + src,
                             static_cast<const T*>(a.v_new) + src, D, lane, kWave);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    asm volatile("" ::: "memory");
  }

  const T* __restrict__ kc = static_cast<const T*>(a.k);
  const T* __restrict__ vc = static_cast<const T*>(a.v);

  __syncthreads();

  float m_run[G], l_run[G];
  float oacc[G][VCH];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int k = 0; k < VCH; ++k) oacc[h][k] = 0.f;
  }

  __shared__ float lds_p[NW][G][kPage];
  const int half = lane % LPR;  // which EPC-key slice of the page this lane's V chunk covers

  // One page: q.k and the online softmax of every head (keys with key_ok false
  // are masked), then `mid` (which issues the next page's V loads once this page's
  // K registers are dead), then P.V.
  auto attend = [&](const uint4 (&kf)[KCH], const uint4 (&vf)[VCH], bool key_ok, auto&& mid) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        const uint4 qk = q_lds[h][k][lane];
        if constexpr (kBf16) {
          s = __builtin_amdgcn_fdot2_f32_bf16(bit_cast_to<bf16x2_t>(kf[k].x), bit_cast_to<bf16x2_t>(qk.x), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(bit_cast_to<bf16x2_t>(kf[k].y), bit_cast_to<bf16x2_t>(qk.y), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(bit_cast_to<bf16x2_t>(kf[k].z), bit_cast_to<bf16x2_t>(qk.z), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(bit_cast_to<bf16x2_t>(kf[k].w), bit_cast_to<bf16x2_t>(qk.w), s, false);
        } else {
          s = fmaf(__uint_as_float(kf[k].x), __uint_as_float(qk.x), s);
          s = fmaf(__uint_as_float(kf[k].y), __uint_as_float(qk.y), s);
          s = fmaf(__uint_as_float(kf[k].z), __uint_as_float(qk.z), s);
          s = fmaf(__uint_as_float(kf[k].w), __uint_as_float(qk.w), s);
        }
      }
      s = cross_row_sum(s);  // full q.k of key r16, identical in all four rows
      const float sv = key_ok ? s * a.scale_log2 : -INFINITY;
      const float mx = row16_max(sv);
      const float m_new = fmaxf(m_run[h], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[h] - m_use);
      const float p = fast_exp2(sv - m_use);
      l_run[h] = l_run[h] * alpha + p;
      m_run[h] = m_new;
#pragma unroll
      for (int k = 0; k < VCH; ++k) oacc[h][k] *= alpha;
      if (grp == 0) lds_p[wave][h][r16] = p;
    }
    mid();
    // LDS traffic of one wave is processed in order: the reads below see the
    // writes above. The asm statements only keep the compiler from moving
    // memory operations across them.
    asm volatile("" ::: "memory");
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* pp = &lds_p[wave][h][half * EPC];
      if constexpr (kBf16) {
        const float4 p0 = *reinterpret_cast<const float4*>(pp);
        const float4 p1 = *reinterpret_cast<const float4*>(pp + 4);
        const bf16x2_t w0 = bit_cast_to<bf16x2_t>(pack_bf16x2(p0.x, p0.y));
        const bf16x2_t w1 = bit_cast_to<bf16x2_t>(pack_bf16x2(p0.z, p0.w));
        const bf16x2_t w2 = bit_cast_to<bf16x2_t>(pack_bf16x2(p1.x, p1.y));
        const bf16x2_t w3 = bit_cast_to<bf16x2_t>(pack_bf16x2(p1.z, p1.w));
#pragma unroll
        for (int k = 0; k < VCH; ++k) {
          float o = oacc[h][k];
          o = __builtin_amdgcn_fdot2_f32_bf16(w0, bit_cast_to<bf16x2_t>(vf[k].x), o, false);
          o = __builtin_amdgcn_fdot2_f32_bf16(w1, bit_cast_to<bf16x2_t>(vf[k].y), o, false);
          o = __builtin_amdgcn_fdot2_f32_bf16(w2, bit_cast_to<bf16x2_t>(vf[k].z), o, false);
          o = __builtin_amdgcn_fdot2_f32_bf16(w3, bit_cast_to<bf16x2_t>(vf[k].w), o, false);
          oacc[h][k] = o;
        }
      } else {
        const float4 p0 = *reinterpret_cast<const float4*>(pp);
#pragma unroll
        for (int k = 0; k < VCH; ++k) {
          float o = oacc[h][k];
          o = fmaf(p0.x, __uint_as_float(vf[k].x), o);
          o = fmaf(p0.y, __uint_as_float(vf[k].y), o);
          o = fmaf(p0.z, __uint_as_float(vf[k].z), o);
          o = fmaf(p0.w, __uint_as_float(vf[k].w), o);
          oacc[h][k] = o;
        }
      }
    }
    asm volatile("" ::: "memory");
  };

  for (int base = 0; base < n_ent; base += NW * 64) {
    const int2 pb = base == 0 ? first_pb : resolve(base);
    const int my_page = pb.x, my_blk = min(max(pb.y, 0), a.num_blocks - 1);
    const int rem = n_ent - base - wave;
    const int n_it = rem <= 0 ? 0 : min(64, (rem + NW - 1) / NW);

    auto load_k = [&](int it, uint4 (&kf)[KCH]) {
      const int blk = __builtin_amdgcn_readlane(my_blk, it);
      const char* kp = reinterpret_cast<const char*>(kc + (static_cast<size_t>(blk) * a.hkv + kvh) * (kPage * D));
#pragma unroll
      for (int k = 0; k < KCH; ++k) kf[k] = ld_stream16(kp + r16 * (D * kElem) + (4 * k + grp) * 16);
    };
    auto load_v = [&](int it, uint4 (&vf)[VCH]) {
      const int blk = __builtin_amdgcn_readlane(my_blk, it);
      const char* vp = reinterpret_cast<const char*>(vc + (static_cast<size_t>(blk) * a.hkv + kvh) * (kPage * D));
#pragma unroll
      for (int k = 0; k < VCH; ++k) vf[k] = ld_stream16(vp + k * 1024 + lane * 16);
    };

    // One page of this loop: entry e's keys past the last cache position attended
    // are masked on the tail pages.
    auto consume = [&](int it, const uint4 (&kf)[KCH], const uint4 (&vf)[VCH], auto&& mid) {
      const int e = base + wave + NW * it;
      const int page = __builtin_amdgcn_readlane(my_page, it);
      const bool tail = e >= ns;
      attend(kf, vf, !tail || (page * kPage + r16 <= last_cache), mid);
    };

    // Ring of NS register slots; see verify_main: an unconditional prologue and a
    // steady-state loop with unconditional prefetch keep DEPTH pages in flight.
    // K of page it + DEPTH is issued before page it's q.k, its V after it.
    uint4 kf[NS][KCH], vf[NS][VCH];
    auto step = [&](int it, int s_cur, int s_next, bool prefetch) {
      if (prefetch) load_k(it + DEPTH, kf[s_next]);
      consume(it, kf[s_cur], vf[s_cur], [&] {
        if (prefetch) load_v(it + DEPTH, vf[s_next]);
      });
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
  }

  // Draft-row mode: the in-flight rows are one more page (16 keys at a time),
  // taken by the wave that has the fewest cache pages, from the LDS staging (rows
  // past the first 16 are staged by that wave here).
  if constexpr (kRows) {
    if (wave == n_ent % NW) {
      for (int g0 = 0; g0 < a.step; g0 += kPage) {
        if (g0 > 0)
          for (int c = lane; c < kPage * CPR; c += kWave) stage_chunk(g0, c);
        // one wave's LDS accesses are processed in order; the asm keeps the
        // compiler from moving them across
        asm volatile("" ::: "memory");
        uint4 kf[KCH], vf[VCH];
#pragma unroll
        for (int k = 0; k < KCH; ++k) kf[k] = rows_k[r16 * CPR + 4 * k + grp];
#pragma unroll
        for (int k = 0; k < VCH; ++k) vf[k] = reinterpret_cast<const uint4*>(rows_v)[k * (1024 / 16) + lane];
        attend(kf, vf, g0 + r16 < a.step, [] {});
        asm volatile("" ::: "memory");
      }
    }
  }

  // combine the LPR lanes that share a dim, and the row's keys of l
  __shared__ float lds_m[NW][G], lds_l[NW][G];
  __shared__ float lds_o[NW][G][D];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = row16_sum(l_run[h]);
#pragma unroll
    for (int k = 0; k < VCH; ++k) {
      float o = oacc[h][k];
      o += __shfl_xor(o, 1);
      if constexpr (LPR == 4) o += __shfl_xor(o, 2);
      if (half == 0) lds_o[wave][h][k * DPS + lane / LPR] = o;
    }
    if (lane == 0) {
      lds_m[wave][h] = m_run[h];
      lds_l[wave][h] = lt;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mstar = fmaxf(mstar, lds_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = lds_m[w][h];
      const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mstar);
      num += wt * lds_o[w][h][d];
      den += wt * lds_l[w][h];
    }
    const float o = den > 0.f ? num / den : 0.f;
    const size_t oi = (static_cast<size_t>(b) * a.hq + kvh * G + h) * D + d;
    if constexpr (kBf16)
      static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(o);
    else
      static_cast<float*>(a.out)[oi] = o;
  }
}

template <typename T, int D, int G, int NW>
hipError_t launch_nw(const DraftArgs& a, int depth, int units, hipStream_t stream) {
  switch (depth) {
    case 1: hipLaunchKernelGGL((draft_kernel<T, D, G, NW, 1, false>), dim3(units), dim3(NW * 64), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((draft_kernel<T, D, G, NW, 3, false>), dim3(units), dim3(NW * 64), 0, stream, a); break;
    default: hipLaunchKernelGGL((draft_kernel<T, D, G, NW, 2, false>), dim3(units), dim3(NW * 64), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_g(const DraftArgs& a, int waves, int depth, int units, hipStream_t stream) {
  if (a.k_rows != nullptr) {
    // draft-row mode: the default shape only (four waves, one page in flight for
    // bf16; eight waves for fp32)
    constexpr int NWr = std::is_same<T, float>::value ? 8 : 4;
    if (a.horizons != nullptr)
      hipLaunchKernelGGL((draft_kernel<T, D, G, NWr, 1, true, true>), dim3(units), dim3(NWr * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((draft_kernel<T, D, G, NWr, 1, true>), dim3(units), dim3(NWr * 64), 0, stream, a);
    return hipGetLastError();
  }
  if constexpr (std::is_same<T, float>::value) {
    return launch_nw<T, D, G, 8>(a, 1, units, stream);
  } else {
    return waves == 4 ? launch_nw<T, D, G, 4>(a, depth, units, stream) : launch_nw<T, D, G, 8>(a, depth, units, stream);
  }
}

template <typename T, int D>
hipError_t launch_d(const DraftArgs& a, int g, int waves, int depth, int units, hipStream_t stream) {
  switch (g) {
    case 1: return launch_g<T, D, 1>(a, waves, depth, units, stream);
    case 2: return launch_g<T, D, 2>(a, waves, depth, units, stream);
    case 4: return launch_g<T, D, 4>(a, waves, depth, units, stream);
    default: return launch_g<T, D, 8>(a, waves, depth, units, stream);
  }
}

}  // namespace

hipError_t launch_draft(const KvView& kv, int num_seqs, int hq, int step, const void* q, float scale,
                        const int32_t* sel, const int32_t* nsel, int max_sel, void* out, hipStream_t stream,
                        const void* k_new, const void* v_new, bool sel_per_head, const void* k_rows,
                        const void* v_rows, long long row_stride, long long seq_stride,
                        const int32_t* horizons) {
  DraftArgs a{};
  a.k_rows = k_rows;
  a.horizons = k_rows != nullptr ? horizons : nullptr;
  a.v_rows = v_rows;
  a.row_stride = row_stride;
  a.seq_stride = seq_stride;
  a.k = kv.k;
  a.v = kv.v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.sel_per_head = sel_per_head ? 1 : 0;
  a.table = kv.table;
  a.lens = kv.lens;
  a.q = q;
  a.out = out;
  a.sel = sel;
  a.nsel = nsel;
  a.max_sel = max_sel;
  a.num_blocks = kv.num_blocks;
  a.hkv = kv.hkv;
  a.hq = hq;
  a.maxp = kv.maxp;
  a.step = step;
  a.scale_log2 = scale * kLog2e;
  a.num_seqs = num_seqs;
  const int g = hq / kv.hkv;
  const int units = num_seqs * kv.hkv;
  // Longest-first order pays when the units take a little more than one wave of
  // workgroups (about three draft workgroups per CU run at once) and their
  // lengths spread widely. Its cost is the ranking prologue, about 4 us per call,
  // almost all of it the round trip that loads every sequence's count before the
  // workgroup knows its unit. Measured on MI355X: 98 -> 86-89 us per draft on 128
  // sequences of 2K-16K tokens (1024 units), 108 -> 112 us on 128 of equal length,
  // 89.5 -> 92 us on 256 of 1K-16K (2048 units, where natural order already
  // balances); so the default takes it for at most 128 sequences.
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  a.lpt = (num_seqs <= kDraftLptAutoSeqs && units > 3 * cus) ? 1 : 0;
  if (const char* e = getenv("S3R_DRAFT_ORDER")) a.lpt = (num_seqs <= kDraftLptMaxSeqs && e[0] == 'l') ? 1 : 0;
  // Tuning knobs (environment overrides for measurement sweeps): waves per
  // workgroup (4 or 8) and pages in flight per wave (1 .. 3), bf16 only.
  int waves = 4, depth = 1;  // measured best on MI355X for g = 2 and g = 4
  if (const char* e = getenv("S3R_DRAFT_WAVES")) waves = atoi(e) == 4 ? 4 : 8;
  if (const char* e = getenv("S3R_DRAFT_DEPTH")) {
    const int v = atoi(e);
    if (v >= 1 && v <= 3) depth = v;
  }
  if (kv.bf16)
    return kv.head_dim == 128 ? launch_d<bf16_t, 128>(a, g, waves, depth, units, stream)
                              : launch_d<bf16_t, 64>(a, g, waves, depth, units, stream);
  return kv.head_dim == 128 ? launch_d<float, 128>(a, g, waves, depth, units, stream)
                            : launch_d<float, 64>(a, g, waves, depth, units, stream);
}

}  // namespace s3r
