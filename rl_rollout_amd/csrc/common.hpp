// Shared device helpers for the S3R kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace s3r {

constexpr int kPage = 16;          // tokens per KV page
constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct bf16_t {  // storage tag for bf16 tensors (raw 16-bit patterns)
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats to packed bf16 (lo in the low half), rounded to nearest even by the
// hardware conversion (one v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_cvt_t));
}

template <typename T>
__device__ __forceinline__ T bit_cast_to(uint32_t x) {
  return __builtin_bit_cast(T, x);
}

// ---- cross-lane reductions -------------------------------------------------
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror. Applied in this order they pair every lane of a 16-lane row with
// lanes of the other quad / half-row, so after four steps each lane of the row
// holds the row-wide result, bitwise identical across the row (the operands of
// each step are the same pair in swapped order).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return x;
}

// Sum / max over the four 16-lane rows (lanes l, l^16, l^32, l^48), on the VALU
// with the gfx950 row-swap permutes (no LDS round trip). With both operands equal
// to x, permlane16_swap returns rows [0,0,2,2] and [1,1,3,3] of x, and
// permlane32_swap rows [0,1,0,1] and [2,3,2,3]; combining the pair after each swap
// leaves (x0 op x1) op (x2 op x3) in every row, the same value in all four.
__device__ __forceinline__ float cross_row_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float cross_row_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
  for (int m = 1; m < kWave; m <<= 1) x = max(x, __shfl_xor(x, m));
  return x;
}

// Fast 2^x (v_exp_f32). Inputs of -inf give 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Streaming loads with the non-temporal hint: KV pages and logits are read once
// per call, and on MI355X these loads sustain a markedly higher HBM read rate
// than default-cached loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
}

__device__ __forceinline__ float4 ld_stream16f(const void* p) {
  const uint4 u = ld_stream16(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// Non-temporal stores for data written once per call and read back by a later
// kernel (split partials): while the chip streams KV at full rate, ordinary
// stores of these rows cost far more than their bytes; the streaming hint
// roughly halves that cost on MI355X.
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_stream16f(void* p, float4 v) {
  const f32x4v_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4v_t*>(p));
}

__device__ __forceinline__ void st_stream4f(void* p, float v) {
  __builtin_nontemporal_store(v, reinterpret_cast<float*>(p));
}

// Writes the K/V rows of token positions [pos0, pos0 + n) that fall in `page`
// into the kv head's slab of block blk, with whole-line stores only. K rows are
// contiguous (one 16-slot page is [16][D]) and are copied in 16-byte chunks. A V
// row is one element per dim, 16 slots apart (the page is stored [D][16]), so
// the slab's 16-byte chunks are read, the new slots merged in, and the chunks
// written back whole: partial-line stores are expensive while the chip streams
// KV (the memory controller turns them into read-modify-writes). Row r's K and
// V are ksrc + r * src_stride and vsrc + r * src_stride ([D] elements each).
template <typename T, int D>
__device__ __forceinline__ void put_rows_in_page(void* kc, void* vc, int hkv, int kvh, int blk, int page, int pos0,
                                                 int n, const T* ksrc, const T* vsrc, size_t src_stride, int tid,
                                                 int nthreads) {
  constexpr int E = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPD = kPage / E;      // V chunks per dim (2 for bf16, 4 for fp32)
  const int lo = max(pos0, page * kPage), hi = min(pos0 + n, (page + 1) * kPage);
  if (lo >= hi) return;
  const size_t slab = (static_cast<size_t>(blk) * hkv + kvh) * (kPage * D);
  // K: row (pos & 15) of the slab, D / E chunks per row
  uint4* kd = reinterpret_cast<uint4*>(static_cast<T*>(kc) + slab);
  const int kchunks = (hi - lo) * (D / E);
  for (int c = tid; c < kchunks; c += nthreads) {
    const int r = lo + c / (D / E);
    const uint4* ks = reinterpret_cast<const uint4*>(ksrc + (r - pos0) * src_stride);
    kd[(r & (kPage - 1)) * (D / E) + c % (D / E)] = ks[c % (D / E)];
  }
  // V: chunk c holds slots (c % CPD) * E .. + E - 1 of dim c / CPD
  uint4* vd = reinterpret_cast<uint4*>(static_cast<T*>(vc) + slab);
  for (int c = tid; c < D * CPD; c += nthreads) {
    const int d = c / CPD;
    const int s0 = (c % CPD) * E;
    const int first = max(lo, (lo & ~(kPage - 1)) + s0), last = min(hi, (lo & ~(kPage - 1)) + s0 + E);
    if (first >= last) continue;
    uint4 v = vd[c];
    T* ve = reinterpret_cast<T*>(&v);
    const int pb = (lo & ~(kPage - 1)) + s0;  // position of the chunk's first slot
#pragma unroll
    for (int e = 0; e < E; ++e) {  // constant indices keep the chunk in registers
      const int pos = pb + e;
      if (pos >= first && pos < last) ve[e] = vsrc[(pos - pos0) * src_stride + d];
    }
    vd[c] = v;
  }
}

}  // namespace s3r
