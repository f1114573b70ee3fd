// Device helpers shared by the gfx950 kernels of the Shampoo library.
#pragma once

#include <hip/hip_runtime.h>
#include <cfloat>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "../../include/shampoo.h"

namespace shp {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Workgroups are handed to the XCDs round-robin (id % 8).  This maps the
// hardware id to a logical id so that each XCD receives one contiguous range
// of logical tiles: the tiles of a factor then share one L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t hw, uint32_t total) {
  const uint32_t q = total / kXcds, r = total % kXcds;
  const uint32_t xcd = hw % kXcds, local = hw / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Global-memory access through an explicit global address space.  Pointers
// that the compiler cannot trace to a kernel argument (descriptor tables,
// pointers picked at run time) would otherwise become flat accesses, which
// also count against the LDS wait counter and so serialise LDS waits with
// outstanding global loads.
template <class T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ void stg(T* p, const T& v) {
  *(__attribute__((address_space(1))) T*)p = v;
}

// f(std::integral_constant<int, i>) for i = 0..N-1, expanded at compile time
// (indices stay constants even where a loop would be too large to unroll).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Deterministic sum over a workgroup of `nthreads` threads (fixed tree order).
// `red` must hold nthreads / 64 floats.  Returns the total in every thread.
template <int kThreads>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) t += red[i];
  __syncthreads();
  return t;
}

// fp32 -> bf16, round to nearest even: gfx950's V_CVT_PK_BF16_F32 (NaN stays
// NaN), two values per instruction when packed.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Two bf16 values (a in the low half) in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// 16-bit operand formats of the half-width MFMA products.
enum { H16_BF16 = 0, H16_F16 = 1 };

__device__ __forceinline__ uint16_t to_h16(float x, int fmt) {
  return fmt == H16_F16 ? f32_to_f16_bits(x) : f32_to_bf16_bits(x);
}

// Two 16-bit values of format fmt (a in the low half) in one dword, each
// rounded to nearest even.  Both conversions and a select: a branch on the
// (uniform) format per pair costs more in the store loops of the epilogues.
__device__ __forceinline__ uint32_t pack_h16x2(float a, float b, int fmt) {
  const f32x2_t v = {a, b};
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  const uint32_t g = pack_bf16x2(a, b);
  return fmt == H16_F16 ? h : g;
}

// Four consecutive 16-bit copies of o at p (p 8-byte aligned).
__device__ __forceinline__ void stg4_h16(uint16_t* p, const floatx4& o, int fmt) {
  u32x2 w;
  w.x = pack_h16x2(o[0], o[1], fmt);
  w.y = pack_h16x2(o[2], o[3], fmt);
  stg(reinterpret_cast<u32x2*>(p), w);
}

// Eight consecutive 16-bit copies of lo, hi at p (p 16-byte aligned).
__device__ __forceinline__ void stg8_h16(uint16_t* p, const floatx4& lo, const floatx4& hi, int fmt) {
  u32x4 w;
  w.x = pack_h16x2(lo[0], lo[1], fmt);
  w.y = pack_h16x2(lo[2], lo[3], fmt);
  w.z = pack_h16x2(hi[0], hi[1], fmt);
  w.w = pack_h16x2(hi[2], hi[3], fmt);
  stg(reinterpret_cast<u32x4*>(p), w);
}

__device__ __forceinline__ bool degenerate(int32_t st) {
  return (st & (SHAMPOO_BLK_ZERO | SHAMPOO_BLK_NONPOS_RQ)) != 0;
}

// Scale constant as used by the iterations: a degenerate factor keeps c = 1
// so that its (discarded) iterates stay finite.
__device__ __forceinline__ float safe_c(const shampoo_scale* sc, const int32_t* status, int64_t f) {
  const float c = sc[f].c;
  if (status != nullptr && degenerate(status[f])) return 1.f;
  return c;
}

}  // namespace shp
