// Device-side helpers: element conversions and 16-byte vector access.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "zds.h"

namespace zds {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-bit -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}

template <int D>
__device__ __forceinline__ float lo_of(uint32_t w) {
  return D == ZDS_BF16 ? bf16_lo(w) : f16_lo(w);
}
template <int D>
__device__ __forceinline__ float hi_of(uint32_t w) {
  return D == ZDS_BF16 ? bf16_hi(w) : f16_hi(w);
}

template <int D>
__device__ __forceinline__ float widen1(const void *base, int64_t i) {
  if (D == ZDS_FP32) return static_cast<const float *>(base)[i];
  const uint16_t h = static_cast<const uint16_t *>(base)[i];
  return D == ZDS_BF16 ? __uint_as_float(static_cast<uint32_t>(h) << 16)
                       : __half2float(__ushort_as_half(h));
}

// fp32 -> 16-bit, round to nearest even. bf16 uses gfx950's packed
// conversion instruction, fp16 the IEEE conversion.
template <int D>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if (D == ZDS_BF16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 in = {a, b};
    bf2 r = __builtin_convertvector(in, bf2);
    return __builtin_bit_cast(uint32_t, r);
  } else {
    const uint32_t lo = __half_as_ushort(__float2half_rn(a));
    const uint32_t hi = __half_as_ushort(__float2half_rn(b));
    return lo | (hi << 16);
  }
}

template <int D>
__device__ __forceinline__ uint16_t narrow1(float a) {
  return static_cast<uint16_t>(pack2<D>(a, 0.0f) & 0xffffu);
}

// Streaming 16-byte loads and stores: every byte of the hot arrays is touched
// once per call, so by default they carry the non-temporal hint.
#ifndef ZDS_NT_LOADS
#define ZDS_NT_LOADS 1
#endif
#ifndef ZDS_NT_STORES
#define ZDS_NT_STORES 1
#endif
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) {
#if ZDS_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void st_stream(T *p, T v) {
#if ZDS_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// 8 consecutive 16-bit elements (one 16-byte access) at group index `group`,
// as fp32.
template <int D>
__device__ __forceinline__ void load8(const void *base, int64_t group, float (&x)[8]) {
  static_assert(D != ZDS_FP32, "load8 is for 16-bit data");
  const u32x4 w = ld_stream(static_cast<const u32x4 *>(base) + group);
  x[0] = lo_of<D>(w.x); x[1] = hi_of<D>(w.x);
  x[2] = lo_of<D>(w.y); x[3] = hi_of<D>(w.y);
  x[4] = lo_of<D>(w.z); x[5] = hi_of<D>(w.z);
  x[6] = lo_of<D>(w.w); x[7] = hi_of<D>(w.w);
}

// Quads: 4 consecutive elements per lane, one 16-byte access for fp32 and
// one 8-byte access for 16-bit data; lane l of a wave takes quad base + l so
// each wave-level access covers one contiguous range.
template <int D>
__device__ __forceinline__ void load_quad(const void *base, int64_t q, float (&x)[4]) {
  if (D == ZDS_FP32) {
    const f32x4 a = ld_stream(static_cast<const f32x4 *>(base) + q);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else {
    const u32x2 w = ld_stream(static_cast<const u32x2 *>(base) + q);
    x[0] = lo_of<D>(w.x); x[1] = hi_of<D>(w.x);
    x[2] = lo_of<D>(w.y); x[3] = hi_of<D>(w.y);
  }
}

__device__ __forceinline__ void store_quad(float *base, int64_t q, const float (&x)[4]) {
  const f32x4 a = {x[0], x[1], x[2], x[3]};
  st_stream(reinterpret_cast<f32x4 *>(base) + q, a);
}

template <int D>
__device__ __forceinline__ void store_quad16(void *base, int64_t q, const float (&x)[4]) {
  const u32x2 w = {pack2<D>(x[0], x[1]), pack2<D>(x[2], x[3])};
  st_stream(static_cast<u32x2 *>(base) + q, w);
}

}  // namespace zds
