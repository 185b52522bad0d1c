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

// Streaming loads and stores: every byte of the hot arrays is touched once
// per call, so they carry the non-temporal hint. Loads are the compiler's
// non-temporal loads ("nt"; the policies "sc1 nt" and "sc0 sc1 nt" measured
// no different). The 16- and 8-byte stores use the cache policy
// "sc0 sc1 nt" (system scope, written through), which has no builtin, so
// they are one vector global store in inline assembly; other sizes use the
// compiler's non-temporal store. A store of more than 8 bytes reads its data
// registers late: on gfx950 a VALU write to them needs two wait states after
// the store (the compiler pads a plain 16-byte store that way), which the
// compiler's hazard pass does not insert for a store inside inline assembly,
// so the 16-byte form carries its own s_nop 1. With one wait state only, a
// decode variant whose compiler placed an address computation into the data
// registers right after the store wrote wrong values.
// Measured on the 7B shard, interleaved A/B, store policies "nt" /
// "sc1 nt" / "sc0 sc1 nt": AdamW 6,282 / 6,297 / 6,301 GB/s, flatten + norm
// 5,997 / 6,014 / 6,040 GB/s, a plain copy 6,524 / 6,627 / 6,631; plain
// (write-back) stores: AdamW 5,517 GB/s against 6,215.
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T *p, T v) {
  if constexpr (sizeof(T) == 16) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
  } else if constexpr (sizeof(T) == 8) {
    asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1 nt" : : "v"(p), "v"(v) : "memory");
  } else {
    __builtin_nontemporal_store(v, p);
  }
}
// A pointer that is the same on every lane of the wave, moved to scalar
// registers (the address form below needs its base there).
template <typename T>
__device__ __forceinline__ T *wave_uniform(T *p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<T *>((static_cast<uint64_t>(hi) << 32) | lo);
}
// The same 16- or 8-byte streaming store at a wave-uniform base plus a
// 32-bit per-lane byte offset (the scalar-base address form: the base stays
// in scalar registers and a loop over tiles advances it with scalar adds).
template <typename T>
__device__ __forceinline__ void st_stream_at(void *base, uint32_t byte_off, T v) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte stores only");
  if constexpr (sizeof(T) == 16)
    asm volatile("global_store_dwordx4 %0, %1, %2 sc0 sc1 nt\n\ts_nop 1" : : "v"(byte_off), "v"(v), "s"(base) : "memory");
  else
    asm volatile("global_store_dwordx2 %0, %1, %2 sc0 sc1 nt" : : "v"(byte_off), "v"(v), "s"(base) : "memory");
}
// A 16- or 8-byte streaming load in the same address form that returns only
// once the data has arrived (the wait is part of the same instruction
// sequence), so that a wave issuing several of them has one load in flight at
// a time.
template <typename T>
__device__ __forceinline__ T ld_stream_at_once(const void *base, uint32_t byte_off) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte loads only");
  T r;
  if constexpr (sizeof(T) == 16)
    asm volatile("global_load_dwordx4 %0, %1, %2 nt\n\ts_waitcnt vmcnt(0)" : "=v"(r) : "v"(byte_off), "s"(base) : "memory");
  else
    asm volatile("global_load_dwordx2 %0, %1, %2 nt\n\ts_waitcnt vmcnt(0)" : "=v"(r) : "v"(byte_off), "s"(base) : "memory");
  return r;
}
// A streaming load through a global-address-space pointer, so that it is a
// global (not a flat) load: a flat load also counts against the LDS
// counter, and the wait for LDS before a barrier would then wait for it too.
template <typename T>
__device__ __forceinline__ T ld_stream_global(const T *p) {
  typedef __attribute__((address_space(1))) const T gT;
  return __builtin_nontemporal_load((gT *)p);
}
// Waits until every vector memory access of the wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

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

// fp64 reductions: DPP inside 16-lane rows, readlane across the rows, LDS
// across waves. Fixed order, so sums are run-to-run identical.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffu), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffu), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sum over the 64 lanes of a wave, the same value returned to every lane.
// Needs all 64 lanes active.
__device__ __forceinline__ double wave_sum(double x) {
  x = x + dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]: pairs
  x = x + dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]: quads
  x = x + dpp_f64<0x124>(x);  // row_ror:4
  x = x + dpp_f64<0x128>(x);  // row_ror:8 -> every lane holds its row's sum
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// acc + x^2 in float64; the square of a 16-bit or fp32 value is exact there.
__device__ __forceinline__ double sq_add(float x, double acc) {
  const double d = static_cast<double>(x);
  return fma(d, d, acc);
}

// Sum over a block of BLOCK threads (all of them must call it); the result is
// valid in thread 0. Waves add in lane order, the wave totals in wave order.
template <int BLOCK>
__device__ __forceinline__ double block_sum(double x) {
  static_assert(BLOCK % 64 == 0, "block is whole waves");
  __shared__ double wsum[BLOCK / 64];
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) wsum[w] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    for (int k = 0; k < BLOCK / 64; ++k) t += wsum[k];
  }
  return t;  // valid in thread 0
}

}  // namespace zds
