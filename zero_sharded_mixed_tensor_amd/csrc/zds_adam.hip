// Row a4: fused AdamW + unscale/clip + cast on the rank's fp32 master shard.
//
// The update runs on the fp32 master copy while params and grads are 16-bit
// (devpress.csdn.net DeepSpeed tutorial §2.2; aiqz.cc "DeepSpeed ZeRO引擎深入",
// 混合精度); AdamW with betas, eps and weight decay (same tutorial §3.2
// optimizer block); the two moment recurrences as in aiqz.cc's Python 演示.
//
// Memory-bound stream, no MFMA: per element it reads the grad (2 or 4 B) and
// master/m/v (12 B) and writes master/m/v (12 B) and the 16-bit param (2 B):
// 28 B (16-bit grads) or 30 B (fp32 accumulator).
//
// Access pattern. Every wave-level load or store covers one contiguous range
// so each 128-byte line is requested by exactly one instruction;
// non-temporal hints on all of them. (Two 16-byte pieces per lane at stride
// 32 B make two instructions each touch every line half, which measured far
// slower.) The kernels are wave-specialised: each wave of a block moves one
// array piece of the block's tile (master, m, v, grads in / 16-bit params
// out), and the pieces meet in LDS where every thread updates one element.
// Against a kernel in which each lane moves all arrays of its own 4 elements
// (kept as adam_quad_kernel), this lowers the memory footprint per wave from
// 4 loads + 4 stores to 1 + 1 and raised the pass from about 5.8 to 6.0 TB/s
// on the 7B shard. A block takes 2 consecutive tiles (6.0 -> 6.3 TB/s: half
// the block launches, same footprint per wave) and the grid has one block per
// tile pair, so the dispatcher keeps every CU full as blocks finish. Issuing
// the second tile's loads before the first tile's update (software
// pipelining) measured slower: on this memory system more bytes in flight per
// wave lose to more waves with one access each.
//
// The default is adam_wide_kernel: 8 waves and 512 elements per tile, so that
// the 16-bit grads and params also move as one 1 KiB access per wave (16
// bytes per lane), like the fp32 halves; in A/B runs interleaved with the
// order rotated each round it was 1.0 and 2.7 % faster (two boxes) than
// adam_tile_kernel, the 4-wave form with 256-element tiles and 512-byte
// 16-bit accesses, which remains the path for 16-bit buffers that are 8- but
// not 16-byte aligned.
//
// The step constants (lr / (1 - beta1^t), sqrt(1 - beta2^t), 1 - lr*wd, the
// 1 - beta values) are derived once per call by a single-wave prep kernel
// into the caller's step-scalars struct, so the update kernel only loads them.
#include "zds_device.h"
#include "zds_internal.h"

#ifndef ZDS_ADAM_BLOCK
#define ZDS_ADAM_BLOCK 256
#endif
#ifndef ZDS_ADAM_QUADS
#define ZDS_ADAM_QUADS 1
#endif
// 0: one block per tile; > 0: at most this many resident waves per CU, the
// blocks striding over the tiles.
#ifndef ZDS_ADAM_PERSIST
#define ZDS_ADAM_PERSIST 0
#endif
// 1: remap block ids so each XCD streams one contiguous eighth of the arrays
// (measured 3 % slower for the tile kernel on the 7B shard, so off).
#ifndef ZDS_ADAM_XCD
#define ZDS_ADAM_XCD 0
#endif
// 1: wave-specialised tile kernel (one array per wave, LDS exchange);
// 0: every lane moves all arrays of its own quads.
#ifndef ZDS_ADAM_TILE
#define ZDS_ADAM_TILE 1
#endif
// Consecutive tiles per block in the tile kernel.
#ifndef ZDS_ADAM_TPB
#define ZDS_ADAM_TPB 2
#endif
// Upper bound on the tile kernel's grid (blocks loop over the tiles beyond it).
#ifndef ZDS_ADAM_TILE_GRID
#define ZDS_ADAM_TILE_GRID (int64_t(1) << 23)
#endif

namespace zds {

struct AdamArgs {
  const void *g;
  float *p;
  float *m;
  float *v;
  void *out;
  int64_t n;
  float beta1, beta2, eps;
  const zds_step_scalars *sc;
};

struct ElemConsts {
  float b1, b2, omb1, omb2, eps, step_size, bc2_sqrt, decay, gs;
};

__device__ __forceinline__ ElemConsts load_consts(const AdamArgs &a) {
  ElemConsts c;
  c.b1 = a.beta1;
  c.b2 = a.beta2;
  c.eps = a.eps;
  c.omb1 = a.sc->one_minus_beta1;
  c.omb2 = a.sc->one_minus_beta2;
  c.step_size = a.sc->step_size;
  c.bc2_sqrt = a.sc->bc2_sqrt;
  c.decay = a.sc->decay;
  c.gs = a.sc->grad_scale;
  return c;
}

// One element, fp32, one rounding per operation, in this order.
__device__ __forceinline__ void adam_elem(float x, const ElemConsts &c, float &p, float &m, float &v) {
  const float g = x * c.gs;
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float denom = sqrtf(v) / c.bc2_sqrt + c.eps;
  p = p * c.decay;
  p = p - c.step_size * (m / denom);
}

// Block id after the XCD remap: with G a multiple of 8, hardware block b
// runs on XCD b % 8; it is given tile-block (b % 8) * (G / 8) + b / 8.
__device__ __forceinline__ int64_t remapped_block() {
  const int64_t b = blockIdx.x;
  if (!ZDS_ADAM_XCD) return b;
  const int64_t per = static_cast<int64_t>(gridDim.x) >> 3;
  return (b & 7) * per + (b >> 3);
}

template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(ZDS_ADAM_BLOCK) adam_quad_kernel(AdamArgs a) {
  // Skip on overflow without a host round trip; the flag is uniform.
  if (a.sc->overflow) return;
  const ElemConsts c = load_consts(a);
  constexpr int U = ZDS_ADAM_QUADS;
  constexpr int64_t span = static_cast<int64_t>(ZDS_ADAM_BLOCK) * U;
  const int64_t quads = a.n >> 2;
  const int64_t b0 = remapped_block();
  for (int64_t t = b0; t * span < quads; t += gridDim.x) {
    const int64_t q0 = t * span + threadIdx.x;
    float x[U][4], p[U][4], m[U][4], v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + u * ZDS_ADAM_BLOCK;
      if (q < quads) {
        load_quad<GD>(a.g, q, x[u]);
        load_quad<ZDS_FP32>(a.p, q, p[u]);
        load_quad<ZDS_FP32>(a.m, q, m[u]);
        load_quad<ZDS_FP32>(a.v, q, v[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + u * ZDS_ADAM_BLOCK;
      if (q < quads) {
#pragma unroll
        for (int k = 0; k < 4; ++k) adam_elem(x[u][k], c, p[u][k], m[u][k], v[u][k]);
        store_quad(a.p, q, p[u]);
        store_quad(a.m, q, m[u]);
        store_quad(a.v, q, v[u]);
        if (WRITE_OUT) store_quad16<PD>(a.out, q, p[u]);
      }
    }
  }
  // Ragged tail: the last n % 4 elements, one per lane of tile-block 0.
  const int64_t tail0 = quads << 2;
  if (b0 == 0 && tail0 + threadIdx.x < a.n) {
    const int64_t e = tail0 + threadIdx.x;
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

// Wave-specialised variant. A block of 4 waves owns a tile of 64 quads (256
// elements). Wave 0 moves the master tile, wave 1 m, wave 2 v and wave 3 the
// grad tile in and the 16-bit param tile out, each with one contiguous
// wave-wide access per direction; the tiles meet in LDS, where each of the
// 256 threads updates one element. Every wave thus issues one load and one
// store instead of four of each.
template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(256) adam_tile_kernel(AdamArgs a) {
  __shared__ f32x4 sp[64], sm[64], sv[64];
  __shared__ f32x4 sgf[GD == ZDS_FP32 ? 64 : 1];
  __shared__ u32x2 s16[64];  // 16-bit grads in, then the 16-bit params out
  if (a.sc->overflow) return;
  const ElemConsts c = load_consts(a);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t quads = a.n >> 2;
  // Wave w reads and writes LDS buffer w in the load and store phases and
  // all threads touch every buffer in the update phase, which sits between
  // the two barriers; so a wave may start the next tile's load right after
  // its own store without a third barrier.
  const int64_t ntiles = (quads + 63) >> 6;
  for (int64_t it = remapped_block() * ZDS_ADAM_TPB; it < ntiles; it += static_cast<int64_t>(gridDim.x) * ZDS_ADAM_TPB)
  for (int64_t tile = it; tile < it + ZDS_ADAM_TPB && tile < ntiles; ++tile) {  // uniform per block
    const int64_t q0 = tile * 64;
    const int64_t q = q0 + lane;
    const bool ok = q < quads;
    if (w == 0) {
      if (ok) sp[lane] = ld_stream(reinterpret_cast<const f32x4 *>(a.p) + q);
    } else if (w == 1) {
      if (ok) sm[lane] = ld_stream(reinterpret_cast<const f32x4 *>(a.m) + q);
    } else if (w == 2) {
      if (ok) sv[lane] = ld_stream(reinterpret_cast<const f32x4 *>(a.v) + q);
    } else if (ok) {
      if (GD == ZDS_FP32)
        sgf[lane] = ld_stream(static_cast<const f32x4 *>(a.g) + q);
      else
        s16[lane] = ld_stream(static_cast<const u32x2 *>(a.g) + q);
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (q0 + (t >> 2) < quads) {
      float *fp = reinterpret_cast<float *>(sp);
      float *fm = reinterpret_cast<float *>(sm);
      float *fv = reinterpret_cast<float *>(sv);
      uint16_t *h = reinterpret_cast<uint16_t *>(s16);
      float x;
      if (GD == ZDS_FP32) {
        x = reinterpret_cast<const float *>(sgf)[t];
      } else {
        const uint32_t b = h[t];
        x = GD == ZDS_BF16 ? __uint_as_float(b << 16) : __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
      }
      float p = fp[t], m = fm[t], v = fv[t];
      adam_elem(x, c, p, m, v);
      fp[t] = p;
      fm[t] = m;
      fv[t] = v;
      if (WRITE_OUT) h[t] = narrow1<PD>(p);
    }
    __syncthreads();
    if (w == 0) {
      if (ok) st_stream(reinterpret_cast<f32x4 *>(a.p) + q, sp[lane]);
    } else if (w == 1) {
      if (ok) st_stream(reinterpret_cast<f32x4 *>(a.m) + q, sm[lane]);
    } else if (w == 2) {
      if (ok) st_stream(reinterpret_cast<f32x4 *>(a.v) + q, sv[lane]);
    } else if (WRITE_OUT && ok) {
      st_stream(static_cast<u32x2 *>(a.out) + q, s16[lane]);
    }
  }
  // Ragged tail: the last n % 4 elements, one per lane of block 0.
  const int64_t tail0 = quads << 2;
  if (blockIdx.x == 0 && tail0 + threadIdx.x < a.n) {
    const int64_t e = tail0 + threadIdx.x;
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

// Wide wave-specialised variant. A block of 8 waves owns a tile of 512
// elements: waves 0-1 move the two 1 KiB halves of the master tile, 2-3 m,
// 4-5 v; 16-bit grads come in through wave 6 (8 elements per lane, one 1 KiB
// access) and the 16-bit params go out through wave 7; fp32 grads come in
// through waves 6 and 7 (a half each). Each of the 512 threads updates one
// element. The tiles cover the first n & ~7 elements; block 0 takes the rest
// element-wise. As in the 4-wave kernel, outside the update phase each wave
// writes and reads only its own part of the LDS tiles, so two barriers per
// tile suffice.
template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(512) adam_wide_kernel(AdamArgs a) {
  __shared__ f32x4 sf[3][128];
  __shared__ f32x4 sgf[GD == ZDS_FP32 ? 128 : 1];
  __shared__ u32x4 sg16[GD == ZDS_FP32 ? 1 : 64];
  __shared__ u32x4 so16[64];
  if (a.sc->overflow) return;
  const ElemConsts c = load_consts(a);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t nv = a.n & ~int64_t(7);
  const int64_t quads = nv >> 2;
  const int64_t octs = nv >> 3;
  const int64_t ntiles = (nv + 511) >> 9;
  // This wave's half of a 128-quad tile (waves 0-5, and 6-7 for fp32 grads).
  const int half = (w & 1) * 64 + lane;
  float *arr = w < 2 ? a.p : (w < 4 ? a.m : a.v);
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * ZDS_ADAM_TPB; it < ntiles;
       it += static_cast<int64_t>(gridDim.x) * ZDS_ADAM_TPB)
  for (int64_t tile = it; tile < it + ZDS_ADAM_TPB && tile < ntiles; ++tile) {  // uniform per block
    const int64_t q = tile * 128 + half;
    const int64_t o = tile * 64 + lane;
    if (w < 6) {
      if (q < quads) sf[w >> 1][half] = ld_stream(reinterpret_cast<const f32x4 *>(arr) + q);
    } else if (GD == ZDS_FP32) {
      if (q < quads) sgf[half] = ld_stream(static_cast<const f32x4 *>(a.g) + q);
    } else if (w == 6) {
      if (o < octs) sg16[lane] = ld_stream(static_cast<const u32x4 *>(a.g) + o);
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (tile * 512 + t < nv) {
      float *fp = reinterpret_cast<float *>(sf[0]);
      float *fm = reinterpret_cast<float *>(sf[1]);
      float *fv = reinterpret_cast<float *>(sf[2]);
      float x;
      if (GD == ZDS_FP32) {
        x = reinterpret_cast<const float *>(sgf)[t];
      } else {
        const uint32_t b = reinterpret_cast<const uint16_t *>(sg16)[t];
        x = GD == ZDS_BF16 ? __uint_as_float(b << 16) : __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
      }
      float p = fp[t], m = fm[t], v = fv[t];
      adam_elem(x, c, p, m, v);
      fp[t] = p;
      fm[t] = m;
      fv[t] = v;
      if (WRITE_OUT) reinterpret_cast<uint16_t *>(so16)[t] = narrow1<PD>(p);
    }
    __syncthreads();
    if (w < 6) {
      if (q < quads) st_stream(reinterpret_cast<f32x4 *>(arr) + q, sf[w >> 1][half]);
    } else if (WRITE_OUT && w == 7) {
      if (o < octs) st_stream(static_cast<u32x4 *>(a.out) + o, so16[lane]);
    }
  }
  // Ragged tail: the last n % 8 elements, one per lane of block 0.
  if (blockIdx.x == 0 && nv + threadIdx.x < a.n) {
    const int64_t e = nv + threadIdx.x;
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

// Element-wise path for buffers without the vector alignment.
template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(ZDS_ADAM_BLOCK) adam_scalar_kernel(AdamArgs a) {
  if (a.sc->overflow) return;
  const ElemConsts c = load_consts(a);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ZDS_ADAM_BLOCK;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * ZDS_ADAM_BLOCK + threadIdx.x; e < a.n;
       e += stride) {
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

// Derives the step constants for t = state.t + 1 into the scalars struct.
__global__ void __launch_bounds__(64) adam_prep_kernel(zds_adamw_hparams hp, const zds_step_state *state,
                                                       zds_step_scalars *sc) {
  if (threadIdx.x != 0) return;
  const AdamConsts c = adam_constants(hp, state->beta1_pow, state->beta2_pow);
  sc->step_size = c.step_size;
  sc->bc2_sqrt = c.bc2_sqrt;
  sc->decay = c.decay;
  sc->one_minus_beta1 = c.omb1;
  sc->one_minus_beta2 = c.omb2;
}

// Blocks of `kernel` that fit on one CU at once (queried once per kernel).
template <typename K>
static int resident_blocks_per_cu(K kernel) {
  static int cached = 0;
  if (cached == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, ZDS_ADAM_BLOCK, 0) != hipSuccess || nb < 1)
      nb = 1;
    cached = nb;
  }
  return cached;
}

static int64_t round8(int64_t g) { return ZDS_ADAM_XCD ? ((g + 7) / 8) * 8 : g; }

template <int GD, int PD, bool WO>
static void launch_one(bool vec, bool vec16, hipStream_t s, const AdamArgs &a) {
  if (vec16 && ZDS_ADAM_TILE) {
    // One block per ZDS_ADAM_TPB tiles up to max_blocks(512); larger arrays loop.
    int64_t g = round8((((a.n & ~int64_t(7)) + 511) / 512 + ZDS_ADAM_TPB - 1) / ZDS_ADAM_TPB);
    if (g < 8) g = 8;
    if (g > max_blocks(512)) g = max_blocks(512) & ~int64_t(7);
    if (g > ZDS_ADAM_TILE_GRID) g = ZDS_ADAM_TILE_GRID;
    hipLaunchKernelGGL((adam_wide_kernel<GD, PD, WO>), dim3(static_cast<uint32_t>(g)), dim3(512), 0, s, a);
  } else if (vec && ZDS_ADAM_TILE) {
    // One block per tile up to max_blocks(256) (a dispatch holds fewer than 2^32
    // work-items); larger arrays loop over the tiles.
    int64_t g = round8((((a.n >> 2) + 63) / 64 + ZDS_ADAM_TPB - 1) / ZDS_ADAM_TPB);
    if (g < 8) g = 8;
    if (g > max_blocks(256)) g = max_blocks(256) & ~int64_t(7);
    if (g > ZDS_ADAM_TILE_GRID) g = ZDS_ADAM_TILE_GRID;
    hipLaunchKernelGGL((adam_tile_kernel<GD, PD, WO>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a);
  } else if (vec) {
    const int64_t span = static_cast<int64_t>(ZDS_ADAM_BLOCK) * ZDS_ADAM_QUADS;
    int64_t tiles = ((a.n >> 2) + span - 1) / span;
    if (tiles < 1) tiles = 1;
    int64_t g = tiles;
    if (ZDS_ADAM_PERSIST > 0) {
      int64_t cap = static_cast<int64_t>(device_cu_count()) * ZDS_ADAM_PERSIST * 64 / ZDS_ADAM_BLOCK;
      const int64_t res = static_cast<int64_t>(device_cu_count()) *
                          resident_blocks_per_cu(adam_quad_kernel<GD, PD, WO>);
      if (cap > res) cap = res;
      if (g > cap) g = cap;
    }
    g = round8(g);
    if (g > max_blocks(ZDS_ADAM_BLOCK)) g = max_blocks(ZDS_ADAM_BLOCK) & ~int64_t(7);
    hipLaunchKernelGGL((adam_quad_kernel<GD, PD, WO>), dim3(static_cast<uint32_t>(g)), dim3(ZDS_ADAM_BLOCK),
                       0, s, a);
  } else {
    int64_t g = (a.n + ZDS_ADAM_BLOCK - 1) / ZDS_ADAM_BLOCK;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) *
                        resident_blocks_per_cu(adam_scalar_kernel<GD, PD, WO>);
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    hipLaunchKernelGGL((adam_scalar_kernel<GD, PD, WO>), dim3(static_cast<uint32_t>(g)), dim3(ZDS_ADAM_BLOCK),
                       0, s, a);
  }
}

template <int GD>
static void launch_gd(zds_dtype pdt, bool wo, bool vec, bool vec16, hipStream_t s, const AdamArgs &a) {
  if (!wo) {
    launch_one<GD, ZDS_FP16, false>(vec, vec16, s, a);
  } else if (pdt == ZDS_BF16) {
    launch_one<GD, ZDS_BF16, true>(vec, vec16, s, a);
  } else {
    launch_one<GD, ZDS_FP16, true>(vec, vec16, s, a);
  }
}

zds_status launch_adam(const zds_adamw_hparams &hp, const void *grads, zds_dtype gdt, float *master,
                       float *m, float *v, void *out, zds_dtype pdt, int64_t n, zds_step_scalars *scalars,
                       const zds_step_state *state, hipStream_t stream) {
  hipLaunchKernelGGL(adam_prep_kernel, dim3(1), dim3(64), 0, stream, hp, state, scalars);
  zds_status st = check_launch("adam_step constants kernel");
  if (st != ZDS_OK) return st;
  AdamArgs a{grads, master, m, v, out, n, hp.beta1, hp.beta2, hp.eps, scalars};
  const bool vec = aligned(grads, gdt == ZDS_FP32 ? 16 : 8) && aligned(master, 16) && aligned(m, 16) &&
                   aligned(v, 16) && (out == nullptr || aligned(out, 8));
  const bool vec16 = vec && aligned(grads, 16) && (out == nullptr || aligned(out, 16));
  switch (gdt) {
    case ZDS_FP16: launch_gd<ZDS_FP16>(pdt, out != nullptr, vec, vec16, stream, a); break;
    case ZDS_BF16: launch_gd<ZDS_BF16>(pdt, out != nullptr, vec, vec16, stream, a); break;
    default: launch_gd<ZDS_FP32>(pdt, out != nullptr, vec, vec16, stream, a); break;
  }
  return check_launch("adam_step kernel");
}

}  // namespace zds
