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
// out), and the pieces meet in LDS where every thread updates its elements.
// Against a kernel in which each lane moves all arrays of its own 4 elements,
// this lowers the memory footprint per wave from 4 loads + 4 stores to 1 + 1
// and raised the pass from about 5.8 to 6.0 TB/s on the 7B shard.
//
// The default is adam_wide_kernel: 8 waves and one 1024-element tile per
// block, the grid one block per tile, so the dispatcher keeps every CU full
// with short-lived blocks that each stream one contiguous piece of every
// array. Each wave moves its part of the tile as 1 KiB accesses (16 bytes per
// lane) and issues the next only after the previous one has completed, for
// its loads and for its stores: this memory system rewards many waves with
// one access each in flight. The tile's two halves are pipelined: the second
// half's loads are in flight while the first half is updated, and the first
// half's stores while the second half is updated, so the arithmetic is hidden
// behind the memory accesses. Measured on the 7B shard, library builds swapped
// between bench runs, three rounds on one box: 3.609-3.616 ms (0.815-0.817 of
// 8 TB/s) against 3.696-3.701 for the same tile without the pipelining and
// 3.720-3.724 for the kernel before (2 consecutive 512-element tiles per
// block, one 1 KiB access per wave per tile). In probes (bit-exact), the
// pipelined kernel ran as fast as the unpipelined one with the arithmetic left
// out; a wave's two accesses back to back, or only its loads or only its
// stores one at a time, were slower than the 2-tile kernel (-0.7, -2.0,
// -2.9 %), and so were 2048-element tiles (4 accesses per wave, -1.6 %).
// 16-bit buffers that are 8- but not 16-byte aligned take the same kernel
// with 8-byte 16-bit accesses (two 512-byte wave accesses per half tile;
// wave 7's two loads of the second half are in flight together); that form
// replaced a 4-wave kernel with 256-element tiles. The
// wave's role index is made wave-uniform (readfirstlane), so role branches,
// array bases and tile counters are scalar.
//
// The update's instruction count showed in the bandwidth of the earlier,
// unpipelined kernels, where a block's update phase was time with nothing in
// flight. Two measures came from that and are kept. (1) The division by the
// per-step constant sqrt(1 - beta2^t) is a float64 multiplication by its
// float64 reciprocal, rounded to fp32 (3 instructions instead of the 11 of a
// correctly rounded fp32 divide), +2.2 % on the 7B shard then; it gives the
// correctly rounded quotient for every input, see adam_elem. (2) The waves
// raise their scheduling priority while they issue loads and stores and drop
// it for the update, so that a block's memory accesses are not queued behind
// other blocks' arithmetic on the same SIMD: +0.3 to 1 % in four A/B runs
// then, neutral to -0.3 % on the unpipelined 1024-element tile and neutral on
// the pipelined one (3.623-3.626 ms against 3.623-3.628 without it, four
// rounds on one box).
//
// The step constants (lr / (1 - beta1^t), sqrt(1 - beta2^t) and its float64
// reciprocal, 1 - lr*wd, the 1 - beta values) are derived once per call by a
// single-wave prep kernel into the caller's step-scalars struct, so the
// update kernel only loads them. (Deriving them in every block instead, by
// one wave while its loads are in flight, measured 0.4 % slower.)
#include "zds_device.h"
#include "zds_internal.h"

namespace {
// Threads per block of the element-wise kernel.
constexpr int kScalarBlock = 256;
// Upper bound on the tile kernel's grid (blocks loop over the tiles beyond it).
constexpr int64_t kTileGridCap = int64_t(1) << 23;
}  // namespace

namespace zds {

// The arguments of every update kernel; every other scalar of the update
// comes from the step-scalars struct, read once per block with one batch of
// scalar loads. (A kernel argument loaded in the same batch as the struct's
// fields made the compiler reuse a register still being loaded and wait for
// the whole batch in between: a second round trip before a block's first
// access, 1 % of the pass. Passing the 64-bit pointers and size as separate
// arguments, preloaded into SGPRs at wave launch, measured no faster.)
struct AdamArgs {
  const zds_step_scalars *sc;
  const void *g;
  float *p;
  float *m;
  float *v;
  void *out;
  int64_t n;
};

struct ElemConsts {
  float b1, b2, omb1, omb2, eps, step_size, decay, gs;
  double inv_bc2;
};

// 1 - beta is formed here in fp32, as the step's definition does (one fp32
// subtraction; exact for beta in [0.5, 1]).
__device__ __forceinline__ ElemConsts load_consts(const zds_step_scalars *sc) {
  ElemConsts c;
  c.b1 = sc->beta1;
  c.b2 = sc->beta2;
  c.eps = sc->eps;
  c.omb1 = 1.0f - c.b1;
  c.omb2 = 1.0f - c.b2;
  c.step_size = sc->step_size;
  c.inv_bc2 = sc->inv_bc2_sqrt;
  c.decay = sc->decay;
  c.gs = sc->grad_scale;
  return c;
}

// One element, fp32, one rounding per operation, in this order.
//
// sqrt(v) / bc2 (bc2 = sqrt(1 - beta2^t) in fp32) is formed as
// fp32(float64(sqrt(v)) * r) with r = 1 / float64(bc2) correctly rounded.
// That is the correctly rounded fp32 quotient: r carries a relative error of
// at most 2^-53 and the float64 product another 2^-53, so the product is
// within 2^-52 (relatively) of the exact quotient; the exact quotient a/b of
// two fp32 numbers is never a point halfway between two fp32 numbers (a
// halfway point times b would need more than 24 significant bits), and lies at
// least 2^-49 (relatively) away from every such point, because
// |a - b*M| is a non-zero multiple of the coarser of a's and b*M's
// granularities. So no rounding boundary separates the product from the
// exact quotient. Here a = sqrt(v) is 0, NaN, inf or at least 2^-74.5, and
// the quotient stays in the normal range; bc2 = 0 (beta2 = 1) gives
// r = inf and the same inf / NaN as the division.
__device__ __forceinline__ void adam_elem(float x, const ElemConsts &c, float &p, float &m, float &v) {
  const float g = x * c.gs;
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float q = static_cast<float>(static_cast<double>(sqrtf(v)) * c.inv_bc2);
  const float denom = q + c.eps;
  p = p * c.decay;
  p = p - c.step_size * (m / denom);
}

// Scheduling priority of a wave: raised while it issues its loads and stores,
// lowered for the update.
__device__ __forceinline__ void memory_phase() { __builtin_amdgcn_s_setprio(3); }
__device__ __forceinline__ void update_phase() { __builtin_amdgcn_s_setprio(0); }

// Wide wave-specialised variant: one tile of 1024 elements per 8-wave block,
// in two halves of 512. Waves 0-1 move the master tile, 2-3 m, 4-5 v: wave w
// holds quarter (w & 1) of each half, one 1 KiB access per half. 16-bit
// grads: wave 6 loads the first half's (1 KiB), wave 7 the second half's, and
// the 16-bit params go out the same way; fp32 grads are moved by waves 6 and 7
// like a fourth fp32 array, and the params by wave 6 (first half) and 7.
// Each wave has one access in flight at a time, and the halves are pipelined
// so that the arithmetic overlaps the memory accesses:
//   load half 0 (and wait); issue the load of half 1      | barrier 1
//   update half 0 (each thread one element); store half 1's data in LDS
//                                                          | barrier 2
//   store half 0; update half 1; wait for the store         | barrier 3
//   store half 1
// Outside the update phases each wave writes and reads only its own part of
// the LDS tiles; the update of a half reads and writes only that half. The
// tiles cover the first n & ~7 elements; block 0 takes the rest element-wise.
// Whole tiles take a path without per-lane bounds checks (the test is uniform
// per block); only the last, partial tile checks each lane.
template <int GD>
struct WideTile {
  f32x4 sf[3][256];
  u32x4 sg16[128];
  u32x4 so16[128];
  __device__ f32x4 *sgf() { return sf[0]; }  // unused for 16-bit grads
};
template <>
struct WideTile<ZDS_FP32> {
  f32x4 sf[3][256];
  f32x4 sgf_[256];
  u32x4 so16[128];
  u32x4 sg16[1];
  __device__ f32x4 *sgf() { return sgf_; }
};

// Elements per tile of the wide kernel.
constexpr int kWideTile = 1024;

// Update of element h * 512 + threadIdx.x of the tile in LDS.
template <int GD, int PD, bool WRITE_OUT, bool FULL>
__device__ __forceinline__ void wide_update(const ElemConsts &c, WideTile<GD> &sh, int h, int64_t first, int64_t nv) {
  const int t = threadIdx.x + 512 * h;
  if (!FULL && first + t >= nv) return;
  float *fp = reinterpret_cast<float *>(sh.sf[0]);
  float *fm = reinterpret_cast<float *>(sh.sf[1]);
  float *fv = reinterpret_cast<float *>(sh.sf[2]);
  float x;
  if (GD == ZDS_FP32) {
    x = reinterpret_cast<const float *>(sh.sgf())[t];
  } else {
    const uint32_t b = reinterpret_cast<const uint16_t *>(sh.sg16)[t];
    x = GD == ZDS_BF16 ? __uint_as_float(b << 16) : __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
  }
  float p = fp[t], m = fm[t], v = fv[t];
  adam_elem(x, c, p, m, v);
  fp[t] = p;
  fm[t] = m;
  fv[t] = v;
  if (WRITE_OUT) reinterpret_cast<uint16_t *>(sh.so16)[t] = narrow1<PD>(p);
}

// The 16-bit accesses of the wide kernel: V16 = 16 bytes per lane (8
// elements; one 1 KiB wave access per half tile) when the 16-bit buffers are
// 16-byte aligned, else 8 bytes per lane (4 elements; two 512-byte wave
// accesses per half tile).
template <int V16>
struct Vec16 {
  typedef u32x4 T;
};
template <>
struct Vec16<8> {
  typedef u32x2 T;
};

// One tile. fp32 role (waves 0-5, and 6-7 for fp32 grads): `base` is this
// wave's array, `lt` its LDS tile. The quads of half h this wave moves are
// qa + 128 h (qa = 64 (w & 1) + lane). 16-bit role (waves 6 and 7): half
// (w & 1)'s grads and params, as V16-byte pieces j of the tile, j counted
// in units of V16 / 2 elements.
template <int GD, int PD, bool WRITE_OUT, bool FULL, int V16>
__device__ __forceinline__ void wide_tile(const AdamArgs &a, const ElemConsts &c, WideTile<GD> &sh, float *base, int w,
                                          uint32_t tile, int64_t nv) {
  typedef typename Vec16<V16>::T V;
  constexpr int E16 = V16 / 2;                 // 16-bit elements per piece
  constexpr int PH = 512 / E16;                // pieces per half tile: 64 (16 B) or 128 (8 B)
  const int lane = threadIdx.x & 63;
  const uint32_t qa = 64 * (w & 1) + lane;
  const int64_t first = static_cast<int64_t>(tile) * kWideTile;  // first element of the tile
  const int64_t quads = nv >> 2;
  const int64_t pieces = nv / E16;             // whole V16 pieces of the 16-bit arrays
  const int64_t p0 = first / E16;              // the tile's first piece
  V *sg = reinterpret_cast<V *>(sh.sg16);
  V *so = reinterpret_cast<V *>(sh.so16);
  const bool fp32_role = w < 6 || GD == ZDS_FP32;
  if (fp32_role) {
    f32x4 *lt = w < 6 ? sh.sf[w >> 1] : sh.sgf();
    float *tp = wave_uniform(base + first);
    const bool in0 = FULL || first / 4 + qa < quads;
    const bool in1 = FULL || first / 4 + qa + 128 < quads;
    memory_phase();
    if (in0) lt[qa] = ld_stream_at_once<f32x4>(tp, qa * 16);
    f32x4 b4;
    if (in1) b4 = ld_stream_global(reinterpret_cast<const f32x4 *>(tp) + qa + 128);
    update_phase();
    __syncthreads();
    wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 0, first, nv);
    if (in1) lt[qa + 128] = b4;
    __syncthreads();
    if (w < 6) {
      memory_phase();
      if (in0) st_stream_at(tp, qa * 16, lt[qa]);
      update_phase();
      wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 1, first, nv);
      wait_vmem();
      __syncthreads();
      memory_phase();
      if (in1) st_stream_at(tp, (qa + 128) * 16, lt[qa + 128]);
      update_phase();
      return;
    }
  } else if (w == 6) {  // 16-bit grads of half 0, one piece access at a time
    const uint16_t *tg = wave_uniform(static_cast<const uint16_t *>(a.g) + first);
    memory_phase();
#pragma unroll
    for (int k = 0; k < PH / 64; ++k) {
      const int j = 64 * k + lane;
      if (FULL || p0 + j < pieces) sg[j] = ld_stream_at_once<V>(tg, j * V16);
    }
    update_phase();
    __syncthreads();
    wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 0, first, nv);
    __syncthreads();
  } else {  // w == 7: 16-bit grads of half 1, in flight during the update of half 0
    const uint16_t *tg = wave_uniform(static_cast<const uint16_t *>(a.g) + first);
    memory_phase();
    V gb[PH / 64];
#pragma unroll
    for (int k = 0; k < PH / 64; ++k) {
      const int j = PH + 64 * k + lane;
      if (FULL || p0 + j < pieces) gb[k] = ld_stream_global(reinterpret_cast<const V *>(tg) + j);
    }
    update_phase();
    __syncthreads();
    wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 0, first, nv);
#pragma unroll
    for (int k = 0; k < PH / 64; ++k) {
      const int j = PH + 64 * k + lane;
      if (FULL || p0 + j < pieces) sg[j] = gb[k];
    }
    __syncthreads();
  }
  // waves 6 and 7 from barrier 2 on: 16-bit params of half 0 (wave 6) and
  // half 1 (wave 7), one piece access at a time
  uint16_t *to = wave_uniform(static_cast<uint16_t *>(a.out) + first);
  const int j0 = PH * (w & 1) + lane;
  if (w == 6) {
    memory_phase();
#pragma unroll
    for (int k = 0; k < PH / 64; ++k) {
      if (k > 0) wait_vmem();
      const int j = j0 + 64 * k;
      if (WRITE_OUT && (FULL || p0 + j < pieces)) st_stream_at(to, j * V16, so[j]);
    }
    update_phase();
    wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 1, first, nv);
    wait_vmem();
    __syncthreads();
  } else {
    wide_update<GD, PD, WRITE_OUT, FULL>(c, sh, 1, first, nv);
    __syncthreads();
    memory_phase();
#pragma unroll
    for (int k = 0; k < PH / 64; ++k) {
      if (k > 0) wait_vmem();
      const int j = j0 + 64 * k;
      if (WRITE_OUT && (FULL || p0 + j < pieces)) st_stream_at(to, j * V16, so[j]);
    }
    update_phase();
  }
}

template <int GD, int PD, bool WRITE_OUT, int V16>
__global__ void __launch_bounds__(512) adam_wide_kernel(const zds_step_scalars *__restrict__ sc,
                                                        const void *__restrict__ g, float *__restrict__ p,
                                                        float *__restrict__ m, float *__restrict__ v,
                                                        void *__restrict__ out, int64_t n) {
  __shared__ WideTile<GD> sh;
  const AdamArgs a{sc, g, p, m, v, out, n};
  // The role index is the same on every lane of a wave; read through
  // readfirstlane the compiler knows it, so role branches, array bases and
  // tile counters are scalar.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nv = n & ~int64_t(7);
  const uint32_t full = static_cast<uint32_t>(nv / kWideTile);  // whole tiles
  const uint32_t ntiles = static_cast<uint32_t>((nv + kWideTile - 1) / kWideTile);
  // the fp32 array this wave moves (waves 6-7: the fp32 grads, if any)
  float *base = w < 2 ? p : (w < 4 ? m : (w < 6 ? v : static_cast<float *>(const_cast<void *>(g))));
  if (sc->overflow) return;  // the step is skipped: uniform, nothing is touched
  const ElemConsts c = load_consts(sc);
  // One tile per block; a grid capped below the tile count loops. Every
  // tile ends with the last wave stores after barrier 3; the next tile's
  // loads write only the issuing wave's own LDS part, which no other wave
  // reads before that tile's barrier 1.
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {  // uniform per block
    if (tile < full)
      wide_tile<GD, PD, WRITE_OUT, true, V16>(a, c, sh, base, w, tile, nv);
    else
      wide_tile<GD, PD, WRITE_OUT, false, V16>(a, c, sh, base, w, tile, nv);
  }
  // Ragged tail: the last n % 8 elements, one per lane of block 0.
  if (blockIdx.x == 0 && nv + threadIdx.x < n) {
    const int64_t e = nv + threadIdx.x;
    float pe = p[e], me = m[e], ve = v[e];
    adam_elem(widen1<GD>(g, e), c, pe, me, ve);
    p[e] = pe;
    m[e] = me;
    v[e] = ve;
    if (WRITE_OUT) static_cast<uint16_t *>(out)[e] = narrow1<PD>(pe);
  }
}

// Element-wise path for buffers without the vector alignment.
template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(kScalarBlock) adam_scalar_kernel(const zds_step_scalars *__restrict__ sc,
                                                                  const void *__restrict__ g,
                                                                  float *__restrict__ p, float *__restrict__ m,
                                                                  float *__restrict__ v, void *__restrict__ out,
                                                                  int64_t n) {
  const AdamArgs a{sc, g, p, m, v, out, n};
  if (sc->overflow) return;
  const ElemConsts c = load_consts(sc);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kScalarBlock;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kScalarBlock + threadIdx.x; e < a.n;
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
  sc->inv_bc2_sqrt = c.inv_bc2_sqrt;
  sc->step_size = c.step_size;
  sc->bc2_sqrt = c.bc2_sqrt;
  sc->decay = c.decay;
  sc->beta1 = c.b1;
  sc->beta2 = c.b2;
  sc->eps = c.eps;
}

// Blocks of the element-wise kernel that fit on one CU at once (queried once
// per instantiation).
template <typename K>
static int resident_blocks_per_cu(K kernel) {
  static int cached = 0;
  if (cached == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kScalarBlock, 0) != hipSuccess || nb < 1)
      nb = 1;
    cached = nb;
  }
  return cached;
}

// One block per kWideTile elements, at most max_blocks(512) (a dispatch
// holds fewer than 2^32 work-items) and kTileGridCap; larger arrays loop
// over the tiles.
static uint32_t wide_grid(int64_t elems) {
  int64_t g = (elems + kWideTile - 1) / kWideTile;
  if (g < 1) g = 1;
  if (g > max_blocks(512)) g = max_blocks(512);
  if (g > kTileGridCap) g = kTileGridCap;
  return static_cast<uint32_t>(g);
}

template <int GD, int PD, bool WO>
static void launch_one(bool vec, bool vec16, hipStream_t s, const AdamArgs &a) {
  if (vec16) {
    hipLaunchKernelGGL((adam_wide_kernel<GD, PD, WO, 16>), dim3(wide_grid(a.n & ~int64_t(7))), dim3(512), 0, s,
                       a.sc, a.g, a.p, a.m, a.v, a.out, a.n);
  } else if (vec) {
    hipLaunchKernelGGL((adam_wide_kernel<GD, PD, WO, 8>), dim3(wide_grid(a.n & ~int64_t(7))), dim3(512), 0, s,
                       a.sc, a.g, a.p, a.m, a.v, a.out, a.n);
  } else {
    int64_t g = (a.n + kScalarBlock - 1) / kScalarBlock;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) *
                        resident_blocks_per_cu(adam_scalar_kernel<GD, PD, WO>);
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    hipLaunchKernelGGL((adam_scalar_kernel<GD, PD, WO>), dim3(static_cast<uint32_t>(g)), dim3(kScalarBlock),
                       0, s, a.sc, a.g, a.p, a.m, a.v, a.out, a.n);
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
  const AdamArgs a{scalars, grads, master, m, v, out, n};
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
