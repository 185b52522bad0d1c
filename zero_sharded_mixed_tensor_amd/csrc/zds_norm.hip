// Row a2: overflow flag + global L2 norm + clip/unscale factor, two stages.
//
// Overflow of fp16 grads under the loss scale has to be caught before the
// update, and the scale lowered (devpress.csdn.net DeepSpeed tutorial §2.2,
// loss scaling). The global-norm clip is the conventional one.
//
// Stage 1 streams the grads once (2 B/element for 16-bit, 4 B for the fp32
// accumulator) and forms float64 partial sums of x^2: every 16-bit or fp32
// value squares exactly in float64, so each element costs one exact
// convert and one fma(x, x, acc) == acc + x^2. The wave sum uses DPP
// (quad_perm and row_ror) inside each 16-lane row and readlane across the four
// rows; waves meet in LDS; one partial per block. Stage 2 is one block that
// adds the partials in index order and derives the scalars. The grid is a
// fixed function of n, so the summation order, and the result, are the same
// on every call.
//
// The overflow flag comes from the sum itself: a square of a finite 16-bit or
// fp32 value is at most 2^256, so a sum of fewer than 2^63 of them stays far
// below the float64 maximum, while an inf or NaN element makes the sum inf or
// NaN (squares are never negative, so inf - inf cannot occur). Hence the sum
// is finite exactly when every element is.
#include "zds_device.h"
#include "zds_internal.h"

#ifndef ZDS_NORM_BLOCK
#define ZDS_NORM_BLOCK 256
#endif
#ifndef ZDS_NORM_MAX_GRID
#define ZDS_NORM_MAX_GRID 2048
#endif

namespace zds {

static_assert(ZDS_NORM_BLOCK % 64 == 0, "block is whole waves");

template <int D>
__device__ __forceinline__ double sq_acc(float x, double acc) {
  const double d = static_cast<double>(x);
  return fma(d, d, acc);
}

template <int D, bool VEC>
__global__ void __launch_bounds__(ZDS_NORM_BLOCK) norm_stage1(const void *x, int64_t n, double *partials) {
  double acc0 = 0.0, acc1 = 0.0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ZDS_NORM_BLOCK;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * ZDS_NORM_BLOCK + threadIdx.x;
  int64_t done = 0;
  if constexpr (VEC && D == ZDS_FP32) {
    // fp32: one 16-byte quad per lane, lane-contiguous
    const int64_t quads = n >> 2;
    for (int64_t i = tid; i < quads; i += stride) {
      float v[4];
      load_quad<D>(x, i, v);
      acc0 = sq_acc<D>(v[0], acc0);
      acc1 = sq_acc<D>(v[1], acc1);
      acc0 = sq_acc<D>(v[2], acc0);
      acc1 = sq_acc<D>(v[3], acc1);
    }
    done = quads << 2;
    if (blockIdx.x == 0 && done + threadIdx.x < n) acc0 = sq_acc<D>(widen1<D>(x, done + threadIdx.x), acc0);
  } else if constexpr (VEC) {
    // 16-bit: 8 elements (16 bytes) per lane, lane-contiguous
    const int64_t groups = n >> 3;
    for (int64_t i = tid; i < groups; i += stride) {
      float v[8];
      load8<D>(x, i, v);
      acc0 = sq_acc<D>(v[0], acc0);
      acc1 = sq_acc<D>(v[1], acc1);
      acc0 = sq_acc<D>(v[2], acc0);
      acc1 = sq_acc<D>(v[3], acc1);
      acc0 = sq_acc<D>(v[4], acc0);
      acc1 = sq_acc<D>(v[5], acc1);
      acc0 = sq_acc<D>(v[6], acc0);
      acc1 = sq_acc<D>(v[7], acc1);
    }
    done = groups << 3;
    if (blockIdx.x == 0 && done + threadIdx.x < n) acc0 = sq_acc<D>(widen1<D>(x, done + threadIdx.x), acc0);
  } else {
    for (int64_t e = tid; e < n; e += stride) acc0 = sq_acc<D>(widen1<D>(x, e), acc0);
  }
  const double b = block_sum<ZDS_NORM_BLOCK>(acc0 + acc1);
  if (threadIdx.x == 0) partials[blockIdx.x] = b;
}

__global__ void __launch_bounds__(ZDS_NORM_BLOCK) norm_stage2(const double *partials, int64_t nparts,
                                                               const zds_step_state *state,
                                                               int32_t accum_steps, float max_norm,
                                                               zds_step_scalars *out) {
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < nparts; i += ZDS_NORM_BLOCK) acc += partials[i];
  const double total = block_sum<ZDS_NORM_BLOCK>(acc);
  if (threadIdx.x == 0) {
    zds_step_scalars s = {};
    clip_scalars(total, state->scale, accum_steps, max_norm, s);
    *out = s;
  }
}

int norm_grid(int64_t n) {
  const int64_t per_block = static_cast<int64_t>(ZDS_NORM_BLOCK) * 8 * 4;
  int64_t g = (n + per_block - 1) / per_block;
  if (g > ZDS_NORM_MAX_GRID) g = ZDS_NORM_MAX_GRID;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

template <int D>
static void launch_d(bool vec, int grid, hipStream_t s, const void *x, int64_t n, double *partials) {
  if (vec)
    hipLaunchKernelGGL((norm_stage1<D, true>), dim3(grid), dim3(ZDS_NORM_BLOCK), 0, s, x, n, partials);
  else
    hipLaunchKernelGGL((norm_stage1<D, false>), dim3(grid), dim3(ZDS_NORM_BLOCK), 0, s, x, n, partials);
}

zds_status launch_norm(const void *grads, zds_dtype dtype, int64_t n, int32_t accum_steps,
                       float max_norm, const zds_step_state *state, zds_step_scalars *out,
                       double *partials, hipStream_t stream) {
  const int grid = norm_grid(n);
  const bool vec = aligned(grads, 16);
  switch (dtype) {
    case ZDS_FP16: launch_d<ZDS_FP16>(vec, grid, stream, grads, n, partials); break;
    case ZDS_BF16: launch_d<ZDS_BF16>(vec, grid, stream, grads, n, partials); break;
    default: launch_d<ZDS_FP32>(vec, grid, stream, grads, n, partials); break;
  }
  zds_status st = check_launch("overflow_and_norm stage 1");
  if (st != ZDS_OK) return st;
  return launch_norm_stage2(partials, grid, state, accum_steps, max_norm, out, stream);
}

// Block b adds partials [b*kReduceSpan, (b+1)*kReduceSpan) in a fixed order.
constexpr int64_t kReduceSpan = 8 * ZDS_NORM_BLOCK;

__global__ void __launch_bounds__(ZDS_NORM_BLOCK) norm_reduce(const double *in, int64_t n, double *out) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kReduceSpan;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t i = base + k * ZDS_NORM_BLOCK + threadIdx.x;
    if (i < n) acc += in[i];
  }
  const double b = block_sum<ZDS_NORM_BLOCK>(acc);
  if (threadIdx.x == 0) out[blockIdx.x] = b;
}

int64_t partials_workspace_doubles(int64_t nparts) {
  int64_t total = nparts;
  for (int64_t k = nparts; k > kReduceSpan; k = (k + kReduceSpan - 1) / kReduceSpan)
    total += (k + kReduceSpan - 1) / kReduceSpan;
  return total;
}

// Many partials (one per block of a one-block-per-chunk kernel) are first
// folded kReduceSpan at a time by parallel blocks, in index order, into the
// workspace after them; the last level goes to the single-block stage 2.
zds_status launch_norm_stage2(double *partials, int64_t nparts, const zds_step_state *state,
                              int32_t accum_steps, float max_norm, zds_step_scalars *out,
                              hipStream_t stream) {
  double *p = partials;
  double *next = partials + nparts;
  int64_t k = nparts;
  while (k > kReduceSpan) {
    const int64_t blocks = (k + kReduceSpan - 1) / kReduceSpan;
    hipLaunchKernelGGL(norm_reduce, dim3(static_cast<uint32_t>(blocks)), dim3(ZDS_NORM_BLOCK), 0, stream, p, k,
                       next);
    zds_status st = check_launch("overflow_and_norm partial reduction");
    if (st != ZDS_OK) return st;
    p = next;
    next += blocks;
    k = blocks;
  }
  hipLaunchKernelGGL(norm_stage2, dim3(1), dim3(ZDS_NORM_BLOCK), 0, stream, p, k, state, accum_steps, max_norm,
                     out);
  return check_launch("overflow_and_norm stage 2");
}

}  // namespace zds
