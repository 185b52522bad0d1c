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
// adds the partials in index order and derives the scalars. Each block of
// stage 1 reads one contiguous unit of kNormUnitBytes (every load of
// a whole unit issued before the sums, a unit per block as long as the grid
// allows), and its partial is that unit's sum in a fixed order, so the
// summation order, and the result, are the same on every call. (A grid of at
// most 2048 blocks striding over the array ran the 7B shard's bf16 grads at
// 6.3 TB/s; strided streams lose on this memory system.)
//
// The overflow flag comes from the sum itself: a square of a finite 16-bit or
// fp32 value is at most 2^256, so a sum of fewer than 2^63 of them stays far
// below the float64 maximum, while an inf or NaN element makes the sum inf or
// NaN (squares are never negative, so inf - inf cannot occur). Hence the sum
// is finite exactly when every element is.
#include "zds_device.h"
#include "zds_internal.h"

namespace zds {

constexpr int kNormBlock = 256;
// Bytes per block in the vector paths: 2 accesses of 16 bytes per lane
// (4096 16-bit or 2048 fp32 elements).
constexpr int64_t kNormUnitBytes = 8192;
static_assert(kNormBlock % 64 == 0, "block is whole waves");

template <int D>
__device__ __forceinline__ double sq_acc(float x, double acc) {
  const double d = static_cast<double>(x);
  return fma(d, d, acc);
}

// Loads UPT vector groups of a unit (lane-contiguous per access) and adds
// their squares; FULL: the whole unit is in range, so no load is guarded.
// 16-bit grads: the loads issue back to back. fp32: each wave has one load
// in flight at a time (an explicit wait after each but the last), which the
// fp32 accumulator reads faster (C3's 842M-element accumulator, library
// builds swapped between bench runs, three rounds: 0.477-0.478 ms against
// 0.503-0.507 back to back; the 16-bit grads the other way round, 0.247-0.250
// back to back against 0.266-0.268).
template <int D, int UPT, bool FULL>
__device__ __forceinline__ void unit_sumsq(const void *x, int64_t base, int64_t groups, double &acc0, double &acc1) {
  constexpr int PER = D == ZDS_FP32 ? 4 : 8;
  float v[UPT][PER];
#pragma unroll
  for (int r = 0; r < UPT; ++r) {
    const int64_t i = base + r * kNormBlock;
    if (FULL || i < groups) {
      if constexpr (D == ZDS_FP32) load_quad<D>(x, i, v[r]);
      else load8<D>(x, i, v[r]);
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) v[r][j] = 0.0f;
    }
    // vmcnt(0), expcnt and lgkmcnt left at their maxima (GFX9 encoding)
    if (D == ZDS_FP32 && r + 1 < UPT) __builtin_amdgcn_s_waitcnt(0x0F70);
  }
#pragma unroll
  for (int r = 0; r < UPT; ++r) {
#pragma unroll
    for (int j = 0; j < PER; j += 2) {
      acc0 = sq_acc<D>(v[r][j], acc0);
      acc1 = sq_acc<D>(v[r][j + 1], acc1);
    }
  }
}

template <int D>
constexpr int64_t norm_unit() { return kNormUnitBytes / (D == ZDS_FP32 ? 4 : 2); }

template <int D, bool VEC>
__global__ void __launch_bounds__(kNormBlock) norm_stage1(const void *x, int64_t n, double *partials) {
  double acc0 = 0.0, acc1 = 0.0;
  if constexpr (VEC) {
    // lane-contiguous 16-byte accesses: fp32 quads or 8 16-bit elements
    constexpr int PER = D == ZDS_FP32 ? 4 : 8;
    constexpr int UPT = static_cast<int>(norm_unit<D>() / PER / kNormBlock);
    static_assert(UPT >= 1 && UPT * PER * kNormBlock == norm_unit<D>(), "a unit is whole accesses");
    const int64_t groups = n / PER;
    const int64_t units = (groups + UPT * kNormBlock - 1) / (UPT * kNormBlock);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {  // uniform per block
      const int64_t first = u * UPT * kNormBlock;
      if (first + UPT * kNormBlock <= groups)
        unit_sumsq<D, UPT, true>(x, first + threadIdx.x, groups, acc0, acc1);
      else
        unit_sumsq<D, UPT, false>(x, first + threadIdx.x, groups, acc0, acc1);
    }
    const int64_t done = groups * PER;
    if (blockIdx.x == 0 && done + threadIdx.x < n) acc0 = sq_acc<D>(widen1<D>(x, done + threadIdx.x), acc0);
  } else {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kNormBlock;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kNormBlock + threadIdx.x; e < n; e += stride)
      acc0 = sq_acc<D>(widen1<D>(x, e), acc0);
  }
  const double b = block_sum<kNormBlock>(acc0 + acc1);
  if (threadIdx.x == 0) partials[blockIdx.x] = b;
}

__global__ void __launch_bounds__(kNormBlock) norm_stage2(const double *partials, int64_t nparts,
                                                               const zds_step_state *state,
                                                               int32_t accum_steps, float max_norm,
                                                               zds_step_scalars *out) {
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < nparts; i += kNormBlock) acc += partials[i];
  const double total = block_sum<kNormBlock>(acc);
  if (threadIdx.x == 0) {
    zds_step_scalars s = {};
    clip_scalars(total, state->scale, accum_steps, max_norm, s);
    *out = s;
  }
}

static int grid_for(int64_t n, int64_t unit) {
  int64_t g = (n + unit - 1) / unit;
  if (g > max_blocks(kNormBlock)) g = max_blocks(kNormBlock);
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

// The most blocks (partials) stage 1 uses for n elements of any dtype.
int norm_grid(int64_t n) { return grid_for(n, norm_unit<ZDS_FP32>()); }

template <int D>
static int launch_d(bool vec, hipStream_t s, const void *x, int64_t n, double *partials) {
  const int grid = grid_for(n, norm_unit<D>());
  if (vec)
    hipLaunchKernelGGL((norm_stage1<D, true>), dim3(grid), dim3(kNormBlock), 0, s, x, n, partials);
  else
    hipLaunchKernelGGL((norm_stage1<D, false>), dim3(grid), dim3(kNormBlock), 0, s, x, n, partials);
  return grid;
}

zds_status launch_norm(const void *grads, zds_dtype dtype, int64_t n, int32_t accum_steps,
                       float max_norm, const zds_step_state *state, zds_step_scalars *out,
                       double *partials, hipStream_t stream) {
  const bool vec = aligned(grads, 16);
  int grid;
  switch (dtype) {
    case ZDS_FP16: grid = launch_d<ZDS_FP16>(vec, stream, grads, n, partials); break;
    case ZDS_BF16: grid = launch_d<ZDS_BF16>(vec, stream, grads, n, partials); break;
    default: grid = launch_d<ZDS_FP32>(vec, stream, grads, n, partials); break;
  }
  zds_status st = check_launch("overflow_and_norm stage 1");
  if (st != ZDS_OK) return st;
  return launch_norm_stage2(partials, grid, state, accum_steps, max_norm, out, stream);
}

// Block b adds partials [b*kReduceSpan, (b+1)*kReduceSpan) in a fixed order.
constexpr int64_t kReduceSpan = 8 * kNormBlock;

__global__ void __launch_bounds__(kNormBlock) norm_reduce(const double *in, int64_t n, double *out) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kReduceSpan;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t i = base + k * kNormBlock + threadIdx.x;
    if (i < n) acc += in[i];
  }
  const double b = block_sum<kNormBlock>(acc);
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
    hipLaunchKernelGGL(norm_reduce, dim3(static_cast<uint32_t>(blocks)), dim3(kNormBlock), 0, stream, p, k,
                       next);
    zds_status st = check_launch("overflow_and_norm partial reduction");
    if (st != ZDS_OK) return st;
    p = next;
    next += blocks;
    k = blocks;
  }
  hipLaunchKernelGGL(norm_stage2, dim3(1), dim3(kNormBlock), 0, stream, p, k, state, accum_steps, max_norm,
                     out);
  return check_launch("overflow_and_norm stage 2");
}

}  // namespace zds
