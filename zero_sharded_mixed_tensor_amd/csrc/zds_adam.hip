// Row a4: fused AdamW + unscale/clip + cast on the rank's fp32 master shard.
//
// The update runs on the fp32 master copy while params and grads are 16-bit
// (devpress.csdn.net DeepSpeed tutorial §2.2; aiqz.cc "DeepSpeed ZeRO引擎深入",
// 混合精度); AdamW with betas, eps and weight decay (same tutorial §3.2
// optimizer block); the two moment recurrences as in aiqz.cc's Python 演示.
//
// Memory-bound stream, no MFMA: per element it reads the grad (2 or 4 B) and
// master/m/v (12 B) and writes master/m/v (12 B) and the 16-bit param (2 B):
// 28 B (16-bit grads) or 30 B (fp32 accumulator). Each thread owns groups of
// 8 consecutive elements, so every access is a 16-byte global load/store
// (two per fp32 group); UNROLL groups are loaded before any is computed to
// keep enough bytes in flight per CU. The grid is a fixed multiple of the CU
// count and strides over the groups.
#include "zds_device.h"
#include "zds_internal.h"

#ifndef ZDS_ADAM_UNROLL
#define ZDS_ADAM_UNROLL 2
#endif
#ifndef ZDS_ADAM_BLOCK
#define ZDS_ADAM_BLOCK 256
#endif
#ifndef ZDS_ADAM_WAVES_PER_CU
#define ZDS_ADAM_WAVES_PER_CU 32
#endif

namespace zds {

struct AdamArgs {
  const void *g;
  float *p;
  float *m;
  float *v;
  void *out;
  int64_t n;
  zds_adamw_hparams hp;
  const zds_step_scalars *scalars;
  const zds_step_state *state;
};

// One element, fp32, one rounding per operation, in this order.
__device__ __forceinline__ void adam_elem(float x, float gs, const AdamConsts &c, float &p, float &m,
                                          float &v) {
  const float g = x * gs;
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float denom = sqrtf(v) / c.bc2_sqrt + c.eps;
  p = p * c.decay;
  p = p - c.step_size * (m / denom);
}

template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(ZDS_ADAM_BLOCK) adam_vec_kernel(AdamArgs a) {
  // Skip on overflow without a host round trip; the flag is uniform.
  if (a.scalars->overflow) return;
  const float gs = a.scalars->grad_scale;
  const AdamConsts c = adam_constants(a.hp, a.state->beta1_pow, a.state->beta2_pow);

  const int64_t groups = a.n >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ZDS_ADAM_BLOCK;
  int64_t i = static_cast<int64_t>(blockIdx.x) * ZDS_ADAM_BLOCK + threadIdx.x;

  constexpr int U = ZDS_ADAM_UNROLL;
  for (; i + (U - 1) * stride < groups; i += U * stride) {
    float x[U][8], p[U][8], m[U][8], v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t gi = i + u * stride;
      load8<GD>(a.g, gi, x[u]);
      load8f(a.p, gi, p[u]);
      load8f(a.m, gi, m[u]);
      load8f(a.v, gi, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) adam_elem(x[u][k], gs, c, p[u][k], m[u][k], v[u][k]);
      const int64_t gi = i + u * stride;
      store8f(a.p, gi, p[u]);
      store8f(a.m, gi, m[u]);
      store8f(a.v, gi, v[u]);
      if (WRITE_OUT) store8h<PD>(a.out, gi, p[u]);
    }
  }
  for (; i < groups; i += stride) {
    float x[8], p[8], m[8], v[8];
    load8<GD>(a.g, i, x);
    load8f(a.p, i, p);
    load8f(a.m, i, m);
    load8f(a.v, i, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) adam_elem(x[k], gs, c, p[k], m[k], v[k]);
    store8f(a.p, i, p);
    store8f(a.m, i, m);
    store8f(a.v, i, v);
    if (WRITE_OUT) store8h<PD>(a.out, i, p);
  }
  // Ragged tail: the last n % 8 elements, one per thread of block 0.
  const int64_t tail0 = groups << 3;
  if (blockIdx.x == 0 && tail0 + threadIdx.x < a.n) {
    const int64_t e = tail0 + threadIdx.x;
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), gs, c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

// Element-wise path for buffers that are not 16-byte aligned.
template <int GD, int PD, bool WRITE_OUT>
__global__ void __launch_bounds__(ZDS_ADAM_BLOCK) adam_scalar_kernel(AdamArgs a) {
  if (a.scalars->overflow) return;
  const float gs = a.scalars->grad_scale;
  const AdamConsts c = adam_constants(a.hp, a.state->beta1_pow, a.state->beta2_pow);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ZDS_ADAM_BLOCK;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * ZDS_ADAM_BLOCK + threadIdx.x; e < a.n;
       e += stride) {
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adam_elem(widen1<GD>(a.g, e), gs, c, p, m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (WRITE_OUT) static_cast<uint16_t *>(a.out)[e] = narrow1<PD>(p);
  }
}

template <int GD, int PD, bool WO>
static void launch_one(bool vec, int grid, hipStream_t s, const AdamArgs &a) {
  if (vec)
    hipLaunchKernelGGL((adam_vec_kernel<GD, PD, WO>), dim3(grid), dim3(ZDS_ADAM_BLOCK), 0, s, a);
  else
    hipLaunchKernelGGL((adam_scalar_kernel<GD, PD, WO>), dim3(grid), dim3(ZDS_ADAM_BLOCK), 0, s, a);
}

template <int GD>
static void launch_gd(zds_dtype pdt, bool wo, bool vec, int grid, hipStream_t s, const AdamArgs &a) {
  if (!wo) {
    launch_one<GD, ZDS_FP16, false>(vec, grid, s, a);
  } else if (pdt == ZDS_BF16) {
    launch_one<GD, ZDS_BF16, true>(vec, grid, s, a);
  } else {
    launch_one<GD, ZDS_FP16, true>(vec, grid, s, a);
  }
}

zds_status launch_adam(const zds_adamw_hparams &hp, const void *grads, zds_dtype gdt, float *master,
                       float *m, float *v, void *out, zds_dtype pdt, int64_t n,
                       const zds_step_scalars *scalars, const zds_step_state *state,
                       hipStream_t stream) {
  AdamArgs a{grads, master, m, v, out, n, hp, scalars, state};
  const bool vec = aligned(grads, 16) && aligned(master, 16) && aligned(m, 16) && aligned(v, 16) &&
                   (out == nullptr || aligned(out, 16));
  const int64_t items = vec ? (n >> 3) : n;
  const int64_t per_block = static_cast<int64_t>(ZDS_ADAM_BLOCK) * (vec ? ZDS_ADAM_UNROLL : 1);
  int64_t blocks = (items + per_block - 1) / per_block;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * ZDS_ADAM_WAVES_PER_CU * 64 / ZDS_ADAM_BLOCK;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const int grid = static_cast<int>(blocks);
  const bool wo = out != nullptr;
  switch (gdt) {
    case ZDS_FP16: launch_gd<ZDS_FP16>(pdt, wo, vec, grid, stream, a); break;
    case ZDS_BF16: launch_gd<ZDS_BF16>(pdt, wo, vec, grid, stream, a); break;
    default: launch_gd<ZDS_FP32>(pdt, wo, vec, grid, stream, a); break;
  }
  return check_launch("adam_step kernel");
}

}  // namespace zds
