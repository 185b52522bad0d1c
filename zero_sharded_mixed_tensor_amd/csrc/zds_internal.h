// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "zds.h"

namespace zds {

// ---------------------------------------------------------------------------
// Error reporting (thread-local message behind zds_last_error()).
// ---------------------------------------------------------------------------
zds_status fail(zds_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
zds_status hip_fail(hipError_t e, const char *what);
zds_status check_launch(const char *what);
void clear_error();

// Number of compute units of the current device (cached per device).
int device_cu_count();

inline int dtype_size(zds_dtype d) { return d == ZDS_FP32 ? 4 : 2; }
inline bool valid_dtype(int d) { return d == ZDS_FP16 || d == ZDS_BF16 || d == ZDS_FP32; }
__host__ __device__ inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// ---------------------------------------------------------------------------
// Scalar logic, one definition for host and device.
// ---------------------------------------------------------------------------

struct AdamConsts {
  float b1, b2, omb1, omb2, eps, step_size, bc2_sqrt, decay;
};

// The fp32 scalars of the step that raises t by one. The hyperparameters are
// fp32; 1 - beta is exact in fp32 for beta in [0.5, 1]. The running beta
// powers are float64; each derived scalar is computed in float64 and rounded
// once to fp32.
__host__ __device__ inline AdamConsts adam_constants(const zds_adamw_hparams &hp, double b1pow,
                                                     double b2pow) {
  AdamConsts c;
  c.b1 = hp.beta1;
  c.b2 = hp.beta2;
  c.eps = hp.eps;
  c.omb1 = 1.0f - hp.beta1;
  c.omb2 = 1.0f - hp.beta2;
  const double p1 = b1pow * static_cast<double>(hp.beta1);
  const double p2 = b2pow * static_cast<double>(hp.beta2);
  c.step_size = static_cast<float>(static_cast<double>(hp.lr) / (1.0 - p1));
  c.bc2_sqrt = static_cast<float>(sqrt(1.0 - p2));
  c.decay = static_cast<float>(1.0 - static_cast<double>(hp.lr) * static_cast<double>(hp.weight_decay));
  return c;
}

// Loss-scale transition after a step with the given overflow flag.
__host__ __device__ inline void scaler_transition(zds_step_state &s, uint32_t overflow, float beta1,
                                                  float beta2) {
  s.steps_seen += 1u;
  if (overflow) {
    s.last_skip = 1u;
    s.steps_skipped += 1u;
    if (!s.dynamic) return;
    s.good_steps = 0;
    if (s.hyst_left <= 1) {
      const float half = s.scale * 0.5f;
      s.scale = half < s.min_scale ? s.min_scale : half;
      s.hyst_left = s.hysteresis;
    } else {
      s.hyst_left -= 1;
    }
    return;
  }
  s.last_skip = 0u;
  s.t += 1;
  s.beta1_pow *= static_cast<double>(beta1);
  s.beta2_pow *= static_cast<double>(beta2);
  if (!s.dynamic) return;
  s.hyst_left = s.hysteresis;
  s.good_steps += 1;
  if (s.good_steps == s.window) {
    // fp32 power of two; growth saturates at 2^127 so the scale stays finite
    if (s.scale < 0x1p127f) s.scale *= 2.0f;
    s.good_steps = 0;
  }
}

// Norm, clip coefficient and the single grad factor from the raw sum of
// squares. A finite sum means every element was finite (see the norm kernel).
__host__ __device__ inline void clip_scalars(double sumsq, float scale, int32_t accum_steps,
                                             float max_norm, zds_step_scalars &o) {
  o.sumsq = sumsq;
  o.accum_steps = accum_steps;
  o.scale_used = scale;
  if (!(sumsq <= DBL_MAX)) {  // +inf or NaN
    o.overflow = 1u;
    o.norm = INFINITY;
    o.clip_coef = 1.0f;
    o.grad_scale = 0.0f;
    return;
  }
  o.overflow = 0u;
  const double sk = static_cast<double>(scale) * static_cast<double>(accum_steps);
  const double norm = sqrt(sumsq) / sk;
  double coef = 1.0;
  if (max_norm > 0.0f && norm > static_cast<double>(max_norm)) {
    coef = static_cast<double>(max_norm) / (norm + 1e-6);
  }
  o.norm = static_cast<float>(norm);
  o.clip_coef = static_cast<float>(coef);
  o.grad_scale = static_cast<float>(coef / sk);
}

inline void state_from_config(zds_step_state &s, const zds_scaler_config &cfg, int64_t t0,
                              double b1p, double b2p) {
  s.scale = cfg.dynamic ? std::ldexp(1.0f, cfg.initial_scale_power) : cfg.static_scale;
  s.good_steps = 0;
  s.hyst_left = cfg.hysteresis;
  s.window = cfg.window;
  s.hysteresis = cfg.hysteresis;
  s.min_scale = cfg.min_scale;
  s.dynamic = cfg.dynamic ? 1 : 0;
  s.last_skip = 0u;
  s.t = t0;
  s.beta1_pow = b1p;
  s.beta2_pow = b2p;
  s.steps_seen = 0u;
  s.steps_skipped = 0u;
}

// ---------------------------------------------------------------------------
// Launchers (arguments already validated).
// ---------------------------------------------------------------------------

struct PlanDev {
  const int64_t *table;  // [start E][len E][dst E][chunk0 E+1][entry of each chunk]
  int32_t num_entries;
  int64_t total_chunks;
};

zds_status launch_accumulate(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src,
                             void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                             hipStream_t stream);

int norm_grid(int64_t n);
zds_status launch_norm(const void *grads, zds_dtype dtype, int64_t n, int32_t accum_steps,
                       float max_norm, const zds_step_state *state, zds_step_scalars *out,
                       double *partials, hipStream_t stream);

// Folds nparts float64 partial sums (more levels for large counts, written
// into the workspace after them) and derives the step scalars.
zds_status launch_norm_stage2(double *partials, int64_t nparts, const zds_step_state *state,
                              int32_t accum_steps, float max_norm, zds_step_scalars *out,
                              hipStream_t stream);
// Doubles of workspace launch_norm_stage2 needs for nparts partials.
int64_t partials_workspace_doubles(int64_t nparts);

// Grid of the accumulate kernel for a plan with `total_chunks` chunks (also
// the number of partial sums the fused norm writes).
int64_t accumulate_grid(int64_t total_chunks);

// Same as launch_accumulate, and each block also writes the float64 sum of
// squares of the values it stored to partials[blockIdx].
zds_status launch_accumulate_norm(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src,
                                  void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                  double *partials, hipStream_t stream);

// Most peers zds_reduce_peer_slices sums in one call.
constexpr int kMaxPeers = 16;
zds_status launch_reduce_peers(const void *const *peers, int32_t npeers, zds_dtype src, int64_t n, void *dst,
                               zds_dtype dst_dtype, bool accumulate, hipStream_t stream);

zds_status launch_adam(const zds_adamw_hparams &hp, const void *grads, zds_dtype gdt, float *master,
                       float *m, float *v, void *out, zds_dtype pdt, int64_t n, zds_step_scalars *scalars,
                       const zds_step_state *state, hipStream_t stream);

zds_status launch_scaler(zds_step_state *state, const zds_step_scalars *scalars, float beta1,
                         float beta2, hipStream_t stream);
zds_status launch_state_init(zds_step_state *state, const zds_step_state &init, hipStream_t stream);

// A dispatch packet counts work-items in 32 bits: a launch must stay below
// 2^32 of them. Grids are capped here and the kernels loop over the rest.
constexpr int64_t max_blocks(int threads_per_block) {
  return ((int64_t(1) << 32) - 1) / threads_per_block < (int64_t(1) << 23)
             ? ((int64_t(1) << 32) - 1) / threads_per_block
             : (int64_t(1) << 23);
}

// Chunk size (elements) of the accumulate kernel's work items.
#ifndef ZDS_ACC_CHUNK
#define ZDS_ACC_CHUNK 4096
#endif
constexpr int64_t kAccumChunk = ZDS_ACC_CHUNK;

}  // namespace zds
