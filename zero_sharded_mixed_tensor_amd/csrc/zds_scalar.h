// Scalar logic and small helpers shared by the device kernels, their host
// twins and the host (offload) optimizer: one definition, compiled by hipcc
// for both sides and by the host compiler for the CPU path.
#pragma once

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "zds.h"

#if defined(__HIPCC__) || defined(__HIP__)
#define ZDS_HD __host__ __device__
#else
#define ZDS_HD
#endif

namespace zds {

zds_status fail(zds_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int dtype_size(zds_dtype d) { return d == ZDS_FP32 ? 4 : 2; }
inline bool valid_dtype(int d) { return d == ZDS_FP16 || d == ZDS_BF16 || d == ZDS_FP32; }
ZDS_HD inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// ---------------------------------------------------------------------------
// Scalar logic, one definition for host and device.
// ---------------------------------------------------------------------------

struct AdamConsts {
  float b1, b2, omb1, omb2, eps, step_size, bc2_sqrt, decay;
  double inv_bc2_sqrt;  // 1 / bc2_sqrt in float64, correctly rounded
};

// The fp32 scalars of the step that raises t by one. The hyperparameters are
// fp32; 1 - beta is exact in fp32 for beta in [0.5, 1]. The running beta
// powers are float64; each derived scalar is computed in float64 and rounded
// once to fp32.
ZDS_HD inline AdamConsts adam_constants(const zds_adamw_hparams &hp, double b1pow,
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
  c.inv_bc2_sqrt = 1.0 / static_cast<double>(c.bc2_sqrt);
  return c;
}

// Loss-scale transition after a step with the given overflow flag.
ZDS_HD inline void scaler_transition(zds_step_state &s, uint32_t overflow, float beta1,
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
ZDS_HD inline void clip_scalars(double sumsq, float scale, int32_t accum_steps,
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

}  // namespace zds
