// Offloaded optimizer shard (a next row): the same AdamW update on host
// memory, for a rank whose fp32 master/m/v live in host RAM. ZeRO-Offload
// moves the optimizer state (and its update) to the CPU, trading PCIe and
// host-memory bandwidth for HBM, and a step is then bounded by its slowest
// link (aiqz.cc "DeepSpeed ZeRO引擎深入", 卸载策略; devpress.csdn.net DeepSpeed
// tutorial §4.3; algomooc.com, ZeRO 三阶段).
//
// Bit-identical to the device kernel and the oracle: the same step constants
// (zds_scalar.h), the same fp32 operation order with one rounding each, no
// FMA contraction (-ffp-contract=off), IEEE division and square root
// (vdivps/vsqrtps), round-to-nearest-even casts (F16C for fp16, integer
// rounding for bf16). The range is cut into contiguous pieces, one per
// thread; each thread walks its piece in blocks of 1024 elements: widen the
// grads, update (a loop the compiler vectorises), narrow the params.
// Host-memory bound: 28 B/param (16-bit grads) like the device pass.
#include <immintrin.h>

#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "zds_host.h"
#include "zds_scalar.h"

namespace {

using zds::AdamConsts;

constexpr int64_t kBlock = 1024;

struct HostArgs {
  const void *g;
  zds_dtype gdt;
  float *p, *m, *v;
  void *out;
  zds_dtype pdt;
  float gs;
  AdamConsts c;
};

inline uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

void widen_block(const void *g, zds_dtype d, int64_t off, int64_t len, float *x) {
  if (d == ZDS_FP32) {
    std::memcpy(x, static_cast<const float *>(g) + off, sizeof(float) * len);
  } else if (d == ZDS_BF16) {
    const uint16_t *h = static_cast<const uint16_t *>(g) + off;
    for (int64_t j = 0; j < len; ++j) {
      const uint32_t u = static_cast<uint32_t>(h[j]) << 16;
      std::memcpy(&x[j], &u, 4);
    }
  } else {
    const uint16_t *h = static_cast<const uint16_t *>(g) + off;
    int64_t j = 0;
    for (; j + 8 <= len; j += 8) {
      const __m128i w = _mm_loadu_si128(reinterpret_cast<const __m128i *>(h + j));
      _mm256_storeu_ps(x + j, _mm256_cvtph_ps(w));
    }
    for (; j < len; ++j) x[j] = _cvtsh_ss(h[j]);
  }
}

void narrow_block(const float *p, zds_dtype d, int64_t off, int64_t len, void *out) {
  uint16_t *o = static_cast<uint16_t *>(out) + off;
  if (d == ZDS_BF16) {
    for (int64_t j = 0; j < len; ++j) o[j] = bf16_rne(p[j]);
  } else {
    int64_t j = 0;
    for (; j + 8 <= len; j += 8) {
      const __m128i w = _mm256_cvtps_ph(_mm256_loadu_ps(p + j), _MM_FROUND_TO_NEAREST_INT);
      _mm_storeu_si128(reinterpret_cast<__m128i *>(o + j), w);
    }
    for (; j < len; ++j) o[j] = _cvtss_sh(p[j], _MM_FROUND_TO_NEAREST_INT);
  }
}

// The element update, in the same order as the device kernel.
void update_block(const float *__restrict x, float *__restrict p, float *__restrict m, float *__restrict v,
                  int64_t len, const AdamConsts &c, float gs) {
  const float b1 = c.b1, b2 = c.b2, omb1 = c.omb1, omb2 = c.omb2, eps = c.eps;
  const float step = c.step_size, bc2 = c.bc2_sqrt, decay = c.decay;
  for (int64_t j = 0; j < len; ++j) {
    const float g = x[j] * gs;
    const float mj = b1 * m[j] + omb1 * g;
    const float vj = b2 * v[j] + omb2 * (g * g);
    const float denom = std::sqrt(vj) / bc2 + eps;
    float pj = p[j] * decay;
    pj = pj - step * (mj / denom);
    m[j] = mj;
    v[j] = vj;
    p[j] = pj;
  }
}

void run_range(const HostArgs &a, int64_t lo, int64_t hi) {
  alignas(64) float x[kBlock];
  for (int64_t b = lo; b < hi; b += kBlock) {
    const int64_t len = std::min(kBlock, hi - b);
    widen_block(a.g, a.gdt, b, len, x);
    update_block(x, a.p + b, a.m + b, a.v + b, len, a.c, a.gs);
    if (a.out) narrow_block(a.p + b, a.pdt, b, len, a.out);
  }
}

}  // namespace

extern "C" zds_status zds_cpu_adam_step(const zds_adamw_hparams *hp, const void *grads, zds_dtype grad_dtype,
                                        float *master, float *exp_avg, float *exp_avg_sq, void *params_out,
                                        zds_dtype param_dtype, int64_t n, const zds_step_scalars *scalars,
                                        const zds_step_state *state, int32_t num_threads) {
  using namespace zds;
  clear_error();
  const char *fn = "zds_cpu_adam_step";
  if (!hp || !scalars || !state) return fail(ZDS_EINVAL, "%s: null hparams, scalars or state", fn);
  if (!valid_dtype(grad_dtype)) return fail(ZDS_EINVAL, "%s: bad grad dtype", fn);
  if (params_out && param_dtype != ZDS_FP16 && param_dtype != ZDS_BF16)
    return fail(ZDS_EINVAL, "%s: param dtype must be fp16 or bf16", fn);
  if (n < 0) return fail(ZDS_EINVAL, "%s: n < 0", fn);
  if (!(hp->beta1 >= 0.5f && hp->beta1 < 1.0f && hp->beta2 >= 0.5f && hp->beta2 < 1.0f))
    return fail(ZDS_EINVAL, "%s: betas must lie in [0.5, 1)", fn);
  if (!(hp->eps > 0.0f) || !(hp->lr >= 0.0f) || !(hp->weight_decay >= 0.0f))
    return fail(ZDS_EINVAL, "%s: need eps > 0, lr >= 0, weight_decay >= 0", fn);
  if (num_threads < 0) return fail(ZDS_EINVAL, "%s: num_threads < 0", fn);
  if (n == 0 || scalars->overflow) return ZDS_OK;  // empty, or a skipped step
  if (!grads || !master || !exp_avg || !exp_avg_sq) return fail(ZDS_EINVAL, "%s: null pointer", fn);
  HostArgs a{grads, grad_dtype, master, exp_avg, exp_avg_sq, params_out, param_dtype, scalars->grad_scale,
             adam_constants(*hp, state->beta1_pow, state->beta2_pow)};
  int64_t T = num_threads > 0 ? num_threads : host_thread_budget();
  if (T < 1) T = 1;
  const int64_t blocks = (n + kBlock - 1) / kBlock;
  if (T > blocks) T = blocks;
  const int64_t per = (blocks + T - 1) / T * kBlock;  // contiguous, block-aligned pieces
  std::vector<std::thread> pool;
  pool.reserve(static_cast<size_t>(T - 1));
  for (int64_t t = 1; t < T; ++t) {
    const int64_t lo = t * per, hi = std::min(n, (t + 1) * per);
    if (lo < hi) pool.emplace_back(run_range, std::cref(a), lo, hi);
  }
  run_range(a, 0, std::min(n, per));
  for (auto &th : pool) th.join();
  return ZDS_OK;
}
