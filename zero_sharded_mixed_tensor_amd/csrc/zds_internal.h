// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "zds.h"
#include "zds_scalar.h"

namespace zds {

// ---------------------------------------------------------------------------
// Error reporting (thread-local message behind zds_last_error()); fail() and
// clear_error() are declared in zds_scalar.h.
// ---------------------------------------------------------------------------
zds_status hip_fail(hipError_t e, const char *what);
zds_status check_launch(const char *what);

// Number of compute units of the current device (cached per device).
int device_cu_count();


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

// Grid of the accumulate kernel in `mode` for a plan with `total_chunks`
// chunks (also the number of partial sums the fused norm writes; largest in
// the fp32 modes).
int64_t accumulate_grid(int64_t total_chunks, zds_accum_mode mode);

// Same as launch_accumulate, and each block also writes the float64 sum of
// squares of the values it stored to partials[blockIdx].
zds_status launch_accumulate_norm(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src,
                                  void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                  double *partials, hipStream_t stream);

// Most peers zds_reduce_peer_slices sums in one call.
constexpr int kMaxPeers = 16;
// With partials != null each block also writes the float64 sum of squares of
// the values it stored; *nparts (if given) receives the number of blocks.
zds_status launch_reduce_peers(const void *const *peers, int32_t npeers, zds_dtype src, int64_t n, void *dst,
                               zds_dtype dst_dtype, bool accumulate, double *partials, int64_t *nparts,
                               hipStream_t stream);
// Most partial sums the fused intake norm writes for n elements.
int64_t reduce_grid_max(int64_t n);

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
constexpr int64_t kAccumChunk = 4096;

}  // namespace zds
