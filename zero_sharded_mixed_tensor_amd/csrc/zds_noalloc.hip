// The overflow / norm pass for callers that cannot allocate: the block
// partial sums live in a fixed device array of the library instead of a
// caller workspace (graph capture, serving loops, harnesses that forbid
// hipMalloc). The kernels are those of zds_overflow_and_norm.
#include <atomic>
#include <mutex>

#include "zds_internal.h"

namespace {

// Room for the partial sums (and their folding levels) of
// zds_overflow_and_norm over up to 1,073,217,536 elements (one float64
// partial per 2048).
constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends. In host code this name is
// a host-side stand-in, not a device address: the address on each device
// comes from hipGetSymbolAddress and only that address is handed to kernels.
__device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

std::atomic<double *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, resolved on the
// first call on that device.
zds_status scratch_address(double **out, const char *fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return zds::hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return zds::fail(ZDS_EINVAL, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  double *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return zds::hip_fail(e, fn);
      if (!addr) return zds::fail(ZDS_EHIP, "%s: no device address for the scratch array", fn);
      p = static_cast<double *>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZDS_OK;
}

}  // namespace

using namespace zds;

extern "C" zds_status zds_overflow_and_norm_noalloc(const void *grads, zds_dtype dtype, int64_t n,
                                                    int32_t accum_steps, float max_norm,
                                                    const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                                    void *stream) {
  clear_error();
  const char *fn = "zds_overflow_and_norm_noalloc";
  if (!valid_dtype(dtype)) return fail(ZDS_EINVAL, "%s: bad dtype", fn);
  if (n < 0) return fail(ZDS_EINVAL, "%s: n < 0", fn);
  if (accum_steps < 1) return fail(ZDS_EINVAL, "%s: accum_steps must be >= 1", fn);
  if (!state_dev || !out_dev) return fail(ZDS_EINVAL, "%s: null state or output", fn);
  if (!aligned(state_dev, 8) || !aligned(out_dev, 8)) return fail(ZDS_EALIGN, "%s: state/output not 8-byte aligned", fn);
  if (n > 0 && !grads) return fail(ZDS_EINVAL, "%s: null grads", fn);
  if (n > 0 && !aligned(grads, static_cast<uintptr_t>(dtype_size(dtype))))
    return fail(ZDS_EALIGN, "%s: grads misaligned", fn);
  const size_t need = static_cast<size_t>(partials_workspace_doubles(norm_grid(n))) * sizeof(double);
  if (need > kScratchBytes)
    return fail(ZDS_EINVAL, "%s: n = %lld needs %zu bytes of partial sums, the fixed array holds %zu", fn,
                static_cast<long long>(n), need, kScratchBytes);
  double *partials = nullptr;
  const zds_status st = scratch_address(&partials, fn);
  if (st != ZDS_OK) return st;
  // n == 0 still writes the scalars of an empty shard, as zds_overflow_and_norm.
  return launch_norm(grads, dtype, n, accum_steps, max_norm, state_dev, out_dev, partials,
                     static_cast<hipStream_t>(stream));
}
