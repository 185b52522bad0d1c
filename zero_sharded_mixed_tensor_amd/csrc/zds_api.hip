// The extern "C" boundary: argument checks, plans, host-only geometry and
// the host twins of the scalar logic. Kernels live in the other files.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "zds_internal.h"
#include "zds_onebit.h"

namespace zds {

static thread_local std::string g_err;

void clear_error() { g_err.clear(); }

zds_status fail(zds_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

zds_status hip_fail(hipError_t e, const char *what) {
  return fail(ZDS_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

zds_status check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return ZDS_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<int>(cache.size()) <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    cache[dev] = cu;
  }
  return cache[dev];
}

}  // namespace zds

using namespace zds;

// ---------------------------------------------------------------------------
// Geometry (host only)
// ---------------------------------------------------------------------------

static int64_t align_up(int64_t x, int64_t a) { return ((x + a - 1) / a) * a; }

extern "C" zds_status zds_flat_layout(const int64_t *numel, int32_t num_tensors, int32_t flat_align,
                                      int64_t *offsets_out, int64_t *total_out) {
  clear_error();
  if (num_tensors < 0 || (num_tensors > 0 && !numel) || !total_out)
    return fail(ZDS_EINVAL, "zds_flat_layout: null pointer or negative tensor count");
  if (flat_align < 1) return fail(ZDS_EINVAL, "zds_flat_layout: flat_align must be >= 1");
  int64_t pos = 0;
  for (int32_t i = 0; i < num_tensors; ++i) {
    if (numel[i] < 0) return fail(ZDS_EINVAL, "zds_flat_layout: numel[%d] < 0", i);
    if (offsets_out) offsets_out[i] = pos;
    pos = align_up(pos + numel[i], flat_align);
  }
  *total_out = pos;
  return ZDS_OK;
}

extern "C" zds_status zds_shard_range(int64_t flat_total, int32_t world, int32_t rank,
                                      int32_t flat_align, int64_t *lo, int64_t *hi) {
  clear_error();
  if (!lo || !hi) return fail(ZDS_EINVAL, "zds_shard_range: null output");
  if (world < 1 || rank < 0 || rank >= world || flat_align < 1 || flat_total < 0)
    return fail(ZDS_EINVAL, "zds_shard_range: need world >= 1, 0 <= rank < world, flat_align >= 1");
  const int64_t padded = align_up(flat_total, static_cast<int64_t>(world) * flat_align);
  const int64_t per = padded / world;
  *lo = per * rank;
  *hi = per * (rank + 1);
  return ZDS_OK;
}

static zds_status compute_entries(const int64_t *numel, int32_t T, int32_t align, int64_t lo,
                                  int64_t hi, std::vector<int64_t> &out) {
  if (T < 0 || (T > 0 && !numel)) return fail(ZDS_EINVAL, "tensor table: null numel or T < 0");
  if (align < 1) return fail(ZDS_EINVAL, "tensor table: flat_align must be >= 1");
  if (lo < 0 || hi < lo) return fail(ZDS_EINVAL, "tensor table: need 0 <= lo <= hi");
  out.clear();
  int64_t pos = 0;
  for (int32_t t = 0; t < T; ++t) {
    if (numel[t] < 0) return fail(ZDS_EINVAL, "tensor table: numel[%d] < 0", t);
    const int64_t a = pos > lo ? pos : lo;
    const int64_t end = pos + numel[t];
    const int64_t b = end < hi ? end : hi;
    if (a < b) {
      out.push_back(t);
      out.push_back(a - pos);
      out.push_back(b - a);
      out.push_back(a - lo);
    }
    pos = align_up(end, align);
  }
  return ZDS_OK;
}

extern "C" zds_status zds_shard_entries(const int64_t *numel, int32_t num_tensors, int32_t flat_align,
                                        int64_t lo, int64_t hi, int64_t *out, int32_t max_entries,
                                        int32_t *count) {
  clear_error();
  if (!count || (max_entries > 0 && !out) || max_entries < 0)
    return fail(ZDS_EINVAL, "zds_shard_entries: null output or negative max_entries");
  std::vector<int64_t> e;
  zds_status s = compute_entries(numel, num_tensors, flat_align, lo, hi, e);
  if (s != ZDS_OK) return s;
  const int32_t n = static_cast<int32_t>(e.size() / 4);
  *count = n;
  const int32_t k = n < max_entries ? n : max_entries;
  if (k > 0) memcpy(out, e.data(), sizeof(int64_t) * 4 * k);
  if (n > max_entries) return fail(ZDS_EINVAL, "zds_shard_entries: %d entries, room for %d", n, max_entries);
  return ZDS_OK;
}

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

static constexpr int kRing = 8;

struct zds_plan {
  int device = 0;
  int32_t num_tensors = 0;
  int32_t num_entries = 0;
  std::vector<int64_t> entries;  // 4 per entry
  int64_t total_chunks = 0;
  int64_t *d_table = nullptr;
  const void **d_ptrs = nullptr;  // kRing * E
  const void **h_ptrs = nullptr;  // pinned, kRing * E
  hipEvent_t ev[kRing] = {};
  bool used[kRing] = {};
  bool pinned[kRing] = {};  // read by a captured graph on every replay: never refilled
  uint32_t next = 0;
  int last_slot = -1;                // slot holding the most recently uploaded pointer set
  hipStream_t last_stream = nullptr;  // stream of the most recent launch
};

static void plan_free(zds_plan *p) {
  if (!p) return;
  for (int i = 0; i < kRing; ++i)
    if (p->ev[i]) (void)hipEventDestroy(p->ev[i]);
  if (p->d_table) (void)hipFree(p->d_table);
  if (p->d_ptrs) (void)hipFree(p->d_ptrs);
  if (p->h_ptrs) (void)hipHostFree(p->h_ptrs);
  delete p;
}

extern "C" zds_status zds_plan_create(zds_plan **out, const int64_t *numel, int32_t num_tensors,
                                      int32_t flat_align, int64_t lo, int64_t hi) {
  clear_error();
  if (!out) return fail(ZDS_EINVAL, "zds_plan_create: null out");
  *out = nullptr;
  std::vector<int64_t> e;
  zds_status s = compute_entries(numel, num_tensors, flat_align, lo, hi, e);
  if (s != ZDS_OK) return s;
  zds_plan *p = new (std::nothrow) zds_plan;
  if (!p) return fail(ZDS_ENOMEM, "zds_plan_create: host allocation failed");
  p->num_tensors = num_tensors;
  p->entries = e;
  const int32_t E = static_cast<int32_t>(e.size() / 4);
  p->num_entries = E;
  hipError_t he = hipGetDevice(&p->device);
  if (he != hipSuccess) { plan_free(p); return hip_fail(he, "zds_plan_create: hipGetDevice"); }
  // device table: [start E][length E][dst E][first chunk E+1][entry of each chunk]
  int64_t chunks = 0;
  for (int32_t i = 0; i < E; ++i) chunks += (e[4 * i + 2] + kAccumChunk - 1) / kAccumChunk;
  std::vector<int64_t> table(4 * static_cast<size_t>(E) + 1 + static_cast<size_t>(chunks));
  int64_t c = 0;
  for (int32_t i = 0; i < E; ++i) {
    table[i] = e[4 * i + 1];
    table[E + i] = e[4 * i + 2];
    table[2 * E + i] = e[4 * i + 3];
    table[3 * E + i] = c;
    const int64_t k = (e[4 * i + 2] + kAccumChunk - 1) / kAccumChunk;
    for (int64_t j = 0; j < k; ++j) table[4 * static_cast<size_t>(E) + 1 + c + j] = i;
    c += k;
  }
  table[4 * E] = chunks;
  p->total_chunks = chunks;
  const size_t tb = table.size() * sizeof(int64_t);
  he = hipMalloc(reinterpret_cast<void **>(&p->d_table), tb);
  if (he != hipSuccess) { plan_free(p); return fail(ZDS_ENOMEM, "zds_plan_create: hipMalloc table: %s", hipGetErrorString(he)); }
  he = hipMemcpy(p->d_table, table.data(), tb, hipMemcpyHostToDevice);
  if (he != hipSuccess) { plan_free(p); return hip_fail(he, "zds_plan_create: table upload"); }
  const size_t pb = sizeof(void *) * kRing * (E > 0 ? E : 1);
  he = hipMalloc(reinterpret_cast<void **>(&p->d_ptrs), pb);
  if (he != hipSuccess) { plan_free(p); return fail(ZDS_ENOMEM, "zds_plan_create: hipMalloc ptrs: %s", hipGetErrorString(he)); }
  he = hipHostMalloc(reinterpret_cast<void **>(&p->h_ptrs), pb, hipHostMallocDefault);
  if (he != hipSuccess) { plan_free(p); return fail(ZDS_ENOMEM, "zds_plan_create: hipHostMalloc: %s", hipGetErrorString(he)); }
  for (int i = 0; i < kRing; ++i) {
    he = hipEventCreateWithFlags(&p->ev[i], hipEventDisableTiming);
    if (he != hipSuccess) { plan_free(p); return hip_fail(he, "zds_plan_create: hipEventCreate"); }
  }
  *out = p;
  return ZDS_OK;
}

extern "C" void zds_plan_destroy(zds_plan *plan) {
  if (!plan) return;
  for (int i = 0; i < kRing; ++i)
    if (plan->used[i]) (void)hipEventSynchronize(plan->ev[i]);
  plan_free(plan);
}

extern "C" int32_t zds_plan_num_entries(const zds_plan *plan) { return plan ? plan->num_entries : -1; }

extern "C" zds_status zds_plan_entry(const zds_plan *plan, int32_t e, int64_t *out4) {
  clear_error();
  if (!plan || !out4) return fail(ZDS_EINVAL, "zds_plan_entry: null argument");
  if (e < 0 || e >= plan->num_entries) return fail(ZDS_EINVAL, "zds_plan_entry: entry %d out of range", e);
  memcpy(out4, &plan->entries[4 * static_cast<size_t>(e)], 4 * sizeof(int64_t));
  return ZDS_OK;
}

// ---------------------------------------------------------------------------
// Hot calls
// ---------------------------------------------------------------------------

// Checks, staging of the per-call source pointers, and the launch shared by
// zds_grad_accumulate and zds_grad_accumulate_norm. With partials != null the
// kernel also writes one sum of squares per block.
static zds_status accumulate_impl(const char *fn, zds_plan *plan, const void *const *src_ptrs,
                                  zds_dtype src_dtype, void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                  double *partials, void *stream) {
  if (!plan) return fail(ZDS_EINVAL, "%s: null plan", fn);
  if (!valid_dtype(src_dtype) || !valid_dtype(dst_dtype)) return fail(ZDS_EINVAL, "%s: bad dtype", fn);
  if (mode == ZDS_COPY) {
    if (src_dtype == ZDS_FP32 || dst_dtype != src_dtype)
      return fail(ZDS_EINVAL, "%s: copy mode needs the same 16-bit dtype on both sides", fn);
  } else if (mode == ZDS_OVERWRITE || mode == ZDS_ACCUMULATE) {
    if (dst_dtype != ZDS_FP32) return fail(ZDS_EINVAL, "%s: accumulator must be fp32", fn);
  } else {
    return fail(ZDS_EINVAL, "%s: bad mode %d", fn, static_cast<int>(mode));
  }
  const int32_t E = plan->num_entries;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PlanDev pd{plan->d_table, E, plan->total_chunks};
  if (E == 0) {
    if (!partials) return ZDS_OK;
    return launch_accumulate_norm(pd, plan->d_ptrs, src_dtype, dst, dst_dtype, mode, partials, s);
  }
  if (!src_ptrs || !dst) return fail(ZDS_EINVAL, "%s: null src_ptrs or dst", fn);
  const uintptr_t es = static_cast<uintptr_t>(dtype_size(src_dtype));
  if (!aligned(dst, static_cast<uintptr_t>(dtype_size(dst_dtype))))
    return fail(ZDS_EALIGN, "%s: dst not aligned to its element size", fn);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (dev != plan->device) return fail(ZDS_EINVAL, "%s: plan belongs to device %d, current is %d", fn, plan->device, dev);
  for (int32_t i = 0; i < E; ++i) {
    const int64_t t = plan->entries[4 * static_cast<size_t>(i)];
    const void *sp = src_ptrs[t];
    if (!sp) return fail(ZDS_EINVAL, "%s: src_ptrs[%lld] is null", fn, static_cast<long long>(t));
    if (!aligned(sp, es)) return fail(ZDS_EALIGN, "%s: src_ptrs[%lld] misaligned", fn, static_cast<long long>(t));
  }
  // The same source set as the previous call (the usual case: grads live in
  // fixed buffers) reuses that slot's device copy; otherwise the next ring
  // slot is refilled once the launch that last used it has finished.
  bool same = plan->last_slot >= 0;
  if (same) {
    const void **prev = plan->h_ptrs + static_cast<size_t>(plan->last_slot) * E;
    for (int32_t i = 0; i < E && same; ++i) same = prev[i] == src_ptrs[plan->entries[4 * static_cast<size_t>(i)]];
  }
  // Under stream capture the launch is recorded into a graph and replayed
  // later: it may only read an upload that is already complete (the caller
  // ran the same source set eagerly and synchronized), and that slot is then
  // never refilled. No upload, event record or wait is captured.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  he = hipStreamIsCapturing(s, &cap);
  if (he != hipSuccess) return hip_fail(he, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) {
    if (!same)
      return fail(ZDS_EINVAL,
                  "%s: under stream capture the source pointers must be those of the previous call, after that "
                  "call has completed (run it once eagerly and synchronize before capturing)", fn);
    plan->pinned[plan->last_slot] = true;
    const void **dp = plan->d_ptrs + static_cast<size_t>(plan->last_slot) * E;
    return partials ? launch_accumulate_norm(pd, dp, src_dtype, dst, dst_dtype, mode, partials, s)
                    : launch_accumulate(pd, dp, src_dtype, dst, dst_dtype, mode, s);
  }
  uint32_t slot;
  if (same) {
    slot = static_cast<uint32_t>(plan->last_slot);
  } else {
    int k = 0;
    while (k < kRing && plan->pinned[(plan->next + k) % kRing]) ++k;
    if (k == kRing) return fail(ZDS_EINVAL, "%s: every staging slot is held by a captured graph", fn);
    plan->next += static_cast<uint32_t>(k);
    slot = plan->next % kRing;
    if (plan->used[slot]) {
      he = hipEventSynchronize(plan->ev[slot]);
      if (he != hipSuccess) return hip_fail(he, "staging slot wait");
    }
  }
  // a reused upload was enqueued on the stream of an earlier call: another
  // stream must wait for it (ev[slot] follows the upload and that launch)
  if (same && s != plan->last_stream) {
    he = hipStreamWaitEvent(s, plan->ev[slot], 0);
    if (he != hipSuccess) return hip_fail(he, "hipStreamWaitEvent");
  }
  const void **h = plan->h_ptrs + static_cast<size_t>(slot) * E;
  const void **d = plan->d_ptrs + static_cast<size_t>(slot) * E;
  if (!same) {
    for (int32_t i = 0; i < E; ++i) h[i] = src_ptrs[plan->entries[4 * static_cast<size_t>(i)]];
    he = hipMemcpyAsync(d, h, sizeof(void *) * E, hipMemcpyHostToDevice, s);
    if (he != hipSuccess) return hip_fail(he, "pointer upload");
  }
  zds_status st = partials ? launch_accumulate_norm(pd, d, src_dtype, dst, dst_dtype, mode, partials, s)
                           : launch_accumulate(pd, d, src_dtype, dst, dst_dtype, mode, s);
  if (st != ZDS_OK) return st;
  he = hipEventRecord(plan->ev[slot], s);
  if (he != hipSuccess) return hip_fail(he, "hipEventRecord");
  plan->used[slot] = true;
  plan->last_stream = s;
  if (!same) {
    plan->next += 1;
    plan->last_slot = static_cast<int>(slot);
  }
  return ZDS_OK;
}

extern "C" zds_status zds_grad_accumulate(zds_plan *plan, const void *const *src_ptrs,
                                          zds_dtype src_dtype, void *dst, zds_dtype dst_dtype,
                                          zds_accum_mode mode, void *stream) {
  clear_error();
  return accumulate_impl("zds_grad_accumulate", plan, src_ptrs, src_dtype, dst, dst_dtype, mode, nullptr,
                         stream);
}

extern "C" size_t zds_plan_norm_workspace_bytes(const zds_plan *plan) {
  if (!plan) return 0;
  // the accumulate mode launches the most blocks, hence writes the most partials
  return static_cast<size_t>(partials_workspace_doubles(accumulate_grid(plan->total_chunks, ZDS_ACCUMULATE))) *
         sizeof(double);
}

extern "C" zds_status zds_grad_accumulate_norm(zds_plan *plan, const void *const *src_ptrs,
                                               zds_dtype src_dtype, void *dst, zds_dtype dst_dtype,
                                               zds_accum_mode mode, int32_t accum_steps, float max_norm,
                                               const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                               void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  const char *fn = "zds_grad_accumulate_norm";
  if (!plan) return fail(ZDS_EINVAL, "%s: null plan", fn);
  if (accum_steps < 1) return fail(ZDS_EINVAL, "%s: accum_steps must be >= 1", fn);
  if (!state_dev || !out_dev) return fail(ZDS_EINVAL, "%s: null state or output", fn);
  if (!aligned(state_dev, 8) || !aligned(out_dev, 8))
    return fail(ZDS_EALIGN, "%s: state/output not 8-byte aligned", fn);
  const size_t need = zds_plan_norm_workspace_bytes(plan);
  if (!ws || ws_bytes < need || !aligned(ws, 8))
    return fail(ZDS_EINVAL, "%s: workspace of %zu bytes needed (8-byte aligned)", fn, need);
  double *partials = static_cast<double *>(ws);
  zds_status st = accumulate_impl(fn, plan, src_ptrs, src_dtype, dst, dst_dtype, mode, partials, stream);
  if (st != ZDS_OK) return st;
  return launch_norm_stage2(partials, accumulate_grid(plan->total_chunks, mode), state_dev, accum_steps, max_norm,
                            out_dev, static_cast<hipStream_t>(stream));
}

static zds_status reduce_checks(const char *fn, const void *const *peer_ptrs, int32_t num_peers,
                                zds_dtype src_dtype, int64_t n, void *dst, zds_dtype dst_dtype, zds_accum_mode mode) {
  if (num_peers < 1 || num_peers > kMaxPeers) return fail(ZDS_EINVAL, "%s: num_peers must be in [1, %d]", fn, kMaxPeers);
  if (src_dtype != ZDS_FP16 && src_dtype != ZDS_BF16) return fail(ZDS_EINVAL, "%s: peers must be fp16 or bf16", fn);
  if (dst_dtype != ZDS_FP32 && dst_dtype != src_dtype)
    return fail(ZDS_EINVAL, "%s: destination must be fp32 or the peers' dtype", fn);
  if (mode != ZDS_OVERWRITE && mode != ZDS_ACCUMULATE) return fail(ZDS_EINVAL, "%s: mode must be overwrite or accumulate", fn);
  if (n < 0) return fail(ZDS_EINVAL, "%s: n < 0", fn);
  if (n == 0) return ZDS_OK;
  if (!peer_ptrs || !dst) return fail(ZDS_EINVAL, "%s: null pointer", fn);
  for (int k = 0; k < num_peers; ++k) {
    if (!peer_ptrs[k]) return fail(ZDS_EINVAL, "%s: peer %d is null", fn, k);
    if (!aligned(peer_ptrs[k], 2)) return fail(ZDS_EALIGN, "%s: peer %d misaligned", fn, k);
  }
  if (!aligned(dst, static_cast<uintptr_t>(dtype_size(dst_dtype)))) return fail(ZDS_EALIGN, "%s: dst misaligned", fn);
  return ZDS_OK;
}

extern "C" zds_status zds_reduce_peer_slices(const void *const *peer_ptrs, int32_t num_peers, zds_dtype src_dtype,
                                             int64_t n, void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                             void *stream) {
  clear_error();
  zds_status st = reduce_checks("zds_reduce_peer_slices", peer_ptrs, num_peers, src_dtype, n, dst, dst_dtype, mode);
  if (st != ZDS_OK || n == 0) return st;
  return launch_reduce_peers(peer_ptrs, num_peers, src_dtype, n, dst, dst_dtype, mode == ZDS_ACCUMULATE, nullptr,
                             nullptr, static_cast<hipStream_t>(stream));
}

extern "C" size_t zds_reduce_norm_workspace_bytes(int64_t n) {
  const int64_t a = partials_workspace_doubles(reduce_grid_max(n < 0 ? 0 : n));
  const int64_t b = partials_workspace_doubles(norm_grid(0));  // n == 0 runs the plain norm pass
  return static_cast<size_t>(a > b ? a : b) * sizeof(double);
}

extern "C" zds_status zds_reduce_peer_slices_norm(const void *const *peer_ptrs, int32_t num_peers,
                                                  zds_dtype src_dtype, int64_t n, void *dst, zds_dtype dst_dtype,
                                                  zds_accum_mode mode, int32_t accum_steps, float max_norm,
                                                  const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                                  void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  const char *fn = "zds_reduce_peer_slices_norm";
  zds_status st = reduce_checks(fn, peer_ptrs, num_peers, src_dtype, n, dst, dst_dtype, mode);
  if (st != ZDS_OK) return st;
  if (accum_steps < 1) return fail(ZDS_EINVAL, "%s: accum_steps must be >= 1", fn);
  if (!state_dev || !out_dev) return fail(ZDS_EINVAL, "%s: null state or output", fn);
  if (!aligned(state_dev, 8) || !aligned(out_dev, 8)) return fail(ZDS_EALIGN, "%s: state/output not 8-byte aligned", fn);
  const size_t need = zds_reduce_norm_workspace_bytes(n);
  if (!ws || ws_bytes < need || !aligned(ws, 8))
    return fail(ZDS_EINVAL, "%s: workspace of %zu bytes needed (8-byte aligned)", fn, need);
  double *partials = static_cast<double *>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // nothing to sum: the scalars of an empty shard (norm 0), as zds_overflow_and_norm writes them
  if (n == 0) return launch_norm(nullptr, ZDS_FP32, 0, accum_steps, max_norm, state_dev, out_dev, partials, s);
  int64_t nparts = 0;
  st = launch_reduce_peers(peer_ptrs, num_peers, src_dtype, n, dst, dst_dtype, mode == ZDS_ACCUMULATE, partials,
                           &nparts, s);
  if (st != ZDS_OK) return st;
  return launch_norm_stage2(partials, nparts, state_dev, accum_steps, max_norm, out_dev, s);
}

static bool onebit_chunk_ok(int32_t c) {
  return c == 1024 || c == 2048 || c == 4096 || c == 8192 || c == 16384;
}

extern "C" zds_status zds_onebit_compress(const float *x, float *error, int64_t n, int32_t chunk, uint32_t *words,
                                          float *scales, void *stream) {
  clear_error();
  const char *fn = "zds_onebit_compress";
  if (!onebit_chunk_ok(chunk)) return fail(ZDS_EINVAL, "%s: chunk must be 1024, 2048, 4096, 8192 or 16384", fn);
  if (n < 0) return fail(ZDS_EINVAL, "%s: n < 0", fn);
  if (n == 0) return ZDS_OK;
  if (!x || !words || !scales) return fail(ZDS_EINVAL, "%s: null pointer", fn);
  if (!aligned(x, 16) || (error && !aligned(error, 16)))
    return fail(ZDS_EALIGN, "%s: x and error must be 16-byte aligned", fn);
  if (!aligned(words, 4) || !aligned(scales, 4)) return fail(ZDS_EALIGN, "%s: words and scales must be 4-byte aligned", fn);
  return launch_onebit_encode(x, error, n, chunk, words, scales, static_cast<hipStream_t>(stream));
}

extern "C" zds_status zds_onebit_decompress(const uint32_t *const *peer_words, const float *const *peer_scales,
                                            int32_t num_peers, int64_t n, int32_t chunk, float *dst,
                                            zds_accum_mode mode, void *stream) {
  clear_error();
  const char *fn = "zds_onebit_decompress";
  if (num_peers < 1 || num_peers > kMaxPeers) return fail(ZDS_EINVAL, "%s: num_peers must be in [1, %d]", fn, kMaxPeers);
  if (!onebit_chunk_ok(chunk)) return fail(ZDS_EINVAL, "%s: chunk must be 1024, 2048, 4096, 8192 or 16384", fn);
  if (mode != ZDS_OVERWRITE && mode != ZDS_ACCUMULATE) return fail(ZDS_EINVAL, "%s: mode must be overwrite or accumulate", fn);
  if (n < 0) return fail(ZDS_EINVAL, "%s: n < 0", fn);
  if (n == 0) return ZDS_OK;
  if (!peer_words || !peer_scales || !dst) return fail(ZDS_EINVAL, "%s: null pointer", fn);
  for (int k = 0; k < num_peers; ++k) {
    if (!peer_words[k] || !peer_scales[k]) return fail(ZDS_EINVAL, "%s: peer %d is null", fn, k);
    if (!aligned(peer_words[k], 4) || !aligned(peer_scales[k], 4)) return fail(ZDS_EALIGN, "%s: peer %d misaligned", fn, k);
  }
  if (!aligned(dst, 16)) return fail(ZDS_EALIGN, "%s: dst must be 16-byte aligned", fn);
  return launch_onebit_decode(peer_words, peer_scales, num_peers, n, chunk, dst, mode == ZDS_ACCUMULATE,
                              static_cast<hipStream_t>(stream));
}

extern "C" size_t zds_workspace_bytes(int64_t n) {
  return static_cast<size_t>(partials_workspace_doubles(norm_grid(n < 0 ? 0 : n))) * sizeof(double);
}

extern "C" zds_status zds_overflow_and_norm(const void *grads, zds_dtype dtype, int64_t n,
                                            int32_t accum_steps, float max_norm,
                                            const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                            void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  if (!valid_dtype(dtype)) return fail(ZDS_EINVAL, "zds_overflow_and_norm: bad dtype");
  if (n < 0) return fail(ZDS_EINVAL, "zds_overflow_and_norm: n < 0");
  if (accum_steps < 1) return fail(ZDS_EINVAL, "zds_overflow_and_norm: accum_steps must be >= 1");
  if (!state_dev || !out_dev) return fail(ZDS_EINVAL, "zds_overflow_and_norm: null state or output");
  if (!aligned(state_dev, 8) || !aligned(out_dev, 8))
    return fail(ZDS_EALIGN, "zds_overflow_and_norm: state/output not 8-byte aligned");
  if (n > 0 && !grads) return fail(ZDS_EINVAL, "zds_overflow_and_norm: null grads");
  if (n > 0 && !aligned(grads, static_cast<uintptr_t>(dtype_size(dtype))))
    return fail(ZDS_EALIGN, "zds_overflow_and_norm: grads misaligned");
  if (!ws || ws_bytes < zds_workspace_bytes(n) || !aligned(ws, 8))
    return fail(ZDS_EINVAL, "zds_overflow_and_norm: workspace of %zu bytes needed (8-byte aligned)", zds_workspace_bytes(n));
  // n == 0 still writes the scalars: the norm of an empty shard is 0.
  return launch_norm(grads, dtype, n, accum_steps, max_norm, state_dev, out_dev,
                     static_cast<double *>(ws), static_cast<hipStream_t>(stream));
}

extern "C" zds_status zds_adam_step(const zds_adamw_hparams *hp, const void *grads, zds_dtype grad_dtype,
                                    float *master, float *exp_avg, float *exp_avg_sq, void *params_out,
                                    zds_dtype param_dtype, int64_t n, zds_step_scalars *scalars_dev,
                                    const zds_step_state *state_dev, void *stream) {
  clear_error();
  if (!hp) return fail(ZDS_EINVAL, "zds_adam_step: null hparams");
  if (!valid_dtype(grad_dtype)) return fail(ZDS_EINVAL, "zds_adam_step: bad grad dtype");
  if (params_out && param_dtype != ZDS_FP16 && param_dtype != ZDS_BF16)
    return fail(ZDS_EINVAL, "zds_adam_step: param dtype must be fp16 or bf16");
  if (n < 0) return fail(ZDS_EINVAL, "zds_adam_step: n < 0");
  if (n >= (int64_t(1) << 40)) return fail(ZDS_EINVAL, "zds_adam_step: n must be below 2^40");
  if (!(hp->beta1 >= 0.5f && hp->beta1 < 1.0f && hp->beta2 >= 0.5f && hp->beta2 < 1.0f))
    return fail(ZDS_EINVAL, "zds_adam_step: betas must lie in [0.5, 1)");
  if (!(hp->eps > 0.0f) || !(hp->lr >= 0.0f) || !(hp->weight_decay >= 0.0f))
    return fail(ZDS_EINVAL, "zds_adam_step: need eps > 0, lr >= 0, weight_decay >= 0");
  if (n == 0) return ZDS_OK;
  if (!grads || !master || !exp_avg || !exp_avg_sq || !scalars_dev || !state_dev)
    return fail(ZDS_EINVAL, "zds_adam_step: null pointer");
  if (!aligned(grads, static_cast<uintptr_t>(dtype_size(grad_dtype))) || !aligned(master, 4) ||
      !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || (params_out && !aligned(params_out, 2)) ||
      !aligned(scalars_dev, 8) || !aligned(state_dev, 8))
    return fail(ZDS_EALIGN, "zds_adam_step: pointer not aligned to its element size");
  return launch_adam(*hp, grads, grad_dtype, master, exp_avg, exp_avg_sq, params_out, param_dtype, n,
                     scalars_dev, state_dev, static_cast<hipStream_t>(stream));
}

static zds_status check_cfg(const zds_scaler_config *cfg) {
  if (!cfg) return fail(ZDS_EINVAL, "null scaler config");
  if (cfg->dynamic) {
    if (cfg->window < 1 || cfg->hysteresis < 1)
      return fail(ZDS_EINVAL, "scaler config: window and hysteresis must be >= 1");
    if (cfg->initial_scale_power < -126 || cfg->initial_scale_power > 127)
      return fail(ZDS_EINVAL, "scaler config: initial_scale_power out of fp32 range");
    if (!(cfg->min_scale > 0.0f)) return fail(ZDS_EINVAL, "scaler config: min_scale must be > 0");
  } else if (!(cfg->static_scale > 0.0f)) {
    return fail(ZDS_EINVAL, "scaler config: static_scale must be > 0");
  }
  return ZDS_OK;
}

extern "C" zds_status zds_step_state_init(zds_step_state *state_dev, const zds_scaler_config *cfg,
                                          int64_t t0, double beta1_pow0, double beta2_pow0, void *stream) {
  clear_error();
  if (!state_dev) return fail(ZDS_EINVAL, "zds_step_state_init: null state");
  if (!aligned(state_dev, 8)) return fail(ZDS_EALIGN, "zds_step_state_init: state not 8-byte aligned");
  zds_status s = check_cfg(cfg);
  if (s != ZDS_OK) return s;
  if (t0 < 0) return fail(ZDS_EINVAL, "zds_step_state_init: t0 < 0");
  zds_step_state init;
  state_from_config(init, *cfg, t0, beta1_pow0, beta2_pow0);
  return launch_state_init(state_dev, init, static_cast<hipStream_t>(stream));
}

extern "C" zds_status zds_loss_scaler_update(zds_step_state *state_dev, const zds_step_scalars *scalars_dev,
                                             const zds_adamw_hparams *hp, void *stream) {
  clear_error();
  if (!state_dev || !scalars_dev || !hp) return fail(ZDS_EINVAL, "zds_loss_scaler_update: null argument");
  if (!aligned(state_dev, 8) || !aligned(scalars_dev, 8))
    return fail(ZDS_EALIGN, "zds_loss_scaler_update: state/scalars not 8-byte aligned");
  return launch_scaler(state_dev, scalars_dev, hp->beta1, hp->beta2, static_cast<hipStream_t>(stream));
}

extern "C" zds_status zds_step_state_init_host(zds_step_state *state, const zds_scaler_config *cfg,
                                               int64_t t0, double beta1_pow0, double beta2_pow0) {
  clear_error();
  if (!state) return fail(ZDS_EINVAL, "zds_step_state_init_host: null state");
  zds_status s = check_cfg(cfg);
  if (s != ZDS_OK) return s;
  if (t0 < 0) return fail(ZDS_EINVAL, "zds_step_state_init_host: t0 < 0");
  state_from_config(*state, *cfg, t0, beta1_pow0, beta2_pow0);
  return ZDS_OK;
}

extern "C" zds_status zds_loss_scaler_update_host(zds_step_state *state, uint32_t overflow,
                                                  const zds_adamw_hparams *hp) {
  clear_error();
  if (!state || !hp) return fail(ZDS_EINVAL, "zds_loss_scaler_update_host: null argument");
  scaler_transition(*state, overflow ? 1u : 0u, hp->beta1, hp->beta2);
  return ZDS_OK;
}

extern "C" zds_status zds_adam_constants_host(const zds_adamw_hparams *hp, const zds_step_state *state,
                                              float *out5) {
  clear_error();
  if (!hp || !state || !out5) return fail(ZDS_EINVAL, "zds_adam_constants_host: null argument");
  const AdamConsts c = adam_constants(*hp, state->beta1_pow, state->beta2_pow);
  out5[0] = c.step_size;
  out5[1] = c.bc2_sqrt;
  out5[2] = c.decay;
  out5[3] = c.omb1;
  out5[4] = c.omb2;
  return ZDS_OK;
}

extern "C" zds_status zds_clip_scalars_host(double sumsq, float scale, int32_t accum_steps, float max_norm,
                                            zds_step_scalars *out) {
  clear_error();
  if (!out) return fail(ZDS_EINVAL, "zds_clip_scalars_host: null output");
  if (accum_steps < 1) return fail(ZDS_EINVAL, "zds_clip_scalars_host: accum_steps must be >= 1");
  *out = zds_step_scalars{};
  clip_scalars(sumsq, scale, accum_steps, max_norm, *out);
  return ZDS_OK;
}

extern "C" const char *zds_last_error(void) { return g_err.c_str(); }

extern "C" const char *zds_status_string(zds_status s) {
  switch (s) {
    case ZDS_OK: return "ok";
    case ZDS_EINVAL: return "invalid argument";
    case ZDS_EALIGN: return "misaligned pointer";
    case ZDS_ENOMEM: return "out of memory";
    case ZDS_EHIP: return "HIP error";
    case ZDS_EIO: return "file error";
  }
  return "unknown status";
}

extern "C" int32_t zds_abi_version(void) { return ZDS_ABI_VERSION; }

static_assert(sizeof(zds_step_state) == 64, "zds_step_state is 64 bytes");
static_assert(sizeof(zds_step_scalars) == 64, "zds_step_scalars is 64 bytes");
static_assert(sizeof(zds_checkpoint_meta) == 48, "zds_checkpoint_meta is 48 bytes");
