// Row a1: multi-tensor flatten / accumulate into the rank's flat buffer.
//
// Backward produces many small gradient tensors; packing them into one
// contiguous bucket (devpress.csdn.net DeepSpeed tutorial §3.2,
// contiguous_gradients; aiqz.cc "DeepSpeed ZeRO引擎深入", 通信优化) and summing
// micro-batches in memory before a single update (same tutorial §2.3) are done
// here in one launch over the plan's device-side tensor table.
//
// Work is cut into chunks of kAccumChunk elements that never straddle two
// table entries; the plan's table maps every chunk to its entry, so a block
// finds its piece with a few uniform (scalar) loads. Copy mode moves 8
// elements per lane (16-byte accesses); the fp32 modes move quads (8-byte
// 16-bit loads, 16-byte fp32 accesses), lane l on quad l of a wave's range so
// each wave-level access is contiguous. Unaligned entries fall back to
// element-wise moves. Bytes per element: copy 2+2, overwrite 2+4,
// accumulate 2+4+4. One block per chunk by default.
#include "zds_device.h"
#include "zds_internal.h"

#ifndef ZDS_ACC_BLOCK
#define ZDS_ACC_BLOCK 256
#endif
#ifndef ZDS_ACC_WAVES_PER_CU
#define ZDS_ACC_WAVES_PER_CU 32
#endif
// 1: one block per chunk; 0: at most ZDS_ACC_WAVES_PER_CU waves per CU
// striding over the chunks.
#ifndef ZDS_ACC_ONESHOT
#define ZDS_ACC_ONESHOT 1
#endif

namespace zds {

struct AccArgs {
  const int64_t *table;
  int32_t num_entries;
  int64_t total_chunks;
  const void *const *ptrs;
  void *dst;
  double *partials;  // NORM: one sum of squares per block
};

__device__ __forceinline__ double sq_add(float x, double acc) {
  const double d = static_cast<double>(x);
  return fma(d, d, acc);  // x^2 is exact in float64
}

// MODE: ZDS_COPY (16-bit -> same 16-bit), ZDS_OVERWRITE / ZDS_ACCUMULATE
// (SD -> fp32).
template <int SD, int MODE, bool NORM>
__global__ void __launch_bounds__(ZDS_ACC_BLOCK) accumulate_kernel(AccArgs a) {
  double ss = 0.0;
  const int32_t E = a.num_entries;
  const int64_t *start = a.table;
  const int64_t *len = a.table + E;
  const int64_t *dsto = a.table + 2 * E;
  const int64_t *chunk0 = a.table + 3 * E;
  const int64_t *chunk_entry = a.table + 4 * E + 1;
  for (int64_t c = blockIdx.x; c < a.total_chunks; c += gridDim.x) {
    const int64_t e = chunk_entry[c];
    const int64_t local = (c - chunk0[e]) * kAccumChunk;
    const int64_t rem = len[e] - local;
    const int64_t cnt = rem < kAccumChunk ? rem : kAccumChunk;
    const char *src = static_cast<const char *>(a.ptrs[e]) + (start[e] + local) * (SD == ZDS_FP32 ? 4 : 2);
    const int64_t d0 = dsto[e] + local;
    if (MODE == ZDS_COPY) {
      uint16_t *dst = static_cast<uint16_t *>(a.dst) + d0;
      const uint16_t *s = reinterpret_cast<const uint16_t *>(src);
      if (aligned(s, 16) && aligned(dst, 16)) {
        const int64_t groups = cnt >> 3;
        for (int64_t i = threadIdx.x; i < groups; i += ZDS_ACC_BLOCK) {
          const u32x4 w = ld_stream(reinterpret_cast<const u32x4 *>(s) + i);
          st_stream(reinterpret_cast<u32x4 *>(dst) + i, w);
          if (NORM) {
            ss = sq_add(lo_of<SD>(w.x), ss); ss = sq_add(hi_of<SD>(w.x), ss);
            ss = sq_add(lo_of<SD>(w.y), ss); ss = sq_add(hi_of<SD>(w.y), ss);
            ss = sq_add(lo_of<SD>(w.z), ss); ss = sq_add(hi_of<SD>(w.z), ss);
            ss = sq_add(lo_of<SD>(w.w), ss); ss = sq_add(hi_of<SD>(w.w), ss);
          }
        }
        for (int64_t j = (groups << 3) + threadIdx.x; j < cnt; j += ZDS_ACC_BLOCK) {
          dst[j] = s[j];
          if (NORM) ss = sq_add(widen1<SD>(s, j), ss);
        }
      } else {
        for (int64_t j = threadIdx.x; j < cnt; j += ZDS_ACC_BLOCK) {
          dst[j] = s[j];
          if (NORM) ss = sq_add(widen1<SD>(s, j), ss);
        }
      }
    } else {
      float *dst = static_cast<float *>(a.dst) + d0;
      if (aligned(src, SD == ZDS_FP32 ? 16 : 8) && aligned(dst, 16)) {
        const int64_t quads = cnt >> 2;
        for (int64_t q = threadIdx.x; q < quads; q += ZDS_ACC_BLOCK) {
          float x[4];
          load_quad<SD>(src, q, x);
          if (MODE == ZDS_ACCUMULATE) {
            float y[4];
            load_quad<ZDS_FP32>(dst, q, y);
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = y[k] + x[k];
          }
          store_quad(dst, q, x);
          if (NORM) {
#pragma unroll
            for (int k = 0; k < 4; ++k) ss = sq_add(x[k], ss);
          }
        }
        for (int64_t j = (quads << 2) + threadIdx.x; j < cnt; j += ZDS_ACC_BLOCK) {
          const float x = widen1<SD>(src, j);
          const float r = MODE == ZDS_ACCUMULATE ? dst[j] + x : x;
          dst[j] = r;
          if (NORM) ss = sq_add(r, ss);
        }
      } else {
        for (int64_t j = threadIdx.x; j < cnt; j += ZDS_ACC_BLOCK) {
          const float x = widen1<SD>(src, j);
          const float r = MODE == ZDS_ACCUMULATE ? dst[j] + x : x;
          dst[j] = r;
          if (NORM) ss = sq_add(r, ss);
        }
      }
    }
  }
  if (NORM) {
    const double b = block_sum<ZDS_ACC_BLOCK>(ss);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = b;
  }
}

template <int SD, int MODE, bool NORM>
static void go(int64_t grid, hipStream_t s, const AccArgs &a) {
  hipLaunchKernelGGL((accumulate_kernel<SD, MODE, NORM>), dim3(static_cast<uint32_t>(grid)), dim3(ZDS_ACC_BLOCK),
                     0, s, a);
}

int64_t accumulate_grid(int64_t total_chunks) {
  int64_t grid = static_cast<int64_t>(device_cu_count()) * ZDS_ACC_WAVES_PER_CU * 64 / ZDS_ACC_BLOCK;
  if (ZDS_ACC_ONESHOT || grid > total_chunks) grid = total_chunks;
  if (grid > max_blocks(ZDS_ACC_BLOCK)) grid = max_blocks(ZDS_ACC_BLOCK);
  if (grid < 1) grid = 1;
  return grid;
}

template <bool NORM>
static zds_status dispatch(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src, void *dst,
                           zds_accum_mode mode, double *partials, hipStream_t stream) {
  AccArgs a{p.table, p.num_entries, p.total_chunks, dev_ptrs, dst, partials};
  const int64_t g = accumulate_grid(p.total_chunks);
  if (mode == ZDS_COPY) {
    // fp16 and bf16 copies move the same bits; the squares need the type
    if (src == ZDS_BF16) go<ZDS_BF16, ZDS_COPY, NORM>(g, stream, a);
    else go<ZDS_FP16, ZDS_COPY, NORM>(g, stream, a);
  } else if (mode == ZDS_OVERWRITE) {
    if (src == ZDS_FP16) go<ZDS_FP16, ZDS_OVERWRITE, NORM>(g, stream, a);
    else if (src == ZDS_BF16) go<ZDS_BF16, ZDS_OVERWRITE, NORM>(g, stream, a);
    else go<ZDS_FP32, ZDS_OVERWRITE, NORM>(g, stream, a);
  } else {
    if (src == ZDS_FP16) go<ZDS_FP16, ZDS_ACCUMULATE, NORM>(g, stream, a);
    else if (src == ZDS_BF16) go<ZDS_BF16, ZDS_ACCUMULATE, NORM>(g, stream, a);
    else go<ZDS_FP32, ZDS_ACCUMULATE, NORM>(g, stream, a);
  }
  return check_launch(NORM ? "grad_accumulate_norm kernel" : "grad_accumulate kernel");
}

zds_status launch_accumulate(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src,
                             void *dst, zds_dtype /*dst_dtype*/, zds_accum_mode mode,
                             hipStream_t stream) {
  if (p.num_entries == 0 || p.total_chunks == 0) return ZDS_OK;
  return dispatch<false>(p, dev_ptrs, src, dst, mode, nullptr, stream);
}

zds_status launch_accumulate_norm(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src,
                                  void *dst, zds_dtype /*dst_dtype*/, zds_accum_mode mode,
                                  double *partials, hipStream_t stream) {
  return dispatch<true>(p, dev_ptrs, src, dst, mode, partials, stream);
}

}  // namespace zds
