// Row a1: multi-tensor flatten / accumulate into the rank's flat buffer.
//
// Backward produces many small gradient tensors; packing them into one
// contiguous bucket (devpress.csdn.net DeepSpeed tutorial §3.2,
// contiguous_gradients; aiqz.cc "DeepSpeed ZeRO引擎深入", 通信优化) and summing
// micro-batches in memory before a single update (same tutorial §2.3) are done
// here in one launch over the plan's device-side tensor table.
//
// Work is cut into chunks of kAccumChunk (4096) elements that never straddle
// two table entries; the plan's table maps every chunk to its entry, so a
// block finds its piece with two rounds of uniform scalar loads. Copy mode
// moves 8 elements per lane (16-byte accesses); the fp32 modes move quads
// (8-byte 16-bit loads, 16-byte fp32 accesses), lane l on quad l of a wave's
// range so each wave-level access is contiguous. Unaligned entries fall back
// to element-wise moves. Bytes per element: copy 2+2, overwrite 2+4,
// accumulate 2+4+4. A block takes a whole chunk in copy mode (2 accesses per
// lane), half a chunk in overwrite mode and a quarter chunk in accumulate
// mode (1 quad per lane), and issues all of its vector loads before its
// first store (overwrite: see parts_per_chunk). Measured on the 7B shard
// against 8192-element chunks (whole / half): copy with the fused norm
// 0.535 vs 0.543-0.564 ms, 16 accumulated micro-batches 20.5 vs 21.1-22.2 ms,
// the whole 7B model's flatten 4.08-4.15 vs 4.36-4.45 ms. Small units pay
// only because the lookups are scalar loads (see unit_piece).
#include "zds_device.h"
#include "zds_internal.h"

namespace zds {

// Threads per block by mode. The grid has one block per work unit (a
// resident-size grid striding over the units measured slower), capped below
// 2^32 work-items per dispatch with a loop beyond.
constexpr int kAccBlock = 256;

struct AccArgs {
  const int64_t *table;
  int32_t num_entries;
  int64_t total_chunks;
  const void *const *ptrs;
  void *dst;
  double *partials;  // NORM: one sum of squares per block
};

// Work units per chunk. Copy mode takes a whole chunk per block (2 accesses
// of 8 elements per lane); accumulate a quarter chunk (one quad per lane: a
// 16-bit load, an fp32 load and an fp32 store); overwrite half a chunk (its
// block moves only 6 B per element, and with a quarter chunk the two rounds
// of table lookups at each block's start cost 15 %). With 16-bit sources
// that are 16-byte aligned, overwrite loads 8 elements per lane (1 KiB wave
// accesses), re-lays them out through LDS and stores two 1 KiB fp32 wave
// accesses one at a time: 776-778 against 789-790 us on the 7B shard (fp16
// sources, rocprofv3 traces, builds swapped, two rounds); otherwise two
// quads per lane (8-byte 16-bit loads).
// Measured on the 7B shard, fp16 sources, library builds swapped, two
// rounds: overwrite 0.90 ms (5,610 GB/s) with a quarter chunk, 0.80 ms
// (6,330 GB/s) with half a chunk, 0.84 with a whole chunk (4 quads per
// lane), 0.90-0.93 with 512- or 1024-thread blocks at one quad per lane;
// accumulate 1.30 ms (6,480 GB/s) with a quarter chunk against 1.37 / 1.44
// with half / whole chunks.
template <int MODE>
constexpr int parts_per_chunk() { return MODE == ZDS_COPY ? 1 : (MODE == ZDS_OVERWRITE ? 2 : 4); }
static_assert(kAccumChunk % (8 * 4) == 0, "a unit holds whole vector accesses in every mode");

// One work unit: where it reads and writes, and whether the vector path
// applies (both ends 16-byte aligned, or 8-byte for 16-bit sources of the
// fp32 modes).
struct Piece {
  const char *src;
  int64_t d0;   // destination element offset
  int64_t cnt;  // elements (0: nothing to do)
  bool vec;
};

// The plan's table and the call's pointer slots are written before the
// launch and never during it, so the kernel reads them through the constant
// address space: the uniform lookups then compile to scalar loads. (As plain
// global loads behind the previous unit's stores they became vector loads
// queued with the data stream, which made small units slow.)
typedef const __attribute__((address_space(4))) int64_t *ConstI64;
typedef const __attribute__((address_space(4))) char *const __attribute__((address_space(4))) *ConstPtrs;

// Unit u: part u % P of chunk u / P of its entry.
template <int SD, int MODE>
__device__ __forceinline__ Piece unit_piece(const AccArgs &a, int64_t u) {
  constexpr int P = parts_per_chunk<MODE>();
  constexpr int64_t span = kAccumChunk / P;
  const int32_t E = a.num_entries;
  // [start E][len E][dst E][chunk0 E+1][entry of each chunk]
  const ConstI64 t = (ConstI64)a.table;  // address-space cast
  const ConstPtrs ptrs = (ConstPtrs)a.ptrs;
  const int64_t c = u / P;
  const int64_t e = t[4 * E + 1 + c];
  const int64_t local = (c - t[3 * E + e]) * kAccumChunk + (u % P) * span;
  const int64_t rem = t[E + e] - local;
  Piece pc;
  pc.cnt = rem < 0 ? 0 : (rem < span ? rem : span);
  pc.src = (const char *)ptrs[e] + (t[e] + local) * (SD == ZDS_FP32 ? 4 : 2);
  pc.d0 = t[2 * E + e] + local;
  if (MODE == ZDS_COPY)
    pc.vec = aligned(pc.src, 16) && aligned(static_cast<uint16_t *>(a.dst) + pc.d0, 16);
  else
    pc.vec = aligned(pc.src, SD == ZDS_FP32 ? 16 : 8) && aligned(static_cast<float *>(a.dst) + pc.d0, 16);
  return pc;
}

// MODE: ZDS_COPY (16-bit -> same 16-bit), ZDS_OVERWRITE / ZDS_ACCUMULATE
// (SD -> fp32). Every vector load of a block iteration is issued before its
// first store.
template <int SD, int MODE, bool NORM>
__global__ void __launch_bounds__(kAccBlock) accumulate_kernel(AccArgs a) {
  constexpr int P = parts_per_chunk<MODE>();
  constexpr int BLK = kAccBlock;
  constexpr int PER = MODE == ZDS_COPY ? 8 : 4;                         // elements per access
  constexpr int UPT = (kAccumChunk / P / PER + BLK - 1) / BLK;  // accesses per thread
  const int64_t units = a.total_chunks * P;
  double ss = 0.0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {  // uniform per block
    const Piece pc = unit_piece<SD, MODE>(a, u);
    if (MODE == ZDS_COPY) {
      const int64_t groups = pc.vec ? pc.cnt >> 3 : 0;
      const u32x4 *s4 = reinterpret_cast<const u32x4 *>(pc.src);
      u32x4 *d4 = reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.dst) + pc.d0);
      u32x4 w[UPT];
#pragma unroll
      for (int r = 0; r < UPT; ++r) {
        const int64_t i = threadIdx.x + r * BLK;
        if (i < groups) w[r] = ld_stream(s4 + i);
      }
#pragma unroll
      for (int r = 0; r < UPT; ++r) {
        const int64_t i = threadIdx.x + r * BLK;
        if (i < groups) {
          st_stream(d4 + i, w[r]);
          if (NORM) {
            ss = sq_add(lo_of<SD>(w[r].x), ss); ss = sq_add(hi_of<SD>(w[r].x), ss);
            ss = sq_add(lo_of<SD>(w[r].y), ss); ss = sq_add(hi_of<SD>(w[r].y), ss);
            ss = sq_add(lo_of<SD>(w[r].z), ss); ss = sq_add(hi_of<SD>(w[r].z), ss);
            ss = sq_add(lo_of<SD>(w[r].w), ss); ss = sq_add(hi_of<SD>(w[r].w), ss);
          }
        }
      }
      // the tail of a vector piece, or a whole unaligned one
      const uint16_t *s16 = reinterpret_cast<const uint16_t *>(pc.src);
      uint16_t *d16 = static_cast<uint16_t *>(a.dst) + pc.d0;
      for (int64_t j = (groups << 3) + threadIdx.x; j < pc.cnt; j += BLK) {
        d16[j] = s16[j];
        if (NORM) ss = sq_add(widen1<SD>(s16, j), ss);
      }
    } else if (MODE == ZDS_OVERWRITE && SD != ZDS_FP32 && aligned(pc.src, 16) && pc.vec) {
      // 16-bit sources 16-byte aligned: wave w converts elements
      // [512 w, 512 w + 512) of the unit; lane l loads 8 of them (one 1 KiB
      // wave access), the wave re-lays them out through LDS, and stores the
      // 2 KiB of fp32 as two 1 KiB wave accesses, the second issued after the
      // first has completed.
      __shared__ f32x4 xch[BLK / 64][128];
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int lane = threadIdx.x & 63;
      const int64_t groups = pc.cnt >> 3;  // whole 8-element groups of the unit
      const int64_t gi = 64 * w + lane;
      float *d32 = static_cast<float *>(a.dst) + pc.d0 + 512 * w;
      if (gi < groups) {
        float x[8];
        load8<SD == ZDS_FP32 ? ZDS_FP16 : SD>(pc.src, gi, x);  // (never reached for fp32)
        xch[w][2 * lane] = f32x4{x[0], x[1], x[2], x[3]};
        xch[w][2 * lane + 1] = f32x4{x[4], x[5], x[6], x[7]};
      }
      __builtin_amdgcn_wave_barrier();  // the wave's LDS writes before its reads
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int qi = lane + 64 * r;  // quad of the wave's 512 elements
        if (128 * w + qi < 2 * groups) {
          const f32x4 o = xch[w][qi];
          st_stream(reinterpret_cast<f32x4 *>(d32) + qi, o);
          if (NORM) {
            ss = sq_add(o.x, ss); ss = sq_add(o.y, ss); ss = sq_add(o.z, ss); ss = sq_add(o.w, ss);
          }
        }
        if (r == 0) wait_vmem();
      }
      __builtin_amdgcn_wave_barrier();  // reads done before the next unit's writes
      // the ragged tail of the unit
      const uint16_t *s16 = reinterpret_cast<const uint16_t *>(pc.src);
      float *t32 = static_cast<float *>(a.dst) + pc.d0;
      for (int64_t j = (groups << 3) + threadIdx.x; j < pc.cnt; j += BLK) {
        const float v = widen1<SD == ZDS_FP32 ? ZDS_FP16 : SD>(s16, j);
        t32[j] = v;
        if (NORM) ss = sq_add(v, ss);
      }
    } else {
      const int64_t quads = pc.vec ? pc.cnt >> 2 : 0;
      float *d32 = static_cast<float *>(a.dst) + pc.d0;
      float x[UPT][4], y[UPT][4];
#pragma unroll
      for (int r = 0; r < UPT; ++r) {
        const int64_t q = threadIdx.x + r * BLK;
        if (q < quads) {
          load_quad<SD>(pc.src, q, x[r]);
          if (MODE == ZDS_ACCUMULATE) load_quad<ZDS_FP32>(d32, q, y[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < UPT; ++r) {
        const int64_t q = threadIdx.x + r * BLK;
        if (q < quads) {
          if (MODE == ZDS_ACCUMULATE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[r][i] = y[r][i] + x[r][i];
          }
          store_quad(d32, q, x[r]);
          if (NORM) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = sq_add(x[r][i], ss);
          }
        }
      }
      // the tail of a vector piece, or a whole unaligned one
      for (int64_t j = (quads << 2) + threadIdx.x; j < pc.cnt; j += BLK) {
        const float v = widen1<SD>(pc.src, j);
        const float r = MODE == ZDS_ACCUMULATE ? d32[j] + v : v;
        d32[j] = r;
        if (NORM) ss = sq_add(r, ss);
      }
    }
  }
  if (NORM) {
    const double b = block_sum<BLK>(ss);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = b;
  }
}

template <int SD, int MODE, bool NORM>
static void go(int64_t grid, hipStream_t s, const AccArgs &a) {
  hipLaunchKernelGGL((accumulate_kernel<SD, MODE, NORM>), dim3(static_cast<uint32_t>(grid)), dim3(kAccBlock),
                     0, s, a);
}

int64_t accumulate_grid(int64_t total_chunks, zds_accum_mode mode) {
  const int parts = mode == ZDS_COPY ? parts_per_chunk<ZDS_COPY>()
                                     : (mode == ZDS_OVERWRITE ? parts_per_chunk<ZDS_OVERWRITE>()
                                                              : parts_per_chunk<ZDS_ACCUMULATE>());
  int64_t grid = total_chunks * parts;
  if (grid > max_blocks(kAccBlock)) grid = max_blocks(kAccBlock);
  if (grid < 1) grid = 1;
  return grid;
}

template <bool NORM>
static zds_status dispatch(const PlanDev &p, const void *const *dev_ptrs, zds_dtype src, void *dst,
                           zds_accum_mode mode, double *partials, hipStream_t stream) {
  AccArgs a{p.table, p.num_entries, p.total_chunks, dev_ptrs, dst, partials};
  const int64_t g = accumulate_grid(p.total_chunks, mode);
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
