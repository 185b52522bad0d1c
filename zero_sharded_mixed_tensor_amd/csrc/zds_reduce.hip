// Stage-2 reduce-scatter intake on one rank: the sum over N peers of their
// copies of this rank's gradient slice, into the rank's fp32 (or 16-bit)
// shard gradient. Under Stage 2 the grads are reduce-scattered instead of
// all-reduced (aidhplus.com "DeepSpeed", ZeRO-2 section;
// jwzheng96.github.io llm-train-tutorials ch01, §1.2 table); this is the
// arithmetic a rank does with the slices it receives.
//
// Sum order: fp32, peer 0 first, one round-to-nearest add per peer; with
// ZDS_ACCUMULATE the previous destination value is added last; a 16-bit
// destination is rounded once at the end.
//
// HBM-bound: 2N (16-bit peers) + 4 (fp32 out) [+ 4 when accumulating] bytes
// per element. Wave-specialised like the Adam kernel: a block of 4 waves owns
// a tile of 512 elements; wave w loads peers w, w+4, w+8, w+12 (one
// contiguous 1 KiB wave-wide access each) and a share of the destination
// tile, the tiles meet in LDS where each thread sums 2 elements over the
// peers in order, and waves 0 and 1 store the result. A block takes one
// tile (blocks loop only past the grid cap).
//
// NORM (the step's overflow / norm pass fused in): each thread adds the
// float64 square of every value it stores (the rounded value for a 16-bit
// destination) and each block writes one partial sum, so the shard gradient
// is not read a second time.
#include "zds_device.h"
#include "zds_internal.h"

namespace zds {

// Consecutive tiles a block takes per grid step, with or without the norm
// fused in. One: each block streams one tile and ends (8 peers into fp32,
// library builds swapped between bench runs, three rounds on one box: 2.52
// ms against 2.69-2.73 with 2 tiles; with the norm fused in 2.55-2.65 against
// 2.73-2.82 with 2 tiles and 2.93-2.96 with 4). When each wave's peer loads
// were still serialised by the compiler (below), 2 and 4 tiles per block had
// measured best. Blocks loop only past the grid cap.
constexpr int kReduceTilesPerBlock = 1;

struct ReduceArgs {
  const void *peers[kMaxPeers];
  int32_t npeers;
  int64_t n;
  void *dst;
  double *partials;  // NORM: one sum of squares per block
};

template <int SD>
__device__ __forceinline__ float widen16(uint16_t h) {
  return SD == ZDS_BF16 ? __uint_as_float(static_cast<uint32_t>(h) << 16)
                        : __half2float(__ushort_as_half(h));
}

// SD: peer dtype (16-bit). DD: destination dtype (fp32 or SD). ACC: add the
// destination's previous value. S = ceil(npeers / 4): the peer slots of each
// wave (wave w takes peers w, w + 4, ...).
template <int SD, int DD, bool ACC, bool NORM, int S>
__global__ void __launch_bounds__(256) reduce_peers_kernel(ReduceArgs a) {
  __shared__ u32x4 sx[kMaxPeers][64];     // peer tiles, 512 x 16-bit each
  __shared__ f32x4 sd[DD == ZDS_FP32 ? 128 : 1];  // fp32 destination tile
  __shared__ u32x4 sh[DD == ZDS_FP32 ? 1 : 64];   // 16-bit destination tile
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: peer pointers by scalar loads
  const int N = a.npeers;
  const int64_t g8 = a.n >> 3;  // whole groups of 8 elements
  const int64_t ntiles = (g8 + 63) >> 6;
  constexpr int TPB = kReduceTilesPerBlock;
  double ss = 0.0;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * TPB; it < ntiles; it += static_cast<int64_t>(gridDim.x) * TPB)
  for (int64_t tile = it; tile < it + TPB && tile < ntiles; ++tile) {  // uniform per block
    const int64_t grp = tile * 64 + lane;  // this lane's 8-element group
    const bool gok = grp < g8;
    u32x4 r[S];
#pragma unroll
    for (int s = 0; s < S; ++s) r[s] = u32x4{0u, 0u, 0u, 0u};
    if (tile * 64 + 64 <= g8) {
      // A whole tile: the wave's S loads issue back to back with no condition
      // (a slot past the last peer reloads peer 0 and is never summed). With a
      // per-lane guard around each, and the wave index taken as varying per
      // lane (so each peer pointer was a vector load), the compiler waited for
      // every load before issuing the next.
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int k = w + 4 * s;
        r[s] = ld_stream(static_cast<const u32x4 *>(a.peers[k < N ? k : 0]) + grp);
      }
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int k = w + 4 * s;
        if (k < N && gok) r[s] = ld_stream(static_cast<const u32x4 *>(a.peers[k]) + grp);
      }
    }
    // fp32 destination quads of the tile: q = tile*128 + {0..127}; waves 2, 3
    // load them when accumulating (quad j of the tile holds elements 4j..4j+3)
    const int64_t dq = tile * 128 + (w & 1) * 64 + lane;
    const bool dqok = dq < 2 * g8;
    f32x4 dr;
    u32x4 dh;
    if (ACC) {
      if (DD == ZDS_FP32) {
        if (w >= 2 && dqok) dr = ld_stream(static_cast<const f32x4 *>(a.dst) + dq);
      } else if (w == 3 && gok) {
        dh = ld_stream(static_cast<const u32x4 *>(a.dst) + grp);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) sx[w + 4 * s][lane] = r[s];  // slots past the peers or the tile are never read
    if (ACC) {
      if (DD == ZDS_FP32) {
        if (w >= 2 && dqok) sd[(w & 1) * 64 + lane] = dr;
      } else if (w == 3 && gok) {
        sh[lane] = dh;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = threadIdx.x + 256 * h;  // element of the tile
      if (tile * 64 + (e >> 3) < g8) {
        float acc = widen16<SD>(reinterpret_cast<const uint16_t *>(sx[0])[e]);
        for (int k = 1; k < N; ++k) acc = acc + widen16<SD>(reinterpret_cast<const uint16_t *>(sx[k])[e]);
        if constexpr (DD == ZDS_FP32) {
          float *o = reinterpret_cast<float *>(sd);
          const float r = ACC ? o[e] + acc : acc;
          o[e] = r;
          if (NORM) ss = sq_add(r, ss);
        } else {
          uint16_t *o = reinterpret_cast<uint16_t *>(sh);
          const float r2 = ACC ? widen16<DD>(o[e]) + acc : acc;
          const uint16_t h = narrow1<DD>(r2);
          o[e] = h;
          if (NORM) ss = sq_add(widen16<DD>(h), ss);
        }
      }
    }
    __syncthreads();
    if (DD == ZDS_FP32) {
      if (w < 2 && dqok) st_stream(static_cast<f32x4 *>(a.dst) + dq, sd[w * 64 + lane]);
    } else if (w == 0 && gok) {
      st_stream(static_cast<u32x4 *>(a.dst) + grp, sh[lane]);
    }
    // waves 2 and 3 write the destination tile of the next iteration
    // (accumulate mode) while waves 0 and 1 may still read this one
    __syncthreads();
  }
  // Ragged tail: the last n % 8 elements, one per lane of block 0.
  const int64_t tail0 = g8 << 3;
  if (blockIdx.x == 0 && tail0 + threadIdx.x < a.n) {
    const int64_t e = tail0 + threadIdx.x;
    float acc = widen1<SD>(a.peers[0], e);
    for (int k = 1; k < N; ++k) acc = acc + widen1<SD>(a.peers[k], e);
    if constexpr (DD == ZDS_FP32) {
      float *o = static_cast<float *>(a.dst);
      const float r = ACC ? o[e] + acc : acc;
      o[e] = r;
      if (NORM) ss = sq_add(r, ss);
    } else {
      uint16_t *o = static_cast<uint16_t *>(a.dst);
      const float r2 = ACC ? widen1<DD>(a.dst, e) + acc : acc;
      const uint16_t h = narrow1<DD>(r2);
      o[e] = h;
      if (NORM) ss = sq_add(widen16<DD>(h), ss);
    }
  }
  if (NORM) {
    const double b = block_sum<256>(ss);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = b;
  }
}

// Element-wise path for peers or destinations without 16-byte alignment.
template <int SD, int DD, bool ACC, bool NORM>
__global__ void __launch_bounds__(256) reduce_peers_scalar(ReduceArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  double ss = 0.0;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < a.n; e += stride) {
    float acc = widen1<SD>(a.peers[0], e);
    for (int k = 1; k < a.npeers; ++k) acc = acc + widen1<SD>(a.peers[k], e);
    if constexpr (DD == ZDS_FP32) {
      float *o = static_cast<float *>(a.dst);
      const float r = ACC ? o[e] + acc : acc;
      o[e] = r;
      if (NORM) ss = sq_add(r, ss);
    } else {
      uint16_t *o = static_cast<uint16_t *>(a.dst);
      const float r2 = ACC ? widen1<DD>(a.dst, e) + acc : acc;
      const uint16_t h = narrow1<DD>(r2);
      o[e] = h;
      if (NORM) ss = sq_add(widen16<DD>(h), ss);
    }
  }
  if (NORM) {
    const double b = block_sum<256>(ss);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = b;
  }
}

// Grid of the intake kernels (also the number of partials the fused norm
// writes).
static int64_t reduce_grid(int64_t n, bool vec, bool norm) {
  if (vec) {
    const int tpb = kReduceTilesPerBlock;
    int64_t g = (((n >> 3) + 63) / 64 + tpb - 1) / tpb;
    if (g < 1) g = 1;
    if (g > max_blocks(256)) g = max_blocks(256);
    return g;
  }
  int64_t g = (n + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return g;
}

int64_t reduce_grid_max(int64_t n) {
  const int64_t a = reduce_grid(n, true, true), b = reduce_grid(n, false, true);
  return a > b ? a : b;
}

template <int SD, int DD, bool ACC, bool NORM>
static void go(bool vec, int64_t g, hipStream_t s, const ReduceArgs &a) {
  if (vec) {
    switch ((a.npeers + 3) / 4) {
      case 1: hipLaunchKernelGGL((reduce_peers_kernel<SD, DD, ACC, NORM, 1>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((reduce_peers_kernel<SD, DD, ACC, NORM, 2>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a); break;
      case 3: hipLaunchKernelGGL((reduce_peers_kernel<SD, DD, ACC, NORM, 3>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((reduce_peers_kernel<SD, DD, ACC, NORM, 4>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a); break;
    }
  } else
    hipLaunchKernelGGL((reduce_peers_scalar<SD, DD, ACC, NORM>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a);
}

template <int SD, bool NORM>
static void go_sd(zds_dtype dd, bool acc, bool vec, int64_t g, hipStream_t s, const ReduceArgs &a) {
  if (dd == ZDS_FP32) {
    if (acc) go<SD, ZDS_FP32, true, NORM>(vec, g, s, a); else go<SD, ZDS_FP32, false, NORM>(vec, g, s, a);
  } else {
    if (acc) go<SD, SD, true, NORM>(vec, g, s, a); else go<SD, SD, false, NORM>(vec, g, s, a);
  }
}

zds_status launch_reduce_peers(const void *const *peers, int32_t npeers, zds_dtype src, int64_t n, void *dst,
                               zds_dtype dst_dtype, bool accumulate, double *partials, int64_t *nparts,
                               hipStream_t stream) {
  ReduceArgs a{};
  bool vec = aligned(dst, 16);
  for (int k = 0; k < npeers; ++k) {
    a.peers[k] = peers[k];
    vec = vec && aligned(peers[k], 16);
  }
  a.npeers = npeers;
  a.n = n;
  a.dst = dst;
  a.partials = partials;
  const int64_t g = reduce_grid(n, vec, partials != nullptr);
  if (nparts) *nparts = g;
  if (partials) {
    if (src == ZDS_BF16) go_sd<ZDS_BF16, true>(dst_dtype, accumulate, vec, g, stream, a);
    else go_sd<ZDS_FP16, true>(dst_dtype, accumulate, vec, g, stream, a);
  } else {
    if (src == ZDS_BF16) go_sd<ZDS_BF16, false>(dst_dtype, accumulate, vec, g, stream, a);
    else go_sd<ZDS_FP16, false>(dst_dtype, accumulate, vec, g, stream, a);
  }
  return check_launch(partials ? "reduce_peer_slices_norm kernel" : "reduce_peer_slices kernel");
}

}  // namespace zds
