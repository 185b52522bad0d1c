// 1-bit compression with error compensation (a next row): the rank-local
// encode and decode of a sign-compressed exchange. 1-bit Adam sends only the
// sign of each element and compensates the compression error afterwards
// (devpress.csdn.net DeepSpeed tutorial §4.2, 通信压缩).
//
// Encode, per chunk of C elements (C a multiple of 1024; the last chunk may
// be shorter): c = x + error (fp32), scale s = fp32(sqrt(sum c^2 / len)) with
// the squares summed in float64, sign bit 1 for c >= 0, new error = c - s
// (bit 1) or c + s (bit 0).
// Sign words are wave lane masks: bit l of 64-bit word 4g + i is element
// 256g + 4l + i, i.e. when lane l of a wave holds quad l of group g, word
// 4g + i is the ballot of the lanes' i-th sign. The encoder writes a word
// with one ballot; the decoder uses it directly as the per-lane condition of
// a select between s and -s.
// Decode: the fp32 sum over peers, in peer order, of +-s per element.
//
// Both are HBM-bound streams. Encode moves 12 B/element (read x and error,
// write error) plus 1/8 B of signs and 4/C B of scales; one block owns one
// chunk at a time and keeps its c values in registers across the
// block-wide sum. Decode moves N/8 + 4N/C B of payload plus 4 B out (8 B
// when adding to the destination); its vector work per element and peer is
// two readlanes (the sign word into scalar registers), one select and one
// add, so with many peers it is bound by issue rather than by HBM.
#include "zds_device.h"
#include "zds_onebit.h"

namespace zds {

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const uint64_t *words[kMaxPeers];
  const float *scales[kMaxPeers];
  int32_t npeers;
  int64_t n;
  int32_t chunk_shift;  // chunk = 1 << chunk_shift
  float *dst;
};

// R = chunk / 1024: quads per thread per chunk. EF: an error buffer is given.
// Iteration r of a chunk: wave w's lane l holds quad 256 r + 64 w + l, i.e.
// quad l of group (chunk base / 256) + 4 r + w.
template <int R, bool EF>
__global__ void __launch_bounds__(256) onebit_encode_kernel(const float *__restrict__ x, float *__restrict__ err,
                                                            uint64_t *__restrict__ words,
                                                            float *__restrict__ scales, int64_t n) {
  constexpr int64_t C = 1024 * R;
  __shared__ float s_sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nchunks = (n + C - 1) / C;
  for (int64_t j = blockIdx.x; j < nchunks; j += gridDim.x) {  // uniform per block
    const int64_t base = j * C;
    const int64_t len = n - base < C ? n - base : C;
    float c[R][4];
    bool full[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t e0 = base + 4 * (r * 256 + tid);
      full[r] = e0 + 4 <= n;
      if (full[r]) {
        const f32x4 a = ld_stream(reinterpret_cast<const f32x4 *>(x + e0));
        c[r][0] = a.x; c[r][1] = a.y; c[r][2] = a.z; c[r][3] = a.w;
        if (EF) {
          const f32x4 b = ld_stream(reinterpret_cast<const f32x4 *>(err + e0));
          c[r][0] = c[r][0] + b.x; c[r][1] = c[r][1] + b.y; c[r][2] = c[r][2] + b.z; c[r][3] = c[r][3] + b.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[r][i] = 0.0f;
          if (e0 + i < n) c[r][i] = EF ? x[e0 + i] + err[e0 + i] : x[e0 + i];
        }
      }
    }
    double ss = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double d = c[r][i];
        ss = ss + d * d;  // the square of an fp32 value is exact in float64
      }
    const double total = block_sum<256>(ss);
    if (tid == 0) {
      const float s = static_cast<float>(sqrt(total / static_cast<double>(len)));
      s_sh = s;
      scales[j] = s;
    }
    __syncthreads();
    const float s = s_sh;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t e0 = base + 4 * (r * 256 + tid);
      bool pos[4];
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pos[i] = c[r][i] >= 0.0f && e0 + i < n;
        e[i] = pos[i] ? c[r][i] - s : c[r][i] + s;
      }
      if (EF) {
        if (full[r]) {
          const f32x4 o = {e[0], e[1], e[2], e[3]};
          st_stream(reinterpret_cast<f32x4 *>(err + e0), o);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e0 + i < n) err[e0 + i] = e[i];
        }
      }
      const uint64_t m0 = __ballot(pos[0]), m1 = __ballot(pos[1]);
      const uint64_t m2 = __ballot(pos[2]), m3 = __ballot(pos[3]);
      const int64_t g = (base >> 8) + 4 * r + wave;
      if (lane < 2 && (g << 8) < n) {  // 32 bytes of words per group, 16 per lane
        const u64x2 v = lane == 0 ? u64x2{m0, m1} : u64x2{m2, m3};
        *reinterpret_cast<u64x2 *>(words + 4 * g + 2 * lane) = v;
      }
    }
  }
}

// Wave w of block b decodes U consecutive groups (U = 2 for up to 8 peers,
// else 1), starting at group U (4 b + w) and moving on by 4 U groups per
// block of the grid; lane l takes quad l of each group. One vector load per
// iteration brings all signs and scales of the U groups: lane t loads sign
// word i = t % 4 of peer k = (t / 4) % NP for group t / (4 NP), and lane
// t < U NP one scale. Each word then reaches scalar registers by readlane and
// serves as the select condition of one element per lane. The next
// iteration's loads are issued before this one's decode.
template <bool ACC, int NP>
__global__ void __launch_bounds__(256) onebit_decode_kernel(DecodeArgs a) {
  constexpr int U = NP <= 8 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ngroups = (a.n + 255) >> 8;
  const int wk = (lane >> 2) % NP, wu = lane / (4 * NP), wi = lane & 3;
  const int sk = lane % NP, su = lane / NP;
  const uint64_t *myw = a.words[0];
  const float *mys = a.scales[0];
#pragma unroll
  for (int k = 1; k < NP; ++k) {
    if (wk == k) myw = a.words[k];
    if (sk == k) mys = a.scales[k];
  }
  const int64_t step = U * 4 * static_cast<int64_t>(gridDim.x);
  int64_t g = U * (4 * static_cast<int64_t>(blockIdx.x) + wave);
  auto fetch = [&](int64_t g0, uint64_t &w, float &sc) {
    const int64_t gw = g0 + wu, gs = g0 + su;
    if (wu < U && gw < ngroups) w = myw[4 * gw + wi];
    if (su < U && gs < ngroups) sc = mys[(gs << 8) >> a.chunk_shift];
  };
  uint64_t w = 0;
  float sc = 0.0f;
  if (g < ngroups) fetch(g, w, sc);
  for (; g < ngroups; g += step) {
    uint64_t wn = 0;
    float scn = 0.0f;
    if (g + step < ngroups) fetch(g + step, wn, scn);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t gg = g + u;
      if (gg >= ngroups) break;
      const int64_t e0 = (gg << 8) + 4 * lane;
      float acc[4];
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), u * NP + k));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int src = 4 * (u * NP + k) + i;
          const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(w & 0xffffffffu), src);
          const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(w >> 32), src);
          const uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
          const float d = __builtin_amdgcn_inverse_ballot_w64(m) ? s : -s;
          acc[i] = k == 0 ? d : acc[i] + d;
        }
      }
      if (e0 + 4 <= a.n) {
        f32x4 o = {acc[0], acc[1], acc[2], acc[3]};
        if (ACC) {
          const f32x4 old = ld_stream(reinterpret_cast<const f32x4 *>(a.dst + e0));
          o = f32x4{old.x + acc[0], old.y + acc[1], old.z + acc[2], old.w + acc[3]};
        }
        st_stream(reinterpret_cast<f32x4 *>(a.dst + e0), o);
      } else {
        for (int i = 0; i < 4 && e0 + i < a.n; ++i) a.dst[e0 + i] = ACC ? a.dst[e0 + i] + acc[i] : acc[i];
      }
    }
    w = wn;
    sc = scn;
  }
}

template <int R>
static void encode_go(const float *x, float *err, uint64_t *words, float *scales, int64_t n, hipStream_t s) {
  int64_t g = (n + 1024 * R - 1) / (1024 * R);
  if (g > max_blocks(256)) g = max_blocks(256);
  if (err)
    hipLaunchKernelGGL((onebit_encode_kernel<R, true>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, x, err,
                       words, scales, n);
  else
    hipLaunchKernelGGL((onebit_encode_kernel<R, false>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, x, err,
                       words, scales, n);
}

zds_status launch_onebit_encode(const float *x, float *err, int64_t n, int32_t chunk, uint64_t *words, float *scales,
                                hipStream_t s) {
  switch (chunk / 1024) {
    case 1: encode_go<1>(x, err, words, scales, n, s); break;
    case 2: encode_go<2>(x, err, words, scales, n, s); break;
    case 4: encode_go<4>(x, err, words, scales, n, s); break;
    case 8: encode_go<8>(x, err, words, scales, n, s); break;
    case 16: encode_go<16>(x, err, words, scales, n, s); break;
    default: return fail(ZDS_EINVAL, "onebit encode: chunk %d is not 1024, 2048, 4096, 8192 or 16384", chunk);
  }
  return check_launch("onebit encode kernel");
}

template <bool ACC, int NP>
static void decode_go(const DecodeArgs &a, int64_t g, hipStream_t s) {
  hipLaunchKernelGGL((onebit_decode_kernel<ACC, NP>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a);
}

template <bool ACC>
static void decode_np(const DecodeArgs &a, int64_t g, hipStream_t s) {
  switch (a.npeers) {
    case 1: decode_go<ACC, 1>(a, g, s); break;
    case 2: decode_go<ACC, 2>(a, g, s); break;
    case 3: decode_go<ACC, 3>(a, g, s); break;
    case 4: decode_go<ACC, 4>(a, g, s); break;
    case 5: decode_go<ACC, 5>(a, g, s); break;
    case 6: decode_go<ACC, 6>(a, g, s); break;
    case 7: decode_go<ACC, 7>(a, g, s); break;
    case 8: decode_go<ACC, 8>(a, g, s); break;
    case 9: decode_go<ACC, 9>(a, g, s); break;
    case 10: decode_go<ACC, 10>(a, g, s); break;
    case 11: decode_go<ACC, 11>(a, g, s); break;
    case 12: decode_go<ACC, 12>(a, g, s); break;
    case 13: decode_go<ACC, 13>(a, g, s); break;
    case 14: decode_go<ACC, 14>(a, g, s); break;
    case 15: decode_go<ACC, 15>(a, g, s); break;
    default: decode_go<ACC, 16>(a, g, s); break;
  }
}

zds_status launch_onebit_decode(const uint64_t *const *words, const float *const *scales, int32_t npeers, int64_t n,
                                int32_t chunk, float *dst, bool accumulate, hipStream_t s) {
  DecodeArgs a{};
  for (int k = 0; k < npeers; ++k) {
    a.words[k] = words[k];
    a.scales[k] = scales[k];
  }
  a.npeers = npeers;
  a.n = n;
  a.chunk_shift = 0;
  while ((1 << a.chunk_shift) < chunk) ++a.chunk_shift;
  a.dst = dst;
  const int64_t per_block = 4 * (npeers <= 8 ? 2 : 1);  // groups of 256 elements per block
  int64_t g = ((n + 255) / 256 + per_block - 1) / per_block;
  if (g > max_blocks(256)) g = max_blocks(256);
  if (accumulate) decode_np<true>(a, g, s);
  else decode_np<false>(a, g, s);
  return check_launch("onebit decode kernel");
}

}  // namespace zds
