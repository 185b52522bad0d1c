// 1-bit compression with error compensation (a next row): the rank-local
// encode and decode of a sign-compressed exchange. 1-bit Adam sends only the
// sign of each element and compensates the compression error afterwards
// (devpress.csdn.net DeepSpeed tutorial §4.2, 通信压缩).
//
// Encode, per chunk of C elements (C a multiple of 1024; the last chunk may
// be shorter): c = x + error (fp32), scale s = fp32(sqrt(sum c^2 / len)) with
// the squares summed in float64, sign bit 1 for c >= 0, new error = c - s
// (bit 1) or c + s (bit 0).
// Sign words: 32 bits, 64 per unit of 2048 elements; bit 4r + i of word
// 64u + l is element 2048u + 256r + 4l + i. Word l of a unit thus holds the
// 32 signs of the elements a lane l touches when a wave walks the unit's
// eight 256-element groups one quad per lane: the encoder's lane l ORs its
// 4-bit nibble of each group into it, and the decoder's lane l gets all of
// its signs for the unit from one word per peer.
// Decode: the fp32 sum over peers, in peer order, of +-s per element.
//
// Both are HBM-bound streams. Encode moves 12 B/element (read x and error,
// write error) plus 1/8 B of signs and 4/C B of scales; one block owns one
// chunk at a time and keeps its c values in registers across the
// block-wide sum. Decode moves N/8 + 4N/C B of payload plus 4 B out (8 B
// when adding to the destination). For the first 8 peers it does not add
// per peer: every element's result is one of the 2^N in-order fp32 sums of
// +-s_k, which a wave tabulates in LDS per unit; the lane turns its 8 peers'
// words into one 8-bit table index per element with a bit-matrix transpose
// (byte gathers and three masked swap rounds) and reads its results from the
// table. Peers 9..16 are then added in order, one select and add each. With
// 1 or 2 peers a wave takes a quarter of a unit instead, so that it stores
// 2 quads per lane rather than 8.
#include "zds_device.h"
#include "zds_onebit.h"

namespace zds {

struct DecodeArgs {
  const uint32_t *words[kMaxPeers];
  const float *scales[kMaxPeers];
  int32_t npeers;
  int64_t n;
  int32_t chunk_shift;  // chunk = 1 << chunk_shift
  float *dst;
};

// Threads per encode block for a chunk of 1024 R elements. Fewer quads in
// flight per thread pay up to 8192-element chunks; at 16384 the 256-thread
// block is best again (7B shard, encode GB/s for 256 / 512 / 1024 threads,
// interleaved on one box: chunk 2048 5,985 / 6,149 / 6,161 (512 is the most
// a 2048 chunk allows), 4096 5,943 / 6,124 / 6,336, 8192 5,626 / 5,686 /
// 5,882, 16384 5,423 / 5,278 / 5,365).
template <int R>
constexpr int enc_block() {
  return R == 2 ? 512 : (R == 4 || R == 8) ? 1024 : 256;
}

// R = chunk / 1024, B threads, Q = 256 R / B quads per thread. EF: an error
// buffer is given. Iteration r of a chunk: wave w's lane l holds quad
// B r + 64 w + l, i.e. quad l of group (chunk base / 256) + (B / 64) r + w.
template <int R, bool EF, int B>
__global__ void __launch_bounds__(B) onebit_encode_kernel(const float *__restrict__ x, float *__restrict__ err,
                                                          uint32_t *__restrict__ words,
                                                          float *__restrict__ scales, int64_t n) {
  constexpr int64_t C = 1024 * R;
  constexpr int Q = 256 * R / B;  // quads per thread
  constexpr int WPB = B / 64;     // waves per block
  constexpr int UNITS = R >= 2 ? R / 2 : 1;  // sign-word units a chunk covers (half of one when C = 1024)
  __shared__ float s_sh;
  __shared__ uint32_t sw[UNITS][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nchunks = (n + C - 1) / C;
  const int64_t nunits = (n + 2047) >> 11;
  for (int64_t j = blockIdx.x; j < nchunks; j += gridDim.x) {  // uniform per block
    const int64_t base = j * C;
    const int64_t len = n - base < C ? n - base : C;
    for (int k = tid; k < UNITS * 64; k += B) (&sw[0][0])[k] = 0u;
    float c[Q][4];
    bool full[Q];
#pragma unroll
    for (int r = 0; r < Q; ++r) {
      const int64_t e0 = base + 4 * (r * B + tid);
      full[r] = e0 + 4 <= n;
      if (full[r]) {
        const f32x4 a = ld_stream(reinterpret_cast<const f32x4 *>(x + e0));
        c[r][0] = a.x; c[r][1] = a.y; c[r][2] = a.z; c[r][3] = a.w;
        if (EF) {
          // With one quad per thread, the error quad is loaded only after the
          // input quad has arrived: one load in flight per wave (chunk 2048,
          // the 7B shard, library builds swapped between bench runs, three
          // rounds: 1.558-1.562 ms against 1.618 back to back).
          if (Q == 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt at their maxima
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
    for (int r = 0; r < Q; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double d = c[r][i];
        ss = ss + d * d;  // the square of an fp32 value is exact in float64
      }
    const double total = block_sum<B>(ss);  // its barrier also orders the zeroing of sw before the ORs
    if (tid == 0) {
      const float s = static_cast<float>(sqrt(total / static_cast<double>(len)));
      s_sh = s;
      scales[j] = s;
    }
    __syncthreads();
    const float s = s_sh;
#pragma unroll
    for (int r = 0; r < Q; ++r) {
      const int64_t e0 = base + 4 * (r * B + tid);
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
      // group g = base / 256 + 4 r + wave: unit g >> 3, nibble g & 7
      const int64_t g = (base >> 8) + WPB * r + wave;
      const uint32_t nib = (pos[0] ? 1u : 0u) | (pos[1] ? 2u : 0u) | (pos[2] ? 4u : 0u) | (pos[3] ? 8u : 0u);
      const int ul = R >= 2 ? (WPB * r + wave) >> 3 : 0;
      if (nib) atomicOr(&sw[ul][lane], nib << (4 * (g & 7)));
    }
    __syncthreads();
    if constexpr (R >= 2) {
      // the chunk's whole units, 64 words each
      const int64_t u0 = base >> 11;
      for (int k = tid; k < UNITS * 64; k += B)
        if (u0 + (k >> 6) < nunits) words[64 * u0 + k] = (&sw[0][0])[k];
    } else {
      // half a unit: the 16-bit half of each word that holds this chunk's
      // groups; when the unit ends with this first half, the whole word (its
      // upper half is past n, hence 0)
      const int64_t u = base >> 11, h = (base >> 10) & 1;
      if (tid < 64) {
        if (h == 0 && base + 1024 >= n)
          words[64 * u + tid] = sw[0][tid];
        else
          reinterpret_cast<uint16_t *>(words)[2 * (64 * u + tid) + h] = static_cast<uint16_t>(sw[0][tid] >> (16 * h));
      }
    }
    __syncthreads();  // the words are read out before the next chunk clears them
  }
}

// Bit-matrix transpose of the 8 peers' sign words of a lane. In: w[k] bit j
// = sign of the lane's element j for peer k. Out: byte c of x[2b] (c < 4) or
// of x[2b + 1] (c >= 4, byte c - 4) = sum over k of (bit 8b + c of w[k]) << k,
// the table index of element 8b + c. Per byte b the 8x8 block (row k = byte b
// of w[k]) is gathered into a 64-bit pair and transposed by three masked
// swap rounds (distances 7, 14 and 28 bits).
__device__ __forceinline__ void transpose8x8(const uint32_t (&w)[8], int b, uint32_t &xlo, uint32_t &xhi) {
  const int sh = 8 * b;
  uint32_t lo = ((w[0] >> sh) & 0xffu) | (((w[1] >> sh) & 0xffu) << 8) | (((w[2] >> sh) & 0xffu) << 16) |
                (((w[3] >> sh) & 0xffu) << 24);
  uint32_t hi = ((w[4] >> sh) & 0xffu) | (((w[5] >> sh) & 0xffu) << 8) | (((w[6] >> sh) & 0xffu) << 16) |
                (((w[7] >> sh) & 0xffu) << 24);
  uint32_t t;
  t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
  lo = lo ^ t ^ (t << 7);
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
  hi = hi ^ t ^ (t << 7);
  t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
  lo = lo ^ t ^ (t << 14);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
  hi = hi ^ t ^ (t << 14);
  t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  xlo = lo ^ t;
  xhi = hi ^ (t >> 4);
}

__device__ __forceinline__ void transpose8x32(const uint32_t (&w)[8], uint32_t (&x)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int sh = 8 * b;
    uint32_t lo = ((w[0] >> sh) & 0xffu) | (((w[1] >> sh) & 0xffu) << 8) | (((w[2] >> sh) & 0xffu) << 16) |
                  (((w[3] >> sh) & 0xffu) << 24);
    uint32_t hi = ((w[4] >> sh) & 0xffu) | (((w[5] >> sh) & 0xffu) << 8) | (((w[6] >> sh) & 0xffu) << 16) |
                  (((w[7] >> sh) & 0xffu) << 24);
    uint32_t t;
    t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
    lo = lo ^ t ^ (t << 7);
    t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
    hi = hi ^ t ^ (t << 7);
    t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
    lo = lo ^ t ^ (t << 14);
    t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
    hi = hi ^ t ^ (t << 14);
    t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
    lo = lo ^ t;
    hi = hi ^ (t >> 4);
    x[2 * b] = lo;
    x[2 * b + 1] = hi;
  }
}

// Wave w of block b decodes unit 4 b + w (2048 elements) and moves on by 4
// units per block of the grid; lane l takes quad l of each of the unit's 8
// groups. Per unit: each lane loads its word of every peer and the peers'
// scales; the wave writes the table of the 2^min(N, 8) in-order sums (two
// tables when a chunk is 1024 elements, one per half unit); the lane
// transposes its 8 words into table indices, reads its 32 results and adds
// peers 9..N in order; then it stores its 8 quads (the wave's store of
// quad r covers 1 KiB).
template <bool ACC, int NP>
__global__ void __launch_bounds__(256) onebit_decode_kernel(DecodeArgs a) {
  constexpr int NT = NP < 8 ? NP : 8;  // peers in the table
  constexpr int TS = 1 << NT;         // table entries
  __shared__ float tab[4][2][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float *T0 = tab[wave][0];
  float *T1 = tab[wave][1];
  const int64_t nunits = (a.n + 2047) >> 11;
  const bool halves = a.chunk_shift == 10;  // a unit spans two chunks
  // lane k < NP loads peer k's scale of the unit's first chunk, lane 16 + k
  // that of its second half's chunk
  const int sk = lane & 15;
  const float *mys = a.scales[0];
#pragma unroll
  for (int k = 1; k < NP; ++k)
    if (sk == k) mys = a.scales[k];
  for (int64_t u = 4 * static_cast<int64_t>(blockIdx.x) + wave; u < nunits;
       u += 4 * static_cast<int64_t>(gridDim.x)) {
    uint32_t w[NP < 8 ? 8 : NP];
#pragma unroll
    for (int k = 0; k < (NP < 8 ? 8 : NP); ++k) w[k] = k < NP ? a.words[k][64 * u + lane] : 0u;
    float scl = 0.0f;
    const int64_t e_half = (u << 11) + (lane >> 4) * 1024;  // first element of the half this lane's scale is for
    if (sk < NP && lane < 32 && e_half < a.n) scl = mys[e_half >> a.chunk_shift];
    float s0[NP], s1[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      s0[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl), k));
      s1[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl), 16 + k));
    }
    // tables: entry e = the in-order sum over k < NT of (bit k of e ? s_k : -s_k).
    // Lane l writes entries l + 64 m; bits 0..5 come from the lane, 6 and 7 from m.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 1 && !halves) break;
      const float *s = t == 0 ? s0 : s1;
      float *T = t == 0 ? T0 : T1;
      constexpr int KL = NT < 6 ? NT : 6;
      float p = (lane & 1) ? s[0] : -s[0];
#pragma unroll
      for (int k = 1; k < KL; ++k) p = p + (((lane >> k) & 1) ? s[k] : -s[k]);
      if constexpr (NT <= 6) {
        if (lane < TS) T[lane] = p;
      } else {
#pragma unroll
        for (int m = 0; m < TS / 64; ++m) {
          float q = p + ((m & 1) ? s[6] : -s[6]);
          if constexpr (NT == 8) q = q + ((m & 2) ? s[7] : -s[7]);
          T[64 * m + lane] = q;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t wt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) wt[k] = w[k];
    uint32_t ix[8];
    transpose8x32(wt, ix);
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t idx = (ix[2 * (j >> 3) + ((j >> 2) & 1)] >> (8 * (j & 3))) & 0xffu;
      const int r = j >> 2;  // the group of element j (its bit is 4 r + i)
      // element j of the lane is bit j of its words, i.e. quad r = j / 4
      v[j] = (halves && r >= 4 ? T1 : T0)[idx];
    }
    // peers past the table, in order
#pragma unroll
    for (int k = NT; k < NP; ++k) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float sc = (halves && (j >> 2) >= 4) ? s1[k] : s0[k];
        v[j] = v[j] + (((w[k] >> j) & 1u) ? sc : -sc);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the table is read before the next unit rewrites it
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t e0 = (u << 11) + 256 * r + 4 * lane;
      if (e0 + 4 <= a.n) {
        f32x4 o = {v[4 * r], v[4 * r + 1], v[4 * r + 2], v[4 * r + 3]};
        if (ACC) {
          const f32x4 old = ld_stream(reinterpret_cast<const f32x4 *>(a.dst + e0));
          o = f32x4{old.x + o.x, old.y + o.y, old.z + o.z, old.w + o.w};
        }
        st_stream(reinterpret_cast<f32x4 *>(a.dst + e0), o);
        // Up to 8 peers, one store in flight per wave. 7B shard, library
        // builds swapped between runs: 8 peers 0.709-0.714 ms against
        // 0.762-0.768 with the 8 stores back to back in the bench (a wait
        // after every second store: 0.736-0.739); peer-count sweeps on three
        // boxes: 3 / 5 / 8 peers 0.61-0.62 / 0.62 / 0.67-0.71 against
        // 0.69-0.70 / 0.67-0.72 / 0.79 on two of them, while the third ran 3
        // and 4 peers slower with the waits (0.75-0.77 against 0.68-0.71) and
        // 8 peers faster. Past 8 peers, where each element also takes an add
        // per extra peer, the waits cost more than they save (16 peers 1.08
        // against 0.97 ms).
        if (NP <= 8 && r < 7) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt at their maxima
      } else {
        for (int i = 0; i < 4 && e0 + i < a.n; ++i) a.dst[e0 + i] = ACC ? a.dst[e0 + i] + v[4 * r + i] : v[4 * r + i];
      }
    }
  }
}

// The same for 1 or 2 peers, where the table and the transpose cost little
// and the stores dominate: block b decodes unit b (moving on by the grid),
// wave w the unit's groups 2w and 2w + 1, i.e. byte w of every lane word;
// each wave builds its own copy of the unit's table and stores 2 quads per
// lane instead of 8 (decoding into the 7B shard, interleaved A/B: 1 / 2
// peers 0.533 / 0.537 ms against 0.608 / 0.610 for the unit kernel; at 3 / 8
// peers 0.722 / 0.865 against 0.667 / 0.796, the quarter kernel reloading
// every word and rebuilding the table for a quarter of the elements).
template <bool ACC, int NP>
__global__ void __launch_bounds__(256) onebit_decode_quarter_kernel(DecodeArgs a) {
  constexpr int NT = NP < 8 ? NP : 8;
  constexpr int TS = 1 << NT;
  constexpr int WN = NP < 8 ? 8 : NP;
  __shared__ float tab[4][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float *T = tab[wave];
  const int64_t nunits = (a.n + 2047) >> 11;
  const int sk = lane & 15;
  const float *mys = a.scales[0];
#pragma unroll
  for (int k = 1; k < NP; ++k)
    if (sk == k) mys = a.scales[k];
  for (int64_t u = blockIdx.x; u < nunits; u += gridDim.x) {
    const int64_t ebase = (u << 11) + 512 * wave;  // the wave's 512 elements lie in one chunk
    if (ebase >= a.n) continue;                    // uniform per wave
    uint32_t w[WN];
#pragma unroll
    for (int k = 0; k < WN; ++k) w[k] = k < NP ? a.words[k][64 * u + lane] : 0u;
    float scl = 0.0f;
    if (sk < NP && lane < 16) scl = mys[ebase >> a.chunk_shift];
    float sv[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k)
      sv[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl), k));
    {
      constexpr int KL = NT < 6 ? NT : 6;
      float p = (lane & 1) ? sv[0] : -sv[0];
#pragma unroll
      for (int k = 1; k < KL; ++k) p = p + (((lane >> k) & 1) ? sv[k] : -sv[k]);
      if constexpr (NT <= 6) {
        if (lane < TS) T[lane] = p;
      } else {
#pragma unroll
        for (int m = 0; m < TS / 64; ++m) {
          float q = p + ((m & 1) ? sv[6] : -sv[6]);
          if constexpr (NT == 8) q = q + ((m & 2) ? sv[7] : -sv[7]);
          T[64 * m + lane] = q;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t wt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) wt[k] = w[k];
    uint32_t xlo, xhi;
    transpose8x8(wt, wave, xlo, xhi);
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = T[((c < 4 ? xlo : xhi) >> (8 * (c & 3))) & 0xffu];
#pragma unroll
    for (int k = NT; k < NP; ++k) {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = v[c] + (((w[k] >> (8 * wave + c)) & 1u) ? sv[k] : -sv[k]);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t e0 = (u << 11) + 256 * (2 * wave + q) + 4 * lane;
      if (e0 + 4 <= a.n) {
        f32x4 o = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        if (ACC) {
          const f32x4 old = ld_stream(reinterpret_cast<const f32x4 *>(a.dst + e0));
          o = f32x4{old.x + o.x, old.y + o.y, old.z + o.z, old.w + o.w};
        }
        st_stream(reinterpret_cast<f32x4 *>(a.dst + e0), o);
        // one store in flight per wave: 1 / 2 peers 0.506-0.515 / 0.510-0.517
        // ms against 0.541 / 0.537-0.538 with the 2 stores back to back
        if (q == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
      } else {
        for (int i = 0; i < 4 && e0 + i < a.n; ++i) a.dst[e0 + i] = ACC ? a.dst[e0 + i] + v[4 * q + i] : v[4 * q + i];
      }
    }
  }
}

template <int R>
static void encode_go(const float *x, float *err, uint32_t *words, float *scales, int64_t n, hipStream_t s) {
  constexpr int B = enc_block<R>();
  int64_t g = (n + 1024 * R - 1) / (1024 * R);
  if (g > max_blocks(B)) g = max_blocks(B);
  if (err)
    hipLaunchKernelGGL((onebit_encode_kernel<R, true, B>), dim3(static_cast<uint32_t>(g)), dim3(B), 0, s, x, err,
                       words, scales, n);
  else
    hipLaunchKernelGGL((onebit_encode_kernel<R, false, B>), dim3(static_cast<uint32_t>(g)), dim3(B), 0, s, x, err,
                       words, scales, n);
}

zds_status launch_onebit_encode(const float *x, float *err, int64_t n, int32_t chunk, uint32_t *words, float *scales,
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
static void decode_go(const DecodeArgs &a, hipStream_t s) {
  const int64_t nunits = (a.n + 2047) / 2048;
  int64_t g = NP <= 2 ? nunits : (nunits + 3) / 4;  // units per block: 1 (quarter kernel) or 4
  if (g > max_blocks(256)) g = max_blocks(256);
  if constexpr (NP <= 2)
    hipLaunchKernelGGL((onebit_decode_quarter_kernel<ACC, NP>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((onebit_decode_kernel<ACC, NP>), dim3(static_cast<uint32_t>(g)), dim3(256), 0, s, a);
}

template <bool ACC>
static void decode_np(const DecodeArgs &a, hipStream_t s) {
  switch (a.npeers) {
    case 1: decode_go<ACC, 1>(a, s); break;
    case 2: decode_go<ACC, 2>(a, s); break;
    case 3: decode_go<ACC, 3>(a, s); break;
    case 4: decode_go<ACC, 4>(a, s); break;
    case 5: decode_go<ACC, 5>(a, s); break;
    case 6: decode_go<ACC, 6>(a, s); break;
    case 7: decode_go<ACC, 7>(a, s); break;
    case 8: decode_go<ACC, 8>(a, s); break;
    case 9: decode_go<ACC, 9>(a, s); break;
    case 10: decode_go<ACC, 10>(a, s); break;
    case 11: decode_go<ACC, 11>(a, s); break;
    case 12: decode_go<ACC, 12>(a, s); break;
    case 13: decode_go<ACC, 13>(a, s); break;
    case 14: decode_go<ACC, 14>(a, s); break;
    case 15: decode_go<ACC, 15>(a, s); break;
    default: decode_go<ACC, 16>(a, s); break;
  }
}

zds_status launch_onebit_decode(const uint32_t *const *words, const float *const *scales, int32_t npeers, int64_t n,
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
  if (accumulate) decode_np<true>(a, s);
  else decode_np<false>(a, s);
  return check_launch("onebit decode kernel");
}

}  // namespace zds
