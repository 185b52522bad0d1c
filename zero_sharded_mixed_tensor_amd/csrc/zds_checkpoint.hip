// Sharded checkpoint / resume and consolidation (a next row).
//
// A run resumes from its per-rank shard files when the library version, the
// data-parallel topology and the configuration match the ones that wrote
// them; merging the ZeRO shards into one full fp32 state is a separate
// export step, not part of resuming (algomooc.com interview answer, 训练与恢复
// 边界 and the spoken answer's checkpoint paragraph). A rank's resumable state
// is its fp32 master/m/v shard plus the 64-byte step state (loss scale and
// its counters, the Adam step count and beta powers, the scaler settings).
//
// File layout (little-endian), produced and parsed only here:
//   [0, 256)        header: magic "ZDSCKPT1", format version, header size,
//                   zds_checkpoint_meta, zds_step_state, shard length n,
//                   four 64-bit hashes (tensor table, master, m, v)
//   [256, +8T)      the tensor table: numel of each of the T tensors
//   then            master[n], exp_avg[n], exp_avg_sq[n], fp32 each
// A save writes "<path>.tmp" and renames it over <path> when complete, so a
// crash mid-save leaves the previous checkpoint intact.
//
// Device arrays move through two pinned staging buffers, so the copy of one
// chunk overlaps the file I/O and hashing of the other.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zds_internal.h"

namespace {

using namespace zds;

constexpr char kMagic[8] = {'Z', 'D', 'S', 'C', 'K', 'P', 'T', '1'};
constexpr uint32_t kHeaderBytes = 256;
constexpr size_t kChunk = size_t(64) << 20;  // bytes per staging buffer

struct Header {
  char magic[8];
  uint32_t format;
  uint32_t header_bytes;
  zds_checkpoint_meta meta;
  zds_step_state state;
  int64_t n;
  uint64_t hash[4];  // tensor table, master, exp_avg, exp_avg_sq
};
static_assert(sizeof(Header) <= kHeaderBytes, "the header fits its slot");

// 64-bit hash of a byte stream: four lanes over 8-byte words with
// multiply-rotate mixing, folded at the end. Chunks fed to update() must be
// multiples of 32 bytes except the last.
struct Hash64 {
  uint64_t h[4] = {0x9E3779B97F4A7C15ull, 0xC2B2AE3D27D4EB4Full, 0x165667B19E3779F9ull, 0x27D4EB2F165667C5ull};
  uint64_t len = 0;
  static uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
  static uint64_t mix(uint64_t acc, uint64_t w) {
    return rotl(acc ^ (w * 0x87C37B91114253D5ull), 31) * 0x4CF5AD432745937Full;
  }
  void update(const void *p, size_t bytes) {
    const unsigned char *c = static_cast<const unsigned char *>(p);
    size_t i = 0;
    for (; i + 32 <= bytes; i += 32) {
      uint64_t w[4];
      std::memcpy(w, c + i, 32);
      for (int k = 0; k < 4; ++k) h[k] = mix(h[k], w[k]);
    }
    for (; i < bytes; ++i) h[i & 3] = mix(h[i & 3], c[i]);
    len += bytes;
  }
  uint64_t digest() const {
    uint64_t x = len * 0x9E3779B97F4A7C15ull;
    for (int k = 0; k < 4; ++k) x = rotl(x ^ h[k], 27) * 0x87C37B91114253D5ull + 0x52DCE729ull;
    x ^= x >> 33;
    x *= 0xFF51AFD7ED558CCDull;
    x ^= x >> 33;
    return x;
  }
};

uint64_t hash_of(const void *p, size_t bytes) {
  Hash64 h;
  h.update(p, bytes);
  return h.digest();
}

struct File {
  FILE *f = nullptr;
  File() = default;
  File(const File &) = delete;
  File &operator=(const File &) = delete;
  ~File() {
    if (f) std::fclose(f);
  }
};

struct Staging {
  void *p[2] = {nullptr, nullptr};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool busy[2] = {false, false};
  Staging() = default;
  Staging(const Staging &) = delete;
  Staging &operator=(const Staging &) = delete;
  ~Staging() {
    for (int i = 0; i < 2; ++i) {
      if (busy[i]) (void)hipEventSynchronize(ev[i]);
      if (ev[i]) (void)hipEventDestroy(ev[i]);
      if (p[i]) (void)hipHostFree(p[i]);
    }
  }
  zds_status init(const char *fn) {
    for (int i = 0; i < 2; ++i) {
      if (hipHostMalloc(&p[i], kChunk, hipHostMallocDefault) != hipSuccess) {
        p[i] = nullptr;
        return fail(ZDS_ENOMEM, "%s: pinned staging buffer of %zu bytes", fn, kChunk);
      }
      if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) {
        ev[i] = nullptr;
        return fail(ZDS_EHIP, "%s: hipEventCreateWithFlags", fn);
      }
    }
    return ZDS_OK;
  }
  zds_status wait(int i, const char *fn) {
    if (!busy[i]) return ZDS_OK;
    busy[i] = false;
    if (hipEventSynchronize(ev[i]) != hipSuccess) return fail(ZDS_EHIP, "%s: waiting for a staging copy", fn);
    return ZDS_OK;
  }
};

bool same_meta(const zds_checkpoint_meta &a, const zds_checkpoint_meta &b) {
  return a.world == b.world && a.rank == b.rank && a.flat_align == b.flat_align && a.stage == b.stage &&
         a.offload == b.offload && a.num_tensors == b.num_tensors && a.flat_total == b.flat_total &&
         a.lo == b.lo && a.hi == b.hi;
}

// The meta must describe rank's shard of the layout of numel exactly.
zds_status check_meta(const zds_checkpoint_meta &m, const int64_t *numel, const char *fn) {
  if (m.world < 1 || m.rank < 0 || m.rank >= m.world || m.flat_align < 1 || m.stage < 1 || m.stage > 3 ||
      (m.offload != 0 && m.offload != 1) || m.num_tensors < 0 || (m.num_tensors > 0 && !numel))
    return fail(ZDS_EINVAL, "%s: bad meta (world %d, rank %d, flat_align %d, stage %d, offload %d, %d tensors)", fn,
                m.world, m.rank, m.flat_align, m.stage, m.offload, m.num_tensors);
  int64_t total = 0;
  if (zds_flat_layout(numel, m.num_tensors, m.flat_align, nullptr, &total) != ZDS_OK)
    return fail(ZDS_EINVAL, "%s: bad tensor table", fn);
  int64_t lo = 0, hi = 0;
  if (zds_shard_range(total, m.world, m.rank, m.flat_align, &lo, &hi) != ZDS_OK)
    return fail(ZDS_EINVAL, "%s: bad partition", fn);
  if (total != m.flat_total || lo != m.lo || hi != m.hi)
    return fail(ZDS_EINVAL,
                "%s: meta says total %lld, range [%lld, %lld); the tensor table gives total %lld, rank %d of %d "
                "owns [%lld, %lld)",
                fn, static_cast<long long>(m.flat_total), static_cast<long long>(m.lo),
                static_cast<long long>(m.hi), static_cast<long long>(total), m.rank, m.world,
                static_cast<long long>(lo), static_cast<long long>(hi));
  return ZDS_OK;
}

zds_status write_bytes(FILE *f, const void *p, size_t bytes, const char *fn) {
  if (bytes && std::fwrite(p, 1, bytes, f) != bytes) return fail(ZDS_EIO, "%s: write failed", fn);
  return ZDS_OK;
}

zds_status read_bytes(FILE *f, void *p, size_t bytes, const char *fn, const char *path) {
  if (bytes && std::fread(p, 1, bytes, f) != bytes) return fail(ZDS_EIO, "%s: %s is truncated", fn, path);
  return ZDS_OK;
}

size_t piece(size_t bytes, size_t off) { return bytes - off < kChunk ? bytes - off : kChunk; }

// One fp32 array to the file, hashing what is written.
zds_status save_array(FILE *f, const float *src, int64_t n, bool on_host, hipStream_t s, Staging *stg,
                      uint64_t *hash, const char *fn) {
  const size_t bytes = sizeof(float) * static_cast<size_t>(n);
  const char *p = reinterpret_cast<const char *>(src);
  Hash64 h;
  if (on_host) {
    for (size_t off = 0; off < bytes; off += kChunk) {  // hash and write piece by piece, while in cache
      const size_t len = piece(bytes, off);
      h.update(p + off, len);
      zds_status st = write_bytes(f, p + off, len, fn);
      if (st != ZDS_OK) return st;
    }
    *hash = h.digest();
    return ZDS_OK;
  }
  // chunk c copies into buffer c % 2 while chunk c - 1 is hashed and written
  const size_t chunks = (bytes + kChunk - 1) / kChunk;
  for (size_t c = 0; c <= chunks; ++c) {
    if (c < chunks) {
      const int b = static_cast<int>(c & 1);
      const size_t off = c * kChunk;
      if (hipMemcpyAsync(stg->p[b], p + off, piece(bytes, off), hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipEventRecord(stg->ev[b], s) != hipSuccess)
        return fail(ZDS_EHIP, "%s: device-to-host copy", fn);
      stg->busy[b] = true;
    }
    if (c > 0) {
      const int b = static_cast<int>((c - 1) & 1);
      const size_t len = piece(bytes, (c - 1) * kChunk);
      zds_status st = stg->wait(b, fn);
      if (st != ZDS_OK) return st;
      h.update(stg->p[b], len);
      st = write_bytes(f, stg->p[b], len, fn);
      if (st != ZDS_OK) return st;
    }
  }
  *hash = h.digest();
  return ZDS_OK;
}

// One fp32 array from the file, checked against its hash.
zds_status load_array(FILE *f, float *dst, int64_t n, bool on_host, hipStream_t s, Staging *stg, uint64_t hash,
                      const char *fn, const char *path, const char *what) {
  const size_t bytes = sizeof(float) * static_cast<size_t>(n);
  char *p = reinterpret_cast<char *>(dst);
  Hash64 h;
  if (on_host) {
    for (size_t off = 0; off < bytes; off += kChunk) {
      const size_t len = piece(bytes, off);
      zds_status st = read_bytes(f, p + off, len, fn, path);
      if (st != ZDS_OK) return st;
      h.update(p + off, len);
    }
  } else {
    for (size_t off = 0, c = 0; off < bytes; off += kChunk, ++c) {
      const int b = static_cast<int>(c & 1);
      const size_t len = piece(bytes, off);
      zds_status st = stg->wait(b, fn);  // the copy out of this buffer two chunks ago
      if (st != ZDS_OK) return st;
      st = read_bytes(f, stg->p[b], len, fn, path);
      if (st != ZDS_OK) return st;
      h.update(stg->p[b], len);
      if (hipMemcpyAsync(p + off, stg->p[b], len, hipMemcpyHostToDevice, s) != hipSuccess ||
          hipEventRecord(stg->ev[b], s) != hipSuccess)
        return fail(ZDS_EHIP, "%s: host-to-device copy", fn);
      stg->busy[b] = true;
    }
    for (int b = 0; b < 2; ++b) {
      zds_status st = stg->wait(b, fn);
      if (st != ZDS_OK) return st;
    }
  }
  if (h.digest() != hash) return fail(ZDS_EIO, "%s: %s is corrupt (%s does not match its hash)", fn, path, what);
  return ZDS_OK;
}

// Header and tensor table of a checkpoint file; the file is left positioned at
// the start of the master section.
zds_status read_head(FILE *f, const char *path, Header *hd, std::vector<int64_t> *numel, const char *fn) {
  unsigned char buf[kHeaderBytes];
  zds_status st = read_bytes(f, buf, kHeaderBytes, fn, path);
  if (st != ZDS_OK) return st;
  std::memcpy(hd, buf, sizeof *hd);
  if (std::memcmp(hd->magic, kMagic, 8) != 0)
    return fail(ZDS_EIO, "%s: %s is not a checkpoint of this library", fn, path);
  if (hd->format != ZDS_CHECKPOINT_FORMAT || hd->header_bytes != kHeaderBytes)
    return fail(ZDS_EIO, "%s: %s has format %u; this library reads format %d", fn, path, hd->format,
                ZDS_CHECKPOINT_FORMAT);
  const int32_t T = hd->meta.num_tensors;
  if (T < 0 || T > (1 << 24)) return fail(ZDS_EIO, "%s: %s has a bad tensor count %d", fn, path, T);
  numel->assign(static_cast<size_t>(T), 0);
  st = read_bytes(f, numel->data(), sizeof(int64_t) * static_cast<size_t>(T), fn, path);
  if (st != ZDS_OK) return st;
  if (hash_of(numel->data(), sizeof(int64_t) * static_cast<size_t>(T)) != hd->hash[0])
    return fail(ZDS_EIO, "%s: %s is corrupt (the tensor table does not match its hash)", fn, path);
  if (check_meta(hd->meta, numel->data(), fn) != ZDS_OK) {
    const std::string why = zds_last_error();
    return fail(ZDS_EIO, "%s: %s: %s", fn, path, why.c_str());
  }
  if (hd->n != hd->meta.hi - hd->meta.lo)
    return fail(ZDS_EIO, "%s: %s: the shard length does not match its range", fn, path);
  const long here = std::ftell(f);
  const long long want = static_cast<long long>(kHeaderBytes) + 8LL * T + 12LL * hd->n;
  if (here < 0 || std::fseek(f, 0, SEEK_END) != 0) return fail(ZDS_EIO, "%s: cannot seek in %s", fn, path);
  const long size = std::ftell(f);
  if (size != want) return fail(ZDS_EIO, "%s: %s has %ld bytes, its header says %lld", fn, path, size, want);
  if (std::fseek(f, here, SEEK_SET) != 0) return fail(ZDS_EIO, "%s: cannot seek in %s", fn, path);
  return ZDS_OK;
}

}  // namespace

extern "C" zds_status zds_checkpoint_save(const char *path, const zds_checkpoint_meta *meta, const int64_t *numel,
                                          const float *master, const float *exp_avg, const float *exp_avg_sq,
                                          const zds_step_state *state, zds_location loc, void *stream) {
  clear_error();
  const char *fn = "zds_checkpoint_save";
  if (!path || !meta || !state) return fail(ZDS_EINVAL, "%s: null path, meta or state", fn);
  if (loc != ZDS_ON_DEVICE && loc != ZDS_ON_HOST) return fail(ZDS_EINVAL, "%s: bad location %d", fn, loc);
  zds_status st = check_meta(*meta, numel, fn);
  if (st != ZDS_OK) return st;
  const int64_t n = meta->hi - meta->lo;
  if (n > 0 && (!master || !exp_avg || !exp_avg_sq)) return fail(ZDS_EINVAL, "%s: null array", fn);
  const bool on_host = loc == ZDS_ON_HOST;
  hipStream_t s = static_cast<hipStream_t>(stream);

  Header hd{};
  std::memcpy(hd.magic, kMagic, 8);
  hd.format = ZDS_CHECKPOINT_FORMAT;
  hd.header_bytes = kHeaderBytes;
  hd.meta = *meta;
  hd.n = n;
  const size_t table_bytes = sizeof(int64_t) * static_cast<size_t>(meta->num_tensors);
  hd.hash[0] = hash_of(numel, table_bytes);
  Staging stg;
  if (on_host) {
    hd.state = *state;
  } else {
    // the state and arrays as left by the work already enqueued on stream
    if (hipMemcpyAsync(&hd.state, state, sizeof(zds_step_state), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(ZDS_EHIP, "%s: state download", fn);
    st = stg.init(fn);
    if (st != ZDS_OK) return st;
  }

  const std::string tmp = std::string(path) + ".tmp";
  {
    File out;
    out.f = std::fopen(tmp.c_str(), "wb");
    if (!out.f) return fail(ZDS_EIO, "%s: cannot create %s", fn, tmp.c_str());
    unsigned char head[kHeaderBytes] = {};
    st = write_bytes(out.f, head, kHeaderBytes, fn);  // rewritten once the hashes are known
    if (st == ZDS_OK) st = write_bytes(out.f, numel, table_bytes, fn);
    const float *arr[3] = {master, exp_avg, exp_avg_sq};
    for (int k = 0; k < 3 && st == ZDS_OK; ++k)
      st = save_array(out.f, arr[k], n, on_host, s, &stg, &hd.hash[k + 1], fn);
    if (st == ZDS_OK) {
      std::memcpy(head, &hd, sizeof hd);
      if (std::fseek(out.f, 0, SEEK_SET) != 0) st = fail(ZDS_EIO, "%s: seek failed", fn);
      else st = write_bytes(out.f, head, kHeaderBytes, fn);
    }
    if (st == ZDS_OK && std::fflush(out.f) != 0) st = fail(ZDS_EIO, "%s: flush failed", fn);
    const int rc = std::fclose(out.f);
    out.f = nullptr;
    if (st == ZDS_OK && rc != 0) st = fail(ZDS_EIO, "%s: close failed", fn);
  }
  if (st != ZDS_OK) {
    std::remove(tmp.c_str());
    return st;
  }
  if (std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return fail(ZDS_EIO, "%s: cannot rename %s to %s", fn, tmp.c_str(), path);
  }
  return ZDS_OK;
}

extern "C" zds_status zds_checkpoint_read_meta(const char *path, zds_checkpoint_meta *meta, zds_step_state *state,
                                               int64_t *numel_out, int32_t max_tensors) {
  clear_error();
  const char *fn = "zds_checkpoint_read_meta";
  if (!path || !meta) return fail(ZDS_EINVAL, "%s: null path or meta", fn);
  if (max_tensors < 0 || (max_tensors > 0 && !numel_out)) return fail(ZDS_EINVAL, "%s: bad tensor buffer", fn);
  File in;
  in.f = std::fopen(path, "rb");
  if (!in.f) return fail(ZDS_EIO, "%s: cannot open %s", fn, path);
  Header hd;
  std::vector<int64_t> numel;
  zds_status st = read_head(in.f, path, &hd, &numel, fn);
  if (st != ZDS_OK) return st;
  *meta = hd.meta;
  if (state) *state = hd.state;
  const int32_t T = hd.meta.num_tensors;
  if (numel_out) std::memcpy(numel_out, numel.data(), sizeof(int64_t) * static_cast<size_t>(T < max_tensors ? T : max_tensors));
  if (numel_out && T > max_tensors)
    return fail(ZDS_EINVAL, "%s: %s has %d tensors, room for %d", fn, path, T, max_tensors);
  return ZDS_OK;
}

extern "C" zds_status zds_checkpoint_load(const char *path, const zds_checkpoint_meta *expect, const int64_t *numel,
                                          float *master, float *exp_avg, float *exp_avg_sq, zds_step_state *state,
                                          zds_location loc, void *stream) {
  clear_error();
  const char *fn = "zds_checkpoint_load";
  if (!path || !expect || !state) return fail(ZDS_EINVAL, "%s: null path, meta or state", fn);
  if (loc != ZDS_ON_DEVICE && loc != ZDS_ON_HOST) return fail(ZDS_EINVAL, "%s: bad location %d", fn, loc);
  zds_status st = check_meta(*expect, numel, fn);
  if (st != ZDS_OK) return st;
  File in;
  in.f = std::fopen(path, "rb");
  if (!in.f) return fail(ZDS_EIO, "%s: cannot open %s", fn, path);
  Header hd;
  std::vector<int64_t> table;
  st = read_head(in.f, path, &hd, &table, fn);
  if (st != ZDS_OK) return st;
  const zds_checkpoint_meta &m = hd.meta;
  const bool same_tensors =
      m.num_tensors == expect->num_tensors &&
      (m.num_tensors == 0 || std::memcmp(table.data(), numel, sizeof(int64_t) * static_cast<size_t>(m.num_tensors)) == 0);
  if (!same_meta(m, *expect) || !same_tensors)
    return fail(ZDS_EINVAL,
                "%s: %s was written by rank %d of %d (stage %d, offload %d, align %d, %d tensors, %lld elements, "
                "range [%lld, %lld)); this run is rank %d of %d (stage %d, offload %d, align %d, %d tensors, "
                "%lld elements, range [%lld, %lld))%s",
                fn, path, m.rank, m.world, m.stage, m.offload, m.flat_align, m.num_tensors,
                static_cast<long long>(m.flat_total), static_cast<long long>(m.lo), static_cast<long long>(m.hi),
                expect->rank, expect->world, expect->stage, expect->offload, expect->flat_align, expect->num_tensors,
                static_cast<long long>(expect->flat_total), static_cast<long long>(expect->lo),
                static_cast<long long>(expect->hi), same_tensors ? "" : "; the tensor tables differ");
  const int64_t n = hd.n;
  if (n > 0 && (!master || !exp_avg || !exp_avg_sq)) return fail(ZDS_EINVAL, "%s: null array", fn);
  const bool on_host = loc == ZDS_ON_HOST;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Staging stg;
  if (!on_host) {
    st = stg.init(fn);
    if (st != ZDS_OK) return st;
  }
  float *arr[3] = {master, exp_avg, exp_avg_sq};
  const char *what[3] = {"master", "exp_avg", "exp_avg_sq"};
  for (int k = 0; k < 3; ++k) {
    st = load_array(in.f, arr[k], n, on_host, s, &stg, hd.hash[k + 1], fn, path, what[k]);
    if (st != ZDS_OK) return st;
  }
  if (on_host) {
    *state = hd.state;
    return ZDS_OK;
  }
  st = launch_state_init(state, hd.state, s);
  if (st != ZDS_OK) return st;
  if (hipStreamSynchronize(s) != hipSuccess) return fail(ZDS_EHIP, "%s: stream sync", fn);
  return ZDS_OK;
}

extern "C" zds_status zds_consolidate_fp32(const char *const *paths, int32_t num_files, int32_t section, float *out,
                                           int64_t out_numel) {
  clear_error();
  const char *fn = "zds_consolidate_fp32";
  if (!paths || num_files < 1) return fail(ZDS_EINVAL, "%s: no files", fn);
  if (section < 0 || section > 2) return fail(ZDS_EINVAL, "%s: section must be 0 (master), 1 or 2", fn);
  std::vector<Header> hd(static_cast<size_t>(num_files));
  std::vector<int64_t> numel, other;
  for (int i = 0; i < num_files; ++i) {
    if (!paths[i]) return fail(ZDS_EINVAL, "%s: null path", fn);
    File in;
    in.f = std::fopen(paths[i], "rb");
    if (!in.f) return fail(ZDS_EIO, "%s: cannot open %s", fn, paths[i]);
    zds_status st = read_head(in.f, paths[i], &hd[i], i == 0 ? &numel : &other, fn);
    if (st != ZDS_OK) return st;
    if (i > 0 && other != numel)
      return fail(ZDS_EINVAL, "%s: %s has another tensor table than %s", fn, paths[i], paths[0]);
  }
  // the files must be ranks 0 .. world-1 of one run at one step, in any order
  const zds_checkpoint_meta &m0 = hd[0].meta;
  if (num_files != m0.world) return fail(ZDS_EINVAL, "%s: %d files for a world of %d", fn, num_files, m0.world);
  std::vector<int> by_rank(static_cast<size_t>(num_files), -1);
  for (int i = 0; i < num_files; ++i) {
    const zds_checkpoint_meta &m = hd[i].meta;
    if (m.world != m0.world || m.flat_align != m0.flat_align || m.stage != m0.stage)
      return fail(ZDS_EINVAL, "%s: %s belongs to another run than %s", fn, paths[i], paths[0]);
    if (hd[i].state.t != hd[0].state.t)
      return fail(ZDS_EINVAL, "%s: %s is at step %lld, %s at step %lld", fn, paths[i],
                  static_cast<long long>(hd[i].state.t), paths[0], static_cast<long long>(hd[0].state.t));
    if (by_rank[m.rank] >= 0) return fail(ZDS_EINVAL, "%s: rank %d appears twice", fn, m.rank);
    by_rank[m.rank] = i;
  }
  const int32_t T = m0.num_tensors;
  std::vector<int64_t> offs(static_cast<size_t>(T)), out_off(static_cast<size_t>(T));
  int64_t total = 0;
  if (zds_flat_layout(numel.data(), T, m0.flat_align, offs.data(), &total) != ZDS_OK)
    return fail(ZDS_EIO, "%s: bad tensor table in %s", fn, paths[0]);
  int64_t want = 0;
  for (int t = 0; t < T; ++t) {
    out_off[t] = want;
    want += numel[t];
  }
  if (want > 0 && !out) return fail(ZDS_EINVAL, "%s: null output", fn);
  if (out_numel != want)
    return fail(ZDS_EINVAL, "%s: the tensors hold %lld elements, the output %lld", fn, static_cast<long long>(want),
                static_cast<long long>(out_numel));
  // Each rank's slice [lo, hi) of the flat buffer goes to the pieces of the
  // tensors it covers; padding is dropped.
  std::vector<float> buf(kChunk / sizeof(float));
  for (int r = 0; r < num_files; ++r) {
    const Header &h = hd[by_rank[r]];
    const char *path = paths[by_rank[r]];
    File in;
    in.f = std::fopen(path, "rb");
    const size_t skip = kHeaderBytes + sizeof(int64_t) * static_cast<size_t>(T) +
                        sizeof(float) * static_cast<size_t>(h.n) * static_cast<size_t>(section);
    if (!in.f || std::fseek(in.f, static_cast<long>(skip), SEEK_SET) != 0)
      return fail(ZDS_EIO, "%s: cannot read %s", fn, path);
    Hash64 hash;
    int t = 0;
    for (int64_t pos = h.meta.lo; pos < h.meta.hi;) {
      const int64_t room = static_cast<int64_t>(buf.size());
      const int64_t len = h.meta.hi - pos < room ? h.meta.hi - pos : room;
      zds_status st = read_bytes(in.f, buf.data(), sizeof(float) * static_cast<size_t>(len), fn, path);
      if (st != ZDS_OK) return st;
      hash.update(buf.data(), sizeof(float) * static_cast<size_t>(len));
      while (t < T && offs[t] + numel[t] <= pos) ++t;
      for (int u = t; u < T && offs[u] < pos + len; ++u) {
        const int64_t a = offs[u] > pos ? offs[u] : pos;
        const int64_t b = offs[u] + numel[u] < pos + len ? offs[u] + numel[u] : pos + len;
        if (a < b)
          std::memcpy(out + out_off[u] + (a - offs[u]), buf.data() + (a - pos),
                      sizeof(float) * static_cast<size_t>(b - a));
      }
      pos += len;
    }
    if (hash.digest() != h.hash[section + 1])
      return fail(ZDS_EIO, "%s: %s is corrupt (section %d does not match its hash)", fn, path, section);
  }
  return ZDS_OK;
}
