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
// A section's hash is the hash of the sequence of its 32 MiB pieces' hashes,
// so pieces can be hashed in parallel. A save writes "<path>.tmp" and
// renames it over <path> when complete, so a crash mid-save leaves the
// previous checkpoint intact.
//
// The sections move piece by piece on up to 8 host threads; for device
// arrays each thread owns a pinned buffer and a stream, so copies over PCIe,
// hashing and file I/O of different pieces overlap. A save writes through a
// shared mapping of the preallocated file.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <cstdio>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "zds_host.h"
#include "zds_internal.h"

namespace {

using namespace zds;

constexpr char kMagic[8] = {'Z', 'D', 'S', 'C', 'K', 'P', 'T', '1'};
constexpr uint32_t kHeaderBytes = 256;
constexpr size_t kPiece = size_t(32) << 20;  // bytes per hashed and transferred piece
constexpr int kMaxWorkers = 8;
// A save writes through a shared mapping of the preallocated file, not
// through pwrite (a 10.1 GB rank file saved to /tmp: 7.3-9.8 GB/s mapped;
// 10.7 GB/s for a first pwrite save, 3.4-4.6 for the next ones); it falls
// back to pwrite where the file cannot be mapped.

struct Header {
  char magic[8];
  uint32_t format;
  uint32_t header_bytes;
  zds_checkpoint_meta meta;
  zds_step_state state;
  int64_t n;
  uint64_t hash[4];   // tensor table, master, exp_avg, exp_avg_sq
  uint64_t head_hash; // every field above (the step state included)
};
static_assert(sizeof(Header) <= kHeaderBytes, "the header fits its slot");
static_assert(offsetof(Header, head_hash) == 168, "no padding before the header's own hash");

// 64-bit hash of a byte stream: four lanes over 8-byte words with
// multiply-rotate mixing, folded at the end.
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

// A section's hash from its pieces' hashes.
uint64_t fold(const std::vector<uint64_t> &pieces) { return hash_of(pieces.data(), 8 * pieces.size()); }

size_t num_pieces(size_t bytes) { return (bytes + kPiece - 1) / kPiece; }

struct Fd {
  int fd = -1;
  Fd() = default;
  Fd(const Fd &) = delete;
  Fd &operator=(const Fd &) = delete;
  ~Fd() {
    if (fd >= 0) ::close(fd);
  }
};

bool pwrite_all(int fd, const void *p, size_t n, off_t off) {
  const char *c = static_cast<const char *>(p);
  while (n > 0) {
    const ssize_t w = ::pwrite(fd, c, n, off);
    if (w < 0 && errno == EINTR) continue;
    if (w <= 0) return false;
    c += w;
    n -= static_cast<size_t>(w);
    off += w;
  }
  return true;
}

bool pread_all(int fd, void *p, size_t n, off_t off) {
  char *c = static_cast<char *>(p);
  while (n > 0) {
    const ssize_t r = ::pread(fd, c, n, off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    c += r;
    n -= static_cast<size_t>(r);
    off += r;
  }
  return true;
}

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

// Moves the three fp32 sections (sec_bytes each, starting at file offset
// data_off) between memory and the file, piece by piece, on up to
// kMaxWorkers threads, and records every piece's hash in dig[section].
// to_file: memory -> file (into `map`, the file mapped shared, when given:
// writes through one descriptor are serialised by the kernel, page faults
// of a mapping are not); otherwise file -> memory.
zds_status transfer(int fd, char *map, bool to_file, bool on_host, float *const arr[3], size_t sec_bytes,
                    off_t data_off, std::vector<uint64_t> dig[3], const char *fn, const char *path) {
  const size_t per = num_pieces(sec_bytes);
  for (int k = 0; k < 3; ++k) dig[k].assign(per, 0);
  const size_t jobs = 3 * per;
  if (jobs == 0) return ZDS_OK;
  int dev = 0;
  if (!on_host && hipGetDevice(&dev) != hipSuccess) return fail(ZDS_EHIP, "%s: hipGetDevice", fn);
  const size_t workers =
      std::min<size_t>({static_cast<size_t>(kMaxWorkers), static_cast<size_t>(host_thread_budget()), jobs});

  std::atomic<size_t> next(0);
  std::atomic<bool> bad(false);
  std::mutex mu;
  zds_status why_st = ZDS_OK;
  std::string why;
  auto stop = [&](zds_status st, const std::string &msg) {
    std::lock_guard<std::mutex> lock(mu);
    if (!bad.load()) {
      why_st = st;
      why = msg;
    }
    bad.store(true);
  };
  auto work = [&]() {
    void *buf = nullptr;
    hipStream_t s = nullptr;
    if (!on_host) {
      if (hipSetDevice(dev) != hipSuccess) return stop(ZDS_EHIP, std::string(fn) + ": hipSetDevice");
      if (hipHostMalloc(&buf, kPiece, hipHostMallocDefault) != hipSuccess) {
        buf = nullptr;
        return stop(ZDS_ENOMEM, std::string(fn) + ": pinned staging buffer");
      }
      if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
        (void)hipHostFree(buf);
        return stop(ZDS_EHIP, std::string(fn) + ": hipStreamCreateWithFlags");
      }
    }
    for (;;) {
      if (bad.load()) break;
      const size_t j = next.fetch_add(1);
      if (j >= jobs) break;
      const size_t sec = j / per, p = j % per;
      const size_t off = p * kPiece;
      const size_t len = std::min(kPiece, sec_bytes - off);
      char *mem = reinterpret_cast<char *>(arr[sec]) + off;
      const off_t foff = data_off + static_cast<off_t>(sec * sec_bytes + off);
      if (to_file) {
        const char *src = mem;
        if (!on_host) {
          if (hipMemcpyAsync(buf, mem, len, hipMemcpyDeviceToHost, s) != hipSuccess ||
              hipStreamSynchronize(s) != hipSuccess) {
            stop(ZDS_EHIP, std::string(fn) + ": device-to-host copy");
            break;
          }
          src = static_cast<const char *>(buf);
        }
        dig[sec][p] = hash_of(src, len);
        if (map) {
          std::memcpy(map + foff, src, len);
        } else if (!pwrite_all(fd, src, len, foff)) {
          stop(ZDS_EIO, std::string(fn) + ": write to " + path + " failed");
          break;
        }
      } else {
        char *dst = on_host ? mem : static_cast<char *>(buf);
        if (!pread_all(fd, dst, len, foff)) {
          stop(ZDS_EIO, std::string(fn) + ": " + path + " is truncated");
          break;
        }
        dig[sec][p] = hash_of(dst, len);
        if (!on_host && (hipMemcpyAsync(mem, buf, len, hipMemcpyHostToDevice, s) != hipSuccess ||
                         hipStreamSynchronize(s) != hipSuccess)) {
          stop(ZDS_EHIP, std::string(fn) + ": host-to-device copy");
          break;
        }
      }
    }
    if (s) (void)hipStreamDestroy(s);
    if (buf) (void)hipHostFree(buf);
  };
  std::vector<std::thread> pool;
  pool.reserve(workers - 1);
  for (size_t w = 1; w < workers; ++w) pool.emplace_back(work);
  work();
  for (auto &t : pool) t.join();
  if (bad.load()) return fail(why_st, "%s", why.c_str());
  return ZDS_OK;
}

// Header and tensor table of an open checkpoint file, checked against each
// other and against the file's size.
zds_status read_head(int fd, const char *path, Header *hd, std::vector<int64_t> *numel, const char *fn) {
  unsigned char buf[kHeaderBytes];
  if (!pread_all(fd, buf, kHeaderBytes, 0)) return fail(ZDS_EIO, "%s: %s is truncated", fn, path);
  std::memcpy(hd, buf, sizeof *hd);
  if (std::memcmp(hd->magic, kMagic, 8) != 0)
    return fail(ZDS_EIO, "%s: %s is not a checkpoint of this library", fn, path);
  if (hd->format != ZDS_CHECKPOINT_FORMAT || hd->header_bytes != kHeaderBytes)
    return fail(ZDS_EIO, "%s: %s has format %u; this library reads format %d", fn, path, hd->format,
                ZDS_CHECKPOINT_FORMAT);
  if (hash_of(hd, offsetof(Header, head_hash)) != hd->head_hash)
    return fail(ZDS_EIO, "%s: %s is corrupt (the header, step state included, does not match its hash)", fn, path);
  const int32_t T = hd->meta.num_tensors;
  if (T < 0 || T > (1 << 24)) return fail(ZDS_EIO, "%s: %s has a bad tensor count %d", fn, path, T);
  numel->assign(static_cast<size_t>(T), 0);
  if (!pread_all(fd, numel->data(), sizeof(int64_t) * static_cast<size_t>(T), kHeaderBytes))
    return fail(ZDS_EIO, "%s: %s is truncated", fn, path);
  if (hash_of(numel->data(), sizeof(int64_t) * static_cast<size_t>(T)) != hd->hash[0])
    return fail(ZDS_EIO, "%s: %s is corrupt (the tensor table does not match its hash)", fn, path);
  if (check_meta(hd->meta, numel->data(), fn) != ZDS_OK) {
    const std::string why = zds_last_error();
    return fail(ZDS_EIO, "%s: %s: %s", fn, path, why.c_str());
  }
  if (hd->n != hd->meta.hi - hd->meta.lo)
    return fail(ZDS_EIO, "%s: %s: the shard length does not match its range", fn, path);
  struct stat sb;
  const long long want = static_cast<long long>(kHeaderBytes) + 8LL * T + 12LL * hd->n;
  if (::fstat(fd, &sb) != 0) return fail(ZDS_EIO, "%s: cannot stat %s", fn, path);
  if (static_cast<long long>(sb.st_size) != want)
    return fail(ZDS_EIO, "%s: %s has %lld bytes, its header says %lld", fn, path,
                static_cast<long long>(sb.st_size), want);
  return ZDS_OK;
}

zds_status open_read(const char *path, Fd *f, const char *fn) {
  f->fd = ::open(path, O_RDONLY | O_CLOEXEC);
  if (f->fd < 0) return fail(ZDS_EIO, "%s: cannot open %s", fn, path);
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

  Header hd{};
  std::memcpy(hd.magic, kMagic, 8);
  hd.format = ZDS_CHECKPOINT_FORMAT;
  hd.header_bytes = kHeaderBytes;
  hd.meta = *meta;
  hd.n = n;
  const size_t table_bytes = sizeof(int64_t) * static_cast<size_t>(meta->num_tensors);
  hd.hash[0] = hash_of(numel, table_bytes);
  if (on_host) {
    hd.state = *state;
  } else {
    // the state and arrays as left by the work already enqueued on stream
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&hd.state, state, sizeof(zds_step_state), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(ZDS_EHIP, "%s: state download", fn);
  }

  const std::string tmp = std::string(path) + ".tmp";
  {
    Fd out;
    out.fd = ::open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
    if (out.fd < 0) return fail(ZDS_EIO, "%s: cannot create %s", fn, tmp.c_str());
    if (table_bytes && !pwrite_all(out.fd, numel, table_bytes, kHeaderBytes))
      st = fail(ZDS_EIO, "%s: write to %s failed", fn, tmp.c_str());
    std::vector<uint64_t> dig[3];
    float *arr[3] = {const_cast<float *>(master), const_cast<float *>(exp_avg), const_cast<float *>(exp_avg_sq)};
    const size_t data_off = kHeaderBytes + table_bytes;
    const size_t file_bytes = data_off + 3 * sizeof(float) * static_cast<size_t>(n);
    // reserve the blocks first, so a full disk is an error here and not a
    // fault in the mapping
    char *map = nullptr;
    if (st == ZDS_OK && n > 0) {
      const int rc = ::posix_fallocate(out.fd, 0, static_cast<off_t>(file_bytes));
      if (rc != 0) {
        st = fail(ZDS_EIO, "%s: cannot reserve %zu bytes for %s (%s)", fn, file_bytes, tmp.c_str(), std::strerror(rc));
      } else {
        void *m = ::mmap(nullptr, file_bytes, PROT_READ | PROT_WRITE, MAP_SHARED, out.fd, 0);
        map = m == MAP_FAILED ? nullptr : static_cast<char *>(m);  // no mapping: plain writes
      }
    }
    if (st == ZDS_OK)
      st = transfer(out.fd, map, true, on_host, arr, sizeof(float) * static_cast<size_t>(n),
                    static_cast<off_t>(data_off), dig, fn, tmp.c_str());
    if (map && ::munmap(map, file_bytes) != 0 && st == ZDS_OK) st = fail(ZDS_EIO, "%s: munmap failed", fn);
    if (st == ZDS_OK) {
      for (int k = 0; k < 3; ++k) hd.hash[k + 1] = fold(dig[k]);
      hd.head_hash = hash_of(&hd, offsetof(Header, head_hash));
      unsigned char head[kHeaderBytes] = {};
      std::memcpy(head, &hd, sizeof hd);
      if (!pwrite_all(out.fd, head, kHeaderBytes, 0)) st = fail(ZDS_EIO, "%s: header write failed", fn);
    }
    const int rc = ::close(out.fd);
    out.fd = -1;
    if (st == ZDS_OK && rc != 0) st = fail(ZDS_EIO, "%s: close failed", fn);
  }
  if (st != ZDS_OK) {
    ::unlink(tmp.c_str());
    return st;
  }
  if (std::rename(tmp.c_str(), path) != 0) {
    ::unlink(tmp.c_str());
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
  Fd in;
  zds_status st = open_read(path, &in, fn);
  if (st != ZDS_OK) return st;
  Header hd;
  std::vector<int64_t> numel;
  st = read_head(in.fd, path, &hd, &numel, fn);
  if (st != ZDS_OK) return st;
  *meta = hd.meta;
  if (state) *state = hd.state;
  const int32_t T = hd.meta.num_tensors;
  const int32_t copy = T < max_tensors ? T : max_tensors;
  if (numel_out && copy > 0) std::memcpy(numel_out, numel.data(), sizeof(int64_t) * static_cast<size_t>(copy));
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
  Fd in;
  st = open_read(path, &in, fn);
  if (st != ZDS_OK) return st;
  Header hd;
  std::vector<int64_t> table;
  st = read_head(in.fd, path, &hd, &table, fn);
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
  float *arr[3] = {master, exp_avg, exp_avg_sq};
  std::vector<uint64_t> dig[3];
  st = transfer(in.fd, nullptr, false, on_host, arr, sizeof(float) * static_cast<size_t>(n),
                static_cast<off_t>(kHeaderBytes + 8 * table.size()), dig, fn, path);
  if (st != ZDS_OK) return st;
  const char *what[3] = {"master", "exp_avg", "exp_avg_sq"};
  for (int k = 0; k < 3; ++k)
    if (fold(dig[k]) != hd.hash[k + 1])
      return fail(ZDS_EIO, "%s: %s is corrupt (%s does not match its hash)", fn, path, what[k]);
  if (on_host) {
    *state = hd.state;
    return ZDS_OK;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
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
    Fd in;
    zds_status st = open_read(paths[i], &in, fn);
    if (st != ZDS_OK) return st;
    st = read_head(in.fd, paths[i], &hd[i], i == 0 ? &numel : &other, fn);
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
  // tensors it covers; padding is dropped. Read piece by piece, so the
  // section's piece hashes come out as a side effect.
  std::vector<float> buf(kPiece / sizeof(float));
  for (int r = 0; r < num_files; ++r) {
    const Header &h = hd[by_rank[r]];
    const char *path = paths[by_rank[r]];
    Fd in;
    zds_status st = open_read(path, &in, fn);
    if (st != ZDS_OK) return st;
    const off_t base = static_cast<off_t>(kHeaderBytes + sizeof(int64_t) * static_cast<size_t>(T) +
                                          sizeof(float) * static_cast<size_t>(h.n) * static_cast<size_t>(section));
    std::vector<uint64_t> dig;
    int t = 0;
    for (int64_t pos = h.meta.lo; pos < h.meta.hi;) {
      const int64_t room = static_cast<int64_t>(buf.size());
      const int64_t len = h.meta.hi - pos < room ? h.meta.hi - pos : room;
      const size_t bytes = sizeof(float) * static_cast<size_t>(len);
      if (!pread_all(in.fd, buf.data(), bytes, base + static_cast<off_t>(sizeof(float) * (pos - h.meta.lo))))
        return fail(ZDS_EIO, "%s: %s is truncated", fn, path);
      dig.push_back(hash_of(buf.data(), bytes));
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
    if (fold(dig) != h.hash[section + 1])
      return fail(ZDS_EIO, "%s: %s is corrupt (section %d does not match its hash)", fn, path, section);
  }
  return ZDS_OK;
}
