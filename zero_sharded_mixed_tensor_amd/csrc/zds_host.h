// Host-side helpers of the library's CPU paths (offloaded optimizer,
// checkpoint I/O).
#pragma once

#include <sched.h>

#include <thread>

namespace zds {

// Threads the process may run at once: the CPUs of its affinity mask (a
// container or a job's CPU share), else the hardware's count; at least 1.
inline int host_thread_budget() {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  const unsigned hc = std::thread::hardware_concurrency();
  return hc > 0 ? static_cast<int>(hc) : 1;
}

}  // namespace zds
