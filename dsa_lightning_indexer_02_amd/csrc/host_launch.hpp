// Host-side launch helpers shared by the kernel launchers.
//
//  - set_max_dynamic_lds(kernel): raises a kernel's dynamic-LDS limit to gfx950's 160 KB once per
//    (kernel, device), under a mutex, so concurrent callers on several host threads or devices
//    neither race on the flag nor skip the attribute on a second GPU.
//  - device_props(): compute-unit count and LDS per CU of the current device, queried once per
//    device and cached (launchers that size their grid to the resident workgroups read it on every
//    call without a runtime query).
//  - occupancy_without_lds(kernel, threads): resident workgroups per CU allowed by the kernel's
//    registers and static LDS, queried once per (kernel, device, threads); a launcher divides the
//    LDS per CU by its dynamic LDS bytes for the rest of the bound.
//  - traced launch: with the environment variable DSA_TRACE set to a non-empty value other than
//    "0", every launch writes one line to stderr: kernel, grid, block, dynamic LDS, stream.
//  - stage events: between dsa_profile_begin and dsa_profile_end on a host thread, every launch
//    records the caller's next event on its stream right after the kernel, so consecutive events
//    bracket each kernel of a fused call.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

namespace dsa {

constexpr size_t kLdsPerWorkgroupMax = 160 * 1024;  // gfx950: 160 KB of LDS per compute unit

inline std::mutex& launch_cache_mutex() {
  static std::mutex m;
  return m;
}

// A failed runtime call also leaves its error as the thread's "last error", which the next
// unrelated check (ours or the caller's framework) would report: clear it and return it here.
inline hipError_t take_error(hipError_t e) {
  if (e != hipSuccess) (void)hipGetLastError();
  return e;
}

inline hipError_t set_max_dynamic_lds(const void* kernel) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return take_error(e);
  std::lock_guard<std::mutex> lock(launch_cache_mutex());
  static std::set<std::pair<const void*, int>> done;
  if (done.count({kernel, dev})) return hipSuccess;
  // the kernel's static LDS and its dynamic LDS share the 160 KB
  hipFuncAttributes attr{};
  e = hipFuncGetAttributes(&attr, kernel);
  if (e != hipSuccess) return take_error(e);
  const int dyn = (int)(kLdsPerWorkgroupMax - std::min<size_t>(attr.sharedSizeBytes, kLdsPerWorkgroupMax));
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  if (e == hipSuccess) done.insert({kernel, dev});
  return take_error(e);
}

struct DeviceProps {
  int cu_count;
  size_t lds_per_cu;
};

inline hipError_t device_props(DeviceProps* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return take_error(e);
  std::lock_guard<std::mutex> lock(launch_cache_mutex());
  static std::map<int, DeviceProps> cache;
  auto it = cache.find(dev);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int cus = 0, lds = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return take_error(e);
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e != hipSuccess) return take_error(e);
  DeviceProps p{cus, lds > 0 ? (size_t)lds : kLdsPerWorkgroupMax};
  cache.emplace(dev, p);
  *out = p;
  return hipSuccess;
}

inline hipError_t occupancy_without_lds(const void* kernel, int threads, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return take_error(e);
  std::lock_guard<std::mutex> lock(launch_cache_mutex());
  static std::map<std::tuple<const void*, int, int>, int> cache;
  const auto key = std::make_tuple(kernel, dev, threads);
  auto it = cache.find(key);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return take_error(e);
  cache.emplace(key, per_cu);
  *out = per_cu;
  return hipSuccess;
}

inline bool trace_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("DSA_TRACE");
    return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
  }();
  return on;
}

inline void trace_launch(const char* name, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  if (!trace_enabled()) return;
  std::fprintf(stderr, "[dsa] launch %s grid=(%u,%u,%u) block=%u lds=%zu stream=%p\n", name, grid.x, grid.y,
               grid.z, block.x * block.y * block.z, lds, (void*)stream);
}

// Stage timing of this host thread (a profiling aid): while active, each launch records the next
// caller-created event on its stream right after the kernel.
struct ProfileState {
  hipEvent_t* events = nullptr;
  int32_t capacity = 0;
  int32_t count = 0;
  std::vector<const char*> names;
};

inline ProfileState& profile_state() {
  thread_local ProfileState s;
  return s;
}

// Enqueue kernel<<<grid, block, lds, stream>>>(args...) after the optional trace line; returns the
// launch status.
template <typename Kernel, typename... Args>
inline hipError_t launch(const char* name, Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         Args... args) {
  trace_launch(name, grid, block, lds, stream);
  hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  hipError_t e = hipGetLastError();
  ProfileState& ps = profile_state();
  if (e == hipSuccess && ps.events && ps.count < ps.capacity) {
    e = take_error(hipEventRecord(ps.events[ps.count], stream));
    ps.names.push_back(name);
    ++ps.count;
  }
  return e;
}

// One line per C-ABI call that carves a caller workspace (under DSA_TRACE).
inline void trace_call(const char* name, size_t workspace_bytes, size_t workspace_used) {
  if (!trace_enabled()) return;
  std::fprintf(stderr, "[dsa] call %s workspace=%zu used=%zu\n", name, workspace_bytes, workspace_used);
}

}  // namespace dsa
