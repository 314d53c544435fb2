// A host-memory stand-in for the HIP runtime, for the host-only check of the
// library under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// with no GPU. Test infrastructure: it is linked into the check program only,
// never into the library that applications load.
//
// Device allocations are host allocations (so an overrun by the library's host
// code of a buffer it sized itself shows up as a heap overflow), copies and
// fills are memcpy / memset, events and streams are tokens, and a kernel
// launch records the kernel's name and launch shape instead of running: the
// check program then verifies the shapes. Nothing here runs device code.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "hip_stub.h"

namespace {

std::mutex g_mu;
std::map<const void*, std::string> g_kernels;   // host stub -> kernel name
std::map<void*, size_t> g_allocs;               // live device allocations
std::vector<StubLaunch> g_launches;
std::vector<std::vector<unsigned char>> g_first_args;  // per launch: the kept copy
std::vector<std::pair<std::string, size_t>> g_capture;  // name part, bytes
int g_fail_malloc_after = -1;                   // fail the n-th next hipMalloc
struct CallConfig {
  dim3 grid, block;
  size_t shmem;
  hipStream_t stream;
};
thread_local std::vector<CallConfig> g_config;
int g_dummy_module;

}  // namespace

extern "C" {

void** __hipRegisterFatBinary(const void*) { return reinterpret_cast<void**>(&g_dummy_module); }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void* host_function, char*, const char* device_name, unsigned int,
                           uint3*, uint3*, dim3*, dim3*, int*) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_kernels[host_function] = device_name ? device_name : "?";
}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_config.push_back({grid, block, shmem, stream});
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  if (g_config.empty()) return hipErrorInvalidConfiguration;
  const CallConfig c = g_config.back();
  g_config.pop_back();
  *grid = c.grid;
  *block = c.block;
  *shmem = c.shmem;
  *stream = c.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* f, dim3 grid, dim3 block, void** args, size_t shmem, hipStream_t) {
  std::lock_guard<std::mutex> lk(g_mu);
  StubLaunch l;
  auto it = g_kernels.find(f);
  const std::string name = it == g_kernels.end() ? "<unregistered>" : it->second;
  std::snprintf(l.name, sizeof(l.name), "%s", name.c_str());
  l.grid[0] = grid.x; l.grid[1] = grid.y; l.grid[2] = grid.z;
  l.block[0] = block.x; l.block[1] = block.y; l.block[2] = block.z;
  l.shmem = shmem;
  g_launches.push_back(l);
  std::vector<unsigned char> kept;
  for (const auto& c : g_capture)
    if (args && args[0] && name.find(c.first) != std::string::npos) {
      const unsigned char* p = static_cast<const unsigned char*>(args[0]);
      kept.assign(p, p + c.second);
      break;
    }
  g_first_args.push_back(std::move(kept));
  return hipSuccess;
}

hipError_t hipMalloc(void** p, size_t bytes) {
  if (!p) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_fail_malloc_after == 0) {
    g_fail_malloc_after = -1;
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  if (g_fail_malloc_after > 0) --g_fail_malloc_after;
  // 256-byte aligned like device allocations; at least one byte
  *p = std::aligned_alloc(256, (bytes + 255) / 256 * 256 + (bytes == 0 ? 256 : 0));
  if (!*p) return hipErrorOutOfMemory;
  g_allocs[*p] = bytes;
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  if (!p) return hipSuccess;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_allocs.find(p);
  if (it == g_allocs.end()) {
    std::fprintf(stderr, "hip_stub: hipFree of %p, which hipMalloc did not return\n", p);
    std::abort();
  }
  g_allocs.erase(it);
  std::free(p);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  if (bytes) std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipMemset(void* dst, int value, size_t bytes) {
  if (bytes) std::memset(dst, value, bytes);
  return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
  // the host shadow of a __device__ array has the array's size
  *p = const_cast<void*>(symbol);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = reinterpret_cast<hipEvent_t>(new int(0));
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<int*>(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) { return e ? hipSuccess : hipErrorInvalidHandle; }
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidHandle; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  if (!a || !b) return hipErrorInvalidHandle;
  *ms = 0.001f;
  return hipSuccess;
}

// ---- queries for the check program
size_t stub_live_allocations(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_allocs.size();
}
size_t stub_allocation_size(const void* p) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_allocs.find(const_cast<void*>(p));
  return it == g_allocs.end() ? 0 : it->second;
}
size_t stub_launch_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_launches.size();
}
StubLaunch stub_launch(size_t i) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_launches.at(i);
}
void stub_clear_launches(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_launches.clear();
  g_first_args.clear();
}
void stub_fail_malloc_after(int n) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_fail_malloc_after = n;
}
void stub_capture_first_arg(const char* name_part, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_capture.size() < 4) g_capture.emplace_back(name_part, bytes);
}
size_t stub_launch_first_arg(size_t i, void* out, size_t max) {
  std::lock_guard<std::mutex> lk(g_mu);
  const std::vector<unsigned char>& k = g_first_args.at(i);
  if (out && max >= k.size() && !k.empty()) std::memcpy(out, k.data(), k.size());
  return k.size();
}

}  // extern "C"
