// hip_stub.cpp - the recording HIP runtime of the bounds-check build: the
// library's host code runs on the CPU against it. Allocations are host
// memory whose extents are recorded (bounds::inside checks spans against
// them), copies and fills act on that memory, kernel launches are counted
// and do nothing (the launchers' bounds hooks have already checked them),
// and the device reports the MI355X's 256 compute units. Host code only.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>

#include "../../../include/fno.h"
#include "../common.hpp"

namespace {

std::mutex mu;
std::map<uintptr_t, size_t> live;  // base -> bytes
long n_launch = 0, n_report = 0;

}  // namespace

namespace fno {
namespace bounds {

bool inside(const void *p, size_t n) {
  if (n == 0) return true;
  const uintptr_t a = (uintptr_t)p;
  std::lock_guard<std::mutex> g(mu);
  auto it = live.upper_bound(a);
  if (it == live.begin()) return false;
  --it;
  return a >= it->first && a - it->first <= it->second && n <= it->second - (a - it->first);
}

void report(const char *launch, const char *what) {
  std::lock_guard<std::mutex> g(mu);
  if (n_report < 50) std::fprintf(stderr, "bounds: %s: %s\n", launch, what);
  ++n_report;
}

}  // namespace bounds
}  // namespace fno

long check_launches() { return n_launch; }
long check_reports() { return n_report; }

// ---- the runtime entry points the library calls

hipError_t hipMalloc(void **ptr, size_t size) {
  if (!ptr) return hipErrorInvalidValue;
  if (size > ((size_t)8 << 30)) return hipErrorOutOfMemory;  // a small host stands in for the device
  void *p = nullptr;
  if (posix_memalign(&p, 256, size ? size : 1) != 0) return hipErrorOutOfMemory;
  std::memset(p, 0, size);
  std::lock_guard<std::mutex> g(mu);
  live[(uintptr_t)p] = size;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFree(void *ptr) {
  if (!ptr) return hipSuccess;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = live.find((uintptr_t)ptr);
    if (it == live.end()) return hipErrorInvalidValue;
    live.erase(it);
  }
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
  if (n && (!dst || !src)) return hipErrorInvalidValue;
  std::memmove(dst, src, n);
  return hipSuccess;
}

hipError_t hipMemset(void *dst, int v, size_t n) {
  if (n && !dst) return hipErrorInvalidValue;
  if (n && !fno::bounds::inside(dst, n)) fno::bounds::report("hipMemset", "outside every allocation");
  else std::memset(dst, v, n);
  return hipSuccess;
}

hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipGetDeviceCount(int *n) {
  *n = 1;
  return hipSuccess;
}
hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }

hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t attr, int) {
  switch (attr) {
    case hipDeviceAttributeMultiprocessorCount: *v = 256; break;
    case hipDeviceAttributeCooperativeLaunch: *v = 1; break;
    case hipDeviceAttributeMaxSharedMemoryPerBlock: *v = 160 * 1024; break;
    default: *v = 0;
  }
  return hipSuccess;
}

hipError_t hipFuncSetAttribute(const void *, hipFuncAttribute, int) { return hipSuccess; }

// resident workgroups per CU from threads (32 waves per CU) and LDS only
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int *n, const void *, int threads, size_t lds) {
  int by_t = threads > 0 ? 2048 / threads : 1;
  int by_l = lds > 0 ? (int)((160 * 1024) / lds) : 64;
  *n = by_t < by_l ? by_t : by_l;
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void **ptr, const void *symbol) {
  *ptr = const_cast<void *>(symbol);
  std::lock_guard<std::mutex> g(mu);
  live[(uintptr_t)symbol] = FNO_NOALLOC_SCRATCH_BYTES;  // the library's only symbol of this kind
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void *, dim3 grid, dim3 block, void **, size_t lds, hipStream_t) {
  if (grid.x < 1 || grid.y < 1 || grid.z < 1 || block.x < 1 || block.x > 1024) return hipErrorInvalidConfiguration;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> g(mu);
  ++n_launch;
  return hipSuccess;
}

hipError_t hipLaunchCooperativeKernel(const void *f, dim3 grid, dim3 block, void **args, unsigned int lds,
                                      hipStream_t s) {
  return hipLaunchKernel(f, grid, block, args, lds, s);
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *cs) {
  *cs = hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned int) {
  static int dummy;
  *s = reinterpret_cast<hipStream_t>(&dummy);
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { return hipSuccess; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t *g) {
  static int dummy;
  *g = reinterpret_cast<hipGraph_t>(&dummy);
  return hipSuccess;
}
hipError_t hipGraphInstantiate(hipGraphExec_t *e, hipGraph_t, hipGraphNode_t *, char *, size_t) {
  static int dummy;
  *e = reinterpret_cast<hipGraphExec_t>(&dummy);
  return hipSuccess;
}
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { return hipSuccess; }
hipError_t hipGraphDestroy(hipGraph_t) { return hipSuccess; }
hipError_t hipGraphExecDestroy(hipGraphExec_t) { return hipSuccess; }

// ---- what compiler-generated host code registers and calls

extern "C" {
void **__hipRegisterFatBinary(const void *) {
  static void *h = nullptr;
  return &h;
}
void __hipUnregisterFatBinary(void **) {}
void __hipRegisterFunction(void **, const void *, char *, const char *, unsigned int, void *, void *, void *, void *,
                           int *) {}
void __hipRegisterVar(void **, void *, char *, const char *, int, size_t, int, int) {}

// the <<<...>>> configuration, handed from the push to the generated stub's pop
namespace {
thread_local dim3 cfg_grid(1), cfg_block(1);
thread_local size_t cfg_lds = 0;
thread_local hipStream_t cfg_stream = nullptr;
}  // namespace

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  cfg_grid = grid;
  cfg_block = block;
  cfg_lds = lds;
  cfg_stream = s;
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3 *grid, dim3 *block, size_t *lds, hipStream_t *s) {
  *grid = cfg_grid;
  *block = cfg_block;
  *lds = cfg_lds;
  *s = cfg_stream;
  return hipSuccess;
}
}
