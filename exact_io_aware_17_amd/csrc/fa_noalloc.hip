// Device scratch for fa_fwd_ex_noalloc: the split-KV workspace (arrival
// counters, partial softmax states) in a file-scope device array, so that the
// entry point allocates nothing. Each GPU the library runs on holds its own
// copy of the array, at its own address, until the process ends; the host
// finds that address once per device with hipGetSymbolAddress and passes it
// to the kernels like any caller-provided workspace. The array's name is
// never used as an address on the host.
#include "fa_internal.h"

#include <map>
#include <mutex>

namespace fa {
namespace {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// Sets n ints to zero (the arrival counters a split launch uses); a kernel
// rather than a memset, so the clear can sit in a captured graph.
__global__ __launch_bounds__(256) void clear_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

void* noalloc_scratch() {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of its copy of `scratch`
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next call
    return nullptr;
  }
  addr.emplace(dev, ptr);
  return ptr;
}

hipError_t clear_ints(int* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_ints_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p,
                     n);
  return hipGetLastError();
}

}  // namespace fa
