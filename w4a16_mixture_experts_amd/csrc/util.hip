// Small utility kernels: the plain device copy (the kernel of known traffic used to
// calibrate HBM byte counters), span slot reset and the expert->slot table upload.
#include "common.h"

namespace exmoe {

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Launch span slots back to "not run": min start = all ones, max end = 0.
__global__ __launch_bounds__(256) void span_fill_kernel(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    p[2 * i] = ~0ull;
    p[2 * i + 1] = 0ull;
  }
}

hipError_t span_fill(unsigned long long* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(span_fill_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// An expert->slot table passed by value: the launch copies it into the kernel arguments, so
// the host buffer is free as soon as the call returns and nothing waits for the stream.
struct SlotTableArg {
  int32_t v[kMaxExperts];
};

__global__ __launch_bounds__(kMaxExperts) void table_fill_kernel(int32_t* __restrict__ dst, SlotTableArg t, int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = t.v[i];
}

hipError_t table_upload(int32_t* dst, const int32_t* host, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxExperts) return hipErrorInvalidValue;
  SlotTableArg t;
  for (int i = 0; i < n; i++) t.v[i] = host[i];
  hipLaunchKernelGGL(table_fill_kernel, dim3(1), dim3(kMaxExperts), 0, s, dst, t, n);
  return hipGetLastError();
}

// Every expert with rows must have been in one of the waves (mask bit set); otherwise its
// rows were never computed and the output of its tokens is undefined: flag it.
struct WaveMaskArg {
  uint32_t m[kMaxExperts / 32];
};

__global__ __launch_bounds__(kMaxExperts) void wave_union_kernel(const int32_t* __restrict__ offsets, int E, WaveMaskArg mk,
                                                                 uint32_t* __restrict__ debug) {
  const int e = threadIdx.x;
  if (e < E && offsets[e + 1] > offsets[e] && !((mk.m[e >> 5] >> (e & 31)) & 1u))
    atomicOr(debug, (uint32_t)EXMOE_FLAG_EXPERT_WITHOUT_SLOT);
}

hipError_t check_wave_union(const int32_t* offsets, int E, const uint32_t mask[kMaxExperts / 32], uint32_t* debug,
                            hipStream_t s) {
  WaveMaskArg mk;
  for (int i = 0; i < kMaxExperts / 32; i++) mk.m[i] = mask[i];
  hipLaunchKernelGGL(wave_union_kernel, dim3(1), dim3(kMaxExperts), 0, s, offsets, E, mk, debug);
  return hipGetLastError();
}

}  // namespace exmoe

using namespace exmoe;

extern "C" int exmoe_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "exmoe_device_copy: NULL pointer");
  if (bytes % 16 || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "exmoe_device_copy: size and pointers must be 16-byte multiples");
  if (bytes == 0) return EXMOE_OK;
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  ProfScope prof("copy", stream);
  EXMOE_LAUNCH(prof, copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const uint4*>(src),
               static_cast<uint4*>(dst), n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? EXMOE_OK : hip_error(e, "copy_kernel launch");
}
