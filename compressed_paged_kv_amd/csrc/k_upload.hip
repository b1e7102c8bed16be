// Copy of the per-call tables (layer pointers, source and target block ids)
// from a pinned, device-visible host buffer into the workspace.  A kernel
// read of host memory costs one fabric round trip; the runtime's
// host-to-device copy of the same few kilobytes costs several times more on
// the stream.
#include "zp_device.h"
#include "zp_internal.h"

namespace zp {
namespace {

constexpr int kUploadThreads = 256;

__global__ __launch_bounds__(kUploadThreads) void k_upload(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kUploadThreads + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

}  // namespace

hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || (uintptr_t)host_src % 16 != 0 || (uintptr_t)dst % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t grid = (n16 + kUploadThreads - 1) / kUploadThreads;
  prof_begin(ZP_PHASE_UPLOAD, s);
  hipLaunchKernelGGL(k_upload, dim3((unsigned)grid), dim3(kUploadThreads), 0, s, static_cast<const uint4*>(host_src),
                     static_cast<uint4*>(dst), n16);
  prof_end(ZP_PHASE_UPLOAD, s);
  return hipGetLastError();
}

}  // namespace zp
