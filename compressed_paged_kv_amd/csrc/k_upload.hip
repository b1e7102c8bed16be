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

// Per request, the lowest evicted slot over all its (layer, head) units
// (the evicted lists are ascending): every slot below it keeps its place in
// every layer and head.  Written straight to host-mapped memory.
__global__ __launch_bounds__(kUploadThreads) void k_first_evict(const int32_t* __restrict__ evicted,
                                                                int32_t* out, int R, int H, int L,
                                                                int E) {
  const int r = blockIdx.x * kUploadThreads + threadIdx.x;
  if (r >= R) return;
  int m = 0x7fffffff;
  for (int l = 0; l < L; l++)
    for (int h = 0; h < H; h++) m = min(m, evicted[(((size_t)l * R + r) * H + h) * E]);
  out[r] = m;
}

}  // namespace

hipError_t launch_first_evict(const int32_t* evicted, int32_t* host_out, int R, int H, int L, int E,
                              hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_first_evict, dim3((unsigned)((R + kUploadThreads - 1) / kUploadThreads)),
                     dim3(kUploadThreads), 0, s, evicted, host_out, R, H, L, E);
  return hipGetLastError();
}

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
