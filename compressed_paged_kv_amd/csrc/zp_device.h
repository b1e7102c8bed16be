// Device helpers shared by the kernels: 16-byte global loads and stores.
//
// Pool and query pointers reach the kernels through parameter structs and a
// device-side pointer table, so the compiler cannot prove they point to
// global memory and would emit flat instructions (which also occupy the LDS
// counter).  Casting to address space 1 selects global_load / global_store.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zp {

// HIP's uint4 is a struct, and loads of it through an address-space-1
// pointer still become flat instructions; a native vector type does not.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t g_cu32x4;
typedef __attribute__((address_space(1))) u32x4_t g_u32x4;

__device__ inline uint4 ldg16(const void* p) {
  const u32x4_t v = *(g_cu32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void stg16(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  *(g_u32x4*)(p) = w;
}

// Streaming variants: the data is touched once, so ask the memory system not
// to keep it (non-temporal hint on the global load / store).
__device__ inline uint4 ldg16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((g_cu32x4*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void stg16_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (g_u32x4*)(p));
}

// Blocks request r holds when rows are ragged: the index of the first
// negative entry of its source row, clamped to [n_max, n_src]; otherwise
// n_src.  Every lane of a wave gets the same value.
__device__ inline int unit_blocks(const int32_t* src, int src_stride, int r, int n_src, int n_max,
                                  int ragged) {
  if (!ragged) return n_src;
  const int32_t* row = src + (size_t)r * src_stride;
  const int lane = threadIdx.x & 63;
  int first = n_src;
  for (int k0 = 0; k0 < n_src; k0 += 64) {
    const int k = k0 + lane;
    const unsigned long long neg = __ballot(k < n_src && row[k] < 0);
    if (neg) {
      first = k0 + __builtin_ctzll(neg);
      break;
    }
  }
  return first < n_max ? n_max : first;
}

}  // namespace zp
