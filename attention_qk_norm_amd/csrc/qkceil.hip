// qkceil.hip -- streaming copy, read-only, write-only and empty kernels for
// gfx950: the bandwidth ceiling the QK-Norm kernels are measured against;
// and a probe of the shader clock between launches.
// They move data the way the QK-Norm kernels move rows (raw 16-byte buffer
// accesses with the non-temporal policy, every load of a lane issued before
// its stores), with no arithmetic in between.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkceil.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kLanes = 256;                 // 4 wavefronts per workgroup
constexpr int kRsrcConfig = 0x00020000;     // raw, untyped, 32-bit data format
constexpr uint64_t kMaxBytes = uint64_t{1} << 35;  // keeps grid.x * 256 below 2^32

// A workgroup's chunk as a buffer resource: accesses past `bytes` (the
// ragged last chunk) read zeros and drop their stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcConfig);
}

template <int U>
__device__ __forceinline__ uint32_t chunk_len(uint64_t total, uint64_t base) {
  constexpr uint64_t chunk = uint64_t{U} * kLanes * 16;
  return total - base < chunk ? static_cast<uint32_t>(total - base) : static_cast<uint32_t>(chunk);
}

template <int U>
__global__ void __launch_bounds__(kLanes) copy_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                      uint64_t bytes) {
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * U * kLanes * 16;
  const uint32_t len = chunk_len<U>(bytes, base);
  const auto r = chunk_rsrc(src + base, len);
  const auto w = chunk_rsrc(dst + base, len);
  u32x4 d[U];
#pragma unroll
  for (int j = 0; j < U; ++j)
    d[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (j * kLanes + threadIdx.x) * 16u, 0, 2);
#pragma unroll
  for (int j = 0; j < U; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(d[j], w, (j * kLanes + threadIdx.x) * 16u, 0, 2);
}

template <int U>
__global__ void __launch_bounds__(kLanes) read_kernel(const char* __restrict__ src, uint64_t bytes,
                                                      uint32_t* __restrict__ sink) {
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * U * kLanes * 16;
  const auto r = chunk_rsrc(src + base, chunk_len<U>(bytes, base));
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, (j * kLanes + threadIdx.x) * 16u, 0, 2);
    acc ^= d.x ^ d.y ^ d.z ^ d.w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

template <int U>
__global__ void __launch_bounds__(kLanes) write_kernel(char* __restrict__ dst, uint64_t bytes) {
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * U * kLanes * 16;
  const auto w = chunk_rsrc(dst + base, chunk_len<U>(bytes, base));
  const u32x4 v = {threadIdx.x, blockIdx.x, 0x51ED270Bu, static_cast<uint32_t>(base >> 4)};
#pragma unroll
  for (int j = 0; j < U; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(v, w, (j * kLanes + threadIdx.x) * 16u, 0, 2);
}

__global__ void __launch_bounds__(kLanes) empty_kernel() {}

// Cycles of this compute unit's clock over 200 ticks (2 us) of the 100 MHz
// real-time clock; the loop ends when the real-time clock has advanced.
__global__ void __launch_bounds__(64) clock_kernel(uint64_t* out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_readcyclecounter();
  uint64_t r1 = r0;
  while (r1 - r0 < 200) r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_readcyclecounter();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check(const void* a, const void* b, uint64_t bytes, int vpl) {
  if (a == nullptr || b == nullptr) return QKCEIL_ERR_NULL;
  if (bytes % 16 != 0 || bytes > kMaxBytes) return QKCEIL_ERR_SIZE;
  if (!aligned16(a) || !aligned16(b)) return QKCEIL_ERR_ALIGN;
  if (vpl != 1 && vpl != 2 && vpl != 4 && vpl != 8) return QKCEIL_ERR_CONFIG;
  return QKCEIL_OK;
}

dim3 grid_for(uint64_t bytes, int vpl) {
  const uint64_t chunk = static_cast<uint64_t>(vpl) * kLanes * 16;
  return dim3(static_cast<unsigned>((bytes + chunk - 1) / chunk));
}

int launched() { return hipGetLastError() == hipSuccess ? QKCEIL_OK : QKCEIL_ERR_DEVICE; }

}  // namespace

extern "C" {

int qkceil_copy(const void* src, void* dst, uint64_t bytes, int vectors_per_lane, void* stream) {
  const int st = check(src, dst, bytes, vectors_per_lane);
  if (st != QKCEIL_OK || bytes == 0) return st;
  const auto s = static_cast<hipStream_t>(stream);
  const dim3 g = grid_for(bytes, vectors_per_lane), b(kLanes);
  const auto* x = static_cast<const char*>(src);
  auto* y = static_cast<char*>(dst);
  switch (vectors_per_lane) {
    case 1: hipLaunchKernelGGL(copy_kernel<1>, g, b, 0, s, x, y, bytes); break;
    case 2: hipLaunchKernelGGL(copy_kernel<2>, g, b, 0, s, x, y, bytes); break;
    case 4: hipLaunchKernelGGL(copy_kernel<4>, g, b, 0, s, x, y, bytes); break;
    default: hipLaunchKernelGGL(copy_kernel<8>, g, b, 0, s, x, y, bytes); break;
  }
  return launched();
}

int qkceil_read(const void* src, uint64_t bytes, int vectors_per_lane, void* sink, void* stream) {
  const int st = check(src, sink, bytes, vectors_per_lane);
  if (st != QKCEIL_OK || bytes == 0) return st;
  const auto s = static_cast<hipStream_t>(stream);
  const dim3 g = grid_for(bytes, vectors_per_lane), b(kLanes);
  const auto* x = static_cast<const char*>(src);
  auto* k = static_cast<uint32_t*>(sink);
  switch (vectors_per_lane) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, g, b, 0, s, x, bytes, k); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, g, b, 0, s, x, bytes, k); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, g, b, 0, s, x, bytes, k); break;
    default: hipLaunchKernelGGL(read_kernel<8>, g, b, 0, s, x, bytes, k); break;
  }
  return launched();
}

int qkceil_write(void* dst, uint64_t bytes, int vectors_per_lane, void* stream) {
  const int st = check(dst, dst, bytes, vectors_per_lane);
  if (st != QKCEIL_OK || bytes == 0) return st;
  const auto s = static_cast<hipStream_t>(stream);
  const dim3 g = grid_for(bytes, vectors_per_lane), b(kLanes);
  auto* y = static_cast<char*>(dst);
  switch (vectors_per_lane) {
    case 1: hipLaunchKernelGGL(write_kernel<1>, g, b, 0, s, y, bytes); break;
    case 2: hipLaunchKernelGGL(write_kernel<2>, g, b, 0, s, y, bytes); break;
    case 4: hipLaunchKernelGGL(write_kernel<4>, g, b, 0, s, y, bytes); break;
    default: hipLaunchKernelGGL(write_kernel<8>, g, b, 0, s, y, bytes); break;
  }
  return launched();
}

int qkceil_empty(unsigned workgroups, void* stream) {
  if (workgroups == 0) return QKCEIL_ERR_CONFIG;
  hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(kLanes), 0, static_cast<hipStream_t>(stream));
  return launched();
}

int qkceil_clock(uint64_t* out, void* stream) {
  if (out == nullptr) return QKCEIL_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return QKCEIL_ERR_ALIGN;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out);
  return launched();
}

}  // extern "C"
