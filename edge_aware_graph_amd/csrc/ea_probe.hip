// Achievable-bandwidth probes: a plain device copy and a plain device read,
// so that a benchmark can report the HBM rate this GPU reaches on a simple
// stream next to the layer's kernels (measurement context only; nothing in
// the layer uses them).
#include <hip/hip_runtime.h>

#include "ea_internal.h"

namespace ea {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte pieces in flight per thread and step
constexpr int kProbeBlocksPerCU = 8;

// dst[k] = src[k] for n16 16-byte pieces. Each step a thread moves
// kProbeUnroll pieces kProbeThreads apart (every load of a step is issued
// before the first store); the tail past the last whole step is moved one
// piece per thread.
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, size_t n16) {
  const size_t step = (size_t)kProbeThreads * kProbeUnroll;
  const size_t whole = n16 / step;
  for (size_t s = blockIdx.x; s < whole; s += gridDim.x) {
    const size_t base = s * step + threadIdx.x;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = src[base + (size_t)k * kProbeThreads];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) dst[base + (size_t)k * kProbeThreads] = v[k];
  }
  for (size_t k = whole * step + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; k < n16;
       k += (size_t)gridDim.x * kProbeThreads)
    dst[k] = src[k];
}

// XOR of every 32-bit word of n16 16-byte pieces into *out (one atomic per
// block), so that no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                   uint32_t* out) {
  const size_t step = (size_t)kProbeThreads * kProbeUnroll;
  const size_t whole = n16 / step;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t s = blockIdx.x; s < whole; s += gridDim.x) {
    const size_t base = s * step + threadIdx.x;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = src[base + (size_t)k * kProbeThreads];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k];
  }
  for (size_t k = whole * step + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; k < n16;
       k += (size_t)gridDim.x * kProbeThreads)
    acc ^= src[k];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0u;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= part[w];
    atomicXor(out, y);
  }
}

unsigned probe_blocks(size_t n16) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const size_t want = (size_t)cus * kProbeBlocksPerCU;
  const size_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  return (unsigned)(need < want ? (need > 0 ? need : 1) : want);
}

}  // namespace

// Launchers: n16 16-byte pieces (the caller checks pointers and alignment).
hipError_t launch_probe_copy(const void* src, void* dst, size_t n16, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(probe_blocks(n16)), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}
hipError_t launch_probe_read(const void* src, size_t n16, uint32_t* xor_out, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(probe_blocks(n16)), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(src), n16, xor_out);
  return hipGetLastError();
}

}  // namespace ea
