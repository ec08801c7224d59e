// Streaming probes of the memory system: a read of a large buffer and a copy
// between two, with 16-byte accesses spread over the whole chip.  They are
// not steps of the method: they measure the read and copy ceilings the
// kernels are compared with, and give the byte counters a transfer of known
// size to be calibrated against.
#include "kernels.h"

namespace logra {

namespace {

constexpr int kProbeThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeUnroll = 4;

// Every thread reads kProbeUnroll 16-byte words per pass, grid-strided, and
// folds them by XOR; one word per block is stored (blocks share 256 slots:
// the values only keep the loads from being removed).
__global__ void __launch_bounds__(kProbeThreads) probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                  u32x4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      acc ^= v[u];
    }
  }
  for (; i < n16; i += stride) {
    acc ^= src[i];
  }
  __shared__ u32x4 red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 t = u32x4{0u, 0u, 0u, 0u};
    for (int j = 0; j < kProbeThreads; ++j) {
      t ^= red[j];
    }
    out[blockIdx.x & 255] = t;
  }
}

// Copy: non-temporal loads, plain stores (the faster pair on this part).
__global__ void __launch_bounds__(kProbeThreads) probe_copy_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_probe(bool copy, const void* src, void* dst, int64_t bytes, int blocks_per_cu,
                        hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const dim3 grid((unsigned)(blocks_per_cu * compute_units()));
  if (copy)
    hipLaunchKernelGGL(probe_copy_kernel, grid, dim3(kProbeThreads), 0, s, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
  else
    hipLaunchKernelGGL(probe_read_kernel, grid, dim3(kProbeThreads), 0, s, static_cast<const u32x4*>(src),
                       n16, static_cast<u32x4*>(dst));
  return hipGetLastError();
}

}  // namespace logra
