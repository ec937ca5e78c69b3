// On-device peak probes (include/w4a8_peaks.h): a streaming read for the HBM
// roofline and chains of int8 matrix-core instructions for the MFMA one,
// both measured in the same run as the kernels they are compared with.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kPeakThreads = 256;
// The folded value is stored only if it equals this constant, which keeps
// every load alive while (in practice) nothing is written.
constexpr uint32_t kNever = 0x9E3779B9u;

// Each workgroup reads one contiguous share of the n16 16-byte pieces,
// eight 1 KiB wavefront loads in flight per wavefront (whole HBM pages per
// workgroup rather than a grid-wide stride).
constexpr int kStreamUnroll = 8;
__global__ void __launch_bounds__(kPeakThreads)
stream_read_kernel(const v4i* __restrict__ p, int64_t n16, uint32_t* sink) {
  const int64_t share = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * share;
  const int64_t b1 = b0 + share < n16 ? b0 + share : n16;
  constexpr int kStep = kPeakThreads * kStreamUnroll;
  v4i acc = {0, 0, 0, 0};
  int64_t i = b0 + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * kPeakThreads < b1; i += kStep) {
    v4i r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) r[u] = __builtin_nontemporal_load(&p[i + u * kPeakThreads]);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= r[u];
  }
  for (; i < b1; i += kPeakThreads) acc ^= p[i];
  const uint32_t v = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (v == kNever) sink[blockIdx.x] = v;
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Eight independent accumulators per wavefront, so the matrix core never
// waits on a result; two operand sets alternate so the operands keep
// changing as they do in a real product.
__global__ void __launch_bounds__(kPeakThreads)
mfma_chain_kernel(int iters, int32_t* sink, uint64_t* clocks) {
  const uint32_t t = blockIdx.x * kPeakThreads + threadIdx.x;
  v4i a0, b0, a1, b1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] = (int)mix32(t * 16 + i);
    b0[i] = (int)mix32(t * 16 + 4 + i);
    a1[i] = (int)mix32(t * 16 + 8 + i);
    b1[i] = (int)mix32(t * 16 + 12 + i);
  }
  v4i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4i{0, 0, 0, 0};
  const uint64_t c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[j], 0, 0, 0);
    if (it + 1 < iters) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[j], 0, 0, 0);
    }
  }
  v4i f = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) f ^= acc[j];
  sink[t] = f[0] ^ f[1] ^ f[2] ^ f[3];
  if (clocks && threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = clock64() - c0;
    clocks[2 * blockIdx.x + 1] = wall_clock64() - r0;
  }
}

}  // namespace

hipError_t launch_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                   hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st,
                     static_cast<const v4i*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_peak_mfma_i8(int iters, int32_t* sink, uint64_t* clocks, int blocks,
                               hipStream_t st) {
  hipLaunchKernelGGL(mfma_chain_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0, st, iters,
                     sink, clocks);
  return hipGetLastError();
}

}  // namespace w4a8
