// Load-time weight packing (and its inverse) for the gfx950 layout.
//
// "The 4-bit CPU path", section "The weight layout, measured": deinterleaving
// per call cost 1.63x prefill, so every layout transform here runs once at
// load and the GEMM kernels read the packed planes directly.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

// One thread per 16-byte lane run of a codes block: reads the run's two
// 16-code slices of q (input channels 16j..16j+15 and 64+16j..64+16j+15 of
// the group) and interleaves them as low/high nibbles.
__global__ void __launch_bounds__(256)
pack_codes_kernel(const uint8_t* __restrict__ q, int64_t K, int64_t G, int64_t runs,
                  uint8_t* __restrict__ codes) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= runs) return;
  const int64_t blk = t >> 6;
  const int L = (int)(t & 63);
  const int64_t nb = blk / G, g = blk % G;
  const int j = L >> 4, c = L & 15;
  const uint8_t* row = q + (16 * nb + c) * K + 128 * g + 16 * j;
  uint4 lo = *reinterpret_cast<const uint4*>(row);
  uint4 hi = *reinterpret_cast<const uint4*>(row + 64);
  uint4 out;
  out.x = (lo.x & 0x0F0F0F0Fu) | ((hi.x & 0x0F0F0F0Fu) << 4);
  out.y = (lo.y & 0x0F0F0F0Fu) | ((hi.y & 0x0F0F0F0Fu) << 4);
  out.z = (lo.z & 0x0F0F0F0Fu) | ((hi.z & 0x0F0F0F0Fu) << 4);
  out.w = (lo.w & 0x0F0F0F0Fu) | ((hi.w & 0x0F0F0F0Fu) << 4);
  *reinterpret_cast<uint4*>(codes + t * 16) = out;
}

// One thread per (block, column): scale copy; even columns also write the
// zeros byte for columns c and c+1.
__global__ void __launch_bounds__(256)
pack_meta_kernel(const uint8_t* __restrict__ z, const float* __restrict__ s, int64_t G,
                 int64_t cells, uint8_t* __restrict__ zeros, float* __restrict__ scales) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= cells) return;
  const int64_t blk = t >> 4;
  const int c = (int)(t & 15);
  const int64_t nb = blk / G, g = blk % G;
  const int64_t n = 16 * nb + c;
  scales[t] = s[n * G + g];
  if ((c & 1) == 0) {
    // no zero points: the symmetric grid, every zero point 8
    uint32_t lo = z ? z[n * G + g] & 0xFu : 8u;
    uint32_t hi = z ? z[(n + 1) * G + g] & 0xFu : 8u;
    zeros[blk * kZeroBlockBytes + (c >> 1)] = (uint8_t)(lo | (hi << 4));
  }
}

// Zero the alignment gaps between the planes so that a packed buffer's bytes
// are fully determined by (q, z, s).
__global__ void __launch_bounds__(256)
zero_gaps_kernel(uint8_t* __restrict__ packed, int64_t a0, int64_t a1, int64_t b0, int64_t b1) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t na = a1 - a0;
  if (t < na)
    packed[a0 + t] = 0;
  else if (t < na + (b1 - b0))
    packed[b0 + t - na] = 0;
}

__global__ void __launch_bounds__(256)
unpack_codes_kernel(const uint8_t* __restrict__ codes, int64_t K, int64_t G, int64_t runs,
                    uint8_t* __restrict__ q) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= runs) return;
  const int64_t blk = t >> 6;
  const int L = (int)(t & 63);
  const int64_t nb = blk / G, g = blk % G;
  const int j = L >> 4, c = L & 15;
  uint4 v = *reinterpret_cast<const uint4*>(codes + t * 16);
  uint4 lo, hi;
  lo.x = v.x & 0x0F0F0F0Fu; hi.x = (v.x >> 4) & 0x0F0F0F0Fu;
  lo.y = v.y & 0x0F0F0F0Fu; hi.y = (v.y >> 4) & 0x0F0F0F0Fu;
  lo.z = v.z & 0x0F0F0F0Fu; hi.z = (v.z >> 4) & 0x0F0F0F0Fu;
  lo.w = v.w & 0x0F0F0F0Fu; hi.w = (v.w >> 4) & 0x0F0F0F0Fu;
  uint8_t* row = q + (16 * nb + c) * K + 128 * g + 16 * j;
  *reinterpret_cast<uint4*>(row) = lo;
  *reinterpret_cast<uint4*>(row + 64) = hi;
}

__global__ void __launch_bounds__(256)
unpack_meta_kernel(const uint8_t* __restrict__ zeros, const float* __restrict__ scales, int64_t G,
                   int64_t cells, uint8_t* __restrict__ z, float* __restrict__ s) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= cells) return;
  const int64_t blk = t >> 4;
  const int c = (int)(t & 15);
  const int64_t nb = blk / G, g = blk % G;
  const int64_t n = 16 * nb + c;
  s[n * G + g] = scales[t];
  z[n * G + g] = (uint8_t)zero_of(zeros + blk * kZeroBlockBytes, c);
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

// W8A8 weights: one thread per 16-byte run of a packed block.  Run t is
// (block nb*G + g, half h, lane L = 16j + c) and holds qw[16nb+c][128g +
// 64h + 16j .. +15]: the int8 codes of the MFMA B operand, copied as they are.
__global__ void __launch_bounds__(256)
w8_pack_codes_kernel(const int8_t* __restrict__ qw, int64_t K, int64_t G, int64_t runs,
                     uint8_t* __restrict__ codes) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= runs) return;
  const int64_t blk = t >> 7;
  const int h = (int)((t >> 6) & 1), L = (int)(t & 63);
  const int64_t nb = blk / G, g = blk % G;
  const int j = L >> 4, c = L & 15;
  const int8_t* src = qw + (16 * nb + c) * K + 128 * g + 64 * h + 16 * j;
  *reinterpret_cast<uint4*>(codes + 16 * t) = *reinterpret_cast<const uint4*>(src);
}

__global__ void __launch_bounds__(256)
w8_unpack_codes_kernel(const uint8_t* __restrict__ codes, int64_t K, int64_t G, int64_t runs,
                       int8_t* __restrict__ qw) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= runs) return;
  const int64_t blk = t >> 7;
  const int h = (int)((t >> 6) & 1), L = (int)(t & 63);
  const int64_t nb = blk / G, g = blk % G;
  const int j = L >> 4, c = L & 15;
  int8_t* dst = qw + (16 * nb + c) * K + 128 * g + 64 * h + 16 * j;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(codes + 16 * t);
}

__global__ void __launch_bounds__(256)
copy_f32_kernel(const float* __restrict__ src, int64_t n, float* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) dst[t] = src[t];
}

}  // namespace

// Packs a [N_part][K] weight into channels [n_offset, n_offset + N_part) of a
// buffer packed for N_total channels: every plane holds its channel blocks in
// order, so the part is one contiguous range of each plane.
hipError_t launch_pack_into(const uint8_t* q, const uint8_t* z, const float* s, int64_t N_part,
                            int64_t K, uint8_t* packed, int64_t N_total, int64_t n_offset,
                            hipStream_t st) {
  const int64_t G = K / kGroup;
  const int64_t b0 = n_offset / kBlockCols;  // first channel block of the part
  const int64_t runs = N_part * K / 32;      // 16-byte runs
  const int64_t cells = N_part * G;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(runs)), dim3(256), 0, st, q, K, G, runs,
                     packed + b0 * G * kBlockBytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_meta_kernel, dim3(blocks_for(cells)), dim3(256), 0, st, z, s, G, cells,
                     packed + zeros_offset(N_total, K) + b0 * G * kZeroBlockBytes,
                     reinterpret_cast<float*>(packed + scales_offset(N_total, K)) + b0 * G * 16);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the alignment gaps of the whole buffer (idempotent, so every part may)
  const int64_t a0 = N_total * K / 2, a1 = zeros_offset(N_total, K);
  const int64_t c0 = zeros_offset(N_total, K) + N_total * G / 2, c1 = scales_offset(N_total, K);
  const int64_t gaps = (a1 - a0) + (c1 - c0);
  if (gaps > 0) {
    hipLaunchKernelGGL(zero_gaps_kernel, dim3(blocks_for(gaps)), dim3(256), 0, st, packed, a0, a1,
                       c0, c1);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_pack(const uint8_t* q, const uint8_t* z, const float* s, int64_t N, int64_t K,
                       uint8_t* packed, hipStream_t st) {
  return launch_pack_into(q, z, s, N, K, packed, N, 0, st);
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, uint8_t* q, uint8_t* z,
                         float* s, hipStream_t st) {
  const int64_t G = K / kGroup;
  const int64_t runs = N * K / 32;
  const int64_t cells = N * G;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(runs)), dim3(256), 0, st, packed, K, G,
                     runs, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unpack_meta_kernel, dim3(blocks_for(cells)), dim3(256), 0, st,
                     packed + zeros_offset(N, K),
                     reinterpret_cast<const float*>(packed + scales_offset(N, K)), G, cells, z, s);
  return hipGetLastError();
}

// W8A8: codes plane [N/16][G][2][64][16] at 0, scales [N] at w8_scales_offset.
hipError_t launch_w8_pack(const int8_t* qw, const float* sw, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t st) {
  const int64_t G = K / kGroup, runs = N * K / 16;
  hipLaunchKernelGGL(w8_pack_codes_kernel, dim3(blocks_for(runs)), dim3(256), 0, st, qw, K, G, runs,
                     packed);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks_for(N)), dim3(256), 0, st, sw, N,
                     reinterpret_cast<float*>(packed + w8_scales_offset(N, K)));
  return hipGetLastError();
}

hipError_t launch_w8_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* qw, float* sw,
                            hipStream_t st) {
  const int64_t G = K / kGroup, runs = N * K / 16;
  hipLaunchKernelGGL(w8_unpack_codes_kernel, dim3(blocks_for(runs)), dim3(256), 0, st, packed, K, G,
                     runs, qw);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks_for(N)), dim3(256), 0, st,
                     reinterpret_cast<const float*>(packed + w8_scales_offset(N, K)), N, sw);
  return hipGetLastError();
}

}  // namespace w4a8
