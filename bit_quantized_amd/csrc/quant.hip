// Per-token symmetric int8 activation quantisation.
//
// "The 4-bit CPU path", section "W4A8": activations are quantised to int8
// before the int4 x int8 product.  Reading taken here: one scale per token
// (row), sa = absmax / 127 with IEEE float division, codes rint(x / sa) with
// ties to even, clamped to [-127, 127]; an all-zero row has sa = 0, codes 0.
// The division is the correctly rounded one (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt and without fast-math), so the
// codes match any IEEE implementation of the same rule bit for bit.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kQuantThreads = 256;

template <typename T>
struct Chunk8;  // eight consecutive activations widened to float

template <>
struct Chunk8<uint16_t> {  // bfloat16 bits
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

template <>
struct Chunk8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ float wave_max(float v) { return wave_max64(v); }

// Codes of eight activations under one row scale (a zero row: codes 0).
__device__ __forceinline__ uint2 quant8(const float* v, float amax, float scale) {
  return amax != 0.0f ? quant8_codes(v, scale, 1.0f / scale) : make_uint2(0u, 0u);
}


// Row maximum over the block's wavefronts (all threads get it).
template <int THREADS>
__device__ __forceinline__ float block_max(float amax, float* red) {
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) amax = fmaxf(amax, red[w]);
  return amax;
}

// Long rows: the row is read twice (maximum, then codes) in a strided loop.
// HAD: rotated first (recomputed identically in the second pass); the
// stride of 256 chunks keeps every group in one 16-lane row.
template <typename T, bool HAD>
__global__ void __launch_bounds__(kQuantThreads)
quant_act_kernel(const T* __restrict__ x, int64_t K, int8_t* __restrict__ qa,
                 float* __restrict__ sa) {
  __shared__ float red[kQuantThreads / 64];
  const int64_t m = blockIdx.x;
  const T* row = x + m * K;
  const int64_t chunks = K / 8;

  float amax = 0.0f;
  for (int64_t ch = threadIdx.x; ch < chunks; ch += kQuantThreads) {
    float v[8];
    Chunk8<T>::load(row + ch * 8, v);
    if (HAD) hadamard_chunk(v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max<kQuantThreads>(amax, red);
  const float scale = amax / 127.0f;
  if (threadIdx.x == 0) sa[m] = scale;

  int8_t* out = qa + m * K;
  for (int64_t ch = threadIdx.x; ch < chunks; ch += kQuantThreads) {
    float v[8];
    Chunk8<T>::load(row + ch * 8, v);
    if (HAD) hadamard_chunk(v);
    *reinterpret_cast<uint2*>(out + ch * 8) = quant8(v, amax, scale);
  }
}

// Eight activations as float from their raw 16-byte loads (bf16: one
// load, f32: two).
template <typename T>
struct Raw8 {
  static constexpr int kLoads = sizeof(T) / 2;
  static __device__ __forceinline__ void widen(const uint4* r, float* v) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
};

// Byte offset of the eight codes of chunk ch (input channels 8 ch ..) of
// row m.  Row-major: m K + 8 ch.  TILED, [K / 16][16 rows][16 B] for at
// most 16 rows: 256 (ch / 2) + 16 m + 8 (ch % 2).  A 16-byte load per lane
// at 2048 g + 1024 h + 16 lane then gives lane 16 j + r the channels
// 128 g + 64 h + 16 j .. + 16 of row r: the int8 MFMA's A operand for half
// of group g, one contiguous KiB per wavefront, with no exchange between
// lanes.
template <bool TILED>
__device__ __forceinline__ int64_t code_offset(int64_t m, int64_t K, int ch) {
  if constexpr (TILED)
    return (int64_t)(ch >> 1) * 256 + m * 16 + (ch & 1) * 8;
  else
    return m * K + (int64_t)ch * 8;
}

// Rows of up to 8 * THREADS * NPT activations: every thread issues its NPT
// chunk loads back to back (through a descriptor over the row, so a chunk
// past the row reads zeros instead of branching around its load, which
// would make each load wait for the one before), keeps them in registers,
// and the block waits for memory once.  1024 threads per row serve few
// rows, where each block's latency is the whole cost; 256 serve many rows,
// which fill the machine by themselves.
template <typename T, int NPT, bool HAD, int kRowThreads, bool TILED>
__global__ void __launch_bounds__(kRowThreads)
quant_row_kernel(const T* __restrict__ x, int64_t K, int8_t* __restrict__ qa,
                 float* __restrict__ sa) {
  __shared__ float red[kRowThreads / 64];
  constexpr int L = Raw8<T>::kLoads;
  const int64_t m = blockIdx.x;
  const int chunks = (int)(K / 8);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(x + m * K, K * (int64_t)sizeof(T));
  uint4 raw[NPT][L];
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int ch = threadIdx.x + c * kRowThreads;
    const int off = ch < chunks ? ch * 8 * (int)sizeof(T) : kOob;
#pragma unroll
    for (int l = 0; l < L; ++l)
      raw[c][l] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off == kOob ? kOob : off + 16 * l, 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first wait
  float v[NPT][8];
#pragma unroll
  for (int c = 0; c < NPT; ++c) Raw8<T>::widen(raw[c], v[c]);
  if (HAD) {
    // whole groups are either all present or all absent (K % 128 == 0), so
    // the lanes of a group agree on every branch here
#pragma unroll
    for (int c = 0; c < NPT; ++c)
      if (threadIdx.x + c * kRowThreads < chunks) hadamard_chunk(v[c]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NPT; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
  amax = block_max<kRowThreads>(amax, red);
  const float scale = amax / 127.0f;
  if (threadIdx.x == 0) sa[m] = scale;
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int ch = threadIdx.x + c * kRowThreads;
    if (ch < chunks)
      *reinterpret_cast<uint2*>(qa + code_offset<TILED>(m, K, ch)) = quant8(v[c], amax, scale);
  }
}

template <typename T, bool HAD, int THREADS, bool TILED = false>
void launch_rows(const T* x, int64_t M, int64_t K, int8_t* qa, float* sa, hipStream_t st) {
  const int64_t chunks = K / 8;
  const dim3 grid((unsigned)M), block(THREADS);
  if (chunks <= THREADS)
    hipLaunchKernelGGL((quant_row_kernel<T, 1, HAD, THREADS, TILED>), grid, block, 0, st, x, K, qa, sa);
  else if (chunks <= 2 * THREADS)
    hipLaunchKernelGGL((quant_row_kernel<T, 2, HAD, THREADS, TILED>), grid, block, 0, st, x, K, qa, sa);
  else if (chunks <= 4 * THREADS)
    hipLaunchKernelGGL((quant_row_kernel<T, 4, HAD, THREADS, TILED>), grid, block, 0, st, x, K, qa, sa);
  else
    hipLaunchKernelGGL((quant_row_kernel<T, 8, HAD, THREADS, TILED>), grid, block, 0, st, x, K, qa, sa);
}

template <typename T, bool HAD>
void launch_typed(const T* x, int64_t M, int64_t K, int8_t* qa, float* sa, hipStream_t st) {
  const int64_t chunks = K / 8;
  if (M <= 64 && chunks <= 8 * 1024)
    launch_rows<T, HAD, 1024>(x, M, K, qa, sa, st);
  else if (M > 64 && chunks <= 8 * 256)
    launch_rows<T, HAD, 256>(x, M, K, qa, sa, st);
  else if (M > 64 && chunks <= 8 * 512)
    launch_rows<T, HAD, 512>(x, M, K, qa, sa, st);
  else
    hipLaunchKernelGGL((quant_act_kernel<T, HAD>), dim3((unsigned)M), dim3(kQuantThreads), 0, st, x,
                       K, qa, sa);
}

}  // namespace

hipError_t launch_quant(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* qa, float* sa,
                        hipStream_t st, bool hadamard) {
  if (x_dtype == 0) {
    if (hadamard)
      launch_typed<uint16_t, true>(static_cast<const uint16_t*>(x), M, K, qa, sa, st);
    else
      launch_typed<uint16_t, false>(static_cast<const uint16_t*>(x), M, K, qa, sa, st);
  } else {
    if (hadamard)
      launch_typed<float, true>(static_cast<const float*>(x), M, K, qa, sa, st);
    else
      launch_typed<float, false>(static_cast<const float*>(x), M, K, qa, sa, st);
  }
  return hipGetLastError();
}

hipError_t launch_quant_tiled(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* qa,
                              float* sa, hipStream_t st, bool hadamard) {
  if (M < 1 || M > 16 || K / 8 > 8 * 1024) return hipErrorInvalidValue;
  if (x_dtype == 0) {
    auto p = static_cast<const uint16_t*>(x);
    if (hadamard)
      launch_rows<uint16_t, true, 1024, true>(p, M, K, qa, sa, st);
    else
      launch_rows<uint16_t, false, 1024, true>(p, M, K, qa, sa, st);
  } else {
    auto p = static_cast<const float*>(x);
    if (hadamard)
      launch_rows<float, true, 1024, true>(p, M, K, qa, sa, st);
    else
      launch_rows<float, false, 1024, true>(p, M, K, qa, sa, st);
  }
  return hipGetLastError();
}

}  // namespace w4a8
