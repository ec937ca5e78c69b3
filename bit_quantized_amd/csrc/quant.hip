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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <typename T>
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
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);

  const float scale = amax / 127.0f;
  if (threadIdx.x == 0) sa[m] = scale;

  int8_t* out = qa + m * K;
  for (int64_t ch = threadIdx.x; ch < chunks; ch += kQuantThreads) {
    float v[8];
    Chunk8<T>::load(row + ch * 8, v);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = 0.0f;
      if (amax != 0.0f) {
        r = rintf(v[i] / scale);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
      }
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
      packed[i >> 2] |= b << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(out + ch * 8) = make_uint2(packed[0], packed[1]);
  }
}

}  // namespace

hipError_t launch_quant(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* qa, float* sa,
                        hipStream_t st) {
  if (x_dtype == 0) {
    hipLaunchKernelGGL(quant_act_kernel<uint16_t>, dim3((unsigned)M), dim3(kQuantThreads), 0, st,
                       static_cast<const uint16_t*>(x), K, qa, sa);
  } else {
    hipLaunchKernelGGL(quant_act_kernel<float>, dim3((unsigned)M), dim3(kQuantThreads), 0, st,
                       static_cast<const float*>(x), K, qa, sa);
  }
  return hipGetLastError();
}

}  // namespace w4a8
