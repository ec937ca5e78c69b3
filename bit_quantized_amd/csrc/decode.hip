// Decode-side kernels: the 2 <= M <= 16 skinny GEMM and the deterministic
// split-K reduction it (and the M == 1 GEMV) use when N alone cannot fill the
// chip.
//
// "The 4-bit CPU path", section "W4A16": at decode a kernel whose cost is
// reading each weight once per call is good enough; these kernels
// stream every packed weight byte exactly once with 1 KiB-per-wavefront
// coalesced loads and unpack the nibbles in registers.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / 64;

// Balanced split of [0, n) into `parts` contiguous slices.
__device__ __forceinline__ int64_t slice_begin(int64_t n, int parts, int idx) {
  return n * idx / parts;
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, float v) {
  if (a.ksplit == 1) {
    if (a.y) a.y[m * a.N + n] = f32_to_bf16_rne(a.sa[m] * v);
  } else {
    a.workspace[((int64_t)blockIdx.y * a.M + m) * a.N + n] = v;
  }
}

// ------------------------------------------------------------- 2 <= M <= 16
//
// One v_mfma_i32_16x16x64_i8 pair per 16-channel block and group.  A is the
// activation tile (rows >= M read as zero), B the unpacked q - z bytes.  Lane
// l supplies A row l%16 and B column l%16 with the same 16 input channels
// (16j..16j+15 for the first step, 64+16j.. for the second, j = l/16); the
// instruction sums over all 64 slots, so the group's exact int32 product
// comes out per (row, column) without any cross-lane work.  Result layout:
// lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3.
template <bool DEBUG>
__global__ void __launch_bounds__(kThreads)
skinny_kernel(GemmArgs a) {
  __shared__ float red[kWaves][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int64_t G = a.K / kGroup;
  const int parts = a.ksplit * kWaves;
  const int pidx = blockIdx.y * kWaves + wave;
  const int64_t gb = slice_begin(G, parts, pidx), ge = slice_begin(G, parts, pidx + 1);
  const uint8_t* codes = a.w.codes + nb * G * kBlockBytes + 16 * lane;
  const uint8_t* zeros = a.w.zeros + nb * G * kZeroBlockBytes;
  const float* scales = a.w.scales + nb * G * 16 + r16;
  const bool row_ok = r16 < a.M;
  const int8_t* act = a.qa + (row_ok ? r16 : 0) * a.K + 16 * j;

  float accf[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int64_t g0 = gb; g0 < ge; g0 += U) {
    uint4 wv[U];
    v4i a0[U], a1[U];
    float sv[U];
    uint32_t zv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u < ge) {
        const int64_t g = g0 + u;
        wv[u] = *reinterpret_cast<const uint4*>(codes + g * kBlockBytes);
        if (row_ok) {
          a0[u] = *reinterpret_cast<const v4i*>(act + g * kGroup);
          a1[u] = *reinterpret_cast<const v4i*>(act + g * kGroup + 64);
        } else {
          a0[u] = v4i{0, 0, 0, 0};
          a1[u] = v4i{0, 0, 0, 0};
        }
        sv[u] = scales[g * 16];
        zv[u] = zero_of(zeros + g * kZeroBlockBytes, r16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u < ge) {
        const uint32_t zz = zv[u] * 0x01010101u;
        const uint32_t d[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
        v4i b0, b1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          b0[w] = (int)sub_zero_bytes(d[w] & 0x0F0F0F0Fu, zz);
          b1[w] = (int)sub_zero_bytes((d[w] >> 4) & 0x0F0F0F0Fu, zz);
        }
        v4i acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[u], b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[u], b1, acc, 0, 0, 0);
        if (DEBUG && a.partials) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t m = 4 * j + r;
            if (m < a.M && m >= a.m_begin && m < a.m_end)
              a.partials[((m - a.m_begin) * a.N + 16 * nb + r16) * G + (g0 + u)] = acc[r];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[r] += sv[u] * (float)acc[r];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = accf[r];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = red[0][r][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += red[w][r][lane];
      const int64_t m = 4 * j + r;
      if (m < a.M) store_out(a, m, 16 * nb + r16, t);
    }
  }
}

// y[m][n] = bf16(sa[m] * sum_k ws[k][m][n]), summed in split order.  The
// per-token scale comes from `sa` (a device array written before this kernel
// runs: by the caller, or by the fused-quant GEMV).
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ ws, int ksplit, const float* __restrict__ sa,
                     int64_t M, int64_t N, uint16_t* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M * N) return;
  const int64_t m = t / N;
  float v = ws[t];
  for (int k = 1; k < ksplit; ++k) v += ws[k * M * N + t];
  y[t] = f32_to_bf16_rne(sa[m] * v);
}

// Split K until the grid has about 4 workgroups per compute unit, keeping at
// least 2 groups per wavefront.
int pick_ksplit(int64_t N, int64_t K) {
  const int64_t nb = N / kBlockCols, G = K / kGroup;
  int ks = 1;
  while (nb * ks < 1024 && G >= (int64_t)ks * 2 * kWaves * 2) ks *= 2;
  return ks;
}

}  // namespace

int skinny_ksplit(int64_t, int64_t N, int64_t K) { return pick_ksplit(N, K); }

hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.N / kBlockCols), (unsigned)a.ksplit);
  if (a.partials)
    hipLaunchKernelGGL(skinny_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(skinny_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, int ksplit, const float* sa, int64_t M,
                                int64_t N, uint16_t* y, hipStream_t st) {
  const int64_t total = M * N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, ws, ksplit, sa, M, N, y);
  return hipGetLastError();
}

}  // namespace w4a8
