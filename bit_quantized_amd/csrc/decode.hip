// Decode-side kernels: the 2 <= M <= 16 skinny GEMM and the deterministic
// split-K reduction it uses when N alone cannot fill the chip.
//
// "The 4-bit CPU path", section "W4A16": at decode a kernel whose cost is
// reading each weight once per call is good enough; these kernels
// stream every packed weight byte exactly once with 1 KiB-per-wavefront
// coalesced loads and unpack the nibbles in registers.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 1024;  // 16 wavefronts, one workgroup per compute unit
constexpr int kWaves = kThreads / 64;
constexpr int D = 4;            // units a wavefront keeps in flight
constexpr int kBufferWord3 = 0x00020000;  // raw byte buffer, gfx9 descriptor format
constexpr int kNontemporal = 2;           // cache policy bit: nt

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, float v) {
  if (a.ksplit == 1) {
    if (a.y) a.y[m * a.N + n] = f32_to_bf16_rne(a.sa[m] * v);
  } else {
    a.workspace[((int64_t)blockIdx.y * a.M + m) * a.N + n] = v;
  }
}

// One unit (16-channel block x one group) of a wavefront's run, as loaded.
struct Slot {
  v4u w;        // packed codes of this lane
  v4i a0, a1;   // activation row r16, input channels 16j.. and 64+16j.. of the group
  float s;      // scale of channel r16
  uint32_t zw;  // the zero block's dword holding channel r16's zero point
};

// ------------------------------------------------------------- 2 <= M <= 16
//
// One workgroup per 16-channel block (and K slice when the blocks alone
// cannot fill the machine); its 16 wavefronts split the slice's groups into
// contiguous runs and stream them through a ring of D register slots, as the
// GEMV does.  Every operand is read through a buffer descriptor bounded to
// what exists (the run's codes, scales and zeros; the M activation rows), so
// rows >= M and units past a run read as zeros with no memory request and
// every wavefront issues the same, compile-time count of loads (exact waits,
// no branches around loads).
//
// Per unit: one v_mfma_i32_16x16x64_i8 pair.  A is the activation tile, B
// the unpacked q - z bytes.  Lane l supplies A row l%16 and B column l%16
// with the same 16 input channels (16j..16j+15 for the first step, 64+16j..
// for the second, j = l/16); the instruction sums over all 64 slots, so the
// group's exact int32 product comes out per (row, column) without any
// cross-lane work.  Result layout: lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.  The wavefronts' pieces are summed in LDS in fixed
// wavefront order.
template <bool DEBUG>
__global__ void __launch_bounds__(kThreads)
skinny_kernel(GemmArgs a) {
  __shared__ float red[kWaves][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int64_t G = a.K / kGroup;
  // this wavefront's slice of the groups: G = gq * (ksplit * 16) + gr, the
  // first gr slices one group longer (quotient and remainder from the host,
  // so no division delays the first loads)
  const int pidx = blockIdx.y * kWaves + wave;
  const int gb = pidx * a.gq + min(pidx, a.gr);
  const int nrun = a.gq + (pidx < a.gr ? 1 : 0);
  const int64_t blk0 = nb * G + gb;  // first unit of the run in the packed planes

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.w.codes + blk0 * kBlockBytes, (int64_t)nrun * kBlockBytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.w.scales + blk0 * 16, (int64_t)nrun * 64);
  const __amdgpu_buffer_rsrc_t rz = rsrc_of(a.w.zeros + blk0 * kZeroBlockBytes, (int64_t)nrun * kZeroBlockBytes);
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(a.qa, a.M * a.K);
  const int oob = 0x7FFFFFF0;                       // beyond every descriptor
  const int act_lane = r16 < a.M ? r16 * (int)a.K + 16 * j : oob;

  auto load = [&](int r, Slot& sl) __attribute__((always_inline)) {
    const bool live = r < nrun;  // wave-uniform
    const int g = gb + r;
    const v4u w = __builtin_amdgcn_raw_buffer_load_b128(rc, live ? r * kBlockBytes + 16 * lane : oob, 0,
                                                        kNontemporal);
    const int ao = live && act_lane != oob ? act_lane + g * kGroup : oob;
    sl.w = w;
    sl.a0 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, ao, 0, 0));
    sl.a1 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                        ra, ao == oob ? oob : ao + 64, 0, 0));
    sl.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rs, live ? r * 64 + 4 * r16 : oob, 0, 0));
    sl.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, live ? r * kZeroBlockBytes + (r16 >> 3) * 4 : oob,
                                                 0, 0);
  };

  float accf[4] = {0.f, 0.f, 0.f, 0.f};
  Slot ring[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    load(i, ring[i]);
    __builtin_amdgcn_sched_barrier(0);  // slot order = issue order, so waits stay exact
  }
  const int zshift = (r16 & 7) * 4;  // nibble of channel r16 in its dword
  for (int ub = 0; ub < nrun; ub += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      // a slot past the run holds zeros (codes, zero point, activations and
      // scale all read as 0), so computing it adds exactly nothing: no branch
      const int r = ub + i;
      {
        const Slot& sl = ring[i];
        const uint32_t zz = ((sl.zw >> zshift) & 0xFu) * 0x01010101u;
        v4i b0, b1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t d = sl.w[w];
          b0[w] = (int)sub_zero_bytes(d & 0x0F0F0F0Fu, zz);
          b1[w] = (int)sub_zero_bytes((d >> 4) & 0x0F0F0F0Fu, zz);
        }
        v4i acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(sl.a0, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(sl.a1, b1, acc, 0, 0, 0);
        if (DEBUG && a.partials && r < nrun) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = 4 * j + q;
            if (m < a.M && m >= a.m_begin && m < a.m_end)
              a.partials[((m - a.m_begin) * a.N + 16 * nb + r16) * G + (gb + r)] = acc[q];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) accf[q] += sl.s * (float)acc[q];
      }
      load(r + D, ring[i]);  // refill with the unit D ahead (zeros past the run)
      __builtin_amdgcn_sched_barrier(0);  // keep the ring order: refill before the next slot
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave][q][lane] = accf[q];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t = red[0][q][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += red[w][q][lane];
      const int64_t m = 4 * j + q;
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

// Split K only while the channel blocks alone leave compute units idle, and
// never below one group per wavefront.
int pick_ksplit(int64_t N, int64_t K) {
  const int64_t nb = N / kBlockCols, G = K / kGroup;
  const int64_t cus = device_cus();
  int ks = 1;
  while (nb * ks * 2 <= cus && G >= (int64_t)ks * 2 * kWaves) ks *= 2;
  return ks;
}

}  // namespace

int skinny_ksplit(int64_t, int64_t N, int64_t K) { return pick_ksplit(N, K); }

hipError_t launch_skinny(GemmArgs a, hipStream_t st) {
  const int64_t G = a.K / kGroup, parts = (int64_t)a.ksplit * kWaves;
  a.gq = (int)(G / parts);
  a.gr = (int)(G % parts);
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
