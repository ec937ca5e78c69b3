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

// ------------------------------------------------------------- 2 <= M <= 16
//
// One workgroup per 16-channel block (and K slice when the blocks alone
// cannot fill the machine); its 16 wavefronts split the slice's groups into
// contiguous runs and walk them four units (16 channels x one group) at a
// time.  Every operand is read through a buffer descriptor bounded to what
// exists (the run's codes, scales and zeros; the M activation rows), so
// units past a run read as zeros with no memory request and the compute
// needs no branch.
//
// Per unit: one v_mfma_i32_16x16x64_i8 pair.  A is the activation tile, B
// the unpacked q - z bytes.  Lane l supplies A row l%16 and B column l%16
// with the same 16 input channels (16j..16j+15 for the first step, 64+16j..
// for the second, j = l/16); the instruction sums over all 64 slots, so the
// group's exact int32 product comes out per (row, column) without any
// cross-lane work.  Result layout: lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.  The wavefronts' pieces are summed in LDS in fixed
// wavefront order.
//
// The cost of this kernel is its count of memory instructions more than its
// bytes, so each kind of operand is fetched with as few as its size allows
// and moved to the lanes that need it with ds_bpermute:
//   codes        one 1 KiB load per unit;
//   activations  coalesced row segments of the row-major int8 matrix: for
//                MP = 2, 4, 8 (M rounded up to a power of two) one load
//                holds MP rows x 1024/MP bytes, i.e. 8/MP units; for MP = 16
//                one load holds the 16 rows x 64 bytes of one unit-half;
//   scales       one load per four units (lane 16i+c: unit i, channel c);
//   zeros        one load per four units (lanes 0..7: the four 8-byte blocks).
// Loads are issued four units ahead (the next quad's per-quad operands
// first, then each unit's own as its slot frees), and the last quad issues
// nothing, so no load is made for a unit that a wavefront never computes
// beyond the at most three that pad its last quad.
template <int MP>
struct ActShape {
  static constexpr int kUnitsPerLoad = MP >= 8 ? 1 : 8 / MP;     // units one load covers
  static constexpr int kSlotLoads = MP == 16 ? 2 : (MP == 8 ? 1 : 0);  // loads per unit slot
  static constexpr int kQuadLoads = MP >= 8 ? 0 : 4 / kUnitsPerLoad;   // loads per quad
  static constexpr int kLanesPerRow = MP == 16 ? 4 : 64 / MP;
};

template <bool DEBUG, int MP>
__global__ void __launch_bounds__(kThreads)
skinny_kernel(GemmArgs a) {
  using S = ActShape<MP>;
  constexpr int QL = S::kQuadLoads > 0 ? S::kQuadLoads : 1;
  constexpr int SL = S::kSlotLoads > 0 ? S::kSlotLoads : 1;
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
  const int nq = (nrun + 3) >> 2;
  const int64_t blk0 = nb * G + gb;  // first unit of the run in the packed planes

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.w.codes + blk0 * kBlockBytes, (int64_t)nrun * kBlockBytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.w.scales + blk0 * 16, (int64_t)nrun * 64);
  const __amdgpu_buffer_rsrc_t rz = rsrc_of(a.w.zeros + blk0 * kZeroBlockBytes, (int64_t)nrun * kZeroBlockBytes);
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(a.qa, a.M * a.K);
  const int oob = 0x7FFFFFF0;  // beyond every descriptor

  // activation row segment this lane fetches (row >= M: none)
  const int arow = lane / S::kLanesPerRow, aseg = lane % S::kLanesPerRow;
  const int act_base = arow < a.M ? arow * (int)a.K + gb * kGroup + 16 * aseg : oob;
  const int z_base = lane < 8 ? 4 * lane : oob;

  auto act_off = [&](int u) __attribute__((always_inline)) {  // unit u of the run, first byte
    return act_base == oob ? oob : act_base + u * kGroup;
  };
  // per-quad operands of quad q: scales, zeros, and (MP <= 4) the activations
  auto load_quad = [&](int q, uint32_t& s, uint32_t& z, v4i* act) __attribute__((always_inline)) {
    s = __builtin_amdgcn_raw_buffer_load_b32(rs, (4 * q + j) * 64 + 4 * r16, 0, 0);
    z = __builtin_amdgcn_raw_buffer_load_b32(rz, z_base == oob ? oob : 4 * q * kZeroBlockBytes + z_base, 0, 0);
    if constexpr (S::kQuadLoads > 0) {
#pragma unroll
      for (int n = 0; n < S::kQuadLoads; ++n)
        act[n] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, act_off(4 * q + n * S::kUnitsPerLoad), 0, 0));
    }
  };
  // per-unit operands of unit u: codes and (MP >= 8) the activations
  auto load_unit = [&](int u, v4u& w, v4i* act) __attribute__((always_inline)) {
    if constexpr (S::kSlotLoads > 0) {
#pragma unroll
      for (int h = 0; h < S::kSlotLoads; ++h)
        act[h] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, act_off(u) == oob ? oob : act_off(u) + 64 * h, 0, 0));
    }
    w = __builtin_amdgcn_raw_buffer_load_b128(rc, u * kBlockBytes + 16 * lane, 0, kNontemporal);
  };

  // ds_bpermute byte addresses: source lane of this lane's A operand for
  // (unit-in-load du, half h) is base + 8 du + 4 h (MP <= 8) or 4 r + j
  // (MP == 16, one load per half)
  const int perm_a = MP == 16 ? 4 * (4 * r16 + j) : 4 * (S::kLanesPerRow * (r16 % MP) + j);
  const int perm_s = 4 * r16;              // + 64 i: scale of unit i, channel r16
  const int perm_z = 4 * (r16 >> 3);       // + 8 i: zero dword of unit i holding channel r16
  const int zshift = (r16 & 7) * 4;        // nibble of channel r16 in that dword

  float accf[4] = {0.f, 0.f, 0.f, 0.f};
  v4u wr[4];                 // codes ring, one slot per unit of the quad
  v4i ar[4][SL];             // per-unit activations (MP >= 8)
  v4i aq[2][QL];             // per-quad activations (MP <= 4), current and next quad
  uint32_t sq[2], zq[2];     // per-quad scales and zeros, current and next quad

  auto compute = [&](int q, int i, const v4u& w, const v4i* au, const v4i* aqc, uint32_t sc,
                     uint32_t zc) __attribute__((always_inline)) {
    v4i a0, a1;
    if constexpr (MP == 16) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0[t] = __builtin_amdgcn_ds_bpermute(perm_a, au[0][t]);
        a1[t] = __builtin_amdgcn_ds_bpermute(perm_a, au[1][t]);
      }
    } else {
      const int n = i / S::kUnitsPerLoad, du = i % S::kUnitsPerLoad;
      const v4i& src = MP == 8 ? au[0] : aqc[n];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0[t] = __builtin_amdgcn_ds_bpermute(perm_a + 32 * du, src[t]);
        a1[t] = __builtin_amdgcn_ds_bpermute(perm_a + 32 * du + 16, src[t]);
      }
    }
    const float s = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(perm_s + 64 * i, (int)sc));
    const uint32_t zw = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_z + 8 * i, (int)zc);
    const uint32_t zz = ((zw >> zshift) & 0xFu) * 0x01010101u;
    v4i b0, b1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t d = w[t];
      b0[t] = (int)sub_zero_bytes(d & 0x0F0F0F0Fu, zz);
      b1[t] = (int)sub_zero_bytes((d >> 4) & 0x0F0F0F0Fu, zz);
    }
    v4i acc = {0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
    const int r = 4 * q + i;
    if (DEBUG && a.partials && r < nrun) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t m = 4 * j + t;
        if (m < a.M && m >= a.m_begin && m < a.m_end)
          a.partials[((m - a.m_begin) * a.N + 16 * nb + r16) * G + (gb + r)] = acc[t];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) accf[t] += s * (float)acc[t];
  };

  load_quad(0, sq[0], zq[0], aq[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    load_unit(i, wr[i], ar[i]);
    __builtin_amdgcn_sched_barrier(0);  // slot order = issue order, so waits stay exact
  }
  int q = 0;
  for (; q < nq - 1; ++q) {
    load_quad(q + 1, sq[1], zq[1], aq[1]);  // next quad's shared operands first
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      compute(q, i, wr[i], ar[i], aq[0], sq[0], zq[0]);
      load_unit(4 * (q + 1) + i, wr[i], ar[i]);  // refill the slot with the next quad's unit
      __builtin_amdgcn_sched_barrier(0);
    }
    sq[0] = sq[1];
    zq[0] = zq[1];
#pragma unroll
    for (int n = 0; n < QL; ++n) aq[0][n] = aq[1][n];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) compute(q, i, wr[i], ar[i], aq[0], sq[0], zq[0]);

#pragma unroll
  for (int t = 0; t < 4; ++t) red[wave][t][lane] = accf[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += red[w][t][lane];
      const int64_t m = 4 * j + t;
      if (m < a.M) store_out(a, m, 16 * nb + r16, v);
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

template <int MP>
void launch_mp(const GemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.partials)
    hipLaunchKernelGGL((skinny_kernel<true, MP>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((skinny_kernel<false, MP>), grid, dim3(kThreads), 0, st, a);
}

hipError_t launch_skinny(GemmArgs a, hipStream_t st) {
  const int64_t G = a.K / kGroup, parts = (int64_t)a.ksplit * kWaves;
  a.gq = (int)(G / parts);
  a.gr = (int)(G % parts);
  dim3 grid((unsigned)(a.N / kBlockCols), (unsigned)a.ksplit);
  if (a.M <= 2)
    launch_mp<2>(a, grid, st);
  else if (a.M <= 4)
    launch_mp<4>(a, grid, st);
  else if (a.M <= 8)
    launch_mp<8>(a, grid, st);
  else
    launch_mp<16>(a, grid, st);
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
