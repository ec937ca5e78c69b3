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

typedef unsigned int v4u __attribute__((ext_vector_type(4)));


typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Four codes q (one per byte, 0..15) minus a zero point z (0..15) as four
// bfloat16, two per dword in byte order.  q + 16 - z lies in 1..31, so the
// per-byte subtraction borrows nothing; each byte converts exactly to float
// as an unsigned value and 16 is taken off exactly; small integers are exact
// in bf16, so the float's high half is the bf16.
__device__ __forceinline__ void codes_to_bf16x2(uint32_t nib4, uint32_t zz, int& lo, int& hi) {
  const uint32_t u = (nib4 + 0x10101010u) - zz;
  const float f0 = (float)(u & 0xFFu) - 16.0f, f1 = (float)((u >> 8) & 0xFFu) - 16.0f;
  const float f2 = (float)((u >> 16) & 0xFFu) - 16.0f, f3 = (float)(u >> 24) - 16.0f;
  lo = (int)__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = (int)__builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
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

// Raw activations of the fused-quantisation variant: NPT chunks of eight per
// thread, kept in registers between the row maximum and the codes.
template <typename T> struct XChunk {  // unused (int8 input): no raw activations
  static constexpr int kLoads = 1;
  static __device__ __forceinline__ float absmax(const v4u (*)[1], int) { return 0.0f; }
};
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <> struct XChunk<uint16_t> {  // bfloat16 bits: one 16-byte load
  static constexpr int kLoads = 1;
  // max |x| of n chunks: the magnitudes of finite bfloat16 values order as
  // their sign-cleared bit patterns, two per packed 16-bit maximum
  static __device__ __forceinline__ float absmax(const v4u (*r)[1], int n) {
    u16x2 m = {0, 0};
    for (int c = 0; c < n; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, r[c][0][i] & 0x7FFF7FFFu));
    return __uint_as_float((uint32_t)(m.x > m.y ? m.x : m.y) << 16);
  }
  static __device__ __forceinline__ void widen(const v4u* r, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[0][i] << 16);
      v[2 * i + 1] = __uint_as_float(r[0][i] & 0xFFFF0000u);
    }
  }
};
template <> struct XChunk<float> {  // two 16-byte loads
  static constexpr int kLoads = 2;
  static __device__ __forceinline__ float absmax(const v4u (*r)[2], int n) {
    float m = 0.0f;
    for (int c = 0; c < n; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(__uint_as_float(r[c][i >> 2][i & 3])));
    return m;
  }
  static __device__ __forceinline__ void widen(const v4u* r, float* v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(r[i >> 2][i & 3]);
  }
};

// NPT == 0: activations are the caller's int8 codes (row-major [M][K]).
// NPT > 0: the kernel quantises x (bf16 or f32, [M][K]) itself, with the
// rule of the stand-alone quantiser (sa = absmax / 127 by IEEE division,
// codes rint(x / sa) ties to even, clamped to +-127; a zero row gives sa 0
// and codes 0), into LDS: every workgroup covers all of K, so each one sees
// whole rows.  The row is split over 1024 / MP threads, each loading its NPT
// chunks of eight before the first weight loads (so waiting for them leaves
// the weight loads in flight); the wavefronts then read their A operands
// from LDS (row stride K + 16 bytes, which keeps a 16-lane read on distinct
// banks) instead of from memory.
//
// W8: the W8A8 weights instead (int8 per channel, packed as two 1 KiB halves
// per unit in MFMA operand order, one float scale per channel).  The bytes
// are the B operand as loaded, the products accumulate in int32 over all of
// K (exact), and the two scales are applied once, to the total.
//
// A16: W4A16 instead (bf16 activations, no quantisation).  Each workgroup
// copies its K slice of the M rows into LDS (row stride 2 * slice + 16
// bytes) and the wavefronts run four v_mfma_f32_16x16x32_bf16 per unit: B is
// q - z converted exactly to bf16, A the matching eight activations per lane
// (the four steps take input channels 16j.., 16j+8.., 64+16j.., 64+16j+8..
// of the group, the same slots in A and B), and the fp32 group sum is scaled
// by s into the accumulator.
constexpr int kA16Slack = 1536;  // LDS past the staged rows that padded quads may read
//
// A16 with NPT == 0 instead reads each unit's A operands straight from the
// row-major bf16 rows, four 16-byte loads per lane per unit (step t's eight
// values, exactly the MFMA layout), so the rows need no LDS and K no split.
// Units past a wavefront's run and rows >= M read as zeros.
//
// TILED (MP == 16, int8 codes from the caller, no debug): qa is in the
// [K / 16][16 rows][16 B] layout of launch_quant_tiled, so each lane's two
// A operands of a unit are two 16-byte loads at consecutive lane addresses
// (one contiguous KiB per wavefront), with no exchange between lanes (the
// row-major layout needs eight ds_bpermute per unit).  Rows M..15 of the
// layout are never written, and their lanes load nothing.  A layout with
// whole 128-byte row lines per group ([K / 128][16 rows][128 B]) was
// slower: its loads split into 16 pieces of 64 bytes.

// The operands the first loads need also lead the argument list as scalars,
// so that they arrive preloaded in scalar registers (kernel-argument preload)
// rather than behind a memory round trip; they overwrite the same fields of
// the by-value GemmArgs, which supplies everything else.
template <bool DEBUG, int MP, int NPT, typename T, bool W8, bool A16 = false, bool TILED = false>
__global__ void __launch_bounds__(kThreads)
skinny_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
              const uint8_t* __restrict__ zeros, const int8_t* __restrict__ qa,
              const void* __restrict__ x, int M, int K, int gq, int gr, GemmArgs a) {
  a.w.codes = codes;
  a.w.scales = scales;
  a.w.zeros = zeros;
  a.qa = qa;
  a.x = x;
  a.M = M;
  a.K = K;
  a.gq = gq;
  a.gr = gr;
  constexpr bool STAGE = NPT > 0;            // activations staged in LDS
  constexpr bool FUSED = STAGE && !A16;      // ... as int8 codes quantised here
  constexpr bool DIRECT16 = A16 && !STAGE;   // bf16 A operands loaded per unit
  constexpr int kUnitBytes = W8 ? 2 * kBlockBytes : kBlockBytes;  // codes per unit
  constexpr int CW = W8 ? 2 : 1;                                  // code loads per unit
  using S = ActShape<MP>;
  constexpr int kQuadLoads = STAGE || DIRECT16 ? 0 : S::kQuadLoads;
  constexpr int kSlotLoads = STAGE ? 0 : (DIRECT16 ? 4 : S::kSlotLoads);
  constexpr int QL = kQuadLoads > 0 ? kQuadLoads : 1;
  constexpr int SL = kSlotLoads > 0 ? kSlotLoads : 1;
  static_assert(!TILED || (MP == 16 && NPT == 0 && !A16 && !DEBUG), "tiled codes: M <= 16 GEMM only");
  __shared__ float red[kWaves][4][64];
  __shared__ float s_wmax[kWaves];
  __shared__ float s_sa[16];
  extern __shared__ __attribute__((aligned(16))) int8_t qs[];  // fused: [M][K + 16] codes
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int64_t G = a.K / kGroup;
  const int rstride = (int)a.K + 16;  // fused: LDS row stride of the codes

  // A16: groups [g_first, g_last) of K are this workgroup's slice
  const int g_first = (int)blockIdx.y * kWaves * a.gq + min((int)blockIdx.y * kWaves, a.gr);
  const int g_last = ((int)blockIdx.y + 1) * kWaves * a.gq + min(((int)blockIdx.y + 1) * kWaves, a.gr);
  const int rs16 = 2 * kGroup * (g_last - g_first) + 16;  // A16: LDS row stride in bytes

  // staged: this thread's row and chunks of eight, loaded before anything else
  constexpr int XL = STAGE ? XChunk<T>::kLoads : 1;
  constexpr int NX = STAGE ? NPT : 1;
  constexpr int kRowThreads = kThreads / MP;
  const int xrow = threadIdx.x / kRowThreads, xt = threadIdx.x % kRowThreads;
  const int cpr = A16 ? kGroup / 8 * (g_last - g_first) : (int)(a.K / 8);  // chunks per row
  // chunks xt, xt + 1024/MP, ... of row xrow: the first nx of them exist
  const int nx = xrow < a.M && xt < cpr ? (cpr - xt + kRowThreads - 1) / kRowThreads : 0;
  v4u xr[NX][XL];
  if constexpr (STAGE) {
    const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.x, a.M * a.K * (int64_t)sizeof(T));
    const int oob = 0x7FFFFFF0;
    const int off0 = (xrow * (int)a.K + (A16 ? kGroup * g_first : 0) + 8 * xt) * (int)sizeof(T);
#pragma unroll
    for (int c = 0; c < NPT; ++c) {
      const int off = c < nx ? off0 + c * 8 * kRowThreads * (int)sizeof(T) : oob;
#pragma unroll
      for (int l = 0; l < XL; ++l)
        xr[c][l] = __builtin_amdgcn_raw_buffer_load_b128(rx, off == oob ? oob : off + 16 * l, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // this wavefront's slice of the groups: G = gq * (ksplit * 16) + gr, the
  // first gr slices one group longer (quotient and remainder from the host,
  // so no division delays the first loads)
  const int pidx = blockIdx.y * kWaves + wave;
  const int gb = pidx * a.gq + min(pidx, a.gr);
  const int nrun = a.gq + (pidx < a.gr ? 1 : 0);
  const int nq = (nrun + 3) >> 2;
  const int64_t blk0 = nb * G + gb;  // first unit of the run in the packed planes

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.w.codes + blk0 * kUnitBytes, (int64_t)nrun * kUnitBytes);
  const __amdgpu_buffer_rsrc_t rs =
      W8 ? rsrc_of(a.w.scales, 0) : rsrc_of(a.w.scales + blk0 * 16, (int64_t)nrun * 64);
  const __amdgpu_buffer_rsrc_t rz =
      W8 ? rsrc_of(a.w.scales, 0)
         : rsrc_of(a.w.zeros + blk0 * kZeroBlockBytes, (int64_t)nrun * kZeroBlockBytes);
  const __amdgpu_buffer_rsrc_t ra =
      DIRECT16 ? rsrc_of(a.x, a.M * a.K * 2)
               : rsrc_of(a.qa, FUSED ? 0 : (TILED ? 16 : a.M) * a.K);
  const int oob = 0x7FFFFFF0;  // beyond every descriptor

  // activation row segment this lane fetches (row >= M: none)
  const int arow = lane / S::kLanesPerRow, aseg = lane % S::kLanesPerRow;
  const int act_base = arow < a.M ? arow * (int)a.K + gb * kGroup + 16 * aseg : oob;
  const int z_base = lane < 8 ? 4 * lane : oob;
  // fused: LDS byte offset of this lane's A operand for unit 0 of the run
  // (rows >= M read row M-1; their products are never stored)
  const int lds_a = A16 ? min(r16, (int)a.M - 1) * rs16 + (gb - g_first) * 2 * kGroup + 32 * j
                        : min(r16, (int)a.M - 1) * rstride + gb * kGroup + 16 * j;

  auto act_off = [&](int u) __attribute__((always_inline)) {  // unit u of the run, first byte
    return act_base == oob ? oob : act_base + u * kGroup;
  };
  // per-quad operands of quad q: scales, zeros, and (MP <= 4) the activations
  auto load_quad = [&](int q, uint32_t& s, uint32_t& z, v4i* act) __attribute__((always_inline)) {
    if constexpr (!W8) {
      s = __builtin_amdgcn_raw_buffer_load_b32(rs, (4 * q + j) * 64 + 4 * r16, 0, 0);
      z = __builtin_amdgcn_raw_buffer_load_b32(rz, z_base == oob ? oob : 4 * q * kZeroBlockBytes + z_base, 0, 0);
    } else {
      s = z = 0u;
    }
    if constexpr (kQuadLoads > 0) {
#pragma unroll
      for (int n = 0; n < kQuadLoads; ++n)
        act[n] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, act_off(4 * q + n * S::kUnitsPerLoad), 0, 0));
    }
  };
  // per-unit operands of unit u: codes and (MP >= 8) the activations
  // DIRECT16: byte offset of this lane's step-0 operand in unit u (row r16,
  // input channels 16j.. of the group; step t adds 128 (t / 2) + 16 (t % 2))
  const int a16_lane = r16 < a.M ? r16 * (int)a.K * 2 + gb * 2 * kGroup + 32 * j : oob;
  auto load_unit = [&](int u, v4u* w, v4i* act) __attribute__((always_inline)) {
    if constexpr (DIRECT16) {
      const int o = u < nrun && a16_lane != oob ? a16_lane + u * 2 * kGroup : oob;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        act[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, o == oob ? oob : o + 128 * (t >> 1) + 16 * (t & 1), 0, 0));
    } else if constexpr (TILED) {
      // unit gb + u of the layout: 2 KiB, half h at + 1024 h (rows >= M
      // read zeros, with no memory request)
      const int o = u < nrun && r16 < a.M ? (gb + u) * 2 * kBlockBytes + 16 * lane : oob;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        act[h] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, o == oob ? oob : o + h * kBlockBytes, 0, 0));
    } else if constexpr (kSlotLoads > 0) {
#pragma unroll
      for (int h = 0; h < kSlotLoads; ++h)
        act[h] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, act_off(u) == oob ? oob : act_off(u) + 64 * h, 0, 0));
    }
#pragma unroll
    for (int h = 0; h < CW; ++h)
      w[h] = __builtin_amdgcn_raw_buffer_load_b128(rc, u * kUnitBytes + h * kBlockBytes + 16 * lane,
                                                   0, kNontemporal);
  };

  // ds_bpermute byte addresses: source lane of this lane's A operand for
  // (unit-in-load du, half h) is base + 8 du + 4 h (MP <= 8) or 4 r + j
  // (MP == 16, one load per half)
  const int perm_a = MP == 16 ? 4 * (4 * r16 + j) : 4 * (S::kLanesPerRow * (r16 % MP) + j);
  const int perm_s = 4 * r16;              // + 64 i: scale of unit i, channel r16
  const int perm_z = 4 * (r16 >> 3);       // + 8 i: zero dword of unit i holding channel r16
  const int zshift = (r16 & 7) * 4;        // nibble of channel r16 in that dword

  float accf[4] = {0.f, 0.f, 0.f, 0.f};
  v4i acci = {0, 0, 0, 0};   // W8: int32 total over the run
  v4u wr[4][CW];             // codes ring, one slot per unit of the quad
  v4i ar[4][SL];             // per-unit activations (MP >= 8)
  v4i aq[2][QL];             // per-quad activations (MP <= 4), current and next quad
  uint32_t sq[2], zq[2];     // per-quad scales and zeros, current and next quad

  auto compute = [&](int q, int i, const v4u* w, const v4i* au, const v4i* aqc, uint32_t sc,
                     uint32_t zc) __attribute__((always_inline)) {
    if constexpr (A16) {
      const float s = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(perm_s + 64 * i, (int)sc));
      const uint32_t zw = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_z + 8 * i, (int)zc);
      const uint32_t zz = ((zw >> zshift) & 0xFu) * 0x01010101u;
      const int off = lds_a + (4 * q + i) * 2 * kGroup;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // step t: nibble half t / 2, code bytes 8 (t % 2) ..
        v4i av;
        if constexpr (DIRECT16)
          av = au[t];
        else
          av = *reinterpret_cast<const v4i*>(qs + off + (t >> 1) * kGroup + (t & 1) * 16);
        const int sh = (t >> 1) * 4;
        int b0, b1, b2, b3;
        codes_to_bf16x2((w[0][2 * (t & 1)] >> sh) & 0x0F0F0F0Fu, zz, b0, b1);
        codes_to_bf16x2((w[0][2 * (t & 1) + 1] >> sh) & 0x0F0F0F0Fu, zz, b2, b3);
        const v4i bv = {b0, b1, b2, b3};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                      __builtin_bit_cast(v8bf, bv), acc, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) accf[t] += s * acc[t];
      return;
    }
    v4i a0, a1;
    if constexpr (FUSED) {
      const int off = lds_a + (4 * q + i) * kGroup;
      a0 = *reinterpret_cast<const v4i*>(qs + off);
      a1 = *reinterpret_cast<const v4i*>(qs + off + 64);
    } else if constexpr (TILED) {
      a0 = au[0];
      a1 = au[1];
    } else if constexpr (MP == 16) {
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
    if constexpr (W8) {
      acci = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, __builtin_bit_cast(v4i, w[0]), acci, 0, 0, 0);
      acci = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, __builtin_bit_cast(v4i, w[1]), acci, 0, 0, 0);
      // The running total is otherwise only read after the loop, so the
      // compiler sinks every product there and keeps all slots' operands
      // live; an empty statement that reads and writes it pins each unit's
      // products in place (no instruction is emitted).
      asm volatile("" : "+v"(acci));
      return;
    }
    const float s = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(perm_s + 64 * i, (int)sc));
    const uint32_t zw = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_z + 8 * i, (int)zc);
    const uint32_t zz = ((zw >> zshift) & 0xFu) * 0x01010101u;
    v4i b0, b1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t d = w[0][t];
      b0[t] = (int)sub_zero_bytes(d & 0x0F0F0F0Fu, zz);
      b1[t] = (int)sub_zero_bytes((d >> 4) & 0x0F0F0F0Fu, zz);
    }
    v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, kBiasSeed, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
    const int r = 4 * q + i;
    if (DEBUG && a.partials && r < nrun) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t m = 4 * j + t;
        if (m < a.M && m >= a.m_begin && m < a.m_end)
          a.partials[((m - a.m_begin) * a.N + 16 * nb + r16) * G + (gb + r)] = acc[t] - kBiasBits;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) accf[t] += s * unbias(acc[t]);
  };

  // the first quad's loads (fused: after every wavefront has its
  // activations, which would otherwise queue behind these weight reads)
  auto load_first = [&]() __attribute__((always_inline)) {
    load_quad(0, sq[0], zq[0], aq[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_unit(i, wr[i], ar[i]);
      __builtin_amdgcn_sched_barrier(0);  // slot order = issue order, so waits stay exact
    }
  };
  if constexpr (A16 && STAGE) {
    // copy the slice's rows to LDS as they are, then the first weight loads.
    // The units that pad a run's last quad multiply zero weights by whatever
    // lies past the run (row pads, the slack after the rows): zeroed here,
    // since 0 times a bf16 NaN pattern would not be 0.
    int8_t* qrow = qs + xrow * rs16 + 16 * xt;
#pragma unroll
    for (int c = 0; c < NPT; ++c)
      if (c < nx) *reinterpret_cast<v4u*>(qrow + c * 16 * kRowThreads) = xr[c][0];
    if (threadIdx.x < (unsigned)a.M)
      *reinterpret_cast<v4u*>(qs + threadIdx.x * rs16 + rs16 - 16) = v4u{0u, 0u, 0u, 0u};
    if (threadIdx.x < kA16Slack / 16)
      *reinterpret_cast<v4u*>(qs + a.M * rs16 + 16 * threadIdx.x) = v4u{0u, 0u, 0u, 0u};
    __syncthreads();
    load_first();
  }
  if constexpr (!STAGE) load_first();
  if constexpr (FUSED) {
    // row maximum: this thread's chunks, its wavefront (one row per
    // wavefront, as a row spans 1024 / MP >= 64 threads), then the row's
    // wavefronts through LDS
    // (the raw chunks stay packed in registers; they are widened twice)
    float amax = XChunk<T>::absmax(xr, NPT);
    amax = wave_max64(amax);
    if (lane == 0) s_wmax[wave] = amax;
    __syncthreads();
    load_first();
    constexpr int kRowWaves = kRowThreads / 64;
    amax = s_wmax[xrow * kRowWaves];
#pragma unroll
    for (int w = 1; w < kRowWaves; ++w) amax = fmaxf(amax, s_wmax[xrow * kRowWaves + w]);
    const float scale = amax / 127.0f;
    const float inv = 1.0f / scale;
    if (xt == 0 && xrow < a.M) s_sa[xrow] = scale;
    int8_t* qrow = qs + xrow * rstride + 8 * xt;
#pragma unroll
    for (int c = 0; c < NPT; ++c) {
      if (c < nx) {
        float v[8];
        XChunk<T>::widen(xr[c], v);
        // a zero row gives codes 0 (its quotients would be 0/0)
        const uint2 codes = amax != 0.0f ? quant8_codes(v, scale, inv) : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(qrow + c * 8 * kRowThreads) = codes;
      }
    }
    __syncthreads();
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

  if constexpr (W8) {
    // exact int32 totals: the sum over wavefronts is order-free
    int (*redi)[4][64] = reinterpret_cast<int (*)[4][64]>(red);
#pragma unroll
    for (int t = 0; t < 4; ++t) redi[wave][t][lane] = acci[t];
    __syncthreads();
    if (wave == 0) {
      const int64_t n = 16 * nb + r16;
      const float swn = a.w.scales[n];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int p = redi[0][t][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) p += redi[w][t][lane];
        const int64_t m = 4 * j + t;
        if (m >= a.M) continue;
        if (a.ksplit > 1) {
          reinterpret_cast<int32_t*>(a.workspace)[((int64_t)blockIdx.y * a.M + m) * a.N + n] = p;
          continue;
        }
        if (DEBUG && a.partials && m >= a.m_begin && m < a.m_end) a.partials[(m - a.m_begin) * a.N + n] = p;
        float sam;
        if constexpr (FUSED)
          sam = s_sa[m];
        else
          sam = a.sa[m];
        if (a.y) a.y[m * a.N + n] = f32_to_bf16_rne(sam * (swn * (float)p));
      }
    }
    return;
  }
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
      if (m < a.M) {
        if constexpr (FUSED) {
          a.y[m * a.N + 16 * nb + r16] = f32_to_bf16_rne(s_sa[m] * v);
        } else if constexpr (A16) {
          if (a.ksplit == 1)
            a.y[m * a.N + 16 * nb + r16] = f32_to_bf16_rne(v);
          else
            a.workspace[((int64_t)blockIdx.y * a.M + m) * a.N + 16 * nb + r16] = v;
        } else {
          store_out(a, m, 16 * nb + r16, v);
        }
      }
    }
  }
}

// y[m][n] = bf16(sa[m] * sum_k ws[k][m][n]), summed in split order.  The
// per-token scale comes from `sa` (a device array written before this kernel
// runs: by the caller, or by the fused-quant GEMV).
// The slices cover columns [n0, N) of y: ws is [ksplit][M][N - n0].  Each
// thread takes eight consecutive outputs of one row (N - n0 is a multiple of
// 16): 16-byte loads of every slice, one 16-byte store.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ ws, int ksplit, const float* __restrict__ sa,
                     int64_t M, int64_t N, uint16_t* __restrict__ y, int64_t n0) {
  const int64_t W = N - n0;
  const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (t >= M * W) return;
  const int64_t m = t / W;
  float v[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(ws + t);
    const float4 b = *reinterpret_cast<const float4*>(ws + t + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  for (int k = 1; k < ksplit; ++k) {
    const float4 a = *reinterpret_cast<const float4*>(ws + k * M * W + t);
    const float4 b = *reinterpret_cast<const float4*>(ws + k * M * W + t + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  const float s = sa ? sa[m] : 1.0f;  // 1 * v == v exactly
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16_rne(s * v[2 * i]) | ((uint32_t)f32_to_bf16_rne(s * v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(y + m * N + n0 + t % W) = make_uint4(o[0], o[1], o[2], o[3]);
}

// W8A8 split-K: the exact int32 totals summed over the slices (order-free),
// then y[m][n] = bf16(sa[m] * (sw[n] * P)); totals also written for rows in
// [m_begin, m_end) when asked.
__global__ void __launch_bounds__(256)
w8_splitk_reduce_kernel(const int32_t* __restrict__ ws, int ksplit, const float* __restrict__ sa,
                        const float* __restrict__ sw, int64_t M, int64_t N, uint16_t* __restrict__ y,
                        int32_t* __restrict__ totals, int64_t m_begin, int64_t m_end, int64_t n0) {
  const int64_t W = N - n0;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M * W) return;
  const int64_t m = t / W, n = n0 + t % W;
  int p = ws[t];
  for (int k = 1; k < ksplit; ++k) p += ws[k * M * W + t];
  if (totals && m >= m_begin && m < m_end) totals[(m - m_begin) * N + n] = p;
  if (y) y[m * N + n] = f32_to_bf16_rne(sa[m] * (sw[n] * (float)p));
}

// Split K only while the channel blocks alone leave compute units idle, and
// never below one group per wavefront.
// Launch arguments of skinny_kernel: the preloaded scalars, then the struct.
#define SKINNY_ARGS(a) \
  (a).w.codes, (a).w.scales, (a).w.zeros, (a).qa, (a).x, (int)(a).M, (int)(a).K, (a).gq, (a).gr, (a)

int pick_ksplit(int64_t N, int64_t K) {
  const int64_t nb = N / kBlockCols, G = K / kGroup;
  const int64_t cus = device_cus();
  int ks = 1;
  while (nb * ks * 2 <= cus && G >= (int64_t)ks * 2 * kWaves) ks *= 2;
  return ks;
}

template <int MP, bool W8>
void launch_mp(const GemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.partials)
    hipLaunchKernelGGL((skinny_kernel<true, MP, 0, uint8_t, W8>), grid, dim3(kThreads), 0, st, SKINNY_ARGS(a));
  else if (MP == 16 && a.qa_tiled)
    hipLaunchKernelGGL((skinny_kernel<false, 16, 0, uint8_t, W8, false, true>), grid, dim3(kThreads), 0, st,
                       SKINNY_ARGS(a));
  else
    hipLaunchKernelGGL((skinny_kernel<false, MP, 0, uint8_t, W8>), grid, dim3(kThreads), 0, st, SKINNY_ARGS(a));
}

// Chunks of eight activations per thread of the fused variant, or 0 when it
// does not apply: one workgroup per channel block covering all of K, the
// M x (K + 16) codes within the LDS budget, and the thread's share of the
// row within the register budget.
constexpr int64_t kFusedLdsBytes = 128 * 1024;

int pow2_rows(int64_t M) { return M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// Every workgroup quantises all M rows again, so the fused form also needs
// the channel blocks to fit one round of workgroups: past that, the separate
// quantiser and the GEMM on its codes are faster (M = 4, K = 3584 -> N =
// 18944, 1184 blocks: 22.3 us fused against about 20 us; M = 16 there: 32.4
// against about 22 us).
int fused_chunks(int64_t M, int64_t N, int64_t K, int x_dtype) {
  if (M < 1 || M > 16 || pick_ksplit(N, K) != 1 || N / kBlockCols > device_cus()) return 0;
  if (M * (K + 16) + 512 > kFusedLdsBytes) return 0;
  const int64_t per_thread = (K / 8 + kThreads / pow2_rows(M) - 1) / (kThreads / pow2_rows(M));
  const int64_t limit = x_dtype == 0 ? 10 : 4;
  if (per_thread > limit) return 0;
  return per_thread <= 4 ? 4 : per_thread <= 8 ? 8 : 10;
}

template <int MP, typename T, bool W8>
void launch_fused_mp(const GemmArgs& a, dim3 grid, int npt, hipStream_t st) {
  const size_t lds = (size_t)(a.M * (a.K + 16) + 512);
  if (npt == 4)
    hipLaunchKernelGGL((skinny_kernel<false, MP, 4, T, W8>), grid, dim3(kThreads), lds, st, SKINNY_ARGS(a));
  else if constexpr (sizeof(T) == 2) {
    if (npt == 8)
      hipLaunchKernelGGL((skinny_kernel<false, MP, 8, T, W8>), grid, dim3(kThreads), lds, st, SKINNY_ARGS(a));
    else
      hipLaunchKernelGGL((skinny_kernel<false, MP, 10, T, W8>), grid, dim3(kThreads), lds, st, SKINNY_ARGS(a));
  }
}

template <typename T, bool W8>
void launch_fused(const GemmArgs& a, dim3 grid, int npt, hipStream_t st) {
  if (a.M <= 2)
    launch_fused_mp<2, T, W8>(a, grid, npt, st);
  else if (a.M <= 4)
    launch_fused_mp<4, T, W8>(a, grid, npt, st);
  else if (a.M <= 8)
    launch_fused_mp<8, T, W8>(a, grid, npt, st);
  else
    launch_fused_mp<16, T, W8>(a, grid, npt, st);
}

template <bool W8>
void launch_any(const GemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.x) {
    const int npt = fused_chunks(a.M, a.N, a.K, a.x_dtype);
    if (a.x_dtype == 0)
      launch_fused<uint16_t, W8>(a, grid, npt, st);
    else
      launch_fused<float, W8>(a, grid, npt, st);
  } else if (a.M <= 2) {
    launch_mp<2, W8>(a, grid, st);
  } else if (a.M <= 4) {
    launch_mp<4, W8>(a, grid, st);
  } else if (a.M <= 8) {
    launch_mp<8, W8>(a, grid, st);
  } else {
    launch_mp<16, W8>(a, grid, st);
  }
}

}  // namespace

bool skinny_fuses_quant(int64_t M, int64_t N, int64_t K, int x_dtype) {
  return fused_chunks(M, N, K, x_dtype) > 0;
}

int skinny_ksplit(int64_t, int64_t N, int64_t K) { return pick_ksplit(N, K); }

// The K split is the one that fills the machine (as for W4A8).  The rows are
// staged in LDS when the workgroup's slice of them fits (read once, with
// coalesced loads); otherwise each wavefront loads its A operands per unit
// straight from memory (npt 0).  Measured at K = 18944 -> N = 3584: staging
// that needed a further K split took 21.4 / 29.2 / 85.7 us at M = 4 / 8 / 16,
// direct loads 16.5 / 18.0 / 23.1 us; where the rows fit, staging is as fast
// or faster (M = 4, K = 3584 -> N = 18944: 23.8 us against 30.3 us).
A16Plan skinny_a16_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t G = K / kGroup;
  const int ks = pick_ksplit(N, K);
  // the first workgroup's slice is the longest: 16 runs of gq groups, plus
  // one more group for each of the first gr runs
  const int64_t parts = (int64_t)ks * kWaves, gq = G / parts, gr = G % parts;
  const int64_t slice = kWaves * gq + (gr < kWaves ? gr : kWaves);
  // (slack: a wavefront's padded last quad reads up to three units, 3 x 256
  // bytes, plus one operand span past its run)
  const int64_t lds = M * (2 * kGroup * slice + 16) + kA16Slack;
  const int64_t mp = pow2_rows(M);
  const int64_t npt = (kGroup / 8 * slice + kThreads / mp - 1) / (kThreads / mp);
  if (lds <= kFusedLdsBytes && npt <= 8) return A16Plan{ks, npt <= 4 ? 4 : 8, (size_t)lds};
  // direct loads address the rows with 32-bit offsets
  if (M * K * 2 <= kPrefillMaxBytes) return A16Plan{ks, 0, 0};
  return A16Plan{0, 0, 0};
}

hipError_t launch_skinny_a16(GemmArgs a, hipStream_t st) {
  const A16Plan p = skinny_a16_plan(a.M, a.N, a.K);
  if (p.ksplit == 0 || p.ksplit != a.ksplit || a.x_dtype != 0) return hipErrorInvalidValue;
  const int64_t G = a.K / kGroup, parts = (int64_t)a.ksplit * kWaves;
  a.gq = (int)(G / parts);
  a.gr = (int)(G % parts);
  const dim3 grid((unsigned)(a.N / kBlockCols), (unsigned)a.ksplit), block(kThreads);
  if (p.npt == 0) {
    hipLaunchKernelGGL((skinny_kernel<false, 16, 0, uint16_t, false, true>), grid, block, 0, st,
                       SKINNY_ARGS(a));
    return hipGetLastError();
  }
  const int mp = pow2_rows(a.M);
#define W4A16_LAUNCH(MPV, NPTV) \
  hipLaunchKernelGGL((skinny_kernel<false, MPV, NPTV, uint16_t, false, true>), grid, block, p.lds, st, SKINNY_ARGS(a))
  if (p.npt == 4) {
    if (mp == 2) W4A16_LAUNCH(2, 4); else if (mp == 4) W4A16_LAUNCH(4, 4);
    else if (mp == 8) W4A16_LAUNCH(8, 4); else W4A16_LAUNCH(16, 4);
  } else {
    if (mp == 2) W4A16_LAUNCH(2, 8); else if (mp == 4) W4A16_LAUNCH(4, 8);
    else if (mp == 8) W4A16_LAUNCH(8, 8); else W4A16_LAUNCH(16, 8);
  }
#undef W4A16_LAUNCH
  return hipGetLastError();
}

hipError_t launch_skinny(GemmArgs a, hipStream_t st) {
  const int64_t G = a.K / kGroup, parts = (int64_t)a.ksplit * kWaves;
  a.gq = (int)(G / parts);
  a.gr = (int)(G % parts);
  dim3 grid((unsigned)(a.N / kBlockCols), (unsigned)a.ksplit);
  if (a.x && (fused_chunks(a.M, a.N, a.K, a.x_dtype) == 0 || a.ksplit != 1 || a.partials))
    return hipErrorInvalidValue;
  if (a.qa_tiled && (a.x || a.partials || a.M <= 8 || a.M > 16)) return hipErrorInvalidValue;
  if (a.w8)
    launch_any<true>(a, grid, st);
  else
    launch_any<false>(a, grid, st);
  return hipGetLastError();
}

hipError_t launch_w8_splitk_reduce(const int32_t* ws, int ksplit, const float* sa, const float* sw,
                                   int64_t M, int64_t N, uint16_t* y, int32_t* totals,
                                   int64_t m_begin, int64_t m_end, hipStream_t st, int64_t n0) {
  const int64_t total = M * (N - n0);
  hipLaunchKernelGGL(w8_splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, ws, ksplit, sa, sw, M, N, y, totals, m_begin, m_end, n0);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, int ksplit, const float* sa, int64_t M,
                                int64_t N, uint16_t* y, hipStream_t st, int64_t n0) {
  if ((N - n0) % 16 || n0 % 16) return hipErrorInvalidValue;
  const int64_t total = M * (N - n0) / 8;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, ws, ksplit, sa, M, N, y, n0);
  return hipGetLastError();
}

}  // namespace w4a8
