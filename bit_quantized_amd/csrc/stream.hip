// 1 <= M <= 16 GEMM for wide, short layers (N / 16 at least the number of
// compute units, K <= 4096): the weights are dealt out by bytes, whole
// channel blocks per workgroup, and each workgroup stages the activations
// once.
//
// "The 4-bit CPU path", section "W4A16": at decode a call costs what
// streaming the weights costs.  The M <= 16 kernel of decode.hip runs one
// workgroup per 16-channel block, so an up projection (K = 3584 ->
// N = 18944) is 1184 workgroups of 28 KiB each over several rounds of the
// compute units, every one of them fetching its own activation operands.
// Here a grid of C workgroups (a whole number of rounds, as the M == 1 GEMV
// does) takes channel blocks [cb0, cb1) each: C = 256 gives the up
// projection 4-5 blocks (112-140 KiB) per workgroup.
//
// The activation codes (all 16 operand rows: rows >= M repeat row M - 1,
// whose products are never stored) are copied once per workgroup into LDS in
// MFMA operand order, 2 KiB per group: half h of group g, lane L = 16j + r,
// holds row r, input channels 128g + 64h + 16j .. +15.  A fragment read is
// then one conflict-free ds_read_b128 per lane.
//
// The workgroup's units (16-channel block x group, 1 KiB of codes each,
// adjacent in the codes plane) are cut into 16 contiguous runs, one per
// wavefront; a run is at most as long as K has groups, so it meets at most
// two channel blocks.  Each wavefront stages its run's scales and zero points
// in LDS with two loads, streams its codes through a ring of D register
// slots (one 1 KiB load per unit; out-of-range offsets past the run return
// zeros and make no request), and runs one v_mfma_i32_16x16x64_i8 pair per
// unit: A the staged activations, B the codes unpacked to q - z bytes, the
// exact int32 group product per (row, channel) rescaled by s[n][g] into
// float accumulators.  At a channel-block boundary the wavefront's 16 x 16
// piece goes to LDS; the pieces of a block are summed in wavefront order, so
// the result never depends on timing.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int D = 4;                      // code blocks a wavefront keeps in flight
constexpr int kMaxRun = 12;               // units per wavefront
constexpr int kMaxGroups = 32;            // K / 128 (2 KiB of staged activations each)
constexpr int kMaxRounds = 8;             // workgroups per compute unit, at most

typedef unsigned int v4u __attribute__((ext_vector_type(4)));


// The leading scalars arrive preloaded in SGPRs (kernel-argument preload).
// N / 16 = cb_q * gridDim.x + cb_r: workgroup b takes cb_q blocks, one more
// when b < cb_r.  inv_g is 1 / G rounded to float.
template <bool DEBUG>
__global__ void __launch_bounds__(kThreads)
stream_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
              const uint8_t* __restrict__ zeros, const int8_t* __restrict__ qa, int K, int M,
              int cb_q, int cb_r, float inv_g, GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_act[];  // [G][2][64][16 B]
  __shared__ __attribute__((aligned(16))) float s_scale[kWaves][kMaxRun][16];
  __shared__ __attribute__((aligned(16))) uint2 s_zero[kWaves][kMaxRun];
  __shared__ __attribute__((aligned(16))) float4 part[kWaves][2][64];
  __shared__ int s_first[kWaves], s_last[kWaves];  // local blocks of each run, -1: none

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = K / kGroup;
  const int bx = blockIdx.x;
  const int cb0 = bx * cb_q + min(bx, cb_r);
  const int ncb = cb_q + (bx < cb_r ? 1 : 0);

  // The activations first: chunk t < 128 G is half (t / 64) % 2 of group
  // t / 128, lane t % 64 (row t % 16, channels 16 ((t % 64) / 16) ..).
  constexpr int kAChunks = kMaxGroups * 128 / kThreads;
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(qa, (int64_t)M * K);
  v4u ach[kAChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int t = tid + i * kThreads;
    const int r = min(t & 15, M - 1), jj = (t >> 4) & 3, h = (t >> 6) & 1, g = t >> 7;
    const int off = t < 128 * G ? r * K + g * kGroup + 64 * h + 16 * jj : kOob;
    ach[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // this wavefront's run: units [u0, u1) of the workgroup's ncb x G, channel
  // block by channel block (contiguous in the codes plane); it starts at
  // local block f.  (u0 < 2^12 and G <= 32, so the float product of u0 + 1/2
  // and 1 / G floors exactly: the quotient lies at least 1 / (2 G) from an
  // integer, far more than the rounding.)
  const int units = ncb * G;
  const int u0 = units * wave / kWaves, u1 = units * (wave + 1) / kWaves;
  const int nrun = u1 - u0;
  const int f = (int)(((float)u0 + 0.5f) * inv_g);
  const int64_t first = (int64_t)cb0 * G + u0;  // codes-plane block of run unit 0
  const int last = nrun > 0 ? nrun - 1 : 0;
  const int oob = nrun * kBlockBytes;
  const __amdgpu_buffer_rsrc_t rc = rsrc_of(codes + first * kBlockBytes, (int64_t)oob);
  // metadata: lane l holds unit l / 4's scales of channels 4 (l % 4) .. + 3
  // and unit l's zero block, clamped to the run (a wavefront with an empty
  // run reads block 0's)
  const int64_t mb = nrun > 0 ? first : 0;
  const uint4 s4 = *reinterpret_cast<const uint4*>(scales + (mb + min(lane >> 2, last)) * 16 +
                                                   4 * (lane & 3));
  const uint2 z2 = *reinterpret_cast<const uint2*>(zeros + (mb + min(lane, last)) * kZeroBlockBytes);

  // the ring: unit lu of the run
  uint4 wv[D];
  int lu = 0;
  auto load_next = [&](uint4& w) __attribute__((always_inline)) {
    const int off = lu < nrun ? lu * kBlockBytes + 16 * lane : oob;  // wave-uniform choice
    const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, kNontemporal);
    w = make_uint4(t.x, t.y, t.z, t.w);
    ++lu;
  };
#pragma unroll
  for (int i = 0; i < D; ++i) load_next(wv[i]);
  __builtin_amdgcn_sched_barrier(0);

  // staged activations, metadata tables, run bounds -> LDS; then one
  // barrier that waits for LDS writes only (the code blocks stay in flight)
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int t = tid + i * kThreads;
    if (t < 128 * G) *reinterpret_cast<v4u*>(s_act + 16 * t) = ach[i];
  }
  if ((lane >> 2) < kMaxRun) *reinterpret_cast<uint4*>(&s_scale[wave][lane >> 2][4 * (lane & 3)]) = s4;
  if (lane < kMaxRun) s_zero[wave][lane] = z2;
  if (lane == 0) {
    s_first[wave] = nrun > 0 ? f : -1;
    s_last[wave] = nrun > 0 ? (int)(((float)(u1 - 1) + 0.5f) * inv_g) : -1;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  float accf[4] = {0.f, 0.f, 0.f, 0.f};
  int slot = 0, cp = u0 - f * G;  // piece slot, group of the next unit
  const int zshift = 4 * (c & 7);
  for (int ub = 0; ub < nrun; ub += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int r = ub + i;
      if (r < nrun) {
        const float sc = s_scale[wave][r][c];
        const uint2 zb = s_zero[wave][r];
        const uint32_t zz = (((c < 8 ? zb.x : zb.y) >> zshift) & 0xFu) * 0x01010101u;
        const v4i a0 = *reinterpret_cast<const v4i*>(s_act + (2 * cp) * 1024 + 16 * lane);
        const v4i a1 = *reinterpret_cast<const v4i*>(s_act + (2 * cp + 1) * 1024 + 16 * lane);
        v4i b0, b1;
        const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          b0[t] = (int)sub_zero_bytes(d[t] & 0x0F0F0F0Fu, zz);
          b1[t] = (int)sub_zero_bytes((d[t] >> 4) & 0x0F0F0F0Fu, zz);
        }
        v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, kBiasSeed, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
        if (DEBUG && a.partials) {
          const int64_t n = (int64_t)(cb0 + f + slot) * 16 + c;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int64_t m = 4 * j + t;
            if (m < M && m >= a.m_begin && m < a.m_end)
              a.partials[((m - a.m_begin) * a.N + n) * G + cp] = acc[t] - kBiasBits;
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) accf[t] += sc * unbias(acc[t]);
        ++cp;
        const bool wrap = cp == G;
        if (wrap || r == nrun - 1) {  // the end of this channel block's piece
          part[wave][slot][lane] = make_float4(accf[0], accf[1], accf[2], accf[3]);
          accf[0] = accf[1] = accf[2] = accf[3] = 0.f;
          ++slot;
        }
        if (wrap) cp = 0;
      }
      // refill the slot with the unit D ahead: on every path, so that each
      // pass issues D loads and the waits for the ring stay exact
      load_next(wv[i]);
    }
  }
  __syncthreads();

  // the workgroup's outputs: block k, row m, channel cc of [cb0, cb0 + ncb),
  // summed over the wavefronts whose runs meet block k, in wavefront order
  for (int o = tid; o < ncb * 256; o += kThreads) {
    const int k = o >> 8, m = (o >> 4) & 15, cc = o & 15;
    if (m >= M) continue;
    const int src = 16 * (m >> 2) + cc, e = m & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int fw = s_first[w];
      if (fw >= 0 && k >= fw && k <= s_last[w]) {
        const float4 p = part[w][k - fw][src];
        v += e == 0 ? p.x : e == 1 ? p.y : e == 2 ? p.z : p.w;
      }
    }
    if (a.y) a.y[m * a.N + (int64_t)(cb0 + k) * 16 + cc] = f32_to_bf16_rne(a.sa[m] * v);
  }
}

}  // namespace

// The grid for an M x K -> N product with 1 <= M <= 16, or C == 0 where it
// does not apply: at least one channel block per compute unit (else the
// M <= 16 kernel of decode.hip, whose K slices fill the machine, serves
// better: measured at K = 3584 -> N = 3584, M = 16, 7.7 against 5.1 us), all
// of K staged (G <= kMaxGroups), and wavefront runs of at most kMaxRun units
// and at most G.
// C is a whole number R of rounds of the compute units; of R in [1,
// kMaxRounds] the one with the least work per compute unit (R times the
// largest workgroup's units, plus half a unit per group for staging the
// activations in every workgroup) wins.
StreamPlan stream_plan(int64_t M, int64_t N, int64_t K) {
  StreamPlan best{0, 0, 0};
  if (M < 1 || M > 16 || N % kBlockCols || K % kGroup) return best;
  const int64_t NB = N / kBlockCols, G = K / kGroup, cus = device_cus();
  if (G > kMaxGroups || NB < cus || NB >= (1 << 24)) return best;
  int64_t best_cost = 0;
  for (int64_t R = 1; R <= kMaxRounds; ++R) {
    const int64_t C = R * cus < NB ? R * cus : NB;
    const int64_t ncb = (NB + C - 1) / C, run = (ncb * G + kWaves - 1) / kWaves;
    if (run <= kMaxRun && run <= G) {  // (a run then meets at most two blocks)
      const int64_t cost = R * (2 * ncb * G + G);
      if (best.C == 0 || cost < best_cost) {
        best = StreamPlan{(int)C, 1, (size_t)G * 2 * 1024};
        best_cost = cost;
      }
    }
    if (C == NB) break;
  }
  return best;
}

hipError_t launch_stream(const GemmArgs& a, hipStream_t st) {
  const StreamPlan p = stream_plan(a.M, a.N, a.K);
  if (p.C == 0 || a.x || a.w8 || a.ksplit != 1) return hipErrorInvalidValue;
  const int NB = (int)(a.N / kBlockCols);
  const int cb_q = NB / p.C, cb_r = NB % p.C;
  const float inv_g = 1.0f / (float)(a.K / kGroup);
  if (a.partials)
    hipLaunchKernelGGL((stream_kernel<true>), dim3((unsigned)p.C), dim3(kThreads), p.lds, st,
                       a.w.codes, a.w.scales, a.w.zeros, a.qa, (int)a.K, (int)a.M, cb_q, cb_r,
                       inv_g, a);
  else
    hipLaunchKernelGGL((stream_kernel<false>), dim3((unsigned)p.C), dim3(kThreads), p.lds, st,
                       a.w.codes, a.w.scales, a.w.zeros, a.qa, (int)a.K, (int)a.M, cb_q, cb_r,
                       inv_g, a);
  return hipGetLastError();
}

}  // namespace w4a8
