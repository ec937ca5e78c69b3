// M == 1 decode GEMV, optionally with the per-token activation quantisation
// fused into it.
//
// "The 4-bit CPU path", section "W4A16": at decode a kernel that reads each
// weight once per call is good enough, because the call costs what streaming
// the packed weights costs; everything else must hide under that stream.  Each compute
// unit draws a fixed share of HBM bandwidth through a short queue; a
// wavefront that waits in that queue cannot take part in anything else, and a
// workgroup barrier would make every wavefront wait for the slowest one.  So
// one 1024-thread workgroup per compute unit (the grid is a whole number of
// rounds over the compute units) splits into two roles that never meet at a
// barrier before the last reduction:
//   - kQ quantiser wavefronts load the token first (their requests lead the
//     queue), take its absmax, quantise it into LDS (the rule of
//     w4a8_quant_act bit for bit, ties to even) with per-quarter code sums added by
//     integer LDS atomics (exact, so order-free), and raise an LDS flag; they
//     synchronise among themselves through LDS counters, and stream their
//     own (shorter) runs once every quantiser has raised the flag, since a
//     run reads codes and sums that all of them wrote;
//   - the other wavefronts put D code blocks of their runs in flight at once
//     (after the set-up barrier, so the token's requests go first), wait for
//     the flag, and stream.
// Both waits on the LDS counters are unbounded spins (with s_sleep): they end
// only because each of the kQ quantiser (or, for W4A16, stager) wavefronts
// increments each counter it owns exactly once, on a path with no branch
// around the increment.  Any edit that lets one of those wavefronts skip an
// increment would leave the others spinning for ever; the increments are
// marked "kQ increments" below.
// The workgroup's (16-channel block, group) units are dealt out as contiguous
// runs of the codes plane (1 KiB per wavefront per unit, nontemporal loads:
// every byte is read once), the quantisers taking a smaller share since they
// start late.  Each wavefront stages its run's scales and zero points in LDS
// with two wide loads and streams the run through a ring of D register slots:
// consume a unit, refill its slot with the unit D ahead.
// Lane l = 16j + c owns channel c and input channels
// {16j..16j+15} u {64+16j..64+16j+15} of each group: the raw codes q (0..15,
// valid signed int8) go straight into eight v_dot4_i32_i8 and the zero point
// is applied once per group as  sum qa*q - z * sum qa.  The float rescale
// s[n][g] * P is linear, so each lane rescales its quarter; quarters are
// summed with cross-lane shuffles and the pieces of a channel block (several
// wavefronts may share one) in fixed wavefront order through LDS, so the
// result never depends on timing.
// The same grid and stream serve two more weight/activation pairs:
//   - W4A16 (X_A16): the quantisers become stagers that copy the bf16 token
//     into LDS with its per-quarter float sums; lanes take bf16 pair dots;
//   - W8A8 (W8): 2 KiB units of int8 weights in operand order, raw dot4,
//     exact int32 totals and one per-channel scale in the epilogue.
#include <atomic>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kQ = 4;                       // quantiser wavefronts
constexpr int kQWeight = 2;                 // run share of a quantiser (a streamer's is 4)
constexpr int kShareTotal = kQ * kQWeight + (kWaves - kQ) * 4;
constexpr int D = 4;                        // code blocks a wavefront keeps in flight
constexpr int kDeepD = 6;                   // ... over a long token (see launch_ks)
constexpr int kMaxRun = 12;                 // units per wavefront
constexpr int kMaxCb = 12;                  // channel blocks per workgroup

// X_A16: W4A16, the bf16 token is used as it is (no quantisation)
enum { X_BF16 = 0, X_F32 = 1, X_QUANTISED = 2, X_A16 = 3 };

// Start of wavefront w's run in share units.
__host__ __device__ constexpr int share_prefix(int w) {
  return w <= kQ ? w * kQWeight : kQ * kQWeight + (w - kQ) * 4;
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntload16(const uint8_t* p) {
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ float wave_max(float v) { return wave_max64(v); }

// Sum of the 8 signed bytes in a uint2.
__device__ __forceinline__ int byte_sum8(uint2 v) {
  return __builtin_amdgcn_sdot4((int)v.y, 0x01010101,
                                __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false), false);
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
// a.lo * b.lo + a.hi * b.hi + c over two bf16 pairs, in float
__device__ __forceinline__ float bf16_dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c,
                                         false);
}

// Codes-plane block index of unit u of a workgroup's run.
// floor(total * i / parts) in 32-bit arithmetic (parts <= 65536, checked on
// the host): total = q parts + r, so total i / parts = q i + r i / parts.
__device__ __forceinline__ int split_point(unsigned total, unsigned parts, unsigned i) {
  const unsigned q = total / parts, r = total % parts;
  return (int)(q * i + (r * i) / parts);
}

template <bool KSPLIT>
__device__ __forceinline__ int64_t unit_block(int u, int nb0, int G, int g0, int gk) {
  if constexpr (!KSPLIT) return (int64_t)nb0 * G + u;  // whole blocks: the run is contiguous
  return (int64_t)(nb0 + u / gk) * G + g0 + u % gk;
}

// Load the next unit of the run into a ring slot.  The wavefront reads its
// run through a buffer descriptor that spans exactly the run's blocks; past
// the end of the run the load still issues (so every wavefront has the same,
// compile-time count of loads in flight and waits stay exact) but with an
// offset beyond the descriptor's range, which the hardware answers with zeros
// and no memory request.  Branch-free on purpose.
// A unit is H KiB: H = 1 for the int4 codes, 2 for the W8A8 weights (two
// 1 KiB halves, input channels 0-63 and 64-127 of the group).
template <int H>
__device__ __forceinline__ void load_next(__amdgpu_buffer_rsrc_t rsrc, int oob, int u1, int G,
                                          int gk, int lane, int& lu, int& lg, int& rel,
                                          uint4 (&w)[H]) {
  const int live = lu < u1 ? 1 : 0;  // wave-uniform
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int off = live ? (rel * H + h) * kBlockBytes + 16 * lane : oob;
    const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kNontemporal);
    w[h] = make_uint4(t.x, t.y, t.z, t.w);
  }
  lu += live;
  lg += live;
  const int wrap = (lg == gk) ? 1 : 0;
  lg -= wrap * gk;
  rel += live + wrap * (G - gk);  // next group, or the next block's first group
}

// One 8-element chunk of the token (chunk ch), raw: bf16 -> one uint4, f32 ->
// two, pre-quantised codes -> one uint2 (in .x, .y).
template <int XT>
__device__ __forceinline__ void load_chunk(const void* x, int ch, uint4* r) {
  if constexpr (XT == X_BF16 || XT == X_A16) {
    r[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + 8 * ch);
  } else if constexpr (XT == X_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + 8 * ch);
    r[0] = p[0];
    r[1] = p[1];
  } else {
    const uint2 c2 = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(x) + 8 * ch);
    r[0] = make_uint4(c2.x, c2.y, 0u, 0u);
  }
}

template <int XT>
__device__ __forceinline__ float chunk_value(const uint4* r, int e) {
  if constexpr (XT == X_BF16 || XT == X_A16) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
  } else {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
    return __uint_as_float(w[e]);
  }
}

// The flag: every wavefront of the workgroup (streamers, and quantisers or
// stagers once their own share is written) waits until all kQ quantisers or
// stagers have made their one increment of s_sync[2], which releases their
// LDS writes (codes, code sums, staged token).  An unbounded spin with
// s_sleep: it ends because each of the kQ wavefronts reaches its increment
// exactly once, on a path with no branch around it and no wait before it
// other than the quantisers' row-maximum wait, which ends the same way.
__device__ __forceinline__ void wait_flag(uint32_t* s_sync) {
  while (__hip_atomic_load(&s_sync[2], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
         (unsigned)kQ)
    __builtin_amdgcn_s_sleep(1);
}

// kQChunks: token chunks (8 elements) a quantiser thread holds at once; the
// whole token fits in one batch when K / 8 <= 256 * kQChunks.
// The operands the first loads need lead the argument list as scalars, so
// that they arrive preloaded in scalar registers (kernel-argument preload)
// instead of behind a memory round trip; the rest stays in GemmArgs.
// xin: the token (bf16 / f32) or, pre-quantised, its codes.
// W8: the W8A8 weights (two 1 KiB halves per unit, already in operand order;
// one scale per channel in `scales`, no zero points): raw int8 dots, int32
// totals over the run, the scales applied once in the epilogue.
// EARLY: the streamers' first code blocks go out beside the token's
// requests instead of after the set-up barrier (chosen on the host).
template <int XT, bool DEBUG, bool KSPLIT, int kQChunks, bool W8 = false, bool HAD = false,
          bool EARLY = false, int DR = D>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
            const uint8_t* __restrict__ zeros, const void* __restrict__ xin, int K, int cb_q,
            int cb_r, GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ __attribute__((aligned(16))) float s_scale[kWaves][kMaxRun][16];
  __shared__ __attribute__((aligned(16))) uint2 s_zero[kWaves][kMaxRun];
  __shared__ float part[kMaxCb][kWaves][16];
  // [0] token absmax bits, [1] quantisers past the absmax, [2] quantisers done
  __shared__ unsigned s_sync[4];
  const int G = K / kGroup, NB = (int)(a.N / kBlockCols);
  int8_t* qs = reinterpret_cast<int8_t*>(smem);               // [K] activation codes
  int* rs = reinterpret_cast<int*>(smem + K);                  // [4G] per-quarter code sums
  // W4A16 instead: the bf16 token [K] and its per-quarter float sums [4G]
  constexpr bool A16 = XT == X_A16;
  float* xsum = reinterpret_cast<float*>(smem + 2 * K);
  constexpr int H = W8 ? 2 : 1;  // KiB per unit
  int (*part_i)[kWaves][16] = reinterpret_cast<int (*)[kWaves][16]>(part);  // W8: int32 pieces

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int c = lane & 15, j = lane >> 4;
  // The quantisers' (stagers') token requests go out first of all, before
  // the run set-up below: that set-up is scalar work which the kernel's 16
  // wavefronts issue in turn, and the token is on every wavefront's
  // critical path.
  const int nch = K / 8;
  constexpr int RW = XT == X_F32 ? 2 : 1;
  constexpr int kQThreads = 64 * kQ;
  uint4 xr[kQChunks][RW];
  if (wave < kQ) {
#pragma unroll
    for (int i = 0; i < kQChunks; ++i) load_chunk<XT>(xin, min(i * kQThreads + tid, nch - 1), xr[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // This workgroup: channel blocks [nb0, nb1) x groups [g0, g0 + gk).  The
  // host passes NB = cb_q * gridDim.x + cb_r, so no division is needed here;
  // everything up to the first loads is kept short, because those loads
  // start the memory pipe.
  const int bx = blockIdx.x;
  const int nb0 = bx * cb_q + min(bx, cb_r);
  const int nb1 = nb0 + cb_q + (bx < cb_r ? 1 : 0);
  int g0 = 0, gk = G;
  if constexpr (KSPLIT) {
    g0 = split_point(G, gridDim.y, blockIdx.y);
    gk = split_point(G, gridDim.y, blockIdx.y + 1) - g0;
  }
  const int units = (nb1 - nb0) * gk;
  const int u0 = units * share_prefix(wave) / kShareTotal;
  const int u1 = units * share_prefix(wave + 1) / kShareTotal;
  const int nrun = u1 - u0;

  // the run's metadata: scales (lane l: unit l/4, channels 4(l%4)..+3) and
  // zero blocks (lane l: unit l), clamped to the run's last unit
  const int last = nrun > 0 ? nrun - 1 : 0;
  const int64_t bs = unit_block<KSPLIT>(u0 + min(lane >> 2, last), nb0, G, g0, gk);
  const int64_t bz = unit_block<KSPLIT>(u0 + min(lane & 15, last), nb0, G, g0, gk);
  const float* hot_s = scales + bs * 16 + 4 * (lane & 3);
  // the run's blocks: [first, first + span) of the codes plane
  const int64_t first = unit_block<KSPLIT>(u0, nb0, G, g0, gk);
  const int span = nrun > 0 ? (int)(unit_block<KSPLIT>(u1 - 1, nb0, G, g0, gk) - first + 1) : 0;
  const int oob = span * H * kBlockBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + (nrun > 0 ? first : 0) * H * kBlockBytes), (short)0, oob,
      kBufferWord3);
  uint4 wv[DR][H];
  int lu = u0, lg = 0, rel = 0;  // next unit to load (lg: its group within the slice)
  if constexpr (KSPLIT) lg = nrun > 0 ? u0 % gk : 0;
  uint4 s4;
  uint2 z2;
  float scale;
  // then every wavefront's run metadata (two small loads) and, EARLY, the
  // streamers' first code blocks
  if constexpr (!W8) {  // (W8: one scale per channel, read in the epilogue)
    s4 = *reinterpret_cast<const uint4*>(hot_s);
    z2 = *reinterpret_cast<const uint2*>(zeros + bz * kZeroBlockBytes);
  }
  if constexpr (EARLY) {
    if (wave >= kQ) {
#pragma unroll
      for (int i = 0; i < DR; ++i) load_next<H>(rsrc, oob, u1, G, gk, lane, lu, lg, rel, wv[i]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads above issue before the set-up below

  for (int t = tid; t < kMaxCb * kWaves * 16; t += kThreads) (&part[0][0][0])[t] = 0.0f;
  if constexpr (!A16 && !W8)
    for (int t = tid; t < 4 * G; t += kThreads) rs[t] = 0;
  if (tid < 4) s_sync[tid] = 0u;
  __syncthreads();
  // otherwise the streamers' first DR code blocks only now, so that every
  // quantiser's token requests are ahead of them in this compute unit's
  // memory queue (the token is on every wavefront's critical path)
  if (!EARLY && wave >= kQ) {
#pragma unroll
    for (int i = 0; i < DR; ++i) load_next<H>(rsrc, oob, u1, G, gk, lane, lu, lg, rel, wv[i]);
  }

  if (wave < kQ && A16) {
    // ---- W4A16 stager: the token chunks go to LDS as they are, with the
    // float sum of each lane quarter (chunks 2j, 2j+1, 8+2j, 9+2j of a
    // group: the 32 inputs a streamer lane multiplies) taken in a fixed
    // order across the four lanes that hold them
    const int nbatch = (nch + kQChunks * kQThreads - 1) / (kQChunks * kQThreads);
    for (int b = 0; b < nbatch; ++b) {
      if (b > 0) {
#pragma unroll
        for (int i = 0; i < kQChunks; ++i)
          load_chunk<XT>(xin, min((b * kQChunks + i) * kQThreads + tid, nch - 1), xr[i]);
      }
#pragma unroll
      for (int i = 0; i < kQChunks; ++i) {
        const int ch = (b * kQChunks + i) * kQThreads + tid;  // ch % 16 == lane % 16
        const bool live = ch < nch;  // the same for the 16 lanes of a row (nch % 16 == 0)
        float v = 0.0f;
        if (live) {
          *reinterpret_cast<uint4*>(smem + 16 * ch) = xr[i][0];
#pragma unroll
          for (int e = 0; e < 8; ++e) v += chunk_value<XT>(xr[i], e);
        }
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 8);
        if (live && (lane & 9) == 0) xsum[4 * (ch >> 4) + ((ch & 7) >> 1)] = v;
      }
    }
    scale = 1.0f;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wavefront's LDS writes done (lgkmcnt(0))
    // kQ increments: every stager reaches this line exactly once; the
    // unbounded waits for s_sync[2] == kQ (wait_flag) depend on it
    if (lane == 0)
      __hip_atomic_fetch_add(&s_sync[2], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int i = 0; i < DR; ++i)
      load_next<H>(rsrc, oob, u1, G, gk, lane, lu, lg, rel, wv[i]);
    // this stager's run reads the token and sums the others staged: the
    // streamers' wait (below), which ends after the kQ increments
    wait_flag(s_sync);
  } else if (wave < kQ) {
    // ---- quantiser: token chunks (8 elements) qt, qt + 256, ... in batches
    // of kQChunks (the first batch is in flight already); the last batch
    // stays in registers for the second pass
    const int qt = tid;                                         // 0 .. 64 kQ - 1
    const int nbatch = (nch + kQChunks * kQThreads - 1) / (kQChunks * kQThreads);
    float amax = 0.0f;
    for (int b = 0; b < nbatch; ++b) {
      if (b > 0) {
#pragma unroll
        for (int i = 0; i < kQChunks; ++i)
          load_chunk<XT>(xin, min((b * kQChunks + i) * kQThreads + qt, nch - 1), xr[i]);
      }
      if constexpr (XT != X_QUANTISED) {
#pragma unroll
        for (int i = 0; i < kQChunks; ++i) {
          // (liveness is the same for the 16 lanes of a row: nch % 16 == 0)
          const bool live = (b * kQChunks + i) * kQThreads + qt < nch;
          if constexpr (HAD) {  // the rotated values set the scale
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = chunk_value<XT>(xr[i], e);
            hadamard_chunk(v);
            if (live)
#pragma unroll
              for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
          } else if (live) {
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(chunk_value<XT>(xr[i], e)));
          }
        }
      }
    }
    if constexpr (XT == X_QUANTISED) {
      scale = a.sa[0];
    } else {
      // row absmax: every quantiser publishes its wavefront max (non-negative
      // floats order as their bit patterns), then waits for the others
      amax = wave_max(amax);
      // kQ increments: every quantiser reaches this line exactly once; the
      // unbounded wait just below (all quantisers) depends on it
      if (lane == 0) {
        __hip_atomic_fetch_max(&s_sync[0], __float_as_uint(amax), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&s_sync[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      while (__hip_atomic_load(&s_sync[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
             (unsigned)kQ)
        __builtin_amdgcn_s_sleep(1);
      scale = __uint_as_float(
          __hip_atomic_load(&s_sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) / 127.0f;
    }
    const float inv = scale != 0.0f ? 1.0f / scale : 0.0f;  // correctly rounded
    for (int b = nbatch - 1; b >= 0; --b) {
      if (b != nbatch - 1) {
#pragma unroll
        for (int i = 0; i < kQChunks; ++i)
          load_chunk<XT>(xin, min((b * kQChunks + i) * kQThreads + qt, nch - 1), xr[i]);
      }
#pragma unroll
      for (int i = 0; i < kQChunks; ++i) {
        const int ch = (b * kQChunks + i) * kQThreads + qt;
        float v[8];
        if constexpr (XT != X_QUANTISED) {
          // (rotated, when asked, outside the branch: the rotation exchanges
          // values across the 16 lanes of a row)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = chunk_value<XT>(xr[i], e);
          if constexpr (HAD) hadamard_chunk(v);
        }
        if (ch < nch) {
          uint2 pk;
          if constexpr (XT == X_QUANTISED) {
            pk = make_uint2(xr[i][0].x, xr[i][0].y);
          } else {
            // the rule of w4a8_quant_act (or w4a8_quant_act_hadamard), bit
            // for bit (quant8_codes); an all-zero token has scale 0 and
            // all-zero codes
            pk = scale != 0.0f ? quant8_codes(v, scale, inv) : make_uint2(0u, 0u);
          }
          *reinterpret_cast<uint2*>(qs + 8 * ch) = pk;
          // chunk ch covers elements 8(ch%16)..+7 of group ch/16: quarter
          // ((ch % 16) % 8) / 2 of the lane layout (0..63 and 64..127 fold)
          if constexpr (!W8) atomicAdd(&rs[4 * (ch >> 4) + ((ch & 7) >> 1)], byte_sum8(pk));
        }
      }
    }
    if (a.sa_ws && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.sa_ws[0] = scale;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wavefront's LDS writes done (lgkmcnt(0))
    // kQ increments: every quantiser reaches this line exactly once; the
    // unbounded waits for s_sync[2] == kQ (wait_flag) depend on it
    if (lane == 0)
      __hip_atomic_fetch_add(&s_sync[2], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    // then the quantiser streams its own (shorter) run, which reads codes
    // and sums the other quantisers wrote: it waits for them as the
    // streamers do (below), once its loads are in flight
#pragma unroll
    for (int i = 0; i < DR; ++i)
      load_next<H>(rsrc, oob, u1, G, gk, lane, lu, lg, rel, wv[i]);
    wait_flag(s_sync);
  } else {
    // ---- streamer: metadata and DR code blocks are in flight; the flag
    // (an unbounded spin that ends once all kQ quantisers or stagers have
    // made their one increment of s_sync[2])
    if constexpr (XT == X_QUANTISED) scale = a.sa[0];
    wait_flag(s_sync);
    if constexpr (A16)
      scale = 1.0f;
    else if constexpr (XT != X_QUANTISED)
      scale = __uint_as_float(
          __hip_atomic_load(&s_sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) / 127.0f;
  }
  if constexpr (!W8) {
    if ((lane >> 2) < kMaxRun) *reinterpret_cast<uint4*>(&s_scale[wave][lane >> 2][4 * (lane & 3)]) = s4;
    if (lane < kMaxRun) s_zero[wave][lane] = z2;
  }

  // the run, through the ring
  {
    float accf = 0.0f;
    int acci = 0;  // W8: int32 total of the current channel block
    int ccb = nrun > 0 ? u0 / gk : 0, cg = nrun > 0 ? u0 % gk : 0;  // compute position
    int cur = ccb;
    const int zshift = (c & 1) * 4;
    for (int ub = 0; ub < nrun; ub += DR) {
#pragma unroll
      for (int i = 0; i < DR; ++i) {
        const int r = ub + i;  // position in the run
        if (r < nrun) {
          if (ccb != cur) {
            if constexpr (W8) {
              acci += __shfl_xor(acci, 16);
              acci += __shfl_xor(acci, 32);
              if (j == 0) part_i[cur][wave][c] = acci;
              acci = 0;
            } else {
              accf += __shfl_xor(accf, 16);
              accf += __shfl_xor(accf, 32);
              if (j == 0) part[cur][wave][c] = accf;
              accf = 0.0f;
            }
            cur = ccb;
          }
          const int g = g0 + cg;
          if constexpr (A16) {
            // sum x (128 + q) over the lane's 32 inputs with bf16 pair dots:
            // a code q (0..15) below the bf16 of 128 (0x4300) is exactly
            // 128 + q; then minus (128 + z) times the quarter's sum of x
            const uint8_t* xb = smem + 2 * (kGroup * g + 16 * j);
            const uint4 xl0 = *reinterpret_cast<const uint4*>(xb);
            const uint4 xl1 = *reinterpret_cast<const uint4*>(xb + 16);
            const uint4 xh0 = *reinterpret_cast<const uint4*>(xb + 128);
            const uint4 xh1 = *reinterpret_cast<const uint4*>(xb + 144);
            const uint32_t xl[8] = {xl0.x, xl0.y, xl0.z, xl0.w, xl1.x, xl1.y, xl1.z, xl1.w};
            const uint32_t xh[8] = {xh0.x, xh0.y, xh0.z, xh0.w, xh1.x, xh1.y, xh1.z, xh1.w};
            const uint32_t d[4] = {wv[i][0].x, wv[i][0].y, wv[i][0].z, wv[i][0].w};
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              // code bytes 4w, 4w+1 (and 4w+2, 4w+3) into the low bytes of two halves
              const uint32_t t01 = __builtin_amdgcn_perm(d[w], d[w], 0x0C010C00u);
              const uint32_t t23 = __builtin_amdgcn_perm(d[w], d[w], 0x0C030C02u);
              acc = bf16_dot2(xl[2 * w], (t01 & 0x000F000Fu) | 0x43004300u, acc);
              acc = bf16_dot2(xl[2 * w + 1], (t23 & 0x000F000Fu) | 0x43004300u, acc);
              acc = bf16_dot2(xh[2 * w], ((t01 >> 4) & 0x000F000Fu) | 0x43004300u, acc);
              acc = bf16_dot2(xh[2 * w + 1], ((t23 >> 4) & 0x000F000Fu) | 0x43004300u, acc);
            }
            const uint32_t zbyte = reinterpret_cast<const uint8_t*>(&s_zero[wave][r])[c >> 1];
            const float zf = (float)(int)(((zbyte >> zshift) & 0xFu) + 128u);
            accf += s_scale[wave][r][c] * fmaf(-zf, xsum[4 * g + j], acc);
          } else if constexpr (W8) {
            // the two halves' int8 weights against the codes of the same
            // input channels: no unpacking, no zero point, no per-group scale
            const uint4 al = *reinterpret_cast<const uint4*>(qs + kGroup * g + 16 * j);
            const uint4 ah = *reinterpret_cast<const uint4*>(qs + kGroup * g + 64 + 16 * j);
            const uint32_t w0[4] = {wv[i][0].x, wv[i][0].y, wv[i][0].z, wv[i][0].w};
            const uint32_t w1[4] = {wv[i][1].x, wv[i][1].y, wv[i][1].z, wv[i][1].w};
            const uint32_t l4[4] = {al.x, al.y, al.z, al.w};
            const uint32_t h4[4] = {ah.x, ah.y, ah.z, ah.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              acci = __builtin_amdgcn_sdot4((int)w0[w], (int)l4[w], acci, false);
              acci = __builtin_amdgcn_sdot4((int)w1[w], (int)h4[w], acci, false);
            }
          } else {
          const uint4 al = *reinterpret_cast<const uint4*>(qs + kGroup * g + 16 * j);
          const uint4 ah = *reinterpret_cast<const uint4*>(qs + kGroup * g + 64 + 16 * j);
          const uint32_t d[4] = {wv[i][0].x, wv[i][0].y, wv[i][0].z, wv[i][0].w};
          const uint32_t l4[4] = {al.x, al.y, al.z, al.w};
          const uint32_t h4[4] = {ah.x, ah.y, ah.z, ah.w};
          int acc = kBiasBits;  // read back as a float by unbias below
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc = __builtin_amdgcn_sdot4((int)(d[w] & 0x0F0F0F0Fu), (int)l4[w], acc, false);
            acc = __builtin_amdgcn_sdot4((int)((d[w] >> 4) & 0x0F0F0F0Fu), (int)h4[w], acc,
                                         false);
          }
          const uint32_t zbyte = reinterpret_cast<const uint8_t*>(&s_zero[wave][r])[c >> 1];
          const int z = (int)((zbyte >> zshift) & 0xFu);
          const int pb = acc - z * rs[4 * g + j];  // kBiasBits + the quarter's product
          if (DEBUG) {
            const int p = pb - kBiasBits;
            int pg = p + __shfl_xor(p, 16);
            pg += __shfl_xor(pg, 32);
            if (j == 0 && a.partials && a.m_begin == 0 && a.m_end > 0)
              a.partials[((int64_t)16 * (nb0 + ccb) + c) * G + g] = pg;
          }
          accf += s_scale[wave][r][c] * unbias(pb);
          }
          ++cg;
          const int wrap = (cg == gk) ? 1 : 0;
          cg -= wrap * gk;
          ccb += wrap;
        }
        // refill this slot with the unit DR ahead
        load_next<H>(rsrc, oob, u1, G, gk, lane, lu, lg, rel, wv[i]);
      }
    }
    if constexpr (W8) {
      acci += __shfl_xor(acci, 16);
      acci += __shfl_xor(acci, 32);
      if (nrun > 0 && j == 0) part_i[cur][wave][c] = acci;
    } else {
      accf += __shfl_xor(accf, 16);
      accf += __shfl_xor(accf, 32);
      if (nrun > 0 && j == 0) part[cur][wave][c] = accf;
    }
  }
  __syncthreads();

  // each channel block: its wavefront pieces in wavefront order
  const int ncb = nb1 - nb0;
  for (int t = tid; t < ncb * 16; t += kThreads) {
    const int cbl = t >> 4, cc = t & 15;
    if constexpr (W8) {
      // exact int32 total (order-free), then y = sa * (sw * P) as on every
      // W8A8 path; split K: the slice's total to the int32 workspace
      int total = part_i[cbl][0][cc];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) total += part_i[cbl][w][cc];
      const int64_t n = (int64_t)16 * (nb0 + cbl) + cc;
      if (gridDim.y == 1) {
        if (DEBUG && a.partials && a.m_begin == 0 && a.m_end > 0) a.partials[n] = total;
        if (a.y) a.y[n] = f32_to_bf16_rne(scale * (scales[n] * (float)total));
      } else {
        reinterpret_cast<int32_t*>(a.workspace)[(int64_t)blockIdx.y * a.N + n] = total;
      }
      continue;
    }
    float total = part[cbl][0][cc];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) total += part[cbl][w][cc];
    const int64_t n = (int64_t)16 * (nb0 + cbl) + cc;
    if (gridDim.y == 1) {
      if (a.y) a.y[n] = f32_to_bf16_rne(scale * total);
    } else {
      a.workspace[(int64_t)blockIdx.y * a.N + n] = total;
    }
  }
}

template <int XT, bool KSPLIT, int QC, bool W8>
hipError_t launch_ks(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  dim3 grid((unsigned)a.cb, (unsigned)a.ksplit);
  const size_t lds = (XT == X_A16 ? 2 : 1) * (size_t)a.K + 16 * (size_t)G;
  const void* xin = XT == X_QUANTISED ? static_cast<const void*>(a.qa) : a.x;
  if constexpr ((XT == X_BF16 || XT == X_F32) && !W8) {
    // the rotated token (w4a8_linear_hadamard): its own instantiation, so the
    // plain kernel carries none of the rotation's code
    if (a.hadamard) {
      if (a.partials) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemv_kernel<XT, false, KSPLIT, QC, false, true>), grid, dim3(kThreads), lds,
                         st, a.w.codes, a.w.scales, a.w.zeros, xin, (int)a.K, a.cb_q, a.cb_r, a);
      return hipGetLastError();
    }
  }
  if (a.hadamard) return hipErrorInvalidValue;
  if (a.partials) {
    hipLaunchKernelGGL((gemv_kernel<XT, true, KSPLIT, QC, W8>), grid, dim3(kThreads), lds, st, a.w.codes,
                       a.w.scales, a.w.zeros, xin, (int)a.K, a.cb_q, a.cb_r, a);
    return hipGetLastError();
  }
  if constexpr (!KSPLIT && (XT == X_BF16 || XT == X_F32) && !W8 && QC >= 4) {
    // A long token (at least 16384 inputs) keeps the streamers waiting for
    // the flag longest: a deeper ring puts more of their runs in flight
    // meanwhile (MI355X, K = 18944 -> N = 3584: 9.06 against 9.49 us).  On
    // shorter tokens the extra requests only queue ahead of the token's
    // (K = 3584 -> N = 18944: 8.62 against 7.94 us).
    if (a.K >= 16384) {
      hipLaunchKernelGGL((gemv_kernel<XT, false, false, QC, false, false, false, kDeepD>), grid,
                         dim3(kThreads), lds, st, a.w.codes, a.w.scales, a.w.zeros, xin, (int)a.K,
                         a.cb_q, a.cb_r, a);
      return hipGetLastError();
    }
  }
  if constexpr (!KSPLIT) {
    // One round of workgroups with long runs over a short token: the token's
    // round trip does not shorten when its requests go first, and the weight
    // stream then starts later (MI355X, K = 3584 -> N = 18944: 8.06 us early
    // against 8.31).  Elsewhere the token goes first (K = 18944 -> N = 3584:
    // 10.1 against 10.9 us; K = 3584 -> N = 3584 5.1 against 5.5 us;
    // N = 152064, eight rounds: 45.4 against 48.3 us).
    const int64_t NB = a.N / kBlockCols;
    const int64_t units = (NB + a.cb - 1) / a.cb * G;
    if ((int64_t)a.cb <= device_cus() && a.K <= 8192 && units >= 64) {
      hipLaunchKernelGGL((gemv_kernel<XT, false, false, QC, W8, false, true>), grid, dim3(kThreads),
                         lds, st, a.w.codes, a.w.scales, a.w.zeros, xin, (int)a.K, a.cb_q, a.cb_r, a);
      return hipGetLastError();
    }
  }
    hipLaunchKernelGGL((gemv_kernel<XT, false, KSPLIT, QC, W8>), grid, dim3(kThreads), lds, st,
                       a.w.codes, a.w.scales, a.w.zeros, xin, (int)a.K, a.cb_q, a.cb_r, a);
  return hipGetLastError();
}

// Token chunks per quantiser thread: as few as hold the token in one batch
// (fewer, shorter loads on the critical path); past 20480 inputs (float
// tokens: past 8192) the token is quantised in batches of 4 chunks.
template <int XT, bool KSPLIT, bool W8>
hipError_t launch_qc(const GemmArgs& a, hipStream_t st) {
  const int64_t nch = a.K / 8, per = 64 * kQ;
  if (nch <= 2 * per) return launch_ks<XT, KSPLIT, 2, W8>(a, st);
  if (nch <= 4 * per || XT == X_F32) return launch_ks<XT, KSPLIT, 4, W8>(a, st);
  if (nch <= 10 * per) return launch_ks<XT, KSPLIT, 10, W8>(a, st);
  return launch_ks<XT, KSPLIT, 4, W8>(a, st);
}

template <int XT, bool W8 = false>
hipError_t launch_xt(GemmArgs a, hipStream_t st) {
  const int NB = (int)(a.N / kBlockCols);
  a.cb_q = NB / a.cb;  // workgroup b holds cb_q blocks, plus one if b < cb_r
  a.cb_r = NB % a.cb;
  return a.ksplit > 1 ? launch_qc<XT, true, W8>(a, st) : launch_qc<XT, false, W8>(a, st);
}

}  // namespace

// Compute units of the current device (cached per device; 256 when the
// runtime cannot say, e.g. on a host without a GPU).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
    (void)hipGetLastError();
    v = 256;
  }
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Grid for an N x K weight.  One 1024-thread workgroup fills a compute unit,
// so the grid is a whole number of rounds of the compute units (no tail of
// late workgroups) with about 128 (block, group) units per workgroup.  K is
// split across workgroups (into >= 16-group slices) when one block's groups
// exceed what the streamers of a workgroup hold, or when the channel blocks
// fill less than half the compute units.  `cb` carries the number of
// workgroups along N.
GemvShape gemv_shape(int64_t N, int64_t K) {
  const int64_t NB = N / kBlockCols, G = K / kGroup;
  const int64_t cus = device_cus();
  // a streamer's run is at most ceil(units * 4 / kShareTotal) units
  const int64_t max_units = (int64_t)kMaxRun * kShareTotal / 4;
  GemvShape s{1, kWaves, 1};
  while ((G + s.ksplit - 1) / s.ksplit > max_units) s.ksplit *= 2;
  const int64_t gk = (G + s.ksplit - 1) / s.ksplit;
  if (NB >= cus) {
    int64_t rounds = NB * G / (128 * cus);
    if (rounds < 1) rounds = 1;
    int64_t w = rounds * cus;
    if (w > NB) w = NB;
    while (w < NB && ((NB + w - 1) / w > kMaxCb || (NB + w - 1) / w * gk > max_units)) w += cus;
    if (w > NB) w = NB;
    s.cb = (int)w;
  } else {
    // fewer channel blocks than compute units: split K while the doubled grid
    // still fits in one round (a second round would cost more than it saves)
    s.cb = (int)NB;
    while ((int64_t)s.cb * s.ksplit * 2 <= cus && G / (s.ksplit * 2) >= 16) s.ksplit *= 2;
  }
  return s;
}

// What the kernel's fixed LDS tables hold: <= kMaxCb channel blocks per
// workgroup and <= kMaxRun units per streamer wavefront.
bool gemv_shape_ok(int64_t N, int64_t K, const GemvShape& s) {
  const int64_t NB = N / kBlockCols, G = K / kGroup;
  if (s.cb < 1 || s.cb > 65536 || s.ksplit < 1 || s.ksplit > G || s.ksplit > 65536) return false;
  const int64_t ncb = (NB + s.cb - 1) / s.cb;
  const int64_t gk_max = (G + s.ksplit - 1) / s.ksplit;
  const int64_t run = (ncb * gk_max * 4 + kShareTotal - 1) / kShareTotal;
  return ncb <= kMaxCb && run <= kMaxRun;
}

hipError_t launch_gemv_a16(const GemmArgs& a, hipStream_t st) { return launch_xt<X_A16>(a, st); }

hipError_t launch_gemv(const GemmArgs& a, hipStream_t st) {
  if (a.w8) {  // W8A8 weights (a.w.scales: one per channel)
    if (!a.x) return launch_xt<X_QUANTISED, true>(a, st);
    if (a.x_dtype == 0) return launch_xt<X_BF16, true>(a, st);
    return launch_xt<X_F32, true>(a, st);
  }
  if (!a.x) return launch_xt<X_QUANTISED>(a, st);
  if (a.x_dtype == 0) return launch_xt<X_BF16>(a, st);
  return launch_xt<X_F32>(a, st);
}

}  // namespace w4a8
