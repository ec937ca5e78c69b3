// M == 1 decode GEMV, optionally with the per-token activation quantisation
// fused into it.
//
// "The 4-bit CPU path", section "W4A16": a kernel that touches every weight
// once per call is "fine for decode" — its cost is the stream of packed
// weights, and everything else must hide under that stream.  One 1024-thread
// workgroup per compute unit (the grid is a whole number of rounds over the
// compute units), with two roles:
//   - 12 streamer wavefronts each own an equal contiguous run of the
//     workgroup's (16-channel block, group) units, i.e. one contiguous run of
//     the codes plane.  At entry each stages its run's scales and zero points
//     in LDS with two wide loads and puts its first D code blocks in flight
//     (1 KiB per wavefront per unit, nontemporal: every byte is read once);
//   - 4 quantiser wavefronts meanwhile turn the token into int8 codes in LDS.
//     Each reads the whole row to form the absmax itself (so they need no
//     synchronisation among themselves), then quantises every fourth group
//     (IEEE division, ties to even — the rule of w4a8_quant_act) and forms the
//     per-quarter code sums of those groups.  Given pre-quantised codes they
//     only copy them.
// One workgroup barrier joins the two, then the streamers run a ring of D
// register slots: consume a unit, refill its slot with the unit D ahead.
// Lane l = 16j + c owns channel c and input channels
// {16j..16j+15} u {64+16j..64+16j+15} of each group: the raw codes q (0..15,
// valid signed int8) go straight into eight v_dot4_i32_i8 and the zero point
// is applied once per group as  sum qa*q - z * sum qa.  The float rescale
// s[n][g] * P is linear, so each lane rescales its quarter; quarters are summed
// with cross-lane shuffles and the pieces of a channel block (several
// wavefronts may share one) in fixed wavefront order through LDS, so the
// result never depends on timing.
#include <atomic>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kQWaves = 4;                  // quantiser wavefronts
constexpr int kSWaves = kWaves - kQWaves;   // streamer wavefronts
constexpr int kMaxRun = 16;                 // units per streamer wavefront
constexpr int D = 4;                        // code blocks a streamer keeps in flight
constexpr int kSmallK = 4096;               // rows a quantiser wavefront holds in registers
constexpr int kMaxCb = 16;                  // channel blocks per workgroup

enum { X_BF16 = 0, X_F32 = 1, X_QUANTISED = 2 };

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntload16(const uint8_t* p) {
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Eight activations (chunk ch) widened to float.
template <int XT>
__device__ __forceinline__ void load8(const void* x, int ch, float* v) {
  if constexpr (XT == X_BF16) {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + 8 * ch);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float* p = static_cast<const float*>(x) + 8 * ch;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Sum of the 16 signed bytes in a uint4.
__device__ __forceinline__ int byte_sum16(uint4 v) {
  int s = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false);
  s = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, s, false);
  return __builtin_amdgcn_sdot4((int)v.w, 0x01010101, s, false);
}

// Codes-plane block index of unit u of a workgroup's run.
__device__ __forceinline__ int64_t unit_block(int u, int nb0, int G, int g0, int gk) {
  return (int64_t)(nb0 + u / gk) * G + g0 + u % gk;
}

// Step the load position (unit lu at block lcb, group lg of the slice).
__device__ __forceinline__ void advance(int& lu, int& lcb, int& lg, int gk) {
  ++lu;
  ++lg;
  const int wrap = (lg == gk) ? 1 : 0;  // a select, not a branch
  lg -= wrap * gk;
  lcb += wrap;
}

// The first loads of a quantiser wavefront, issued before the streamers put
// their code blocks in flight: the first 8 activation chunks of this lane
// (bf16: chunk lane + 64 i) or, for pre-quantised codes, the codes of its
// first group.
struct QPrefetch {
  uint4 v[8];
};

template <int XT>
__device__ __forceinline__ void quantise_prefetch(const GemmArgs& a, int qw, int lane, int K,
                                                  QPrefetch& pf) {
  if constexpr (XT == X_BF16) {
    const int nch = K / 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pf.v[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) +
                                                8 * min(64 * i + lane, nch - 1));
  } else if constexpr (XT == X_QUANTISED) {
    const int g = min(qw + 4 * (lane >> 4), K / kGroup - 1);
    const uint2 c2 = *reinterpret_cast<const uint2*>(a.qa + 8 * (g * 16 + (lane & 15)));
    pf.v[0] = make_uint4(c2.x, c2.y, 0u, 0u);
  }
}

// Quantiser wavefront qw: the token's codes for groups qw, qw+4, ... into qs,
// with their per-quarter sums into rs.
template <int XT>
__device__ __forceinline__ void quantise_groups(const GemmArgs& a, int qw, int lane, int K, int G,
                                                const QPrefetch& pf, int8_t* qs, int* rs,
                                                float* scale_out) {
  float scale;
  float amax = 0.0f;
  if constexpr (XT == X_QUANTISED) {
    scale = a.sa[0];
  } else {
    // absmax over the whole row, eight chunks per lane in flight at a time
    const int nch = K / 8;
    for (int base = 0; base < nch; base += 64 * 8) {
      float v[8][8];
      if (XT == X_BF16 && base == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w[4] = {pf.v[i].x, pf.v[i].y, pf.v[i].z, pf.v[i].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[i][2 * k] = __uint_as_float(w[k] << 16);
            v[i][2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) load8<XT>(a.x, min(base + 64 * i + lane, nch - 1), v[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    }
    amax = wave_max(amax);
    scale = amax / 127.0f;
  }
  *scale_out = scale;
  // 16 lanes per group, one 8-element chunk per lane; 4 groups per pass
  const int t = lane >> 4, cq = lane & 15;
  for (int g = qw + 4 * t; g < G; g += 16) {
    const int ch = g * 16 + cq;
    uint2 pk;
    if constexpr (XT == X_QUANTISED) {
      pk = (g == qw + 4 * t) ? make_uint2(pf.v[0].x, pf.v[0].y)
                             : *reinterpret_cast<const uint2*>(a.qa + 8 * ch);
    } else {
      float v[8];
      load8<XT>(a.x, ch, v);
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = 0.0f;
        if (amax != 0.0f) r = fminf(fmaxf(rintf(v[e] / scale), -127.0f), 127.0f);
        w[e >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu) << (8 * (e & 3));
      }
      pk = make_uint2(w[0], w[1]);
    }
    *reinterpret_cast<uint2*>(qs + 8 * ch) = pk;
  }
  // the same wavefront reads back what it wrote: order it at wavefront scope
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (cq < 4) {
    for (int g = qw + 4 * t; g < G; g += 16) {
      rs[4 * g + cq] = byte_sum16(*reinterpret_cast<const uint4*>(qs + kGroup * g + 16 * cq)) +
                       byte_sum16(*reinterpret_cast<const uint4*>(qs + kGroup * g + 64 + 16 * cq));
    }
  }
}

// Load the next unit of the run into a ring slot.  Past the end of the run the
// load still issues (so every wavefront has the same, compile-time count of
// loads in flight and waits stay exact) but reads the lane's own scale bytes,
// fetched moments ago; its value is never used.  Branch-free on purpose.
__device__ __forceinline__ void load_next(const uint8_t* base, int64_t hot_off, int u1, int nb0,
                                          int G, int g0, int gk, int lane, int& lu, int& lcb,
                                          int& lg, uint4& w) {
  const int live = lu < u1 ? 1 : 0;  // wave-uniform
  const int64_t code_off = unit_block(0, nb0 + lcb, G, g0 + lg, gk) * kBlockBytes + 16 * lane;
  w = ntload16(base + (live ? code_off : hot_off));
  lu += live;
  lg += live;
  const int wrap = (lg == gk) ? 1 : 0;
  lg -= wrap * gk;
  lcb += wrap;
}

// Quantiser wavefront qw, row held in registers (K <= kSmallK): lane chunk i
// is chunk lane + 64 i of the row (8 activations or codes), i.e. group
// 4i + lane/16.  The wavefront converts the chunks with i % 4 == qw, so each
// group is handled by exactly one wavefront, and forms those groups'
// per-quarter sums from what it has just written.
template <int XT>
__device__ __forceinline__ void quantise_held(const uint4* xr, int qw, int lane, int K, int G,
                                              float scale, float amax, int8_t* qs, int* rs) {
  const int nch = K / 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = lane + 64 * i;
    if ((i & 3) == qw && ch < nch) {
      uint2 pk;
      if constexpr (XT == X_QUANTISED) {
        pk = make_uint2(xr[i].x, xr[i].y);
      } else {
        const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = __uint_as_float((e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16));
          float r = 0.0f;
          if (amax != 0.0f) r = fminf(fmaxf(rintf(v / scale), -127.0f), 127.0f);
          w[e >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu) << (8 * (e & 3));
        }
        pk = make_uint2(w[0], w[1]);
      }
      *reinterpret_cast<uint2*>(qs + 8 * ch) = pk;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int cq = lane & 15;
  if (cq < 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 4 * i + (lane >> 4);
      if ((i & 3) == qw && g < G)
        rs[4 * g + cq] = byte_sum16(*reinterpret_cast<const uint4*>(qs + kGroup * g + 16 * cq)) +
                         byte_sum16(*reinterpret_cast<const uint4*>(qs + kGroup * g + 64 + 16 * cq));
    }
  }
}

template <int XT, bool SMALL, bool DEBUG>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ __attribute__((aligned(16))) float s_scale[kSWaves][kMaxRun][16];
  __shared__ __attribute__((aligned(16))) uint2 s_zero[kSWaves][kMaxRun];
  __shared__ float part[kMaxCb][kSWaves][16];
  __shared__ float s_sa;
  const int K = (int)a.K, G = K / kGroup, NB = (int)(a.N / kBlockCols);
  int8_t* qs = reinterpret_cast<int8_t*>(smem);               // [K] activation codes
  int* rs = reinterpret_cast<int*>(smem + K);                  // [4G] per-quarter code sums

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int c = lane & 15, j = lane >> 4;
  // This workgroup: channel blocks [nb0, nb1) x groups [g0, g1), dealt to
  // the streamers as equal contiguous runs of (block, group) units in
  // block-major order (the order of the codes plane).
  const int nb0 = (int)((int64_t)NB * blockIdx.x / gridDim.x);
  const int nb1 = (int)((int64_t)NB * (blockIdx.x + 1) / gridDim.x);
  const int g0 = (int)((int64_t)G * blockIdx.y / gridDim.y);
  const int g1 = (int)((int64_t)G * (blockIdx.y + 1) / gridDim.y);
  const int gk = g1 - g0, units = (nb1 - nb0) * gk;
  const int sw = wave - kQWaves;                                // streamer index
  const int u0 = sw >= 0 ? units * sw / kSWaves : 0;
  const int u1 = sw >= 0 ? units * (sw + 1) / kSWaves : 0;
  const int nrun = u1 - u0;

  // The quantisers' activation loads go out before any code block: requests
  // queued behind the weight stream wait microseconds.  With a short row
  // (SMALL) the quantisers hold all of it, form the absmax, and only then let
  // the streamers start (barrier 0); otherwise the first chunks are in
  // flight before the stream begins.
  QPrefetch pf;
  float sscale = 0.0f, samax = 0.0f;
  if (sw < 0) {
    if constexpr (SMALL) {
      const int nch = K / 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = min(lane + 64 * i, nch - 1);
        if constexpr (XT == X_QUANTISED) {
          const uint2 c2 = *reinterpret_cast<const uint2*>(a.qa + 8 * ch);
          pf.v[i] = make_uint4(c2.x, c2.y, 0u, 0u);
        } else {
          pf.v[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + 8 * ch);
        }
      }
      if constexpr (XT == X_QUANTISED) {
        sscale = a.sa[0];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w4[4] = {pf.v[i].x, pf.v[i].y, pf.v[i].z, pf.v[i].w};
#pragma unroll
          for (int k = 0; k < 4; ++k)
            samax = fmaxf(samax, fmaxf(fabsf(__uint_as_float(w4[k] << 16)),
                                       fabsf(__uint_as_float(w4[k] & 0xFFFF0000u))));
        }
        samax = wave_max(samax);
        sscale = samax / 127.0f;
      }
    } else {
      quantise_prefetch<XT>(a, wave, lane, K, pf);
    }
  }
  for (int t = tid; t < kMaxCb * kSWaves * 16; t += kThreads) (&part[0][0][0])[t] = 0.0f;
  __syncthreads();

  uint4 wv[D];
  int lcb = 0, lg = 0, lu = u0;  // next unit to load
  int64_t hot_off = 0;  // offset of this lane's 16 scale bytes (just fetched, cache-resident)
  if (sw >= 0) {
    // run metadata: scales (lane l: unit l/4, channels 4(l%4)..+3) and zero
    // blocks (lane l < 16: unit l), clamped to the run's last unit
    const int last = nrun > 0 ? nrun - 1 : 0;
    const int64_t bs = unit_block(u0 + min(lane >> 2, last), nb0, G, g0, gk);
    const int64_t bz = unit_block(u0 + min(lane & 15, last), nb0, G, g0, gk);
    const float* hot_s = a.w.scales + bs * 16 + 4 * (lane & 3);
    hot_off = reinterpret_cast<const uint8_t*>(hot_s) - a.w.codes;  // same packed buffer
    // the first D code blocks of the run, then its metadata
    lcb = nrun > 0 ? u0 / gk : 0;
    lg = nrun > 0 ? u0 % gk : 0;
#pragma unroll
    for (int i = 0; i < D; ++i)
      load_next(a.w.codes, hot_off, u1, nb0, G, g0, gk, lane, lu, lcb, lg, wv[i]);
    const uint4 s4 = *reinterpret_cast<const uint4*>(hot_s);
    const uint2 z2 = *reinterpret_cast<const uint2*>(a.w.zeros + bz * kZeroBlockBytes);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait
    if ((lane >> 2) < kMaxRun)
      *reinterpret_cast<uint4*>(&s_scale[sw][lane >> 2][4 * (lane & 3)]) = s4;
    if (lane < kMaxRun) s_zero[sw][lane] = z2;
  } else {
    float scale = sscale;
    if constexpr (SMALL)
      quantise_held<XT>(pf.v, wave, lane, K, G, sscale, samax, qs, rs);
    else
      quantise_groups<XT>(a, wave, lane, K, G, pf, qs, rs, &scale);
    if (wave == 0 && lane == 0) {
      s_sa = scale;
      if (a.sa_ws && blockIdx.x == 0 && blockIdx.y == 0) a.sa_ws[0] = scale;
    }
  }
  __syncthreads();

  if (sw >= 0) {
    float accf = 0.0f;
    int ccb = nrun > 0 ? u0 / gk : 0, cg = nrun > 0 ? u0 % gk : 0;  // compute position
    int cur = ccb;
    const int zshift = (c & 1) * 4;
    for (int ub = 0; ub < nrun; ub += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int r = ub + i;  // position in the run
        if (r < nrun) {
          if (ccb != cur) {
            accf += __shfl_xor(accf, 16);
            accf += __shfl_xor(accf, 32);
            if (j == 0) part[cur][sw][c] = accf;
            accf = 0.0f;
            cur = ccb;
          }
          const int g = g0 + cg;
          const uint4 al = *reinterpret_cast<const uint4*>(qs + kGroup * g + 16 * j);
          const uint4 ah = *reinterpret_cast<const uint4*>(qs + kGroup * g + 64 + 16 * j);
          const uint32_t d[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
          const uint32_t l4[4] = {al.x, al.y, al.z, al.w};
          const uint32_t h4[4] = {ah.x, ah.y, ah.z, ah.w};
          int acc = 0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc = __builtin_amdgcn_sdot4((int)(d[w] & 0x0F0F0F0Fu), (int)l4[w], acc, false);
            acc = __builtin_amdgcn_sdot4((int)((d[w] >> 4) & 0x0F0F0F0Fu), (int)h4[w], acc,
                                         false);
          }
          const uint32_t zbyte = reinterpret_cast<const uint8_t*>(&s_zero[sw][r])[c >> 1];
          const int z = (int)((zbyte >> zshift) & 0xFu);
          const int p = acc - z * rs[4 * g + j];
          if (DEBUG) {
            int pg = p + __shfl_xor(p, 16);
            pg += __shfl_xor(pg, 32);
            if (j == 0 && a.partials && a.m_begin == 0 && a.m_end > 0)
              a.partials[((int64_t)16 * (nb0 + ccb) + c) * G + g] = pg;
          }
          accf += s_scale[sw][r][c] * (float)p;
          ++cg;
          const int wrap = (cg == gk) ? 1 : 0;
          cg -= wrap * gk;
          ccb += wrap;
        }
        // refill this slot with the unit D ahead (a ring only when runs can
        // be longer than the ring)
        if constexpr (D < kMaxRun)
          load_next(a.w.codes, hot_off, u1, nb0, G, g0, gk, lane, lu, lcb, lg, wv[i]);
      }
    }
    accf += __shfl_xor(accf, 16);
    accf += __shfl_xor(accf, 32);
    if (nrun > 0 && j == 0) part[cur][sw][c] = accf;
  }
  __syncthreads();

  // each channel block: its streamer pieces in streamer order
  const int ncb = nb1 - nb0;
  const float scale = s_sa;
  for (int t = tid; t < ncb * 16; t += kThreads) {
    const int cbl = t >> 4, cc = t & 15;
    float total = part[cbl][0][cc];
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) total += part[cbl][w][cc];
    const int64_t n = (int64_t)16 * (nb0 + cbl) + cc;
    if (gridDim.y == 1) {
      if (a.y) a.y[n] = f32_to_bf16_rne(scale * total);
    } else {
      a.workspace[(int64_t)blockIdx.y * a.N + n] = total;
    }
  }
}

template <int XT, bool SMALL>
hipError_t launch_small(const GemmArgs& a, hipStream_t st) {
  const int64_t G = a.K / kGroup;
  dim3 grid((unsigned)a.cb, (unsigned)a.ksplit);
  const size_t lds = (size_t)a.K + 16 * (size_t)G;
  if (a.partials)
    hipLaunchKernelGGL((gemv_kernel<XT, SMALL, true>), grid, dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((gemv_kernel<XT, SMALL, false>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int XT>
hipError_t launch_xt(const GemmArgs& a, hipStream_t st) {
  if (XT != X_F32 && a.K <= kSmallK) return launch_small<XT, XT != X_F32>(a, st);
  return launch_small<XT, false>(a, st);
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
// split across workgroups (into >= 16-group slices) when there are too few
// channel blocks to give every compute unit one, or when one block's groups
// exceed what the streamers of a workgroup hold.  `cb` carries the number of
// workgroups along N.
GemvShape gemv_shape(int64_t N, int64_t K) {
  const int64_t NB = N / kBlockCols, G = K / kGroup;
  const int64_t cus = device_cus();
  const int64_t max_units = (int64_t)kSWaves * kMaxRun;
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
    s.cb = (int)NB;
    while ((int64_t)s.cb * s.ksplit < cus && G / (s.ksplit * 2) >= 16) s.ksplit *= 2;
  }
  return s;
}

// What the kernel's fixed LDS tables hold: <= kMaxCb channel blocks per
// workgroup and <= kMaxRun units per streamer wavefront.
bool gemv_shape_ok(int64_t N, int64_t K, const GemvShape& s) {
  const int64_t NB = N / kBlockCols, G = K / kGroup;
  if (s.cb < 1 || s.ksplit < 1 || s.ksplit > G) return false;
  const int64_t ncb = (NB + s.cb - 1) / s.cb;
  const int64_t gk_max = (G + s.ksplit - 1) / s.ksplit;
  const int64_t run = (ncb * gk_max + kSWaves - 1) / kSWaves;
  return ncb <= kMaxCb && run <= kMaxRun;
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t st) {
  if (!a.x) return launch_xt<X_QUANTISED>(a, st);
  if (a.x_dtype == 0) return launch_xt<X_BF16>(a, st);
  return launch_xt<X_F32>(a, st);
}

}  // namespace w4a8
