// Prefill GEMM (M > 16) on the int8 matrix cores.
//
// "The 4-bit CPU path", section "W4A16": dequantising per row is far too
// slow once many tokens share the weights, so large batches take a separate
// GEMM path.  Here that path keeps the weights as 4-bit codes in LDS, unpacks
// them in registers to q - z bytes and runs v_mfma_i32_16x16x64_i8 per group,
// so the weights are never expanded in HBM.
//
// Tile: 256 tokens x 128 output channels per 512-thread workgroup, eight
// wavefronts of 64 x 64.  Per group of 128 input channels the workgroup
// stages the activation tile (256 x 128 int8), the eight code blocks of the
// tile unpacked once to q - z bytes, and their scales in LDS, double-buffered,
// with the next group's loads in flight while the current group computes.
// The activation tile goes from memory straight into LDS (buffer loads with
// the LDS bit: no registers, no LDS store instructions); its 16-byte chunks
// are swizzled by row so that both the 1 KiB load chunks and the MFMA
// fragment reads are free of bank conflicts.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 512;           // 8 wavefronts, 2 per SIMD
constexpr int BM = 256;                 // tokens per tile
constexpr int BN = 128;                 // output channels per tile
constexpr int NCB = BN / kBlockCols;    // packed blocks per tile (8)
constexpr int kAOff = 0;                              // activation tile [BM][128], chunks swizzled
constexpr int kBOff = kAOff + BM * kGroup;            // unpacked q - z, [NCB][2][64 lanes][16 B]
constexpr int kSOff = kBOff + NCB * 2 * kBlockBytes;  // scales [NCB][16]
constexpr int kBufBytes = kSOff + NCB * 16 * 4;
constexpr int kADmaRows = 1024 / kGroup;                      // tile rows per 1 KiB load (8)
constexpr int kADma = BM / kADmaRows / (kThreads / 64);       // such loads per wavefront (4)

// 16-byte chunk c (input channels 16c..16c+15 of the group) of tile row r
// sits at chunk c ^ (r % 8) of the row's 128 bytes.
__device__ __forceinline__ int a_chunk(int r, int c) { return c ^ (r & 7); }

// One group's W4 weight operands as they come from HBM, held in registers
// while the previous group computes.  (W8 weights go straight into LDS.)
struct Stage {
  v4i b;          // this thread's 16 packed bytes: block t/64, lane t%64
  uint32_t zb;    // the byte holding that lane's zero point
  float s;        // scale of channel t%16 of block (t/16)%8
};

// Per-thread byte offsets of its operands within group 0; group g adds a
// uniform g * (bytes per group) to the plane base.  Rows and blocks past the
// matrix read the last valid one: they only reach outputs that are never
// stored, so nothing needs masking and every thread issues the same loads.
// (The host keeps M*K and N*K/2 below 2^31 on this path.)
struct Offsets {
  uint32_t a[kADma];  // activation bytes this lane brings into LDS chunk kADma * wave + i
  uint32_t b, z, s;
  int zshift;
};

template <bool W8>
__device__ __forceinline__ Offsets make_offsets(const GemmArgs& a, int64_t m0, int64_t cb0,
                                                int64_t NB, int64_t G) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Offsets o;
  // 1 KiB load chunk i of the wavefront holds tile rows kADmaRows (kADma wave
  // + i) + lane / 8; lane writes physical chunk lane % 8 of its row
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int r = kADmaRows * (kADma * wave + i) + (lane >> 3);
    o.a[i] = (uint32_t)(min(m0 + r, a.M - 1) * a.K + 16 * a_chunk(r, lane & 7));
  }
  const int64_t nb = min(cb0 + (tid >> 6), NB - 1);
  o.b = (uint32_t)(nb * G * (W8 ? 2 : 1) * kBlockBytes + (tid & 63) * 16);
  o.z = (uint32_t)(nb * G * kZeroBlockBytes + ((tid & 15) >> 1));
  o.zshift = (tid & 1) * 4;
  const int64_t nbs = min(cb0 + ((tid >> 4) & (NCB - 1)), NB - 1);
  o.s = (uint32_t)(nbs * G * 16 + (tid & 15));
  return o;
}

__device__ __forceinline__ void load_stage(const GemmArgs& a, const Offsets& o, int64_t g,
                                           Stage& st) {
  const uint8_t* codes = a.w.codes + g * kBlockBytes;
  const uint8_t* zeros = a.w.zeros + g * kZeroBlockBytes;
  const float* scales = a.w.scales + g * 16;
  st.b = *reinterpret_cast<const v4i*>(codes + o.b);
  st.zb = zeros[o.z];
  st.s = scales[o.s];
}

// Stage -> LDS.  The packed codes are unpacked here, once per workgroup, to
// signed q - z bytes in exactly the order the MFMA B operand is read: block
// u, half h (low nibbles = input channels 16j..16j+15 of the group, high =
// 64+16j..), lane L.
__device__ __forceinline__ void store_stage(uint8_t* buf, const Stage& st, int zshift) {
  const int tid = threadIdx.x;
  const uint32_t zz = ((st.zb >> zshift) & 0xFu) * 0x01010101u;
  v4i lo, hi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t d = (uint32_t)st.b[w];
    lo[w] = (int)sub_zero_bytes(d & 0x0F0F0F0Fu, zz);
    hi[w] = (int)sub_zero_bytes((d >> 4) & 0x0F0F0F0Fu, zz);
  }
  const int u = tid >> 6, L = tid & 63;
  *reinterpret_cast<v4i*>(buf + kBOff + (u * 2 + 0) * kBlockBytes + L * 16) = lo;
  *reinterpret_cast<v4i*>(buf + kBOff + (u * 2 + 1) * kBlockBytes + L * 16) = hi;
  // every thread holds the scale of entry tid % 128 (four identical writers
  // per entry), so the store needs no branch
  reinterpret_cast<float*>(buf + kSOff)[tid & (NCB * 16 - 1)] = st.s;
}

// Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
// run of tiles (tokens fastest) so the packed weights of a tile column are
// fetched into one XCD's L2 and the tiles running together on an XCD share
// their operands there.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t T) {
  const int64_t xcd = b % 8, local = b / 8;
  const int64_t per = T / 8, rem = T % 8;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// One group on the matrix cores: fragments from LDS, the 16 tiles' MFMA
// pairs, and the per-group rescale into the fp32 accumulators.
template <bool DEBUG>
__device__ __forceinline__ void compute_group(const GemmArgs& a, const uint8_t* buf, int64_t g,
                                              int64_t m0, int64_t cb0, int64_t NB, int64_t G,
                                              float (&accf)[4][4][4]);

// W8: one group's MFMA pairs into the int32 totals (no per-group rescale).
__device__ __forceinline__ void compute_group_w8(const uint8_t* buf, v4i (&acci)[16]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  v4i b0[4], b1[4], a0[4], a1[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cb = wn * 4 + u;
    b0[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 0) * kBlockBytes + lane * 16);
    b1[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 1) * kBlockBytes + lane * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // rows wm*64 + 16i + r16: the swizzle is r16 % 8
    const uint8_t* arow = buf + kAOff + (wm * 64 + i * 16 + r16) * kGroup;
    a0[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, j));
    a1[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, 4 + j));
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int i = t >> 2, u = t & 3;
    acci[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b0[u], acci[t], 0, 0, 0);
    acci[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[i], b1[u], acci[t], 0, 0, 0);
  }
  // the totals are otherwise only read after the loop, and the compiler would
  // sink every group's products there; reading and writing them in an empty
  // statement keeps this group's products here (no instruction is emitted)
#pragma unroll
  for (int t = 0; t < 16; ++t) asm volatile("" : "+v"(acci[t]));
}

template <bool DEBUG>
__device__ __forceinline__ void compute_group(const GemmArgs& a, const uint8_t* buf, int64_t g,
                                              int64_t m0, int64_t cb0, int64_t NB, int64_t G,
                                              float (&accf)[4][4][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  v4i b0[4], b1[4];
  float sv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cb = wn * 4 + u;
    b0[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 0) * kBlockBytes + lane * 16);
    b1[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 1) * kBlockBytes + lane * 16);
    sv[u] = reinterpret_cast<const float*>(buf + kSOff)[cb * 16 + r16];
  }
  v4i a0[4], a1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // rows wm*64 + 16i + r16: the swizzle is r16 % 8
    const uint8_t* arow = buf + kAOff + (wm * 64 + i * 16 + r16) * kGroup;
    a0[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, j));
    a1[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, 4 + j));
  }
  // MFMA pair of tile t, then the rescale of tile t - 2 (whose result is
  // ready by then): the vector ALU and the matrix cores work side by side.
  // The fences keep the compiler from regrouping them.
  v4i acc[16];
#pragma unroll
  for (int t = 0; t < 18; ++t) {
    if (t < 16) {
      const int i = t >> 2, u = t & 3;
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b0[u], kBiasSeed, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[i], b1[u], acc[t], 0, 0, 0);
    }
    if (t >= 2) {
      const int e = t - 2, i = e >> 2, u = e & 3;
      if (DEBUG && a.partials) {
        const int64_t nb = cb0 + wn * 4 + u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
          if (nb < NB && m < a.M && m >= a.m_begin && m < a.m_end)
            a.partials[((m - a.m_begin) * a.N + nb * 16 + r16) * G + g] = acc[e][r] - kBiasBits;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] += sv[u] * unbias(acc[e][r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// W8: the W8A8 weights (two 1 KiB halves per block, already in MFMA operand
// order, one scale per channel).  Each group's products accumulate in int32
// over the workgroup's whole K slice, and the scales are applied once.
template <bool DEBUG, bool W8>
__global__ void __launch_bounds__(kThreads)
prefill_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][kBufBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 3, wn = wave >> 2;   // 4 x 2 wavefronts of 64 x 64
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t G = a.K / kGroup;
  const int64_t NB = a.N / kBlockCols;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (NB + NCB - 1) / NCB;
  // Tiles [0, main_tiles) run whole (or as gridDim.y K slices).  With a tail
  // split, workgroup main_tiles + r takes K slice r / tail_tiles of tile
  // main_tiles + r % tail_tiles; those tiles are whole column tiles, the
  // channels from tail_n0 on, and their slices go to the workspace
  // [tail_split][M][N - tail_n0].
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t main_tiles = a.tail_split > 1 ? tiles - a.tail_tiles : tiles;
  int64_t t;
  int slice = blockIdx.y, nslices = gridDim.y;
  int64_t wn0 = 0;  // first channel of the workspace rows
  if ((int64_t)blockIdx.x < main_tiles) {
    t = xcd_tile(blockIdx.x, main_tiles);
  } else {
    const int64_t r = blockIdx.x - main_tiles;
    t = main_tiles + r % a.tail_tiles;
    slice = (int)(r / a.tail_tiles);
    nslices = a.tail_split;
    wn0 = a.tail_n0;
  }
  const bool split = nslices > 1;
  const int64_t ldw = a.N - wn0;  // workspace row length
  const int64_t tm = t % tiles_m, tn = t / tiles_m;
  const int64_t m0 = tm * BM, cb0 = tn * NCB;
  // K slice of this workgroup: groups [gb, ge) (all of K unless split)
  const int64_t gb = G * slice / nslices, ge = G * (slice + 1) / nslices;

  float accf[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] = 0.0f;
  v4i acci[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acci[t] = v4i{0, 0, 0, 0};
  auto compute = [&](const uint8_t* buf, int64_t g) __attribute__((always_inline)) {
    if constexpr (W8)
      compute_group_w8(buf, acci);
    else
      compute_group<DEBUG>(a, buf, g, m0, cb0, NB, G, accf);
  };

  // One group of 128 input channels per step: while group g computes from
  // one LDS buffer, group g + 1's activation tile streams into the other and
  // its weight operands into registers, unpacked there after the compute.
  // The buffers alternate, so the loop is unrolled by two.  (The barrier
  // waits for this wavefront's loads, the LDS ones included.)
  const Offsets off = make_offsets<W8>(a, m0, cb0, NB, G);
  const __amdgpu_buffer_rsrc_t rqa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.qa), (short)0, (int)(a.M * a.K),
                                        kBufferWord3);
  // W8: the weight halves are MFMA operands as stored, so they too go
  // straight into LDS: block u = wave, half h to chunk 2u + h of the B area
  const __amdgpu_buffer_rsrc_t rcw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w.codes), (short)0, W8 ? (int)(a.N * a.K) : 0, kBufferWord3);
  // group g's LDS-direct operands into buffer B (wave-uniform LDS addresses)
#define PREFILL_DMA(B, g)                                                                        \
  do {                                                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < kADma; ++i_)                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                  \
          rqa, &smem[B][kAOff + (kADma * wave + i_) * 1024], 16, off.a[i_],                      \
          (unsigned)__builtin_amdgcn_readfirstlane((int)((g) * kGroup)), 0, 0);                  \
    if constexpr (W8) {                                                                          \
      _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_)                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
            rcw, &smem[B][kBOff + (2 * wave + h_) * kBlockBytes], 16, off.b + h_ * kBlockBytes, \
            (unsigned)__builtin_amdgcn_readfirstlane((int)((g) * 2 * kBlockBytes)), 0, 0);       \
    }                                                                                            \
  } while (0)
  Stage sb;  // W4 only
  PREFILL_DMA(0, gb);
  if constexpr (!W8) {
    load_stage(a, off, gb, sb);
    store_stage(smem[0], sb, off.zshift);
  }
  __syncthreads();
  for (int64_t g = gb; g < ge; g += 2) {
    if (g + 1 < ge) {  // buffer 1 was last read before the previous barrier
      PREFILL_DMA(1, g + 1);
      if constexpr (!W8) load_stage(a, off, g + 1, sb);
    }
    compute(smem[0], g);
    if constexpr (!W8)
      if (g + 1 < ge) store_stage(smem[1], sb, off.zshift);
    __syncthreads();
    if (g + 1 >= ge) break;
    if (g + 2 < ge) {
      PREFILL_DMA(0, g + 2);
      if constexpr (!W8) load_stage(a, off, g + 2, sb);
    }
    compute(smem[1], g + 1);
    if constexpr (!W8)
      if (g + 2 < ge) store_stage(smem[0], sb, off.zshift);
    __syncthreads();
  }
#undef PREFILL_DMA

  if constexpr (W8) {
    // int32 totals: to the workspace when K is split, else scaled to y (and
    // written out for the debug row window)
    float swv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) swv[u] = a.w.scales[min(cb0 + wn * 4 + u, NB - 1) * 16 + r16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
        if (m >= a.M) continue;
        const float sam = split ? 0.0f : a.sa[m];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t nb = cb0 + wn * 4 + u;
          if (nb >= NB) continue;
          const int64_t n = nb * 16 + r16;
          const int p = acci[i * 4 + u][r];
          if (split) {
            reinterpret_cast<int32_t*>(a.workspace)[((int64_t)slice * a.M + m) * ldw + n - wn0] = p;
            continue;
          }
          if (DEBUG && a.partials && m >= a.m_begin && m < a.m_end)
            a.partials[(m - a.m_begin) * a.N + n] = p;
          if (a.y) a.y[m * a.N + n] = f32_to_bf16_rne(sam * (swv[u] * (float)p));
        }
      }
    return;
  }

  if (split) {
    // split K: this slice's float sums, reduced (and scaled) by a second kernel
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
        if (m >= a.M) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t nb = cb0 + wn * 4 + u;
          if (nb < NB)
            a.workspace[((int64_t)slice * a.M + m) * ldw + nb * 16 + r16 - wn0] = accf[i][u][r];
        }
      }
    return;
  }
  if (!a.y) return;
  // all row scales first (one wait), then the stores
  float sam[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sam[i][r] = a.sa[min(m0 + wm * 64 + i * 16 + 4 * j + r, a.M - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t nb = cb0 + wn * 4 + u;
        if (nb < NB) a.y[m * a.N + nb * 16 + r16] = f32_to_bf16_rne(sam[i][r] * accf[i][u][r]);
      }
    }
  }
}

// --------------------------------------------------------------- wide tiles
//
// The same product on 256 x 256 output tiles: eight wavefronts of 64 tokens x
// 128 channels (4 x 8 tiles of 16 x 16), still two per SIMD.  Per group of
// 128 input channels the workgroup moves the activation tile (32 KiB, straight
// into LDS) and the 16 code blocks (16 KiB, unpacked once to 32 KiB of q - z
// bytes in LDS) for twice the products of the 256 x 128 tile: half the
// activation bytes per product, and a quarter fewer fragment reads per product
// (64 x 128 wave tiles read 24 KiB per 1 MiB products instead of 16 KiB per
// 0.5 MiB).  Both the LDS and the path from L2 into the compute unit bound the
// 256 x 128 tile well before its matrix cores do.
//
// When the wide tiles fill whole rounds of the compute units plus a partial
// round that half as many compute units could not finish faster in halves,
// the partial round's channels run instead as 256 x 128 tiles of the same
// kernel (wavefronts of 64 x 64: NU = 4 column tiles each), all in one round:
// no K split, no partial sums in memory and no second kernel.
namespace wide {

constexpr int BN = 256;                       // output channels per tile
constexpr int NCB = BN / kBlockCols;          // packed blocks per tile (16)
constexpr int kAOff = 0;                      // activation tile [BM][128], chunks swizzled
constexpr int kBOff = kAOff + BM * kGroup;    // unpacked q - z, [NCB][2][64 lanes][16 B]
constexpr int kSOff = kBOff + NCB * 2 * kBlockBytes;  // scales [16 channels][NCB]
constexpr int kBufBytes = kSOff + NCB * 16 * 4;

// One group's weight operands in registers: thread t holds lane t % 64 of
// code blocks t / 64 and t / 64 + 8 of the tile, their zero-point bytes, and
// the scale of scale-table entry t % 256.  (Half tiles use the first of the
// two blocks and entries below 128 only.)
struct Stage {
  v4i b[2];
  uint32_t zb[2];
  float s;
};

struct Offsets {
  uint32_t a[kADma];
  uint32_t b[2], z[2], s;
  int zshift;
};

// Channel blocks per tile: 16 for whole tiles (NU = 8), 8 for half tiles.
template <int NU>
__device__ __forceinline__ Offsets make_offsets(const GemmArgs& a, int64_t m0, int64_t cb0,
                                                int64_t NB, int64_t G) {
  constexpr int kBlocks = 2 * NU;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Offsets o;
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int r = kADmaRows * (kADma * wave + i) + (lane >> 3);
    o.a[i] = (uint32_t)(min(m0 + r, a.M - 1) * a.K + 16 * a_chunk(r, lane & 7));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int64_t nb = min(cb0 + wave + 8 * k, NB - 1);
    o.b[k] = (uint32_t)(nb * G * kBlockBytes + lane * 16);
    o.z[k] = (uint32_t)(nb * G * kZeroBlockBytes + ((lane & 15) >> 1));
  }
  o.zshift = (lane & 1) * 4;
  const int64_t nbs = min(cb0 + ((tid >> 4) & (kBlocks - 1)), NB - 1);
  o.s = (uint32_t)(nbs * G * 16 + (tid & 15));
  return o;
}

template <int NU>
__device__ __forceinline__ void load_stage(const GemmArgs& a, const Offsets& o, int64_t g,
                                           Stage& st) {
  const uint8_t* codes = a.w.codes + g * kBlockBytes;
  const uint8_t* zeros = a.w.zeros + g * kZeroBlockBytes;
#pragma unroll
  for (int k = 0; k < NU / 4; ++k) {
    st.b[k] = *reinterpret_cast<const v4i*>(codes + o.b[k]);
    st.zb[k] = zeros[o.z[k]];
  }
  st.s = (a.w.scales + g * 16)[o.s];
}

// Stage -> LDS: code block k (of the thread's two) unpacked to q - z bytes in
// MFMA operand order (block u, half h, lane L) ...
__device__ __forceinline__ void store_block(uint8_t* buf, const Stage& st, int zshift, int k) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t zz = ((st.zb[k] >> zshift) & 0xFu) * 0x01010101u;
  v4i lo, hi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t d = (uint32_t)st.b[k][w];
    lo[w] = (int)sub_zero_bytes(d & 0x0F0F0F0Fu, zz);
    hi[w] = (int)sub_zero_bytes((d >> 4) & 0x0F0F0F0Fu, zz);
  }
  const int u = wave + 8 * k;
  *reinterpret_cast<v4i*>(buf + kBOff + (u * 2 + 0) * kBlockBytes + lane * 16) = lo;
  *reinterpret_cast<v4i*>(buf + kBOff + (u * 2 + 1) * kBlockBytes + lane * 16) = hi;
}
// ... and the scale table, transposed to [channel][block] so that a lane's
// scales are contiguous.
template <int NU>
__device__ __forceinline__ void store_scale(uint8_t* buf, const Stage& st) {
  const int e = threadIdx.x & (NCB * 16 - 1);  // entry (block e / 16, channel e % 16)
  if (NU == 8 || e < 128) reinterpret_cast<float*>(buf + kSOff)[(e & 15) * NCB + (e >> 4)] = st.s;
}
template <int NU>
__device__ __forceinline__ void store_stage(uint8_t* buf, const Stage& st, int zshift) {
  store_block(buf, st, zshift, 0);
  if (NU == 8) store_block(buf, st, zshift, 1);
  store_scale<NU>(buf, st);
}

// One group: the wavefront's 4 x NU tiles, an MFMA pair each, and the rescale
// of the tile two steps behind into the float accumulators.  A fragments are
// read once; B fragments column tile by column tile, one ahead.  With `next`
// set, the next group's weights (already loaded into `st`) are unpacked into
// `next` between the MFMA pairs, where the other wavefront of the SIMD keeps
// the matrix core busy, rather than in a burst after them.
template <bool DEBUG, int NU>
__device__ __forceinline__ void compute_group(const GemmArgs& a, const uint8_t* buf, int64_t g,
                                              int64_t m0, int64_t cb0, int64_t NB, int64_t G,
                                              float (&accf)[4][NU][4], uint8_t* next,
                                              const Stage& st, int zshift) {
  constexpr int T = 4 * NU;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  v4i a0[4], a1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // rows wm*64 + 16i + r16: the swizzle is r16 % 8
    const uint8_t* arow = buf + kAOff + (wm * 64 + i * 16 + r16) * kGroup;
    a0[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, j));
    a1[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, 4 + j));
  }
  const float* srow = reinterpret_cast<const float*>(buf + kSOff) + r16 * NCB + wn * NU;
  float sv[NU];
#pragma unroll
  for (int q = 0; q < NU / 4; ++q) {
    const v4i sq = *reinterpret_cast<const v4i*>(srow + 4 * q);
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[4 * q + u] = __int_as_float(sq[u]);
  }
  v4i b0[NU], b1[NU];
  auto load_b = [&](int u) __attribute__((always_inline)) {
    const int cb = wn * NU + u;
    b0[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 0) * kBlockBytes + lane * 16);
    b1[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 1) * kBlockBytes + lane * 16);
  };
  load_b(0);
  v4i acc[T];
#pragma unroll
  for (int t = 0; t < T + 2; ++t) {
    if (t < T) {
      const int u = t >> 2, i = t & 3;
      if (i == 0 && u + 1 < NU) load_b(u + 1);  // one column tile ahead
      if (next && t == T / 2) store_block(next, st, zshift, 0);
      if (NU == 8 && next && t == 22) store_block(next, st, zshift, 1);
      if (next && t == T - 4) store_scale<NU>(next, st);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b0[u], kBiasSeed, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[i], b1[u], acc[t], 0, 0, 0);
    }
    if (t >= 2) {
      const int e = t - 2, u = e >> 2, i = e & 3;
      if (DEBUG && a.partials) {
        const int64_t nb = cb0 + wn * NU + u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
          if (nb < NB && m < a.M && m >= a.m_begin && m < a.m_end)
            a.partials[((m - a.m_begin) * a.N + nb * 16 + r16) * G + g] = acc[e][r] - kBiasBits;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] += sv[u] * unbias(acc[e][r]);
      // The next MFMA pair takes its A operand through this empty statement,
      // which reads the tile just rescaled: the compiler cannot run the
      // pairs ahead of the rescales (which would keep every tile's int32
      // results live at once) nor delay the rescales behind them.
      if (t + 1 < T) {
        const int in = (t + 1) & 3;
        asm volatile("" : "+v"(a0[in]) : "v"(accf[i][u][0]), "v"(accf[i][u][1]), "v"(accf[i][u][2]),
                     "v"(accf[i][u][3]));
      }
    }
  }
}

// One output tile (rows m0.., channel blocks cb0..) over groups [gb, ge):
// NU = 8 a whole 256 x 256 tile, NU = 4 a half tile of 256 x 128.  With
// `split`, this K slice's float sums go to the workspace (rows of ldw
// channels from wn0) instead of y.
template <bool DEBUG, int NU>
__device__ __forceinline__ void tile(const GemmArgs& a, uint8_t (&smem)[2][kBufBytes], int64_t m0,
                                     int64_t cb0, int64_t gb, int64_t ge, bool split, int slice,
                                     int64_t wn0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t G = a.K / kGroup;
  const int64_t NB = a.N / kBlockCols;
  const int64_t ldw = a.N - wn0;

  float accf[4][NU][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] = 0.0f;

  const Offsets off = make_offsets<NU>(a, m0, cb0, NB, G);
  const __amdgpu_buffer_rsrc_t rqa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.qa), (short)0, (int)(a.M * a.K),
                                        kBufferWord3);
#define WIDE_DMA(B, g)                                                                        \
  do {                                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < kADma; ++i_)                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                               \
          rqa, &smem[B][kAOff + (kADma * wave + i_) * 1024], 16, off.a[i_],                   \
          (unsigned)__builtin_amdgcn_readfirstlane((int)((g) * kGroup)), 0, 0);               \
  } while (0)
  Stage sb;
  WIDE_DMA(0, gb);
  load_stage<NU>(a, off, gb, sb);
  store_stage<NU>(smem[0], sb, off.zshift);
  __syncthreads();
  for (int64_t g = gb; g < ge; g += 2) {
    if (g + 1 < ge) {  // buffer 1 was last read before the previous barrier
      WIDE_DMA(1, g + 1);
      load_stage<NU>(a, off, g + 1, sb);
    }
    compute_group<DEBUG, NU>(a, smem[0], g, m0, cb0, NB, G, accf, g + 1 < ge ? smem[1] : nullptr,
                             sb, off.zshift);
    __syncthreads();
    if (g + 1 >= ge) break;
    if (g + 2 < ge) {
      WIDE_DMA(0, g + 2);
      load_stage<NU>(a, off, g + 2, sb);
    }
    compute_group<DEBUG, NU>(a, smem[1], g + 1, m0, cb0, NB, G, accf,
                             g + 2 < ge ? smem[0] : nullptr, sb, off.zshift);
    __syncthreads();
  }
#undef WIDE_DMA

  if (split) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
        if (m >= a.M) continue;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int64_t nb = cb0 + wn * NU + u;
          if (nb < NB)
            a.workspace[((int64_t)slice * a.M + m) * ldw + nb * 16 + r16 - wn0] = accf[i][u][r];
        }
      }
    return;
  }
  if (!a.y) return;
  float sam[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sam[i][r] = a.sa[min(m0 + wm * 64 + i * 16 + 4 * j + r, a.M - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int64_t nb = cb0 + wn * NU + u;
        if (nb < NB) a.y[m * a.N + nb * 16 + r16] = f32_to_bf16_rne(sam[i][r] * accf[i][u][r]);
      }
    }
  }
}

// W8A8 on the same tiles: the weights ([N/16][G][2][1 KiB], already MFMA
// operands) go straight into LDS like the activations, each group's MFMA
// pairs accumulate into int32 totals over the tile's K range, and the
// per-channel scales apply once at the end.  With no unpack and no
// per-group rescale the loop is matrix-core and LDS work only.
template <int NU>
__device__ __forceinline__ void compute_group_w8(const uint8_t* buf, int (&tot)[4][NU][4]) {
  constexpr int T = 4 * NU;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  v4i a0[4], a1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // rows wm*64 + 16i + r16: the swizzle is r16 % 8
    const uint8_t* arow = buf + kAOff + (wm * 64 + i * 16 + r16) * kGroup;
    a0[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, j));
    a1[i] = *reinterpret_cast<const v4i*>(arow + 16 * a_chunk(r16, 4 + j));
  }
  v4i b0[NU], b1[NU];
  auto load_b = [&](int u) __attribute__((always_inline)) {
    const int cb = wn * NU + u;
    b0[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 0) * kBlockBytes + lane * 16);
    b1[u] = *reinterpret_cast<const v4i*>(buf + kBOff + (cb * 2 + 1) * kBlockBytes + lane * 16);
  };
  load_b(0);
  // as for W4A8: each tile's pair from zero, then added into the int32
  // totals two tiles later (an MFMA accumulating into a total that lives
  // across the loop was given a fresh register every time and spilled)
  v4i acc[T];
#pragma unroll
  for (int t = 0; t < T + 2; ++t) {
    if (t < T) {
      const int u = t >> 2, i = t & 3;
      if (i == 0 && u + 1 < NU) load_b(u + 1);  // one column tile ahead
      const v4i zero = {0, 0, 0, 0};
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[i], b0[u], zero, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[i], b1[u], acc[t], 0, 0, 0);
    }
    if (t >= 2) {
      const int e = t - 2, u = e >> 2, i = e & 3;
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[i][u][r] += acc[e][r];
      if (t + 1 < T) {  // keeps the pairs and the adds interleaved, as for W4A8
        const int in = (t + 1) & 3;
        asm volatile("" : "+v"(a0[in]) : "v"(tot[i][u][0]), "v"(tot[i][u][1]), "v"(tot[i][u][2]),
                     "v"(tot[i][u][3]));
      }
    }
  }
}

// One W8A8 tile, as tile() for W4A8: with `split`, this K slice's int32
// totals go to the workspace (rows of ldw channels from wn0).
template <bool DEBUG, int NU>
__device__ __forceinline__ void tile_w8(const GemmArgs& a, uint8_t (&smem)[2][kBufBytes], int64_t m0,
                                        int64_t cb0, int64_t gb, int64_t ge, bool split, int slice,
                                        int64_t wn0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t G = a.K / kGroup;
  const int64_t NB = a.N / kBlockCols;
  const int64_t ldw = a.N - wn0;

  int tot[4][NU][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[i][u][r] = 0;

  const Offsets off = make_offsets<NU>(a, m0, cb0, NB, G);
  // weight block wave + 8k of the tile, both halves, lane 16 B
  uint32_t ob[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    ob[k] = (uint32_t)(min(cb0 + wave + 8 * k, NB - 1) * G * 2 * kBlockBytes + lane * 16);
  const __amdgpu_buffer_rsrc_t rqa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.qa), (short)0, (int)(a.M * a.K),
                                        kBufferWord3);
  const __amdgpu_buffer_rsrc_t rcw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w.codes), (short)0, (int)(a.N * a.K), kBufferWord3);
#define WIDE_W8_DMA(B, g)                                                                     \
  do {                                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < kADma; ++i_)                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                               \
          rqa, &smem[B][kAOff + (kADma * wave + i_) * 1024], 16, off.a[i_],                   \
          (unsigned)__builtin_amdgcn_readfirstlane((int)((g) * kGroup)), 0, 0);               \
    _Pragma("unroll") for (int k_ = 0; k_ < NU / 4; ++k_)                                    \
      _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_)                                       \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                             \
            rcw, &smem[B][kBOff + ((wave + 8 * k_) * 2 + h_) * kBlockBytes], 16,              \
            ob[k_] + h_ * kBlockBytes,                                                        \
            (unsigned)__builtin_amdgcn_readfirstlane((int)((g) * 2 * kBlockBytes)), 0, 0);    \
  } while (0)
  WIDE_W8_DMA(0, gb);
  __syncthreads();
  for (int64_t g = gb; g < ge; g += 2) {
    if (g + 1 < ge) WIDE_W8_DMA(1, g + 1);  // buffer 1 was last read before the previous barrier
    compute_group_w8<NU>(smem[0], tot);
    __syncthreads();
    if (g + 1 >= ge) break;
    if (g + 2 < ge) WIDE_W8_DMA(0, g + 2);
    compute_group_w8<NU>(smem[1], tot);
    __syncthreads();
  }
#undef WIDE_W8_DMA

  float swv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) swv[u] = a.w.scales[min(cb0 + wn * NU + u, NB - 1) * 16 + r16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 64 + i * 16 + 4 * j + r;
      if (m >= a.M) continue;
      const float sam = split ? 0.0f : a.sa[m];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int64_t nb = cb0 + wn * NU + u;
        if (nb >= NB) continue;
        const int64_t n = nb * 16 + r16;
        const int p = tot[i][u][r];
        if (split) {
          reinterpret_cast<int32_t*>(a.workspace)[((int64_t)slice * a.M + m) * ldw + n - wn0] = p;
          continue;
        }
        if (DEBUG && a.partials && m >= a.m_begin && m < a.m_end)
          a.partials[(m - a.m_begin) * a.N + n] = p;
        if (a.y) a.y[m * a.N + n] = f32_to_bf16_rne(sam * (swv[u] * (float)p));
      }
    }
}

// Workgroups [0, main) take the whole tiles (XCD-aware order, tokens
// fastest); the rest take the tail: with a.tail_split > 1, K slice r /
// tail_tiles of whole tile main + r % tail_tiles; with a.tail_split == -1
// (half tiles), half tile r of the channels from tail_n0 on.
template <bool DEBUG, bool W8>
__global__ void __launch_bounds__(kThreads)
prefill_wide_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][kBufBytes];
  const int64_t G = a.K / kGroup;
  const int64_t NB = a.N / kBlockCols;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (NB + NCB - 1) / NCB;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t main_tiles = a.tail_split > 1 || a.tail_split == -1 ? tiles - a.tail_tiles : tiles;
  if ((int64_t)blockIdx.x < main_tiles) {
    const int64_t t = xcd_tile(blockIdx.x, main_tiles);
    const int slice = blockIdx.y, nslices = gridDim.y;
    const int64_t tm = t % tiles_m, tn = t / tiles_m;
    if constexpr (W8)
      tile_w8<DEBUG, 8>(a, smem, tm * BM, tn * NCB, G * slice / nslices, G * (slice + 1) / nslices,
                        nslices > 1, slice, 0);
    else
      tile<DEBUG, 8>(a, smem, tm * BM, tn * NCB, G * slice / nslices, G * (slice + 1) / nslices,
                     nslices > 1, slice, 0);
    return;
  }
  const int64_t r = blockIdx.x - main_tiles;
  if (a.tail_split == -1) {
    const int64_t tm = r % tiles_m, tn = r / tiles_m;
    if constexpr (W8)
      tile_w8<DEBUG, 4>(a, smem, tm * BM, a.tail_n0 / kBlockCols + tn * (NCB / 2), 0, G, false, 0, 0);
    else
      tile<DEBUG, 4>(a, smem, tm * BM, a.tail_n0 / kBlockCols + tn * (NCB / 2), 0, G, false, 0, 0);
    return;
  }
  const int64_t t = main_tiles + r % a.tail_tiles;
  const int slice = (int)(r / a.tail_tiles);
  const int64_t tm = t % tiles_m, tn = t / tiles_m;
  if constexpr (W8)
    tile_w8<DEBUG, 8>(a, smem, tm * BM, tn * NCB, G * slice / a.tail_split,
                      G * (slice + 1) / a.tail_split, true, slice, a.tail_n0);
  else
    tile<DEBUG, 8>(a, smem, tm * BM, tn * NCB, G * slice / a.tail_split,
                   G * (slice + 1) / a.tail_split, true, slice, a.tail_n0);
}

}  // namespace wide

// --------------------------------------------------------------- W4A16
//
// "The 4-bit CPU path", section "W4A16": large batches of bf16 activations
// take their own GEMM path, the int4 weights expanded once per batch rather
// than per activation row.  Here they are expanded once per workgroup and
// group, in LDS, to exact bf16 q - z, and multiplied on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, float32 sums); each group's float sum is
// scaled by s[n][g] into the accumulators, as the W4A8 path does with its
// integer sums.
//
// Tile: 128 tokens x 128 channels per 512-thread workgroup, eight wavefronts
// of 32 x 64 (the bf16 activation tile is twice the int8 one, so the token
// side is halved to keep two stages in LDS).  Per group the wavefront runs
// its 8 tiles x 4 steps; step t takes input channels 16j + 8t'.. of half
// t / 2 (t' = t % 2) in both operands.
namespace a16 {

constexpr int BM = 128;
constexpr int kAStride = 2 * kGroup + 16;             // bf16 row of one group, bank-spread
constexpr int kAOff = 0;
constexpr int kBOff = kAOff + BM * kAStride;          // bf16 q - z, [NCB][4 steps][64 lanes][16 B]
constexpr int kSOff = kBOff + NCB * 4 * kBlockBytes;  // scales [NCB][16]
constexpr int kBufBytes = kSOff + NCB * 16 * 4;
constexpr int kAChunks = BM * 2 * kGroup / 16 / kThreads;  // 16-B activation chunks per thread (4)

struct Stage {
  v4i a[kAChunks];
  v4i b;          // 16 packed code bytes: block t/64, lane t%64
  uint32_t zb;    // the byte holding that lane's zero point
  float s;        // scale of channel t%16 of block (t/16)%8
};

struct Offsets {
  uint32_t a[kAChunks];
  uint32_t b, z, s;
  int zshift;
};

__device__ __forceinline__ Offsets make_offsets(const GemmArgs& a, int64_t m0, int64_t cb0,
                                                int64_t NB, int64_t G) {
  const int tid = threadIdx.x;
  Offsets o;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int ch = tid + kThreads * i;  // 16 chunks of 16 B per row and group
    o.a[i] = (uint32_t)((min(m0 + (ch >> 4), a.M - 1) * a.K + (ch & 15) * 8) * 2);
  }
  const int64_t nb = min(cb0 + (tid >> 6), NB - 1);
  o.b = (uint32_t)(nb * G * kBlockBytes + (tid & 63) * 16);
  o.z = (uint32_t)(nb * G * kZeroBlockBytes + ((tid & 15) >> 1));
  o.zshift = (tid & 1) * 4;
  const int64_t nbs = min(cb0 + ((tid >> 4) & (NCB - 1)), NB - 1);
  o.s = (uint32_t)(nbs * G * 16 + (tid & 15));
  return o;
}

__device__ __forceinline__ void load_stage(const GemmArgs& a, const Offsets& o, int64_t g,
                                           Stage& st) {
  const uint8_t* x = static_cast<const uint8_t*>(a.x) + g * kGroup * 2;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) st.a[i] = *reinterpret_cast<const v4i*>(x + o.a[i]);
  st.b = *reinterpret_cast<const v4i*>(a.w.codes + g * kBlockBytes + o.b);
  st.zb = (a.w.zeros + g * kZeroBlockBytes)[o.z];
  st.s = (a.w.scales + g * 16)[o.s];
}

// Four codes (0..15, one per byte) minus a zero point as four bf16, two per
// dword in byte order: q + 16 - z (1..31, no borrow across bytes) converts
// exactly from each unsigned byte, 16 comes off exactly, and small integers
// are exact in bf16 (the float's high half).
__device__ __forceinline__ void codes_to_bf16x2(uint32_t nib4, uint32_t zz, int& lo, int& hi) {
  const uint32_t u = (nib4 + 0x10101010u) - zz;
  const float f0 = (float)(u & 0xFFu) - 16.0f, f1 = (float)((u >> 8) & 0xFFu) - 16.0f;
  const float f2 = (float)((u >> 16) & 0xFFu) - 16.0f, f3 = (float)(u >> 24) - 16.0f;
  lo = (int)__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = (int)__builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// Stage -> LDS: the activation rows as they are, the codes expanded once to
// bf16 q - z in MFMA operand order (block u, step t, lane L), the scales.
__device__ __forceinline__ void store_stage(uint8_t* buf, const Stage& st, int zshift) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int ch = tid + kThreads * i;
    *reinterpret_cast<v4i*>(buf + kAOff + (ch >> 4) * kAStride + (ch & 15) * 16) = st.a[i];
  }
  const uint32_t zz = ((st.zb >> zshift) & 0xFu) * 0x01010101u;
  const int u = tid >> 6, L = tid & 63;
#pragma unroll
  for (int t = 0; t < 4; ++t) {  // step t: nibble half t / 2, code bytes 8 (t % 2) .. + 7
    const int sh = (t >> 1) * 4;
    int b0, b1, b2, b3;
    codes_to_bf16x2(((uint32_t)st.b[2 * (t & 1)] >> sh) & 0x0F0F0F0Fu, zz, b0, b1);
    codes_to_bf16x2(((uint32_t)st.b[2 * (t & 1) + 1] >> sh) & 0x0F0F0F0Fu, zz, b2, b3);
    *reinterpret_cast<v4i*>(buf + kBOff + (u * 4 + t) * kBlockBytes + L * 16) = v4i{b0, b1, b2, b3};
  }
  reinterpret_cast<float*>(buf + kSOff)[tid & (NCB * 16 - 1)] = st.s;
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// One group: fragments from LDS, 8 tiles x 4 bf16 MFMA steps, and the
// group's float sums scaled into the accumulators.
__device__ __forceinline__ void compute_group(const uint8_t* buf, float (&accf)[2][4][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  float sv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sv[u] = reinterpret_cast<const float*>(buf + kSOff)[(wn * 4 + u) * 16 + r16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint8_t* arow = buf + kAOff + (wm * 32 + i * 16 + r16) * kAStride + 32 * j;
    v4i av[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const v4i*>(arow + (t >> 1) * kGroup + (t & 1) * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i bv = *reinterpret_cast<const v4i*>(buf + kBOff + ((wn * 4 + u) * 4 + t) * kBlockBytes + lane * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[t]),
                                                      __builtin_bit_cast(v8bf, bv), acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] += sv[u] * acc[r];
    }
  }
}

__global__ void __launch_bounds__(kThreads)
prefill_a16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][kBufBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r16 = lane & 15, j = lane >> 4;
  const int64_t G = a.K / kGroup;
  const int64_t NB = a.N / kBlockCols;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (NB + NCB - 1) / NCB;
  // tiles and tail slices as in the W4A8 kernel
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t main_tiles = a.tail_split > 1 ? tiles - a.tail_tiles : tiles;
  int64_t t;
  int slice = blockIdx.y, nslices = gridDim.y;
  int64_t wn0 = 0;
  if ((int64_t)blockIdx.x < main_tiles) {
    t = xcd_tile(blockIdx.x, main_tiles);
  } else {
    const int64_t r = blockIdx.x - main_tiles;
    t = main_tiles + r % a.tail_tiles;
    slice = (int)(r / a.tail_tiles);
    nslices = a.tail_split;
    wn0 = a.tail_n0;
  }
  const int64_t ldw = a.N - wn0;
  const int64_t tm = t % tiles_m, tn = t / tiles_m;
  const int64_t m0 = tm * BM, cb0 = tn * NCB;
  const int64_t gb = G * slice / nslices, ge = G * (slice + 1) / nslices;

  float accf[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][u][r] = 0.0f;

  const Offsets off = make_offsets(a, m0, cb0, NB, G);
  Stage s0, s1;
  load_stage(a, off, gb, s0);
  load_stage(a, off, min(gb + 1, ge - 1), s1);
  store_stage(smem[0], s0, off.zshift);
  __syncthreads();
  for (int64_t g = gb; g < ge; g += 2) {
    load_stage(a, off, min(g + 2, ge - 1), s0);
    compute_group(smem[0], accf);
    store_stage(smem[1], s1, off.zshift);
    __syncthreads();
    if (g + 1 >= ge) break;
    load_stage(a, off, min(g + 3, ge - 1), s1);
    compute_group(smem[1], accf);
    store_stage(smem[0], s0, off.zshift);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm * 32 + i * 16 + 4 * j + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t nb = cb0 + wn * 4 + u;
        if (nb >= NB) continue;
        const int64_t n = nb * 16 + r16;
        if (nslices > 1)
          a.workspace[((int64_t)slice * a.M + m) * ldw + n - wn0] = accf[i][u][r];
        else
          a.y[m * a.N + n] = f32_to_bf16_rne(accf[i][u][r]);
      }
    }
}

}  // namespace a16

}  // namespace

namespace {
// Output tile of a prefill kernel: rows (tokens) and 16-channel blocks.
int64_t tile_rows(int tile) { return tile == kTileA16 ? a16::BM : BM; }
int64_t tile_blocks(int tile) { return tile == kTile256x256 ? wide::NCB : NCB; }
int64_t tile_count(int64_t M, int64_t N, int tile) {
  const int64_t bm = tile_rows(tile), ncb = tile_blocks(tile);
  return ((M + bm - 1) / bm) * ((N / kBlockCols + ncb - 1) / ncb);
}
}  // namespace

// 256 x 256 tiles halve the activation bytes per product and cut the fragment
// reads by a quarter, but fewer than one round of them leaves compute units
// idle that 256 x 128 tiles (with their K split) would use.  Measured
// (quantised GEMM, us, 256 x 128 against 256 x 256): M = 2048, K = 3584 ->
// N = 18944 200 / 187; M = 512 -> N = 37888 119 / 107; M = 512 -> N = 18944
// 63 / 73; M = 2048 -> N = 4608 62 / 71.
int prefill_auto_tile(int64_t M, int64_t N, int64_t K) {
  (void)K;
  return tile_count(M, N, kTile256x256) >= (int64_t)device_cus() ? kTile256x256 : kTile256x128;
}

// Split K only while the output tiles leave compute units idle, keeping at
// least two groups per slice.
int prefill_ksplit(int64_t M, int64_t N, int64_t K, int tile) {
  const int64_t tiles = tile_count(M, N, tile);
  const int64_t G = K / kGroup, cus = device_cus();
  int ks = 1;
  while (tiles * ks * 2 <= cus && G >= (int64_t)ks * 2 * 2) ks *= 2;
  return ks;
}

// Measured at M = 512, K = 3584 -> N = 18944 (296 tiles of 256 x 128: one
// round and 40 tiles): with the last 40 tiles as 6 K slices each,
// quantisation + GEMM takes 68.6 us instead of 87 us.
PrefillTail prefill_tail(int64_t M, int64_t N, int64_t K, int tile) {
  const int64_t bm = tile_rows(tile), ncb = tile_blocks(tile);
  const int64_t tiles_m = (M + bm - 1) / bm, tiles_n = (N / kBlockCols + ncb - 1) / ncb;
  const int64_t tiles = tiles_m * tiles_n, cus = device_cus(), G = K / kGroup;
  const PrefillTail none{0, 0, 0};
  if (tiles <= cus || tiles % cus == 0) return none;
  const int64_t cols = (tiles % cus + tiles_m - 1) / tiles_m;  // whole column tiles
  const int64_t tail = cols * tiles_m;
  const int64_t n0 = (tiles_n - cols) * ncb * kBlockCols;
  int64_t s = cus / tail;
  if (s > G / 2) s = G / 2;  // at least two groups per slice
  // 256 x 256 tiles: the tail's channels may instead run over all of K as
  // 256 x 128 half tiles when those fit one round (split -1). The last round
  // then takes about 0.72 of a tile's time (a half tile still loads the whole
  // activation tile), against 1/s of it plus writing and re-reading the
  // slices' float sums, which moved at about 4 TB/s each way. Fitted on
  // MI355X at K = 3584, where a tile took about 67 us: M = 2048, N = 18944
  // (3 slices) ran 190 us split and 182 us in half tiles; M = 512,
  // N = 37888 (6 slices) 109 us split and 116 us in half tiles.
  if (tile == kTile256x256) {
    const int64_t halves = tiles_m * ((N / kBlockCols - n0 / kBlockCols + ncb / 2 - 1) / (ncb / 2));
    if (halves <= cus) {
      const double tile_us = 67.0 * (double)K / 3584.0;
      const double half_us = 0.72 * tile_us;
      double split_us = tile_us;
      if (s >= 2) {
        const double sums = (double)s * (double)M * (double)(N - n0) * 4.0;
        split_us = tile_us / (double)s + 2.0 * sums / 4.0e6;
      }
      if (half_us < split_us) return PrefillTail{-1, tail, n0};
    }
  }
  if (s < 2) return none;
  return PrefillTail{(int)s, tail, n0};
}

hipError_t launch_prefill(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles = tile_count(a.M, a.N, a.wide ? kTile256x256 : kTile256x128);
  if ((a.tail_split > 1 || a.tail_split == -1) &&
      (a.ksplit != 1 || a.tail_tiles <= 0 || a.tail_tiles > tiles))
    return hipErrorInvalidValue;
  if (a.tail_split == -1 && (!a.wide || a.tail_n0 % (wide::NCB * kBlockCols) != 0))
    return hipErrorInvalidValue;
  int64_t wgs = tiles;
  if (a.tail_split > 1) wgs = tiles - a.tail_tiles + a.tail_tiles * a.tail_split;
  if (a.tail_split == -1)  // the tail's channels as 256 x 128 half tiles
    wgs = tiles - a.tail_tiles +
          ((a.M + BM - 1) / BM) * ((a.N / kBlockCols - a.tail_n0 / kBlockCols + NCB - 1) / NCB);
  const dim3 grid((unsigned)wgs, (unsigned)a.ksplit);
  if (a.wide && a.w8) {
    if (a.partials)
      hipLaunchKernelGGL((wide::prefill_wide_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((wide::prefill_wide_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
  } else if (a.wide) {
    if (a.partials)
      hipLaunchKernelGGL((wide::prefill_wide_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((wide::prefill_wide_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
  } else if (a.w8) {
    if (a.partials)
      hipLaunchKernelGGL((prefill_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
  } else if (a.partials) {
    hipLaunchKernelGGL((prefill_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

// W4A16 prefill: K is split (float partials, deterministic reduce) only while
// the output tiles leave compute units idle.
int prefill_a16_ksplit(int64_t M, int64_t N, int64_t K) { return prefill_ksplit(M, N, K, kTileA16); }

hipError_t launch_prefill_a16(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles = tile_count(a.M, a.N, kTileA16);
  if (a.tail_split > 1 && (a.ksplit != 1 || a.tail_tiles <= 0 || a.tail_tiles > tiles))
    return hipErrorInvalidValue;
  const int64_t wgs = a.tail_split > 1 ? tiles - a.tail_tiles + a.tail_tiles * a.tail_split : tiles;
  hipLaunchKernelGGL(a16::prefill_a16_kernel, dim3((unsigned)wgs, (unsigned)a.ksplit),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace w4a8
