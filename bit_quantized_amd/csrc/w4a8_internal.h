// Internal declarations shared by the HIP translation units of libw4a8.
// Device helpers here are used by the kernels only; nothing in this file is
// part of the public ABI (include/w4a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a8 {

constexpr int kGroup = 128;          // input channels per quantisation group
constexpr int kBlockCols = 16;       // output channels per packed block
constexpr int kBlockBytes = 1024;    // 16 channels x 128 codes x 4 bits
constexpr int kZeroBlockBytes = 8;   // 16 zero points x 4 bits

typedef int v4i __attribute__((ext_vector_type(4)));

struct PackedView {
  const uint8_t* codes;   // [N/16][G][1024]
  const uint8_t* zeros;   // [N/16][G][8]
  const float* scales;    // [N/16][G][16]
};

inline int64_t round_up256(int64_t v) { return (v + 255) / 256 * 256; }
inline int64_t zeros_offset(int64_t N, int64_t K) { return round_up256(N * K / 2); }
inline int64_t scales_offset(int64_t N, int64_t K) {
  return round_up256(zeros_offset(N, K) + N * (K / kGroup) / 2);
}
inline int64_t packed_bytes(int64_t N, int64_t K) {
  return scales_offset(N, K) + 4 * N * (K / kGroup);
}
// W8A8 packed weights: int8 codes [N/16][K/128][2 halves][64 lanes][16 B],
// then one float scale per channel.
inline int64_t w8_scales_offset(int64_t N, int64_t K) { return round_up256(N * K); }
inline int64_t w8_packed_bytes(int64_t N, int64_t K) { return w8_scales_offset(N, K) + 4 * N; }

// ---------------------------------------------------------------- device helpers

// Raw byte-buffer descriptors: a load at an offset past `bytes` returns
// zeros and issues no memory request, so a bounds check becomes an offset
// (kOob lies beyond every descriptor) instead of a branch around the load.
constexpr int kBufferWord3 = 0x00020000;  // raw byte buffer, gfx9 descriptor format
constexpr int kNontemporal = 2;           // cache policy bit: nt
constexpr int kOob = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// An integer product chain that starts from kBiasBits instead of zero (a
// group's first MFMA, or a chain of v_dot4) ends at 0x4B400000 + P.  Read as
// a float those bits are exactly 1.5 * 2^23 + P whenever |P| < 2^22 (a
// group product is at most 128 * 127 * 15 < 2^18 in magnitude), and one
// float subtraction returns P exactly: the same value as an int -> float
// conversion, from an instruction that issues at a higher rate.
constexpr int kBiasBits = 0x4B400000;
constexpr v4i kBiasSeed = {kBiasBits, kBiasBits, kBiasBits, kBiasBits};
__device__ __forceinline__ float unbias(int r) { return __int_as_float(r) - 12582912.0f; }

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four unsigned 4-bit codes (one per byte, 0..15) minus a zero point z
// (0..15) as four signed bytes q - z in [-15, 15].  Setting bit 7 of every
// byte first makes each byte >= 128 > z, so the 32-bit subtraction never
// borrows across bytes; flipping bit 7 back maps 128 + v to v mod 256.
__device__ __forceinline__ uint32_t sub_zero_bytes(uint32_t nib4, uint32_t zz) {
  return ((nib4 | 0x80808080u) - zz) ^ 0x80808080u;
}

// Maximum of v over the 64 lanes of a wavefront, in every lane.  Max is
// exact in any order, so the value is that of any reduction tree: DPP moves
// take each 16-lane row to its maximum (quad swaps, half-row mirror, row
// mirror), then the four row maxima are read into scalar registers.
template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float v) {
  const float o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
  return fmaxf(v, o);
}
__device__ __forceinline__ float wave_max64(float v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v = dpp_max_step<0x141>(v);  // row_half_mirror: the other quad of the half-row
  v = dpp_max_step<0x140>(v);  // row_mirror: the other half of the row
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Codes of eight finite activations under a row scale s > 0 with inv the
// correctly rounded 1 / s: rint(x / s) (IEEE quotient, ties to even) clamped
// to [-127, 127], as bytes.  The quotient is taken as x * inv, which differs
// from the IEEE x / s by less than 2.3e-5 for |x / s| <= 127.5 (each is
// within 2 ulp-of-1 relative rounding of the real quotient); the two can
// round to different integers only when the product lies within that
// distance of a boundary n + 1/2, so such elements (|t - rint(t)| > 1/2 -
// 2^-14) are redone with the IEEE quotient.  Adding 1.5 * 2^23 rounds a
// float of magnitude <= 127 to an integer (round to nearest even) whose
// low byte is then the two's-complement code.
__device__ __forceinline__ uint2 quant8_codes(const float* v, float s, float inv) {
  constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
  uint32_t b[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = __builtin_amdgcn_fmed3f(v[i] * inv, -127.0f, 127.0f);
    const float f = t + kRound;
    near |= fabsf(t - (f - kRound)) > 0.5f - 0x1p-14f;
    b[i] = __float_as_uint(f);
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = fminf(fmaxf(rintf(v[i] / s), -127.0f), 127.0f);
      b[i] = static_cast<uint32_t>(static_cast<int32_t>(r));
    }
  }
  // v_perm_b32 picks bytes of {src0:src1}: selector 0..3 = src1, 4..7 = src0
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm(b[4 * h + 1], b[4 * h], 0x0400u);      // b0, b1 low bytes
    const uint32_t hi = __builtin_amdgcn_perm(b[4 * h + 3], b[4 * h + 2], 0x0400u);  // b2, b3 low bytes
    w[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return make_uint2(w[0], w[1]);
}

// v of lane (lane ^ d) for d = 1, 2, 4, 8, within each 16-lane row, by DPP
// moves (no LDS traffic).  Only symmetric lane maps are used, so the result
// does not depend on the direction conventions of shifts: quad permutations
// [1,0,3,2] and [2,3,0,1] for d = 1, 2; for d = 4 a mirror of each 8-lane
// half (p -> 7 - p) and then a reversal of each quad: position p of a half
// reads mirror position 7 - q(p), q(p) = (p & 4) | (3 - (p & 3)), which is
// p ^ 4; for d = 8 a rotation of the 16-lane row by half its length.
__device__ __forceinline__ float lane_xor_in_row(float v, int d) {
  constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kQuadReverse = 0x1B;
  constexpr int kRowHalfMirror = 0x141, kRowRotate8 = 0x128;
  int x = __float_as_int(v);
  if (d == 1) {
    x = __builtin_amdgcn_mov_dpp(x, kQuadSwap1, 0xF, 0xF, true);
  } else if (d == 2) {
    x = __builtin_amdgcn_mov_dpp(x, kQuadSwap2, 0xF, 0xF, true);
  } else if (d == 4) {
    x = __builtin_amdgcn_mov_dpp(x, kRowHalfMirror, 0xF, 0xF, true);
    x = __builtin_amdgcn_mov_dpp(x, kQuadReverse, 0xF, 0xF, true);
  } else {
    x = __builtin_amdgcn_mov_dpp(x, kRowRotate8, 0xF, 0xF, true);
  }
  return __int_as_float(x);
}

// Online Hadamard rotation of one chunk of eight, in place: this thread's
// chunk is chunk (threadIdx.x & 15) of a group of 128 input channels whose
// other 15 chunks sit in the neighbouring threads of the same 16-lane row.
// The group is multiplied by the unnormalised 128 x 128 Walsh-Hadamard
// matrix (Sylvester order) by radix-2 butterflies of increasing stride
// h = 1, ..., 64, each pair (i, i + h) becoming (a + b, a - b): strides below
// 8 inside the chunk, the rest across lanes.  Every element sees the same
// float32 operations in the same order as the straightforward in-place
// transform, so the rotated values are exact reproductions of it.
__device__ __forceinline__ void hadamard_chunk(float* v) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  const int pos = threadIdx.x & 15;
#pragma unroll
  for (int d = 1; d < 16; d *= 2) {  // stride 8 d: the partner chunk is lane ^ d
    const bool upper = (pos & d) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float u = lane_xor_in_row(v[i], d);
      v[i] = upper ? u - v[i] : v[i] + u;
    }
  }
}

// Zero point of column c in a zeros block.
__device__ __forceinline__ uint32_t zero_of(const uint8_t* zblk, int c) {
  uint32_t b = zblk[c >> 1];
  return (c & 1) ? (b >> 4) : (b & 0xFu);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the
// caller (abi.hip) before any of these runs.

hipError_t launch_pack(const uint8_t* q, const uint8_t* z, const float* s, int64_t N, int64_t K,
                       uint8_t* packed, hipStream_t st);
hipError_t launch_pack_into(const uint8_t* q, const uint8_t* z, const float* s, int64_t N_part,
                            int64_t K, uint8_t* packed, int64_t N_total, int64_t n_offset,
                            hipStream_t st);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, uint8_t* q, uint8_t* z,
                         float* s, hipStream_t st);
// hadamard: rotate every group of 128 by the unnormalised Walsh-Hadamard
// matrix before quantising (the online rotation of QuaRot).
hipError_t launch_quant(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* qa, float* sa,
                        hipStream_t st, bool hadamard = false);
// The same codes and scales for 1 <= M <= 16 rows (K <= 65536), qa in the
// [K / 16][16 rows][16 B] layout the M <= 16 GEMM reads as MFMA operands
// (16 K bytes; rows M..15 left unwritten).
hipError_t launch_quant_tiled(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* qa,
                              float* sa, hipStream_t st, bool hadamard = false);
hipError_t launch_w8_pack(const int8_t* qw, const float* sw, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t st);
hipError_t launch_w8_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* qw, float* sw,
                            hipStream_t st);

struct GemmArgs {
  const int8_t* qa;       // quantised activations [M][K] (null when x is quantised in-kernel)
  const float* sa;        // per-token scales [M]
  const void* x;          // raw activations quantised in-kernel (GEMV; skinny when it fuses), else null
  int x_dtype;            // W4A8_BF16 / W4A8_F32 when x is set
  PackedView w;
  int64_t M, N, K;
  uint16_t* y;            // may be null in debug mode
  int32_t* partials;      // debug only, may be null
  int64_t m_begin, m_end; // debug row window
  float* workspace;       // split-K partial sums [ksplit][M][N]
  float* sa_ws;           // fused quant + split-K: the scale, for the reduction
  int ksplit;
  int cb, ks;             // GEMV: workgroups along N, wavefronts per workgroup
  int cb_q, cb_r;         // GEMV: N/16 = cb_q * cb + cb_r (set by the launcher)
  int gq, gr;             // skinny: G = gq * (ksplit * 16) + gr (set by the launcher)
  bool w8;                // W8A8 weights (codes [N/16][G][2][1024], scales [N]); partials
                          // are then the int32 totals [m_end-m_begin][N]
  // prefill: the last tail_tiles tiles (channels >= tail_n0) each run as
  // tail_split K slices into workspace [tail_split][M][N - tail_n0]; or, with
  // tail_split == -1 (256 x 256 tiles), as 256 x 128 half tiles
  int tail_split = 0;
  int64_t tail_tiles = 0, tail_n0 = 0;
  // prefill (W4A8): 256 x 256 output tiles instead of 256 x 128
  bool wide = false;
  // the GEMV's in-kernel quantisation (bf16 / f32 token, not debug): rotate
  // each group of 128 by the Walsh-Hadamard matrix first (hadamard_chunk), as
  // w4a8_quant_act_hadamard
  bool hadamard = false;
  // qa in the [K / 16][16 rows][16 B] layout of launch_quant_tiled (skinny
  // kernel, 12 <= M <= 16, no debug)
  bool qa_tiled = false;
};

// Largest K the GEMV keeps in LDS (activation codes + per-quarter sums).
constexpr int64_t kGemvMaxK = 32768;
// The prefill kernel addresses the activation and code planes with 32-bit
// per-thread offsets.
constexpr int64_t kPrefillMaxBytes = ((int64_t)1 << 31) - 1;

struct GemvShape {
  int cb, ks, ksplit;
};
int device_cus();  // compute units of the current device (cached)
GemvShape gemv_shape(int64_t N, int64_t K);
bool gemv_shape_ok(int64_t N, int64_t K, const GemvShape& s);
int skinny_ksplit(int64_t M, int64_t N, int64_t K);
// Whether the 2 <= M <= 16 kernel can quantise raw activations of this shape
// itself (GemmArgs::x set); x_dtype as in GemmArgs.
bool skinny_fuses_quant(int64_t M, int64_t N, int64_t K, int x_dtype);
// Output tiles of the prefill kernels: 256 tokens x 128 channels (W4A8 and
// W8A8), 256 x 256 (W4A8, large grids), 128 x 128 (W4A16).
enum PrefillTile { kTile256x128 = 0, kTile256x256 = 1, kTileA16 = 2 };
// The W4A8 tile for an M x N x K product: 256 x 256 when its tiles fill at
// least one round of the compute units, else 256 x 128.
int prefill_auto_tile(int64_t M, int64_t N, int64_t K);
int prefill_ksplit(int64_t M, int64_t N, int64_t K, int tile);
// Prefill grid beyond prefill_ksplit: when the tiles fill R whole rounds of
// the compute units plus a partial one, the partial round's tiles (rounded up
// to whole column tiles) run as `split` K slices each, so the last round is
// 1/split as long.  split 0: no tail split.  split -1 (256 x 256 tiles
// only): the partial round's channels (from n0) run as 256 x 128 half tiles
// over all of K instead, in the same launch.
struct PrefillTail {
  int split;
  int64_t tiles, n0;
};
PrefillTail prefill_tail(int64_t M, int64_t N, int64_t K, int tile);
hipError_t launch_gemv(const GemmArgs& a, hipStream_t st);
// W4A16 (bf16 token in GemmArgs::x, M == 1) on the GEMV kernel; same grid rules.
hipError_t launch_gemv_a16(const GemmArgs& a, hipStream_t st);
hipError_t launch_skinny(GemmArgs a, hipStream_t st);
// W4A16 (bf16 activations in GemmArgs::x, x_dtype 0) on the M <= 16 kernel:
// its K split, chunks per thread and dynamic LDS; ksplit 0 when no split fits.
struct A16Plan {
  int ksplit;
  int npt;
  size_t lds;
};
A16Plan skinny_a16_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_skinny_a16(GemmArgs a, hipStream_t st);
// 1 <= M <= 16 on the weight-streaming grid of stream.hip (W4A8, quantised
// activations, N / 16 >= compute units, K <= 4096): C workgroups of one
// pass over K (S == 1), `lds` bytes of staged activations each; C == 0 where
// the grid does not apply.
struct StreamPlan {
  int C, S;
  size_t lds;
};
StreamPlan stream_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_stream(const GemmArgs& a, hipStream_t st);
hipError_t launch_prefill(const GemmArgs& a, hipStream_t st);
// W4A16 prefill (bf16 activations in GemmArgs::x): K split and launch.
int prefill_a16_ksplit(int64_t M, int64_t N, int64_t K);
hipError_t launch_prefill_a16(const GemmArgs& a, hipStream_t st);
// ws is [ksplit][M][N - n0]: the columns [n0, N) of y (n0 = 0: all).
hipError_t launch_splitk_reduce(const float* ws, int ksplit, const float* sa, int64_t M,
                                int64_t N, uint16_t* y, hipStream_t st, int64_t n0 = 0);
// Sets the thread's w4a8_last_error() message (abi.hip); returns status.
int report_error(int status, const char* msg);

// on-device peak probes (include/w4a8_peaks.h)
hipError_t launch_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                   hipStream_t st);
hipError_t launch_peak_mfma_i8(int iters, int32_t* sink, uint64_t* clocks, int blocks,
                               hipStream_t st);
hipError_t launch_w8_splitk_reduce(const int32_t* ws, int ksplit, const float* sa, const float* sw,
                                   int64_t M, int64_t N, uint16_t* y, int32_t* totals,
                                   int64_t m_begin, int64_t m_end, hipStream_t st,
                                   int64_t n0 = 0);

}  // namespace w4a8
