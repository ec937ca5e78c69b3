// Public C ABI (include/w4a8.h): host-side validation, path choice and
// launches.  Every check runs before anything is enqueued, so a rejected call
// launches nothing and writes nothing.  No C++ exception crosses the ABI.
//
// "The 4-bit CPU path", section "The weight layout, measured": a shape that
// does not tile the packed block is refused instead of being misread.
// "Serve a pre-quantized int8 weight-only DiT ...", comment "Amendment ...":
// a path is only advertised where its kernel runs; the debug entry point lets
// tests force every path at every bucket edge.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/w4a8.h"
#include "../../include/w4a8_peaks.h"
#include "w4a8_internal.h"

using namespace w4a8;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return W4A8_OK;
}

}  // namespace

// Records the message w4a8_last_error() returns for a failing call made from
// another translation unit of the library; returns status.
int w4a8::report_error(int status, const char* msg) { return fail(status, "%s", msg); }

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_weight_shape(int64_t N, int64_t K, int32_t group) {
  if (N <= 0 || K <= 0) return fail(W4A8_ERR_INVALID_ARG, "N=%lld and K=%lld must be positive",
                                    (long long)N, (long long)K);
  if (group != kGroup)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "group=%d unsupported (only 128)", (int)group);
  if (K % kGroup)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (N % kBlockCols)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE,
                "N=%lld is not a multiple of 16 (no partial channel blocks)", (long long)N);
  if (N > (int64_t)1 << 26 || K > (int64_t)1 << 24 || N * K > ((int64_t)1 << 40))
    return fail(W4A8_ERR_INVALID_ARG, "N=%lld K=%lld too large", (long long)N, (long long)K);
  return W4A8_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(W4A8_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Overlap test for [p, p+n) and [q, q+m).
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

int pick_path(int64_t M, int64_t K) {
  if (M == 1 && K <= kGemvMaxK) return W4A8_PATH_GEMV;
  if (M <= 16) return W4A8_PATH_SKINNY;
  return W4A8_PATH_PREFILL;
}

// The prefill kernels address the activation plane with 32-bit offsets.
// Taller matrices run as consecutive row chunks on the stream, each chunk at
// most kPrefillMaxBytes of activations (whole 256-row tiles where a tile
// fits); 0 when a single row is already too long.
int64_t prefill_chunk_rows(int64_t K, int64_t bytes_per_value) {
  const int64_t rows = kPrefillMaxBytes / (K * bytes_per_value);
  return rows >= 256 ? rows / 256 * 256 : rows;
}

// Row window [m_begin, m_end) of a debug call, restricted to the chunk of
// rows [m0, m0 + mc): the chunk-local window and the row offset of its first
// row in the caller's partials (empty window: begin == end == 0).
struct ChunkWindow {
  int64_t begin, end, out_row;
};
ChunkWindow chunk_window(int64_t m_begin, int64_t m_end, int64_t m0, int64_t mc) {
  const int64_t b = m_begin > m0 ? m_begin : m0;
  const int64_t e = m_end < m0 + mc ? m_end : m0 + mc;
  if (b >= e) return ChunkWindow{0, 0, 0};
  return ChunkWindow{b - m0, e - m0, b - m_begin};
}

// The prefill's tail split for a tile width (none when the rows run as
// several chunks) and the workspace bytes its slices take ([split][M][N -
// n0], 4 bytes each).
PrefillTail prefill_tail_for(int64_t M, int64_t N, int64_t K, int tile) {
  if (M > prefill_chunk_rows(K, 1)) return PrefillTail{0, 0, 0};
  return prefill_tail(M, N, K, tile);
}
size_t tail_workspace(const PrefillTail& t, int64_t M, int64_t N) {
  if (t.split < 2) return 0;  // none, or half tiles (split -1)
  return ((size_t)t.split * (size_t)M * (size_t)(N - t.n0) * 4 + 255) / 256 * 256;
}

// Whether w4a8_linear runs 2 <= M <= 16 as one launch (the skinny kernel
// quantising the rows itself): only where the balanced grid does not apply,
// so that the linear and quant + w4a8_gemm run the same GEMM kernel.
bool linear_fuses_quant(int64_t M, int64_t N, int64_t K, int x_dtype) {
  return stream_plan(M, N, K).C == 0 && skinny_fuses_quant(M, N, K, x_dtype);
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

// Whether the two-launch linears hand the skinny kernel its codes in the
// tiled [K / 16][16 rows][16 B] layout (12 <= M <= 16, where the row-major
// codes cost the kernel eight lane exchanges per unit): the same codes and
// the same GEMM arithmetic, so the output is bitwise that of quant + gemm.
// Measured at K = 18944 -> N = 3584: 18.5 -> 16.9 us at M = 16, 16.2 ->
// 15.9 at M = 12; slower below (15.6 -> 15.8 at M = 10), where the lanes
// of the absent rows no longer cost their exchanges.
bool linear_tiles_codes(int64_t M, int64_t N, int64_t K) {
  return M >= 12 && M <= 16 && K <= 65536 && pick_path(M, K) == W4A8_PATH_SKINNY &&
         stream_plan(M, N, K).C == 0;
}

// Bytes of the codes region of a two-launch linear's workspace.
size_t linear_codes_bytes(int64_t M, int64_t N, int64_t K) {
  return round256((size_t)(linear_tiles_codes(M, N, K) ? 16 : M) * K);
}

// `tile` (PrefillTile) matters for the PREFILL path only.
int ksplit_for(int path, int64_t M, int64_t N, int64_t K, int tile) {
  if (path == W4A8_PATH_GEMV) return gemv_shape(N, K).ksplit;
  if (path == W4A8_PATH_SKINNY) {
    return stream_plan(M, N, K).C > 0 ? 1 : skinny_ksplit(M, N, K);
  }
  if (path == W4A8_PATH_PREFILL) return prefill_ksplit(M, N, K, tile);
  return 1;
}

// Split-K partial sums [ksplit][M][N] float, then (GEMV only) one 256-byte
// slot for the scale the fused quantiser computes.
size_t workspace_for(int path, int64_t M, int64_t N, int64_t K, int tile) {
  const int ks = ksplit_for(path, M, N, K, tile);
  if (ks <= 1)
    return path == W4A8_PATH_PREFILL ? tail_workspace(prefill_tail_for(M, N, K, tile), M, N) : 0;
  size_t b = (size_t)ks * (size_t)M * (size_t)N * sizeof(float);
  b = (b + 255) / 256 * 256;
  return path == W4A8_PATH_GEMV ? b + 256 : b;
}

// The most any path (and either prefill tile width, which the debug entry
// point can force) needs.
size_t gemm_workspace_any(int64_t M, int64_t N, int64_t K) {
  size_t need = 0;
  for (int p = W4A8_PATH_GEMV; p <= W4A8_PATH_PREFILL; ++p) {
    if (p == W4A8_PATH_GEMV && (M != 1 || K > kGemvMaxK)) continue;
    if (p == W4A8_PATH_SKINNY && M > 16) continue;
    for (int tile : {kTile256x128, kTile256x256}) {
      const size_t w = workspace_for(p, M, N, K, tile);
      if (w > need) need = w;
    }
  }
  return need;
}


// Activations for a GEMM: either quantised (qa, sa) or raw x that the M == 1
// GEMV quantises in its prologue.
struct ActIn {
  const int8_t* qa;
  const float* sa;
  const void* x;
  int x_dtype;
  bool tiled = false;  // qa in the layout of launch_quant_tiled
};

int run_gemm(const ActIn& act, const void* packed, size_t packed_bytes_, int64_t M, int64_t N,
             int64_t K, int32_t group, int32_t path, int64_t m_begin, int64_t m_end,
             int32_t* partials, uint16_t* y, void* workspace, size_t workspace_bytes,
             void* stream, bool debug, bool validate_only = false, bool hadamard = false) {
  int rc = check_weight_shape(N, K, group);
  if (rc) return rc;
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  const bool fused = act.x != nullptr;
  if (!packed || (!fused && (!act.qa || !act.sa)))
    return fail(W4A8_ERR_INVALID_ARG, "null input pointer");
  if (!debug && !validate_only && !y) return fail(W4A8_ERR_INVALID_ARG, "null output pointer");
  if (!aligned16(packed) || (y && !aligned16(y)) ||
      (!fused && (!aligned16(act.qa) || !aligned16(act.sa))) || (fused && !aligned16(act.x)))
    return fail(W4A8_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
  const size_t need = (size_t)packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  if (path == W4A8_PATH_AUTO) path = pick_path(M, K);
  int tile = -1;  // prefill tile width: forced by the debug-only paths, else by shape
  if (path == W4A8_PATH_PREFILL_N128 || path == W4A8_PATH_PREFILL_N256) {
    if (!debug)
      return fail(W4A8_ERR_INVALID_ARG, "path %d is accepted by w4a8_gemm_debug only", (int)path);
    tile = path == W4A8_PATH_PREFILL_N256 ? kTile256x256 : kTile256x128;
    path = W4A8_PATH_PREFILL;
  }
  if (path < W4A8_PATH_GEMV || path > W4A8_PATH_PREFILL)
    return fail(W4A8_ERR_INVALID_ARG, "unknown path %d", (int)path);
  if (path == W4A8_PATH_PREFILL && tile < 0) tile = prefill_auto_tile(M, N, K);
  if (path == W4A8_PATH_GEMV && M != 1)
    return fail(W4A8_ERR_INVALID_ARG, "GEMV path needs M == 1 (M=%lld)", (long long)M);
  if (path == W4A8_PATH_GEMV && K > kGemvMaxK)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "GEMV path needs K <= %lld (K=%lld)",
                (long long)kGemvMaxK, (long long)K);
  if (path == W4A8_PATH_SKINNY && M > 16)
    return fail(W4A8_ERR_INVALID_ARG, "SKINNY path needs M <= 16 (M=%lld)", (long long)M);
  if (path == W4A8_PATH_PREFILL && (prefill_chunk_rows(K, 1) == 0 || N * K / 2 > kPrefillMaxBytes))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE,
                "PREFILL path addresses a row of activations and the codes with 32-bit offsets "
                "(K=%lld, N*K/2=%lld, limit %lld)",
                (long long)K, (long long)(N * K / 2), (long long)kPrefillMaxBytes);
  if (fused && path != W4A8_PATH_GEMV &&
      !(path == W4A8_PATH_SKINNY && linear_fuses_quant(M, N, K, act.x_dtype) && !debug))
    return fail(W4A8_ERR_INVALID_ARG, "no in-kernel quantisation for this path and shape");
  if (act.tiled && (fused || debug || path != W4A8_PATH_SKINNY || !linear_tiles_codes(M, N, K)))
    return fail(W4A8_ERR_INVALID_ARG, "tiled codes are read by the 12 <= M <= 16 skinny kernel only");
  const size_t qa_bytes = (size_t)(act.tiled ? 16 : M) * K;
  if (debug) {
    if (m_begin < 0 || m_end > M || m_begin > m_end)
      return fail(W4A8_ERR_INVALID_ARG, "row window [%lld, %lld) outside [0, %lld)",
                  (long long)m_begin, (long long)m_end, (long long)M);
    if (partials && !aligned16(partials))
      return fail(W4A8_ERR_MISALIGNED, "partials must be 16-byte aligned");
  }
  const int ks = ksplit_for(path, M, N, K, tile);
  const size_t ws_need = workspace_for(path, M, N, K, tile);
  if (ws_need && (!workspace || workspace_bytes < ws_need))
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                ws_need);
  if (ws_need && !aligned16(workspace))
    return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const size_t ybytes = (size_t)M * (size_t)N * 2;
  const size_t xbytes = (size_t)M * K * (act.x_dtype == W4A8_F32 ? 4 : 2);
  if (y && ((!fused && (overlaps(y, ybytes, act.qa, qa_bytes) ||
                        overlaps(y, ybytes, act.sa, (size_t)M * 4))) ||
            (fused && overlaps(y, ybytes, act.x, xbytes)) || overlaps(y, ybytes, packed, need) ||
            (ws_need && overlaps(y, ybytes, workspace, ws_need))))
    return fail(W4A8_ERR_INVALID_ARG, "output aliases an input or the workspace");
  if (validate_only) return ok();

  const uint8_t* base = static_cast<const uint8_t*>(packed);
  GemmArgs a;
  a.qa = act.qa;
  a.sa = act.sa;
  a.x = act.x;
  a.x_dtype = act.x_dtype;
  a.w.codes = base;
  a.w.zeros = base + zeros_offset(N, K);
  a.w.scales = reinterpret_cast<const float*>(base + scales_offset(N, K));
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = y;
  a.partials = debug ? partials : nullptr;
  a.m_begin = debug ? m_begin : 0;
  a.m_end = debug ? m_end : 0;
  a.workspace = static_cast<float*>(workspace);
  a.sa_ws = nullptr;
  a.ksplit = ks;
  a.cb = a.ks = 0;
  a.w8 = false;
  a.wide = path == W4A8_PATH_PREFILL && tile == kTile256x256;
  a.hadamard = fused && hadamard;
  a.qa_tiled = act.tiled;
  const float* sa_for_reduce = act.sa;
  if (path == W4A8_PATH_GEMV) {
    const GemvShape gs = gemv_shape(N, K);
    if (!gemv_shape_ok(N, K, gs))
      return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "no GEMV grid for N=%lld K=%lld", (long long)N,
                  (long long)K);
    a.cb = gs.cb;
    a.ks = gs.ks;
    if (fused && ks > 1) {
      a.sa_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws_need - 256);
      sa_for_reduce = a.sa_ws;
    }
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  hipError_t e;
  if (path == W4A8_PATH_PREFILL) {
    // row chunks (one chunk unless M*K exceeds the 32-bit offsets); a split
    // K reuses the front of the workspace, chunk after chunk on the stream
    const int64_t rows = prefill_chunk_rows(K, 1);
    const int64_t G = K / kGroup;
    const PrefillTail tail = ks > 1 ? PrefillTail{0, 0, 0} : prefill_tail_for(M, N, K, tile);
    a.tail_split = tail.split;
    a.tail_tiles = tail.tiles;
    a.tail_n0 = tail.n0;
    e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += rows) {
      const int64_t mc = M - m0 < rows ? M - m0 : rows;
      GemmArgs c = a;
      c.qa = a.qa + m0 * K;
      c.sa = a.sa + m0;
      c.M = mc;
      c.y = y ? y + m0 * N : nullptr;
      if (a.partials) {
        const ChunkWindow w = chunk_window(a.m_begin, a.m_end, m0, mc);
        c.m_begin = w.begin;
        c.m_end = w.end;
        c.partials = w.begin < w.end ? a.partials + w.out_row * N * G : nullptr;
      }
      e = launch_prefill(c, st);
      if (e == hipSuccess && ks > 1 && c.y)
        e = launch_splitk_reduce(c.workspace, ks, c.sa, mc, N, c.y, st);
      if (e == hipSuccess && tail.split > 1 && c.y)
        e = launch_splitk_reduce(c.workspace, tail.split, c.sa, mc, N, c.y, st, tail.n0);
    }
    return device_status(e, "gemm launch");
  }
  if (path == W4A8_PATH_GEMV)
    e = launch_gemv(a, st);
  else if (!fused && stream_plan(M, N, K).C > 0)
    e = launch_stream(a, st);
  else
    e = launch_skinny(a, st);
  if (e == hipSuccess && ks > 1 && y)
    e = launch_splitk_reduce(a.workspace, ks, sa_for_reduce, M, N, y, st);
  return device_status(e, "gemm launch");
}

// Workspace of w4a8_linear: the fused GEMV's own, or quantised activations
// (qa, sa) followed by the GEMM's workspace.
size_t linear_workspace(int64_t M, int64_t N, int64_t K) {
  if (pick_path(M, K) == W4A8_PATH_GEMV) return workspace_for(W4A8_PATH_GEMV, M, N, K, 0);
  return linear_codes_bytes(M, N, K) + round256((size_t)M * 4) + gemm_workspace_any(M, N, K);
}

// ------------------------------------------------------------------ W4A16

// The GEMV serves W4A16 at M == 1 when the token and its quarter sums fit LDS
// and the grid fits the kernel's tables.
bool a16_gemv_ok(int64_t M, int64_t N, int64_t K) {
  return M == 1 && K <= kGemvMaxK && gemv_shape_ok(N, K, gemv_shape(N, K));
}

int a16_ksplit(int path, int64_t M, int64_t N, int64_t K) {
  if (path == W4A8_PATH_GEMV) return gemv_shape(N, K).ksplit;
  return path == W4A8_PATH_SKINNY ? skinny_a16_plan(M, N, K).ksplit : prefill_a16_ksplit(M, N, K);
}

// The W4A16 prefill's tail split (none when the rows run as several chunks).
PrefillTail a16_tail_for(int64_t M, int64_t N, int64_t K) {
  if (M > prefill_chunk_rows(K, 2)) return PrefillTail{0, 0, 0};
  return prefill_tail(M, N, K, kTileA16);
}

size_t a16_workspace_for(int path, int64_t M, int64_t N, int64_t K) {
  const int ks = a16_ksplit(path, M, N, K);
  if (ks <= 1) return path == W4A8_PATH_PREFILL ? tail_workspace(a16_tail_for(M, N, K), M, N) : 0;
  return round256((size_t)ks * (size_t)M * (size_t)N * 4);
}

// M <= 16 takes the M <= 16 kernel whenever it has a plan (it beat the
// 128-token prefill tiles at every shape measured: M = 16, K = 18944 -> N =
// 3584 23 us against 34 us; K = 3584 -> N = 18944 34 us against 42 us).
int pick_a16_path(int64_t M, int64_t N, int64_t K) {
  if (a16_gemv_ok(M, N, K)) return W4A8_PATH_GEMV;
  if (M <= 16 && skinny_a16_plan(M, N, K).ksplit > 0) return W4A8_PATH_SKINNY;
  return W4A8_PATH_PREFILL;
}

size_t a16_workspace_any(int64_t M, int64_t N, int64_t K) {
  size_t need = a16_workspace_for(W4A8_PATH_PREFILL, M, N, K);
  if (M <= 16 && skinny_a16_plan(M, N, K).ksplit > 0) {
    const size_t w = a16_workspace_for(W4A8_PATH_SKINNY, M, N, K);
    if (w > need) need = w;
  }
  if (a16_gemv_ok(M, N, K)) {
    const size_t w = a16_workspace_for(W4A8_PATH_GEMV, M, N, K);
    if (w > need) need = w;
  }
  return need;
}

int run_a16(const uint16_t* x, const void* packed, size_t packed_bytes_, int64_t M, int64_t N,
            int64_t K, int32_t group, int32_t path, uint16_t* y, void* workspace,
            size_t workspace_bytes, void* stream) {
  int rc = check_weight_shape(N, K, group);
  if (rc) return rc;
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  if (!x || !packed || !y) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(packed) || !aligned16(y))
    return fail(W4A8_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
  const size_t need = (size_t)packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  if (path == W4A8_PATH_AUTO) path = pick_a16_path(M, N, K);
  if (path == W4A8_PATH_SKINNY && (M > 16 || skinny_a16_plan(M, N, K).ksplit == 0))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "no W4A16 M <= 16 plan for M=%lld K=%lld",
                (long long)M, (long long)K);
  if (path == W4A8_PATH_GEMV && !a16_gemv_ok(M, N, K))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "no W4A16 GEMV plan for M=%lld N=%lld K=%lld",
                (long long)M, (long long)N, (long long)K);
  if (path != W4A8_PATH_GEMV && path != W4A8_PATH_SKINNY && path != W4A8_PATH_PREFILL)
    return fail(W4A8_ERR_INVALID_ARG, "W4A16 paths are GEMV, SKINNY and PREFILL (got %d)",
                (int)path);
  if (path == W4A8_PATH_PREFILL && (prefill_chunk_rows(K, 2) == 0 || N * K / 2 > kPrefillMaxBytes))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE,
                "PREFILL path addresses a row of activations and the codes with 32-bit offsets");
  const int ks = a16_ksplit(path, M, N, K);
  const size_t ws_need = a16_workspace_for(path, M, N, K);
  if (ws_need && (!workspace || workspace_bytes < ws_need))
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                ws_need);
  if (ws_need && !aligned16(workspace))
    return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const size_t ybytes = (size_t)M * (size_t)N * 2, xbytes = (size_t)M * (size_t)K * 2;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, packed, need) ||
      (ws_need && (overlaps(y, ybytes, workspace, ws_need) ||
                   overlaps(workspace, ws_need, x, xbytes) ||
                   overlaps(workspace, ws_need, packed, need))))
    return fail(W4A8_ERR_INVALID_ARG, "output or workspace aliases another buffer");
  const uint8_t* base = static_cast<const uint8_t*>(packed);
  GemmArgs a;
  a.qa = nullptr;
  a.sa = nullptr;
  a.x = x;
  a.x_dtype = W4A8_BF16;
  a.w.codes = base;
  a.w.zeros = base + zeros_offset(N, K);
  a.w.scales = reinterpret_cast<const float*>(base + scales_offset(N, K));
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = y;
  a.partials = nullptr;
  a.m_begin = a.m_end = 0;
  a.workspace = static_cast<float*>(workspace);
  a.sa_ws = nullptr;
  a.ksplit = ks;
  a.cb = a.ks = 0;
  a.w8 = false;
  if (path == W4A8_PATH_GEMV) {
    const GemvShape gs = gemv_shape(N, K);
    a.cb = gs.cb;
    a.ks = gs.ks;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (path == W4A8_PATH_PREFILL) {
    // row chunks, as for W4A8 (bf16 rows: two bytes per value)
    const int64_t rows = prefill_chunk_rows(K, 2);
    const PrefillTail tail = ks > 1 ? PrefillTail{0, 0, 0} : a16_tail_for(M, N, K);
    a.tail_split = tail.split;
    a.tail_tiles = tail.tiles;
    a.tail_n0 = tail.n0;
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += rows) {
      const int64_t mc = M - m0 < rows ? M - m0 : rows;
      GemmArgs c = a;
      c.x = x + m0 * K;
      c.M = mc;
      c.y = y + m0 * N;
      e = launch_prefill_a16(c, st);
      if (e == hipSuccess && ks > 1) e = launch_splitk_reduce(c.workspace, ks, nullptr, mc, N, c.y, st);
      if (e == hipSuccess && tail.split > 1)
        e = launch_splitk_reduce(c.workspace, tail.split, nullptr, mc, N, c.y, st, tail.n0);
    }
    return device_status(e, "w4a16 launch");
  }
  hipError_t e = path == W4A8_PATH_GEMV ? launch_gemv_a16(a, st) : launch_skinny_a16(a, st);
  if (e == hipSuccess && ks > 1) e = launch_splitk_reduce(a.workspace, ks, nullptr, M, N, y, st);
  return device_status(e, "w4a16 launch");
}

// ------------------------------------------------------------------ W8A8

// Exact int32 totals need |sum_k qa*qw| <= 127 * 127 * K < 2^31.
constexpr int64_t kW8MaxK = 131072;

int check_w8_shape(int64_t N, int64_t K) {
  int rc = check_weight_shape(N, K, kGroup);
  if (rc) return rc;
  if (K > kW8MaxK)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE,
                "W8A8 keeps exact int32 totals, so K <= %lld (K=%lld)", (long long)kW8MaxK,
                (long long)K);
  return W4A8_OK;
}

// The GEMV serves W8A8 at M == 1 when the token fits its LDS and the grid its
// tables (the same rule as W4A8).
bool w8_gemv_ok(int64_t M, int64_t N, int64_t K) {
  return M == 1 && K <= kGemvMaxK && gemv_shape_ok(N, K, gemv_shape(N, K));
}

int pick_w8_path(int64_t M, int64_t N, int64_t K) {
  if (w8_gemv_ok(M, N, K)) return W4A8_PATH_GEMV;
  return M <= 16 ? W4A8_PATH_SKINNY : W4A8_PATH_PREFILL;
}

// w8a8_linear's two-launch route at 14 <= M <= 16 hands the M <= 16 kernel
// the tiled codes, as the W4A8 linear does (linear_tiles_codes).  Measured
// at K = 18944 -> N = 3584: 22.2 -> 20.9 us at M = 16, but 19.4 -> 19.7 at
// M = 12 (the W8A8 kernel does less arithmetic per unit, so the exchanges
// the layout saves weigh less than the absent rows' loads).
bool w8_linear_tiles_codes(int64_t M, int64_t N, int64_t K) {
  return M >= 14 && M <= 16 && K <= 65536 && pick_w8_path(M, N, K) == W4A8_PATH_SKINNY;
}
size_t w8_linear_codes_bytes(int64_t M, int64_t N, int64_t K) {
  return round256((size_t)(w8_linear_tiles_codes(M, N, K) ? 16 : M) * K);
}

int w8_ksplit(int path, int64_t M, int64_t N, int64_t K) {
  if (path == W4A8_PATH_GEMV) return gemv_shape(N, K).ksplit;
  return path == W4A8_PATH_SKINNY ? skinny_ksplit(M, N, K)
                                  : prefill_ksplit(M, N, K, prefill_auto_tile(M, N, K));
}

// int32 split-K partials [ksplit][M][N], then (GEMV only) one 256-byte slot
// for the scale the fused quantiser computes.  The prefill takes the same
// tile width as W4A8 (256 x 256 when those tiles fill a round).
size_t w8_workspace_for(int path, int64_t M, int64_t N, int64_t K) {
  const int ks = w8_ksplit(path, M, N, K);
  if (ks <= 1)
    return path == W4A8_PATH_PREFILL
               ? tail_workspace(prefill_tail_for(M, N, K, prefill_auto_tile(M, N, K)), M, N)
               : 0;
  return round256((size_t)ks * (size_t)M * (size_t)N * 4) + (path == W4A8_PATH_GEMV ? 256 : 0);
}

size_t w8_gemm_workspace_any(int64_t M, int64_t N, int64_t K) {
  size_t need = w8_workspace_for(W4A8_PATH_PREFILL, M, N, K);
  if (M <= 16) {
    const size_t w = w8_workspace_for(W4A8_PATH_SKINNY, M, N, K);
    if (w > need) need = w;
  }
  if (w8_gemv_ok(M, N, K)) {
    const size_t w = w8_workspace_for(W4A8_PATH_GEMV, M, N, K);
    if (w > need) need = w;
  }
  return need;
}

size_t w8_linear_workspace(int64_t M, int64_t N, int64_t K) {
  return w8_linear_codes_bytes(M, N, K) + round256((size_t)M * 4) + w8_gemm_workspace_any(M, N, K);
}

int run_w8_gemm(const ActIn& act, const void* packed, size_t packed_bytes_, int64_t M, int64_t N,
                int64_t K, int32_t path, int64_t m_begin, int64_t m_end, int32_t* totals,
                uint16_t* y, void* workspace, size_t workspace_bytes, void* stream, bool debug,
                bool validate_only = false) {
  int rc = check_w8_shape(N, K);
  if (rc) return rc;
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  const bool fused = act.x != nullptr;
  if (!packed || (!fused && (!act.qa || !act.sa)))
    return fail(W4A8_ERR_INVALID_ARG, "null input pointer");
  if (!debug && !validate_only && !y) return fail(W4A8_ERR_INVALID_ARG, "null output pointer");
  if (!aligned16(packed) || (y && !aligned16(y)) ||
      (!fused && (!aligned16(act.qa) || !aligned16(act.sa))) || (fused && !aligned16(act.x)))
    return fail(W4A8_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
  const size_t need = (size_t)w8_packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  if (path == W4A8_PATH_AUTO) path = pick_w8_path(M, N, K);
  if (path != W4A8_PATH_GEMV && path != W4A8_PATH_SKINNY && path != W4A8_PATH_PREFILL)
    return fail(W4A8_ERR_INVALID_ARG,
                "W8A8 paths are GEMV (M == 1), SKINNY (M <= 16) and PREFILL (got %d)", (int)path);
  if (path == W4A8_PATH_GEMV && !w8_gemv_ok(M, N, K))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "no W8A8 GEMV plan for M=%lld N=%lld K=%lld",
                (long long)M, (long long)N, (long long)K);
  if (path == W4A8_PATH_SKINNY && M > 16)
    return fail(W4A8_ERR_INVALID_ARG, "SKINNY path needs M <= 16 (M=%lld)", (long long)M);
  if (path == W4A8_PATH_PREFILL && (prefill_chunk_rows(K, 1) == 0 || N * K > kPrefillMaxBytes))
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE,
                "PREFILL path addresses a row of activations and the codes with 32-bit offsets "
                "(K=%lld, N*K=%lld, limit %lld)",
                (long long)K, (long long)(N * K), (long long)kPrefillMaxBytes);
  if (fused && (debug || !(path == W4A8_PATH_GEMV ||
                            (path == W4A8_PATH_SKINNY && skinny_fuses_quant(M, N, K, act.x_dtype)))))
    return fail(W4A8_ERR_INVALID_ARG, "no in-kernel quantisation for this path and shape");
  if (act.tiled && (fused || debug || path != W4A8_PATH_SKINNY || !w8_linear_tiles_codes(M, N, K)))
    return fail(W4A8_ERR_INVALID_ARG, "tiled codes are read by the 14 <= M <= 16 skinny kernel only");
  const size_t qa_bytes = (size_t)(act.tiled ? 16 : M) * K;
  if (debug) {
    if (m_begin < 0 || m_end > M || m_begin > m_end)
      return fail(W4A8_ERR_INVALID_ARG, "row window [%lld, %lld) outside [0, %lld)",
                  (long long)m_begin, (long long)m_end, (long long)M);
    if (totals && !aligned16(totals))
      return fail(W4A8_ERR_MISALIGNED, "totals must be 16-byte aligned");
  }
  const int ks = w8_ksplit(path, M, N, K);
  const size_t ws_need = w8_workspace_for(path, M, N, K);
  if (ws_need && (!workspace || workspace_bytes < ws_need))
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                ws_need);
  if (ws_need && !aligned16(workspace))
    return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const size_t ybytes = (size_t)M * (size_t)N * 2;
  const size_t xbytes = (size_t)M * K * (act.x_dtype == W4A8_F32 ? 4 : 2);
  if (y && ((!fused && (overlaps(y, ybytes, act.qa, qa_bytes) ||
                        overlaps(y, ybytes, act.sa, (size_t)M * 4))) ||
            (fused && overlaps(y, ybytes, act.x, xbytes)) || overlaps(y, ybytes, packed, need) ||
            (ws_need && overlaps(y, ybytes, workspace, ws_need))))
    return fail(W4A8_ERR_INVALID_ARG, "output aliases an input or the workspace");
  if (totals && m_end > m_begin) {
    const size_t tb = (size_t)(m_end - m_begin) * (size_t)N * 4;
    if ((y && overlaps(totals, tb, y, ybytes)) || overlaps(totals, tb, packed, need) ||
        (ws_need && overlaps(totals, tb, workspace, ws_need)))
      return fail(W4A8_ERR_INVALID_ARG, "totals alias another buffer");
  }
  if (validate_only) return ok();

  const uint8_t* base = static_cast<const uint8_t*>(packed);
  GemmArgs a;
  a.qa = act.qa;
  a.sa = act.sa;
  a.x = act.x;
  a.x_dtype = act.x_dtype;
  a.w.codes = base;
  a.w.zeros = nullptr;
  a.w.scales = reinterpret_cast<const float*>(base + w8_scales_offset(N, K));
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = y;
  a.partials = debug ? totals : nullptr;
  a.m_begin = debug ? m_begin : 0;
  a.m_end = debug ? m_end : 0;
  a.workspace = static_cast<float*>(workspace);
  a.sa_ws = nullptr;
  a.ksplit = ks;
  a.cb = a.ks = 0;
  a.w8 = true;
  a.qa_tiled = act.tiled;
  const float* sa_for_reduce = act.sa;
  if (path == W4A8_PATH_GEMV) {
    const GemvShape gs = gemv_shape(N, K);
    a.cb = gs.cb;
    a.ks = gs.ks;
    if (fused && ks > 1) {  // the in-kernel scale, for the reduction
      a.sa_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws_need - 256);
      sa_for_reduce = a.sa_ws;
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (path == W4A8_PATH_PREFILL) {
    // row chunks, as for W4A8; the totals of the debug window per chunk
    const int64_t rows = prefill_chunk_rows(K, 1);
    const int tile = prefill_auto_tile(M, N, K);
    a.wide = tile == kTile256x256;
    const PrefillTail tail = ks > 1 ? PrefillTail{0, 0, 0} : prefill_tail_for(M, N, K, tile);
    a.tail_split = tail.split;
    a.tail_tiles = tail.tiles;
    a.tail_n0 = tail.n0;
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += rows) {
      const int64_t mc = M - m0 < rows ? M - m0 : rows;
      GemmArgs c = a;
      c.qa = a.qa + m0 * K;
      c.sa = a.sa + m0;
      c.M = mc;
      c.y = y ? y + m0 * N : nullptr;
      if (a.partials) {
        const ChunkWindow w = chunk_window(a.m_begin, a.m_end, m0, mc);
        c.m_begin = w.begin;
        c.m_end = w.end;
        c.partials = w.begin < w.end ? a.partials + w.out_row * N : nullptr;
      }
      e = launch_prefill(c, st);
      if (e == hipSuccess && ks > 1 && (c.y || c.partials))
        e = launch_w8_splitk_reduce(reinterpret_cast<const int32_t*>(workspace), ks, c.sa,
                                    a.w.scales, mc, N, c.y, c.partials, c.m_begin, c.m_end, st);
      if (e == hipSuccess && tail.split > 1 && (c.y || c.partials))
        e = launch_w8_splitk_reduce(reinterpret_cast<const int32_t*>(workspace), tail.split, c.sa,
                                    a.w.scales, mc, N, c.y, c.partials, c.m_begin, c.m_end, st,
                                    tail.n0);
    }
    return device_status(e, "w8a8 gemm launch");
  }
  hipError_t e = path == W4A8_PATH_GEMV ? launch_gemv(a, st) : launch_skinny(a, st);
  if (e == hipSuccess && ks > 1 && (y || a.partials))
    e = launch_w8_splitk_reduce(reinterpret_cast<const int32_t*>(workspace), ks, sa_for_reduce,
                                a.w.scales, M, N, y, a.partials, a.m_begin, a.m_end, st);
  return device_status(e, "w8a8 gemm launch");
}

}  // namespace

extern "C" {

int w4a8_abi_version(void) { return W4A8_ABI_VERSION; }
int w4a8_layout_version(void) { return W4A8_LAYOUT_VERSION; }

const char* w4a8_status_string(int status) {
  switch (status) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_INVALID_ARG: return "invalid argument";
    case W4A8_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case W4A8_ERR_MISALIGNED: return "misaligned pointer";
    case W4A8_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case W4A8_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* w4a8_last_error(void) { return g_err; }

size_t w4a8_packed_weight_bytes(int64_t N, int64_t K, int32_t group) {
  if (check_weight_shape(N, K, group)) return 0;
  return (size_t)packed_bytes(N, K);
}

int w4a8_pack_weights_into(const uint8_t* q, const uint8_t* z, const float* s, int64_t N_part,
                           int64_t K, int32_t group, void* packed, size_t packed_bytes_,
                           int64_t N_total, int64_t n_offset, void* stream) {
  int rc = check_weight_shape(N_part, K, group);
  if (rc) return rc;
  rc = check_weight_shape(N_total, K, group);
  if (rc) return rc;
  if (n_offset < 0 || n_offset % kBlockCols || n_offset + N_part > N_total)
    return fail(W4A8_ERR_INVALID_ARG,
                "channels [%lld, %lld) are not a 16-aligned range of the %lld packed ones",
                (long long)n_offset, (long long)(n_offset + N_part), (long long)N_total);
  if (!q || !s || !packed) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(packed) || !aligned16(s))
    return fail(W4A8_ERR_MISALIGNED, "q, s and packed must be 16-byte aligned");
  const size_t need = (size_t)packed_bytes(N_total, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  const size_t G = (size_t)(K / kGroup);
  if (overlaps(packed, need, q, (size_t)(N_part * K)) ||
      (z && overlaps(packed, need, z, (size_t)N_part * G)) ||
      overlaps(packed, need, s, (size_t)N_part * G * 4))
    return fail(W4A8_ERR_INVALID_ARG, "packed buffer aliases an input");
  (void)hipGetLastError();
  return device_status(launch_pack_into(q, z, s, N_part, K, static_cast<uint8_t*>(packed), N_total,
                                        n_offset, static_cast<hipStream_t>(stream)),
                       "pack launch");
}

int w4a8_pack_weights(const uint8_t* q, const uint8_t* z, const float* s, int64_t N, int64_t K,
                      int32_t group, void* packed, size_t packed_bytes_, void* stream) {
  return w4a8_pack_weights_into(q, z, s, N, K, group, packed, packed_bytes_, N, 0, stream);
}

int w4a8_unpack_weights(const void* packed, size_t packed_bytes_, int64_t N, int64_t K,
                        int32_t group, uint8_t* q, uint8_t* z, float* s, void* stream) {
  int rc = check_weight_shape(N, K, group);
  if (rc) return rc;
  if (!q || !z || !s || !packed) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(packed) || !aligned16(s))
    return fail(W4A8_ERR_MISALIGNED, "q, s and packed must be 16-byte aligned");
  const size_t need = (size_t)packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  (void)hipGetLastError();
  return device_status(launch_unpack(static_cast<const uint8_t*>(packed), N, K, q, z, s,
                                     static_cast<hipStream_t>(stream)),
                       "unpack launch");
}

// tiled: qa in the layout of launch_quant_tiled (16 K bytes, M <= 16).
static int quant_act_any(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* qa,
                         float* sa, void* stream, bool hadamard, bool tiled = false) {
  if (!x || !qa || !sa) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (x_dtype != W4A8_BF16 && x_dtype != W4A8_F32)
    return fail(W4A8_ERR_INVALID_ARG, "unknown activation dtype %d", (int)x_dtype);
  if (M <= 0 || M > ((int64_t)1 << 24) || K <= 0 || K > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld K=%lld out of range", (long long)M, (long long)K);
  if (K % kGroup)
    return fail(W4A8_ERR_UNSUPPORTED_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (!aligned16(x) || !aligned16(qa) || !aligned16(sa))
    return fail(W4A8_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
  const size_t xb = (size_t)M * K * (x_dtype == W4A8_BF16 ? 2 : 4);
  const size_t qb = (size_t)(tiled ? 16 : M) * K;
  if (overlaps(qa, qb, x, xb) || overlaps(sa, (size_t)M * 4, x, xb) ||
      overlaps(qa, qb, sa, (size_t)M * 4))
    return fail(W4A8_ERR_INVALID_ARG, "outputs alias the input or each other");
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return device_status(tiled ? launch_quant_tiled(x, x_dtype, M, K, qa, sa, st, hadamard)
                             : launch_quant(x, x_dtype, M, K, qa, sa, st, hadamard),
                       "quant launch");
}

int w4a8_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* qa, float* sa,
                   void* stream) {
  return quant_act_any(x, x_dtype, M, K, qa, sa, stream, false);
}

int w4a8_quant_act_hadamard(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* qa,
                            float* sa, void* stream) {
  return quant_act_any(x, x_dtype, M, K, qa, sa, stream, true);
}

size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (check_weight_shape(N, K, group) || M <= 0) return 0;
  return gemm_workspace_any(M, N, K);
}

int w4a8_select_path(int64_t M, int64_t, int64_t K) { return M <= 0 ? 0 : pick_path(M, K); }

int w4a8_gemm(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes_,
              int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y, void* workspace,
              size_t workspace_bytes, void* stream) {
  return run_gemm(ActIn{qa, sa, nullptr, 0}, packed, packed_bytes_, M, N, K, group,
                  W4A8_PATH_AUTO, 0, 0, nullptr, y, workspace, workspace_bytes, stream, false);
}

int w4a8_gemm_debug(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes_,
                    int64_t M, int64_t N, int64_t K, int32_t group, int32_t path, int64_t m_begin,
                    int64_t m_end, int32_t* partials, uint16_t* y_or_null, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return run_gemm(ActIn{qa, sa, nullptr, 0}, packed, packed_bytes_, M, N, K, group, path, m_begin,
                  m_end, partials, y_or_null, workspace, workspace_bytes, stream, true);
}

size_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (check_weight_shape(N, K, group) || M <= 0) return 0;
  return linear_workspace(M, N, K);
}

int w4a8_linear(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes_,
                int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y, void* workspace,
                size_t workspace_bytes, void* stream) {
  int rc = check_weight_shape(N, K, group);
  if (rc) return rc;
  if (!x || !y) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (x_dtype != W4A8_BF16 && x_dtype != W4A8_F32)
    return fail(W4A8_ERR_INVALID_ARG, "unknown activation dtype %d", (int)x_dtype);
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  if (pick_path(M, K) == W4A8_PATH_GEMV)
    return run_gemm(ActIn{nullptr, nullptr, x, x_dtype}, packed, packed_bytes_, M, N, K, group,
                    W4A8_PATH_GEMV, 0, 0, nullptr, y, workspace, workspace_bytes, stream, false);
  // The workspace is required at its documented size on every path, so a
  // caller's sizing does not depend on which kernels run.
  const size_t need = linear_workspace(M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  // One launch when the skinny kernel can quantise these rows itself.
  if (pick_path(M, K) == W4A8_PATH_SKINNY && linear_fuses_quant(M, N, K, x_dtype))
    return run_gemm(ActIn{nullptr, nullptr, x, x_dtype}, packed, packed_bytes_, M, N, K, group,
                    W4A8_PATH_SKINNY, 0, 0, nullptr, y, workspace, workspace_bytes, stream, false);
  // Two launches: quantise into the workspace, then the GEMM.
  if (!aligned16(workspace)) return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const size_t xbytes = (size_t)M * K * (x_dtype == W4A8_F32 ? 4 : 2);
  if (overlaps(workspace, need, x, xbytes) || overlaps(workspace, need, packed, packed_bytes_))
    return fail(W4A8_ERR_INVALID_ARG, "workspace aliases an input");
  if (overlaps(y, (size_t)M * N * 2, x, xbytes))
    return fail(W4A8_ERR_INVALID_ARG, "output aliases the activations");
  const bool tiled = linear_tiles_codes(M, N, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qa = reinterpret_cast<int8_t*>(ws);
  float* sa = reinterpret_cast<float*>(ws + linear_codes_bytes(M, N, K));
  uint8_t* gws = ws + linear_codes_bytes(M, N, K) + round256((size_t)M * 4);
  // Validate the GEMM before launching the quantiser, so a rejected call
  // launches nothing.
  rc = run_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K, group,
                W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false,
                /*validate_only=*/true);
  if (rc) return rc;
  rc = quant_act_any(x, x_dtype, M, K, qa, sa, stream, false, tiled);
  if (rc) return rc;
  return run_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K, group,
                  W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false);
}

// The layer with the online rotation: rotated quantisation into the
// workspace, then the GEMM of w4a8_gemm against weights that carry the
// inverse rotation (two launches on every path).
size_t w4a8_linear_hadamard_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (check_weight_shape(N, K, group) || M <= 0) return 0;
  return linear_codes_bytes(M, N, K) + round256((size_t)M * 4) + gemm_workspace_any(M, N, K);
}

int w4a8_linear_hadamard(const void* x, int32_t x_dtype, const void* packed,
                         size_t packed_bytes_, int64_t M, int64_t N, int64_t K, int32_t group,
                         uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_weight_shape(N, K, group);
  if (rc) return rc;
  if (!x || !y) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (x_dtype != W4A8_BF16 && x_dtype != W4A8_F32)
    return fail(W4A8_ERR_INVALID_ARG, "unknown activation dtype %d", (int)x_dtype);
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  const size_t need =
      linear_codes_bytes(M, N, K) + round256((size_t)M * 4) + gemm_workspace_any(M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const size_t xbytes = (size_t)M * K * (x_dtype == W4A8_F32 ? 4 : 2);
  if (overlaps(workspace, need, x, xbytes) || overlaps(workspace, need, packed, packed_bytes_))
    return fail(W4A8_ERR_INVALID_ARG, "workspace aliases an input");
  if (overlaps(y, (size_t)M * N * 2, x, xbytes))
    return fail(W4A8_ERR_INVALID_ARG, "output aliases the activations");
  // At M == 1 one launch: the GEMV's quantiser rotates the token first.  (In
  // the M <= 16 kernel every workgroup would rotate all rows again; measured
  // slower than the two launches at every shape tried, e.g. M = 4, K = 18944
  // -> N = 3584: 26.5 against 15.8 us.)
  if (pick_path(M, K) == W4A8_PATH_GEMV)
    return run_gemm(ActIn{nullptr, nullptr, x, x_dtype}, packed, packed_bytes_, M, N, K, group,
                    W4A8_PATH_GEMV, 0, 0, nullptr, y, workspace, workspace_bytes, stream, false,
                    false, /*hadamard=*/true);
  const bool tiled = linear_tiles_codes(M, N, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qa = reinterpret_cast<int8_t*>(ws);
  float* sa = reinterpret_cast<float*>(ws + linear_codes_bytes(M, N, K));
  uint8_t* gws = ws + linear_codes_bytes(M, N, K) + round256((size_t)M * 4);
  rc = run_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K, group,
                W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false,
                /*validate_only=*/true);
  if (rc) return rc;
  rc = quant_act_any(x, x_dtype, M, K, qa, sa, stream, true, tiled);
  if (rc) return rc;
  return run_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K, group,
                  W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false);
}

// ------------------------------------------------------------------ W8A8

int w8a8_layout_version(void) { return W8A8_LAYOUT_VERSION; }

size_t w8a8_packed_weight_bytes(int64_t N, int64_t K) {
  if (check_w8_shape(N, K)) return 0;
  return (size_t)w8_packed_bytes(N, K);
}

int w8a8_pack_weights(const int8_t* qw, const float* sw, int64_t N, int64_t K, void* packed,
                      size_t packed_bytes_, void* stream) {
  int rc = check_w8_shape(N, K);
  if (rc) return rc;
  if (!qw || !sw || !packed) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(qw) || !aligned16(packed) || !aligned16(sw))
    return fail(W4A8_ERR_MISALIGNED, "qw, sw and packed must be 16-byte aligned");
  const size_t need = (size_t)w8_packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  if (overlaps(packed, need, qw, (size_t)(N * K)) || overlaps(packed, need, sw, (size_t)N * 4))
    return fail(W4A8_ERR_INVALID_ARG, "packed buffer aliases an input");
  (void)hipGetLastError();
  return device_status(launch_w8_pack(qw, sw, N, K, static_cast<uint8_t*>(packed),
                                      static_cast<hipStream_t>(stream)),
                       "w8a8 pack launch");
}

int w8a8_unpack_weights(const void* packed, size_t packed_bytes_, int64_t N, int64_t K, int8_t* qw,
                        float* sw, void* stream) {
  int rc = check_w8_shape(N, K);
  if (rc) return rc;
  if (!qw || !sw || !packed) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(qw) || !aligned16(packed) || !aligned16(sw))
    return fail(W4A8_ERR_MISALIGNED, "qw, sw and packed must be 16-byte aligned");
  const size_t need = (size_t)w8_packed_bytes(N, K);
  if (packed_bytes_ < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "packed buffer %zu bytes, need %zu", packed_bytes_, need);
  if (overlaps(packed, need, qw, (size_t)(N * K)) || overlaps(packed, need, sw, (size_t)N * 4) ||
      overlaps(qw, (size_t)(N * K), sw, (size_t)N * 4))
    return fail(W4A8_ERR_INVALID_ARG, "buffers alias");
  (void)hipGetLastError();
  return device_status(launch_w8_unpack(static_cast<const uint8_t*>(packed), N, K, qw, sw,
                                        static_cast<hipStream_t>(stream)),
                       "w8a8 unpack launch");
}

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_w8_shape(N, K) || M <= 0) return 0;
  return w8_gemm_workspace_any(M, N, K);
}

int w8a8_select_path(int64_t M, int64_t N, int64_t K) { return M <= 0 ? 0 : pick_w8_path(M, N, K); }

int w8a8_gemm(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes_,
              int64_t M, int64_t N, int64_t K, uint16_t* y, void* workspace,
              size_t workspace_bytes, void* stream) {
  return run_w8_gemm(ActIn{qa, sa, nullptr, 0}, packed, packed_bytes_, M, N, K, W4A8_PATH_AUTO, 0,
                     0, nullptr, y, workspace, workspace_bytes, stream, false);
}

int w8a8_gemm_debug(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes_,
                    int64_t M, int64_t N, int64_t K, int32_t path, int64_t m_begin, int64_t m_end,
                    int32_t* totals, uint16_t* y_or_null, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return run_w8_gemm(ActIn{qa, sa, nullptr, 0}, packed, packed_bytes_, M, N, K, path, m_begin,
                     m_end, totals, y_or_null, workspace, workspace_bytes, stream, true);
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_w8_shape(N, K) || M <= 0) return 0;
  return w8_linear_workspace(M, N, K);
}

int w8a8_linear(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes_, int64_t M,
                int64_t N, int64_t K, uint16_t* y, void* workspace, size_t workspace_bytes,
                void* stream) {
  int rc = check_w8_shape(N, K);
  if (rc) return rc;
  if (!x || !y) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (x_dtype != W4A8_BF16 && x_dtype != W4A8_F32)
    return fail(W4A8_ERR_INVALID_ARG, "unknown activation dtype %d", (int)x_dtype);
  if (M <= 0 || M > ((int64_t)1 << 24))
    return fail(W4A8_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  const size_t need = w8_linear_workspace(M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(W4A8_ERR_BUFFER_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(W4A8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  // One launch when the GEMV (M == 1) or the M <= 16 kernel can quantise
  // these rows itself.
  const int fpath = pick_w8_path(M, N, K);
  if (fpath == W4A8_PATH_GEMV ||
      (fpath == W4A8_PATH_SKINNY && skinny_fuses_quant(M, N, K, x_dtype)))
    return run_w8_gemm(ActIn{nullptr, nullptr, x, x_dtype}, packed, packed_bytes_, M, N, K, fpath,
                       0, 0, nullptr, y, workspace, workspace_bytes, stream, false);
  const size_t xbytes = (size_t)M * K * (x_dtype == W4A8_F32 ? 4 : 2);
  if (overlaps(workspace, need, x, xbytes) || overlaps(workspace, need, packed, packed_bytes_))
    return fail(W4A8_ERR_INVALID_ARG, "workspace aliases an input");
  if (overlaps(y, (size_t)M * N * 2, x, xbytes))
    return fail(W4A8_ERR_INVALID_ARG, "output aliases the activations");
  const bool tiled = w8_linear_tiles_codes(M, N, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qa = reinterpret_cast<int8_t*>(ws);
  float* sa = reinterpret_cast<float*>(ws + w8_linear_codes_bytes(M, N, K));
  uint8_t* gws = ws + w8_linear_codes_bytes(M, N, K) + round256((size_t)M * 4);
  rc = run_w8_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K,
                   W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false,
                   /*validate_only=*/true);
  if (rc) return rc;
  rc = quant_act_any(x, x_dtype, M, K, qa, sa, stream, false, tiled);
  if (rc) return rc;
  return run_w8_gemm(ActIn{qa, sa, nullptr, 0, tiled}, packed, packed_bytes_, M, N, K,
                     W4A8_PATH_AUTO, 0, 0, nullptr, y, gws, need - (size_t)(gws - ws), stream, false);
}

// ------------------------------------------------------------------ W4A16

size_t w4a16_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (check_weight_shape(N, K, group) || M <= 0) return 0;
  return a16_workspace_any(M, N, K);
}

int w4a16_select_path(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % kGroup || N % kBlockCols) return 0;
  return pick_a16_path(M, N, K);
}

int w4a16_linear(const uint16_t* x, const void* packed, size_t packed_bytes_, int64_t M, int64_t N,
                 int64_t K, int32_t group, uint16_t* y, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return run_a16(x, packed, packed_bytes_, M, N, K, group, W4A8_PATH_AUTO, y, workspace,
                 workspace_bytes, stream);
}

int w4a16_linear_path(const uint16_t* x, const void* packed, size_t packed_bytes_, int64_t M,
                      int64_t N, int64_t K, int32_t group, int32_t path, uint16_t* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return run_a16(x, packed, packed_bytes_, M, N, K, group, path, y, workspace, workspace_bytes,
                 stream);
}

// ------------------------------------------------------------ peak probes

int w4a8_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                          void* stream) {
  if (!buf || !sink) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (bytes == 0 || bytes % 16) return fail(W4A8_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 16", bytes);
  if (blocks < 1 || blocks > 65536) return fail(W4A8_ERR_INVALID_ARG, "blocks=%d out of [1, 65536]", (int)blocks);
  if (!aligned16(buf) || !aligned16(sink)) return fail(W4A8_ERR_MISALIGNED, "buffers must be 16-byte aligned");
  if (overlaps(buf, bytes, sink, (size_t)blocks * 4)) return fail(W4A8_ERR_INVALID_ARG, "sink aliases the buffer");
  (void)hipGetLastError();
  return device_status(launch_peak_stream_read(buf, bytes, sink, blocks, static_cast<hipStream_t>(stream)),
                       "stream probe launch");
}

int w4a8_peak_mfma_i8(int32_t iters, int32_t* sink, uint64_t* clocks, int32_t blocks, void* stream) {
  if (!sink) return fail(W4A8_ERR_INVALID_ARG, "null pointer");
  if (iters < 1 || iters > (1 << 20)) return fail(W4A8_ERR_INVALID_ARG, "iters=%d out of [1, 2^20]", (int)iters);
  if (blocks < 1 || blocks > 65536) return fail(W4A8_ERR_INVALID_ARG, "blocks=%d out of [1, 65536]", (int)blocks);
  if (!aligned16(sink) || (clocks && !aligned16(clocks)))
    return fail(W4A8_ERR_MISALIGNED, "buffers must be 16-byte aligned");
  if (clocks && overlaps(sink, (size_t)blocks * 256 * 4, clocks, (size_t)blocks * 16))
    return fail(W4A8_ERR_INVALID_ARG, "sink aliases clocks");
  (void)hipGetLastError();
  return device_status(launch_peak_mfma_i8(iters, sink, clocks, blocks, static_cast<hipStream_t>(stream)),
                       "mfma probe launch");
}

}  // extern "C"
