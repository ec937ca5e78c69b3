/*
 * w4a8.h — C ABI of the MI355X (gfx950) W4A8 linear-layer library.
 *
 * The layer: activations quantised per token to symmetric int8, multiplied by
 * GPTQ-style int4 weights that carry a scale and an integer zero point per
 * group of 128 input channels; every group is accumulated exactly in int32,
 * rescaled by sa[m] * s[n][g], and the result is written as bfloat16.
 *
 * Passages this interface follows:
 *   "The 4-bit CPU path", section "W4A8": the kernel takes GPTQ-packed int4
 *     weights and quantises activations to int8; it uses the checkpoint's
 *     zero points (the constant 8 is only a symmetric-grid special case).
 *   "The 4-bit CPU path", section "Building a checkpoint": group size 128.
 *   "The 4-bit CPU path", section "The weight layout, measured": layout
 *     transforms happen once, at load; shapes that do not tile the layout's
 *     block are refused rather than misread.
 *   "The 4-bit CPU path", section "W4A16": small and large batches take
 *     different kernels (here the M buckets GEMV / SKINNY / PREFILL).
 *   "EgoPQ Real-Serving Handoff", section "2. External Artifacts": the packed
 *     path needs the exact per-group scale and zero metadata.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory on the current device;
 *     the caller allocates and owns every buffer.  The library allocates and
 *     frees nothing in these calls and keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work: they never synchronise the device.
 *   - Return value: W4A8_OK (0) or a negative W4A8_ERR_* status.  All
 *     argument checks run on the host before anything is enqueued: a rejected
 *     call launches nothing and writes nothing.  A failed launch returns
 *     W4A8_ERR_DEVICE.  w4a8_last_error() gives a thread-local message.
 *   - Device pointers must be 16-byte aligned.  Outputs must not alias inputs.
 *   - Inputs must be finite; non-finite activations give undefined codes.
 *   - All calls are deterministic: the same inputs give bitwise-identical
 *     outputs (reductions run in a fixed order; no floating-point atomics).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A8_ABI_VERSION 1
#define W4A8_LAYOUT_VERSION 1

/* status codes */
#define W4A8_OK 0
#define W4A8_ERR_INVALID_ARG (-1)       /* null pointer, M/N/K out of range, bad enum */
#define W4A8_ERR_UNSUPPORTED_SHAPE (-2) /* group != 128, K % 128 != 0, N % 16 != 0 */
#define W4A8_ERR_MISALIGNED (-3)        /* a device pointer is not 16-byte aligned */
#define W4A8_ERR_BUFFER_TOO_SMALL (-4)  /* packed or workspace buffer smaller than required */
#define W4A8_ERR_DEVICE (-5)            /* the HIP runtime reported an error */

/* activation dtypes for w4a8_quant_act */
#define W4A8_BF16 0
#define W4A8_F32 1

/* GEMM paths (M buckets).  AUTO picks GEMV for M == 1 (K <= 32768, else
 * SKINNY), SKINNY for 2 <= M <= 16, PREFILL for M > 16; the choice depends on
 * (M, N, K) only.  PREFILL addresses the codes and each launch's activations
 * with 32-bit offsets: an activation matrix of 2^31 bytes or more runs as
 * consecutive row chunks (one launch each, in order on the stream, with the
 * same results as one launch); N*K/2 >= 2^31 (N*K for W8A8 weights) or a
 * single row of 2^31 bytes returns W4A8_ERR_UNSUPPORTED_SHAPE. */
#define W4A8_PATH_AUTO 0
#define W4A8_PATH_GEMV 1
#define W4A8_PATH_SKINNY 2
#define W4A8_PATH_PREFILL 3
/* PREFILL computes 256-token x 256-channel output tiles when they fill at
 * least one round of the compute units, else 256 x 128 tiles.  For tests,
 * w4a8_gemm_debug (and only it) also takes these two paths, which force the
 * tile width at any shape; w4a8_select_path never returns them. */
#define W4A8_PATH_PREFILL_N128 4
#define W4A8_PATH_PREFILL_N256 5

int w4a8_abi_version(void);
/* Bumped whenever the packed weight format changes; a packed buffer is only
 * meaningful together with (N, K, group, layout version). */
int w4a8_layout_version(void);
const char* w4a8_status_string(int status);
/* Message for the last failing call on this thread ("" if none). */
const char* w4a8_last_error(void);

/*
 * Size in bytes of the packed weight buffer for an N x K weight with the
 * given group size; 0 if the shape is unsupported.
 */
size_t w4a8_packed_weight_bytes(int64_t N, int64_t K, int32_t group);

/*
 * w4a8_pack_weights — load-time conversion of GPTQ metadata into the gfx950
 * packed format (layout version 1).
 *   q  device uint8 [N][K], int4 codes 0..15, one per byte, row-major
 *   z  device uint8 [N][K/group], integer zero points 0..15; or NULL for a
 *      symmetric grid, where every zero point is the constant 8 ("The 4-bit
 *      CPU path", section "W4A8": the kernel takes the checkpoint's zero
 *      points when it has them and synthesises 8 otherwise)
 *   s  device float [N][K/group], per-group scales (copied bit for bit)
 *   packed  device buffer of at least w4a8_packed_weight_bytes(N, K, group)
 * Requirements: group == 128, K % 128 == 0, N % 16 == 0, N, K > 0.
 * Only the low 4 bits of q and z are used (callers pass 0..15).
 *
 * Format (G = K/128, NB = N/16), three planes in one buffer:
 *   codes,  N*K/2 bytes at offset 0: block (nb, g) is 1024 bytes at
 *     (nb*G + g)*1024; inside it lane L = 16*j + c (j = 0..3, c = 0..15)
 *     owns bytes [16L, 16L+16), and byte i of that run holds
 *     q[16nb+c][128g+16j+i] in its low nibble and q[16nb+c][128g+64+16j+i]
 *     in its high nibble;
 *   zeros,  N*G/2 bytes at Z0 = round_up(N*K/2, 256): block (nb, g) is 8
 *     bytes at Z0 + (nb*G + g)*8; byte c/2 holds z[16nb+c][g] in its low
 *     nibble (even c) or high nibble (odd c);
 *   scales, 4*N*G bytes at S0 = round_up(Z0 + N*G/2, 256): float at index
 *     (nb*G + g)*16 + c is s[16nb+c][g].
 * One 64-lane wavefront load of a codes block gives every lane the operands
 * of two int8 matrix-core steps (or eight 4-way dot products) for one output
 * channel and 32 input channels of one group.
 */
int w4a8_pack_weights(const uint8_t* q, const uint8_t* z, const float* s,
                      int64_t N, int64_t K, int32_t group,
                      void* packed, size_t packed_bytes, void* stream);

/*
 * w4a8_pack_weights_into — sibling projections of one input (query/key/value,
 * gate/up) packed side by side as ONE weight of N_total output channels, so a
 * single activation quantisation and a single GEMM serve all of them.  Packs
 * the [N_part][K] weight (q, z, s as for w4a8_pack_weights) into output
 * channels [n_offset, n_offset + N_part) of a buffer of
 * w4a8_packed_weight_bytes(N_total, K, group) bytes; packing every part of a
 * partition of [0, N_total) gives the bytes w4a8_pack_weights makes from the
 * parts stacked along N.  Parts may be packed in any order; the alignment
 * gaps between the planes are zeroed by each call.
 * ("Serve a pre-quantized int8 weight-only DiT ...", comments "Verdict in
 * brief" and "Round two": query/key/value weights load as one fused
 * projection; "The 4-bit CPU path", section "The weight layout, measured": a
 * fused gate/up projection.)
 * Requirements: as w4a8_pack_weights for both N_part and N_total;
 * n_offset % 16 == 0 and n_offset + N_part <= N_total (else
 * W4A8_ERR_INVALID_ARG).
 */
int w4a8_pack_weights_into(const uint8_t* q, const uint8_t* z, const float* s,
                           int64_t N_part, int64_t K, int32_t group,
                           void* packed, size_t packed_bytes,
                           int64_t N_total, int64_t n_offset, void* stream);

/* Inverse of w4a8_pack_weights (for tests and inspection): writes q, z, s in
 * the logical layouts described above. */
int w4a8_unpack_weights(const void* packed, size_t packed_bytes,
                        int64_t N, int64_t K, int32_t group,
                        uint8_t* q, uint8_t* z, float* s, void* stream);

/*
 * w4a8_quant_act — per-token symmetric int8 activation quantisation
 * ("The 4-bit CPU path", section "W4A8": activations are quantised to int8).
 *   x   device [M][K], bfloat16 (x_dtype = W4A8_BF16) or float (W4A8_F32)
 *   qa  device int8 [M][K]: qa = clamp(rint(x / sa), -127, 127), ties to even
 *   sa  device float [M]:   sa = max_k |x[m][k]| / 127 (IEEE float division);
 *       an all-zero row gives sa = 0 and qa = 0
 * Requirements: M >= 1, K >= 128, K % 128 == 0.
 */
int w4a8_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                   int8_t* qa, float* sa, void* stream);

/* Workspace bytes any path of w4a8_gemm / w4a8_gemm_debug may need for these
 * shapes (split-K partial sums: K split over all tiles when they leave
 * compute units idle, or over the tiles of a partial last round); 0 if none.
 * The plan depends on the device's compute-unit count (256 on MI355X). */
size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);

/* The path W4A8_PATH_AUTO takes for these shapes. */
int w4a8_select_path(int64_t M, int64_t N, int64_t K);

/*
 * w4a8_gemm — y[m][n] = bf16_rne( sa[m] * sum_g s[n][g] * P[m][n][g] ),
 *   P[m][n][g] = sum_{k in group g} qa[m][k] * (q[n][k] - z[n][g])  (exact int32)
 *   qa  device int8 [M][K] and sa device float [M] (from w4a8_quant_act)
 *   packed  device buffer from w4a8_pack_weights for the same (N, K, group)
 *   y   device bfloat16 bits [M][N], row-major
 *   workspace  device scratch of w4a8_gemm_workspace_bytes(M, N, K, group)
 *     bytes (may be NULL when that is 0); contents on entry are ignored
 * The float rescale is accumulated in float32; the result is rounded to
 * bfloat16 with round-to-nearest-even.
 */
int w4a8_gemm(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes,
              int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a8_gemm_debug — the same kernels as w4a8_gemm, with a forced path and the
 * per-group int32 partials written out for rows [m_begin, m_end):
 *   partials  device int32 [m_end - m_begin][N][K/group] (may be NULL)
 *   y_or_null device bfloat16 [M][N] or NULL (then y is not written)
 * path must be AUTO, GEMV (requires M == 1 and K <= 32768), SKINNY
 * (M <= 16), PREFILL, or PREFILL_N128 / PREFILL_N256 (PREFILL with the tile
 * width forced).
 */
int w4a8_gemm_debug(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes,
                    int64_t M, int64_t N, int64_t K, int32_t group, int32_t path,
                    int64_t m_begin, int64_t m_end, int32_t* partials, uint16_t* y_or_null,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a8_linear — the whole layer from raw activations: per-token int8
 * quantisation (the rule of w4a8_quant_act) followed by the GEMM of
 * w4a8_gemm.  For M == 1 (and K <= 32768) both run in ONE launch: the decode
 * GEMV quantises the token in its prologue, so a decode step has no separate
 * quantisation kernel.  For 2 <= M <= 16 it is also one launch when the rows
 * fit: M*(K+16) <= 128 KiB, at most 10240*8/MP bf16 (4096*8/MP float) values
 * per row with MP = M rounded up to a power of two >= 2, N large enough that
 * K is not split and small enough that its 16-channel blocks fit one round
 * of workgroups (N/16 <= the compute units; every workgroup quantises all
 * rows again), and not a shape that SKINNY runs on its weight-streaming grid
 * (N/16 >= the compute units and K <= 4096: whole 16-channel blocks per
 * workgroup, the activations staged once per workgroup); the SKINNY kernel
 * then quantises the rows into LDS.  Otherwise the codes are written to the
 * workspace and the GEMM of the selected path follows (two launches); for
 * 12 <= M <= 16 on the SKINNY kernel (not its weight-streaming grid) the
 * workspace holds them in an internal 16-row tiled layout that the kernel
 * reads as matrix-core operands.  The result is bitwise identical to
 * w4a8_quant_act followed by w4a8_gemm.
 *   x   device [M][K], bfloat16 (W4A8_BF16) or float (W4A8_F32)
 *   y   device bfloat16 bits [M][N]
 *   workspace  device scratch of w4a8_linear_workspace_bytes(M, N, K, group)
 *     bytes (may be NULL when that is 0), required at that size on every path
 */
size_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);
int w4a8_linear(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes,
                int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a8_linear_noalloc — w4a8_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments and result are those of w4a8_linear (bitwise
 * the same output), without the workspace: the quantised activations, their
 * scales and any split-K partial sums live in a static device array of
 * W4A8_NOALLOC_SCRATCH_BYTES bytes that each GPU the library runs on holds
 * from the library's first use on it until the process ends.  Its address is
 * looked up once per device, on the first call with that device current.
 * The call allocates and frees nothing.
 *   - Shapes whose w4a8_linear_workspace_bytes(M, N, K, group) exceeds the
 *     scratch return W4A8_ERR_BUFFER_TOO_SMALL before anything is enqueued.
 *   - Every call on one GPU uses that GPU's single scratch, which keeps the
 *     last call's contents (nothing in it has to start at zero: each call
 *     writes what it reads).  Calls that overlap in time on one GPU — on two
 *     streams, or from two host threads without ordering between them — race
 *     on it; the caller must serialise them (e.g. one stream).
 */
#define W4A8_NOALLOC_SCRATCH_BYTES (64u << 20)
int w4a8_linear_noalloc(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes,
                        int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y,
                        void* stream);

/* ------------------------------------------------------- online rotation
 *
 * The per-token quantisation preceded by an online Hadamard rotation, as in
 * the packed QuaRot model of "EgoPQ Real-Serving Handoff" (section "1.
 * Source Checkpoint"; its caches in section "2. External Artifacts"): the
 * rotation spreads a token's few large channels over the group, so they no
 * longer set the token's absmax.  Each group of 128 input channels of every
 * row is multiplied by the unnormalised 128 x 128 Walsh-Hadamard matrix H
 * (Sylvester order, H[i][j] = (-1)^popcount(i & j)), in float32, by the
 * radix-2 butterflies of increasing stride 1, 2, ..., 64 (pair (i, i + h)
 * becomes (a + b, a - b)); the rotated row is then quantised by the rule of
 * w4a8_quant_act.  Weights used with it must carry the inverse rotation
 * W' = W H / 128 (group by group), made offline.
 */

/* Arguments as w4a8_quant_act; K % 128 == 0. */
int w4a8_quant_act_hadamard(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* qa,
                            float* sa, void* stream);

/*
 * w4a8_linear_hadamard — w4a8_quant_act_hadamard, then w4a8_gemm with
 * weights packed from the rotated W'.  At M == 1 (the GEMV path) one launch:
 * the GEMV's quantiser rotates the token first, with the same codes and
 * scale; otherwise two launches through the workspace.  The result is bitwise that
 * of the two calls.  Arguments as w4a8_linear; workspace of
 * w4a8_linear_hadamard_workspace_bytes(M, N, K, group) bytes (required on
 * every path).
 */
size_t w4a8_linear_hadamard_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);
int w4a8_linear_hadamard(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes,
                         int64_t M, int64_t N, int64_t K, int32_t group, uint16_t* y,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- W4A16
 *
 * W4A16 ("The 4-bit CPU path", section "W4A16": the same int4 weights with
 * the activations kept in bf16; small batches expand the weights per row,
 * large ones once per batch).  Weights are the W4A8 packed buffer
 * (w4a8_pack_weights).  No activation quantisation:
 *   y[m][n] = bf16_rne( sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g]) )
 * with q - z expanded exactly to bf16 and each group's products summed in
 * float32 on the bf16 matrix cores, then scaled by s in float32 (the M == 1
 * GEMV sums x * (128 + q) with float32 bf16-pair dots and subtracts
 * (128 + z) times the float32 sum of x over the same inputs).
 *   x   device bfloat16 bits [M][K]
 *   y   device bfloat16 bits [M][N]
 *   workspace  device scratch of w4a16_linear_workspace_bytes(M, N, K, group)
 *     bytes (float split-K partials; may be NULL when that is 0)
 * Paths: GEMV (M == 1, K <= 32768: the W4A8 GEMV's grid and weight stream,
 * the bf16 token staged in LDS), SKINNY (M <= 16; each workgroup stages its
 * K slice of the rows in LDS when it fits, else loads the A operands straight
 * from the rows, which needs 2*M*K < 2^31) and PREFILL (128-token tiles).
 * AUTO takes the GEMV at M == 1 when it fits, else SKINNY at M <= 16, else
 * PREFILL.
 * w4a16_select_path names the path AUTO takes; w4a16_linear_path
 * forces one (AUTO allowed), for tests, and returns
 * W4A8_ERR_UNSUPPORTED_SHAPE when the forced path has no plan for the shape.
 */
size_t w4a16_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);
int w4a16_select_path(int64_t M, int64_t N, int64_t K);
int w4a16_linear(const uint16_t* x, const void* packed, size_t packed_bytes, int64_t M, int64_t N,
                 int64_t K, int32_t group, uint16_t* y, void* workspace, size_t workspace_bytes,
                 void* stream);
int w4a16_linear_path(const uint16_t* x, const void* packed, size_t packed_bytes, int64_t M,
                      int64_t N, int64_t K, int32_t group, int32_t path, uint16_t* y,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ W8A8
 *
 * The W8A8 int8-dynamic linear ("Serve a pre-quantized int8 weight-only DiT
 * ...", comment "Round two ...": int8 weights, activations quantised to int8
 * at run time, an integer matrix product scaled afterwards; the comment's
 * kernel check compares against a float reference that carries the
 * activation scale).  Weights are symmetric int8 with one float scale per
 * output channel, W[n][k] = sw[n] * qw[n][k]; activations use the rule of
 * w4a8_quant_act.  The product over all of K is exact in int32:
 *   P[m][n] = sum_k qa[m][k] * qw[n][k]      (K <= 131072, so |P| < 2^31)
 *   y[m][n] = bf16_rne( sa[m] * (sw[n] * (float)P[m][n]) )
 * As P is exact and the epilogue is fixed, y is the same bits on every path.
 * Shapes: N % 16 == 0, K % 128 == 0, 0 < K <= 131072 (else
 * W4A8_ERR_UNSUPPORTED_SHAPE).  The status codes, alignment, stream and
 * ownership conventions are those of the W4A8 calls above.
 */
#define W8A8_LAYOUT_VERSION 1

int w8a8_layout_version(void);

/* Size in bytes of the packed W8A8 weight buffer; 0 if the shape is unsupported. */
size_t w8a8_packed_weight_bytes(int64_t N, int64_t K);

/*
 * w8a8_pack_weights — load-time conversion into the packed W8A8 format.
 *   qw  device int8 [N][K], row-major
 *   sw  device float [N], per-channel scales (copied bit for bit)
 *   packed  device buffer of at least w8a8_packed_weight_bytes(N, K)
 * Format (W8A8 layout version 1; G = K/128, NB = N/16), two planes:
 *   codes,  N*K bytes at offset 0: block (nb, g) is 2048 bytes at
 *     (nb*G + g)*2048; half h (0, 1) at +1024*h; lane L = 16*j + c
 *     (j = 0..3, c = 0..15) at +16*L; byte i of that run is
 *     qw[16nb+c][128g + 64h + 16j + i].  A lane's 16 bytes are its operand
 *     of one v_mfma_i32_16x16x64_i8 step as loaded.
 *   scales, 4*N bytes at round_up(N*K, 256) = N*K: float sw[n] at index n.
 * w8a8_unpack_weights is the exact inverse (qw [N][K], sw [N]).
 */
int w8a8_pack_weights(const int8_t* qw, const float* sw, int64_t N, int64_t K, void* packed,
                      size_t packed_bytes, void* stream);
int w8a8_unpack_weights(const void* packed, size_t packed_bytes, int64_t N, int64_t K, int8_t* qw,
                        float* sw, void* stream);

/* Path for an M x N x K W8A8 product: W4A8_PATH_GEMV for M == 1 when the
 * token fits the GEMV (K <= 32768, as for W4A8), W4A8_PATH_SKINNY for
 * M <= 16, W4A8_PATH_PREFILL otherwise. */
int w8a8_select_path(int64_t M, int64_t N, int64_t K);

/*
 * w8a8_gemm — y from pre-quantised activations.
 *   qa  device int8 [M][K] and sa device float [M] (from w4a8_quant_act)
 *   packed  from w8a8_pack_weights for the same (N, K)
 *   y   device bfloat16 bits [M][N]
 *   workspace  device scratch of w8a8_gemm_workspace_bytes(M, N, K) bytes
 *     (int32 split-K partials; may be NULL when that is 0)
 */
size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int w8a8_gemm(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes,
              int64_t M, int64_t N, int64_t K, uint16_t* y, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * w8a8_gemm_debug — the same kernels with a forced path (AUTO, GEMV for
 * M == 1, SKINNY for M <= 16, or PREFILL) and the exact int32 totals written for rows
 * [m_begin, m_end):  totals device int32 [m_end - m_begin][N] (may be NULL);
 * y_or_null as in w4a8_gemm_debug.
 */
int w8a8_gemm_debug(const int8_t* qa, const float* sa, const void* packed, size_t packed_bytes,
                    int64_t M, int64_t N, int64_t K, int32_t path, int64_t m_begin, int64_t m_end,
                    int32_t* totals, uint16_t* y_or_null, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * w8a8_linear — quantisation (the rule of w4a8_quant_act) and the W8A8 GEMM
 * from raw activations; bitwise identical to w4a8_quant_act + w8a8_gemm.
 * At M == 1 (the GEMV) and for M <= 16 whose rows fit (the same limits as
 * w4a8_linear) it is one launch: the kernel quantises the rows into LDS
 * itself.  Otherwise two launches through the workspace, which holds the
 * codes for 14 <= M <= 16 in the 16-row tiled layout of w4a8_linear.
 *   x   device [M][K], bfloat16 (W4A8_BF16) or float (W4A8_F32)
 *   workspace  device scratch of w8a8_linear_workspace_bytes(M, N, K) bytes,
 *     required on every path
 */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
int w8a8_linear(const void* x, int32_t x_dtype, const void* packed, size_t packed_bytes, int64_t M,
                int64_t N, int64_t K, uint16_t* y, void* workspace, size_t workspace_bytes,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
