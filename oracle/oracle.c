/*
 * CPU oracle for the W4A8 linear layer — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant with the
 * HIP library: everything below is written out from the definitions, with
 * plain loops, so that it can be checked by eye.
 *
 * What it computes (the layer the pages describe):
 *   "The 4-bit CPU path", section "W4A8": GPTQ-packed int4 weights times
 *   activations quantised to int8; the kernel uses the checkpoint's integer
 *   zero points (or the constant 8 for a symmetric grid).
 *   "The 4-bit CPU path", section "Building a checkpoint": group size 128.
 *   "EgoPQ Real-Serving Handoff", section "2. External Artifacts": the native
 *   packed path needs exact per-group scale and zero metadata, and is not
 *   interchangeable with a float fake-quant path — so the oracle is the exact
 *   integer path, not a float emulation.
 *   "Serve a pre-quantized int8 weight-only DiT ...", comments "Directive ..."
 *   and "Round two ...": isolate one linear against a reference
 *   dequant-then-matmul, and make sure that reference applies the activation
 *   scale.
 *
 * Readings taken where the pages are silent (each also listed in the design doc):
 *   - activations: symmetric per-token (per-row) int8, scale sa = absmax/127
 *     in float32 with IEEE division; codes rint(x/sa) (ties to even) clamped
 *     to [-127, 127]; an all-zero row gives sa = 0 and codes 0;
 *   - weights: W[n][k] = s[n][g] * (q[n][k] - z[n][g]) with q, z integers in
 *     0..15, s float32, g = k / group over contiguous groups of K;
 *   - per group an exact integer P[m][n][g] = sum_k qa[m][k]*(q[n][k]-z[n][g]);
 *   - y[m][n] = sa[m] * sum_g s[n][g] * P[m][n][g], evaluated here in float64
 *     and NOT rounded (the bf16 output is compared against this value).
 *
 * The quantisation decision (which int8 code) is taken in float32, the
 * precision the GPU kernel takes it in; everything after the integer products
 * is float64.
 *
 * The W8A8 int8-dynamic linear (a second layer the pages describe) follows at
 * the end of this file.
 *
 * Parity pins live in tests/test_oracle_pins.py (brute force, closed forms,
 * invariants, planted mutants).  Compile-time ORACLE_MUTANT values plant one
 * plausible mistake each, so the tests can show every mistake is caught.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_NONFINITE (-2)
#define ORACLE_RANGE (-3)

/* Largest |P| one group of 128 can reach: 128 * 127 * 15. */
#define ORACLE_P_BOUND 243840

int oracle_version(void) { return 1 + 100 * ORACLE_MUTANT; }

/* Threads the OpenMP loops below run on (reported beside CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
/* Sets the threads of later calls (n >= 1), for single-threaded timings. */
int oracle_set_threads(int n) {
  if (n < 1) return 1;
  omp_set_num_threads(n);
  return 0;
}
#else
int oracle_threads(void) { return 1; }
int oracle_set_threads(int n) { return n == 1 ? 0 : 1; }
#endif

static float widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Symmetric per-token int8 quantisation of one float32 row. */
static int quant_row(const float* x, int64_t K, int8_t* qa, float* sa_out) {
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        if (!isfinite(x[k])) return ORACLE_NONFINITE;
        float a = fabsf(x[k]);
        if (a > amax) amax = a;
    }
#if ORACLE_MUTANT == 3
    float sa = amax / 128.0f;            /* planted: wrong symmetric range */
#else
    float sa = amax / 127.0f;
#endif
    *sa_out = sa;
    for (int64_t k = 0; k < K; ++k) {
        if (amax == 0.0f) {
            qa[k] = 0;
            continue;
        }
        float t = x[k] / sa;
#if ORACLE_MUTANT == 2
        float r = roundf(t);             /* planted: ties away from zero */
#else
        float r = rintf(t);              /* default mode: ties to even */
#endif
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        qa[k] = (int8_t)r;
    }
    return ORACLE_OK;
}

int oracle_quant_act_f32(const float* x, int64_t M, int64_t K, int8_t* qa, float* sa) {
    if (!x || !qa || !sa || M < 0 || K <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        int r = quant_row(x + m * K, K, qa + m * K, sa + m);
        if (r != ORACLE_OK) rc = r;
    }
    return rc;
}

int oracle_quant_act_bf16(const uint16_t* x, int64_t M, int64_t K, int8_t* qa, float* sa) {
    if (!x || !qa || !sa || M < 0 || K <= 0) return ORACLE_BAD_ARG;
    float* row = (float*)malloc((size_t)K * sizeof(float));
    if (!row) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) row[k] = widen_bf16(x[m * K + k]);
        int r = quant_row(row, K, qa + m * K, sa + m);
        if (r != ORACLE_OK) rc = r;
    }
    free(row);
    return rc;
}

/* One exact per-group integer dot product. */
static int64_t group_dot(const int8_t* qa_row, const uint8_t* q_row, int zero,
                         int64_t k0, int32_t group) {
    int64_t p = 0;
    for (int64_t k = k0; k < k0 + group; ++k) {
#if ORACLE_MUTANT == 1
        p += (int64_t)qa_row[k] * (int64_t)q_row[k];          /* planted: zero point dropped */
#elif ORACLE_MUTANT == 6
        int64_t kk = (k + 1 < k0 + group) ? k + 1 : k0;       /* planted: weights shifted by one k */
        p += (int64_t)qa_row[k] * ((int64_t)q_row[kk] - zero);
#else
        p += (int64_t)qa_row[k] * ((int64_t)q_row[k] - (int64_t)zero);
#endif
    }
    return p;
}

static int zero_at(const uint8_t* z, int64_t N, int64_t G, int64_t n, int64_t g) {
#if ORACLE_MUTANT == 4
    /* planted: zero plane read transposed ([G][N] instead of [N][G]) */
    int64_t idx = g * N + n;
    return z[idx % (N * G)];
#else
    (void)N;
    return z[n * G + g];
#endif
}

/*
 * P[m][n][g] for rows m0..m1-1 (stored at P[(m-m0)][n][g]).
 * Codes q[N][K] and zeros z[N][G] are one unsigned value per byte.
 */
int oracle_group_partials(const int8_t* qa, const uint8_t* q, const uint8_t* z,
                          int64_t M, int64_t N, int64_t K, int32_t group,
                          int64_t m0, int64_t m1, int32_t* P) {
    if (!qa || !q || !z || !P || group <= 0 || K % group || M < 0 || N < 0) return ORACLE_BAD_ARG;
    if (m0 < 0 || m1 > M || m0 > m1) return ORACLE_BAD_ARG;
    int64_t G = K / group;
    int rc = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t g = 0; g < G; ++g) {
                int64_t p = group_dot(qa + m * K, q + n * K, zero_at(z, N, G, n, g), g * group, group);
                if (p > ORACLE_P_BOUND || p < -ORACLE_P_BOUND) {
#pragma omp atomic write
                    rc = ORACLE_RANGE;
                }
                P[((m - m0) * N + n) * G + g] = (int32_t)p;
            }
        }
    }
    return rc;
}

/*
 * y[m][n] (float64, unrounded) for rows m0..m1-1 and columns n0..n1-1,
 * stored at y[(m-m0)*(n1-n0) + (n-n0)].
 */
int oracle_linear(const int8_t* qa, const float* sa, const uint8_t* q, const uint8_t* z,
                  const float* s, int64_t M, int64_t N, int64_t K, int32_t group,
                  int64_t m0, int64_t m1, int64_t n0, int64_t n1, double* y) {
    if (!qa || !sa || !q || !z || !s || !y) return ORACLE_BAD_ARG;
    if (group <= 0 || K % group || m0 < 0 || m1 > M || m0 > m1 || n0 < 0 || n1 > N || n0 > n1)
        return ORACLE_BAD_ARG;
    int64_t G = K / group;
    int64_t W = n1 - n0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = n0; n < n1; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int64_t p = group_dot(qa + m * K, q + n * K, zero_at(z, N, G, n, g), g * group, group);
                acc += (double)s[n * G + g] * (double)p;
            }
#if ORACLE_MUTANT == 5
            y[(m - m0) * W + (n - n0)] = acc;                  /* planted: activation scale missing */
#else
            y[(m - m0) * W + (n - n0)] = (double)sa[m] * acc;
#endif
        }
    }
    return ORACLE_OK;
}

/*
 * The packed weight format of the HIP library, written out from its
 * specification (layout version 1) so that the library's packing can be
 * compared byte for byte.  With G = K/128, NB = N/16:
 *   codes plane,  N*K/2 bytes at offset 0:
 *     block (nb, g) = 1024 bytes at ((nb*G + g) * 1024); inside it, lane
 *     L = 16*j + c (j = 0..3, c = 0..15) owns bytes [16L, 16L+16); byte i of
 *     that run holds q[16nb+c][128g+16j+i] in its low nibble and
 *     q[16nb+c][128g+64+16j+i] in its high nibble;
 *   zeros plane,  N*G/2 bytes at Z0 = round_up(N*K/2, 256):
 *     block (nb, g) = 8 bytes at Z0 + (nb*G + g)*8; byte c/2 holds
 *     z[16nb+c][g] in its low nibble for even c, high nibble for odd c;
 *   scales plane, 4*N*G bytes at S0 = round_up(Z0 + N*G/2, 256):
 *     float32 at index (nb*G + g)*16 + c equals s[16nb+c][g], bit for bit.
 */
static int64_t round_up256(int64_t v) { return (v + 255) / 256 * 256; }

int64_t oracle_layout_bytes(int64_t N, int64_t K) {
    int64_t G = K / 128;
    int64_t z0 = round_up256(N * K / 2);
    int64_t s0 = round_up256(z0 + N * G / 2);
    return s0 + 4 * N * G;
}

int oracle_layout_pack(const uint8_t* q, const uint8_t* z, const float* s,
                       int64_t N, int64_t K, uint8_t* out) {
    if (!q || !z || !s || !out || N <= 0 || K <= 0 || N % 16 || K % 128) return ORACLE_BAD_ARG;
    int64_t G = K / 128, NB = N / 16;
    int64_t z0 = round_up256(N * K / 2);
    int64_t s0 = round_up256(z0 + N * G / 2);
    memset(out, 0, (size_t)oracle_layout_bytes(N, K));
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g) {
            uint8_t* blk = out + (nb * G + g) * 1024;
            for (int j = 0; j < 4; ++j)
                for (int c = 0; c < 16; ++c)
                    for (int i = 0; i < 16; ++i) {
                        int64_t n = 16 * nb + c;
                        uint8_t lo = q[n * K + 128 * g + 16 * j + i] & 0x0F;
                        uint8_t hi = q[n * K + 128 * g + 64 + 16 * j + i] & 0x0F;
                        blk[16 * (16 * j + c) + i] = (uint8_t)(lo | (hi << 4));
                    }
            uint8_t* zb = out + z0 + (nb * G + g) * 8;
            for (int c = 0; c < 16; ++c) {
                uint8_t v = z[(16 * nb + c) * G + g] & 0x0F;
                zb[c / 2] |= (uint8_t)((c % 2) ? (v << 4) : v);
            }
            float* sb = (float*)(out + s0) + (nb * G + g) * 16;
            for (int c = 0; c < 16; ++c) sb[c] = s[(16 * nb + c) * G + g];
        }
    return ORACLE_OK;
}

int oracle_layout_unpack(const uint8_t* in, int64_t N, int64_t K,
                         uint8_t* q, uint8_t* z, float* s) {
    if (!in || !q || !z || !s || N <= 0 || K <= 0 || N % 16 || K % 128) return ORACLE_BAD_ARG;
    int64_t G = K / 128, NB = N / 16;
    int64_t z0 = round_up256(N * K / 2);
    int64_t s0 = round_up256(z0 + N * G / 2);
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g) {
            const uint8_t* blk = in + (nb * G + g) * 1024;
            for (int j = 0; j < 4; ++j)
                for (int c = 0; c < 16; ++c)
                    for (int i = 0; i < 16; ++i) {
                        int64_t n = 16 * nb + c;
                        uint8_t b = blk[16 * (16 * j + c) + i];
                        q[n * K + 128 * g + 16 * j + i] = b & 0x0F;
                        q[n * K + 128 * g + 64 + 16 * j + i] = b >> 4;
                    }
            const uint8_t* zb = in + z0 + (nb * G + g) * 8;
            for (int c = 0; c < 16; ++c)
                z[(16 * nb + c) * G + g] = (c % 2) ? (zb[c / 2] >> 4) : (zb[c / 2] & 0x0F);
            const float* sb = (const float*)(in + s0) + (nb * G + g) * 16;
            for (int c = 0; c < 16; ++c) s[(16 * nb + c) * G + g] = sb[c];
        }
    return ORACLE_OK;
}

/*
 * W8A8 int8-dynamic linear ("Serve a pre-quantized int8 weight-only DiT ...",
 * comment "Round two ...": int8 weights, activations quantised to int8 at run
 * time, an integer matrix product, and the product scaled afterwards; the
 * same comment warns that a reference must carry the activation scale).
 * Readings taken where the page is silent (each also listed in the design doc):
 *   - weights: W[n][k] = sw[n] * qw[n][k], symmetric int8 with one float32
 *     scale per output channel and no zero point;
 *   - activations: the per-token rule of quant_row above;
 *   - P[m][n] = sum over all k of qa[m][k] * qw[n][k], exact (the library
 *     keeps it in int32, so |P| must stay below 2^31);
 *   - y[m][n] = sa[m] * (sw[n] * P[m][n]) in float64, not rounded.
 */
static int64_t w8_dot(const int8_t* a, const int8_t* w, int64_t K) {
    int64_t p = 0;
    for (int64_t k = 0; k < K; ++k) {
#if ORACLE_MUTANT == 8
        p += (int64_t)a[k] * (int64_t)(uint8_t)w[k];         /* planted: weights read unsigned */
#else
        p += (int64_t)a[k] * (int64_t)w[k];
#endif
    }
    return p;
}

/* P[m][n] for rows m0..m1-1 (stored at P[(m-m0)][n]). */
int oracle_w8a8_totals(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K,
                       int64_t m0, int64_t m1, int32_t* P) {
    if (!qa || !qw || !P || M < 0 || N < 0 || K <= 0) return ORACLE_BAD_ARG;
    if (m0 < 0 || m1 > M || m0 > m1) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t p = w8_dot(qa + m * K, qw + n * K, K);
            if (p > 2147483647LL || p < -2147483647LL) {
#pragma omp atomic write
                rc = ORACLE_RANGE;
            }
            P[(m - m0) * N + n] = (int32_t)p;
        }
    }
    return rc;
}

/* y[m][n] (float64, unrounded) for rows m0..m1-1 and columns n0..n1-1. */
int oracle_w8a8_linear(const int8_t* qa, const float* sa, const int8_t* qw, const float* sw,
                       int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1, int64_t n0,
                       int64_t n1, double* y) {
    if (!qa || !sa || !qw || !sw || !y || K <= 0) return ORACLE_BAD_ARG;
    if (m0 < 0 || m1 > M || m0 > m1 || n0 < 0 || n1 > N || n0 > n1) return ORACLE_BAD_ARG;
    int64_t W = n1 - n0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = n0; n < n1; ++n) {
            double p = (double)w8_dot(qa + m * K, qw + n * K, K);
#if ORACLE_MUTANT == 7
            y[(m - m0) * W + (n - n0)] = (double)sa[m] * p;           /* planted: weight scale dropped */
#else
            y[(m - m0) * W + (n - n0)] = (double)sa[m] * ((double)sw[n] * p);
#endif
        }
    }
    return ORACLE_OK;
}

/*
 * The W8A8 packed weight format of the HIP library (W8 layout version 1),
 * written out from its specification.  With G = K/128, NB = N/16:
 *   codes plane, N*K bytes at offset 0: block (nb, g) = 2048 bytes at
 *     (nb*G + g) * 2048; half h (0, 1) at +1024*h; lane L = 16*j + c
 *     (j = 0..3, c = 0..15) at +16*L; byte i of that run is
 *     qw[16nb+c][128g + 64h + 16j + i] (two's complement);
 *   scales plane, 4*N bytes at S0 = round_up(N*K, 256): float32 sw[n] at
 *     index n, bit for bit.
 */
int64_t oracle_w8_layout_bytes(int64_t N, int64_t K) { return round_up256(N * K) + 4 * N; }

int oracle_w8_layout_pack(const int8_t* qw, const float* sw, int64_t N, int64_t K, uint8_t* out) {
    if (!qw || !sw || !out || N <= 0 || K <= 0 || N % 16 || K % 128) return ORACLE_BAD_ARG;
    int64_t G = K / 128, NB = N / 16;
    memset(out, 0, (size_t)oracle_w8_layout_bytes(N, K));
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g)
            for (int h = 0; h < 2; ++h)
                for (int j = 0; j < 4; ++j)
                    for (int c = 0; c < 16; ++c)
                        for (int i = 0; i < 16; ++i) {
                            int64_t n = 16 * nb + c, k = 128 * g + 64 * h + 16 * j + i;
                            out[(nb * G + g) * 2048 + 1024 * h + 16 * (16 * j + c) + i] =
                                (uint8_t)qw[n * K + k];
                        }
    float* sb = (float*)(out + round_up256(N * K));
    for (int64_t n = 0; n < N; ++n) sb[n] = sw[n];
    return ORACLE_OK;
}

int oracle_w8_layout_unpack(const uint8_t* in, int64_t N, int64_t K, int8_t* qw, float* sw) {
    if (!in || !qw || !sw || N <= 0 || K <= 0 || N % 16 || K % 128) return ORACLE_BAD_ARG;
    int64_t G = K / 128, NB = N / 16;
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g)
            for (int h = 0; h < 2; ++h)
                for (int j = 0; j < 4; ++j)
                    for (int c = 0; c < 16; ++c)
                        for (int i = 0; i < 16; ++i) {
                            int64_t n = 16 * nb + c, k = 128 * g + 64 * h + 16 * j + i;
                            qw[n * K + k] =
                                (int8_t)in[(nb * G + g) * 2048 + 1024 * h + 16 * (16 * j + c) + i];
                        }
    const float* sb = (const float*)(in + round_up256(N * K));
    for (int64_t n = 0; n < N; ++n) sw[n] = sb[n];
    return ORACLE_OK;
}

/*
 * Online Hadamard rotation before the per-token quantisation.  "EgoPQ
 * Real-Serving Handoff", section "1. Source Checkpoint", serves a packed
 * QuaRot model, and section "2. External Artifacts" exports it from QuaRot
 * caches; the page names the method and nothing more.  QuaRot (the published
 * method) multiplies activations by a Hadamard matrix before quantising them
 * and folds the inverse rotation into the weights, so that a few large
 * channels no longer set a whole token's absmax.  Readings taken (each also
 * listed in the design doc):
 *   - the rotation is block-diagonal over the quantisation groups: every
 *     group of 128 input channels is multiplied by the 128 x 128
 *     Walsh-Hadamard matrix H (Sylvester order, H[i][j] = (-1)^popcount(i&j)),
 *     unnormalised; the factor 1/128 of H * H^T = 128 I belongs to the
 *     weights (W' = W H / 128), since per-token quantisation is blind to a
 *     common scale;
 *   - the product is taken in float32 by the radix-2 butterflies in order of
 *     increasing stride h = 1, 2, 4, ..., 64, each pair (i, i + h) becoming
 *     (a + b, a - b); the kernel takes the same steps, so the rotated values,
 *     and hence the codes, agree bit for bit;
 *   - then the quantisation rule of quant_row, on the rotated row.
 */
static void fwht128(float* v) {
    for (int h = 1; h < 128; h *= 2)
        for (int i0 = 0; i0 < 128; i0 += 2 * h)
            for (int i = i0; i < i0 + h; ++i) {
                float a = v[i], b = v[i + h];
#if ORACLE_MUTANT == 9
                v[i] = a + b;                      /* planted: upper half not negated */
                v[i + h] = a + b;
#else
                v[i] = a + b;
                v[i + h] = a - b;
#endif
            }
}

/* x float32 or bfloat16 bits (is_bf16) [M][K] -> rotated float32 rows xr [M][K]. */
int oracle_hadamard_rows(const void* x, int is_bf16, int64_t M, int64_t K, float* xr) {
    if (!x || !xr || M < 0 || K <= 0 || K % 128) return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            xr[m * K + k] = is_bf16 ? widen_bf16(((const uint16_t*)x)[m * K + k])
                                    : ((const float*)x)[m * K + k];
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < K / 128; ++g) fwht128(xr + m * K + 128 * g);
    return ORACLE_OK;
}

int oracle_hadamard_quant_act(const void* x, int is_bf16, int64_t M, int64_t K, int8_t* qa,
                              float* sa) {
    if (!x || !qa || !sa || M < 0 || K <= 0 || K % 128) return ORACLE_BAD_ARG;
    float* xr = (float*)malloc((size_t)(M * K) * sizeof(float) + 1);
    if (!xr) return ORACLE_BAD_ARG;
    int rc = oracle_hadamard_rows(x, is_bf16, M, K, xr);
    if (rc == ORACLE_OK) rc = oracle_quant_act_f32(xr, M, K, qa, sa);
    free(xr);
    return rc;
}

/*
 * W4A16 ("The 4-bit CPU path", section "W4A16": activations stay bf16 and
 * multiply the same int4 weights, each weight being s * (q - z)).  Reading
 * taken (also listed in the design doc): the activations enter as given (bf16
 * widened exactly, or float32), no quantisation; per group the exact
 * products x * (q - z) are summed, and y[m][n] = sum_g s[n][g] * that sum,
 * all in float64 and not rounded.
 */
int oracle_w4a16_linear(const void* x, int is_bf16, const uint8_t* q, const uint8_t* z,
                        const float* s, int64_t M, int64_t N, int64_t K, int32_t group,
                        int64_t m0, int64_t m1, int64_t n0, int64_t n1, double* y) {
    if (!x || !q || !z || !s || !y || group <= 0 || K % group) return ORACLE_BAD_ARG;
    if (m0 < 0 || m1 > M || m0 > m1 || n0 < 0 || n1 > N || n0 > n1) return ORACLE_BAD_ARG;
    int64_t G = K / group, W = n1 - n0;
    int rc = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = n0; n < n1; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double p = 0.0;
                int zero = zero_at(z, N, G, n, g);
                for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                    double xv = is_bf16 ? (double)widen_bf16(((const uint16_t*)x)[m * K + k])
                                        : (double)((const float*)x)[m * K + k];
                    if (!isfinite(xv)) {
#pragma omp atomic write
                        rc = ORACLE_NONFINITE;
                    }
#if ORACLE_MUTANT == 10
                    p += xv * (double)q[n * K + k];                 /* planted: zero point dropped */
#else
                    p += xv * ((double)q[n * K + k] - (double)zero);
#endif
                }
                acc += (double)s[n * G + g] * p;
            }
            y[(m - m0) * W + (n - n0)] = acc;
        }
    }
    return rc;
}
