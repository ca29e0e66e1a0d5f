/*
 * CPU oracle for the block-scaled small-M decode GEMV
 *
 *     Y[m, n] = sum_k A[m, k] * dequant(W)[n, k]
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with the
 * HIP library, and it includes nothing from the package.
 *
 * Plain and slow on purpose: every weight element is decoded from its bytes into
 * an exact float64 value, every product a*w is formed in float64 (exact: at most
 * 11+30 significant bits), and the K sum runs in ascending k in float64. Next to
 * each output it also returns S = sum_k |a*w|, which scales the acceptance bound.
 *
 * Sources (titles of the pages; section / paragraph):
 *  - "[CUDA] Block-scaled MatMul decode GEMV: tensor cores, packed FP4 decode and
 *    M-tiling": FP8 mma paragraph (E4M3 weight, per-block scales, widening is
 *    lossless) and FP4 mma paragraph (packed E2M1 with an E4M3 scale per 16
 *    elements; E2M1 has 2 significand bits, E4M3 has 4; largest product 6*448,
 *    smallest 0.5*2^-9).
 *  - "[CUDA] MatMulNBits 8-bit: wide fp16 M=1 kernel for decode GEMVs",
 *    Description: per-block scale and zero point, (q - zp) formed exactly.
 *  - "[CUDA] Batched small-M GEMV for MatMulNBits (4-bit/8-bit)", Description:
 *    the [N, blocks, blob] weight layout with packed 4-bit zero points.
 *
 * Readings where the pages are silent (each listed with its reason in the design
 * notes): E4M3 is the OCP E4M3FN variant (max 448, NaN = S.1111.111, no infinity);
 * nibbles are packed low nibble first, for weights and for 4-bit zero points; the
 * 4-bit zero-point row of a column holds ceil(blocks/2) bytes; a missing zero
 * point means 2^(bits-1); the NVFP4 tensor scale multiplies.
 *
 * Optional bias ("[CUDA] Block-scaled MatMul decode GEMV: ...", reviewed-changes
 * table: the FP8 and FP4 tests cover a bias; "[CUDA] Pin FP8 GEMV residency for
 * grids just past two blocks per SM", a timeline note: the tests cover an optional
 * bias): one value per output column in the activation dtype, added to the product
 * of every row, Y[m, n] = sum_k A[m, k] * dequant(W)[n, k] + bias[n] (the tensor
 * scale is part of dequant(W) and does not touch the bias). S stays the sum of
 * |a*w|: the bias is added once, exactly, in float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_U4 = 1, ORC_U8 = 2, ORC_FP8 = 3, ORC_NVFP4 = 4 };
enum { ORC_F16 = 1, ORC_BF16 = 2 };

/* Mirror of the Python-side ctypes structure. */
typedef struct {
    int32_t format;
    int32_t act_dtype;
    int32_t block_size;
    int32_t pad_;
    int64_t N;
    int64_t K;
    const uint8_t *W;
    const void *scales;
    const uint8_t *zp; /* NULL allowed for u4/u8 */
    double tensor_scale;
    const uint16_t *bias; /* NULL, or [N] activation-dtype bits added to every row */
} orc_problem;

/* ---------------------------------------------------------------------------------
 * Scalar decoders from the bit fields of each format.
 */

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0. Exponent 0 is
 * the subnormal binade with step 0.5. */
static double e2m1_closed_form(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. Exponent 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
static double e4m3_closed_form(unsigned code) {
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double half_bits_to_double(uint16_t h) {
    unsigned s = (h >> 15) & 1u, e = (h >> 10) & 31u, f = h & 1023u;
    double mag;
    if (e == 31) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)f, -24);
    else mag = ldexp(1.0 + (double)f / 1024.0, (int)e - 15);
    return s ? -mag : mag;
}

/* bfloat16: sign, 8-bit exponent (bias 127), 7-bit fraction. */
static double bf16_bits_to_double(uint16_t b) {
    unsigned s = (b >> 15) & 1u, e = (b >> 7) & 255u, f = b & 127u;
    double mag;
    if (e == 255) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)f, -133);
    else mag = ldexp(1.0 + (double)f / 128.0, (int)e - 127);
    return s ? -mag : mag;
}

/* Exhaustive tables built once from the closed forms above. */
static double g_e2m1[16];
static double g_e4m3[256];
static int g_tables_ready = 0;

static void build_tables(void) {
    unsigned c;
    if (g_tables_ready) return;
    for (c = 0; c < 16; ++c) g_e2m1[c] = e2m1_closed_form(c);
    for (c = 0; c < 256; ++c) g_e4m3[c] = e4m3_closed_form(c);
    g_tables_ready = 1;
}

/* ---------------------------------------------------------------------------------
 * Exported decoders (so the test suite can pin them against library routines).
 */
void oracle_tables(double *e2m1_out, double *e4m3_out) {
    build_tables();
    memcpy(e2m1_out, g_e2m1, sizeof g_e2m1);
    memcpy(e4m3_out, g_e4m3, sizeof g_e4m3);
}

void oracle_decode_f16(const uint16_t *bits, int64_t count, double *out) {
    int64_t i;
    for (i = 0; i < count; ++i) out[i] = half_bits_to_double(bits[i]);
}

void oracle_decode_bf16(const uint16_t *bits, int64_t count, double *out) {
    int64_t i;
    for (i = 0; i < count; ++i) out[i] = bf16_bits_to_double(bits[i]);
}

/* ---------------------------------------------------------------------------------
 * One dequantized weight element w[n, k] in float64 (exact in every format).
 */
static double activation(const orc_problem *p, const uint16_t *A, int64_t m, int64_t k) {
    uint16_t bits = A[m * p->K + k];
    return p->act_dtype == ORC_BF16 ? bf16_bits_to_double(bits) : half_bits_to_double(bits);
}

static double dequant_element(const orc_problem *p, int64_t n, int64_t k) {
    const int64_t bs = p->block_size;
    const int64_t nblk = p->K / bs;
    const int64_t b = k / bs;      /* block along K */
    const int64_t j = k - b * bs;  /* position inside the block */
    switch (p->format) {
    case ORC_U4: {
        /* blob of block b of column n: bs/2 bytes; byte j/2, low nibble for even j */
        const uint8_t *blob = p->W + (n * nblk + b) * (bs / 2);
        uint8_t byte = blob[j / 2];
        int q = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        int z = 8;
        double s = half_bits_to_double(((const uint16_t *)p->scales)[n * nblk + b]);
        if (p->zp) {
            int64_t zrow = (nblk + 1) / 2;
            uint8_t zb = p->zp[n * zrow + b / 2];
            z = (b % 2 == 0) ? (zb & 0x0F) : (zb >> 4);
        }
        return s * (double)(q - z); /* integer difference is exact */
    }
    case ORC_U8: {
        const uint8_t *blob = p->W + (n * nblk + b) * bs;
        int q = blob[j];
        int z = p->zp ? p->zp[n * nblk + b] : 128;
        double s = half_bits_to_double(((const uint16_t *)p->scales)[n * nblk + b]);
        return s * (double)(q - z);
    }
    case ORC_FP8: {
        uint8_t code = p->W[n * p->K + k];
        double s = (double)((const float *)p->scales)[n * nblk + b];
        return s * g_e4m3[code];
    }
    case ORC_NVFP4: {
        uint8_t byte = p->W[n * (p->K / 2) + k / 2];
        unsigned code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        double sc = g_e4m3[((const uint8_t *)p->scales)[n * (p->K / 16) + k / 16]];
        return p->tensor_scale * sc * g_e2m1[code];
    }
    default:
        return NAN;
    }
}

/* The bias of column n in float64 (0 without a bias). */
static double bias_value(const orc_problem *p, int64_t n) {
    if (!p->bias) return 0.0;
    return p->act_dtype == ORC_F16 ? half_bits_to_double(p->bias[n]) : bf16_bits_to_double(p->bias[n]);
}

static int check_problem(const orc_problem *p, int M) {
    if (!p || !p->W || !p->scales) return 1;
    if (p->N < 1 || p->K < 1 || M < 1) return 2;
    if (p->block_size < 1 || p->K % p->block_size) return 3;
    if (p->format == ORC_NVFP4 && p->block_size != 16) return 3;
    if ((p->format == ORC_U4 || p->format == ORC_NVFP4) && (p->block_size % 2)) return 3;
    if (p->format < ORC_U4 || p->format > ORC_NVFP4) return 4;
    if (p->act_dtype != ORC_F16 && p->act_dtype != ORC_BF16) return 4;
    return 0;
}

double oracle_dequant(const orc_problem *p, int64_t n, int64_t k) {
    build_tables();
    return dequant_element(p, n, k);
}

/* Dequantize whole columns [n0, n0+count) into out[count, K] (float64). */
int oracle_dequant_columns(const orc_problem *p, int64_t n0, int64_t count, double *out) {
    int64_t i, k;
    int rc = check_problem(p, 1);
    if (rc) return rc;
    build_tables();
    for (i = 0; i < count; ++i)
        for (k = 0; k < p->K; ++k) out[i * p->K + k] = dequant_element(p, n0 + i, k);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Full product. Y and S are [M, N] float64. Columns are independent, so they are
 * shared out over ``nthreads`` OpenMP threads (<= 0: the runtime default).
 */
int oracle_gemv(const orc_problem *p, const uint16_t *A, int M, double *Y, double *S, int nthreads) {
    int64_t n;
    int rc = check_problem(p, M);
    if (rc) return rc;
    if (!A || !Y || !S) return 1;
    build_tables();
#ifdef _OPENMP
    /* a thread count for this call only (the process-wide default stays as it is) */
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
#pragma omp parallel num_threads(nt)
    {
        double *w = (double *)malloc((size_t)p->K * sizeof(double));
#pragma omp for schedule(static)
        for (n = 0; n < p->N; ++n) {
            int64_t k;
            int m;
            for (k = 0; k < p->K; ++k) w[k] = dequant_element(p, n, k);
            for (m = 0; m < M; ++m) {
                double y = 0.0, s = 0.0;
                for (k = 0; k < p->K; ++k) {
                    double t = activation(p, A, m, k) * w[k];
                    y += t;
                    s += fabs(t);
                }
                Y[(int64_t)m * p->N + n] = y + bias_value(p, n);
                S[(int64_t)m * p->N + n] = s;
            }
        }
        free(w);
    }
    return 0;
}

/* Selected outputs only: point i is (ms[i], ns[i]). For full-size checks where the
 * whole product would take too long on the host. */
int oracle_gemv_points(const orc_problem *p, const uint16_t *A, int M, int64_t npts,
                       const int32_t *ms, const int64_t *ns, double *Y, double *S) {
    int64_t i;
    int rc = check_problem(p, M);
    if (rc) return rc;
    if (!A || !ms || !ns || !Y || !S) return 1;
    build_tables();
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < npts; ++i) {
        double y = 0.0, s = 0.0;
        int64_t k;
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= p->N) {
            Y[i] = NAN;
            S[i] = NAN;
            continue;
        }
        for (k = 0; k < p->K; ++k) {
            double t = activation(p, A, ms[i], k) * dequant_element(p, ns[i], k);
            y += t;
            s += fabs(t);
        }
        Y[i] = y + bias_value(p, ns[i]);
        S[i] = s;
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
