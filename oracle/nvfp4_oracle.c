/*
 * nvfp4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU definition of the NVFP4 block-scaled grouped GEMM.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code, header, table or constant with the HIP
 * path in nvfp4_block_scaled_grouped_amd/.
 *
 * What it computes (kernelindex page kernelbot-nvfp4-group-gemm-444497, the
 * kernel-source header comment; page kernelbot-nvfp4-group-gemm-505431,
 * custom_kernel_fallback): for every group i,
 *
 *     C_i[m][n] = fp16( sum_k  a(m,k) * sfa(m, k/16) * b(n,k) * sfb(n, k/16) )
 *
 * with a, b FP4 E2M1 codes (two per byte, K-contiguous), sfa, sfb FP8 E4M3
 * scales, one per 16 consecutive K of a row (page 505431, apply_scale_factors:
 * each scale is repeated 16 times along K), and C_i row-major M_i x N_i fp16.
 *
 * The sum is formed EXACTLY (int64 fixed point, see oracle_dot) and rounded
 * once, to nearest-even, to fp16; overflow gives +-inf.  This is the exact
 * value that the pages' fp32-accumulating hardware approximates, so there is
 * exactly one correct fp16 output per element.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoding */

/* E2M1 from its bit fields: 1 sign bit, 2 exponent bits, 1 mantissa bit,
 * exponent bias 1 (page 505431, "FP4 E2M1 Dequantization" block).  Exponent
 * field 0 is subnormal: 0.5 * mantissa.  Returned as twice the value, an
 * integer in [-12, 12], so later arithmetic stays exact. */
int oracle_e2m1_x2(uint8_t code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int f = code & 1;
    int twice; /* 2 * |value| */
    if (e == 0)
        twice = f;                      /* 0.5 * f  -> 2*value = f        */
    else
        twice = (2 + f) << (e - 1);     /* 2^(e-1) * (1 + f/2) * 2        */
    return s ? -twice : twice;
}

double oracle_e2m1(uint8_t code)
{
    int t = oracle_e2m1_x2(code);
    if (t == 0 && (code & 8)) return -0.0;
    return 0.5 * (double)t;
}

/* E4M3 ("E4M3FN", OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; no infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is
 * subnormal.  Returned as 512 times the value, an integer in
 * [-229376, 229376], with *is_nan set for the NaN codes. */
int64_t oracle_e4m3_x512(uint8_t code, int* is_nan)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int f = code & 7;
    int64_t mag;
    *is_nan = (e == 15 && f == 7);
    if (*is_nan) return 0;
    if (e == 0)
        mag = f;                                   /* f * 2^-9 -> *512 = f */
    else
        mag = (int64_t)(8 + f) << (e - 1);         /* 2^(e-7)(1+f/8)*512   */
    return s ? -mag : mag;
}

double oracle_e4m3(uint8_t code)
{
    int nan;
    int64_t v = oracle_e4m3_x512(code, &nan);
    if (nan) return NAN;
    if (v == 0 && (code & 0x80)) return -0.0;
    return (double)v / 512.0;
}

/* Element k of a packed FP4 row: byte k/2, low nibble for even k, high nibble
 * for odd k (page 505431, dequantize_fp4: low nibble first when the two
 * nibbles of a byte are interleaved). */
static inline uint8_t fp4_at(const uint8_t* row, int64_t k)
{
    uint8_t byte = row[k >> 1];
    return (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
}

/* ------------------------------------------------------------ fp16 rounding */

/* Round the exact value X * 2^-20 to IEEE binary16, round-to-nearest-even,
 * overflow to +-inf, exact zero to +0.  Done on the integer itself so there
 * is exactly one rounding. */
uint16_t oracle_round_f16_fixed20(int64_t X)
{
    uint16_t sign = 0;
    uint64_t v;
    if (X == 0) return 0;
    if (X < 0) { sign = 0x8000; v = (uint64_t)(-(X + 1)) + 1; }
    else v = (uint64_t)X;

    /* Values below 2^-14 (v < 64) are fp16 subnormals, spaced 2^-24, and a
     * multiple of 2^-20 is 16 of those steps: exact. */
    if (v < 64) return (uint16_t)(sign | (uint16_t)(v * 16));

    int e = 63 - __builtin_clzll(v);      /* v in [2^e, 2^(e+1)), e >= 6    */
    int E = e - 20;                        /* unbiased binary exponent       */
    uint64_t q;                            /* 11-bit significand 1.xxxxxxxxxx */
    int shift = e - 10;
    if (shift <= 0) {
        q = v << (-shift);
    } else {
        uint64_t rem = v & ((1ULL << shift) - 1);
        uint64_t half = 1ULL << (shift - 1);
        q = v >> shift;
        if (rem > half || (rem == half && (q & 1))) q++;
        if (q == 2048) { q = 1024; E++; }
    }
    if (E > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024));
}

/* Round a double to fp16 (RNE, overflow to inf) when the double is an exact
 * multiple of 2^-20 below 2^43 in magnitude; NaN maps to 0x7E00. */
uint16_t oracle_round_f16_double(double x)
{
    if (isnan(x)) return 0x7E00;
    return oracle_round_f16_fixed20((int64_t)ldexp(x, 20));
}

/* -------------------------------------------------------------- contraction */

/* One output: the exact sum over k of the four decoded factors, in units of
 * 2^-20 (2*a * 512*sfa * 2*b * 512*sfb = a*sfa*b*sfb * 2^20).  Every term is
 * below 2^43 in magnitude, so K < 2^20 terms cannot overflow int64.
 * *nan is set when any scale used is a NaN code. */
static int64_t oracle_dot(const uint8_t* arow, const uint8_t* sfarow,
                          const uint8_t* brow, const uint8_t* sfbrow,
                          int64_t K, int* nan)
{
    int64_t acc = 0;
    *nan = 0;
    for (int64_t k = 0; k < K; ++k) {
        int na, nb;
        int64_t sa = oracle_e4m3_x512(sfarow[k / 16], &na);
        int64_t sb = oracle_e4m3_x512(sfbrow[k / 16], &nb);
        if (na || nb) { *nan = 1; continue; }
        int64_t a = oracle_e2m1_x2(fp4_at(arow, k));
        int64_t b = oracle_e2m1_x2(fp4_at(brow, k));
        acc += (a * sa) * (b * sb);
    }
    return acc;
}

/* Same output accumulated in double from the decoded real values.  For the
 * inputs used here every partial sum is exactly representable, so this must
 * agree with oracle_dot bit for bit; the tests check that. */
static double oracle_dot_f64(const uint8_t* arow, const uint8_t* sfarow,
                             const uint8_t* brow, const uint8_t* sfbrow,
                             int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = oracle_e2m1(fp4_at(arow, k)) * oracle_e4m3(sfarow[k / 16]);
        double b = oracle_e2m1(fp4_at(brow, k)) * oracle_e4m3(sfbrow[k / 16]);
        acc += a * b;
    }
    return acc;
}

/* One element C_i[m][n] of group i described by single pointers.  Writes the
 * fp16 bits to *c16 and the exact value (as a double; exact below 2^53 units)
 * to *cexact.  Returns 0, or -1 on a bad index. */
int oracle_gemm_element(int M, int N, int K,
                        const uint8_t* A, const uint8_t* B,
                        const uint8_t* SFA, const uint8_t* SFB,
                        int m, int n, uint16_t* c16, double* cexact)
{
    if (m < 0 || m >= M || n < 0 || n >= N || K % 16 != 0) return -1;
    int nan;
    int64_t X = oracle_dot(A + (int64_t)m * (K / 2), SFA + (int64_t)m * (K / 16),
                           B + (int64_t)n * (K / 2), SFB + (int64_t)n * (K / 16),
                           K, &nan);
    if (nan) { *c16 = 0x7E00; *cexact = NAN; return 0; }
    *c16 = oracle_round_f16_fixed20(X);
    *cexact = ldexp((double)X, -20);
    return 0;
}

/* The grouped GEMM.  All arrays are host memory.  Cexact may be NULL; when
 * given, Cexact[i] receives M_i*N_i doubles (row-major) with the exact sums.
 * use_f64 selects the double accumulation instead of int64 (cross-check).
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad sizes. */
int oracle_group_gemm(int g, const int* M, const int* N, const int* K,
                      const uint8_t* const* A, const uint8_t* const* B,
                      const uint8_t* const* SFA, const uint8_t* const* SFB,
                      uint16_t* const* C, double* const* Cexact,
                      int use_f64, int nthreads)
{
    if (g < 0) return -1;
    for (int i = 0; i < g; ++i)
        if (M[i] < 0 || N[i] < 0 || K[i] < 0 || K[i] % 16 != 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int i = 0; i < g; ++i) {
        const int64_t Mi = M[i], Ni = N[i], Ki = K[i];
        const uint8_t *Ai = A[i], *Bi = B[i], *SAi = SFA[i], *SBi = SFB[i];
        uint16_t* Ci = C[i];
        double* Xi = Cexact ? Cexact[i] : NULL;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = 0; m < Mi; ++m) {
            for (int64_t n = 0; n < Ni; ++n) {
                const uint8_t* ar = Ai + m * (Ki / 2);
                const uint8_t* sar = SAi + m * (Ki / 16);
                const uint8_t* br = Bi + n * (Ki / 2);
                const uint8_t* sbr = SBi + n * (Ki / 16);
                uint16_t out;
                double exact;
                if (use_f64) {
                    exact = oracle_dot_f64(ar, sar, br, sbr, Ki);
                    out = oracle_round_f16_double(exact);
                } else {
                    int nan;
                    int64_t X = oracle_dot(ar, sar, br, sbr, Ki, &nan);
                    out = nan ? (uint16_t)0x7E00 : oracle_round_f16_fixed20(X);
                    exact = nan ? NAN : ldexp((double)X, -20);
                }
                Ci[m * Ni + n] = out;
                if (Xi) Xi[m * Ni + n] = exact;
            }
        }
    }
    return 0;
}

/* Decode a packed FP4 matrix with its per-16 E4M3 scales into doubles
 * (rows x K, row-major): the dequantisation step alone. */
int oracle_dequant(int rows, int K, const uint8_t* X, const uint8_t* SFX, double* out)
{
    if (rows < 0 || K < 0 || K % 16 != 0) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = oracle_e2m1(fp4_at(X + r * (K / 2), k)) *
                             oracle_e4m3(SFX[r * (K / 16) + k / 16]);
    return 0;
}

/* ------------------------------------------------------ blocked scale layout
 *
 * The layout the pages' kernels read their scales in (page 482006, function
 * to_blocked_gpu of its cuBLAS path, and the scale-factor layout atom of its
 * CuTe kernel; page 505431, the scale-factor copy comment block).  Taken in
 * the order those passages describe it:
 *   1. the rows x cols scale matrix is padded with zeros to a multiple of 128
 *      rows and of 4 columns;
 *   2. it is cut into blocks of 128 rows x 4 columns; the blocks of one
 *      128-row band follow each other in column order, the bands in row
 *      order, 512 bytes per block;
 *   3. inside a block the 128 rows form 4 groups of 32; the block is 32 runs
 *      of 16 bytes, run j holding, in turn, the 4 columns of rows j, j + 32,
 *      j + 64 and j + 96.
 * oracle_block_scales writes a blocked array (pad bytes = pad_value) from a
 * row-major one; oracle_unblock_scales reads the row-major matrix back. */
static int64_t blocked_pos(int64_t r, int64_t c, int64_t band_blocks)
{
    const int64_t band = r / 128, rb = r % 128;   /* step 2: which band, row in band */
    const int64_t block = band * band_blocks + c / 4;
    const int64_t run = rb % 32, group = rb / 32;  /* step 3 */
    return block * 512 + run * 16 + group * 4 + c % 4;
}

int64_t oracle_blocked_scale_bytes(int rows, int cols)
{
    if (rows < 0 || cols < 0) return -1;
    return ((int64_t)(rows + 127) / 128) * 128 * (((int64_t)cols + 3) / 4 * 4);
}

int oracle_block_scales(int rows, int cols, const uint8_t* plain, uint8_t* blocked, uint8_t pad_value)
{
    const int64_t n = oracle_blocked_scale_bytes(rows, cols);
    if (n < 0) return -1;
    memset(blocked, pad_value, (size_t)n);
    const int64_t band_blocks = ((int64_t)cols + 3) / 4;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) blocked[blocked_pos(r, c, band_blocks)] = plain[r * cols + c];
    return 0;
}

int oracle_unblock_scales(int rows, int cols, const uint8_t* blocked, uint8_t* plain)
{
    if (rows < 0 || cols < 0) return -1;
    const int64_t band_blocks = ((int64_t)cols + 3) / 4;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) plain[r * cols + c] = blocked[blocked_pos(r, c, band_blocks)];
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
