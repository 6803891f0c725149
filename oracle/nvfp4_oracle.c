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

/* ------------------------------------------------------------------- MXFP4
 *
 * The MX form of the product (page 505431 names MX block scaling beside the
 * NVFP4 one: one block-scaled MMA kind covers both, and its instruction
 * descriptor has a scale-type field; page 444497's header comment speaks of
 * MX block scaling).  The pages do not define it; it is read as the OCP MX
 * format: the same E2M1 codes, one E8M0 scale per 32 consecutive K of a row,
 * E8M0 an unsigned 8-bit exponent with value 2^(code - 127) and code 0xFF
 * NaN.  For every group, row m and column n:
 *
 *     C[m][n] = fp16( sum_k a(m,k) 2^(sa(m,k/32) - 127) b(n,k) 2^(sb(n,k/32) - 127) )
 *
 * formed exactly and rounded once (round-to-nearest-even, overflow to inf). */
double oracle_e8m0(uint8_t code)
{
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* Exact dot product.  A term is (2a)(2b) 2^(ea + eb - 256), (2a)(2b) an
 * integer of magnitude <= 144 (oracle_e2m1_x2).  With Emin the least
 * exponent sum ea + eb along the row pair, the sum is S 2^(Emin - 256) with S
 * an integer, accumulated in __int128 as long as no term is shifted by more
 * than 96 bits (K <= 2^20 then keeps |S| < 2^124).  Returns 0 and (S, E =
 * Emin - 256), 1 if a scale is NaN, -1 if the exponent spread is too wide. */
static int mx_dot(const uint8_t* arow, const uint8_t* sarow, const uint8_t* brow,
                  const uint8_t* sbrow, int64_t K, __int128* S, int* E)
{
    int emin = 1 << 30;
    for (int64_t b = 0; b < K / 32; ++b) {
        if (sarow[b] == 0xFF || sbrow[b] == 0xFF) return 1;
        const int e = (int)sarow[b] + (int)sbrow[b];
        if (e < emin) emin = e;
    }
    __int128 s = 0;
    for (int64_t k = 0; k < K; ++k) {
        const int shift = (int)sarow[k / 32] + (int)sbrow[k / 32] - emin;
        if (shift > 96) return -1;
        const int p = oracle_e2m1_x2(fp4_at(arow, k)) * oracle_e2m1_x2(fp4_at(brow, k));
        s += (__int128)p * ((__int128)1 << shift);
    }
    *S = s;
    *E = emin - 256;
    return 0;
}

/* S 2^E rounded once to fp16: round-to-nearest-even on the integer itself,
 * overflow to inf, underflow to a signed zero, an exact zero to +0 (the same
 * rules as oracle_round_f16_fixed20, for any binary exponent).  *exact gets
 * S 2^E as a double (rounded if S needs more than 53 bits). */
static uint16_t round_f16_int128(__int128 S, int E, double* exact)
{
    if (S == 0) {
        if (exact) *exact = 0.0;
        return 0;
    }
    const uint16_t sign = S < 0 ? 0x8000 : 0;
    const unsigned __int128 u = S < 0 ? (unsigned __int128)(-S) : (unsigned __int128)S;
    if (exact) *exact = (sign ? -1.0 : 1.0) * ldexp((double)u, E);
    int e = 0;                                  /* u in [2^e, 2^(e+1)) */
    while ((u >> e) > 1) ++e;
    const int V = e + E;                        /* unbiased exponent of the value */
    const int qexp = V >= -14 ? V - 10 : -24;   /* exponent of the last kept bit */
    const int shift = qexp - E;                 /* bits of u below it */
    unsigned __int128 q;
    if (shift <= 0) {
        q = u << (-shift);
    } else if (shift >= 126) {
        q = 0;                                  /* below half the smallest subnormal */
    } else {
        const unsigned __int128 rem = u & (((unsigned __int128)1 << shift) - 1);
        const unsigned __int128 half = (unsigned __int128)1 << (shift - 1);
        q = u >> shift;
        if (rem > half || (rem == half && (q & 1))) q++;
    }
    if (V < -14) return (uint16_t)(sign | (uint16_t)q);   /* subnormal; q == 1024 is the least normal */
    int Ve = V;
    if (q == 2048) {
        q = 1024;
        ++Ve;
    }
    if (Ve > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((Ve + 15) << 10) | (uint16_t)(q - 1024));
}

/* One output element of an MXFP4 group: fp16 bits and the exact value (as a
 * double).  A NaN scale gives NaN; a too-wide exponent spread returns -2. */
int oracle_mx_gemm_element(int M, int N, int K, const uint8_t* A, const uint8_t* B, const uint8_t* SFA,
                           const uint8_t* SFB, int m, int n, uint16_t* c16, double* exact)
{
    if (m < 0 || m >= M || n < 0 || n >= N || K % 32 != 0) return -1;
    __int128 S;
    int E;
    const int rc = mx_dot(A + (int64_t)m * (K / 2), SFA + (int64_t)m * (K / 32), B + (int64_t)n * (K / 2),
                          SFB + (int64_t)n * (K / 32), K, &S, &E);
    if (rc < 0) return -2;
    if (rc == 1) {
        *c16 = 0x7E00;
        *exact = NAN;
        return 0;
    }
    *c16 = round_f16_int128(S, E, exact);
    return 0;
}

/* The MXFP4 grouped GEMM (layouts as oracle_group_gemm, scales M x K/32 and
 * N x K/32).  Returns -2 if some dot product's exponent spread is too wide
 * for the exact sum. */
int oracle_mx_group_gemm(int g, const int* M, const int* N, const int* K, const uint8_t* const* A,
                         const uint8_t* const* B, const uint8_t* const* SFA, const uint8_t* const* SFB,
                         uint16_t* const* C, double* const* Cexact, int nthreads)
{
    if (g < 0) return -1;
    for (int i = 0; i < g; ++i)
        if (M[i] < 0 || N[i] < 0 || K[i] < 0 || K[i] % 32 != 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
    for (int i = 0; i < g; ++i) {
        const int64_t Mi = M[i], Ni = N[i], Ki = K[i];
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
        for (int64_t m = 0; m < Mi; ++m) {
            for (int64_t n = 0; n < Ni; ++n) {
                uint16_t c;
                double x;
                if (oracle_mx_gemm_element(M[i], N[i], K[i], A[i], B[i], SFA[i], SFB[i], (int)m, (int)n, &c, &x) != 0)
                    bad = 1;
                C[i][m * Ni + n] = c;
                if (Cexact) Cexact[i][m * Ni + n] = x;
            }
        }
        (void)Ki;
    }
    return bad ? -2 : 0;
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
