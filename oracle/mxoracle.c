/*
 * mxoracle.c -- plain, slow CPU oracle for the MXFP4 GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * What it computes (sources are the kernelindex.com pages for the
 * amd-mxfp4-mm leaderboard on MI355X):
 *
 *   - MXFP4 quantisation of a bf16 row-major matrix along K in groups of 32,
 *     following the "Software MXFP4 quant" section of submission 755056
 *     (function _mxfp4_quant_tile); the same rule appears in submission
 *     748756 (hw_pack_mxfp4) and in the HIP quantiser of submission 755056
 *     (mxfp4_quant_shuffled), the latter without the clamp:
 *        1. amax = max |x| over the group, exact in fp32;
 *        2. R = (bits(amax) + 0x00200000) & 0xFF800000   -- amax rounded to
 *           a power of two, rounding up when the significand is >= 1.75;
 *        3. s = clamp(E(R) - 129, -127, 127), scale byte = s + 127 (e8m0);
 *        4. q = x * 2^-s (exact here: fp64 ldexp);
 *        5. e2m1 code = nearest of {0,0.5,1,1.5,2,3,4,6}, ties to the even
 *           code, |q| >= 6 saturates to code 7; bit 3 = sign bit of x
 *           (kept also when the magnitude rounds to 0, so -0.25 -> 0x8);
 *        6. two codes per byte, even k in the low nibble.
 *   - Dequantisation: (-1)^b3 * VAL[code & 7] * 2^(byte - 127).
 *   - The GEMM C[m,n] = bf16_RNE( sum_k deqA[m,k] * deqB[n,k] ), the sum in
 *     fp64 and rounded once from fp64 to bf16.  Every product has at most
 *     4 significant bits, so for inputs whose group scales span a few dozen
 *     binades the fp64 sum is exact and C is the correctly rounded result.
 *
 * Readings where the pages leave room (each also listed in the design notes):
 *   - the clamp of s to [-127, 127] is applied (four of five copies do so);
 *   - a scale byte of 0 means 2^-127, never a division by zero;
 *   - ties of the e2m1 rounding go to the even code (round-to-nearest-even);
 *   - inputs are finite; NaN / Inf inputs are outside the contract.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC mxoracle.c -o libmxoracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The eight e2m1 magnitudes, indexed by the 3-bit code (OCP MX e2m1). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t float_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* e2m1 magnitude code of a non-negative q: nearest representable value,
 * ties to the even code, saturating at 6 (code 7). */
int mxo_e2m1_code(double q) {
    if (q >= 6.0) return 7;
    int best = 0;
    double best_d = fabs(q - kE2M1[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(q - kE2M1[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* e8m0 scale byte of one group from its fp32 amax (steps 2 and 3). */
int mxo_scale_byte(float amax) {
    uint32_t r = (float_bits(amax) + 0x00200000u) & 0xFF800000u;
    int e = (int)(r >> 23);
    int s = e - 129;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s + 127;
}

/* Quantise rows x K bf16 (row stride ld elements) into packed e2m1 codes
 * [rows, K/2] and e8m0 bytes [rows, K/32].  K must be a multiple of 32.
 * Returns 0, or -1 on bad arguments. */
int mxo_quant(const uint16_t* x, int rows, int K, int ld,
              uint8_t* codes, uint8_t* scales) {
    if (rows < 0 || K <= 0 || K % 32 != 0 || ld < K) return -1;
    const int G = K / 32;
    for (int r = 0; r < rows; ++r) {
        const uint16_t* xr = x + (size_t)r * ld;
        for (int g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float v = fabsf(bf16_to_float(xr[g * 32 + i]));
                if (v > amax) amax = v;
            }
            int byte = mxo_scale_byte(amax);
            int s = byte - 127;
            scales[(size_t)r * G + g] = (uint8_t)byte;
            for (int i = 0; i < 32; i += 2) {
                int nib[2];
                for (int j = 0; j < 2; ++j) {
                    uint16_t h = xr[g * 32 + i + j];
                    double q = ldexp((double)bf16_to_float(h), -s);
                    int code = mxo_e2m1_code(fabs(q));
                    if (h & 0x8000u) code |= 8;
                    nib[j] = code;
                }
                codes[(size_t)r * (K / 2) + (g * 32 + i) / 2] =
                    (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
    }
    return 0;
}

/* Value of one code under one scale byte. */
double mxo_decode(int code, int byte) {
    double v = ldexp(kE2M1[code & 7], byte - 127);
    return (code & 8) ? -v : v;
}

/* Dequantise [rows, K/2] codes + [rows, K/32] bytes into fp64 [rows, K]. */
int mxo_dequant(const uint8_t* codes, const uint8_t* scales, int rows, int K,
                double* out) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
    const int G = K / 32;
    for (int r = 0; r < rows; ++r)
        for (int k = 0; k < K; ++k) {
            uint8_t b = codes[(size_t)r * (K / 2) + k / 2];
            int code = (k & 1) ? (b >> 4) : (b & 0xF);
            out[(size_t)r * K + k] = mxo_decode(code, scales[(size_t)r * G + k / 32]);
        }
    return 0;
}

/* Round an fp64 value once to bf16 (round to nearest, ties to even),
 * including bf16 subnormals and overflow to infinity. */
uint16_t mxo_bf16_from_double(double d) {
    if (isnan(d)) return 0x7FC0u;
    uint16_t sign = signbit(d) ? 0x8000u : 0;
    double a = fabs(d);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;        /* bf16 subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - 7);
    double r = nearbyint(a / quantum) * quantum;   /* default mode: RNE */
    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    if (r > ldexp(255.0 / 128.0, 127)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;            /* exact: r has <= 8 significant bits */
    return (uint16_t)(sign | (uint16_t)(float_bits(f) >> 16));
}

/* C[m,n] = bf16_RNE( sum_k Ad[m,k] * Bd[n,k] ) with an fp64 accumulator.
 * Ad is [M,K], Bd is [N,K] (both fp64, row-major), C is [M,N] bf16 bits. */
int mxo_gemm_dequantised(const double* Ad, const double* Bd, int M, int N, int K,
                         uint16_t* C) {
    if (M < 0 || N < 0 || K < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const double* b = Bd + (size_t)n * K;
        for (int m = 0; m < M; ++m) {
            const double* a = Ad + (size_t)m * K;
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += a[k] * b[k];
            C[(size_t)m * N + n] = mxo_bf16_from_double(acc);
        }
    }
    return 0;
}

/* Exact fp64 values of n bf16 bit patterns (a bf16 is the upper half of an
 * fp32, so the widening is exact). */
int mxo_bf16_to_double(const uint16_t* x, long long n, double* out) {
    if (n < 0) return -1;
    for (long long i = 0; i < n; ++i) out[i] = (double)bf16_to_float(x[i]);
    return 0;
}

/* Number of OpenMP threads the GEMM loop uses (1 without OpenMP). */
int mxo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
