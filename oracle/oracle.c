/*
 * Reference oracle for the W3G128 weight format -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct CPU definition that the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or constant with the HIP library, and the library never calls it.
 *
 * Format (GSQ model card "Llama-3.1-70B-Instruct-3Bit-GSQ", sections
 * "Quantization details" and "Storage layout"):
 *   - a quantized Linear with original weight [N = out_features, K = in_features]
 *     stores `weight` as int32 [N, 3K/32] holding exact-width 3-bit codes with no
 *     padding, and `weight_scale` as bf16 [N, K/128], one scale per 128 inputs;
 *   - the codebook is a symmetric integer grid times the group scale, with no
 *     zero point.
 * Readings taken where the card is silent (each is listed with its reason in
 * the design notes):
 *   - bit order: each row is one little-endian bitstream; code k occupies
 *     stream bits 3k, 3k+1, 3k+2 (its least significant bit first), and stream
 *     bit j is bit (j mod 32) of word (j div 32) of that row;
 *   - value map: a code c in 0..7 stands for the integer q = c - 4, so the
 *     weight is s * (c - 4) with s = weight_scale[n][k div 128];
 *   - dequantize-to-bf16 rounds the exact product once, to nearest-even.
 *
 * Every function loops in the most literal way: one bit, one term at a time.
 * Floating point is fp64; each product x * (c - 4) * s is exact in fp64 (at
 * most 8 + 3 + 8 significant bits), so the only rounding is the summation.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* bf16 bit pattern -> double.  bf16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Read stream bit j of one packed row (LSB-first across 32-bit words). */
static int stream_bit(const uint32_t *row_words, int64_t j)
{
    return (int)((row_words[j >> 5] >> (j & 31)) & 1u);
}

/* Code k of one packed row: bits 3k (LSB), 3k+1, 3k+2 (MSB). */
static int code_at(const uint32_t *row_words, int64_t k)
{
    int c = 0;
    for (int b = 0; b < 3; ++b)
        c |= stream_bit(row_words, 3 * k + b) << b;
    return c;
}

/* Words per packed row: 3 bits per weight, 32 bits per word. */
int64_t oracle_words_per_row(int64_t K) { return (3 * K) / 32; }

/* Scales per row: one per group of 128 inputs. */
int64_t oracle_groups_per_row(int64_t K) { return K / 128; }

/* Store code c (0..7) of weight k into a zeroed row: its bit b is stream bit
 * 3k + b, i.e. bit (3k + b) mod 32 of word (3k + b) div 32. */
static void put_code(uint32_t *row, int64_t k, int c)
{
    for (int b = 0; b < 3; ++b) {
        if ((c >> b) & 1) {
            int64_t j = 3 * k + b;
            row[j >> 5] |= 1u << (j & 31);
        }
    }
}

/*
 * pack: codes uint8 [N][K] (values 0..7) -> words uint32 [N][3K/32].
 * Returns -1 if a code is above 7, -2 if K is not a multiple of 128, else 0.
 * Sets one stream bit at a time.
 */
int oracle_pack(const uint8_t *codes, uint32_t *words, int64_t N, int64_t K)
{
    if (K % 128 != 0)
        return -2;
    int64_t W = oracle_words_per_row(K);
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = words + n * W;
        for (int64_t w = 0; w < W; ++w)
            row[w] = 0u;
        for (int64_t k = 0; k < K; ++k) {
            int c = codes[n * K + k];
            if (c > 7)
                return -1;
            put_code(row, k, c);
        }
    }
    return 0;
}

/*
 * repack_w4c: the 4-bit-container intermediate uint32 [N][K/8] -> words
 * uint32 [N][3K/32].  The GSQ model card ("Storage layout", the note on the
 * compressed-tensors pack-quantized shards) says only that training writes
 * the 3-bit codebook padded into a 4-bit INT32 container before the
 * checkpoint is re-packed to exact width.  Reading taken: weight k of row n
 * is nibble k % 8 of word k / 8 of that row, counted from the least
 * significant nibble; the nibble's low 3 bits are its code c (the same code
 * as the exact-width stream) and its top bit is padding, ignored.  The code
 * is then stored exactly as pack() stores it, bit by bit.
 */
int oracle_repack_w4c(const uint32_t *w4, uint32_t *words, int64_t N, int64_t K)
{
    if (K % 128 != 0)
        return -2;
    int64_t W = oracle_words_per_row(K);
    int64_t W4 = K / 8;
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = words + n * W;
        for (int64_t w = 0; w < W; ++w)
            row[w] = 0u;
        for (int64_t k = 0; k < K; ++k) {
            uint32_t nibble = (w4[n * W4 + k / 8] >> (4 * (k % 8))) & 0xFu;
            int c = (int)(nibble & 7u);
            put_code(row, k, c);
        }
    }
    return 0;
}

/* unpack: words uint32 [N][3K/32] -> codes uint8 [N][K]. */
int oracle_unpack(const uint32_t *words, uint8_t *codes, int64_t N, int64_t K)
{
    if (K % 128 != 0)
        return -2;
    int64_t W = oracle_words_per_row(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)code_at(words + n * W, k);
    return 0;
}

/*
 * Round a binary32 value to bf16, nearest-even, on its bit pattern.
 * NaN maps to a quiet NaN of the same sign; infinities pass through.
 */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * dequant: words [N][3K/32] + scales bf16 [N][K/128] -> w bf16 [N][K],
 * w[n][k] = bf16_rne( (c - 4) * s[n][k/128] ).
 * The product is formed in fp64, where it is exact, then narrowed to binary32
 * (still exact: at most 10 significant bits) and rounded once to bf16.
 */
int oracle_dequant_bf16(const uint32_t *words, const uint16_t *scales, uint16_t *w,
                        int64_t N, int64_t K)
{
    if (K % 128 != 0)
        return -2;
    int64_t W = oracle_words_per_row(K);
    int64_t G = oracle_groups_per_row(K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int c = code_at(words + n * W, k);
            double s = bf16_bits_to_double(scales[n * G + k / 128]);
            double v = (double)(c - 4) * s;
            w[n * K + k] = float_to_bf16_rne((float)v);
        }
    }
    return 0;
}

/*
 * gemm over a list of output rows:
 *   y[m][i] = sum_k x[m][k] * (c[row_i][k] - 4) * s[row_i][k/128]
 *   a[m][i] = sum_k | same term |
 * x is bf16 [M][K]; words/scales are the full matrices [N][..]; rows[] lists
 * the nrows output features to evaluate; y and a are fp64 [M][nrows].
 * This is Y = X * dequant(W)^T, the product the fused kernels compute, with
 * the exact (unrounded) weight s * (c - 4).
 * Rows are independent; OpenMP spreads them over the host cores.
 */
int oracle_gemm_rows(const uint16_t *x, const uint32_t *words, const uint16_t *scales,
                     const int64_t *rows, int64_t nrows, int64_t M, int64_t N, int64_t K,
                     double *y, double *a)
{
    if (K % 128 != 0)
        return -2;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= N)
            return -3;
    int64_t W = oracle_words_per_row(K);
    int64_t G = oracle_groups_per_row(K);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = rows[i];
        const uint32_t *row = words + n * W;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int c = code_at(row, k);
                double s = bf16_bits_to_double(scales[n * G + k / 128]);
                double xv = bf16_bits_to_double(x[m * K + k]);
                double t = xv * (double)(c - 4) * s;
                acc += t;
                acc_abs += fabs(t);
            }
            y[m * nrows + i] = acc;
            a[m * nrows + i] = acc_abs;
        }
    }
    return 0;
}

/* Number of OpenMP threads the gemm above will use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
