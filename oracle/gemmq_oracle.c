/*
 * gemmq_oracle.c -- the CPU oracle for the packed-weight linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant with the HIP
 * library; every format constant below is written out again on purpose.
 *
 * What it computes is the operation the PocketLLM pages call gemm_quant: a linear
 * layer y = W x evaluated directly on ggml K-quant packed weights (q2_K, q3_K,
 * q4_K, q5_K, q6_K -- the K-quant rung of the pages' width ladder) with
 * the activations quantized to int8 blocks first (PocketLLM README, "What it runs":
 * the K-quant rung is decoded inside the kernel and never widened; molayo article
 * "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++ engine":
 * the CPU gemm_quant quantizes activations to int8 the way llama.cpp does, then runs
 * a packed dot over each weight row).
 *
 * Plain, single-threaded C, built with -O2 -ffp-contract=off.  Each output is
 * computed on its own, so a call over M rows equals M calls over one row byte for
 * byte (the pages' tiled-equals-single-row rule, molayo article, same row).
 *
 * Byte layouts.  The pages name the formats but print no layout; the layouts below
 * are the public ggml K-quant ones (all little-endian):
 *   q4_K, 144 B per 256 weights: f16 d | f16 dmin | 12 B packed 6-bit scales and
 *         mins | 128 B of 4-bit quants.  Sub-block j (32 weights) decodes as
 *         w = d*sc_j*q - dmin*m_j.
 *   q6_K, 210 B per 256 weights: 128 B low nibbles | 64 B 2-bit highs | 16 int8
 *         sub-scales | f16 d.  Sub-block j (16 weights) decodes as w = d*sc_j*(q-32).
 *   q2_K, 84 B per 256 weights: 16 B sub-block bytes (scale in the low nibble,
 *         min in the high nibble) | 64 B of 2-bit quants | f16 d | f16 dmin.
 *         Sub-block j (16 weights) decodes as w = d*sc_j*q - dmin*m_j, q in 0..3.
 *   q3_K, 110 B per 256 weights: 32 B high-bit mask | 64 B of 2-bit low parts |
 *         12 B packed 6-bit scales | f16 d.  Sub-block j (16 weights) decodes as
 *         w = d*(sc_j - 32)*q, q in -4..3 (low part, minus 4 when the high bit is
 *         clear).
 *   q5_K, 176 B per 256 weights: f16 d | f16 dmin | 12 B scales and mins packed
 *         as in q4_K | 32 B high bits | 128 B of 4-bit low parts.  Sub-block j
 *         (32 weights) decodes as w = d*sc_j*q - dmin*m_j, q in 0..31.
 *   q8_K, 292 B per 256 activations: f32 d | 256 int8 | 16 int16 group sums.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms,
 * brute force, an independent packer, a textbook integer GEMM and exact rational
 * sums).  Parity against ggml's own bytes is unpinned: no llama.cpp build and no
 * GGUF file is available, so the layout reading above is pinned only to itself.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OQ2K_BYTES 84
#define OQ3K_BYTES 110
#define OQ4K_BYTES 144
#define OQ5K_BYTES 176
#define OQ6K_BYTES 210
#define OQ8K_BYTES 292
#define OQK 256

/* ---------------------------------------------------------------- helpers */

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static float rd_f32(const uint8_t *p)
{
    float f;
    memcpy(&f, p, 4);
    return f;
}
static void wr_f32(uint8_t *p, float f) { memcpy(p, &f, 4); }
static void wr_i16(uint8_t *p, int v)
{
    uint16_t u = (uint16_t)(int16_t)v;
    p[0] = (uint8_t)(u & 0xff);
    p[1] = (uint8_t)(u >> 8);
}

/* IEEE 754 binary16 -> double, straight from the format's definition:
 * exponent field 0 means subnormal (man * 2^-24), 31 means inf/nan, otherwise
 * (1024 + man) * 2^(exp - 25).  Every binary16 value is exact in double. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);
    return sign ? -v : v;
}

/* q4_K: 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes.
 * Sub-blocks 0..3 keep their value in the low 6 bits of bytes j (scale) and j+4
 * (min); sub-blocks 4..7 take 4 low bits from byte j+4 (scale: low nibble, min:
 * high nibble) and their top 2 bits from the spare top bits of bytes j-4 (scale)
 * and j (min). */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *mn)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* q4_K: 4-bit quant of weight i (0..255).  Each 64-weight group g owns 32 bytes;
 * its first 32 weights are the low nibbles, the next 32 the high nibbles. */
static int q4k_quant(const uint8_t *qs, int i)
{
    int g = i / 64, r = i % 64;
    uint8_t byte = qs[32 * g + (r % 32)];
    return r < 32 ? (byte & 15) : (byte >> 4);
}

/* q6_K: 6-bit quant of weight i (0..255), before the -32 offset.  Each 128-weight
 * half h owns 64 low-nibble bytes and 32 high-bit bytes; inside it, quarter c
 * (32 weights) takes its low 4 bits from byte 32*(c&1)+l (low nibble for c<2,
 * high nibble for c>=2) and its top 2 bits from bits 2c..2c+1 of qh byte l. */
static int q6k_quant(const uint8_t *ql, const uint8_t *qh, int i)
{
    int h = i / 128, c = (i % 128) / 32, l = i % 32;
    uint8_t lowbyte = ql[64 * h + l + 32 * (c & 1)];
    int low = c < 2 ? (lowbyte & 15) : (lowbyte >> 4);
    int high = (qh[32 * h + l] >> (2 * c)) & 3;
    return low | (high << 4);
}

/* q2_K: 2-bit quant of weight i (0..255).  Each 128-weight half h owns 32 bytes;
 * its 32-weight quarter c takes bits 2c..2c+1 of byte l = i % 32. */
static int q2k_quant(const uint8_t *qs, int i)
{
    int h = i / 128, c = (i % 128) / 32, l = i % 32;
    return (qs[32 * h + l] >> (2 * c)) & 3;
}

/* q3_K: quant of weight i in -4..3.  The low two bits are laid out as q2_K's;
 * the third bit is bit 4h+c of mask byte l (h, c, l as for q2_K), and a clear
 * bit subtracts 4. */
static int q3k_quant(const uint8_t *hmask, const uint8_t *qs, int i)
{
    int h = i / 128, c = (i % 128) / 32, l = i % 32;
    int low = (qs[32 * h + l] >> (2 * c)) & 3;
    int high = (hmask[l] >> (4 * h + c)) & 1;
    return high ? low : low - 4;
}

/* q3_K: 6-bit scale of sub-block j (0..15), before the -32 offset.  For
 * j = 4g + k the low four bits are a nibble of byte k (g = 0: low, g = 2: high)
 * or of byte 4 + k (g = 1: low, g = 3: high); the top two bits are bits
 * 2g..2g+1 of byte 8 + k. */
static int q3k_scale(const uint8_t *s, int j)
{
    int g = j / 4, k = j % 4;
    int low = (s[4 * (g & 1) + k] >> (4 * (g >> 1))) & 15;
    int high = (s[8 + k] >> (2 * g)) & 3;
    return low | (high << 4);
}

/* q5_K: 5-bit quant of weight i (0..255).  The low four bits are laid out as
 * q4_K's quants; the fifth is bit 2g + (r >= 32) of byte l of the high-bit
 * array, for 64-weight group g, r = i % 64 and l = r % 32. */
static int q5k_quant(const uint8_t *qh, const uint8_t *qs, int i)
{
    int g = i / 64, r = i % 64, l = r % 32;
    int high = (qh[l] >> (2 * g + (r >= 32))) & 1;
    return q4k_quant(qs, i) | (high << 4);
}

/* Any of the five formats as integers: quants q[256] (offsets applied), the
 * L-weight sub-blocks' scales sc[] and mins mn[] (0 where the format has none),
 * d and dmin (0 where none).  Weight i of sub-block j is d*sc_j*q_i - dmin*mn_j.
 * Returns L (16 or 32), or 0 for an unknown format. */
static int unpack_block(int fmt, const uint8_t *blk, int *q, int *sc, int *mn, double *d,
                        double *dmin)
{
    switch (fmt) {
    case 10: /* q2_K */
        *d = oracle_f16_to_f64(rd_u16(blk + 80));
        *dmin = oracle_f16_to_f64(rd_u16(blk + 82));
        for (int j = 0; j < 16; ++j) {
            sc[j] = blk[j] & 15;
            mn[j] = blk[j] >> 4;
        }
        for (int i = 0; i < OQK; ++i)
            q[i] = q2k_quant(blk + 16, i);
        return 16;
    case 11: /* q3_K */
        *d = oracle_f16_to_f64(rd_u16(blk + 108));
        *dmin = 0.0;
        for (int j = 0; j < 16; ++j) {
            sc[j] = q3k_scale(blk + 96, j) - 32;
            mn[j] = 0;
        }
        for (int i = 0; i < OQK; ++i)
            q[i] = q3k_quant(blk, blk + 32, i);
        return 16;
    case 12: /* q4_K */
        *d = oracle_f16_to_f64(rd_u16(blk));
        *dmin = oracle_f16_to_f64(rd_u16(blk + 2));
        for (int j = 0; j < 8; ++j)
            q4k_scale_min(blk + 4, j, &sc[j], &mn[j]);
        for (int i = 0; i < OQK; ++i)
            q[i] = q4k_quant(blk + 16, i);
        return 32;
    case 13: /* q5_K */
        *d = oracle_f16_to_f64(rd_u16(blk));
        *dmin = oracle_f16_to_f64(rd_u16(blk + 2));
        for (int j = 0; j < 8; ++j)
            q4k_scale_min(blk + 4, j, &sc[j], &mn[j]);
        for (int i = 0; i < OQK; ++i)
            q[i] = q5k_quant(blk + 16, blk + 48, i);
        return 32;
    case 14: /* q6_K */
        *d = oracle_f16_to_f64(rd_u16(blk + 208));
        *dmin = 0.0;
        for (int j = 0; j < 16; ++j) {
            sc[j] = ((const int8_t *)(blk + 192))[j];
            mn[j] = 0;
        }
        for (int i = 0; i < OQK; ++i)
            q[i] = q6k_quant(blk, blk + 128, i) - 32;
        return 16;
    default:
        return 0;
    }
}

/* ---------------------------------------------------------------- decode */

/* q4_K -> f32.  The exact value d*sc*q - dmin*m is formed in long double (each
 * product has at most 21 significant bits and the f16 exponent range keeps the
 * difference inside a 64-bit significand), then rounded once to f32. */
void oracle_decode_q4K(const uint8_t *W, int64_t nblocks, float *out)
{
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *blk = W + b * OQ4K_BYTES;
        long double d = oracle_f16_to_f64(rd_u16(blk));
        long double dmin = oracle_f16_to_f64(rd_u16(blk + 2));
        const uint8_t *s = blk + 4, *qs = blk + 16;
        for (int i = 0; i < OQK; ++i) {
            int sc, mn;
            q4k_scale_min(s, i / 32, &sc, &mn);
            long double v = d * sc * q4k_quant(qs, i) - dmin * mn;
            out[b * OQK + i] = (float)v;
        }
    }
}

/* q6_K -> f32.  d*sc*(q-32) has at most 23 significant bits: exact in f32. */
void oracle_decode_q6K(const uint8_t *W, int64_t nblocks, float *out)
{
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *blk = W + b * OQ6K_BYTES;
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        long double d = oracle_f16_to_f64(rd_u16(blk + 208));
        for (int i = 0; i < OQK; ++i) {
            long double v = d * sc[i / 16] * (q6k_quant(ql, qh, i) - 32);
            out[b * OQK + i] = (float)v;
        }
    }
}

/* q2_K, q3_K, q5_K -> f32 (fmt 10, 11, 13; also accepts 12 and 14).  The exact
 * value d*sc*q - dmin*m is formed in long double (q5_K: at most 22 + 17
 * significant bits, exponents inside the f16 range, so the difference fits a
 * 64-bit significand; q2_K and q3_K fewer), then rounded once to f32.
 * Returns 0, or -1 for an unknown format. */
int oracle_decode(int fmt, const uint8_t *W, int64_t nblocks, float *out)
{
    static const int bytes[15] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 84, 110, 144, 176, 210};
    if (fmt < 10 || fmt > 14)
        return -1;
    int q[OQK], sc[16], mn[16];
    double d, dmin;
    for (int64_t b = 0; b < nblocks; ++b) {
        int L = unpack_block(fmt, W + b * bytes[fmt], q, sc, mn, &d, &dmin);
        for (int i = 0; i < OQK; ++i) {
            long double v = (long double)d * sc[i / L] * q[i] - (long double)dmin * mn[i / L];
            out[b * OQK + i] = (float)v;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- quantize */

/* f32 activations [M, K] -> q8_K blocks, one per 256 consecutive values of a row.
 * amax = max |x|; d = amax / 127 (f32, correctly rounded); q = round-half-even of
 * x / d (f32 division), clamped to [-127, 127]; group sum g = sum of q over values
 * 16g..16g+15.  A block whose d is zero (all-zero input) stores d = 0 and q = 0.
 * Returns 0, or -1 when K is not a multiple of 256. */
int oracle_quantize_q8K(const float *X, int64_t M, int64_t K, uint8_t *Xq)
{
    if (K % OQK != 0 || M < 0)
        return -1;
    int64_t nb = K / OQK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *x = X + m * K + b * OQK;
            uint8_t *blk = Xq + (m * nb + b) * OQ8K_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < OQK; ++i) {
                float a = fabsf(x[i]);
                if (a > amax)
                    amax = a;
            }
            float d = amax / 127.0f;
            int8_t q[OQK];
            for (int i = 0; i < OQK; ++i) {
                if (d == 0.0f) {
                    q[i] = 0;
                    continue;
                }
                float r = rintf(x[i] / d);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                q[i] = (int8_t)r;
            }
            wr_f32(blk, d);
            memcpy(blk + 4, q, OQK);
            for (int g = 0; g < 16; ++g) {
                int s = 0;
                for (int i = 0; i < 16; ++i)
                    s += q[16 * g + i];
                wr_i16(blk + 260 + 2 * g, s);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- matmul */

#define OFMT_Q2K 10
#define OFMT_Q3K 11
#define OFMT_Q4K 12
#define OFMT_Q5K 13
#define OFMT_Q6K 14

static int fmt_block_bytes(int fmt)
{
    switch (fmt) {
    case OFMT_Q2K: return OQ2K_BYTES;
    case OFMT_Q3K: return OQ3K_BYTES;
    case OFMT_Q4K: return OQ4K_BYTES;
    case OFMT_Q5K: return OQ5K_BYTES;
    case OFMT_Q6K: return OQ6K_BYTES;
    default: return 0;
    }
}

/* Route A for q2_K, q3_K and q5_K: per super-block, I_sc = sum_j sc_j *
 * sum_{i in j} q_i * qx_i and I_min = sum_j m_j * sum_{i in j} qx_i as exact
 * int64, then d_x * (d * I_sc - dmin * I_min) in double. */
static int gemm_int_other(int fmt, const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N,
                          int64_t K, const int64_t *rows, int64_t nrows, double *Y)
{
    int wb = fmt_block_bytes(fmt);
    int64_t nb = K / OQK;
    int q[OQK], sc[16], mn[16];
    double d, dmin;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t n = 0; n < N; ++n)
            Y[r * N + n] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            int L = unpack_block(fmt, W + (n * nb + b) * wb, q, sc, mn, &d, &dmin);
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t m = rows ? rows[r] : r;
                const uint8_t *xb = Xq + (m * nb + b) * OQ8K_BYTES;
                double dx = rd_f32(xb);
                const int8_t *qx = (const int8_t *)(xb + 4);
                int64_t isc = 0, imn = 0;
                for (int j = 0; j < OQK / L; ++j) {
                    int64_t dot = 0, sx = 0;
                    for (int i = L * j; i < L * j + L; ++i) {
                        dot += (int64_t)q[i] * qx[i];
                        sx += qx[i];
                    }
                    isc += sc[j] * dot;
                    imn += mn[j] * sx;
                }
                Y[r * N + n] += dx * (d * (double)isc - dmin * (double)imn);
            }
        }
    }
    return 0;
}

/* Route A (integer decomposition).  For every listed activation row m and every
 * weight row n: y = sum over super-blocks b of d_x * (d * I_sc - dmin * I_min) for
 * q4_K, with I_sc = sum_j sc_j * sum_{i in j} q_i * qx_i and
 * I_min = sum_j m_j * sum_{i in j} qx_i, both exact int64; for q6_K
 * y = sum_b d_x * d * sum_j sc_j * sum_{i in j} (q_i - 32) * qx_i; for q2_K,
 * q3_K and q5_K the same sums over their own sub-blocks (16, 16 and 32 weights;
 * q3_K has no min term) from the integers of unpack_block.  The block
 * terms are combined in double.  This is the exact real sum over k of
 * (unrounded weight) * (d_x * qx), up to double rounding.
 * rows == NULL means all M rows; Y is [nrows, N].  Returns 0 or -1 on bad args. */
int oracle_gemm_int(int fmt, const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N,
                    int64_t K, const int64_t *rows, int64_t nrows, double *Y)
{
    int wb = fmt_block_bytes(fmt);
    if (!wb || K % OQK != 0)
        return -1;
    if (!rows)
        nrows = M;
    int64_t nb = K / OQK;
    if (fmt != OFMT_Q4K && fmt != OFMT_Q6K)
        return gemm_int_other(fmt, W, Xq, M, N, K, rows, nrows, Y);
    int *q = (int *)malloc(sizeof(int) * (size_t)K); /* weight quants of one row */
    int *sc = (int *)malloc(sizeof(int) * (size_t)(K / 16));
    int *mn = (int *)malloc(sizeof(int) * (size_t)(K / 32));
    double *dd = (double *)malloc(sizeof(double) * (size_t)nb);
    double *dm = (double *)malloc(sizeof(double) * (size_t)nb);
    for (int64_t n = 0; n < N; ++n) {
        /* unpack row n once: integer quants and sub-block scales, float d/dmin */
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = W + (n * nb + b) * wb;
            if (fmt == OFMT_Q4K) {
                dd[b] = oracle_f16_to_f64(rd_u16(blk));
                dm[b] = oracle_f16_to_f64(rd_u16(blk + 2));
                for (int j = 0; j < 8; ++j)
                    q4k_scale_min(blk + 4, j, &sc[b * 8 + j], &mn[b * 8 + j]);
                for (int i = 0; i < OQK; ++i)
                    q[b * OQK + i] = q4k_quant(blk + 16, i);
            } else {
                dd[b] = oracle_f16_to_f64(rd_u16(blk + 208));
                for (int j = 0; j < 16; ++j)
                    sc[b * 16 + j] = ((const int8_t *)(blk + 192))[j];
                for (int i = 0; i < OQK; ++i)
                    q[b * OQK + i] = q6k_quant(blk, blk + 128, i) - 32;
            }
        }
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t m = rows ? rows[r] : r;
            double y = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *xb = Xq + (m * nb + b) * OQ8K_BYTES;
                double dx = rd_f32(xb);
                const int8_t *qx = (const int8_t *)(xb + 4);
                const int *qw = q + b * OQK;
                if (fmt == OFMT_Q4K) {
                    int64_t isc = 0, imn = 0;
                    for (int j = 0; j < 8; ++j) {
                        int64_t dot = 0, sx = 0;
                        for (int i = 32 * j; i < 32 * j + 32; ++i) {
                            dot += (int64_t)qw[i] * qx[i];
                            sx += qx[i];
                        }
                        isc += sc[b * 8 + j] * dot;
                        imn += mn[b * 8 + j] * sx;
                    }
                    y += dx * (dd[b] * (double)isc - dm[b] * (double)imn);
                } else {
                    int64_t isc = 0;
                    for (int j = 0; j < 16; ++j) {
                        int64_t dot = 0;
                        for (int i = 16 * j; i < 16 * j + 16; ++i)
                            dot += (int64_t)qw[i] * qx[i];
                        isc += sc[b * 16 + j] * dot;
                    }
                    y += dx * dd[b] * (double)isc;
                }
            }
            Y[r * N + n] = y;
        }
    }
    free(q);
    free(sc);
    free(mn);
    free(dd);
    free(dm);
    return 0;
}

/* Route B (decode, then dot) and the error scale.  w_k is the f32 decode above,
 * xhat_k = d_x * qx_k; Yd = sum_k w_k * xhat_k and S = sum_k |w_k * xhat_k|, both
 * in double.  Either output pointer may be NULL. */
int oracle_gemm_dequant(int fmt, const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N,
                        int64_t K, const int64_t *rows, int64_t nrows, double *Yd, double *S)
{
    int wb = fmt_block_bytes(fmt);
    if (!wb || K % OQK != 0)
        return -1;
    if (!rows)
        nrows = M;
    int64_t nb = K / OQK;
    float *w = (float *)malloc(sizeof(float) * (size_t)K);
    double *xh = (double *)malloc(sizeof(double) * (size_t)(K * nrows));
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *xb = Xq + (m * nb + b) * OQ8K_BYTES;
            double dx = rd_f32(xb);
            for (int i = 0; i < OQK; ++i)
                xh[r * K + b * OQK + i] = dx * ((const int8_t *)(xb + 4))[i];
        }
    }
    for (int64_t n = 0; n < N; ++n) {
        if (fmt == OFMT_Q4K)
            oracle_decode_q4K(W + n * nb * wb, nb, w);
        else if (fmt == OFMT_Q6K)
            oracle_decode_q6K(W + n * nb * wb, nb, w);
        else
            oracle_decode(fmt, W + n * nb * wb, nb, w);
        for (int64_t r = 0; r < nrows; ++r) {
            double y = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = (double)w[k] * xh[r * K + k];
                y += t;
                s += fabs(t);
            }
            if (Yd)
                Yd[r * N + n] = y;
            if (S)
                S[r * N + n] = s;
        }
    }
    free(w);
    free(xh);
    return 0;
}

/* The SiLU-gated product of an MLP's two up-projections, element by element:
 * y = silu(g) * u with silu(g) = g / (1 + e^-g), in double.  The pages name this
 * step silu_mul and run it right after the gate/up matmuls (molayo article
 * "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
 * engine": silu_mul's thread grain sized for decode shapes). */
void oracle_silu_mul(const double *g, const double *u, int64_t n, double *y)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* Load-time repack of a q3_K or q6_K matrix (the GPU counterpart of the pages'
 * q4_K 8-column panels, a layout chosen at load time: molayo article, status row
 * "src/ -- C++ engine"): the same bytes, reordered so that every field of every
 * block starts on a 16-byte boundary.  The matrix's NB = N*K/256 blocks, in row
 * order, are split into their fields and each field is stored for all blocks
 * in a row (structure of arrays):
 *   q6_K: ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
 *   q3_K: hmask[NB][32] | qs[NB][64] | scales[NB][12] | d[NB][2]
 * The layout is this library's own (the pages describe panels for q4_K but no
 * byte layout).  Returns 0, or -1 for another format or bad sizes. */
int oracle_repack(int fmt, const uint8_t *W, int64_t N, int64_t K, uint8_t *out)
{
    static const int f6[] = {128, 64, 16, 2}, f3[] = {32, 64, 12, 2};
    const int *f;
    int bb;
    if (fmt == OFMT_Q6K) {
        f = f6;
        bb = OQ6K_BYTES;
    } else if (fmt == OFMT_Q3K) {
        f = f3;
        bb = OQ3K_BYTES;
    } else {
        return -1;
    }
    if (N < 0 || K <= 0 || K % OQK != 0)
        return -1;
    int64_t nb = N * (K / OQK);
    int64_t dst = 0;
    int src = 0;
    for (int k = 0; k < 4; ++k) {
        for (int64_t i = 0; i < nb; ++i)
            memcpy(out + dst + i * f[k], W + i * bb + src, (size_t)f[k]);
        dst += nb * f[k];
        src += f[k];
    }
    return 0;
}

/* Version of this oracle's interface, for the test loader. */
int oracle_version(void) { return 4; }
