/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the decode-step
 * hot path: block-quantized GEMV (dequantize, dot product), RMSNorm,
 * two-pass LayerNorm, the SiLU-gated glue, the synthetic decode chain, the
 * quantizer from fp32 weights and single-token attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; it shares no header, table or helper with the GPU path.
 * Only the tests, the smoke check and the bench's CPU-baseline leg load it.
 *
 * Arithmetic: every floating-point step is carried out in IEEE double and
 * rounded to float once, at the point where the path stores a float.
 * No fast-math, no reassociation beyond what is written, k ascending.
 *
 * Sources (web pages; cited by short tag):
 *   [one-serial-kernel]  vocodex.ai, "From 22.8 to 42.8 tokens a second without
 *                        touching a matrix multiply"
 *   [mountain-runs]      coderlegion.com S-MoE diary #5, "The Mountain Runs"
 *   [roofline-holds]     research.arkey.ai, "The roofline holds on a second GPU"
 *
 * Weight formats.  The pages fix how many bytes each format spends per weight
 * ([roofline-holds] "The Math": 4.5 bits per weight for the 4-bit tables,
 * 6.5625 for the 6-bit ones; "The search space": 256 weights in 144 and 210
 * bytes) and that 2- and 4-bit codes are unpacked in registers
 * ([mountain-runs] section 3).  The block structure and bit layout below are
 * this library's own definition of those byte budgets:
 *
 *   fmt 0  BF16  plane0 = uint16 words [N][K];  w = float(word << 16)
 *   fmt 1  Q45   plane0 = codes [N][K/2]: byte k>>1, nibble (k&1) (low first)
 *                plane2 = fp16 scale [N][K/32];  w = s * (q - 8)
 *   fmt 2  Q65   plane0 = ql [N][K/2]: low 4 code bits, same nibble order
 *                plane1 = qh [N][K/4]: high 2 code bits, see q65_hi() below
 *                plane2 = int8 sub-scale [N][K/16]
 *                plane3 = fp16 super-scale [N][K/256]
 *                q = lo | hi << 4;  w = d * sc * (q - 32)
 *   fmt 3  Q25   plane0 = codes [N][K/4]: byte k>>2, bits 2*(k&3)
 *                plane2 = fp16 scale [N][K/32];  w = s * (q - 2)
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

#define FMT_BF16 0
#define FMT_Q45 1
#define FMT_Q65 2
#define FMT_Q25 3

/* ------------------------------------------------------------------------ */
/* Scalar decoders                                                           */
/* ------------------------------------------------------------------------ */

/* IEEE-754 binary16 -> double, written out from the encoding: 1 sign bit,
 * 5 exponent bits (bias 15), 10 mantissa bits; exponent 0 is subnormal
 * (m * 2^-24), exponent 31 is inf/NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 word -> double: the word is the top half of a binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

static uint16_t rd16(const void* base, size_t idx)
{
    const uint8_t* p = (const uint8_t*)base + 2 * idx;
    return (uint16_t)(p[0] | (p[1] << 8)); /* little-endian */
}

/* High 2 bits of the 6-bit code of weight k within one row of a Q65 qh plane.
 * Each run of 16 weights g = k>>4 owns the 4 bytes qh[4g .. 4g+3], read as a
 * little-endian 32-bit word W; weight r = k & 15 of the run keeps its high
 * bits at bit Q65_POS[r] of W (bits POS and POS+1). */
static const int Q65_POS[16] = {4, 2, 12, 10, 20, 18, 28, 26, 0, 6, 8, 14, 16, 22, 24, 30};

static int q65_hi(const uint8_t* qh_row, int64_t k)
{
    int64_t g = k >> 4;
    int pos = Q65_POS[k & 15];
    return (qh_row[4 * g + pos / 8] >> (pos % 8)) & 3;
}

/* Integer code of weight (n, k).  BF16 has no code (returns -1). */
int oracle_code(int fmt, const void* const planes[4], int64_t N, int64_t K,
                int64_t n, int64_t k)
{
    (void)N;
    if (fmt == FMT_Q45) {
        const uint8_t* c = (const uint8_t*)planes[0] + n * (K / 2);
        return (c[k >> 1] >> (4 * (k & 1))) & 15;
    }
    if (fmt == FMT_Q25) {
        const uint8_t* c = (const uint8_t*)planes[0] + n * (K / 4);
        return (c[k >> 2] >> (2 * (k & 3))) & 3;
    }
    if (fmt == FMT_Q65) {
        const uint8_t* ql = (const uint8_t*)planes[0] + n * (K / 2);
        const uint8_t* qh = (const uint8_t*)planes[1] + n * (K / 4);
        int lo = (ql[k >> 1] >> (4 * (k & 1))) & 15;
        int hi = q65_hi(qh, k);
        return lo | (hi << 4);
    }
    return -1;
}

/* Dequantized weight (n, k) as a double.  For every format the value is a
 * product of at most three small factors and is exactly representable in
 * binary32 (see the tests), so (float) of it is exact. */
double oracle_weight(int fmt, const void* const planes[4], int64_t N, int64_t K,
                     int64_t n, int64_t k)
{
    if (fmt == FMT_BF16)
        return oracle_bf16_to_f64(rd16(planes[0], (size_t)(n * K + k)));
    int q = oracle_code(fmt, planes, N, K, n, k);
    if (fmt == FMT_Q45) {
        double s = oracle_f16_to_f64(rd16(planes[2], (size_t)(n * (K / 32) + (k >> 5))));
        return s * (double)(q - 8);
    }
    if (fmt == FMT_Q25) {
        double s = oracle_f16_to_f64(rd16(planes[2], (size_t)(n * (K / 32) + (k >> 5))));
        return s * (double)(q - 2);
    }
    if (fmt == FMT_Q65) {
        const int8_t* sc = (const int8_t*)planes[2] + n * (K / 16);
        double d = oracle_f16_to_f64(rd16(planes[3], (size_t)(n * (K / 256) + (k >> 8))));
        return d * (double)sc[k >> 4] * (double)(q - 32);
    }
    return NAN;
}

/* ------------------------------------------------------------------------ */
/* Format bookkeeping (bytes per plane)                                      */
/* ------------------------------------------------------------------------ */

/* Byte size of each plane for an N x K weight.  Returns 0 on success, -1 for
 * an unknown format or a K the format's blocks do not divide. */
int oracle_plane_bytes(int fmt, int64_t N, int64_t K, int64_t out[4])
{
    out[0] = out[1] = out[2] = out[3] = 0;
    if (N < 0 || K < 0) return -1;
    switch (fmt) {
    case FMT_BF16:
        out[0] = 2 * N * K;
        return 0;
    case FMT_Q45:
        if (K % 32) return -1;
        out[0] = N * K / 2;
        out[2] = 2 * N * (K / 32);
        return 0;
    case FMT_Q65:
        if (K % 256) return -1;
        out[0] = N * K / 2;
        out[1] = N * K / 4;
        out[2] = N * (K / 16);
        out[3] = 2 * N * (K / 256);
        return 0;
    case FMT_Q25:
        if (K % 32) return -1;
        out[0] = N * K / 4;
        out[2] = 2 * N * (K / 32);
        return 0;
    }
    return -1;
}

/* Pack one-byte-per-weight codes and their scales into the planes above.
 * Written independently of the product's packer; used by tests to check it.
 * scales: Q45/Q25 fp16 words [N][K/32]; Q65 int8 [N][K/16].
 * supers: Q65 fp16 words [N][K/256].  BF16: codes holds the uint16 words. */
int oracle_pack(int fmt, int64_t N, int64_t K, const uint8_t* codes,
                const void* scales, const void* supers, void* const planes[4])
{
    int64_t sz[4];
    if (oracle_plane_bytes(fmt, N, K, sz)) return -1;
    for (int p = 0; p < 4; p++)
        if (sz[p]) memset(planes[p], 0, (size_t)sz[p]);
    if (fmt == FMT_BF16) {
        memcpy(planes[0], codes, (size_t)sz[0]);
        return 0;
    }
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int q = codes[n * K + k];
            if (fmt == FMT_Q45) {
                if (q > 15) return -1;
                uint8_t* c = (uint8_t*)planes[0] + n * (K / 2);
                c[k >> 1] |= (uint8_t)(q << (4 * (k & 1)));
            } else if (fmt == FMT_Q25) {
                if (q > 3) return -1;
                uint8_t* c = (uint8_t*)planes[0] + n * (K / 4);
                c[k >> 2] |= (uint8_t)(q << (2 * (k & 3)));
            } else {
                if (q > 63) return -1;
                uint8_t* ql = (uint8_t*)planes[0] + n * (K / 2);
                uint8_t* qh = (uint8_t*)planes[1] + n * (K / 4);
                ql[k >> 1] |= (uint8_t)((q & 15) << (4 * (k & 1)));
                int64_t g = k >> 4;
                int pos = Q65_POS[k & 15];
                qh[4 * g + pos / 8] |= (uint8_t)((q >> 4) << (pos % 8));
            }
        }
    }
    if (fmt == FMT_Q65) {
        memcpy(planes[2], scales, (size_t)sz[2]);
        memcpy(planes[3], supers, (size_t)sz[3]);
    } else {
        memcpy(planes[2], scales, (size_t)sz[2]);
    }
    return 0;
}

/* All integer codes of the matrix, one byte per weight (row-major). */
int oracle_codes(int fmt, const void* const planes[4], int64_t N, int64_t K,
                 uint8_t* out)
{
    if (fmt == FMT_BF16) return -1;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = (uint8_t)oracle_code(fmt, planes, N, K, n, k);
    return 0;
}

/* All dequantized weights as binary32 (exact), row-major [N][K]. */
void oracle_dequant(int fmt, const void* const planes[4], int64_t N, int64_t K,
                    float* out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = (float)oracle_weight(fmt, planes, N, K, n, k);
}

/* ------------------------------------------------------------------------ */
/* GEMV: y[m][n] = sum_k w[n][k] * x[m][k]                                   */
/* ------------------------------------------------------------------------ */

/* Rows [row0, row1) of y = W x for M input vectors.  Each term is an exact
 * double product of two binary32 values; the sum runs k ascending in double
 * and is rounded to float once.  accumulate != 0 adds the (double) sum to the
 * float already in y before the single rounding ([roofline-holds]
 * "The tensor, the kernel, the token": multiply this tensor by this vector). */
void oracle_gemv(int fmt, const void* const planes[4], int64_t N, int64_t K,
                 const float* x, int64_t M, int64_t ldx,
                 float* y, int64_t ldy, int accumulate,
                 int64_t row0, int64_t row1)
{
    for (int64_t n = row0; n < row1; n++) {
        for (int64_t m = 0; m < M; m++) {
            double s = accumulate ? (double)y[m * ldy + n] : 0.0;
            double dot = 0.0;
            for (int64_t k = 0; k < K; k++)
                dot += oracle_weight(fmt, planes, N, K, n, k) * (double)x[m * ldx + k];
            y[m * ldy + n] = (float)(s + dot);
        }
    }
}

/* Selected experts: y[e][r] = sum_k W_all[idx[e]*R + r][k] * x[k], for rows
 * r in [r0, r1) of every selected expert ([mountain-runs] section 3, the
 * expert FFN kernels).  W_all stacks the experts along N. */
void oracle_gather(int fmt, const void* const planes[4], int64_t N_all, int64_t K,
                   int64_t R, const int32_t* idx, int64_t n_sel,
                   const float* x, float* y, int64_t r0, int64_t r1)
{
    for (int64_t e = 0; e < n_sel; e++) {
        int64_t base = (int64_t)idx[e] * R;
        for (int64_t r = r0; r < r1; r++) {
            double dot = 0.0;
            for (int64_t k = 0; k < K; k++)
                dot += oracle_weight(fmt, planes, N_all, K, base + r, k) * (double)x[k];
            y[e * R + r] = (float)dot;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Row norms ([one-serial-kernel] "What one token costs", "One thread")      */
/* ------------------------------------------------------------------------ */

/* RMSNorm: y = gamma * x / sqrt(mean(x^2) + eps), statistics in double. */
void oracle_rmsnorm(const float* x, const float* gamma, float eps,
                    int64_t rows, int64_t n, float* y)
{
    for (int64_t r = 0; r < rows; r++) {
        const float* xr = x + r * n;
        double ss = 0.0;
        for (int64_t i = 0; i < n; i++) ss += (double)xr[i] * (double)xr[i];
        double inv = 1.0 / sqrt(ss / (double)n + (double)eps);
        for (int64_t i = 0; i < n; i++)
            y[r * n + i] = (float)((double)gamma[i] * ((double)xr[i] * inv));
    }
}

/* LayerNorm in two passes: mean first, then the biased variance of the
 * centred values; y = (x - mean) / sqrt(var + eps) * gamma + beta. */
void oracle_layernorm(const float* x, const float* gamma, const float* beta,
                      float eps, int64_t rows, int64_t n, float* y)
{
    for (int64_t r = 0; r < rows; r++) {
        const float* xr = x + r * n;
        double s = 0.0;
        for (int64_t i = 0; i < n; i++) s += (double)xr[i];
        double mean = s / (double)n;
        double v = 0.0;
        for (int64_t i = 0; i < n; i++) {
            double c = (double)xr[i] - mean;
            v += c * c;
        }
        double inv = 1.0 / sqrt(v / (double)n + (double)eps);
        for (int64_t i = 0; i < n; i++)
            y[r * n + i] = (float)(((double)xr[i] - mean) * inv * (double)gamma[i]
                                   + (double)beta[i]);
    }
}

/* The serial single-thread versions the cooperative kernels replaced
 * ([one-serial-kernel] "One thread"): float accumulation, left to right. */
void oracle_rmsnorm_serial_f32(const float* x, const float* gamma, float eps,
                               int64_t rows, int64_t n, float* y)
{
    for (int64_t r = 0; r < rows; r++) {
        const float* xr = x + r * n;
        float ss = 0.0f;
        for (int64_t i = 0; i < n; i++) ss += xr[i] * xr[i];
        float inv = 1.0f / sqrtf(ss / (float)n + eps);
        for (int64_t i = 0; i < n; i++) y[r * n + i] = gamma[i] * (xr[i] * inv);
    }
}

void oracle_layernorm_serial_f32(const float* x, const float* gamma,
                                 const float* beta, float eps,
                                 int64_t rows, int64_t n, float* y)
{
    for (int64_t r = 0; r < rows; r++) {
        const float* xr = x + r * n;
        float s = 0.0f;
        for (int64_t i = 0; i < n; i++) s += xr[i];
        float mean = s / (float)n;
        float v = 0.0f;
        for (int64_t i = 0; i < n; i++) v += (xr[i] - mean) * (xr[i] - mean);
        float inv = 1.0f / sqrtf(v / (float)n + eps);
        for (int64_t i = 0; i < n; i++)
            y[r * n + i] = (xr[i] - mean) * inv * gamma[i] + beta[i];
    }
}

/* Float sum of v[0..n) by pairwise halving (the order of a cooperative
 * tree reduction over a power-of-two group). */
static float tree_sum_f32(float* v, int64_t n)
{
    while (n > 1) {
        int64_t h = (n + 1) / 2;
        for (int64_t i = 0; i + h < n; i++) v[i] = v[i] + v[i + h];
        n = h;
    }
    return n ? v[0] : 0.0f;
}

/* Float RMSNorm whose sum of squares is combined as `threads` strided partial
 * sums reduced by a pairwise tree: the order of a cooperative kernel with
 * that many threads per row.  scratch holds `threads` floats. */
void oracle_rmsnorm_tree_f32(const float* x, const float* gamma, float eps,
                             int64_t rows, int64_t n, int64_t threads,
                             float* scratch, float* y)
{
    for (int64_t r = 0; r < rows; r++) {
        const float* xr = x + r * n;
        for (int64_t t = 0; t < threads; t++) {
            float p = 0.0f;
            for (int64_t i = t; i < n; i += threads) p += xr[i] * xr[i];
            scratch[t] = p;
        }
        float ss = tree_sum_f32(scratch, threads);
        float inv = 1.0f / sqrtf(ss / (float)n + eps);
        for (int64_t i = 0; i < n; i++) y[r * n + i] = gamma[i] * (xr[i] * inv);
    }
}

/* ------------------------------------------------------------------------ */
/* Glue of the synthetic decode chain                                        */
/* ------------------------------------------------------------------------ */

/* out = silu(g) * u with silu(t) = t / (1 + exp(-t)), in double. */
void oracle_silu_mul(const float* g, const float* u, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; i++) {
        double t = (double)g[i];
        out[i] = (float)(t / (1.0 + exp(-t)) * (double)u[i]);
    }
}

/* One synthetic decode token, attention omitted ([roofline-holds] "The Math":
 * the per-layer tables; "Where the time goes": the norms and the adds).
 * Every activation is stored as float between steps, exactly as the product
 * path stores it; each step is computed as above.
 *   per layer l:  a = rmsnorm(h, g1[l]);  q = Wq a;  k = Wk a;  v = Wv a
 *                 h += Wo q          (attention output stands in as q;
 *                                     k and v are computed and not consumed)
 *                 b = rmsnorm(h, g2[l]); g = Wg b; u = Wu b; m = silu(g) * u
 *                 h += Wd m
 *   then z = rmsnorm(h, gf); logits = Wvocab z.
 * Weight i of layer l (i = q, k, v, o, gate, up, down) is described by
 * fmts[7*l+i] and planes[4*(7*l+i) + 0..3]; the vocab table by fmts[7*L] and
 * planes[4*7*L + 0..3].  Shapes: Wq [dq, d], Wk and Wv [dkv, d], Wo [d, dq],
 * Wg and Wu [f, d], Wd [d, f], Wvocab [V, d].  ws must hold
 * dq + 2*dkv + 3*f + d floats.  h (d floats) is updated in place; h_trace, if
 * not NULL, receives h after every layer (L * d floats). */
void oracle_decode_token(int L, int64_t d, int64_t dq, int64_t dkv, int64_t f,
                         int64_t V, const int* fmts, const void* const* planes,
                         const float* g1, const float* g2, const float* gf,
                         float eps, float* h, float* logits, float* ws,
                         float* h_trace)
{
    float* q = ws;
    float* kk = q + dq;
    float* vv = kk + dkv;
    float* g = vv + dkv;
    float* u = g + f;
    float* m = u + f;
    float* a = m + f;
#define W_(l, i) fmts[7 * (l) + (i)], planes + 4 * (7 * (l) + (i))
    for (int l = 0; l < L; l++) {
        oracle_rmsnorm(h, g1 + l * d, eps, 1, d, a);
        oracle_gemv(W_(l, 0), dq, d, a, 1, d, q, dq, 0, 0, dq);
        oracle_gemv(W_(l, 1), dkv, d, a, 1, d, kk, dkv, 0, 0, dkv);
        oracle_gemv(W_(l, 2), dkv, d, a, 1, d, vv, dkv, 0, 0, dkv);
        oracle_gemv(W_(l, 3), d, dq, q, 1, dq, h, d, 1, 0, d);
        oracle_rmsnorm(h, g2 + l * d, eps, 1, d, a);
        oracle_gemv(W_(l, 4), f, d, a, 1, d, g, f, 0, 0, f);
        oracle_gemv(W_(l, 5), f, d, a, 1, d, u, f, 0, 0, f);
        oracle_silu_mul(g, u, f, m);
        oracle_gemv(W_(l, 6), d, f, m, 1, f, h, d, 1, 0, d);
        if (h_trace) memcpy(h_trace + (int64_t)l * d, h, (size_t)d * sizeof(float));
    }
    oracle_rmsnorm(h, gf, eps, 1, d, a);
    oracle_gemv(W_(L, 0), V, d, a, 1, d, logits, V, 0, 0, V);
#undef W_
}


/* ------------------------------------------------------------------------ */
/* Quantizer: fp32 weights -> codes and scales                               */
/* ------------------------------------------------------------------------ */

/* fp32 -> IEEE binary16 bit pattern, rounding to nearest with ties to even,
 * written out from the encoding; magnitudes that would round past the
 * largest finite half (65504) saturate to it.  Subnormal halves (exponent
 * 0, units of 2^-24) are produced where the value needs them. */
uint16_t oracle_f32_to_f16_sat(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a == 0.0)
        return sign;
    if (a >= 65504.0)
        return (uint16_t)(sign | 0x7BFF);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; a * 2^24 is exact in double */
        double m = nearbyint(a * 16777216.0);      /* ties to even (default mode) */
        return (uint16_t)(sign | (uint16_t)m);      /* m = 1024 is the smallest normal */
    }
    int e;
    double fr = frexp(a, &e);                       /* a = fr * 2^e, fr in [0.5, 1) */
    e -= 1;                                         /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double m = nearbyint(ldexp(fr, 11));            /* 10 fraction bits: m in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7BFF);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* fp32 -> bfloat16 word, round to nearest with ties to even. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint32_t low = bits & 0xFFFF, up = bits >> 16;
    if (low > 0x8000 || (low == 0x8000 && (up & 1)))
        up += 1;
    return (uint16_t)up;
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Symmetric absmax quantizer (this library's reading; the pages fix only the
 * byte budgets of the formats, [roofline-holds] "The Math" and "The search
 * space").  Every decision that yields an integer is made in fp32, in the
 * order written:
 *   Q45 / Q25, per block of 32:  s = half(max|w| / Qmax), Qmax = 7 / 1;
 *     q = clamp(rint(w / s) + off, 0, 2^b - 1), off = 8 / 2; q = off if s = 0.
 *   Q65, per super-block of 256 (16 sub-blocks of 16):
 *     a_j = max_{sub-block j} |w| / 31;  d = half(max_j a_j / 127);
 *     sc_j = clamp(rint(a_j / d), -128, 127)  (0 if d = 0);
 *     q = clamp(rint(w / (d sc_j)) + 32, 0, 63)  (32 if d sc_j = 0).
 *   BF16: round to nearest even.
 * half() is oracle_f32_to_f16_sat, rint rounds half to even.
 * Outputs: codes one byte per weight [N][K] (BF16: uint16 words),
 * scales fp16 bits [N][K/32] (Q45, Q25) or int8 [N][K/16] (Q65),
 * supers fp16 bits [N][K/256] (Q65).  Returns -1 for a bad format or K. */
int oracle_quantize(int fmt, int64_t N, int64_t K, const float* w, int64_t ldw,
                    void* codes, void* scales, uint16_t* supers)
{
    if (fmt == FMT_BF16) {
        uint16_t* o = (uint16_t*)codes;
        for (int64_t n = 0; n < N; n++)
            for (int64_t k = 0; k < K; k++)
                o[n * K + k] = oracle_f32_to_bf16(w[n * ldw + k]);
        return 0;
    }
    uint8_t* q = (uint8_t*)codes;
    if (fmt == FMT_Q45 || fmt == FMT_Q25) {
        if (K % 32) return -1;
        const int qmax = fmt == FMT_Q45 ? 7 : 1, off = fmt == FMT_Q45 ? 8 : 2;
        const int top = fmt == FMT_Q45 ? 15 : 3;
        uint16_t* sc = (uint16_t*)scales;
        for (int64_t n = 0; n < N; n++)
            for (int64_t b = 0; b < K / 32; b++) {
                const float* wb = w + n * ldw + 32 * b;
                float amax = 0.0f;
                for (int k = 0; k < 32; k++)
                    if (fabsf(wb[k]) > amax) amax = fabsf(wb[k]);
                const float t = amax / (float)qmax;
                const uint16_t sh = oracle_f32_to_f16_sat(t);
                const float s = (float)oracle_f16_to_f64(sh);
                sc[n * (K / 32) + b] = sh;
                for (int k = 0; k < 32; k++) {
                    int code = off;
                    if (s != 0.0f) code = clampi((int)rintf(wb[k] / s) + off, 0, top);
                    q[n * K + 32 * b + k] = (uint8_t)code;
                }
            }
        return 0;
    }
    if (fmt == FMT_Q65) {
        if (K % 256) return -1;
        int8_t* sc = (int8_t*)scales;
        for (int64_t n = 0; n < N; n++)
            for (int64_t sb = 0; sb < K / 256; sb++) {
                const float* ws = w + n * ldw + 256 * sb;
                float a[16], amx = 0.0f;
                for (int j = 0; j < 16; j++) {
                    float m = 0.0f;
                    for (int k = 0; k < 16; k++)
                        if (fabsf(ws[16 * j + k]) > m) m = fabsf(ws[16 * j + k]);
                    a[j] = m / 31.0f;
                    if (a[j] > amx) amx = a[j];
                }
                const uint16_t dh = oracle_f32_to_f16_sat(amx / 127.0f);
                const float d = (float)oracle_f16_to_f64(dh);
                supers[n * (K / 256) + sb] = dh;
                for (int j = 0; j < 16; j++) {
                    int s8 = 0;
                    if (d != 0.0f) s8 = clampi((int)rintf(a[j] / d), -128, 127);
                    sc[n * (K / 16) + 16 * sb + j] = (int8_t)s8;
                    const float step = d * (float)s8;     /* exact: 11 + 7 significant bits */
                    for (int k = 0; k < 16; k++) {
                        int code = 32;
                        if (step != 0.0f) code = clampi((int)rintf(ws[16 * j + k] / step) + 32, 0, 63);
                        q[n * K + 256 * sb + 16 * j + k] = (uint8_t)code;
                    }
                }
            }
        return 0;
    }
    return -1;
}


/* ------------------------------------------------------------------------ */
/* Single-token attention over a KV cache                                    */
/* ------------------------------------------------------------------------ */

/* One new token attends over T cached positions ([roofline-holds] "Said
 * before the run": with 512 tokens loaded each token also reads the
 * conversation's memory, 75.5 MB for the 36-layer model, i.e. 16-bit keys and
 * values 1024 wide per layer).  Plain scaled dot-product attention, the
 * reading this library takes (the pages name no positional encoding or
 * normalisation of q and k):
 *   head h of n_heads reads key/value head g = h / (n_heads / n_kv);
 *   s_t = (q_h . k_{t,g}) / sqrt(d);  p_t = exp(s_t - max s) / sum exp(s - max s);
 *   out_h = sum_t p_t v_{t,g}.
 * q: float [n_heads * d]; kc, vc: fp16 bits, position t's row at t * ld
 * (elements), head g at g * d within it; out: float [n_heads * d].
 * fp64 throughout, one rounding to float per output. */
void oracle_attention_decode(int n_heads, int n_kv, int d, int64_t T, const float* q,
                             const uint16_t* kc, const uint16_t* vc, int64_t ld, float* out,
                             double* scratch /* T doubles */)
{
    const int group = n_heads / n_kv;
    const double scale = 1.0 / sqrt((double)d);
    for (int h = 0; h < n_heads; h++) {
        const int g = h / group;
        double mx = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            double sdot = 0.0;
            for (int i = 0; i < d; i++)
                sdot += (double)q[h * d + i] * oracle_f16_to_f64(kc[t * ld + g * d + i]);
            scratch[t] = sdot * scale;
            if (scratch[t] > mx) mx = scratch[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t < T; t++) {
            scratch[t] = exp(scratch[t] - mx);
            z += scratch[t];
        }
        for (int i = 0; i < d; i++) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; t++)
                acc += scratch[t] * oracle_f16_to_f64(vc[t * ld + g * d + i]);
            out[h * d + i] = (float)(acc / z);
        }
    }
}
