/*
 * Reference oracle for the quantized prefill GEMM path -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously correct CPU code in fp64.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * HIP library never does, and the two share no code, header or table.
 *
 * What it computes (the plain definition the method reaches up to rounding):
 *   1. decode every weight of the canonical codec bytes exactly in fp64;
 *   2. ref[m][n] = sum_k x[m][k] * w[n][k], k ascending, one fp64 accumulator
 *      (Y = X * W^T with fp16 activations X [M,K] and weights W [N,K]);
 *   3. for the fused gate/up projection: out = g / (1 + exp(-g)) * u, fp64
 *      (SwiGLU), or out = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u
 *      (GeGLU with the tanh form of GELU).
 *
 * Sources on the pages (m4-prefill-engine):
 *   - releases page, v0.3.0, "PrismML Q2_0 Ternary Codec": 128-weight block of
 *     34 bytes (fp16 scale then 32 bytes of 2-bit codes), w = (q - 1) * d with
 *     the reserved code q = 3 giving +2d.
 *   - project index, Table B: block_q4_0 (GGUF Q4_0) and block_mlx_4bit weights.
 *   - releases page, v0.3.0, "Quantization Registry Extension": Q8_0 is one of
 *     the registry's built-in formats (no layout given there).
 *   - comparison page, section 2.2: SwiGLU is SiLU(Gate) x Up on one input X.
 *   - releases page, v0.3.0, TransformerBlock: SwiGLU / GeGLU activations, in
 *     the same line as the Gemma 2 RMSNorm variant; GeGLU = GELU(Gate) x Up.
 *   - releases page, v0.2 "Honest Verification Labeling": the check is a CPU
 *     double-precision gold computation.
 * Q4_0 w = (q - 8) * d over 32-weight blocks and MLX w = q * s + b over
 * 64-weight groups are the formulas of the workloads this path is measured on.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - Q4_0 byte order: GGUF convention, fp16 d first, then byte j holds weight
 *     j (low nibble) and weight j + 16 (high nibble).
 *   - MLX4 codes: little-endian uint32 words of 8 codes, element 0 in the low
 *     nibble; scales and biases are fp16; one group per 64 weights along K
 *     (MLX4-G32: per 32 weights, the group of the pages' 20-byte
 *     block_mlx_4bit, comparison page section 4).
 *   - Q2_0 code order: weight i sits in byte i / 4 of the code field at bit
 *     2 * (i % 4); q = 3 is applied without clamping.
 *   - Q8_0: GGUF block_q8_0, 34 bytes per 32 weights: fp16 d, then weight j
 *     as the two's-complement byte 2 + j; w = q * d.
 *   - GELU in GeGLU: the tanh form (the Gemma family's activation).
 *   - Q4_K: the pages name "Q4_K (GGUF Super-Blocks)" among the router's
 *     formats (releases page, v0.2 "Universal Quantization Router"; comparison
 *     page section 2.5) but print no layout.  The layout decoded here is the
 *     GGUF super-block of the public GGUF format description (see
 *     decode_q4_k_row); parity with the pages' own Q4_K kernel is therefore
 *     unpinned -- only the oracle's reading of that layout is pinned.
 *   - Ternary 1.58-bit: the pages name the BitNet ternary format (releases
 *     page v0.2 "Universal Quantization Router"; TERNARY_1_58 in the v0.3.0
 *     registry) without a packing.  Reading: blocks of 256 weights in 54
 *     bytes, fp16 d then five base-3 digits per byte (see
 *     decode_ternary_row); parity with the pages' own kernel is unpinned.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared -lm
 * (no fast-math: every operation is a correctly rounded IEEE fp64 operation).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_Q4_0 1
#define ORC_MLX4_G64 2
#define ORC_Q2_0 3
#define ORC_Q8_0 4
#define ORC_MLX4_G32 5
#define ORC_Q4_K 6
#define ORC_TERNARY 7
/* codec 8 reads the same canonical ternary bytes as codec 7 (the library
 * stores them differently on the device, which the oracle never sees) */
#define ORC_TERNARY_Q2 8

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE binary16 bit pattern -> exact fp64 value (sign, 5-bit exponent with
 * bias 15, 10-bit fraction; exponent 0 is subnormal, 31 is Inf/NaN). */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* f * 2^-10 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* fp64 -> nearest binary16, ties to even, correctly rounded in one step
 * (no detour through fp32, which would round twice).  Overflow gives +-Inf,
 * NaN stays NaN. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7E00;
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                 /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -14)
        e = -14;                   /* subnormal range: fixed quantum 2^-24 */
    /* quantum of the binary16 grid around a is 2^(e-10) */
    double scaled = ldexp(a, 10 - e);   /* exact: power-of-two scaling */
    double fl = floor(scaled);
    double rem = scaled - fl;           /* exact */
    double q = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        q = fl + 1.0;
    /* q * 2^(e-10) is the rounded magnitude; q in [1024, 2048] for normals,
     * [0, 1024] for subnormals. */
    double r = ldexp(q, e - 10);
    if (r > 65504.0)               /* rounds past the largest finite value */
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14)) {
        /* subnormal (or rounded up to the smallest normal, q == 1024) */
        uint16_t fbits = (uint16_t)q;      /* value = q * 2^-24 */
        return sign | fbits;              /* q == 1024 encodes 2^-14 exactly */
    }
    int ee;
    double mm = frexp(r, &ee);          /* r = mm * 2^ee, mm in [0.5,1) */
    int exp16 = ee - 1 + 15;
    uint16_t frac = (uint16_t)(ldexp(mm, 11) - 1024.0);
    return sign | (uint16_t)(exp16 << 10) | frac;
}

void orc_f16_to_f64_array(const uint16_t *h, double *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = orc_f16_to_f64(h[i]);
}

void orc_f64_to_f16_array(const double *x, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = orc_f64_to_f16(x[i]);
}

static uint16_t rd_u16le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd_u32le(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* ------------------------------------------------------------ geometry --- */

/* Weights per block and canonical bytes per block of a codec; 0 on error.
 * Q2_0: 128 weights in 34 bytes = 2.125 bits per weight (releases page,
 * v0.3.0).  MLX4-G64 has no interleaved block in canonical form; the value
 * returned is the per-group byte budget (32 code bytes + fp16 s + fp16 b). */
int orc_block_geometry(int codec, int64_t *weights, int64_t *bytes)
{
    switch (codec) {
    case ORC_Q4_0:     *weights = 32;  *bytes = 18; return 1;
    case ORC_MLX4_G64: *weights = 64;  *bytes = 36; return 1;
    case ORC_Q2_0:     *weights = 128; *bytes = 34; return 1;
    case ORC_Q8_0:     *weights = 32;  *bytes = 34; return 1;
    case ORC_MLX4_G32: *weights = 32;  *bytes = 20; return 1;
    case ORC_Q4_K:     *weights = 256; *bytes = 144; return 1;
    case ORC_TERNARY:  *weights = 256; *bytes = 54; return 1;
    case ORC_TERNARY_Q2: *weights = 256; *bytes = 54; return 1;
    default: return 0;
    }
}

/* -------------------------------------------------------------- decode --- */

/* Q4_0: per 32-weight block, d = fp16 at bytes 0-1; weight j (0..15) is the
 * low nibble of byte 2 + j, weight j + 16 the high nibble; w = (q - 8) * d.
 * Exact in fp64 (a 5-bit integer times an 11-bit significand). */
static void decode_q4_0_row(const uint8_t *row, int64_t k, double *w)
{
    for (int64_t b = 0; b < k / 32; ++b) {
        const uint8_t *blk = row + b * 18;
        double d = orc_f16_to_f64(rd_u16le(blk));
        for (int j = 0; j < 16; ++j) {
            int lo = blk[2 + j] & 0x0F;
            int hi = blk[2 + j] >> 4;
            w[b * 32 + j] = (double)(lo - 8) * d;
            w[b * 32 + j + 16] = (double)(hi - 8) * d;
        }
    }
}

/* Q2_0: per 128-weight block (34 bytes), d = fp16 at bytes 0-1; weight i has
 * q = (byte[2 + i/4] >> (2 * (i % 4))) & 3 and w = (q - 1) * d, so the four
 * codes give -d, 0, +d and (reserved code 3) +2d.  Exact in fp64. */
static void decode_q2_0_row(const uint8_t *row, int64_t k, double *w)
{
    for (int64_t b = 0; b < k / 128; ++b) {
        const uint8_t *blk = row + b * 34;
        double d = orc_f16_to_f64(rd_u16le(blk));
        for (int i = 0; i < 128; ++i) {
            int q = (blk[2 + i / 4] >> (2 * (i % 4))) & 3;
            w[b * 128 + i] = (double)(q - 1) * d;
        }
    }
}

/* Q8_0: per 32-weight block (34 bytes), d = fp16 at bytes 0-1; weight j is
 * the signed byte 2 + j (two's complement, -128..127) and w = q * d.  Exact in
 * fp64 (an 8-bit integer times an 11-bit significand). */
static void decode_q8_0_row(const uint8_t *row, int64_t k, double *w)
{
    for (int64_t b = 0; b < k / 32; ++b) {
        const uint8_t *blk = row + b * 34;
        double d = orc_f16_to_f64(rd_u16le(blk));
        for (int j = 0; j < 32; ++j) {
            int q = blk[2 + j] < 128 ? (int)blk[2 + j] : (int)blk[2 + j] - 256;
            w[b * 32 + j] = (double)q * d;
        }
    }
}

/* Q4_K: super-blocks of 256 weights in 144 bytes -- fp16 d (bytes 0-1), fp16
 * dmin (bytes 2-3), twelve bytes of 6-bit sub-block scales and mins (bytes
 * 4-15), then 128 code bytes.  Sub-block j (weights 32 j .. 32 j + 31) has
 * scale sc[j] and min m[j], and
 *     w = d * sc[j] * q - dmin * m[j].
 * The 6-bit fields, with b = bytes 4-15: for j < 4, sc[j] = b[j] & 63 and
 * m[j] = b[j + 4] & 63; for j >= 4, the low four bits of sc[j] are the low
 * nibble of b[j + 4] and its top two bits are the top two bits of b[j - 4];
 * the low four bits of m[j] are the high nibble of b[j + 4] and its top two
 * bits are the top two bits of b[j].  The codes form four runs of 32 bytes;
 * byte l of run c holds weight 64 c + l in its low nibble and weight
 * 64 c + 32 + l in its high nibble.
 * Exact in fp64 for every finite input: d * sc * q (at most 21 significant
 * bits) and dmin * m (17) are exact products, and their difference is an
 * integer multiple of 2^-24 below 2^27 in magnitude -- at most 51 significant
 * bits -- so the subtraction, whose exact result is representable, returns it. */
static void decode_q4_k_row(const uint8_t *row, int64_t k, double *w)
{
    for (int64_t b = 0; b < k / 256; ++b) {
        const uint8_t *blk = row + b * 144;
        const double d = orc_f16_to_f64(rd_u16le(blk));
        const double dmin = orc_f16_to_f64(rd_u16le(blk + 2));
        const uint8_t *sb = blk + 4, *qs = blk + 16;
        int sc[8], mn[8];
        for (int j = 0; j < 4; ++j) {
            sc[j] = sb[j] & 63;
            mn[j] = sb[j + 4] & 63;
            sc[j + 4] = (sb[j + 8] & 15) | ((sb[j] >> 6) << 4);
            mn[j + 4] = (sb[j + 8] >> 4) | ((sb[j + 4] >> 6) << 4);
        }
        for (int c = 0; c < 4; ++c) {
            for (int l = 0; l < 32; ++l) {
                const int q[2] = {qs[32 * c + l] & 15, qs[32 * c + l] >> 4};
                for (int h = 0; h < 2; ++h) {
                    const int j = 2 * c + h;
                    const int64_t idx = b * 256 + 64 * c + 32 * h + l;
                    w[idx] = d * sc[j] * q[h] - dmin * mn[j];
                }
            }
        }
    }
}

/* Ternary 1.58-bit: blocks of 256 weights in 54 bytes -- fp16 d (bytes 0-1),
 * then byte 2 + j holds weights 5 j .. 5 j + 4 as base-3 digits: weight
 * 5 j + i has t = (byte / 3^i) mod 3 and value (t - 1) * d, so the digits
 * 0, 1, 2 stand for -d, 0, +d.  The last weight (255) is digit 0 of byte 53.
 * A byte above 242 (byte 53: above 2) is not a valid code; returns -1 then.
 * Exact in fp64. */
static int decode_ternary_row(const uint8_t *row, int64_t k, double *w)
{
    for (int64_t b = 0; b < k / 256; ++b) {
        const uint8_t *blk = row + b * 54;
        const double d = orc_f16_to_f64(rd_u16le(blk));
        if (blk[53] > 2)
            return -1;
        for (int i = 0; i < 256; ++i) {
            const int byte = blk[2 + i / 5];
            if (byte > 242)
                return -1;
            int pw = 1;
            for (int e = 0; e < i % 5; ++e)
                pw *= 3;
            const int t = (byte / pw) % 3;
            w[b * 256 + i] = (double)(t - 1) * d;
        }
    }
    return 0;
}

/* MLX4 row n with group size G (64 or 32): q = (word[n][k/8] >> 4*(k%8)) & 15,
 * g = k / G, w = q * s[n][g] + b[n][g].  Exact in fp64: q*s has at most 15
 * significant bits and the sum of two fp16-derived values spans far fewer
 * than 53. */
static void decode_mlx4_row(const uint8_t *codes, const uint8_t *scales,
                            const uint8_t *biases, int64_t n_idx, int64_t k,
                            int64_t group, double *w)
{
    const uint8_t *crow = codes + n_idx * (k / 2);
    const uint8_t *srow = scales + n_idx * (k / group) * 2;
    const uint8_t *brow = biases + n_idx * (k / group) * 2;
    for (int64_t kk = 0; kk < k; ++kk) {
        uint32_t word = rd_u32le(crow + (kk / 8) * 4);
        int q = (int)((word >> (4 * (kk % 8))) & 0xF);
        double s = orc_f16_to_f64(rd_u16le(srow + (kk / group) * 2));
        double b = orc_f16_to_f64(rd_u16le(brow + (kk / group) * 2));
        w[kk] = (double)q * s + b;
    }
}

/* Decode rows [row0, row0 + nrows) of an [n, k] weight matrix held in the
 * canonical bytes `canon` into w[nrows][k].  The MLX stream is codes
 * (n*k/2 bytes), then scales (n*k/64 fp16), then biases (same).
 * Returns 0 on success, -1 on a bad codec or shape, -2 on an invalid code. */
int orc_decode_rows(int codec, const uint8_t *canon, int64_t n, int64_t k,
                    int64_t row0, int64_t nrows, double *w)
{
    int64_t bw, bb;
    if (!orc_block_geometry(codec, &bw, &bb) || k <= 0 || k % bw || row0 < 0 ||
        nrows < 0 || row0 + nrows > n)
        return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t nn = row0 + r;
        double *wr = w + r * k;
        if (codec == ORC_Q4_0)
            decode_q4_0_row(canon + nn * (k / 32) * 18, k, wr);
        else if (codec == ORC_Q2_0)
            decode_q2_0_row(canon + nn * (k / 128) * 34, k, wr);
        else if (codec == ORC_Q8_0)
            decode_q8_0_row(canon + nn * (k / 32) * 34, k, wr);
        else if (codec == ORC_Q4_K)
            decode_q4_k_row(canon + nn * (k / 256) * 144, k, wr);
        else if (codec == ORC_TERNARY || codec == ORC_TERNARY_Q2) {
            if (decode_ternary_row(canon + nn * (k / 256) * 54, k, wr))
                return -2;
        }
        else {
            const int64_t group = codec == ORC_MLX4_G32 ? 32 : 64;
            const uint8_t *codes = canon;
            const uint8_t *scales = canon + n * (k / 2);
            const uint8_t *biases = scales + n * (k / group) * 2;
            decode_mlx4_row(codes, scales, biases, nn, k, group, wr);
        }
    }
    return 0;
}

/* fp16 image of the decoded weights: each exact fp64 weight rounded once to
 * binary16 (nearest, ties to even).  This is the value a kernel must feed to
 * an fp16 matrix unit for its dequantization to be called exact. */
int orc_dequant_f16_rows(int codec, const uint8_t *canon, int64_t n, int64_t k,
                         int64_t row0, int64_t nrows, double *scratch,
                         uint16_t *out)
{
    int rc = orc_decode_rows(codec, canon, n, k, row0, nrows, scratch);
    if (rc)
        return rc;
    orc_f64_to_f16_array(scratch, out, nrows * k);
    return 0;
}

/* -------------------------------------------------------------- matmul --- */

/* ref[i][j] = sum_{kk=0}^{k-1} x[i][kk] * w[j][kk], where x holds fp16 bit
 * patterns with row stride ldx and w is the exact fp64 decode [n][k].  Naive
 * triple loop: k ascending into a single fp64 accumulator per output.  The
 * outer loop over rows is split across threads; no output's order changes. */
void orc_matmul_xwt(const uint16_t *x, int64_t ldx, const double *w, int64_t m,
                    int64_t n, int64_t k, double *ref, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        double *xr = (double *)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
        for (int64_t kk = 0; kk < k; ++kk)
            xr[kk] = orc_f16_to_f64(x[i * ldx + kk]);
        for (int64_t j = 0; j < n; ++j) {
            const double *wr = w + j * k;
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk)
                acc += xr[kk] * wr[kk];
            ref[i * n + j] = acc;
        }
        free(xr);
    }
}

/* SiLU(g) * u = g / (1 + exp(-g)) * u, elementwise in fp64 (comparison page
 * section 2.2: the activation applied to the gate projection, times up). */
void orc_swiglu(const double *g, const double *u, double *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* out = GELU(g) * u with GELU(g) = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))). */
void orc_geglu(const double *g, const double *u, double *out, int64_t count)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    for (int64_t i = 0; i < count; ++i) {
        const double x = g[i];
        out[i] = 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x))) * u[i];
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
