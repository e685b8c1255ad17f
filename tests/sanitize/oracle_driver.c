/* Sanitizer driver for the CPU oracle (oracle/qgemm_oracle.c): every codec's
 * decode and fp16 dequant on exactly sized heap buffers, the matmul, SwiGLU and
 * GeGLU, and both fp16 conversions over all 65536 patterns.  Built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py (without OpenMP, so
 * the runtime's own allocations stay out of the leak report).  Exit status 0
 * means every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double orc_f16_to_f64(uint16_t h);
uint16_t orc_f64_to_f16(double x);
int orc_block_geometry(int codec, int64_t *weights, int64_t *bytes);
int orc_decode_rows(int codec, const uint8_t *canon, int64_t n, int64_t k, int64_t row0, int64_t nrows, double *w);
int orc_dequant_f16_rows(int codec, const uint8_t *canon, int64_t n, int64_t k, int64_t row0, int64_t nrows,
                         double *scratch, uint16_t *out);
void orc_matmul_xwt(const uint16_t *x, int64_t ldx, const double *w, int64_t m, int64_t n, int64_t k, double *ref,
                    int nthreads);
void orc_swiglu(const double *g, const double *u, double *out, int64_t count);
void orc_geglu(const double *g, const double *u, double *out, int64_t count);

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint8_t next_byte(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint8_t)(state >> 56);
}

static size_t canonical_bytes(int codec, int64_t n, int64_t k, int64_t bw, int64_t bb)
{
    if (codec == 2 || codec == 5) /* MLX: codes, scales, biases */
        return (size_t)(n * k / 2 + 2 * n * (k / bw) * 2);
    return (size_t)(n * (k / bw) * bb);
}

int main(void)
{
    int bad = 0;
    for (uint32_t h = 0; h < 65536; ++h) {
        double v = orc_f16_to_f64((uint16_t)h);
        if (v == v && orc_f64_to_f16(v) != h && !((h & 0x7FFF) == 0))
            bad = 1, fprintf(stderr, "fp16 round trip %04x\n", h);
    }
    for (int codec = 1; codec <= 7; ++codec) {
        int64_t bw, bb;
        if (!orc_block_geometry(codec, &bw, &bb)) {
            bad = 1;
            continue;
        }
        const int64_t n = 37, k = 2 * (bw > 256 ? bw : 256), m = 5;
        const size_t cb = canonical_bytes(codec, n, k, bw, bb);
        uint8_t *canon = malloc(cb);
        for (size_t i = 0; i < cb; ++i)
            canon[i] = next_byte();
        for (size_t i = 0; i + 1 < cb; i += 2) /* keep scales finite: clear exponent-all-ones patterns */
            if ((canon[i + 1] & 0x7C) == 0x7C)
                canon[i + 1] &= 0xBB;
        if (codec == 7)
            for (size_t blk = 0; blk < cb / 54; ++blk) {
                for (int j = 2; j < 53; ++j)
                    canon[blk * 54 + j] %= 243;
                canon[blk * 54 + 53] %= 3;
            }
        double *w = malloc(sizeof(double) * n * k), *scratch = malloc(sizeof(double) * n * k);
        uint16_t *w16 = malloc(sizeof(uint16_t) * n * k), *x = malloc(sizeof(uint16_t) * m * k);
        double *ref = malloc(sizeof(double) * m * n), *g2 = malloc(sizeof(double) * m * n);
        if (orc_decode_rows(codec, canon, n, k, 0, n, w) || orc_dequant_f16_rows(codec, canon, n, k, 3, n - 3, scratch, w16))
            bad = 1, fprintf(stderr, "decode codec %d\n", codec);
        if (orc_decode_rows(codec, canon, n, k, 1, n, w) != -1)
            bad = 1, fprintf(stderr, "row range past n accepted, codec %d\n", codec);
        for (int64_t i = 0; i < m * k; ++i)
            x[i] = (uint16_t)(0x3000 + (next_byte() & 0x3FF));
        orc_matmul_xwt(x, k, w, m, n, k, ref, 1);
        orc_swiglu(ref, ref, g2, m * n);
        orc_geglu(ref, g2, g2, m * n);
        free(canon), free(w), free(scratch), free(w16), free(x), free(ref), free(g2);
    }
    if (!bad)
        printf("oracle driver: all calls returned the expected status\n");
    return bad;
}
