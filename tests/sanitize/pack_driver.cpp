// Sanitizer driver for the library's host code (pack.cpp): every codec's
// canonical -> planar repack on exactly sized heap buffers, the KV-cache split,
// plane sizes and the argument errors.  Built with -fsanitize=address,undefined
// by tests/test_sanitizers.py; any out-of-bounds access, leak or undefined
// operation aborts it.  Exit status 0 means every call returned what it should.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "qgemm.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint8_t next_byte()
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return uint8_t(state >> 56);
}

static int fail(const char *what, int codec, long n, long k, int st)
{
    fprintf(stderr, "%s: codec %d n %ld k %ld status %d\n", what, codec, n, k, st);
    return 1;
}

static const int BLOCK[8] = {0, 32, 64, 128, 32, 32, 256, 256};

int main()
{
    int bad = 0;
    for (int codec = 1; codec <= 7; ++codec) {
        const long b = BLOCK[codec];
        const long ns[] = {1, 31, 33, 64, 100};
        const long ks[] = {b, 2 * b, 512 / b * b + (b < 512 ? 0 : b), 1024};
        for (long n : ns)
            for (long k : ks) {
                if (k % b)
                    continue;
                size_t cb = 0, qb = 0, sb = 0;
                int st = qg_canonical_size(codec, n, k, &cb);
                if (st) { bad |= fail("canonical_size", codec, n, k, st); continue; }
                st = qg_packed_sizes(codec, n, k, &qb, &sb);
                if (st) { bad |= fail("packed_sizes", codec, n, k, st); continue; }
                uint8_t *canon = (uint8_t *)malloc(cb);
                for (size_t i = 0; i < cb; ++i)
                    canon[i] = next_byte();
                if (codec == QG_CODEC_TERNARY_1_58)   // digit bytes 0..242, the last byte of a block 0..2
                    for (size_t blk = 0; blk < cb / 54; ++blk) {
                        for (int j = 2; j < 53; ++j)
                            canon[blk * 54 + j] %= 243;
                        canon[blk * 54 + 53] %= 3;
                    }
                uint8_t *qs = (uint8_t *)malloc(qb), *sc = (uint8_t *)malloc(sb);
                st = qg_pack_host(codec, n, k, canon, cb, qs, sc);
                if (st)
                    bad |= fail("pack_host", codec, n, k, st);
                if (qg_pack_host(codec, n, k, canon, cb - 1, qs, sc) != QG_ERR_SIZE)
                    bad |= fail("short canonical accepted", codec, n, k, 0);
                if (codec == QG_CODEC_TERNARY_1_58) {
                    canon[cb - 1] = 3;
                    if (qg_pack_host(codec, n, k, canon, cb, qs, sc) != QG_ERR_CODE)
                        bad |= fail("invalid ternary byte accepted", codec, n, k, 0);
                }
                free(qs);
                free(sc);
                free(canon);
            }
        if (qg_pack_host(codec, 4, b, NULL, 0, NULL, NULL) == QG_OK)
            bad |= fail("null pointers accepted", codec, 4, b, 0);
        if (qg_packed_sizes(codec, 4, b + (b > 1 ? b / 2 : 1), NULL, NULL) != QG_ERR_SHAPE)
            bad |= fail("ragged K accepted", codec, 4, b, 0);
    }
    // KV cache split: rows x head_dim int8 codes, rows x head_dim/32 fp16 scales
    for (long d : {32L, 64L, 128L})
        for (long rows : {1L, 7L, 300L}) {
            const size_t cb = size_t(rows) * (d / 32) * 34;
            uint8_t *canon = (uint8_t *)malloc(cb);
            for (size_t i = 0; i < cb; ++i)
                canon[i] = next_byte();
            uint8_t *codes = (uint8_t *)malloc(rows * d), *scales = (uint8_t *)malloc(rows * (d / 32) * 2);
            int st = qg_pack_kv_host(canon, cb, rows, d, codes, scales);
            if (st)
                bad |= fail("pack_kv_host", 4, rows, d, st);
            if (qg_pack_kv_host(canon, cb - 1, rows, d, codes, scales) != QG_ERR_SIZE)
                bad |= fail("short kv canonical accepted", 4, rows, d, 0);
            free(codes);
            free(scales);
            free(canon);
        }
    for (int s = 0; s >= -8; --s)
        if (!qg_status_str((qg_status)s) || !*qg_status_str((qg_status)s))
            bad |= fail("status_str", 0, 0, 0, s);
    if (!bad)
        printf("pack driver: all calls returned the expected status\n");
    return bad;
}
