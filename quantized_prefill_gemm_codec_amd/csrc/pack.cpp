// Host side of the C-ABI: plane sizes, canonical -> planar repack, status text.
//
// The repack only moves bits: every code keeps its value, every fp16 scale and
// bias keeps its bit pattern.  The layout it produces is described in planar.h.
#include <string.h>

#include "../../include/qgemm.h"
#include "planar.h"

using namespace qg;

namespace {

bool valid_codec(int32_t c)
{
    return c == Q4_0 || c == MLX4_G64 || c == Q2_0 || c == Q8_0 || c == MLX4_G32 || c == Q4_K || c == TERNARY ||
           c == TERNARY_Q2;
}

qg_status check_shape(int32_t codec, int64_t n, int64_t k)
{
    if (!valid_codec(codec))
        return QG_ERR_CODEC;
    if (n < 1 || k < 1 || k % block_size(codec) != 0)
        return QG_ERR_SHAPE;
    if (n > (int64_t(1) << 31) || k > (int64_t(1) << 31))
        return QG_ERR_SHAPE;
    return QG_OK;
}

size_t canonical_size(int32_t codec, int64_t n, int64_t k)
{
    if (codec == Q4_0)
        return size_t(n) * size_t(k / 32) * 18;
    if (codec == Q2_0)
        return size_t(n) * size_t(k / 128) * 34;
    if (codec == Q8_0)
        return size_t(n) * size_t(k / 32) * 34;
    if (codec == Q4_K)
        return size_t(n) * size_t(k / 256) * 144;
    if (codec == TERNARY || codec == TERNARY_Q2)
        return size_t(n) * size_t(k / 256) * 54;
    const int64_t group = codec == MLX4_G32 ? 32 : 64;
    return size_t(n) * size_t(k / 2) + 2 * size_t(n) * size_t(k / group) * 2;
}

inline uint16_t rd16(const uint8_t *p) { return uint16_t(p[0] | (p[1] << 8)); }
inline void wr16(uint8_t *p, uint16_t v)
{
    p[0] = uint8_t(v & 0xFF);
    p[1] = uint8_t(v >> 8);
}

// code of weight (row, kk) in the canonical stream (Q8_0: q + 128, 0..255)
inline int canonical_code(int32_t codec, const uint8_t *c, int64_t row, int64_t kk, int64_t k)
{
    if (codec == Q8_0) {
        const uint8_t *blk = c + (row * (k / 32) + kk / 32) * 34;
        return int(blk[2 + kk % 32] ^ 0x80u);
    }
    if (codec == Q4_0) {
        const uint8_t *blk = c + (row * (k / 32) + kk / 32) * 18;
        int j = int(kk % 32);
        return j < 16 ? (blk[2 + j] & 0xF) : (blk[2 + j - 16] >> 4);
    }
    if (codec == Q4_K) {
        // four 32-byte runs; byte l of run u: weight 64 u + l (low nibble), 64 u + 32 + l (high)
        const uint8_t *blk = c + (row * (k / 256) + kk / 256) * 144;
        const int w = int(kk % 256), l = w % 64;
        const uint8_t b = blk[16 + 32 * (w / 64) + l % 32];
        return l < 32 ? (b & 0xF) : (b >> 4);
    }
    if (codec == TERNARY || codec == TERNARY_Q2) {
        // base-3 digit kk % 5 of byte 2 + (kk % 256) / 5 (digits 0..2); as a
        // 2-bit code (TERNARY_Q2) the digit t is q with w = (q - 1) d
        static const int pw[5] = {1, 3, 9, 27, 81};
        const uint8_t *blk = c + (row * (k / 256) + kk / 256) * 54;
        const int w = int(kk % 256);
        return (blk[2 + w / 5] / pw[w % 5]) % 3;
    }
    if (codec == Q2_0) {
        const uint8_t *blk = c + (row * (k / 128) + kk / 128) * 34;
        int i = int(kk % 128);
        return (blk[2 + i / 4] >> (2 * (i % 4))) & 3;
    }
    const uint8_t *word = c + (row * (k / 8) + kk / 8) * 4;
    int e = int(kk % 8);
    return (word[e / 2] >> (4 * (e % 2))) & 0xF;
}

// Fixed-point base-3 byte of up to five digits (digit 0 most significant):
// ceil(256 v / 243) with v = sum_i t_i 3^(4 - i).
inline uint8_t base3_fixed(const int *t, int nd)
{
    int v = 0;
    for (int i = 0; i < 5; ++i)
        v = v * 3 + (i < nd ? t[i] : 0);
    return uint8_t((256 * v + 242) / 243);
}

bool ternary_codes_valid(const uint8_t *c, int64_t n, int64_t k)
{
    const int64_t blocks = n * (k / 256);
    for (int64_t b = 0; b < blocks; ++b) {
        const uint8_t *blk = c + b * 54;
        for (int j = 2; j < 53; ++j)
            if (blk[j] > 242)
                return false;
        if (blk[53] > 2)
            return false;
    }
    return true;
}

// Ternary digit plane: per chunk A[64] u32, B[64] u16, T[32] u8 (planar.h).
void pack_ternary_codes(const uint8_t *c, int64_t n, int64_t k, const Geometry &g, uint8_t *q)
{
    for (int64_t r = 0; r < g.groups; ++r)
        for (int64_t t = 0; t < g.ksteps; ++t) {
            uint8_t *chunk = q + (r * g.ksteps + t) * TERNARY_CHUNK;
            for (int l = 0; l < 64; ++l) {
                const int gh = l / 32, i = l % 32;
                const int64_t row = r * 32 + i;
                int dig[32];
                for (int j = 0; j < 32; ++j) {
                    const int64_t kk = t * 64 + gh * 32 + j;
                    dig[j] = (row < n && kk < k) ? canonical_code(TERNARY, c, row, kk, k) : 1;   // pad: q = 0
                }
                uint8_t e[3], o[3];
                for (int b = 0; b < 3; ++b) {
                    int de[5], dd[5];
                    for (int u = 0; u < 5; ++u) {
                        de[u] = dig[2 * (5 * b + u)];
                        dd[u] = dig[2 * (5 * b + u) + 1];
                    }
                    e[b] = base3_fixed(de, 5);
                    o[b] = base3_fixed(dd, 5);
                }
                chunk[l * 4 + 0] = e[0];
                chunk[l * 4 + 1] = o[0];
                chunk[l * 4 + 2] = e[1];
                chunk[l * 4 + 3] = o[1];
                chunk[256 + l * 2 + 0] = e[2];
                chunk[256 + l * 2 + 1] = o[2];
            }
            for (int tl = 0; tl < 32; ++tl) {     // tail byte of lanes 2 tl and 2 tl + 1
                int td[4];
                for (int h = 0; h < 2; ++h) {
                    const int l = 2 * tl + h, gh = l / 32, i = l % 32;
                    const int64_t row = r * 32 + i;
                    for (int u = 0; u < 2; ++u) {
                        const int64_t kk = t * 64 + gh * 32 + 30 + u;
                        td[2 * h + u] = (row < n && kk < k) ? canonical_code(TERNARY, c, row, kk, k) : 1;
                    }
                }
                chunk[384 + tl] = base3_fixed(td, 4);
            }
        }
}

}  // namespace

extern "C" {

int32_t qg_version(void) { return 102; }

const char *qg_status_str(qg_status s)
{
    switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "null pointer argument";
    case QG_ERR_CODEC: return "unknown codec id";
    case QG_ERR_SHAPE: return "unsupported shape (M/N/K range, K not a multiple of the block, stride too small)";
    case QG_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
    case QG_ERR_MISMATCH: return "gate and up weights differ in codec, N or K";
    case QG_ERR_LAUNCH: return "kernel launch failed";
    case QG_ERR_SIZE: return "host buffer smaller than the format requires";
    case QG_ERR_CODE: return "canonical code byte outside the codec's range";
    }
    return "unknown status";
}

qg_status qg_packed_sizes(int32_t codec, int64_t n, int64_t k, size_t *qs_bytes,
                          size_t *scales_bytes)
{
    qg_status st = check_shape(codec, n, k);
    if (st != QG_OK)
        return st;
    Geometry g = geometry(codec, n, k);
    if (qs_bytes)
        *qs_bytes = size_t(g.qs_bytes);
    if (scales_bytes)
        *scales_bytes = size_t(g.scale_bytes);
    return QG_OK;
}

qg_status qg_canonical_size(int32_t codec, int64_t n, int64_t k, size_t *bytes)
{
    qg_status st = check_shape(codec, n, k);
    if (st != QG_OK)
        return st;
    if (!bytes)
        return QG_ERR_NULL;
    *bytes = canonical_size(codec, n, k);
    return QG_OK;
}

qg_status qg_pack_host(int32_t codec, int64_t n, int64_t k, const void *canonical,
                       size_t canonical_bytes, void *qs, void *scales)
{
    qg_status st = check_shape(codec, n, k);
    if (st != QG_OK)
        return st;
    if (!canonical || !qs || !scales)
        return QG_ERR_NULL;
    if (canonical_bytes < canonical_size(codec, n, k))
        return QG_ERR_SIZE;
    if ((codec == TERNARY || codec == TERNARY_Q2) && !ternary_codes_valid(static_cast<const uint8_t *>(canonical), n, k))
        return QG_ERR_CODE;

    const uint8_t *c = static_cast<const uint8_t *>(canonical);
    uint8_t *q = static_cast<uint8_t *>(qs);
    uint8_t *s = static_cast<uint8_t *>(scales);
    Geometry g = geometry(codec, n, k);
    const int cb = lane_code_bytes(codec);
    const bool four_bit = codec == Q4_0 || is_mlx(codec) || codec == Q4_K;
    // zero-weight code for padding: Q4_0 q = 8, Q2_0 q = 1, Q8_0 q = 0 (stored
    // 128), MLX and Q4_K q = 0 (zero scale records)
    const int pad_code = codec == Q4_0 ? 8 : (codec == Q2_0 || codec == TERNARY_Q2) ? 1 : codec == Q8_0 ? 128 : 0;

    memset(q, 0, size_t(g.qs_bytes));
    memset(s, 0, size_t(g.scale_bytes));

    if (codec == TERNARY) {
        pack_ternary_codes(c, n, k, g, q);
        const int64_t nb = k / 256;
        for (int64_t row = 0; row < n; ++row)
            for (int64_t blk = 0; blk < nb; ++blk)
                wr16(s + (((row / 32) * nb + blk) * 32 + row % 32) * 2, rd16(c + (row * nb + blk) * 54));
        return QG_OK;
    }

    for (int64_t r = 0; r < g.groups; ++r) {
        for (int64_t t = 0; t < g.ksteps; ++t) {
            uint8_t *chunk = q + (r * g.ksteps + t) * 64 * cb;
            for (int l = 0; l < 64; ++l) {
                const int gh = l / 32, i = l % 32;
                const int64_t row = r * 32 + i;
                uint8_t *lane = chunk + l * (cb == 32 ? 16 : cb);
                for (int j = 0; j < 32; ++j) {
                    const int64_t kk = t * 64 + gh * 32 + j;
                    const int code = (row < n && kk < k) ? canonical_code(codec, c, row, kk, k) : pad_code;
                    int byte, shift;
                    if (codec == Q8_0) {
                        // word 2 s + e / 4 of the lane's 8; words 4 h .. 4 h + 3
                        // sit in the chunk's half h (1 KiB apart)
                        const int s8 = j / 8, e = j % 8, word = 2 * s8 + e / 4, e4 = e % 4;
                        const int bit = 8 * (e4 / 2) + 16 * (e4 % 2);
                        byte = (word / 4) * 1024 + (word % 4) * 4 + bit / 8;
                        shift = 0;
                    } else if (four_bit) {
                        const int dw = j / 8, e = j % 8;
                        const int bit = 4 * (e / 2) + 16 * (e % 2);
                        byte = 4 * dw + bit / 8;
                        shift = bit % 8;
                    } else {
                        const int dw = j / 16, e = j % 16;
                        const int bit = 2 * (e / 2) + 16 * (e % 2);
                        byte = 4 * dw + bit / 8;
                        shift = bit % 8;
                    }
                    lane[byte] = uint8_t(lane[byte] | (code << shift));
                }
            }
        }
    }

    // scale / bias planes (padding entries stay zero -> padded weights decode to 0)
    for (int64_t row = 0; row < n; ++row) {
        const int64_t r = row / 32, i = row % 32;
        if (codec == Q4_0 || codec == Q8_0) {
            const int64_t bb = codec == Q4_0 ? 18 : 34;
            for (int64_t blk = 0; blk < k / 32; ++blk) {
                const int64_t t = blk / 2, gh = blk % 2;
                wr16(s + (((r * g.ksteps + t) * 2 + gh) * 32 + i) * 2, rd16(c + (row * (k / 32) + blk) * bb));
            }
        } else if (codec == Q4_K) {
            // unpack the twelve bytes of 6-bit fields: for j < 4, sc[j] and
            // m[j] are the low 6 bits of bytes j and j + 4; for j >= 4 the low
            // nibble / high nibble of byte j + 4 give the low 4 bits of sc[j] /
            // m[j], and the top 2 bits of bytes j - 4 / j their top 2 bits
            const int64_t nsb = k / 256;
            for (int64_t sbk = 0; sbk < nsb; ++sbk) {
                const uint8_t *blk = c + (row * nsb + sbk) * 144;
                const uint8_t *f = blk + 4;
                uint8_t scv[8], mv[8];
                for (int j = 0; j < 4; ++j) {
                    scv[j] = uint8_t(f[j] & 63);
                    mv[j] = uint8_t(f[j + 4] & 63);
                    scv[j + 4] = uint8_t((f[j + 8] & 15) | ((f[j] >> 6) << 4));
                    mv[j + 4] = uint8_t((f[j + 8] >> 4) | ((f[j + 4] >> 6) << 4));
                }
                uint8_t *rec = s + (r * nsb + sbk) * 640;
                for (int u = 0; u < 4; ++u)
                    for (int gh = 0; gh < 2; ++gh) {
                        uint8_t *e = rec + u * 128 + (gh * 32 + i) * 2;
                        e[0] = scv[2 * u + gh];
                        e[1] = mv[2 * u + gh];
                    }
                memcpy(rec + 512 + i * 4, blk, 4);     // fp16 d, fp16 dmin
            }
        } else if (codec == Q2_0) {
            const int64_t nb = k / 128;
            for (int64_t blk = 0; blk < nb; ++blk)
                wr16(s + ((r * nb + blk) * 32 + i) * 2, rd16(c + (row * nb + blk) * 34));
        } else if (codec == TERNARY_Q2) {
            // the Q2_0 plane: one entry per 128 weights, each 256-weight block's d twice
            const int64_t nb = k / 128;
            for (int64_t blk = 0; blk < nb; ++blk)
                wr16(s + ((r * nb + blk) * 32 + i) * 2, rd16(c + (row * (k / 256) + blk / 2) * 54));
        } else {
            const int64_t group = codec == MLX4_G32 ? 32 : 64;
            const int64_t ng = k / group;
            const uint8_t *sc = c + size_t(n) * size_t(k / 2);
            const uint8_t *bi = sc + size_t(n) * size_t(ng) * 2;
            for (int64_t grp = 0; grp < ng; ++grp) {
                // G64: record (t, i); G32: record (t, g, i) with group = 2t + g
                const int64_t rec = codec == MLX4_G32 ? ((r * g.ksteps + grp / 2) * 2 + grp % 2) * 32 + i
                                                      : (r * g.ksteps + grp) * 32 + i;
                uint8_t *e = s + rec * 4;
                wr16(e, rd16(sc + (row * ng + grp) * 2));
                wr16(e + 2, rd16(bi + (row * ng + grp) * 2));
            }
        }
    }
    return QG_OK;
}

qg_status qg_pack_kv_host(const void *canonical, size_t canonical_bytes, int64_t rows, int64_t head_dim,
                          void *codes, void *scales)
{
    if (!canonical || !codes || !scales)
        return QG_ERR_NULL;
    if (rows < 1 || head_dim < 32 || head_dim % 32 != 0 || rows > (int64_t(1) << 31) || head_dim > 4096)
        return QG_ERR_SHAPE;
    const int64_t nb = head_dim / 32;
    if (canonical_bytes < size_t(rows) * size_t(nb) * 34)
        return QG_ERR_SIZE;
    const uint8_t *c = static_cast<const uint8_t *>(canonical);
    uint8_t *q = static_cast<uint8_t *>(codes);
    uint8_t *sc = static_cast<uint8_t *>(scales);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = c + (r * nb + b) * 34;
            memcpy(sc + (r * nb + b) * 2, blk, 2);
            for (int j = 0; j < 32; ++j)   // q + 128: the two's-complement byte with its top bit flipped
                q[r * head_dim + b * 32 + j] = uint8_t(blk[2 + j] ^ 0x80u);
        }
    return QG_OK;
}

}  // extern "C"
