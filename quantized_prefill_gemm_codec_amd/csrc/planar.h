// Planar device format of the packed weights (host and device).
//
// The pages trace a measured slowdown to interleaved block structs whose size
// is not a multiple of 16 bytes (comparison page, section 4, the 20-byte MLX
// struct: 20 mod 16 = 4); 18-byte Q4_0 and 34-byte Q2_0 blocks share the
// problem (both are 2 mod 16).  The library therefore keeps codes and scales in
// separate planes and orders the codes so that one 64-lane wavefront reads one
// contiguous 1 KiB (4-bit) or 512 B (2-bit) chunk per 128-bit (64-bit) load --
// the "2D block-swizzled" tile-major weight layout of the project index,
// Pillar 1, Brick 2, laid out for gfx950 wavefronts.
//
// Geometry.  W [N, K] is cut into row groups of 32 rows and k-steps of 64
// weights (N and K padded up; padding decodes to zero).  Within a (row group
// r, k-step t) chunk, lane l = 32 * g + i owns row 32 r + i and the 32 weights
// k = 64 t + 32 g + j, j = 0..31.  These are exactly the 8-element K slices a
// lane feeds to v_mfma_f32_32x32x16_f16 over four 16-deep sub-steps:
// sub-step s uses j = 8 s .. 8 s + 7.
//
// Code order inside a lane's bytes (chosen so that unpacking needs one shift,
// one and-or per pair of weights and no byte shuffles):
//  * 4-bit (Q4_0, MLX4-G64, MLX4-G32, Q4_K): 16 bytes = 4 dwords; dword s holds j = 8 s + e,
//    with e = 2p at bits [4p, 4p+4) and e = 2p + 1 at bits [16+4p, 20+4p).
//  * 2-bit (Q2_0): 8 bytes = 2 dwords; dword h holds j = 16 h + e, with
//    e = 2p at bits [2p, 2p+2) and e = 2p + 1 at bits [16+2p, 18+2p).
//  * 8-bit (Q8_0): 32 bytes = 8 dwords, stored as two 16-byte halves 1 KiB
//    apart (the chunk is [half 0 of all 64 lanes][half 1 of all 64 lanes], so
//    each half is one contiguous 128-bit wave load); dword 2 s + h' holds
//    j = 8 s + 4 h' + e, with e = 0, 1, 2, 3 at bits 0, 16, 8, 24, as the
//    unsigned byte q + 128.
// So every extracted pair lands as (low half, high half) = (even e, odd e),
// the element order of a packed fp16 register.
//
// Scale planes, one 64-lane (Q4_0) or 32-lane record per chunk:
//  * Q4_0:     fp16 [N/32][K/64][2][32]  -- d of block 2t+g for lane (g, i)
//  * Q8_0:     same as Q4_0
//  * MLX4-G32: u32  [N/32][K/64][2][32]  -- (s, b) of group 2t+g for lane (g, i)
//  * MLX4-G64: u32  [N/32][K/64][32]     -- (s, b) of group t as two fp16
//                                           (scale low half, bias high half),
//                                           so one 32-bit load brings both
//  * Q2_0:     fp16 [N/32][K/128][32]    -- d of block t/2
//  * Q4_K:     [N/32][K/256][640 bytes], one record per (row group,
//              super-block): bytes 128 u .. 128 u + 127 are u16 [64 lanes]
//              for k-step 4 sb + u, lane (g, i) holding sc | m << 8 of its
//              sub-block 2 u + g (the 6-bit fields unpacked to bytes); bytes
//              512..639 are u32 [32 rows], fp16 d low and fp16 dmin high.
//              4.625 bits per weight (canonical: 4.5).
//  * Ternary:  fp16 [N/32][K/256][32]    -- d of block t/4
//
// Ternary codes keep the canonical density (1.625 bits per weight of digits):
// a (row group, k-step) chunk is 416 bytes -- u32 A[64 lanes], u16 B[64 lanes],
// u8 T[32].  Lane l's 32 weights form pairs p = (j = 2p, 2p + 1); for p < 15
// the even weight is digit p % 5 of byte E[p / 5] and the odd one digit p % 5
// of byte O[p / 5], with A = E0 | O0 << 8 | E1 << 16 | O1 << 24 and
// B = E2 | O2 << 8; weights 30, 31 are digits 2 (l & 1) and 2 (l & 1) + 1 of
// T[l / 2].  Digits are t = q + 1 in {0, 1, 2}.  Each byte stores its (up to
// five) digits in fixed-point base 3: byte = ceil(256 v / 243) with
// v = sum_i t_i 3^(4 - i), so that digit i = ((byte 3^i) mod 256) 3 >> 8 --
// every digit comes out with the same four 16-bit operations, two bytes (one
// per register half) at a time.
#pragma once
#include <stddef.h>
#include <stdint.h>

#define QG_ROWS_PER_GROUP 32
#define QG_KSTEP 64

#ifdef __HIPCC__
#define QG_HD __host__ __device__
#else
#define QG_HD
#endif

namespace qg {

enum Codec : int32_t { Q4_0 = 1, MLX4_G64 = 2, Q2_0 = 3, Q8_0 = 4, MLX4_G32 = 5, Q4_K = 6, TERNARY = 7, TERNARY_Q2 = 8 };

// The kernels a codec's planar format runs on.  TERNARY_Q2 is the ternary
// canonical format repacked as 2-bit codes q = t (the digit, 0..2) with the
// 256-weight block's scale repeated for both 128-weight halves: exactly the
// Q2_0 planar format, w = (q - 1) d.
QG_HD inline int kernel_codec(int codec) { return codec == TERNARY_Q2 ? int(Q2_0) : codec; }

constexpr int TERNARY_CHUNK = 416;   // bytes of ternary digits per (row group, k-step)

QG_HD inline bool is_mlx(int codec) { return codec == MLX4_G64 || codec == MLX4_G32; }

QG_HD inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

QG_HD inline int block_size(int codec)
{
    return codec == Q4_0 ? 32 : codec == MLX4_G64 ? 64 : codec == Q2_0 ? 128 : codec == Q8_0 ? 32 : codec == MLX4_G32 ? 32
         : codec == Q4_K ? 256 : codec == TERNARY ? 256 : codec == TERNARY_Q2 ? 256 : 0;
}

// bytes of codes a lane holds per chunk
QG_HD inline int lane_code_bytes(int codec) { return codec == Q2_0 || codec == TERNARY_Q2 ? 8 : codec == Q8_0 ? 32 : 16; }

struct Geometry {
    int64_t groups;   // row groups (N padded to 32) / 32
    int64_t ksteps;   // K padded to 64, / 64
    int64_t qs_bytes, scale_bytes;
};

QG_HD inline Geometry geometry(int codec, int64_t n, int64_t k)
{
    Geometry g;
    g.groups = ceil_div(n, QG_ROWS_PER_GROUP);
    g.ksteps = ceil_div(k, QG_KSTEP);
    g.qs_bytes = codec == TERNARY ? g.groups * g.ksteps * TERNARY_CHUNK : g.groups * g.ksteps * 64 * lane_code_bytes(codec);
    if (codec == Q4_0 || codec == Q8_0)
        g.scale_bytes = g.groups * g.ksteps * 64 * 2;
    else if (codec == MLX4_G32)
        g.scale_bytes = g.groups * g.ksteps * 64 * 4;
    else if (codec == MLX4_G64)
        g.scale_bytes = g.groups * g.ksteps * 32 * 4;
    else if (codec == Q4_K)
        g.scale_bytes = g.groups * (g.ksteps / 4) * 640;
    else if (codec == TERNARY)
        g.scale_bytes = g.groups * (g.ksteps / 4) * 64;
    else
        g.scale_bytes = g.groups * ceil_div(k, 128) * 32 * 2;
    return g;
}

}  // namespace qg
