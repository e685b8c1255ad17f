// Per-codec unpack stage (device): planar code words -> fp16 weights.
//
// The pages run every codec through one shared unpack contract that feeds the
// matrix-unit GEMM, the SwiGLU core and the GEMV (releases page, v0.2.3,
// TCodec::unpack_column); this header is that stage for gfx950.  All three
// codecs use the same integer trick: OR-ing a code field into the mantissa of
// a binary16 power of two 2^E whose mantissa step 2^(E-10) equals the field's
// own bit weight gives exactly 2^E + q, two codes per 32-bit register (one per
// half).  Choosing E per field position (E = 10 for bits 0.., 6 for bits 4..
// of a 4-bit field; E = 10, 8, 6, 4 for 2-bit fields at bits 0, 2, 4, 6)
// reads each field in place -- one 8-bit shift per code word reaches the rest.
// One packed fp16 subtraction of 2^E + zero point is then exact and yields the
// signed integer weight factor, and a single packed multiply (or fused
// multiply-add) rounds once to the nearest binary16 -- so the fp16 operand
// handed to the MFMA is the correctly rounded value of the exact codec weight:
//   Q4_0      w = (q - 8) * d              (v_pk_add_f16, v_pk_mul_f16)
//   MLX4-G64  w = fma(q, s, b)             (v_pk_add_f16, v_pk_fma_f16)
//   MLX4-G32  the same, one (s, b) per 32 weights
//   Q2_0      w = (q - 1) * d, q=3 -> +2d  (v_pk_add_f16, v_pk_mul_f16)
//   Q8_0      w = q * d, stored q + 128    (v_pk_add_f16, v_pk_mul_f16)
//   ternary   w = (t - 1) * d, digit t of a fixed-point base-3 byte (one
//             v_pk_mul_lo_u16, one v_pk_lshrrev_b16 and one v_pk_mad_u16 per
//             two digits, then the or / v_pk_add_f16 / v_pk_mul_f16 of the
//             others)
//   Q4_K      w = d sc q - dmin m          (no insertion: the masked field is
//             read as the fp16 subnormal q 2^-24 (bits 0..3) or q 2^-20 (bits
//             4..7), and v_fma_mix{lo,hi}_f16 multiply it by the fp32 value
//             d sc 2^24 or d sc 2^20, add the fp32 value -dmin m and round
//             once to fp16; see mix_pair)
// (Q2_0 values are exact; Q4_0, MLX and Q4_K round once.  fp16 subnormals are
// kept: an MLX weight with q = 0 is its bias, which may be subnormal.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "planar.h"

namespace qg {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// A binary16 power of two, twice, held in a VGPR the compiler cannot see
// through: with the mask in an SGPR, mask-and-insert then fits one
// v_and_or_b32 (gfx9 VOP3 encodings take no literal operands).
template <uint32_t V> __device__ __forceinline__ uint32_t opaque_u32()
{
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
    return r;
}
__device__ __forceinline__ uint32_t magic1024() { return opaque_u32<0x64006400u>(); }

// The insertion constants (2^E, 2^E) of the unpack, one register each.
struct Magics {
    uint32_t m1024, m256, m64, m16;
};
__device__ __forceinline__ Magics make_magics()
{
    return Magics{opaque_u32<0x64006400u>(), opaque_u32<0x5C005C00u>(), opaque_u32<0x54005400u>(),
                  opaque_u32<0x4C004C00u>()};
}

// The codes a lane owns in one (row group, k-step) chunk, plus its scales.
template <int CODEC> struct LaneCodes;

// Scales held as raw binary16 bits in the low half of a 32-bit register (as
// the 16-bit loads deliver them): a _Float16 field lets the compiler pack two
// lanes' scales into one register, and the packing then waits for both loads.
template <> struct LaneCodes<Q4_0> {
    u32x4 c;
    uint32_t d;
};
template <> struct LaneCodes<MLX4_G64> {
    u32x4 c;
    uint32_t sb;   // fp16 scale (low half) and fp16 bias (high half)
};
template <> struct LaneCodes<MLX4_G32> {
    u32x4 c;
    uint32_t sb;   // the lane's own group (2t + g): fp16 scale low, fp16 bias high
};
template <> struct LaneCodes<Q2_0> {
    u32x2 c;
    uint32_t d;
};
template <> struct LaneCodes<Q8_0> {
    u32x4 lo, hi;    // dwords 0..3 (sub-steps 0, 1) and 4..7 (sub-steps 2, 3)
    uint32_t d;
};
template <> struct LaneCodes<Q4_K> {
    u32x4 c;
    uint32_t scm;              // the lane's sub-block: sc | m << 8 (low 16 bits)
    uint32_t dd;               // the super-block: fp16 d (low half), fp16 dmin (high half)
    float k0, k1;              // from prepare_lane: d sc 2^24 and d sc 2^20, exact in fp32
    float nm;                  // from prepare_lane: -dmin * m, exact in fp32
};

template <> struct LaneCodes<TERNARY> {
    uint32_t a;                // bytes E0 O0 E1 O1
    uint32_t b;                // bytes E2 O2 (low 16 bits)
    uint32_t tl;               // the tail byte shared with the neighbouring lane (low 8 bits)
    uint32_t d;
    uint32_t r0, r1, r2, r3;   // from prepare_lane: (E_b, O_b) one byte per 16-bit half; tail twice
    uint32_t m3;               // from prepare_lane: 16-bit digit multipliers of the lane's two tail digits
};

// Per-k-step values a lane derives once from its codes and scale record
// before the unpack (Q4_K and ternary).
template <int CODEC> __device__ __forceinline__ void prepare_lane(LaneCodes<CODEC> &lc)
{
    if constexpr (CODEC == TERNARY) {
        // v_perm_b32: selector byte k picks the destination byte k (0x0C: zero)
        lc.r0 = __builtin_amdgcn_perm(lc.a, lc.a, 0x0C010C00u);
        lc.r1 = __builtin_amdgcn_perm(lc.a, lc.a, 0x0C030C02u);
        lc.r2 = __builtin_amdgcn_perm(lc.b, lc.b, 0x0C010C00u);
        lc.r3 = __builtin_amdgcn_perm(lc.tl, lc.tl, 0x0C000C00u);
        lc.m3 = (__lane_id() & 1) ? (9u | (27u << 16)) : (1u | (3u << 16));   // digits 2, 3 or 0, 1
    }
    if constexpr (CODEC == Q4_K) {
        // d (11 significant bits) times sc (0..63) fits fp32's 24 exactly, and
        // so does every power-of-two scaling of it within range (at most
        // 65504 * 63 * 2^24 < 2^47)
        const float dsc = float(as_f16x2(lc.dd)[0]) * float(lc.scm & 0xFFu);
        lc.k0 = dsc * 16777216.0f;    // 2^24
        lc.k1 = dsc * 1048576.0f;     // 2^20
        lc.nm = -(float(as_f16x2(lc.dd)[1]) * float((lc.scm >> 8) & 0xFFu));
    }
}

// fp16 pair (k * v.lo + nm, k * v.hi + nm) for the fp16 pair v.  Written as
// fp16 -> fp32 widening, an fp32 FMA and a narrowing to fp16, which the
// compiler selects as v_fma_mixlo_f16 / v_fma_mixhi_f16; on gfx950 those take
// the fp16 operand (subnormals included) and the fp32 multiplier and addend as
// they are and round only the fp16 result.  With v = q 2^-24 (or q 2^-20) and
// k = d sc 2^24 (or 2^20) the product is d sc q exactly, so each weight is the
// correctly rounded value of the exact d sc q - dmin m.  (Plain C rather than
// inline assembly, so that the compiler sees the instructions and keeps its
// wait states against matrix instructions still reading the registers they
// overwrite.)
__device__ __forceinline__ uint32_t mix_pair(float k, uint32_t v, float nm)
{
    const f16x2 q = as_f16x2(v);
    const f16x2 r = {_Float16(__builtin_fmaf(k, float(q[0]), nm)), _Float16(__builtin_fmaf(k, float(q[1]), nm))};
    return as_u32(r);
}

template <int CODEC> struct CodeZero;
template <> struct CodeZero<Q4_0> { static constexpr int v = 8; };
template <> struct CodeZero<MLX4_G64> { static constexpr int v = 0; };
template <> struct CodeZero<MLX4_G32> { static constexpr int v = 0; };
template <> struct CodeZero<Q2_0> { static constexpr int v = 1; };
template <> struct CodeZero<Q8_0> { static constexpr int v = 128; };   // codes are stored as q + 128
template <> struct CodeZero<Q4_K> { static constexpr int v = 0; };
template <> struct CodeZero<TERNARY> { static constexpr int v = 1; };    // digit t = q + 1

// Base-3 digits of fixed-point bytes, one byte per 16-bit half of r, returned
// bare (t in 0..2 per half).  Digit i of byte B is ((B 3^i) mod 256) 3 >> 8,
// the carry out of the fractional byte of B 3^i times 3; with
// X_j = floor(B 3^j / 256) that is X_(i+1) - 3 X_i, because B 3^(i+1) =
// 3 (256 X_i + (B 3^i mod 256)).  So a digit costs one multiply and one shift
// for X_(i+1) and one multiply-add, and the next digit of the same byte reuses
// X_(i+1).  B <= 242 keeps B 3^5 below 2^16.  mul = 3^i in both halves (or the
// lane's tail multipliers); digit 0 (mul = 1) has X_0 = 0.
__device__ __forceinline__ uint32_t ternary_digits(uint32_t r, uint32_t mul, bool first)
{
    const u16x2 b = __builtin_bit_cast(u16x2, r), m = __builtin_bit_cast(u16x2, mul);
    const u16x2 three = {3, 3}, eight = {8, 8};
    const u16x2 x1 = (b * (m * three)) >> eight;
    if (first)
        return __builtin_bit_cast(uint32_t, x1);
    const u16x2 x0 = (b * m) >> eight;
    return __builtin_bit_cast(uint32_t, x1 - x0 * three);
}

// (2^E + q_even, 2^E + q_odd) -> exact fp16 (q_even - z, q_odd - z)
template <int CODEC, int E>
__device__ __forceinline__ f16x2 factor(uint32_t bits)
{
    constexpr _Float16 off = _Float16(float((1 << E) + CodeZero<CODEC>::v));
    const f16x2 o = {off, off};
    return as_f16x2(bits) - o;
}

// The 8 fp16 weights of sub-step s in MFMA operand order (element e = k offset
// 8 s + e inside the lane's 32-weight slice).  Pair p = elements (2p, 2p+1).
template <int CODEC>
__device__ __forceinline__ f16x8 unpack_substep(const LaneCodes<CODEC> &lc, int s, const Magics &mg)
{
    f16x2 q[4];
    if constexpr (CODEC == TERNARY) {
        // pairs p = 4 s .. 4 s + 3: digit p % 5 of (E, O)[p / 5]; p = 15: the tail
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = 4 * s + u;
            const uint32_t r = p < 5 ? lc.r0 : p < 10 ? lc.r1 : p < 15 ? lc.r2 : lc.r3;
            const uint32_t pw = p % 5 == 0 ? 1u : p % 5 == 1 ? 3u : p % 5 == 2 ? 9u : p % 5 == 3 ? 27u : 81u;
            const uint32_t mul = p == 15 ? lc.m3 : pw | (pw << 16);
            q[u] = factor<CODEC, 10>(ternary_digits(r, mul, p != 15 && p % 5 == 0) | 0x64006400u);
        }
    } else if constexpr (CODEC == Q4_K) {
        // a field left in place under a zero exponent reads as the fp16
        // subnormal q 2^-24 (bits 0..3 of a half) or q 2^-20 (bits 4..7);
        // one mix FMA per weight then scales, offsets and rounds once
        const uint32_t w = lc.c[s], w8 = w >> 8;
        const u32x4 r = {mix_pair(lc.k0, w & 0x000F000Fu, lc.nm), mix_pair(lc.k1, w & 0x00F000F0u, lc.nm),
                         mix_pair(lc.k0, w8 & 0x000F000Fu, lc.nm), mix_pair(lc.k1, w8 & 0x00F000F0u, lc.nm)};
        return __builtin_bit_cast(f16x8, r);
    } else if constexpr (CODEC == Q8_0) {
        // sub-step s: dwords 2s (elements 0..3) and 2s + 1 (4..7), bytes at
        // bits 0, 16 (pair 0 / 2) and 8, 24 (pair 1 / 3 after one shift)
        const u32x4 h = (s < 2) ? lc.lo : lc.hi;
        const uint32_t a = h[2 * (s & 1)], b = h[2 * (s & 1) + 1];
        q[0] = factor<CODEC, 10>((a & 0x00FF00FFu) | mg.m1024);
        q[1] = factor<CODEC, 10>(((a >> 8) & 0x00FF00FFu) | mg.m1024);
        q[2] = factor<CODEC, 10>((b & 0x00FF00FFu) | mg.m1024);
        q[3] = factor<CODEC, 10>(((b >> 8) & 0x00FF00FFu) | mg.m1024);
    } else if constexpr (CODEC == Q2_0) {
        // word s/2 holds sub-steps 2 (s/2) (fields at bits 0..7 of each half)
        // and 2 (s/2) + 1 (bits 8..15, brought down by one shift)
        const uint32_t src = (s & 1) ? (lc.c[s >> 1] >> 8) : lc.c[s >> 1];
        q[0] = factor<CODEC, 10>((src & 0x00030003u) | mg.m1024);
        q[1] = factor<CODEC, 8>((src & 0x000C000Cu) | mg.m256);
        q[2] = factor<CODEC, 6>((src & 0x00300030u) | mg.m64);
        q[3] = factor<CODEC, 4>((src & 0x00C000C0u) | mg.m16);
    } else {
        // pairs 0, 1 at bits 0..7 of each half, pairs 2, 3 at bits 8..15
        const uint32_t w = lc.c[s], w8 = w >> 8;
        q[0] = factor<CODEC, 10>((w & 0x000F000Fu) | mg.m1024);
        q[1] = factor<CODEC, 6>((w & 0x00F000F0u) | mg.m64);
        q[2] = factor<CODEC, 10>((w8 & 0x000F000Fu) | mg.m1024);
        q[3] = factor<CODEC, 6>((w8 & 0x00F000F0u) | mg.m64);
    }
    f16x8 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f16x2 w;
        if constexpr (CODEC == MLX4_G64 || CODEC == MLX4_G32) {
            const f16x2 sb = as_f16x2(lc.sb);
            const f16x2 sc = {sb[0], sb[0]};
            const f16x2 bi = {sb[1], sb[1]};
            w = __builtin_elementwise_fma(q[p], sc, bi);
        } else if constexpr (CODEC != Q4_K) {
            const _Float16 dh = __builtin_bit_cast(_Float16, (unsigned short)lc.d);
            const f16x2 dd = {dh, dh};
            w = q[p] * dd;
        }
        out[2 * p] = w[0];
        out[2 * p + 1] = w[1];
    }
    return out;
}

// Planar plane pointers of one weight matrix (host side).
struct Planes {
    const uint8_t *qs;
    const void *scales;
    uint32_t qs_bytes, scale_bytes;
};

// Raw buffer descriptor over [base, base + bytes).  Loads whose byte offset
// falls outside the range return zero, which is how every kernel masks the
// M, N and K tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), 0x00020000);
}

constexpr uint32_t OOB = 0x80000000u;   // an offset no plane reaches

struct PlaneRsrc {
    __amdgpu_buffer_rsrc_t qs, sc;
};

__device__ __forceinline__ PlaneRsrc plane_rsrc(const Planes &w)
{
    PlaneRsrc r;
    r.qs = make_rsrc(w.qs, w.qs_bytes);
    r.sc = make_rsrc(w.scales, w.scale_bytes);
    return r;
}

__device__ __forceinline__ _Float16 load_f16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(_Float16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}

// Per-lane vector offsets of one row group's chunks.  A row group past the
// end of the matrix gets out-of-range offsets, so its loads return zero
// codes with zero scales (weight 0).  Vector offsets are what the hardware
// range-checks, so the chunk-dependent part that goes in the scalar offset
// must itself stay inside the plane (callers keep 0 <= t < ksteps).
struct LaneOffsets {
    uint32_t q, s, s2;    // s2: Q4_K's super-block record
    uint32_t q2, q3;      // ternary: the B and T parts of the chunk
};

template <int CODEC>
__device__ __forceinline__ LaneOffsets lane_offsets(int rg, int groups, int lane)
{
    LaneOffsets o;
    const uint32_t i = uint32_t(lane & 31);
    o.s2 = OOB;
    o.q2 = OOB;
    o.q3 = OOB;
    if (rg >= groups) {
        o.q = OOB;
        o.s = OOB;
    } else if constexpr (CODEC == TERNARY) {
        o.q = uint32_t(lane) * 4;
        o.q2 = 256u + uint32_t(lane) * 2;
        o.q3 = 384u + uint32_t(lane >> 1);
        o.s = i * 2;
    } else if constexpr (CODEC == Q4_K) {
        o.q = uint32_t(lane) * 16;
        o.s = uint32_t(lane) * 2;
        o.s2 = 512u + i * 4;
    } else if constexpr (CODEC == Q2_0) {
        o.q = uint32_t(lane) * 8;
        o.s = i * 2;
    } else if constexpr (CODEC == Q4_0 || CODEC == Q8_0) {
        o.q = uint32_t(lane) * 16;
        o.s = uint32_t(lane) * 2;
    } else if constexpr (CODEC == MLX4_G32) {
        o.q = uint32_t(lane) * 16;
        o.s = uint32_t(lane) * 4;
    } else {
        o.q = uint32_t(lane) * 16;
        o.s = i * 4;
    }
    return o;
}

// memory instructions one load_lane issues
template <int CODEC> constexpr int lane_loads() { return CODEC == TERNARY ? 4 : (CODEC == Q8_0 || CODEC == Q4_K) ? 3 : 2; }

// Load the chunk (row group rg, k-step t) codes and scales a lane owns.
// `ksteps` = padded K / 64, `kb128` = K / 128 (Q2_0 scale plane pitch).
// rg and t are wave-uniform: the chunk part of each address is a scalar
// offset, the lane part a fixed vector offset.  STREAM marks the loads
// non-temporal, for data read exactly once.
template <int CODEC, bool STREAM = false>
__device__ __forceinline__ LaneCodes<CODEC> load_lane(const PlaneRsrc &w, LaneOffsets o, int rg, int t, int ksteps,
                                                      int kb128)
{
    constexpr int AUX = STREAM ? 2 : 0;   // cache policy bits: 2 = nt
    LaneCodes<CODEC> lc;
    const uint32_t chunk = uint32_t(rg) * uint32_t(ksteps) + uint32_t(t);
    if constexpr (CODEC == TERNARY) {
        const uint32_t base = chunk * uint32_t(TERNARY_CHUNK);
        lc.a = __builtin_amdgcn_raw_buffer_load_b32(w.qs, o.q, base, AUX);
        lc.b = __builtin_amdgcn_raw_buffer_load_b16(w.qs, o.q2, base, AUX);
        lc.tl = __builtin_amdgcn_raw_buffer_load_b8(w.qs, o.q3, base, AUX);
        lc.d = __builtin_amdgcn_raw_buffer_load_b16(w.sc, o.s, (uint32_t(rg) * uint32_t(ksteps >> 2) + uint32_t(t >> 2)) * 64u, 0);
    } else if constexpr (CODEC == Q8_0) {
        lc.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.qs, o.q, chunk * 2048, AUX));
        lc.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.qs, o.q, chunk * 2048 + 1024, AUX));
        lc.d = __builtin_amdgcn_raw_buffer_load_b16(w.sc, o.s, chunk * 128, 0);
    } else if constexpr (CODEC == Q4_K) {
        // record of (row group, super-block): u16 [4 k-steps][64 lanes], then u32 [32 rows]
        lc.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.qs, o.q, chunk * 1024, AUX));
        const uint32_t rec = (uint32_t(rg) * uint32_t(ksteps >> 2) + uint32_t(t >> 2)) * 640u;
        lc.scm = __builtin_amdgcn_raw_buffer_load_b16(w.sc, o.s, rec + uint32_t(t & 3) * 128u, AUX);
        lc.dd = __builtin_amdgcn_raw_buffer_load_b32(w.sc, o.s2, rec, AUX);
    } else if constexpr (CODEC == Q2_0) {
        lc.c = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(w.qs, o.q, chunk * 512, AUX));
        lc.d = __builtin_amdgcn_raw_buffer_load_b16(w.sc, o.s, (uint32_t(rg) * kb128 + uint32_t(t >> 1)) * 64, 0);
    } else {
        lc.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.qs, o.q, chunk * 1024, AUX));
        if constexpr (CODEC == Q4_0)
            lc.d = __builtin_amdgcn_raw_buffer_load_b16(w.sc, o.s, chunk * 128, 0);
        else if constexpr (CODEC == MLX4_G32)
            lc.sb = __builtin_amdgcn_raw_buffer_load_b32(w.sc, o.s, chunk * 256, AUX);
        else
            lc.sb = __builtin_amdgcn_raw_buffer_load_b32(w.sc, o.s, chunk * 128, AUX);
    }
    return lc;
}

}  // namespace qg
