// Attention over a Q8_0 KV cache (prefill), fused with the on-the-fly
// dequantization of K and V.
//
// Pages: comparison page section 2.3 and project index Brick 4 -- a
// FlashAttention core (online softmax, no round trip of the score matrix
// through memory) whose K and V come from a Q8_0-compressed cache and are
// dequantized as they are read; releases page v0.2.3, the attention core is
// templated on the head dimension D in {64, 128}; releases page v0.3.0,
// grouped-query attention and causal masking in the transformer block.
//
// One workgroup of four wave64 handles 128 queries of one head; each wave owns
// 32 of them for the whole key range.  Per tile of 64 keys:
//  * the 256 threads turn the next tile's int8 codes and fp16 block scales
//    into fp16 K [64][D] (row-major) and V^T [D][64] in the other half of a
//    double-buffered LDS area -- each element is the correctly rounded q * d,
//    the weights' Q8_0 rule; V is transposed in registers (8 keys x 4 d per
//    thread) so that it is stored with 16-byte writes.  The raw codes are
//    loaded one tile ahead of that, so one barrier per tile suffices;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (A = K rows, B = the wave's Q
//    fragments, loaded once).  K rows are read in the order pi below, which
//    makes each lane's 32 scores exactly the B fragments P^T needs for the
//    next product: no lane exchange between the two products;
//  * online softmax in fp32 on the log2 scale: the row maximum and sum are
//    lane-local over 32 scores plus one exchange with lane l ^ 32 (the other
//    half of the same query's keys); the O accumulators are rescaled by
//    2^(m_old - m_new);
//  * O^T += V^T P^T (A = V^T rows from LDS, B = P as fp16).
// The epilogue divides by the row sum and writes O [H, M, D] fp16.
// Causal work per query tile grows linearly; workgroups are ordered so that
// each heavy query tile is launched next to a light one (see tile_of).
#include "launch.h"

namespace qg {
namespace {

constexpr int AT_BQ = 128;   // queries per workgroup
constexpr int AT_BK = 64;    // keys per tile
constexpr int AT_NT = 256;   // threads per workgroup

struct AttnArgs {
    const _Float16 *q;
    _Float16 *o;
    const uint8_t *kq, *vq;     // int8 codes [kv_heads * s][D]
    const _Float16 *ks, *vs;    // fp16 scales [kv_heads * s][D / 32]
    int heads, m, kv_heads, s, causal, tiles_q;
    float scale_log2;           // softmax scale times log2(e)
};

// 16 int8 codes (two's complement) of one 32-element block half -> the fp16
// values q * d, in order.  XOR 0x80 turns q into q + 128 in 0..255; one
// v_perm_b32 puts two such bytes under the binary16 exponent byte 0x64 (taken
// from the constant word e64 = 0x64646464), which reads 1024 + q + 128;
// subtracting 1152 is exact, the multiply by d rounds once.
__device__ __forceinline__ void dequant16(u32x4 c, _Float16 d, uint32_t e64, u32x4 &lo, u32x4 &hi)
{
    const f16x2 dd = {d, d};
    const f16x2 off = {_Float16(1152.0f), _Float16(1152.0f)};
    uint32_t r[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x = c[w] ^ 0x80808080u;
        // selector bytes 0-3 pick bytes of x, 4-7 bytes of e64
        const uint32_t p01 = __builtin_amdgcn_perm(e64, x, 0x04010400u);
        const uint32_t p23 = __builtin_amdgcn_perm(e64, x, 0x04030402u);
        r[2 * w] = as_u32((as_f16x2(p01) - off) * dd);
        r[2 * w + 1] = as_u32((as_f16x2(p23) - off) * dd);
    }
    lo = u32x4{r[0], r[1], r[2], r[3]};
    hi = u32x4{r[4], r[5], r[6], r[7]};
}

// Four codes (d .. d + 3 of one key, two's complement) -> two fp16 pairs
// (d, d + 1), (d + 2, d + 3) of q * scale, in the rounding of dequant16.
__device__ __forceinline__ void dequant4(uint32_t c, _Float16 d, uint32_t e64, uint32_t &p01, uint32_t &p23)
{
    const f16x2 dd = {d, d};
    const f16x2 off = {_Float16(1152.0f), _Float16(1152.0f)};
    const uint32_t x = c ^ 0x80808080u;
    p01 = as_u32((as_f16x2(__builtin_amdgcn_perm(e64, x, 0x04010400u)) - off) * dd);
    p23 = as_u32((as_f16x2(__builtin_amdgcn_perm(e64, x, 0x04030402u)) - off) * dd);
}

// Query tile and head of workgroup `lin` (0 .. tiles_q * heads - 1).  The
// query heads [0, H/2) take their tiles longest (causal) first, the heads
// [H/2, H) shortest first, so that workgroups lin and lin + half -- dispatched
// to the same compute unit when all of them are resident -- carry
// tiles_q - 1 key-tile rows of work between them.  A bijection for any H.
__device__ __forceinline__ void tile_of(int lin, int tiles_q, int heads, int &qt, int &h)
{
    const int hh = heads / 2, half = hh * tiles_q;
    if (lin < half) {
        qt = tiles_q - 1 - lin % tiles_q;
        h = lin / tiles_q;
    } else {
        const int l2 = lin - half;
        qt = l2 % tiles_q;
        h = hh + l2 / tiles_q;
    }
}

// V^T row d keeps its chunk c (keys 8 c .. 8 c + 7) at chunk position
// c ^ vswz(d): the MFMA reads (16 rows, one chunk each) hit distinct banks and
// the 16-byte stores of consecutive threads (rows 4 apart) at most two-way.
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

// A-operand row r (0..31) of a 32-key block reads key pi(r): the MFMA puts
// row 8 q + 4 g + e of the product in register 4 q + e of lane half g, and
// pi(8 q + 4 g + e) = 16 (q >> 1) + 8 g + 4 (q & 1) + e hands lane half g the
// keys 16 k + 8 g + 0..7 in registers 8 (k & 1) .. 8 (k & 1) + 7 -- the
// B-operand layout of the 16-deep sub-step k of the P V product.
__device__ __forceinline__ int pi_row(int r)
{
    const int q = r >> 3, g = (r >> 2) & 1, e = r & 3;
    return 16 * (q >> 1) + 8 * g + 4 * (q & 1) + e;
}

template <int D>
__global__ __launch_bounds__(AT_NT, 2) void attn_q8kv_kernel(AttnArgs a)
{
    constexpr int KP = D + 8;              // K tile row pitch (halves); the pad staggers LDS banks
    constexpr int VP = AT_BK;              // V^T tile row pitch (halves): 8 chunks of 8 keys, swizzled
    constexpr int NDB = D / 32;            // 32-row blocks of O^T
    constexpr int NDD = D / 16;            // 16-deep steps over d
    constexpr int CPR = D / 16;            // 16-code chunks per key (K)
    constexpr int IPT = AT_BK * CPR / AT_NT;   // K chunks per thread
    constexpr int VITEMS = AT_BK * D / 32;           // V items of 8 keys x 4 d per tile
    constexpr int VIT = (VITEMS + AT_NT - 1) / AT_NT;   // per thread (D = 64: half the threads)
    constexpr int VDG = D / 4;             // 4-wide d groups per key
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(IPT >= 1 && AT_BK * CPR % AT_NT == 0 && VITEMS % 64 == 0, "tile");

    __shared__ __attribute__((aligned(16))) _Float16 ks[2][AT_BK * KP];
    __shared__ __attribute__((aligned(16))) _Float16 vt[2][D * VP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 31, g = lane >> 5;
    int qt, h;
    tile_of(int(blockIdx.x), a.tiles_q, a.heads, qt, h);
    const int q0 = qt * AT_BQ;
    const int kvh = h / (a.heads / a.kv_heads);
    const int off = a.s - a.m;                        // the queries are the last m positions
    const int qrow = q0 + 32 * wave + i;

    // Q fragments (B operand): lane (i, g) holds Q[qrow][16 dd + 8 g .. + 7]
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + int64_t(h) * a.m * D, uint32_t(a.m) * D * 2u);
    f16x8 qf[NDD];
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) {
        const uint32_t v = qrow < a.m ? (uint32_t(qrow) * D + uint32_t(16 * dd + 8 * g)) * 2u : OOB;
        qf[dd] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, v, 0, 0));
    }

    int t_end = (a.s + AT_BK - 1) / AT_BK;
    if (a.causal)
        t_end = min(t_end, (off + q0 + AT_BQ - 1) / AT_BK + 1);

    // raw codes and scales of one tile, AT_BK * CPR chunks per matrix:
    // chunk j = key j / CPR, 16 codes from d = 16 (j % CPR)
    // descriptors over this KV head's s rows: a vector offset at or past s
    // rows reads as zero
    const int64_t head_row = int64_t(kvh) * a.s;
    const __amdgpu_buffer_rsrc_t kqr = make_rsrc(a.kq + head_row * D, uint32_t(a.s) * D);
    const __amdgpu_buffer_rsrc_t vqr = make_rsrc(a.vq + head_row * D, uint32_t(a.s) * D);
    const __amdgpu_buffer_rsrc_t ksr = make_rsrc(a.ks + head_row * (D / 32), uint32_t(a.s) * (D / 32) * 2u);
    const __amdgpu_buffer_rsrc_t vsr = make_rsrc(a.vs + head_row * (D / 32), uint32_t(a.s) * (D / 32) * 2u);
    // K item j: key j / CPR, codes 16 (j % CPR) .. + 15.  V item j: keys
    // 8 (j / VDG) .. + 7, codes 4 (j % VDG) .. + 3 of each.
    u32x4 kc[IPT];
    _Float16 kd[IPT];
    uint32_t vc[VIT][8];
    _Float16 vd[VIT][8];
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int j = tid + AT_NT * u, kk = j / CPR, c = j % CPR;
            const uint32_t key = uint32_t(t * AT_BK + kk);
            const bool in = key < uint32_t(a.s);
            kc[u] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(kqr, in ? key * D + uint32_t(16 * c) : OOB, 0, 0));
            kd[u] = load_f16(ksr, in ? (key * (D / 32) + uint32_t(c >> 1)) * 2u : OOB, 0);
        }
#pragma unroll
        for (int u = 0; u < VIT; ++u) {
            const int j = tid + AT_NT * u, k8 = j / VDG, c4 = j % VDG;
            if (j >= VITEMS)
                break;
            // keys 8 k8 .. + 7 are D (codes) and D / 16 (scale bytes) apart:
            // inside the sequence one vector offset serves all eight (the key
            // goes into the instruction offset); the tile that crosses s puts
            // each key past it out of range by its vector offset
            const uint32_t key0 = uint32_t(t * AT_BK + 8 * k8);
            const uint32_t cv = key0 * D + uint32_t(4 * c4);
            const uint32_t sv = (key0 * (D / 32) + uint32_t(c4 >> 3)) * 2u;
            if (t * AT_BK + AT_BK <= a.s) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    vc[u][e] = __builtin_amdgcn_raw_buffer_load_b32(vqr, cv + uint32_t(e * D), 0, 0);
                    vd[u][e] = load_f16(vsr, sv + uint32_t(e * (D / 16)), 0);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool in = key0 + uint32_t(e) < uint32_t(a.s);
                    vc[u][e] = __builtin_amdgcn_raw_buffer_load_b32(vqr, in ? cv + uint32_t(e * D) : OOB, 0, 0);
                    vd[u][e] = load_f16(vsr, in ? sv + uint32_t(e * (D / 16)) : OOB, 0);
                }
            }
        }
    };
    const uint32_t e64 = 0x64646464u;
    // dequantize the fetched tile into LDS buffer b
    auto stage = [&](int b) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int j = tid + AT_NT * u, kk = j / CPR, c = j % CPR;
            u32x4 lo, hi;
            dequant16(kc[u], kd[u], e64, lo, hi);
            *reinterpret_cast<u32x4 *>(&ks[b][kk * KP + 16 * c]) = lo;
            *reinterpret_cast<u32x4 *>(&ks[b][kk * KP + 16 * c + 8]) = hi;
        }
#pragma unroll
        for (int u = 0; u < VIT; ++u) {
            const int j = tid + AT_NT * u, k8 = j / VDG, c4 = j % VDG;
            if (j >= VITEMS)
                break;
            uint32_t p01[8], p23[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dequant4(vc[u][e], vd[u][e], e64, p01[e], p23[e]);
            // row d = 4 c4 + r of V^T gets keys 8 k8 .. + 7: the low (r even)
            // or high (r odd) halves of keys e, e + 1 paired by v_perm_b32
            u32x4 rows[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rows[0][e] = __builtin_amdgcn_perm(p01[2 * e + 1], p01[2 * e], 0x05040100u);
                rows[1][e] = __builtin_amdgcn_perm(p01[2 * e + 1], p01[2 * e], 0x07060302u);
                rows[2][e] = __builtin_amdgcn_perm(p23[2 * e + 1], p23[2 * e], 0x05040100u);
                rows[3][e] = __builtin_amdgcn_perm(p23[2 * e + 1], p23[2 * e], 0x07060302u);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 4 * c4 + r;
                *reinterpret_cast<u32x4 *>(&vt[b][d * VP + 8 * (k8 ^ vswz(d))]) = rows[r];
            }
        }
    };
    fetch(0);
    stage(0);
    if (t_end > 1)
        fetch(1);
    __syncthreads();

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[db][e] = 0.0f;
    float mrow = -__builtin_inff(), lrow = 0.0f;   // running maximum (log2 scale) and sum
    const int qpos = off + qrow;

    // K rows this lane reads for the A operand, and the LDS offsets
    const int krow0 = pi_row(i), krow1 = 32 + pi_row(i);

    for (int t = 0; t < t_end; ++t) {
        const int b = t & 1;
        // the tile after this one goes into the other buffer: its last
        // readers finished before the barrier that ended the previous step
        if (t + 1 < t_end) {
            stage(b ^ 1);
            if (t + 2 < t_end)
                fetch(t + 2);
        }

        // S^T for keys 32 kb .. 32 kb + 31 of the tile
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = 0.0f;
            const _Float16 *kp = &ks[b][(kb ? krow1 : krow0) * KP + 8 * g];
#pragma unroll
            for (int dd = 0; dd < NDD; ++dd) {
                const f16x8 ka = *reinterpret_cast<const f16x8 *>(kp + 16 * dd);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[dd], sacc[kb], 0, 0, 0);
            }
        }

        // scores on the log2 scale; keys past the sequence or (causal) past
        // the query's own position are -inf.  Register 4 q + e of block kb
        // holds key 32 kb + 16 (q >> 1) + 8 g + 4 (q & 1) + e of the tile.
        const int kbase = t * AT_BK;
        const bool edge = kbase + AT_BK > a.s || (a.causal && kbase + AT_BK - 1 > off + q0 + 32 * wave);
        // (the maximum is taken on the raw scores: the scale is positive)
        float tmax = -__builtin_inff();
        if (edge) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = r >> 2, e = r & 3;
                    const int key = kbase + 32 * kb + 16 * (q >> 1) + 8 * g + 4 * (q & 1) + e;
                    if (key >= a.s || (a.causal && key > qpos))
                        sacc[kb][r] = -__builtin_inff();
                }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                tmax = __builtin_fmaxf(tmax, sacc[kb][r]);
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32)) * a.scale_log2;
        const float mnew = __builtin_fmaxf(mrow, tmax);
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], a.scale_log2, -mnew));
                sacc[kb][r] = p;
                lsum += p;
            }
        lsum += __shfl_xor(lsum, 32);
        if (__builtin_amdgcn_ballot_w64(mnew != mrow) != 0) {   // some row's maximum moved: rescale
            const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[db][e] *= alpha;
        }
        lrow += lsum;
        mrow = mnew;

        // P as fp16 B fragments: sub-step k takes registers 8 (k & 1) .. + 7 of block k >> 1
        f16x8 pf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pf[k][e] = _Float16(sacc[k >> 1][8 * (k & 1) + e]);

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int d = 32 * db + i;
            const _Float16 *vp = &vt[b][d * VP];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f16x8 va = *reinterpret_cast<const f16x8 *>(vp + 8 * ((2 * k + g) ^ vswz(d)));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[k], oacc[db], 0, 0, 0);
            }
        }
        __syncthreads();   // tile t's buffer is free; tile t + 1's is written
    }

    // O[h][qrow][32 db + 8 q + 4 g + e] = O^T acc / row sum
    if (qrow < a.m) {
        const float inv = 1.0f / lrow;
        _Float16 *orow = a.o + (int64_t(h) * a.m + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f16x2 lo2 = {_Float16(oacc[db][4 * q] * inv), _Float16(oacc[db][4 * q + 1] * inv)};
                const f16x2 hi2 = {_Float16(oacc[db][4 * q + 2] * inv), _Float16(oacc[db][4 * q + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * q + 4 * g) = u32x2{as_u32(lo2), as_u32(hi2)};
            }
    }
}

}  // namespace

hipError_t launch_attention(const AttnProblem &p, hipStream_t stream)
{
    AttnArgs a;
    a.q = p.q;
    a.o = p.o;
    a.kq = p.k_codes;
    a.vq = p.v_codes;
    a.ks = p.k_scales;
    a.vs = p.v_scales;
    a.heads = int(p.heads);
    a.m = int(p.m);
    a.kv_heads = int(p.kv_heads);
    a.s = int(p.s);
    a.causal = p.causal ? 1 : 0;
    a.tiles_q = int(ceil_div(p.m, AT_BQ));
    a.scale_log2 = p.scale * 1.4426950408889634f;
    void *args[] = {&a};
    const dim3 grid(unsigned(a.tiles_q * a.heads)), block(AT_NT);
    const void *fn = p.head_dim == 64 ? reinterpret_cast<const void *>(&attn_q8kv_kernel<64>)
                                      : reinterpret_cast<const void *>(&attn_q8kv_kernel<128>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace qg
