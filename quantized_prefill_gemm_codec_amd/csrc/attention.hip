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
// One workgroup of eight wave64 handles 128 queries of one head.  Its waves
// form two groups of four that take the two halves of the query tile's key
// range at the same time; in each group, wave w owns queries 32 w .. 32 w + 31
// for its half.  Per tile of 64 keys and group:
//  * the group's 256 threads turn the next tile's codes and fp16 block scales
//    into fp16 K [64][D] and V [64][D] (both row-major) in the other half of
//    the group's double-buffered LDS area -- each element is the correctly
//    rounded q * d, the weights' Q8_0 rule.  The raw codes are loaded one tile
//    ahead of that, so one barrier per tile suffices;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (A = K rows, B = the wave's Q
//    fragments, loaded once).  K rows are read in the order pi below, which
//    makes each lane's 32 scores exactly the B fragments P^T needs for the
//    next product: no lane exchange between the two products;
//  * online softmax in fp32 on the log2 scale: each lane holds 32 scores of
//    its query, and lane l ^ 32 the other half of that query's keys.  The
//    halves exchange maxima only in a step where the running maximum moves,
//    and keep their own row sums (over P as rounded to fp16 for the product,
//    so that numerator and denominator use the same P), added once at the
//    end.  The running maximum, and with it the
//    O accumulators (by 2^(m_old - m_new)), moves only when a tile's maximum
//    exceeds it by more than RESCALE_SLACK;
//  * O^T += V^T P^T (A = V^T, read out of the row-major V tile by the LDS
//    transpose load, B = P as fp16).
// At the end the second group hands its (maximum, sum, O^T) to the first
// through LDS, which merges the two halves (each rescaled to the common
// maximum), divides by the row sum and writes O [H, M, D] fp16.
// Why two groups: one wave's per-tile chain (dequantize, QK^T, softmax, PV)
// is a serial dependency of about 2 us that another workgroup on the same
// compute unit barely slows, so the kernel took as long as the longest key
// range -- the last query tile's 32 tiles.  Splitting every range in two
// halves that chain.  Workgroups are ordered heaviest (causal) first.
#include "launch.h"

namespace qg {
namespace {

constexpr int AT_BQ = 128;   // queries per workgroup
constexpr int AT_BK = 64;    // keys per tile
constexpr int AT_GT = 256;   // threads per key-range group (one tile's dequantization)
constexpr int AT_NG = 2;     // key-range groups per workgroup
constexpr int AT_NT = AT_GT * AT_NG;   // threads per workgroup
constexpr float RESCALE_SLACK = 8.0f;   // log2 units a row maximum may rise before the O accumulators are rescaled

struct AttnArgs {
    const _Float16 *q;
    _Float16 *o;
    const uint8_t *kq, *vq;     // int8 codes [kv_heads * s][D]
    const _Float16 *ks, *vs;    // fp16 scales [kv_heads * s][D / 32]
    int heads, m, kv_heads, s, causal, tiles_q;
    float scale_log2;           // softmax scale times log2(e)
};

// 16 codes (stored as q + 128 in 0..255) of one 32-element block half -> the
// fp16 values q * d, in order.  One v_perm_b32 puts two code bytes under the
// binary16 exponent byte 0x64 (taken from the constant word e64 = 0x64646464),
// which reads 1024 + q + 128; subtracting 1152 is exact, the multiply by d
// rounds once.
__device__ __forceinline__ void dequant16(u32x4 c, _Float16 d, uint32_t e64, u32x4 &lo, u32x4 &hi)
{
    const f16x2 dd = {d, d};
    const f16x2 off = {_Float16(1152.0f), _Float16(1152.0f)};
    uint32_t r[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x = c[w];
        // selector bytes 0-3 pick bytes of x, 4-7 bytes of e64
        const uint32_t p01 = __builtin_amdgcn_perm(e64, x, 0x04010400u);
        const uint32_t p23 = __builtin_amdgcn_perm(e64, x, 0x04030402u);
        r[2 * w] = as_u32((as_f16x2(p01) - off) * dd);
        r[2 * w + 1] = as_u32((as_f16x2(p23) - off) * dd);
    }
    lo = u32x4{r[0], r[1], r[2], r[3]};
    hi = u32x4{r[4], r[5], r[6], r[7]};
}

// One fp16 scale, zero-extended into a 32-bit register.  Scales of the
// prefetched tile stay in registers of their own until the tile is staged:
// combining two of them into one register as they arrive would make the wave
// wait for the whole prefetch at once.
__device__ __forceinline__ uint16_t load_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

__device__ __forceinline__ _Float16 f16_of(uint16_t x) { return __builtin_bit_cast(_Float16, x); }

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS transpose load (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// 4 a + c receives element c of the four halves addressed by lanes a, a + 4,
// a + 8 and a + 12 of the group, in that order.
__device__ __forceinline__ f16x4 lds_read_tr16(const _Float16 *p)
{
    return __builtin_bit_cast(
        f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p)));
}

// Query tile and head of workgroup `lin` (0 .. tiles_q * heads - 1): causal
// query tiles in decreasing order of their key range (all heads of the last
// tile first), so that the workgroups dispatched as others finish are the
// short ones; the heads of one tile are adjacent, and every group of
// heads / kv_heads of them reads the same KV head.
__device__ __forceinline__ void tile_of(int lin, int tiles_q, int heads, bool causal, int &qt, int &h)
{
    const int r = lin / heads;
    qt = causal ? tiles_q - 1 - r : r;
    h = lin - r * heads;
}

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
__global__ __launch_bounds__(AT_NT, 1) void attn_q8kv_kernel(AttnArgs a)
{
    constexpr int KP = D + 8;              // K tile row pitch (halves); the pad staggers LDS banks
    constexpr int VP = D + 16;             // V tile row pitch (halves): 4 rows of a transpose load hit distinct banks
    constexpr int NDB = D / 32;            // 32-row blocks of O^T
    constexpr int NDD = D / 16;            // 16-deep steps over d
    constexpr int CPR = D / 16;            // 16-code chunks per key (K)
    constexpr int IPT = AT_BK * CPR / AT_GT;   // K chunks per thread of a group
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(IPT >= 1 && AT_BK * CPR % AT_GT == 0, "tile");
    constexpr int KT = AT_BK * KP, VT = AT_BK * VP;   // halves of one K tile and one V tile
    // the merge area (second group's O^T, maximum and sum) reuses the tiles
    static_assert(4 * (D / 32) * 4 * 64 * 16 + 2 * 4 * 64 * 4 <= AT_NG * 2 * (KT + VT) * 2, "merge area");

    // per group: K tiles [2][KT], then V tiles [2][VT]
    __shared__ __attribute__((aligned(16))) _Float16 tiles[AT_NG][2 * (KT + VT)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, qw = wave & 3;         // key-range group, query sub-tile
    const int gtid = tid & (AT_GT - 1);
    const int i = lane & 31, g = lane >> 5;
    // The SIMD's arbiter favours the older wave of a pair, so without this the
    // second group (waves 4..7, one per SIMD beside a first-group wave) ran
    // behind every step and the first waited for it at the barrier; issue
    // priority for the second group balances the pairs.
    if (grp == 1)
        __builtin_amdgcn_s_setprio(3);
    _Float16 *const ksb = &tiles[grp][0];
    _Float16 *const vtb = &tiles[grp][2 * KT];
    int qt, h;
    tile_of(int(blockIdx.x), a.tiles_q, a.heads, a.causal != 0, qt, h);
    const int q0 = qt * AT_BQ;
    const int kvh = h / (a.heads / a.kv_heads);
    const int off = a.s - a.m;                        // the queries are the last m positions
    const int qrow = q0 + 32 * qw + i;

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
    // the two halves of the key range: group 0 takes tiles [0, th), group 1
    // [th, t_end) -- one fewer when t_end is odd
    const int th = (t_end + 1) >> 1;
    const int tb = grp ? th : 0, tn = grp ? t_end - th : th;

    // raw codes and scales of one tile, AT_BK * CPR chunks per matrix:
    // chunk j = key j / CPR, 16 codes from d = 16 (j % CPR)
    // descriptors over this KV head's s rows: a vector offset at or past s
    // rows reads as zero
    const int64_t head_row = int64_t(kvh) * a.s;
    const __amdgpu_buffer_rsrc_t kqr = make_rsrc(a.kq + head_row * D, uint32_t(a.s) * D);
    const __amdgpu_buffer_rsrc_t vqr = make_rsrc(a.vq + head_row * D, uint32_t(a.s) * D);
    const __amdgpu_buffer_rsrc_t ksr = make_rsrc(a.ks + head_row * (D / 32), uint32_t(a.s) * (D / 32) * 2u);
    const __amdgpu_buffer_rsrc_t vsr = make_rsrc(a.vs + head_row * (D / 32), uint32_t(a.s) * (D / 32) * 2u);
    // item j of either matrix: key j / CPR, codes 16 (j % CPR) .. + 15, and
    // the scale of their 32-element block
    u32x4 kc[IPT], vc[IPT];
    uint16_t kd[IPT], vd[IPT];
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int j = gtid + AT_GT * u, kk = j / CPR, c = j % CPR;
            const uint32_t key = uint32_t(t * AT_BK + kk);
            const bool in = key < uint32_t(a.s);
            const uint32_t co = in ? key * D + uint32_t(16 * c) : OOB;
            const uint32_t so = in ? (key * (D / 32) + uint32_t(c >> 1)) * 2u : OOB;
            kc[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kqr, co, 0, 0));
            kd[u] = load_u16(ksr, so);
            vc[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vqr, co, 0, 0));
            vd[u] = load_u16(vsr, so);
        }
    };
    const uint32_t e64 = 0x64646464u;
    // dequantize the fetched tile into LDS buffer b
    auto stage = [&](int b) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int j = gtid + AT_GT * u, kk = j / CPR, c = j % CPR;
            u32x4 lo, hi;
            dequant16(kc[u], f16_of(kd[u]), e64, lo, hi);
            *reinterpret_cast<u32x4 *>(&ksb[b * KT + kk * KP + 16 * c]) = lo;
            *reinterpret_cast<u32x4 *>(&ksb[b * KT + kk * KP + 16 * c + 8]) = hi;
            dequant16(vc[u], f16_of(vd[u]), e64, lo, hi);
            *reinterpret_cast<u32x4 *>(&vtb[b * VT + kk * VP + 16 * c]) = lo;
            *reinterpret_cast<u32x4 *>(&vtb[b * VT + kk * VP + 16 * c + 8]) = hi;
        }
    };
    if (tn > 0) {
        fetch(tb);
        stage(0);
    }
    // Every load so far, the Q fragments included, is in before the loop
    // starts (after stage(0) this waits for nothing).  Without it the
    // compiler cannot tell on every path that the Q fragments have landed,
    // and makes each step's first MFMAs wait for the prefetch issued just
    // before them.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (tn > 1)
        fetch(tb + 1);
    __syncthreads();

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[db][e] = 0.0f;
    float mrow = -__builtin_inff(), lrow = 0.0f;   // running maximum (log2 scale) and sum
    const int qpos = off + qrow;

    // K rows this lane reads for the A operand
    const int krow0 = pi_row(i), krow1 = 32 + pi_row(i);
    // the V element this lane addresses in a transpose load: within each 16
    // lanes, lane 4 r + c (r, c < 4) names row r, columns 4 c .. 4 c + 3 of a
    // 4 x 16 block (rows 8 g .., columns 16 ((lane >> 4) & 1) ..), and gets
    // back column lane & 15 of the block's four rows
    const int vsrc = (8 * g + ((lane >> 2) & 3)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // both groups step together (one barrier per step); a group whose half
    // is one tile shorter idles through the last step
    for (int it = 0; it < th; ++it) {
      if (it < tn) {
        const int t = tb + it;
        const int b = it & 1;
        // the tile after this one goes into the other buffer: its last
        // readers finished before the barrier that ended the previous step
        auto stage_next = [&]() {
            if (it + 1 < tn) {
                stage(b ^ 1);
                if (it + 2 < tn)
                    fetch(t + 2);
            }
        };
        if constexpr (D != 64)
            stage_next();

        // S^T for keys 32 kb .. 32 kb + 31 of the tile
        f32x16 sacc[2];
        f16x8 ka[2][NDD];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const _Float16 *kp = &ksb[b * KT + (kb ? krow1 : krow0) * KP + 8 * g];
#pragma unroll
            for (int dd = 0; dd < NDD; ++dd)
                ka[kb][dd] = *reinterpret_cast<const f16x8 *>(kp + 16 * dd);
        }
        if constexpr (D == 64) {
            // at D = 64 the next tile is staged after this tile's K-fragment
            // reads are issued, so that they do not queue behind the tile
            // writes (at D = 128 that measured slower: the MFMAs then wait
            // for the staging VALU)
            __builtin_amdgcn_sched_barrier(0);
            stage_next();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = 0.0f;
        }
        // all K-fragment reads issued first, then the MFMAs, both blocks interleaved
#pragma unroll
        for (int dd = 0; dd < NDD; ++dd)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[kb][dd], qf[dd], sacc[kb], 0, 0, 0);
        // keep every K-fragment read ahead of the MFMAs (the scheduler would
        // otherwise keep two in flight)
        if constexpr (D != 64) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDD, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * NDD, 0);
        }

        // scores on the log2 scale; keys past the sequence or (causal) past
        // the query's own position are -inf.  Register 4 q + e of block kb
        // holds key 32 kb + 16 (q >> 1) + 8 g + 4 (q & 1) + e of the tile.
        const int kbase = t * AT_BK;
        const bool edge = kbase + AT_BK > a.s || (a.causal && kbase + AT_BK - 1 > off + q0 + 32 * qw);
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
        {
            // four independent chains: a short dependency path to the maximum
            float mx[4] = {tmax, tmax, tmax, tmax};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx[r & 3] = __builtin_fmaxf(mx[r & 3], sacc[kb][r]);
            tmax = __builtin_fmaxf(__builtin_fmaxf(mx[0], mx[1]), __builtin_fmaxf(mx[2], mx[3]));
        }
        tmax *= a.scale_log2;
        // The running maximum moves only when a score exceeds it by more than
        // 2^RESCALE_SLACK on the exp2 scale: until then P = 2^(s - m) stays at
        // most 2^8 (exact range for fp16 P, and the fp32 sums and accumulators
        // are unaffected), and the O accumulators need no rescale -- after the
        // first tiles the maximum rarely moves that far.  Each lane half sees
        // half of a row's keys: only when some lane's half-row maximum moves
        // does the wave exchange the halves' maxima (lane l ^ 32), so that
        // both halves of a row take the same new maximum; otherwise no lane
        // exchange happens in the step.
        bool moved = tmax > mrow + RESCALE_SLACK;
        float mnew = mrow;
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {
            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
            moved = tmax > mrow + RESCALE_SLACK;
            mnew = moved ? tmax : mrow;
        }
        // a row with no visible key yet (a whole half-range can be masked
        // for the first queries) keeps maximum -inf: its P must be 0, not
        // exp2(-inf + inf)
        const float msub = mnew == -__builtin_inff() ? 0.0f : mnew;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sacc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], a.scale_log2, -msub));
        // P as fp16 B fragments: sub-step k takes registers 8 (k & 1) .. + 7 of block k >> 1
        f16x8 pf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pf[k][e] = _Float16(sacc[k >> 1][8 * (k & 1) + e]);
        // the row sum adds the fp16 P that the product uses, two at a time
        // (v_dot2_f32_f16 against (1, 1), fp32 accumulation)
        const f16x2 one2 = {_Float16(1.0f), _Float16(1.0f)};
        float ls[2] = {0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 pp = {pf[k][2 * e], pf[k][2 * e + 1]};
                ls[e & 1] = __builtin_amdgcn_fdot2(pp, one2, ls[e & 1], false);
            }
        const float lsum = ls[0] + ls[1];   // this lane half's share; the halves add up at the end
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {   // some row's maximum moved: rescale
            // rows whose maximum stayed keep their scale (their mrow may still
            // be -inf, and -inf - -inf is NaN)
            const float alpha = moved ? __builtin_amdgcn_exp2f(mrow - mnew) : 1.0f;
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[db][e] *= alpha;
        }
        lrow += lsum;
        mrow = mnew;

        // O^T += V^T P^T; the A fragment of sub-step k, d block db is two
        // transpose loads: keys 16 k + 8 g + 0..3 and + 4..7 of column 32 db + i
        if constexpr (D == 128) {
            // two d blocks at a time: their 16 transpose loads first, then their
            // MFMAs (at D = 64 the extra registers cost more than the read-ahead gains)
#pragma unroll
            for (int d2 = 0; d2 < NDB; d2 += 2) {
                f16x8 va[2][4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const _Float16 *vp = &vtb[b * VT + 16 * k * VP + 32 * (d2 + u) + vsrc];
                        const f16x4 v0 = lds_read_tr16(vp), v1 = lds_read_tr16(vp + 4 * VP);
                        va[u][k] = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    }
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        oacc[d2 + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[u][k], pf[k], oacc[d2 + u], 0, 0, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        } else {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const _Float16 *vp = &vtb[b * VT + 16 * k * VP + 32 * db + vsrc];
                    const f16x4 v0 = lds_read_tr16(vp), v1 = lds_read_tr16(vp + 4 * VP);
                    const f16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[k], oacc[db], 0, 0, 0);
                }
            }
        }
      }
        __syncthreads();   // tile t's buffer is free; tile t + 1's is written
    }

    lrow += __shfl_xor(lrow, 32);   // the row sum over both lane halves' keys
    // merge the halves: group 1 hands its O^T, maximum and sum to group 0
    f32x4 *mo = reinterpret_cast<f32x4 *>(&tiles[0][0]);                 // [4 qw][NDB][4 q][64 lanes]
    float *mm = reinterpret_cast<float *>(mo + 4 * NDB * 4 * 64);         // [2][4 qw][64 lanes]: maximum, sum
    if (grp == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mo[((qw * NDB + db) * 4 + q) * 64 + lane] =
                    f32x4{oacc[db][4 * q], oacc[db][4 * q + 1], oacc[db][4 * q + 2], oacc[db][4 * q + 3]};
        mm[qw * 64 + lane] = mrow;
        mm[(4 + qw) * 64 + lane] = lrow;
    }
    __syncthreads();
    if (grp == 1)
        return;
    {
        const float m1 = mm[qw * 64 + lane], l1 = mm[(4 + qw) * 64 + lane];
        const float mx = __builtin_fmaxf(mrow, m1);
        // a half with no visible key (maximum -inf) contributes nothing
        const float a0 = mrow == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mrow - mx);
        const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
        lrow = lrow * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 o1 = mo[((qw * NDB + db) * 4 + q) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    oacc[db][4 * q + e] = oacc[db][4 * q + e] * a0 + o1[e] * a1;
            }
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
