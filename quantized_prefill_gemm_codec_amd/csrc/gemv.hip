// Weight-streaming small-M projection (decode GEMV) and the dequantization probe.
//
// Pages: releases page v0.3.0 (the quantized linear layer switches to a GEMV
// for M = 1 on every codec); project index Pillar 4 (decode is bound by bytes
// streamed divided by bandwidth).  The GEMV reads every weight byte once, so it
// is HBM-bound: the design goal is the whole code stream in flight from the
// first cycles and as little VALU per byte as the codec allows.
//
// GEMV kernel (1 <= M <= 4): one workgroup of GEMV_NW waves per 32-row group.
//  * Wave w owns k-steps w, w + NW, w + 2 NW, ... of the row group and keeps
//    GEMV_PF of them in flight: per k-step one 128-bit (64-bit for Q2_0) code
//    load and one scale load per lane, contiguous across the wave, so the
//    eight waves together stream one contiguous run of the row group's codes
//    at a time.  Code loads carry the non-temporal hint (each byte is read
//    once), except ternary's three partial loads of one chunk, which share
//    cache lines.
//  * X [M, K] reaches LDS by DMA issued before the first batch of codes; the
//    wait for it leaves those codes in flight.
//  * The codes sit in a ring of GEMV_PF + 1 register slots, walked with the
//    loop unrolled by the ring size: before a wave waits for k-step j it
//    issues the load of k-step j + GEMV_PF into the slot k-step j - 1 has
//    just left, so a refill never waits for the dot products of the step
//    before it.  (On the 14336 x 4096 decode shape three slots in flight
//    measured fastest -- 7.45 us against 7.72 us for four slots refilled after
//    use; more requests in flight per lane, or sixteen waves, were slower.)
//  * The 1024 offset of the mantissa trick is not subtracted per weight:
//    slice_dots dots the raw (1024 + 2^f q) halves with X and block_sum removes
//    the offsets and the codec zero point once per 32-weight slice with a term
//    that depends on X only (slice_correction, computed once per workgroup).
//  * Lane halves, then waves, are reduced in a fixed order: results are
//    bit-identical from run to run.
#include "../../include/qgemm.h"
#include "launch.h"
#include "lds_dma.h"

namespace qg {
namespace {

constexpr int GEMV_NT = 64 * GEMV_NW;
constexpr int GEMV_PF = 3;               // k-steps of codes in flight per lane

struct GemvArgs {
    Planes w;
    const _Float16 *x;
    _Float16 *y;
    uint32_t x_bytes;
    int m, n, k, ldx, ldy;
    int groups, ksteps, kb128;
    int head_dim;            // 0: row-major Y; > 0: direct-head layout
    int x_lds;               // bytes of the X region
};

template <int CODEC> constexpr int corr_floats() { return CODEC == MLX4_G64 || CODEC == MLX4_G32 || CODEC == Q4_K ? 2 : 1; }

// x_s[p] = x_{2p} + x_{2p+1} summed over the 4 sub-step chunks of the slice.
template <int CODEC>
__device__ __forceinline__ void slice_correction(const u32x4 *chunks, float *out)
{
    float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const f16x8 v = __builtin_bit_cast(f16x8, chunks[c]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            sp[p] += float(v[2 * p]) + float(v[2 * p + 1]);
    }
    if constexpr (CODEC == Q8_0) {
        out[0] = -1152.0f * ((sp[0] + sp[1]) + (sp[2] + sp[3]));
    } else if constexpr (CODEC == TERNARY) {
        out[0] = -((sp[0] + sp[1]) + (sp[2] + sp[3]));
    } else if constexpr (CODEC == Q4_0) {
        out[0] = -1032.0f * (sp[0] + sp[2]) - 72.0f * (sp[1] + sp[3]);
    } else if constexpr (CODEC == MLX4_G64 || CODEC == MLX4_G32 || CODEC == Q4_K) {
        out[0] = -1024.0f * (sp[0] + sp[2]) - 64.0f * (sp[1] + sp[3]);
        out[1] = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    } else {
        out[0] = -1024.0f * (sp[0] + 0.25f * sp[1] + 0.0625f * sp[2] + 0.015625f * sp[3]) -
                 ((sp[0] + sp[1]) + (sp[2] + sp[3]));
    }
}

// Dot products of a lane's 32 codes with the matching X values, taken on the
// codes as they sit in the packed word: OR-ing a code field into the mantissa
// of binary16 1024 gives 1024 + 2^f q for a field at bit f of the half-word
// (f < 10), so no shift per field is needed -- only one 8-bit shift per word
// for the fields above bit 7.  v_dot2_f32_f16 multiplies exactly and sums in
// fp32; per class of fields with the same factor 2^f one fp32 partial sum:
//   Q4_0 / MLX4 / Q4_K: d[0] (fields at bits 0, 8 -> factor 1), d[1] (bits 4, 12 -> 16)
//   Q2_0:         d[p] (fields at bits 2p, 8 + 2p -> factor 4^p), p = 0..3
//   Q8_0:         d[0] (bytes at bits 0, 8 -> factor 1; stored q + 128)
//   ternary:      d[0..3] (digits t = q + 1 as subnormal fp16 t 2^-24, one
//                 accumulator per pair position)
// block_sum then removes the 1024 offsets (and the codec zero point) with the
// precomputed X term: sum_k (q_k - z) x_k = sum_c d[c] / 2^f_c + corr.
template <int CODEC, int MM>
__device__ __forceinline__ void slice_dots(const LaneCodes<CODEC> &lc, const u32x4 *const (&xrow)[MM],
                                           uint32_t magic, float (&d)[4][MM])
{
    if constexpr (CODEC == TERNARY) {
        // The digits t (0..2) are dotted as they come out of the extraction:
        // read as binary16 bit patterns they are the subnormals t 2^-24, so
        // each product is t x 2^-24 exactly and block_sum scales by 2^24.
        // Four independent pair chains and accumulators per sub-step keep the
        // multiply-to-use latencies of the packed integer ops covered.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t h[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int p = 4 * s + u;
                const uint32_t r = p < 5 ? lc.r0 : p < 10 ? lc.r1 : p < 15 ? lc.r2 : lc.r3;
                const uint32_t pw = p % 5 == 0 ? 1u : p % 5 == 1 ? 3u : p % 5 == 2 ? 9u : p % 5 == 3 ? 27u : 81u;
                h[u] = ternary_digits(r, p == 15 ? lc.m3 : pw | (pw << 16), p != 15 && p % 5 == 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int mr = 0; mr < MM; ++mr)
                    d[u][mr] = __builtin_amdgcn_fdot2(as_f16x2(h[u]), as_f16x2(xrow[mr][s][u]), d[u][mr], false);
        }
    } else if constexpr (CODEC == Q8_0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 h = (s < 2) ? lc.lo : lc.hi;
            const uint32_t a = h[2 * (s & 1)], b = h[2 * (s & 1) + 1];
            const uint32_t h0 = (a & 0x00FF00FFu) | magic, h1 = ((a >> 8) & 0x00FF00FFu) | magic;
            const uint32_t h2 = (b & 0x00FF00FFu) | magic, h3 = ((b >> 8) & 0x00FF00FFu) | magic;
#pragma unroll
            for (int mr = 0; mr < MM; ++mr) {
                const u32x4 xv = xrow[mr][s];
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h0), as_f16x2(xv[0]), d[0][mr], false);
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h1), as_f16x2(xv[1]), d[0][mr], false);
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h2), as_f16x2(xv[2]), d[0][mr], false);
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h3), as_f16x2(xv[3]), d[0][mr], false);
            }
        }
    } else if constexpr (CODEC == Q2_0) {
        const u32x2 c = lc.c;
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const uint32_t wv = c[wi];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t src = half ? (wv >> 8) : wv;
                const int s = 2 * wi + half;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t h = (src & (0x00030003u << (2 * p))) | magic;
#pragma unroll
                    for (int mr = 0; mr < MM; ++mr)
                        d[p][mr] = __builtin_amdgcn_fdot2(as_f16x2(h), as_f16x2(xrow[mr][s][p]), d[p][mr], false);
                }
            }
        }
    } else {
        const u32x4 c = lc.c;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t wv = c[s], w8 = wv >> 8;
            const uint32_t h0 = (wv & 0x000F000Fu) | magic, h1 = (wv & 0x00F000F0u) | magic;
            const uint32_t h2 = (w8 & 0x000F000Fu) | magic, h3 = (w8 & 0x00F000F0u) | magic;
#pragma unroll
            for (int mr = 0; mr < MM; ++mr) {
                const u32x4 xv = xrow[mr][s];
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h0), as_f16x2(xv[0]), d[0][mr], false);
                d[0][mr] = __builtin_amdgcn_fdot2(as_f16x2(h2), as_f16x2(xv[2]), d[0][mr], false);
                d[1][mr] = __builtin_amdgcn_fdot2(as_f16x2(h1), as_f16x2(xv[1]), d[1][mr], false);
                d[1][mr] = __builtin_amdgcn_fdot2(as_f16x2(h3), as_f16x2(xv[3]), d[1][mr], false);
            }
        }
    }
}

// acc + scale * sum_k (q_k - z) x_k (+ bias * sum_k x_k for MLX4 and Q4_K),
// with the scale and bias of the lane's 32-weight slice:
//   Q4_0, Q2_0, Q8_0: fp16 d;  MLX4: fp16 s, b;
//   Q4_K: d * sc and -dmin * m, both exact in fp32.
template <int CODEC>
__device__ __forceinline__ float block_sum(const LaneCodes<CODEC> &lc, const float (&d)[4], const float *corr,
                                           float acc)
{
    uint32_t sc = 0;
    if constexpr (CODEC == MLX4_G64 || CODEC == MLX4_G32)
        sc = lc.sb;
    else if constexpr (CODEC == Q4_K)
        sc = lc.dd;
    else
        sc = lc.d;
    const f16x2 sb = as_f16x2(sc);
    if constexpr (CODEC == Q4_K) {
        const float dsc = float(sb[0]) * float(lc.scm & 0xFFu);
        const float nm = -(float(sb[1]) * float((lc.scm >> 8) & 0xFFu));
        const float v = __builtin_fmaf(d[1], 0.0625f, d[0]) + corr[0];
        return __builtin_fmaf(dsc, v, __builtin_fmaf(nm, corr[1], acc));
    } else if constexpr (CODEC == TERNARY) {
        // sum (t - 1) x = 2^24 (sum of the subnormal-digit dots) - sum x
        const float v = __builtin_fmaf((d[0] + d[1]) + (d[2] + d[3]), 16777216.0f, corr[0]);
        return __builtin_fmaf(float(sb[0]), v, acc);
    } else if constexpr (CODEC == Q8_0) {
        return __builtin_fmaf(float(sb[0]), d[0] + corr[0], acc);
    } else if constexpr (CODEC == Q2_0) {
        const float v = __builtin_fmaf(d[3], 0.015625f, __builtin_fmaf(d[2], 0.0625f, __builtin_fmaf(d[1], 0.25f, d[0])));
        return __builtin_fmaf(float(sb[0]), v + corr[0], acc);
    } else if constexpr (CODEC == Q4_0) {
        return __builtin_fmaf(float(sb[0]), __builtin_fmaf(d[1], 0.0625f, d[0]) + corr[0], acc);
    } else {
        const float v = __builtin_fmaf(d[1], 0.0625f, d[0]) + corr[0];
        return __builtin_fmaf(float(sb[0]), v, __builtin_fmaf(float(sb[1]), corr[1], acc));
    }
}

template <int CODEC, int MM>
__global__ __launch_bounds__(GEMV_NT) void gemv_kernel(GemvArgs a)
{
    constexpr int NC = corr_floats<CODEC>();
    constexpr int PF = GEMV_PF;

    extern __shared__ u32x4 smem[];
    char *lds = reinterpret_cast<char *>(smem);
    const int kchunks = a.ksteps * 8;                 // 16-byte chunks per X row
    const u32x4 *xs = smem;                           // [MM][kchunks]
    float *corr = reinterpret_cast<float *>(lds + a.x_lds);   // [MM][ksteps][2][NC]
    float *red = corr + MM * a.ksteps * 2 * NC;       // [GEMV_NW][MM][32]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 31, g = lane >> 5;
    const int rg = blockIdx.x;
    const uint32_t magic = magic1024();

    const int t1 = a.ksteps;
    const PlaneRsrc w = plane_rsrc(a.w);
    const LaneOffsets lo = lane_offsets<CODEC>(rg, a.groups, lane);
    LaneOffsets none = lo;
    none.q = none.s = none.s2 = none.q2 = none.q3 = OOB;
    // codes and scales of k-step t; past the end the vector offsets are out
    // of range (zeros), so every call issues exactly lane_loads<CODEC>()
    // memory instructions
    auto fetch = [&](int t) {
        return load_lane<CODEC, CODEC != TERNARY>(w, t < t1 ? lo : none, rg, min(t, t1 - 1), a.ksteps, a.kb128);
    };
    {
        const u32x4 xw = rsrc_words(a.x, a.x_bytes);
        const uint32_t lbase = lds_u32(lds);
        const int xch = MM * kchunks, nxi = (xch + 63) >> 6;
        for (int j = wave; j < nxi; j += GEMV_NW) {
            const int q = j * 64 + lane;
            const int mr = q / kchunks, ch = q - mr * kchunks;
            const uint32_t off = (q < xch && mr < a.m && ch * 8 < a.k)
                                     ? (uint32_t(mr) * uint32_t(a.ldx) + uint32_t(ch) * 8u) * 2u : OOB;
            dma_b128(xw, off, 0, lbase + uint32_t(j) * 1024u);
        }
    }
    LaneCodes<CODEC> lc[PF + 1];
#pragma unroll
    for (int u = 0; u < PF; ++u)
        lc[u] = fetch(wave + u * GEMV_NW);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<PF * lane_loads<CODEC>()>();   // this wave's X DMAs (issued first) have landed
    __syncthreads();
    for (int q = tid; q < MM * a.ksteps * 2; q += GEMV_NT) {
        const int mr = q / (2 * a.ksteps), h = q - mr * 2 * a.ksteps;   // h = 2 t + g
        slice_correction<CODEC>(xs + mr * kchunks + h * 4, corr + q * NC);
    }
    __syncthreads();

    float acc[MM];
#pragma unroll
    for (int mr = 0; mr < MM; ++mr)
        acc[mr] = 0.0f;

    const int nper = (t1 - wave + GEMV_NW - 1) / GEMV_NW;   // k-steps of this wave
    for (int j0 = 0; j0 < nper; j0 += PF + 1) {
#pragma unroll
        for (int v = 0; v < PF + 1; ++v) {
            const int j = j0 + v;
            // slot (v + PF) % (PF + 1) held k-step j - 1, already consumed
            lc[(v + PF) % (PF + 1)] = fetch(wave + (j + PF) * GEMV_NW);
            __builtin_amdgcn_sched_barrier(0);
            const int t = wave + j * GEMV_NW;
            if (j < nper) {
                const u32x4 *xrow[MM];
#pragma unroll
                for (int mr = 0; mr < MM; ++mr)
                    xrow[mr] = xs + mr * kchunks + t * 8 + 4 * g;
                float dots[4][MM];
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int mr = 0; mr < MM; ++mr)
                        dots[c][mr] = 0.0f;
                prepare_lane<CODEC>(lc[v]);
                slice_dots<CODEC, MM>(lc[v], xrow, magic, dots);
#pragma unroll
                for (int mr = 0; mr < MM; ++mr) {
                    const float d4[4] = {dots[0][mr], dots[1][mr], dots[2][mr], dots[3][mr]};
                    acc[mr] = block_sum<CODEC>(lc[v], d4, corr + ((mr * a.ksteps + t) * 2 + g) * NC, acc[mr]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

#pragma unroll
    for (int mr = 0; mr < MM; ++mr) {
        acc[mr] += __shfl_xor(acc[mr], 32);
        if (g == 0)
            red[(wave * MM + mr) * 32 + i] = acc[mr];
    }
    __syncthreads();
    if (wave == 0 && g == 0) {
        const int n = rg * 32 + i;
        if (n < a.n) {
#pragma unroll
            for (int mr = 0; mr < MM; ++mr) {
                if (mr < a.m) {
                    float v = red[mr * 32 + i];
#pragma unroll
                    for (int w = 1; w < GEMV_NW; ++w)
                        v += red[(w * MM + mr) * 32 + i];
                    *out_at(a.y, a.ldy, a.head_dim, a.m, mr, n) = _Float16(v);
                }
            }
        }
    }
}

template <int CODEC>
__global__ __launch_bounds__(256) void dequant_kernel(Planes wp, int n, int k, int groups, int ksteps, int kb128,
                                                      _Float16 *out, int ldw)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunk = blockIdx.x * 4 + wave;
    if (chunk >= groups * ksteps)
        return;
    const int rg = chunk / ksteps, t = chunk - rg * ksteps;
    const int i = lane & 31, g = lane >> 5;
    const Magics mg = make_magics();
    const PlaneRsrc w = plane_rsrc(wp);
    LaneCodes<CODEC> lc = load_lane<CODEC>(w, lane_offsets<CODEC>(rg, groups, lane), rg, t, ksteps, kb128);
    prepare_lane<CODEC>(lc);
    const int row = rg * 32 + i;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const f16x8 v = unpack_substep<CODEC>(lc, s, mg);
        const int kk = t * 64 + 32 * g + 8 * s;
        if (row < n && kk < k)
            *reinterpret_cast<f16x8 *>(out + int64_t(row) * ldw + kk) = v;
    }
}

template <int CODEC, int MM>
hipError_t launch_gemv_mm(const GemmProblem &p, hipStream_t stream)
{
    GemvArgs a;
    a.w = p.w0;
    a.x = p.x;
    a.y = p.y;
    a.x_bytes = uint32_t(((p.m - 1) * p.ldx + p.k) * 2);
    a.m = int(p.m);
    a.n = int(p.n);
    a.k = int(p.k);
    a.ldx = int(p.ldx);
    a.ldy = int(p.ldy);
    a.head_dim = int(p.head_dim);
    a.groups = int(p.groups);
    a.ksteps = int(p.ksteps);
    a.kb128 = int(p.kb128);
    const GemvLds l = gemv_lds(CODEC, MM, p.ksteps);
    a.x_lds = l.x_lds;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_kernel<CODEC, MM>), dim3(unsigned(a.groups)),
                           dim3(GEMV_NT), args, size_t(l.bytes), stream);
}

template <int CODEC>
hipError_t launch_gemv_codec(const GemmProblem &p, int mm, hipStream_t stream)
{
    if (mm == 1)
        return launch_gemv_mm<CODEC, 1>(p, stream);
    if (mm == 2)
        return launch_gemv_mm<CODEC, 2>(p, stream);
    return launch_gemv_mm<CODEC, 4>(p, stream);
}

}  // namespace

hipError_t launch_gemv(const GemmProblem &p, const Choice &c, hipStream_t stream)
{
    if (c.kern != Kern::GEMV || p.m > c.mm || !gemv_fits(p.codec, p.m, p.ksteps))
        return hipErrorInvalidValue;
    switch (p.codec) {
    case Q4_0: return launch_gemv_codec<Q4_0>(p, c.mm, stream);
    case MLX4_G64: return launch_gemv_codec<MLX4_G64>(p, c.mm, stream);
    case MLX4_G32: return launch_gemv_codec<MLX4_G32>(p, c.mm, stream);
    case Q2_0: return launch_gemv_codec<Q2_0>(p, c.mm, stream);
    case Q8_0: return launch_gemv_codec<Q8_0>(p, c.mm, stream);
    case Q4_K: return launch_gemv_codec<Q4_K>(p, c.mm, stream);
    case TERNARY: return launch_gemv_codec<TERNARY>(p, c.mm, stream);
    }
    return hipErrorInvalidValue;
}

namespace {

// Streaming read: 512 workgroups (two per compute unit) of 512 threads, each
// reading one contiguous share with four 128-bit non-temporal loads in flight
// per lane -- the shape that measured fastest among contiguous and
// grid-stride variants at the 33 MB decode size.
constexpr int SR_NT = 512, SR_PF = 4, SR_GRID = 512;
static_assert(SR_GRID * SR_NT / 64 == QG_STREAM_READ_SLOTS, "one output slot per wave");

__global__ __launch_bounds__(SR_NT) void stream_read_kernel(const u32x4 *__restrict__ src, uint32_t n16,
                                                            uint32_t per_wg, uint32_t *out)
{
    const uint32_t base = blockIdx.x * per_wg;
    const uint32_t end = min(base + per_wg, n16);
    uint32_t acc = 0;
    for (uint32_t o = base + threadIdx.x; o < end; o += SR_NT * SR_PF) {
        u32x4 v[SR_PF];
#pragma unroll
        for (int u = 0; u < SR_PF; ++u) {
            const uint32_t idx = o + uint32_t(u) * SR_NT;
            v[u] = idx < end ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < SR_PF; ++u)
            acc ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
    }
    // wave XOR into the wave's own slot (no two waves share one)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        acc ^= __shfl_xor(acc, d);
    if ((threadIdx.x & 63) == 0)
        out[blockIdx.x * (SR_NT / 64) + (threadIdx.x >> 6)] ^= acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, hipStream_t stream)
{
    const uint32_t n16 = uint32_t(bytes / 16);
    const uint32_t per_wg = (n16 + SR_GRID - 1) / SR_GRID;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    uint32_t n = n16, per = per_wg;
    void *args[] = {&s, &n, &per, &out};
    return hipLaunchKernel(reinterpret_cast<const void *>(&stream_read_kernel), dim3(SR_GRID), dim3(SR_NT), args, 0,
                           stream);
}

hipError_t launch_dequant(const GemmProblem &p, _Float16 *out, int64_t ldw, hipStream_t stream)
{
    const int chunks = int(p.groups * p.ksteps);
    const dim3 grid(unsigned((chunks + 3) / 4)), block(256);
    const int n = int(p.n), k = int(p.k), groups = int(p.groups), ksteps = int(p.ksteps), kb128 = int(p.kb128);
    const int ld = int(ldw);
    Planes w = p.w0;
    void *args[] = {&w, const_cast<int *>(&n), const_cast<int *>(&k), const_cast<int *>(&groups),
                    const_cast<int *>(&ksteps), const_cast<int *>(&kb128), &out, const_cast<int *>(&ld)};
    const void *fn = nullptr;
    switch (p.codec) {
    case Q4_0: fn = reinterpret_cast<const void *>(&dequant_kernel<Q4_0>); break;
    case MLX4_G64: fn = reinterpret_cast<const void *>(&dequant_kernel<MLX4_G64>); break;
    case MLX4_G32: fn = reinterpret_cast<const void *>(&dequant_kernel<MLX4_G32>); break;
    case Q2_0: fn = reinterpret_cast<const void *>(&dequant_kernel<Q2_0>); break;
    case Q8_0: fn = reinterpret_cast<const void *>(&dequant_kernel<Q8_0>); break;
    case Q4_K: fn = reinterpret_cast<const void *>(&dequant_kernel<Q4_K>); break;
    case TERNARY: fn = reinterpret_cast<const void *>(&dequant_kernel<TERNARY>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace qg
