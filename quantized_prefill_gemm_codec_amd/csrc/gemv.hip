// Weight-streaming small-M projection (decode GEMV) and the dequantization probe.
//
// Pages: releases page v0.3.0 (the quantized linear layer switches to a GEMV
// for M = 1 on every codec); project index Pillar 4 (decode is bound by bytes
// streamed divided by bandwidth).  The GEMV reads every weight byte once, so it
// is HBM-bound: the design goal is many 128-bit loads in flight and just
// enough VALU per byte.
//
// GEMV kernel (1 <= M <= 4): one 256-thread workgroup per 32-row group of W.
//  * X [M, K] is staged in LDS once per workgroup; every lane of a half-wave
//    reads the same 16 bytes, so the fragment reads are LDS broadcasts.
//  * The four waves split the k-steps; each lane streams its own 16-byte code
//    slice per k-step (one 128-bit load, contiguous 1 KiB per wave) and its
//    scale, several k-steps ahead of use.
//  * The codes are turned into exact fp16 integers (q - offset) with the same
//    unpack routines as the GEMM, dotted with X by v_dot2_f32_f16 into a per
//    block fp32 sum, and the block scale is applied once per block in fp32:
//      Q4_0 / Q2_0:  acc += d * sum_k x_k (q_k - c)
//      MLX4-G64:     acc += s * sum_k x_k q_k + b * sum_k x_k
//    (the per-group sums of X are computed once per workgroup in LDS).
//  * Lane halves, then waves, are reduced in a fixed order: results are
//    bit-identical from run to run.
#include "launch.h"

namespace qg {
namespace {

constexpr int GEMV_NT = 256;
constexpr int GEMV_PF = 8;   // k-steps of codes in flight per lane

struct GemvArgs {
    Planes w;
    const _Float16 *x;
    _Float16 *y;
    uint32_t x_bytes;
    int m, n, k, ldx, ldy;
    int groups, ksteps, kb128;
};

template <int CODEC> __device__ __forceinline__ float scale_of(const LaneCodes<CODEC> &lc)
{
    if constexpr (CODEC == MLX4_G64)
        return float(as_f16x2(lc.sb)[0]);
    else
        return float(lc.d);
}

template <int CODEC, int MM>
__global__ __launch_bounds__(GEMV_NT) void gemv_kernel(GemvArgs a)
{
    extern __shared__ u32x4 smem[];
    const int kchunks = a.ksteps * 8;                 // 16-byte chunks per X row
    u32x4 *xs = smem;                                 // [MM][kchunks]
    float *xsum = reinterpret_cast<float *>(smem + MM * kchunks);   // [MM][2*ksteps]
    float *red = xsum + (CODEC == MLX4_G64 ? MM * 2 * a.ksteps : 0);  // [4][MM][32]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 31, g = lane >> 5;
    const int rg = blockIdx.x;
    const uint32_t magic = magic1024();
    const PlaneRsrc w = plane_rsrc(a.w);

    const int per = (a.ksteps + 3) >> 2;
    const int t0 = wave * per;
    const int t1 = min(a.ksteps, t0 + per);

    // first batch of codes before the X staging, to overlap the latencies
    const LaneOffsets lo = lane_offsets<CODEC>(rg, a.groups, lane);
    LaneCodes<CODEC> lc[GEMV_PF];
#pragma unroll
    for (int u = 0; u < GEMV_PF; ++u)
        lc[u] = load_lane<CODEC>(w, lo, rg, min(t0 + u, a.ksteps - 1), a.ksteps, a.kb128);

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    for (int q = tid; q < MM * kchunks; q += GEMV_NT) {
        const int mr = q / kchunks, ch = q - mr * kchunks;
        const uint32_t off = (mr < a.m && ch * 8 < a.k) ? (uint32_t(mr) * uint32_t(a.ldx) + uint32_t(ch) * 8u) * 2u : OOB;
        xs[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
    __syncthreads();
    if constexpr (CODEC == MLX4_G64) {
        for (int q = tid; q < MM * 2 * a.ksteps; q += GEMV_NT) {
            const int mr = q / (2 * a.ksteps), h = q - mr * 2 * a.ksteps;
            float sum = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f16x8 v = __builtin_bit_cast(f16x8, xs[mr * kchunks + h * 4 + c]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sum += float(v[e]);
            }
            xsum[q] = sum;
        }
        __syncthreads();
    }

    float acc[MM];
#pragma unroll
    for (int mr = 0; mr < MM; ++mr)
        acc[mr] = 0.0f;

    for (int tb = t0; tb < t1; tb += GEMV_PF) {
#pragma unroll
        for (int u = 0; u < GEMV_PF; ++u) {
            const int t = tb + u;
            if (t < t1) {
                float blk[MM];
#pragma unroll
                for (int mr = 0; mr < MM; ++mr)
                    blk[mr] = 0.0f;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 xv[MM];
#pragma unroll
                    for (int mr = 0; mr < MM; ++mr)
                        xv[mr] = xs[mr * kchunks + t * 8 + 4 * g + s];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const f16x2 f = factor_pair<CODEC>(lc[u], s, p, magic);
#pragma unroll
                        for (int mr = 0; mr < MM; ++mr)
                            blk[mr] = __builtin_amdgcn_fdot2(f, as_f16x2(xv[mr][p]), blk[mr], false);
                    }
                }
                const float sc = scale_of<CODEC>(lc[u]);
#pragma unroll
                for (int mr = 0; mr < MM; ++mr) {
                    if constexpr (CODEC == MLX4_G64)
                        acc[mr] += sc * blk[mr] + float(as_f16x2(lc[u].sb)[1]) * xsum[mr * 2 * a.ksteps + 2 * t + g];
                    else
                        acc[mr] += sc * blk[mr];
                }
            }
            // refill this slot with the k-step one batch ahead
            const int tn = tb + GEMV_PF + u;
            if (tn < t1)
                lc[u] = load_lane<CODEC>(w, lo, rg, tn, a.ksteps, a.kb128);
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
                    const float v = ((red[(0 * MM + mr) * 32 + i] + red[(1 * MM + mr) * 32 + i]) +
                                     red[(2 * MM + mr) * 32 + i]) + red[(3 * MM + mr) * 32 + i];
                    a.y[int64_t(mr) * a.ldy + n] = _Float16(v);
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
    const uint32_t magic = magic1024();
    const PlaneRsrc w = plane_rsrc(wp);
    const LaneCodes<CODEC> lc = load_lane<CODEC>(w, lane_offsets<CODEC>(rg, groups, lane), rg, t, ksteps, kb128);
    const int row = rg * 32 + i;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const f16x8 v = unpack_substep<CODEC>(lc, s, magic);
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
    a.groups = int(p.groups);
    a.ksteps = int(p.ksteps);
    a.kb128 = int(p.kb128);
    const size_t lds = size_t(MM) * size_t(a.ksteps) * 128 +
                       (CODEC == MLX4_G64 ? size_t(MM) * 2 * size_t(a.ksteps) * 4 : 0) + 4 * MM * 32 * 4;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_kernel<CODEC, MM>), dim3(unsigned(a.groups)),
                           dim3(GEMV_NT), args, lds, stream);
}

template <int CODEC>
hipError_t launch_gemv_codec(const GemmProblem &p, hipStream_t stream)
{
    if (p.m == 1)
        return launch_gemv_mm<CODEC, 1>(p, stream);
    if (p.m == 2)
        return launch_gemv_mm<CODEC, 2>(p, stream);
    return launch_gemv_mm<CODEC, 4>(p, stream);
}

}  // namespace

// LDS the VALU GEMV needs; beyond this the tiled MFMA kernel serves small M.
static size_t gemv_lds_bytes(const GemmProblem &p)
{
    const int64_t mm = p.m == 1 ? 1 : p.m == 2 ? 2 : 4;
    return size_t(mm * p.ksteps * 128 + (p.codec == MLX4_G64 ? mm * 2 * p.ksteps * 4 : 0) + 4 * mm * 32 * 4);
}

hipError_t launch_gemv(const GemmProblem &p, hipStream_t stream)
{
    if (p.m > 4 || gemv_lds_bytes(p) > 64 * 1024)
        return launch_gemm(p, false, stream);
    switch (p.codec) {
    case Q4_0: return launch_gemv_codec<Q4_0>(p, stream);
    case MLX4_G64: return launch_gemv_codec<MLX4_G64>(p, stream);
    case Q2_0: return launch_gemv_codec<Q2_0>(p, stream);
    }
    return hipErrorInvalidValue;
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
    case Q2_0: fn = reinterpret_cast<const void *>(&dequant_kernel<Q2_0>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace qg
