// Tiled prefill GEMM and fused SwiGLU for gfx950: in-kernel dequantization
// feeding v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
// Pages: comparison page section 2.1 (matrix units fed by dequantized tiles,
// padded threadgroup tiles, register ping-pong prefetch of the next codes),
// section 2.2 (gate and up in one workgroup sharing X, SiLU(g) * u epilogue on
// chip, only the activation written); project index Pillar 1 (128-bit loads,
// block-swizzled weight layout, conflict-free shared tiles).
//
// Work decomposition (one workgroup of WM x WN wave64 per BM x BN output tile):
//  * Wave (wm, wn) owns a TM x TN sub-tile = FM x FN blocks of 32 x 32.
//  * Per 64-deep k-step the workgroup stages the X tile [BM x 64] fp16 in LDS
//    (double-buffered; 16-byte chunks XOR-swizzled by row so that the 128-bit
//    fragment reads of 16 consecutive rows hit distinct banks).
//  * Each wave streams the planar codes of its own FN row groups straight
//    from memory into registers (one 128-bit load per lane per row group),
//    unpacks them to fp16 in registers in MFMA operand order and issues the
//    MFMAs: A = weights (rows n), B = activations (rows m), so each lane ends
//    with 4 consecutive n of one m -> 8-byte fp16 stores of Y.
//  * The next k-step's X tile and codes are fetched into registers before the
//    current step's MFMAs (the pages' q_next ping-pong) and written to the
//    other LDS buffer afterwards: one barrier per k-step.
//  * With 8 waves (2 per SIMD) one wave's unpack and LDS traffic overlaps the
//    other wave's matrix-core work.
//  * All global loads are raw buffer loads: out-of-range rows, row groups and
//    the K tail read as zero, so tails need no branches.
#include "launch.h"

namespace qg {
namespace {

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Consecutive workgroup ids land on different XCDs (round-robin over 8); give
// each XCD a contiguous run of tiles, m fastest, so the tiles of one XCD share
// weight row groups in its L2.
__device__ __forceinline__ int remap_tile(int bid, int ntiles)
{
    if (ntiles & 7)
        return bid;
    const int per = ntiles >> 3;
    return (bid & 7) * per + (bid >> 3);
}

struct GemmArgs {
    Planes w0, w1;
    const _Float16 *x;
    _Float16 *y;
    uint32_t x_bytes;
    int m, n, k, ldx, ldy;
    int groups, ksteps, kb128;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ float silu_mul(float g, float u)
{
    // SiLU(g) * u = g / (1 + exp(-g)) * u with exp(-g) = 2^(-g log2 e)
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <int CODEC, int BM, int BN, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmArgs a)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int NMAT = SWIGLU ? 2 : 1;
    constexpr int XCH = BM * 8 / NT;
    static_assert(FM >= 1 && FN >= 1 && XCH >= 1 && (BM * 8) % NT == 0, "tile");

    __shared__ u32x4 lds_x[2][BM * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int i = lane & 31, g = lane >> 5;
    const uint32_t magic = magic1024();

    const int tile = remap_tile(blockIdx.x, a.tiles_m * a.tiles_n);
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    const __amdgpu_buffer_rsrc_t xr_rsrc = make_rsrc(a.x, a.x_bytes);
    const PlaneRsrc w0 = plane_rsrc(a.w0);
    const PlaneRsrc w1 = plane_rsrc(SWIGLU ? a.w1 : a.w0);

    // per-thread X chunk coordinates (fixed across k-steps)
    uint32_t xoff[XCH];
    int xlds[XCH];
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
        const int q = tid + NT * c, r = q >> 3, ch = q & 7;
        xoff[c] = (uint32_t(m0 + r) * uint32_t(a.ldx) + uint32_t(ch * 8)) * 2u;
        xlds[c] = r * 8 + (ch ^ swz(r));
    }
    u32x4 xr[XCH];
    auto load_x = [&](int t) {
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int col = t * 64 + ((tid + NT * c) & 7) * 8;
            const uint32_t off = col < a.k ? xoff[c] + uint32_t(t) * 128u : OOB;
            xr[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr_rsrc, off, 0, 0));
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int c = 0; c < XCH; ++c)
            lds_x[buf][xlds[c]] = xr[c];
    };

    const int rg0 = (n0 + wn * TN) >> 5;
    LaneCodes<CODEC> cw[NMAT][FN];
    auto load_w = [&](int t, LaneCodes<CODEC>(&dst)[NMAT][FN]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            dst[0][fn] = load_lane<CODEC>(w0, rg0 + fn, t, a.ksteps, a.kb128, lane);
            if constexpr (SWIGLU)
                dst[NMAT - 1][fn] = load_lane<CODEC>(w1, rg0 + fn, t, a.ksteps, a.kb128, lane);
        }
    };

    f32x16 acc[NMAT][FM][FN];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[mt][fm][fn][e] = 0.0f;

    load_x(0);
    load_w(0, cw);
    store_x(0);
    __syncthreads();

    for (int t = 0; t < a.ksteps; ++t) {
        const int buf = t & 1;
        // prefetch step t+1 (past the end these read harmless in-range or zero data)
        LaneCodes<CODEC> cn[NMAT][FN];
        load_x(t + 1);
        load_w(t + 1, cn);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f16x8 wf[NMAT][FN];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    wf[mt][fn] = unpack_substep<CODEC>(cw[mt][fn], s, magic);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * TM + fm * 32 + i;
                const f16x8 xf = __builtin_bit_cast(f16x8, lds_x[buf][r * 8 + ((4 * g + s) ^ swz(r))]);
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[mt][fm][fn] =
                            __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[mt][fn], xf, acc[mt][fm][fn], 0, 0, 0);
            }
        }
        store_x(buf ^ 1);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                cw[mt][fn] = cn[mt][fn];
        __syncthreads();
    }

    // Epilogue: lane (i, g), register 4q+e of block (fm, fn) holds
    // C[n = fn*32 + 8q + 4g + e][m = fm*32 + i].
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * TM + fm * 32 + i;
        if (m >= a.m)
            continue;
        _Float16 *yrow = a.y + int64_t(m) * a.ldy;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * TN + fn * 32 + 8 * q + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (SWIGLU)
                        v[e] = silu_mul(acc[0][fm][fn][4 * q + e], acc[1][fm][fn][4 * q + e]);
                    else
                        v[e] = acc[0][fm][fn][4 * q + e];
                }
                if (n + 3 < a.n) {
                    f16x2 lo = {_Float16(v[0]), _Float16(v[1])};
                    f16x2 hi = {_Float16(v[2]), _Float16(v[3])};
                    *reinterpret_cast<u32x2 *>(yrow + n) = u32x2{as_u32(lo), as_u32(hi)};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.n)
                            yrow[n + e] = _Float16(v[e]);
                }
            }
        }
    }
}

template <int CODEC, int BM, int BN, int WM, int WN, bool SWIGLU>
hipError_t launch_tile(const GemmProblem &p, hipStream_t stream)
{
    GemmArgs a;
    a.w0 = p.w0;
    a.w1 = p.w1;
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
    a.tiles_m = int(ceil_div(p.m, BM));
    a.tiles_n = int(ceil_div(p.n, BN));
    void *args[] = {&a};
    const dim3 grid(unsigned(a.tiles_m * a.tiles_n)), block(64 * WM * WN);
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<CODEC, BM, BN, WM, WN, SWIGLU>), grid,
                           block, args, 0, stream);
}

int64_t tiles(const GemmProblem &p, int bm, int bn) { return ceil_div(p.m, bm) * ceil_div(p.n, bn); }

template <int CODEC>
hipError_t launch_codec(const GemmProblem &p, bool swiglu, hipStream_t stream)
{
    constexpr int64_t FILL = 256;   // compute units on MI355X
    if (swiglu) {
        if (p.m > 128)
            return launch_tile<CODEC, 256, 128, 2, 4, true>(p, stream);
        if (p.m > 64)
            return launch_tile<CODEC, 128, 128, 2, 2, true>(p, stream);
        return launch_tile<CODEC, 64, 64, 2, 2, true>(p, stream);
    }
    if (p.m > 128 && tiles(p, 256, 256) >= FILL)
        return launch_tile<CODEC, 256, 256, 2, 4, false>(p, stream);
    if (p.m > 128)
        return launch_tile<CODEC, 256, 128, 2, 4, false>(p, stream);
    if (p.m > 64)
        return launch_tile<CODEC, 128, 128, 2, 2, false>(p, stream);
    return launch_tile<CODEC, 64, 64, 2, 2, false>(p, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem &p, bool swiglu, hipStream_t stream)
{
    switch (p.codec) {
    case Q4_0: return launch_codec<Q4_0>(p, swiglu, stream);
    case MLX4_G64: return launch_codec<MLX4_G64>(p, swiglu, stream);
    case Q2_0: return launch_codec<Q2_0>(p, swiglu, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
