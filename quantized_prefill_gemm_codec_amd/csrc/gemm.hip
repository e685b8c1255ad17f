// Tiled prefill GEMM and fused SwiGLU for gfx950: in-kernel dequantization
// feeding v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
// Pages: comparison page section 2.1 (matrix units fed by dequantized tiles,
// padded threadgroup tiles, register ping-pong prefetch of the next codes),
// section 2.2 (gate and up in one workgroup sharing X, SiLU(g) * u epilogue on
// chip, only the activation written); project index Pillar 1 (128-bit loads,
// block-swizzled weight layout, conflict-free shared tiles).
//
// Common to both kernels (one workgroup of WM x WN wave64 per BM x BN tile):
//  * Wave (wm, wn) owns a TM x TN sub-tile = FM x FN blocks of 32 x 32.
//  * Per 64-deep k-step the X tile [BM x 64] fp16 sits in LDS, its 16-byte
//    chunks XOR-swizzled by row so that the 128-bit fragment reads of 16
//    consecutive rows hit distinct banks.
//  * Each wave unpacks the planar codes of its own FN row groups to fp16 in
//    registers, in MFMA operand order, and issues the MFMAs: A = weights (rows
//    n), B = activations (rows m), so each lane ends with 4 consecutive n of
//    one m.
//  * All global loads are raw buffer loads: out-of-range rows, row groups and
//    the K tail read as zero, so tails need no branches.
//
// gemm_kernel (gated Q8_0 up to M = 128): codes stream from memory straight
// into registers and the next k-step's X tile is fetched into registers before
// the current step's MFMAs (the pages' q_next ping-pong), then written to the
// other LDS buffer: one barrier per k-step.
//
// gemm_dma_kernel (M > 128, and M <= 128 with a split k-loop, plain or gated):
// X tiles, code chunks and scale records all reach LDS by hardware DMA a few
// k-steps ahead of use; see the comment above the kernel.
#include "kutil.h"
#include "launch.h"
#include "lds_dma.h"

namespace qg {
namespace {

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
    int head_dim;            // 0: row-major Y; > 0: direct-head [N / head_dim, M, head_dim]
};

__device__ __forceinline__ float sigmoid_mul(float g, float z, float u)
{
    // g * sigmoid(z) * u = g / (1 + exp(-z)) * u with exp(-z) = 2^(-z log2 e)
    const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Gated epilogues on the (gate, up) accumulator pair, in fp32:
//   GLU 1 (SwiGLU): SiLU(g) * u = g * sigmoid(g) * u
//   GLU 2 (GeGLU):  GELU(g) * u with the tanh form of GELU, written as
//                   g * sigmoid(2 sqrt(2/pi) (g + 0.044715 g^3)) * u
//                   (0.5 (1 + tanh(t)) = sigmoid(2 t)).
template <int GLU> __device__ __forceinline__ float glu_mul(float g, float u)
{
    if constexpr (GLU == 1)
        return sigmoid_mul(g, g, u);
    else
        return sigmoid_mul(g, 1.5957691216057308f * __builtin_fmaf(0.044715f * g, g * g, g), u);
}

template <int CODEC, int BM, int BN, int WM, int WN, int GLU>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmArgs a)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int NMAT = GLU ? 2 : 1;
    constexpr int XCH = BM * 8 / NT;        // 16-byte X chunks per thread per k-step
    constexpr int STAGE = BM * 128;         // bytes of one X stage in LDS
    static_assert(FM >= 1 && FN >= 1 && XCH >= 1 && (BM * 8) % NT == 0 && (TM % 64 == 0 || FM == 1), "tile");

    __shared__ u32x4 lds_x[2 * BM * 8];
    char *lds = reinterpret_cast<char *>(lds_x);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int i = lane & 31, g = lane >> 5;
    const Magics mg = make_magics();

    const int tile = remap_tile(blockIdx.x, a.tiles_m * a.tiles_n);
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int last = a.ksteps - 1;
    const int ktail = a.k & 63;             // 32 when the last k-step is half empty (Q4_0)

    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, a.x_bytes);
    const PlaneRsrc w0 = plane_rsrc(a.w0);
    const PlaneRsrc w1 = plane_rsrc(GLU ? a.w1 : a.w0);

    // X staging: thread chunk c covers tile row r = (tid + NT c) / 8 and the
    // 16-byte column ch = tid % 8; rows past M and the K tail get out-of-range
    // vector offsets (zero fill), the k-step goes in the scalar offset.
    const int ch = tid & 7;
    uint32_t xv[XCH], xvt[XCH], xl[XCH];
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
        const int r = (tid + NT * c) >> 3;
        xv[c] = (m0 + r < a.m) ? (uint32_t(m0 + r) * uint32_t(a.ldx) + uint32_t(ch * 8)) * 2u : OOB;
        xvt[c] = (ch * 8 < ktail) ? xv[c] : OOB;
        xl[c] = uint32_t(r * 8 + (ch ^ swz(r))) * 16u;
    }
    auto load_x = [&](int t, u32x4(&dst)[XCH]) {
        const bool tail = (t == last) && ktail != 0;
#pragma unroll
        for (int c = 0; c < XCH; ++c)
            dst[c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, tail ? xvt[c] : xv[c], uint32_t(t) * 128u, 0));
    };
    auto store_x = [&](int buf, const u32x4(&src)[XCH]) {
#pragma unroll
        for (int c = 0; c < XCH; ++c)
            *reinterpret_cast<u32x4 *>(lds + buf * STAGE + xl[c]) = src[c];
    };

    // MFMA B-operand reads: row r = wm*TM + fm*32 + i, 16-byte column 4g + s;
    // swz(r) depends only on i and the parity of fm.
    uint32_t rb[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = wm * TM + p * 32 + i;
            rb[p][s] = uint32_t(r * 8 + ((4 * g + s) ^ swz(r))) * 16u;
        }
    auto read_x = [&](int buf, int s, f16x8(&xf)[FM]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            xf[fm] = *reinterpret_cast<const f16x8 *>(lds + buf * STAGE + rb[fm & 1][s] + (fm & ~1) * 4096);
    };

    const int rg0 = (n0 + wn * TN) >> 5;
    LaneOffsets lo[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        lo[fn] = lane_offsets<CODEC>(rg0 + fn, a.groups, lane);
    auto load_w = [&](int t, LaneCodes<CODEC>(&dst)[NMAT][FN]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            dst[0][fn] = load_lane<CODEC>(w0, lo[fn], rg0 + fn, t, a.ksteps, a.kb128);
            if constexpr (GLU != 0)
                dst[NMAT - 1][fn] = load_lane<CODEC>(w1, lo[fn], rg0 + fn, t, a.ksteps, a.kb128);
        }
    };
    auto unpack = [&](const LaneCodes<CODEC>(&cw)[NMAT][FN], int s, f16x8(&wf)[NMAT][FN]) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                wf[mt][fn] = unpack_substep<CODEC>(cw[mt][fn], s, mg);
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

    // One k-step: codes for t are in cw, X(t) is in LDS stage buf.  Fetch
    // step t+1 (clamped: every scalar offset stays inside its buffer), then
    // run the four 16-deep sub-steps, preparing sub-step s+1 (LDS reads and
    // unpack) while the MFMAs of sub-step s issue.
    auto step = [&](int t, int buf, const LaneCodes<CODEC>(&cw)[NMAT][FN], LaneCodes<CODEC>(&cn)[NMAT][FN]) {
        const int tnx = min(t + 1, last);
        u32x4 xr[XCH];
        load_x(tnx, xr);
        load_w(tnx, cn);
        LaneCodes<CODEC> cp[NMAT][FN];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                cp[mt][fn] = cw[mt][fn];
                prepare_lane<CODEC>(cp[mt][fn]);
            }
        f16x8 xf[2][FM];
        f16x8 wf[2][NMAT][FN];
        read_x(buf, 0, xf[0]);
        unpack(cp, 0, wf[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cur = s & 1;
            if (s < 3) {
                read_x(buf, s + 1, xf[cur ^ 1]);
                unpack(cp, s + 1, wf[cur ^ 1]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[mt][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][mt][fn], xf[cur][fm],
                                                                                 acc[mt][fm][fn], 0, 0, 0);
            {
                constexpr int NMF = FM * FN * NMAT;
                constexpr int NV = (NMAT * FN * 16 + NMF - 1) / NMF;
#pragma unroll
                for (int j = 0; j < NMF; ++j) {
                    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                    if (s < 3)
                        __builtin_amdgcn_sched_group_barrier(SG_VALU, NV, 0);
                    if (s < 3 && j < FM)
                        __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
                    if (s == 0 && j < XCH + 2 * NMAT * FN)
                        __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
                    if (s == 3 && j < XCH)
                        __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
                }
            }
        }
        store_x(buf ^ 1, xr);
        __syncthreads();
    };

    {
        u32x4 xr0[XCH];
        load_x(0, xr0);
        store_x(0, xr0);
    }
    LaneCodes<CODEC> ca[NMAT][FN], cb[NMAT][FN];
    load_w(0, ca);
    __syncthreads();
    int t = 0;
    for (; t + 1 < a.ksteps; t += 2) {
        step(t, 0, ca, cb);
        step(t + 1, 1, cb, ca);
    }
    if (t < a.ksteps)
        step(t, 0, ca, cb);

    // Epilogue: lane (i, g), register 4q+e of block (fm, fn) holds
    // C[n = fn*32 + 8q + 4g + e][m = fm*32 + i].
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * TM + fm * 32 + i;
        if (m >= a.m)
            continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * TN + fn * 32 + 8 * q + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (GLU != 0)
                        v[e] = glu_mul<GLU>(acc[0][fm][fn][4 * q + e], acc[1][fm][fn][4 * q + e]);
                    else
                        v[e] = acc[0][fm][fn][4 * q + e];
                }
                _Float16 *dst = out_at(a.y, a.ldy, a.head_dim, a.m, m, n);
                if (n + 3 < a.n) {
                    f16x2 lo2 = {_Float16(v[0]), _Float16(v[1])};
                    f16x2 hi2 = {_Float16(v[2]), _Float16(v[3])};
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{as_u32(lo2), as_u32(hi2)};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.n)
                            dst[e] = _Float16(v[e]);
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Large-tile kernel: every operand reaches LDS by hardware DMA.
//
// X tiles, code chunks and scale records of k-step t+2 are copied from HBM
// straight into LDS stage (t+2) % 3 with buffer_load ... lds (no registers,
// no ds_write), two k-steps ahead of use.  These loads are issued from inline
// assembly so that the only wait on them is the explicit vmcnt before the
// end-of-step barrier (the compiler would otherwise drain all of them before
// every LDS read).  Waves then read their MFMA operands from LDS: X fragments
// (B operand) and their own row groups' code slices (A operand, unpacked in
// registers).  The epilogue converts the accumulators to fp16 into LDS and
// writes whole rows of Y with 16-byte stores.
// ---------------------------------------------------------------------------
// Tile order: each XCD gets a contiguous run of tiles, and runs are laid out
// in groups of GM m-tiles so that the tiles resident on one XCD at a time
// share both X rows and weight row groups in its L2.
__device__ __forceinline__ void grouped_tile(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int nt = tiles_m * tiles_n;
    int l = bid;
    if ((nt & 7) == 0)
        l = (bid & 7) * (nt >> 3) + (bid >> 3);
    constexpr int GM = 4;
    const int per_group = GM * tiles_n;
    const int group = l / per_group;
    const int first = group * GM;
    const int gsm = min(tiles_m - first, GM);
    const int idx = l - group * per_group;
    tm = first + idx % gsm;
    tn = idx / gsm;
}

// WK > 1 splits the k-steps of a tile into WK contiguous slices, one per
// group of WM x WN waves; each group has its own X / code / scale slice in
// every stage, and the WK fp32 partial tiles are summed in LDS (fixed order)
// in the epilogue.  Used for small M, where the tiles alone would leave most
// SIMDs idle.  LDS holds NSTAGE stages of KS k-steps each: a stage's DMAs are
// issued together, NSTAGE-1 stages ahead of use, and the wait + barrier that
// make a stage visible come once per stage.
template <int CODEC, int BM, int BN, int WM, int WN, int WK, int GLU, int NSTAGE, int KS = 1>
__global__ __launch_bounds__(64 * WM * WN * WK, 1) void gemm_dma_kernel(GemmArgs a)
{
    constexpr int NWT = WM * WN;                           // waves per k-slice
    constexpr int NW = NWT * WK, NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int NMAT = GLU ? 2 : 1;
    constexpr int RG = BN / 32;                            // row groups per matrix per tile
    constexpr bool TERN = CODEC == TERNARY;
    constexpr int CB = CODEC == Q2_0 ? 8 : CODEC == Q8_0 ? 32 : 16;   // code bytes per lane per chunk
    // LDS bytes per (row group, k-step) chunk; ternary chunks (416 bytes in
    // memory) arrive by two dword DMA instructions into a 512-byte slot
    constexpr int WCH = TERN ? 512 : 64 * CB;
    constexpr int WDMA = TERN ? 256 : 1024;                // chunk bytes per code DMA instruction
    // scale bytes staged per (row group, k-step); Q4_K: the k-step's u16 (sc, m)
    // lane records, then the super-block's (d, dmin) row records
    constexpr int SB = (CODEC == Q2_0 || TERN) ? 64 : (CODEC == MLX4_G32 || CODEC == Q4_K) ? 256 : 128;
    constexpr int X_OFF = 0, X_BYTES = BM * 128;
    constexpr int W_OFF = X_BYTES, W_BYTES = NMAT * RG * WCH;
    // each matrix's scale records take a whole number of 256-byte DMA
    // instructions, so that no instruction (one buffer descriptor) spans both
    // matrices of a gated tile
    constexpr int SPM = (RG * SB + 255) / 256 * 256;       // scale bytes per matrix, padded
    constexpr int S_OFF = W_OFF + W_BYTES, S_BYTES = NMAT * SPM;
    constexpr int SLICE = (S_OFF + S_BYTES + 255) / 256 * 256;   // one k-slice of one k-step slot
    constexpr int STAGE = WK * SLICE;                      // one k-step slot
    constexpr int AHEAD = NSTAGE - 1;                      // stages of lead
    constexpr int NSLOT = NSTAGE * KS;                     // k-step slots in LDS
    constexpr int PPITCH = BN * 4 + 16;                    // fp32 partial tile row pitch (WK > 1)
    constexpr int EPI_BYTES = WK == 1 ? BM * BN * 2 : NMAT * WK * BM * PPITCH;   // WK > 1: fp32 partials
    constexpr int LDS_BYTES = NSLOT * STAGE > EPI_BYTES ? NSLOT * STAGE : EPI_BYTES;
    constexpr int NX = X_BYTES / 1024, NWI = W_BYTES / WDMA, NSI = (S_BYTES + 255) / 256;   // DMA ops per slice
    constexpr int XPW = NX / NWT, WPW = (NWI + NWT - 1) / NWT, SPW = (NSI + NWT - 1) / NWT;
    constexpr int VMIN = XPW + NWI / NWT + NSI / NWT;       // fewest DMA ops any wave issues per stage
    constexpr int VMAX = XPW + WPW + SPW;                   // most
    constexpr int VWAIT = (AHEAD - 1) * KS * VMAX;          // DMA ops that may stay in flight, at most
    static_assert(NX % NWT == 0 && W_BYTES % 1024 == 0 && SLICE % 256 == 0, "dma tiling");
    static_assert((FM == 1 || FM % 2 == 0) && VMIN >= 1 && NSTAGE >= 2 && NSLOT >= 3 && VWAIT < 64 &&
                      VMAX - VMIN <= 2, "tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");

    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
    const uint32_t lds0 = lds_u32(lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave / NWT, wr = wave % NWT;            // k-slice, wave inside the slice group
    const int wm = wr % WM, wn = wr / WM;
    const int i = lane & 31, g = lane >> 5;
    const Magics mg = make_magics();

    int tm, tn;
    grouped_tile(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int last = a.ksteps - 1;
    const int ktail = a.k & 63;
    const int rg0 = n0 >> 5;
    const int kq = (a.ksteps + WK - 1) / WK;                // iterations (k-steps per slice)
    const int kbase = wk * kq;                             // first k-step of this wave's slice

    const u32x4 xr = rsrc_words(a.x, a.x_bytes);
    const u32x4 q0 = rsrc_words(a.w0.qs, a.w0.qs_bytes), s0 = rsrc_words(a.w0.scales, a.w0.scale_bytes);
    const u32x4 q1 = GLU ? rsrc_words(a.w1.qs, a.w1.qs_bytes) : q0;
    const u32x4 s1 = GLU ? rsrc_words(a.w1.scales, a.w1.scale_bytes) : s0;

    // ---- per-lane DMA source offsets (fixed across k-steps) ----
    // X: instruction j fills LDS slots 64j..64j+63; slot p holds tile row
    // p/8, 16-byte column (p%8) ^ swz(row).
    uint32_t xv[XPW], xvt[XPW];
#pragma unroll
    for (int u = 0; u < XPW; ++u) {
        const int p = (wr + NWT * u) * 64 + lane;
        const int r = p >> 3, ch = (p & 7) ^ swz(r);
        xv[u] = (m0 + r < a.m) ? (uint32_t(m0 + r) * uint32_t(a.ldx) + uint32_t(ch * 8)) * 2u : OOB;
        xvt[u] = (ch * 8 < ktail) ? xv[u] : OOB;
    }
    // codes: instruction j covers chunk bytes [1024 j, 1024 j + 1024) of the
    // stage's code area (one 4-bit chunk, two 2-bit chunks, or one half of an
    // 8-bit chunk)
    uint32_t wv[WPW];
    int wmat[WPW];
#pragma unroll
    for (int u = 0; u < WPW; ++u) {
        const int j = wr + NWT * u;
        if constexpr (TERN) {
            // instruction j: bytes [256 (j & 1), + 256) of chunk j / 2 (valid below 416)
            const int c = j >> 1, rg = c % RG;
            const uint32_t lo = uint32_t(j & 1) * 256u + uint32_t(lane) * 4u;
            wmat[u] = c / RG;
            wv[u] = (j < NWI && rg0 + rg < a.groups && lo < uint32_t(TERNARY_CHUNK))
                        ? uint32_t(rg0 + rg) * uint32_t(a.ksteps) * uint32_t(TERNARY_CHUNK) + lo
                        : OOB;
            continue;
        }
        const int c = CB == 16 ? j : CB == 32 ? (j >> 1) : 2 * j + (lane >> 5);
        const int rg = c % RG;
        const uint32_t lo = CB == 16 ? uint32_t(lane) * 16
                          : CB == 32 ? uint32_t(j & 1) * 1024 + uint32_t(lane) * 16
                                     : uint32_t(lane & 31) * 16;
        wmat[u] = (CB == 16 ? j : CB == 32 ? (j >> 1) : 2 * j) / RG;     // wave-uniform: RG is even
        wv[u] = (j < NWI && rg0 + rg < a.groups) ? uint32_t(rg0 + rg) * uint32_t(a.ksteps) * WCH + lo : OOB;
    }
    // scales: dword instruction j covers bytes [256 j, 256 j + 256) of the
    // stage's scale area: per matrix SPM bytes, SB per row group, then padding
    uint32_t sv[SPW], sk[SPW];
    int smat[SPW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int j = wr + NWT * u;
        const int b = 256 * j + 4 * lane;
        const int bm = b % SPM;                     // byte inside the matrix's area
        const int rg = bm / SB, o = bm % SB;
        smat[u] = (256 * j) / SPM;                  // wave-uniform: SPM is a multiple of 256
        const uint32_t pitch = CODEC == Q2_0   ? uint32_t(a.kb128) * 64u
                             : TERN          ? uint32_t(a.ksteps >> 2) * 64u   // one record per 4 k-steps
                             : CODEC == Q4_K ? uint32_t(a.ksteps) * 160u      // 640 B per 4 k-steps
                                             : uint32_t(a.ksteps) * uint32_t(SB);
        // Q4_K: bytes [0, 128) of a chunk come from the k-step's lane records
        // (+ 128 (t % 4) at issue), bytes [128, 256) from the row records at 512
        const uint32_t src = CODEC == Q4_K && o >= 128 ? uint32_t(o) - 128u + 512u : uint32_t(o);
        sv[u] = (j < NSI && b < S_BYTES && bm < RG * SB && rg0 + rg < a.groups) ? uint32_t(rg0 + rg) * pitch + src
                                                                                : OOB;
        // Q4_K: the lane records move by 128 bytes per k-step inside their
        // 4-k-step record, the row records do not
        sk[u] = CODEC == Q4_K && o < 128 ? 128u : 0u;
    }

    // Waves issue different numbers of DMA ops per stage (the code and scale
    // instructions are spread over the slice's waves), so each waits for its
    // own count: stage t+1 has landed once at most this wave's ops of the
    // AHEAD-1 newer stages remain.  Waiting for fewer (a shared, smaller
    // count) would also wait for loads just issued for the newest stage.
    int nops = XPW;
#pragma unroll
    for (int u = 0; u < WPW; ++u)
        nops += (wr + NWT * u < NWI) ? 1 : 0;
#pragma unroll
    for (int u = 0; u < SPW; ++u)
        nops += (wr + NWT * u < NSI) ? 1 : 0;
    nops = __builtin_amdgcn_readfirstlane(nops);
    auto wait_stage = [&]() {
        if (nops >= VMIN + 2)
            wait_vmcnt<(AHEAD - 1) * KS * (VMIN + 2 <= VMAX ? VMIN + 2 : VMIN)>();
        else if (nops == VMIN + 1)
            wait_vmcnt<(AHEAD - 1) * KS * (VMIN + 1 <= VMAX ? VMIN + 1 : VMIN)>();
        else
            wait_vmcnt<(AHEAD - 1) * KS * VMIN>();
    };

    // iteration i of this wave's slice = k-step kbase + i; past the end of K
    // (last slice of a ragged split) every vector offset is out of range, so
    // the stage fills with zeros and the MFMAs add nothing.
    auto issue_stage = [&](int i, int stage) {
        const uint32_t base = lds0 + uint32_t(stage * STAGE + wk * SLICE);
        const int t = min(kbase + i, last);
        const bool in = kbase + i <= last;
        const bool tail = (t == last) && ktail != 0;
#pragma unroll
        for (int u = 0; u < XPW; ++u)
            dma_b128(xr, in ? (tail ? xvt[u] : xv[u]) : OOB, uint32_t(t) * 128u,
                     base + X_OFF + uint32_t((wr + NWT * u) * 1024));
#pragma unroll
        for (int u = 0; u < WPW; ++u) {
            const int j = wr + NWT * u;
            if (j < NWI) {
                if constexpr (TERN)
                    dma_b32(wmat[u] ? q1 : q0, in ? wv[u] : OOB, uint32_t(t) * uint32_t(TERNARY_CHUNK),
                            base + W_OFF + uint32_t(j * 256));
                else
                    dma_b128(wmat[u] ? q1 : q0, in ? wv[u] : OOB, uint32_t(t) * WCH, base + W_OFF + uint32_t(j * 1024));
            }
        }
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int j = wr + NWT * u;
            const uint32_t so = CODEC == Q2_0   ? uint32_t(t >> 1) * 64u
                              : TERN          ? uint32_t(t >> 2) * 64u
                              : CODEC == Q4_K ? uint32_t(t >> 2) * 640u
                                              : uint32_t(t) * uint32_t(SB);
            // (an out-of-range offset stays out of range with the record step added)
            const uint32_t v = in ? (CODEC == Q4_K ? sv[u] + uint32_t(t & 3) * sk[u] : sv[u]) : OOB;
            if (j < NSI)
                dma_b32(smat[u] ? s1 : s0, v, so, base + S_OFF + uint32_t(j * 256));
        }
    };

    // ---- MFMA operand reads from a stage ----
    uint32_t rb[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = wm * TM + p * 32 + i;
            rb[p][s] = uint32_t(r * 8 + ((4 * g + s) ^ swz(r))) * 16u;
        }
    auto read_x = [&](const char *st, int s, f16x8(&xf)[FM]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            xf[fm] = *reinterpret_cast<const f16x8 *>(st + X_OFF + rb[fm & 1][s] + (fm & ~1) * 4096);
    };
    auto read_w = [&](const char *st, LaneCodes<CODEC>(&cw)[NMAT][FN]) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int c = mt * RG + wn * FN + fn;
                const char *wp = st + W_OFF + c * WCH + lane * (CB == 32 ? 16 : CB);
                const char *sp = st + S_OFF + mt * SPM + (wn * FN + fn) * SB;
                if constexpr (TERN) {
                    const char *cp = st + W_OFF + c * WCH;
                    cw[mt][fn].a = *reinterpret_cast<const uint32_t *>(cp + lane * 4);
                    cw[mt][fn].b = *reinterpret_cast<const unsigned short *>(cp + 256 + lane * 2);
                    cw[mt][fn].tl = *reinterpret_cast<const unsigned char *>(cp + 384 + (lane >> 1));
                    cw[mt][fn].d = *reinterpret_cast<const unsigned short *>(sp + i * 2);
                    prepare_lane<CODEC>(cw[mt][fn]);
                } else if constexpr (CODEC == Q4_K) {
                    cw[mt][fn].c = *reinterpret_cast<const u32x4 *>(wp);
                    cw[mt][fn].scm = *reinterpret_cast<const unsigned short *>(sp + lane * 2);
                    cw[mt][fn].dd = *reinterpret_cast<const uint32_t *>(sp + 128 + i * 4);
                    prepare_lane<CODEC>(cw[mt][fn]);
                } else if constexpr (CODEC == Q8_0) {
                    cw[mt][fn].lo = *reinterpret_cast<const u32x4 *>(wp);
                    cw[mt][fn].hi = *reinterpret_cast<const u32x4 *>(wp + 1024);
                    cw[mt][fn].d = *reinterpret_cast<const unsigned short *>(sp + lane * 2);
                } else if constexpr (CODEC == Q2_0) {
                    cw[mt][fn].c = *reinterpret_cast<const u32x2 *>(wp);
                    cw[mt][fn].d = *reinterpret_cast<const unsigned short *>(sp + i * 2);
                } else {
                    cw[mt][fn].c = *reinterpret_cast<const u32x4 *>(wp);
                    if constexpr (CODEC == Q4_0)
                        cw[mt][fn].d = *reinterpret_cast<const unsigned short *>(sp + lane * 2);
                    else if constexpr (CODEC == MLX4_G32)
                        cw[mt][fn].sb = *reinterpret_cast<const uint32_t *>(sp + lane * 4);
                    else
                        cw[mt][fn].sb = *reinterpret_cast<const uint32_t *>(sp + i * 4);
                }
            }
    };
    auto unpack = [&](const LaneCodes<CODEC>(&cw)[NMAT][FN], int s, f16x8(&wf)[NMAT][FN]) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                wf[mt][fn] = unpack_substep<CODEC>(cw[mt][fn], s, mg);
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

#pragma unroll
    for (int i = 0; i < AHEAD * KS; ++i)
        issue_stage(min(i, kq - 1), i);
    // With one wave per k-slice (NWT = 1) every wave's DMA writes and LDS
    // reads stay inside its own slice of each stage, and its own vmcnt wait
    // is all it needs: the k-loop then runs without workgroup barriers.
    wait_stage();
    if constexpr (NWT > 1)
        __syncthreads();
    LaneCodes<CODEC> cw[NMAT][FN];
    const int slice = wk * SLICE;
    read_w(lds + slice, cw);
    // Operands of sub-step 0 are prepared during sub-step 3 of the previous
    // k-step, so the k-step boundary (wait + barrier + first LDS reads and
    // unpack) overlaps matrix-core work instead of draining it.
    f16x8 xf[2][FM];
    f16x8 wf[2][NMAT][FN];
    read_x(lds + slice, 0, xf[0]);
    unpack(cw, 0, wf[0]);
    // one k-step; ST = t % NSLOT is a compile-time constant (the loop below
    // is unrolled by NSLOT), so every LDS slot address folds to a constant.
    // The first k-step of a stage issues the DMAs of the stage AHEAD on; the
    // last one waits for the next stage and ends with the barrier.
    auto kstep = [&](int t, auto stc) {
        constexpr int ST = decltype(stc)::value;
        if constexpr (ST % KS == 0) {
            // Without a barrier (one wave per k-slice) nothing else orders this
            // wave's reads of the slot it refills (read in the previous k-step)
            // before the refill's DMA writes: wait for them explicitly.  The
            // reads still in flight here are this step's sub-step 0 operands,
            // which its first MFMAs wait for anyway.
            if constexpr (NWT == 1)
                wait_lds_reads();
#pragma unroll
            for (int h = 0; h < KS; ++h)
                issue_stage(min(t + AHEAD * KS + h, kq - 1), (ST + AHEAD * KS + h) % NSLOT);
        }
        const char *sp = lds + ST * STAGE + slice;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cur = s & 1;
            if (s < 3) {
                read_x(sp, s + 1, xf[cur ^ 1]);
                unpack(cw, s + 1, wf[cur ^ 1]);
            } else {
                // at a stage's last k-step: the next stage has landed once at
                // most this wave's DMAs of the newest AHEAD-1 stages remain
                // (wait_stage); after the barrier nobody reads this stage again.
                // sched_barrier: sub-step 3's operands stay ahead of the wait.
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (ST % KS == KS - 1) {
                    wait_stage();
                    if constexpr (NWT > 1)
                        __syncthreads();
                }
                const char *np = lds + ((ST + 1) % NSLOT) * STAGE + slice;
                read_w(np, cw);
                read_x(np, 0, xf[cur ^ 1]);
                unpack(cw, 0, wf[cur ^ 1]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[mt][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][mt][fn], xf[cur][fm],
                                                                                 acc[mt][fm][fn], 0, 0, 0);
            constexpr int NMF = FM * FN * NMAT;
            constexpr int NV = (NMAT * FN * 16 + NMF - 1) / NMF;
#pragma unroll
            for (int j = 0; j < NMF; ++j) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, NV, 0);
                if (j < FM)
                    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
            }
        }
    };
    for (int t0 = 0; t0 < kq; t0 += NSLOT)
        static_for<NSLOT>([&](auto u) {
            if (t0 + int(decltype(u)::value) < kq)
                kstep(t0 + int(decltype(u)::value), u);
        });

    // ---- epilogue: fp16 tile staged in LDS, then whole-row 16-byte stores ----
    // The stores carry the non-temporal hint: Y is written once and not read
    // back here.  When every tile finishes in the same round (the 2048 x 2048
    // x 8192 prefill is 256 tiles), the whole of Y leaves in one burst after
    // the last k-step; with the hint that burst costs about 2 us of the
    // kernel instead of 4.5 (63.8 -> 61.6 us; the other prefill shapes gain
    // 2-3 us).  (The attention kernel's output measured slower with it.)
    wait_vmcnt<0>();
    __syncthreads();
    constexpr int CPR = BN / 8;                           // 16-byte chunks per tile row
    if constexpr (WK > 1) {
        // fp32 partial tile of each k-slice (gated: of the gate, then of the
        // up projection), then the fixed-order sum and, gated, the epilogue
        constexpr int PMAT = WK * BM * PPITCH;              // bytes of one matrix's partials
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int ml = wm * TM + fm * 32 + i;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = wn * TN + fn * 32 + 8 * q + 4 * g;
                        f32x4 v = {acc[mt][fm][fn][4 * q], acc[mt][fm][fn][4 * q + 1], acc[mt][fm][fn][4 * q + 2],
                                   acc[mt][fm][fn][4 * q + 3]};
                        *reinterpret_cast<f32x4 *>(lds + mt * PMAT + (wk * BM + ml) * PPITCH + nl * 4) = v;
                    }
            }
        __syncthreads();
        for (int idx = tid; idx < BM * CPR; idx += NT) {
            const int ml = idx / CPR, c = idx % CPR;
            const int m = m0 + ml, n = n0 + c * 8;
            if (m >= a.m || n >= a.n)
                continue;
            f32x4 lo[NMAT], hi[NMAT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const char *pp = lds + mt * PMAT + ml * PPITCH + c * 32;
                lo[mt] = *reinterpret_cast<const f32x4 *>(pp);
                hi[mt] = *reinterpret_cast<const f32x4 *>(pp + 16);
#pragma unroll
                for (int k = 1; k < WK; ++k) {
                    lo[mt] += *reinterpret_cast<const f32x4 *>(pp + k * BM * PPITCH);
                    hi[mt] += *reinterpret_cast<const f32x4 *>(pp + k * BM * PPITCH + 16);
                }
            }
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (GLU != 0) {
                    v[e] = glu_mul<GLU>(lo[0][e], lo[NMAT - 1][e]);
                    v[4 + e] = glu_mul<GLU>(hi[0][e], hi[NMAT - 1][e]);
                } else {
                    v[e] = lo[0][e];
                    v[4 + e] = hi[0][e];
                }
            }
            const f16x8 h = {_Float16(v[0]), _Float16(v[1]), _Float16(v[2]), _Float16(v[3]),
                             _Float16(v[4]), _Float16(v[5]), _Float16(v[6]), _Float16(v[7])};
            _Float16 *dst = out_at(a.y, a.ldy, a.head_dim, a.m, m, n);
            if (n + 7 < a.n) {
                __builtin_nontemporal_store(h, reinterpret_cast<f16x8 *>(dst));
            } else {
                for (int e = 0; e < 8 && n + e < a.n; ++e)
                    dst[e] = h[e];
            }
        }
        return;
    }
    static_assert(WK > 1 || CPR >= 16, "epilogue swizzle");
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int ml = wm * TM + fm * 32 + i;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * TN + fn * 32 + 8 * q + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (GLU != 0)
                        v[e] = glu_mul<GLU>(acc[0][fm][fn][4 * q + e], acc[1][fm][fn][4 * q + e]);
                    else
                        v[e] = acc[0][fm][fn][4 * q + e];
                }
                const f16x2 lo2 = {_Float16(v[0]), _Float16(v[1])};
                const f16x2 hi2 = {_Float16(v[2]), _Float16(v[3])};
                const int pc = (nl >> 3) ^ (ml & 15);
                *reinterpret_cast<u32x2 *>(lds + ml * (BN * 2) + pc * 16 + (nl & 4) * 2) = u32x2{as_u32(lo2), as_u32(hi2)};
            }
    }
    __syncthreads();
    for (int idx = tid; idx < BM * CPR; idx += NT) {
        const int ml = idx / CPR, c = idx % CPR;
        const int m = m0 + ml, n = n0 + c * 8;
        if (m >= a.m || n >= a.n)
            continue;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + ml * (BN * 2) + ((c ^ (ml & 15)) * 16));
        _Float16 *dst = out_at(a.y, a.ldy, a.head_dim, a.m, m, n);
        if (n + 7 < a.n) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
        } else {
            const f16x8 h = __builtin_bit_cast(f16x8, v);
            for (int e = 0; e < 8 && n + e < a.n; ++e)
                dst[e] = h[e];
        }
    }
}

template <int CODEC, int BM, int BN, int WM, int WN, int WK, int GLU, int NSTAGE, int KS = 1>
hipError_t launch_dma(const GemmProblem &p, hipStream_t stream)
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
    a.head_dim = int(p.head_dim);
    void *args[] = {&a};
    const dim3 grid(unsigned(a.tiles_m * a.tiles_n)), block(64 * WM * WN * WK);
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&gemm_dma_kernel<CODEC, BM, BN, WM, WN, WK, GLU, NSTAGE, KS>), grid, block,
        args, 0, stream);
}

template <int CODEC, int BM, int BN, int WM, int WN, int GLU>
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
    a.head_dim = int(p.head_dim);
    void *args[] = {&a};
    const dim3 grid(unsigned(a.tiles_m * a.tiles_n)), block(64 * WM * WN);
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<CODEC, BM, BN, WM, WN, GLU>), grid,
                           block, args, 0, stream);
}

// Gated kernels (glu 1 = SwiGLU, 2 = GeGLU) run with the gate and up
// projections in one workgroup.  M > 128: 128 x 256 tiles with the eight waves
// side by side along N (each 128 x 32 of both matrices), so every weight is
// unpacked by one wave and a k-step moves 25 KB by DMA; 256 x 128 tiles with
// 2 x 4 waves unpacked each weight twice and moved 36.5 KB (424 against 399 us
// on the 2048 x 4096 x 14336 SwiGLU).  M <= 128: the split-k small-M tile, as
// for the plain GEMM (both matrices' partial tiles summed in LDS before the
// gated epilogue), except Q8_0, whose two 2 KB code chunks per k-step and
// slice would need 198 KB of stages: it keeps the register-staged kernel.
//
// Plain kernels, M > 128: the eight waves sit side by side along N, so every
// weight is unpacked by one wave: 128 x 512 tiles (waves of 128 x 64) while
// they fill the chip, else 128 x 256 (waves of 128 x 32).  Per k-step a 128 x
// 512 tile moves 34 KB by DMA where a 256 x 256 tile with 2 x 4 waves of the
// same 128 x 64 moved 41 KB (64.1 -> 62.1 us for the 2048 x 2048 x 8192 Q4_0
// prefill); 128 x 256 against 256 x 128 with 2 x 4 waves took the 2048 x 4096 x
// 4096 Q2_0 prefill from 74.0 to 67.5 us.  The 128 x 256 tile's k-steps move
// less (25 KB), and two stages of two k-steps each -- half the barriers, the
// same lead -- measured faster there (Q2_0 61.4 -> 58.7 us, q-projection 65.8 ->
// 64.0 us), but not for 128 x 512 (57.9 -> 58.8 us) or the gated tiles.
// Plain kernels, M <= 128 (one or two 64-row tiles): 64 x 64 tiles with the
// k-steps split four ways inside the workgroup, one wave per k-slice, so that
// N / 64 tiles keep the SIMDs busy and the k-loop needs no barrier.  (The
// register-staged 128 x 128 kernel took 92 us for M = 65..128 on the 4096 x
// 14336 decode weight, this one 30-32 us; at M = 64 the barrier-free four waves
// take 15.1-15.4 us where eight waves, two per k-slice, took 15.9.)
template <int CODEC>
hipError_t launch_codec(const GemmProblem &p, const Choice &c, hipStream_t stream)
{
    switch (c.kern) {
    case Kern::DMA_WIDE: return launch_dma<CODEC, 128, 512, 1, 8, 1, 0, 3>(p, stream);
    case Kern::DMA_NARROW: return launch_dma<CODEC, 128, 256, 1, 8, 1, 0, 2, 2>(p, stream);
    case Kern::DMA_SMALL: return launch_dma<CODEC, 64, 64, 1, 1, 4, 0, 3>(p, stream);
    case Kern::GLU_DMA:
        return c.glu == 1 ? launch_dma<CODEC, 128, 256, 1, 8, 1, 1, 3>(p, stream)
                          : launch_dma<CODEC, 128, 256, 1, 8, 1, 2, 3>(p, stream);
    case Kern::GLU_DMA_SMALL:
        if constexpr (CODEC != Q8_0)
            return c.glu == 1 ? launch_dma<CODEC, 64, 64, 1, 2, 4, 1, 3>(p, stream)
                              : launch_dma<CODEC, 64, 64, 1, 2, 4, 2, 3>(p, stream);
        break;
    case Kern::GLU_REG_64:
        if constexpr (CODEC == Q8_0)
            return c.glu == 1 ? launch_tile<CODEC, 64, 64, 2, 2, 1>(p, stream)
                              : launch_tile<CODEC, 64, 64, 2, 2, 2>(p, stream);
        break;
    case Kern::GLU_REG_128:
        if constexpr (CODEC == Q8_0)
            return c.glu == 1 ? launch_tile<CODEC, 128, 128, 2, 2, 1>(p, stream)
                              : launch_tile<CODEC, 128, 128, 2, 2, 2>(p, stream);
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmProblem &p, const Choice &c, hipStream_t stream)
{
    switch (p.codec) {
    case Q4_0: return launch_codec<Q4_0>(p, c, stream);
    case MLX4_G64: return launch_codec<MLX4_G64>(p, c, stream);
    case MLX4_G32: return launch_codec<MLX4_G32>(p, c, stream);
    case Q2_0: return launch_codec<Q2_0>(p, c, stream);
    case Q8_0: return launch_codec<Q8_0>(p, c, stream);
    case Q4_K: return launch_codec<Q4_K>(p, c, stream);
    case TERNARY: return launch_codec<TERNARY>(p, c, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
