// Kernel selection (host).  Every launcher asks choose_kernel which kernel
// instantiation serves a call, and qg_kernel_for reports the same choice by
// name, so the host can tell -- without a GPU -- which instantiations a set
// of shapes reaches.
//
// Pages: releases page v0.3.0 (the quantized linear layer picks a GEMV for
// M = 1 and a GEMM otherwise, for every codec); comparison page section 2.2
// (the gate/up pair is one fused kernel).
#pragma once
#include <stdint.h>
#include <stdio.h>

#include "planar.h"

namespace qg {

// Call sites of the C-ABI that reach a GEMM / GEMV kernel.
enum Entry : int32_t { E_PREFILL = 0, E_HEADS = 1, E_SWIGLU = 2, E_GEGLU = 3, E_GEMV = 4 };

enum class Kern : int32_t {
    GEMV,              // gemv_kernel<CODEC, MM>, MM = 1, 2 or 4 rows
    DMA_WIDE,          // gemm_dma_kernel 128 x 512, eight waves of 128 x 64
    DMA_NARROW,        // gemm_dma_kernel 128 x 256, eight waves of 128 x 32, stages of two k-steps
    DMA_SMALL,         // gemm_dma_kernel 64 x 64, k split over four waves
    GLU_DMA,           // gemm_dma_kernel 128 x 256 gated
    GLU_DMA_SMALL,     // gemm_dma_kernel 64 x 64 gated, k split over four pairs of waves
    GLU_REG_64,        // gemm_kernel 64 x 64 gated (register-staged)
    GLU_REG_128,       // gemm_kernel 128 x 128 gated (register-staged)
};

struct Choice {
    Kern kern;
    int mm;    // GEMV rows (1, 2, 4)
    int glu;   // 0 none, 1 SwiGLU, 2 GeGLU
};

constexpr int GEMV_NW = 8;                  // waves per GEMV workgroup
constexpr int64_t GEMV_X_LDS_MAX = 64 * 1024;   // largest staged X (MM x K fp16) the GEMV takes
constexpr int64_t GEMV_LDS_MAX = 64 * 1024;     // dynamic LDS of one GEMV workgroup, at most

inline int gemv_rows(int64_t m) { return m == 1 ? 1 : m == 2 ? 2 : 4; }

// LDS layout of one GEMV workgroup: X (whole 1 KB DMA rows), the per-slice X
// corrections, the wave partial sums.
struct GemvLds {
    int x_lds;
    int64_t bytes;
};
inline GemvLds gemv_lds(int codec, int64_t mm, int64_t ksteps)
{
    GemvLds l;
    l.x_lds = int((mm * ksteps * 128 + 1023) / 1024 * 1024);
    const int64_t nc = is_mlx(codec) || codec == Q4_K ? 2 : 1;
    l.bytes = l.x_lds + mm * ksteps * 2 * nc * 4 + GEMV_NW * mm * 32 * 4;
    return l;
}

inline bool gemv_fits(int codec, int64_t m, int64_t ksteps)
{
    const int64_t mm = gemv_rows(m);
    return m <= 4 && mm * ksteps * 128 <= GEMV_X_LDS_MAX && gemv_lds(codec, mm, ksteps).bytes <= GEMV_LDS_MAX;
}

constexpr int64_t FILL = 256;   // compute units on MI355X

// glu: 0 for plain projections.  gemv_entry: qgemv_decode, or qgemm_prefill /
// qgemm_prefill_heads with M <= 4 (both take the weight-streaming kernel when
// X fits its LDS).
inline Choice choose_kernel(int codec, int glu, bool gemv_entry, int64_t m, int64_t n, int64_t k)
{
    const int64_t ksteps = ceil_div(k, QG_KSTEP);
    Choice c{Kern::DMA_SMALL, 0, glu};
    if (glu == 0 && gemv_entry && gemv_fits(codec, m, ksteps)) {
        c.kern = Kern::GEMV;
        c.mm = gemv_rows(m);
        return c;
    }
    if (glu != 0) {
        if (m > 128)
            c.kern = Kern::GLU_DMA;
        else if (codec != Q8_0)
            c.kern = Kern::GLU_DMA_SMALL;
        else   // Q8_0's two 2 KB code chunks per k-step and slice would need 198 KB of stages
            c.kern = m > 64 ? Kern::GLU_REG_128 : Kern::GLU_REG_64;
        return c;
    }
    if (m > 128)
        c.kern = ceil_div(m, 128) * ceil_div(n, 512) >= FILL ? Kern::DMA_WIDE : Kern::DMA_NARROW;
    else
        c.kern = Kern::DMA_SMALL;
    return c;
}

// The kernel's name as a kernel trace prints it (template arguments in
// order, codec as its number).
inline int kernel_name(const Choice &c, int codec, char *buf, size_t cap)
{
    switch (c.kern) {
    case Kern::GEMV: return snprintf(buf, cap, "gemv_kernel<%d, %d>", codec, c.mm);
    case Kern::DMA_WIDE: return snprintf(buf, cap, "gemm_dma_kernel<%d, 128, 512, 1, 8, 1, 0, 3, 1>", codec);
    case Kern::DMA_NARROW: return snprintf(buf, cap, "gemm_dma_kernel<%d, 128, 256, 1, 8, 1, 0, 2, 2>", codec);
    case Kern::DMA_SMALL: return snprintf(buf, cap, "gemm_dma_kernel<%d, 64, 64, 1, 1, 4, 0, 3, 1>", codec);
    case Kern::GLU_DMA: return snprintf(buf, cap, "gemm_dma_kernel<%d, 128, 256, 1, 8, 1, %d, 3, 1>", codec, c.glu);
    case Kern::GLU_DMA_SMALL: return snprintf(buf, cap, "gemm_dma_kernel<%d, 64, 64, 1, 2, 4, %d, 3, 1>", codec, c.glu);
    case Kern::GLU_REG_64: return snprintf(buf, cap, "gemm_kernel<%d, 64, 64, 2, 2, %d>", codec, c.glu);
    case Kern::GLU_REG_128: return snprintf(buf, cap, "gemm_kernel<%d, 128, 128, 2, 2, %d>", codec, c.glu);
    }
    return snprintf(buf, cap, "?");
}

}  // namespace qg
