// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dispatch.h"
#include "unpack.h"

namespace qg {

struct GemmProblem {
    int codec;
    Planes w0, w1;             // w1: up projection for the fused SwiGLU
    const _Float16 *x;
    _Float16 *y;
    int64_t m, n, k, ldx, ldy;
    int64_t groups, ksteps, kb128;
    int64_t head_dim = 0;      // > 0: Y is written head-major [N / head_dim, M, head_dim]
};

// Address of output element (m, n): row-major [M, ldy], or, with head_dim = D
// > 0, the direct-head layout [N / D, M, D] (element (m, h D + d) at
// (h M + m) D + d).  Callers pass n at a multiple of the store width, which
// divides D, so a store never crosses heads.
__device__ __forceinline__ _Float16 *out_at(_Float16 *y, int ldy, int head_dim, int rows, int m, int n)
{
    if (head_dim == 0)
        return y + int64_t(m) * ldy + n;
    const int h = n / head_dim;
    return y + (int64_t(h) * rows + m) * head_dim + (n - h * head_dim);
}

// Tiled MFMA kernels (every choice but Kern::GEMV).  Return a hipError_t of the launch.
hipError_t launch_gemm(const GemmProblem &p, const Choice &c, hipStream_t stream);
// Weight-streaming kernel (Kern::GEMV, 1 <= m <= 4).
hipError_t launch_gemv(const GemmProblem &p, const Choice &c, hipStream_t stream);
// fp16 image of the weights, [n, ldw].
hipError_t launch_dequant(const GemmProblem &p, _Float16 *out, int64_t ldw, hipStream_t stream);
// Plain streaming read of `bytes` (a multiple of 16) bytes; XOR checksum into *out.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, hipStream_t stream);

// Attention over a Q8_0 KV cache: Q, O [heads, m, head_dim] fp16; K, V as int8
// codes [kv_heads * s, head_dim] and fp16 scales [kv_heads * s, head_dim / 32].
struct AttnProblem {
    const _Float16 *q;
    _Float16 *o;
    const uint8_t *k_codes, *v_codes;
    const _Float16 *k_scales, *v_scales;
    int64_t heads, m, head_dim, kv_heads, s;
    bool causal;
    float scale;
};
hipError_t launch_attention(const AttnProblem &p, hipStream_t stream);

}  // namespace qg
