// C-ABI entry points: argument validation, then one asynchronous launch on the
// caller's stream.  Nothing is launched when an argument is rejected.
#include "../../include/qgemm.h"
#include "launch.h"

using namespace qg;

namespace {

constexpr int64_t LIMIT = int64_t(1) << 31;   // bytes per buffer, and M/N/K

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_codec(int32_t c)
{
    return c == Q4_0 || c == MLX4_G64 || c == Q2_0 || c == Q8_0 || c == MLX4_G32 || c == Q4_K || c == TERNARY ||
           c == TERNARY_Q2;
}

qg_status check_weight(const qg_weight *w)
{
    if (!w || !w->qs || !w->scales)
        return QG_ERR_NULL;
    if (!valid_codec(w->codec))
        return QG_ERR_CODEC;
    if (w->flags != 0 || w->n < 1 || w->k < 1 || w->n >= LIMIT || w->k >= LIMIT ||
        w->k % block_size(w->codec) != 0)
        return QG_ERR_SHAPE;
    const Geometry g = geometry(w->codec, w->n, w->k);
    if (g.qs_bytes >= LIMIT || g.scale_bytes >= LIMIT)
        return QG_ERR_SHAPE;
    if (!aligned16(w->qs) || !aligned16(w->scales))
        return QG_ERR_ALIGN;
    return QG_OK;
}

qg_status check_act(const void *p, int64_t rows, int64_t cols, int64_t ld)
{
    if (!p)
        return QG_ERR_NULL;
    // kernels form 32-bit byte offsets up to one 256-row tile past the last row
    if (rows < 1 || rows >= LIMIT || ld < cols || ld >= LIMIT || ((rows - 1) * ld + cols) * 2 >= LIMIT ||
        (rows + 256) * ld * 2 >= (int64_t(1) << 32))
        return QG_ERR_SHAPE;
    if (!aligned16(p) || ld % 8 != 0)
        return QG_ERR_ALIGN;
    return QG_OK;
}

Planes planes_of(const qg_weight *w)
{
    const Geometry g = geometry(w->codec, w->n, w->k);
    Planes p;
    p.qs = static_cast<const uint8_t *>(w->qs);
    p.scales = w->scales;
    p.qs_bytes = uint32_t(g.qs_bytes);
    p.scale_bytes = uint32_t(g.scale_bytes);
    return p;
}

GemmProblem problem(const qg_weight *w, const void *x, int64_t m, int64_t ldx, void *y, int64_t ldy)
{
    const Geometry g = geometry(w->codec, w->n, w->k);
    GemmProblem p;
    p.codec = kernel_codec(w->codec);
    p.w0 = planes_of(w);
    p.w1 = p.w0;
    p.x = static_cast<const _Float16 *>(x);
    p.y = static_cast<_Float16 *>(y);
    p.m = m;
    p.n = w->n;
    p.k = w->k;
    p.ldx = ldx;
    p.ldy = ldy;
    p.groups = g.groups;
    p.ksteps = g.ksteps;
    p.kb128 = w->k / 128;
    return p;
}

qg_status launched(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH; }

bool finite_positive(float v) { return v > 0.0f && v <= 3.4e38f; }

// The kernel choose_kernel picks for the call, launched on the stream.
hipError_t run(const GemmProblem &p, int glu, bool gemv_entry, hipStream_t stream)
{
    const Choice c = choose_kernel(p.codec, glu, gemv_entry, p.m, p.n, p.k);
    return c.kern == Kern::GEMV ? launch_gemv(p, c, stream) : launch_gemm(p, c, stream);
}

qg_status check_gemm(const qg_weight *w, const void *x, int64_t m, int64_t ldx, void *y, int64_t ldy)
{
    qg_status st = check_weight(w);
    if (st != QG_OK)
        return st;
    if ((st = check_act(x, m, w->k, ldx)) != QG_OK)
        return st;
    return check_act(y, m, w->n, ldy);
}

}  // namespace

extern "C" {

qg_status qgemm_prefill(const qg_weight *w, const void *x, int64_t m, int64_t ldx, void *y, int64_t ldy,
                        void *stream)
{
    const qg_status st = check_gemm(w, x, m, ldx, y, ldy);
    if (st != QG_OK)
        return st;
    return launched(run(problem(w, x, m, ldx, y, ldy), 0, true, static_cast<hipStream_t>(stream)));
}

qg_status qgemm_prefill_heads(const qg_weight *w, const void *x, int64_t m, int64_t ldx, void *y, int64_t head_dim,
                              void *stream)
{
    qg_status st = check_weight(w);
    if (st != QG_OK)
        return st;
    if (head_dim < 8 || head_dim % 8 != 0 || w->n % head_dim != 0)
        return QG_ERR_SHAPE;
    // y holds M x N elements: validated as a dense [M, N] buffer
    if ((st = check_gemm(w, x, m, ldx, y, w->n)) != QG_OK)
        return st;
    GemmProblem p = problem(w, x, m, ldx, y, w->n);
    p.head_dim = head_dim;
    return launched(run(p, 0, true, static_cast<hipStream_t>(stream)));
}

// gate/up projection pair with a gated epilogue (glu 1 = SwiGLU, 2 = GeGLU)
static qg_status gated(const qg_weight *wg, const qg_weight *wu, const void *x, int64_t m, int64_t ldx, void *out,
                       int64_t ldo, void *stream, int glu)
{
    qg_status st = check_gemm(wg, x, m, ldx, out, ldo);
    if (st != QG_OK)
        return st;
    if ((st = check_weight(wu)) != QG_OK)
        return st;
    if (wu->codec != wg->codec || wu->n != wg->n || wu->k != wg->k)
        return QG_ERR_MISMATCH;
    GemmProblem p = problem(wg, x, m, ldx, out, ldo);
    p.w1 = planes_of(wu);
    return launched(run(p, glu, false, static_cast<hipStream_t>(stream)));
}

qg_status qgemm_swiglu(const qg_weight *wg, const qg_weight *wu, const void *x, int64_t m, int64_t ldx, void *out,
                       int64_t ldo, void *stream)
{
    return gated(wg, wu, x, m, ldx, out, ldo, stream, 1);
}

qg_status qgemm_geglu(const qg_weight *wg, const qg_weight *wu, const void *x, int64_t m, int64_t ldx, void *out,
                      int64_t ldo, void *stream)
{
    return gated(wg, wu, x, m, ldx, out, ldo, stream, 2);
}

qg_status qgemv_decode(const qg_weight *w, const void *x, int64_t m, int64_t ldx, void *y, int64_t ldy,
                       void *stream)
{
    const qg_status st = check_gemm(w, x, m, ldx, y, ldy);
    if (st != QG_OK)
        return st;
    if (m > 64)
        return QG_ERR_SHAPE;
    return launched(run(problem(w, x, m, ldx, y, ldy), 0, true, static_cast<hipStream_t>(stream)));
}

qg_status qg_dequant(const qg_weight *w, void *w_fp16, int64_t ldw, void *stream)
{
    qg_status st = check_weight(w);
    if (st != QG_OK)
        return st;
    if ((st = check_act(w_fp16, w->n, w->k, ldw)) != QG_OK)
        return st;
    const GemmProblem p = problem(w, nullptr, 1, w->k, nullptr, w->n);
    return launched(launch_dequant(p, static_cast<_Float16 *>(w_fp16), ldw, static_cast<hipStream_t>(stream)));
}

qg_status qg_kernel_for(int32_t entry, int32_t codec, int64_t m, int64_t n, int64_t k, char *name, size_t cap)
{
    if (!name || cap == 0)
        return QG_ERR_NULL;
    if (!valid_codec(codec))
        return QG_ERR_CODEC;
    if (entry < E_PREFILL || entry > E_GEMV || m < 1 || n < 1 || k < 1 || m >= LIMIT || n >= LIMIT || k >= LIMIT ||
        k % block_size(codec) != 0 || (entry == E_GEMV && m > 64))
        return QG_ERR_SHAPE;
    const int glu = entry == E_SWIGLU ? 1 : entry == E_GEGLU ? 2 : 0;
    const int kc = kernel_codec(codec);
    const Choice c = choose_kernel(kc, glu, glu == 0, m, n, k);
    const int len = kernel_name(c, kc, name, cap);
    return (len > 0 && size_t(len) < cap) ? QG_OK : QG_ERR_SIZE;
}

qg_status qg_stream_read(const void *src, size_t bytes, uint32_t *out, void *stream)
{
    if (!src || !out)
        return QG_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || bytes >= size_t(LIMIT))
        return QG_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(out))
        return QG_ERR_ALIGN;
    return launched(launch_stream_read(src, bytes, out, static_cast<hipStream_t>(stream)));
}

qg_status qattn_prefill_q8kv(const void *q, void *o, int64_t heads, int64_t m, int64_t head_dim,
                             const void *k_codes, const void *k_scales, const void *v_codes, const void *v_scales,
                             int64_t kv_heads, int64_t s, int32_t causal, float scale, void *stream)
{
    if (!q || !o || !k_codes || !k_scales || !v_codes || !v_scales)
        return QG_ERR_NULL;
    if ((head_dim != 64 && head_dim != 128) || heads < 1 || heads > 65535 || kv_heads < 1 || heads % kv_heads != 0 ||
        m < 1 || s < m || (causal != 0 && causal != 1) || !finite_positive(scale))
        return QG_ERR_SHAPE;
    if (heads * m * head_dim * 2 >= LIMIT || kv_heads * s * head_dim >= LIMIT)
        return QG_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(o) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) ||
        !aligned16(v_scales))
        return QG_ERR_ALIGN;
    AttnProblem p;
    p.q = static_cast<const _Float16 *>(q);
    p.o = static_cast<_Float16 *>(o);
    p.k_codes = static_cast<const uint8_t *>(k_codes);
    p.v_codes = static_cast<const uint8_t *>(v_codes);
    p.k_scales = static_cast<const _Float16 *>(k_scales);
    p.v_scales = static_cast<const _Float16 *>(v_scales);
    p.heads = heads;
    p.m = m;
    p.head_dim = head_dim;
    p.kv_heads = kv_heads;
    p.s = s;
    p.causal = causal != 0;
    p.scale = scale;
    return launched(launch_attention(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
