/*
 * qgemm.h -- C-ABI of the MI355X (gfx950) quantized prefill GEMM library.
 *
 * Y = X * W^T where X holds fp16 activations [M, K] and W is a block-quantized
 * weight matrix [N, K] whose codes are dequantized inside the kernels and
 * contracted on the fp16 matrix cores with fp32 accumulation.
 *
 * Sources (m4-prefill-engine pages):
 *  - comparison page, section 2.1: quantized GEMM on matrix units fed by
 *    in-kernel dequantization; section 2.2: fused SiLU(Gate) x Up with X loaded
 *    once and the gate / up products kept on chip; section 4: planar 16-byte
 *    aligned code arrays read with 128-bit loads.
 *  - releases page, v0.3.0: a C-ABI bridge over caller-owned device buffers;
 *    a quantized linear layer that dispatches GEMV (M = 1) or GEMM (M > 1) for
 *    every codec; PrismML Q2_0 codec (128 weights, 34 bytes, w = (q - 1) d,
 *    q = 3 -> +2d).
 *  - project index, Table B: block_q4_0 (GGUF Q4_0) and block_mlx_4bit weights.
 *
 * Conventions shared by every entry point
 *  - Pointers marked "device" are HIP device pointers; "host" ones are CPU
 *    memory.  The caller owns every buffer.  The library allocates nothing,
 *    keeps no pointer after a call returns and holds no mutable global state.
 *  - Compute entry points enqueue work on `stream` (a hipStream_t; NULL is the
 *    default stream) and return without synchronising.  A kernel fault shows
 *    up at the caller's next synchronisation, as for any HIP launch.
 *  - Errors are status codes; nothing is thrown across the ABI.  Argument
 *    errors are detected before any launch, and then nothing is launched.
 *  - Activations and outputs are row-major binary16.  Row strides are in
 *    elements and must be multiples of 8 (16-byte rows); the base pointers of
 *    x, y and of both weight planes must be 16-byte aligned.
 *  - Each of x, y and the weight planes must span less than 2 GiB, and M, N
 *    and K must be below 2^31 (QG_ERR_SHAPE otherwise).
 *  - Weights are in the library's planar device format, produced from the
 *    canonical codec bytes by qg_pack_host and sized by qg_packed_sizes.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight codecs.  Canonical byte formats (the input of qg_pack_host):
 *  QG_CODEC_Q4_0     32-weight blocks of 18 bytes: fp16 d (little-endian),
 *                    then 16 bytes, byte j = weight j (low nibble) and weight
 *                    j + 16 (high nibble); w = (q - 8) * d.
 *  QG_CODEC_MLX4_G64 codes as little-endian uint32 words [N, K/8] (element 0
 *                    in the low nibble), then fp16 scales [N, K/64], then fp16
 *                    biases [N, K/64]; w = q * s + b per 64-weight group.
 *  QG_CODEC_Q2_0     128-weight blocks of 34 bytes: fp16 d, then 32 bytes of
 *                    2-bit codes, weight i in byte i/4 at bit 2*(i%4);
 *                    w = (q - 1) * d, so q = 3 gives +2d.
 *  QG_CODEC_MLX4_G32 as QG_CODEC_MLX4_G64 with one fp16 scale and bias per 32
 *                    weights ([N, K/32] each): the group of the pages'
 *                    20-byte block_mlx_4bit (comparison page, section 4).
 *  QG_CODEC_Q8_0     32-weight blocks of 34 bytes: fp16 d, then weight j as
 *                    the two's-complement byte 2 + j; w = q * d.  (Q8_0 is in
 *                    the quantization registry of the releases page, v0.3.0;
 *                    the byte layout is GGUF's block_q8_0.)
 *  QG_CODEC_Q4_K     256-weight super-blocks of 144 bytes: fp16 d, fp16 dmin,
 *                    12 bytes of eight 6-bit sub-block scales sc[j] and mins
 *                    m[j], then 128 code bytes in four 32-byte runs (byte l
 *                    of run u: weight 64u + l in the low nibble, 64u + 32 + l
 *                    in the high); w = d * sc[j] * q - dmin * m[j] over
 *                    sub-block j = weights 32j .. 32j + 31.  (The pages list
 *                    "Q4_K (GGUF Super-Blocks)" among the router's formats,
 *                    releases page v0.2; the layout is the public GGUF one.)
 *  QG_CODEC_TERNARY_1_58  256-weight blocks of 54 bytes: fp16 d, then byte
 *                    2 + j holds weights 5j .. 5j + 4 as base-3 digits t
 *                    (weight 5j + i contributes t * 3^i; weight 255 is digit
 *                    0 of byte 53); w = (t - 1) * d, so -d, 0 or +d.  Bytes
 *                    above 242 (byte 53: above 2) are invalid (QG_ERR_CODE).
 *                    (BitNet ternary: releases page v0.2, router formats;
 *                    TERNARY_1_58 in the v0.3.0 registry.  The pages give no
 *                    packing; 1.6875 bits per weight.)
 *  QG_CODEC_TERNARY_1_58_Q2  the same canonical bytes as QG_CODEC_TERNARY_1_58,
 *                    held on the device as 2-bit codes q = t with each block's
 *                    d repeated per 128 weights -- the QG_CODEC_Q2_0 planar
 *                    format (w = (q - 1) d), run by the Q2_0 kernels.  2.125
 *                    bits per weight in device memory instead of 1.625 + 1/16,
 *                    in exchange for a decode without base-3 arithmetic (the
 *                    pages' question whether a ternary codec's byte saving
 *                    survives its decode cost: releases page v0.2). */
typedef enum {
    QG_CODEC_Q4_0 = 1,
    QG_CODEC_MLX4_G64 = 2,
    QG_CODEC_Q2_0 = 3,
    QG_CODEC_Q8_0 = 4,
    QG_CODEC_MLX4_G32 = 5,
    QG_CODEC_Q4_K = 6,
    QG_CODEC_TERNARY_1_58 = 7,
    QG_CODEC_TERNARY_1_58_Q2 = 8
} qg_codec;

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = -1,      /* a required pointer is NULL                       */
    QG_ERR_CODEC = -2,     /* unknown codec id                                 */
    QG_ERR_SHAPE = -3,     /* M/N/K out of range, K not a multiple of the block,
                              stride smaller than the row, M > 64 for a GEMV,
                              a buffer of 2 GiB or more, flags != 0           */
    QG_ERR_ALIGN = -4,     /* pointer or stride not 16-byte aligned            */
    QG_ERR_MISMATCH = -5,  /* gate/up descriptors differ in codec, N or K      */
    QG_ERR_LAUNCH = -6,    /* the HIP launch itself failed                     */
    QG_ERR_SIZE = -7,      /* a host buffer is smaller than the format needs   */
    QG_ERR_CODE = -8       /* a canonical code byte outside the codec's range  */
} qg_status;

/* A packed weight matrix W [n, k] in the planar device format.
 *  qs      device, code plane (qs_bytes from qg_packed_sizes)
 *  scales  device, scale plane (scale_bytes): fp16 d for Q4_0 and Q2_0; for
 *          MLX4-G64 each entry is the pair (fp16 scale, fp16 bias)
 *  flags   must be 0 (reserved for layout variants)
 * The descriptor itself is host memory and is only read during the call. */
typedef struct {
    int32_t codec;
    int32_t flags;
    int64_t n;
    int64_t k;
    const void *qs;
    const void *scales;
} qg_weight;

/* Prefill projection Y[m, n] = sum_k X[m, k] * W[n, k]  (Y = X W^T): the
 * quantized GEMM of prompt prefill, weights dequantized inside the kernel and
 * fed to the matrix cores (comparison page, section 2.1; project index,
 * Pillar 1, Brick 1).
 *  w    host descriptor of W [N, K]
 *  x    device fp16 [m, ldx], rows of K used       (m >= 1, ldx >= K)
 *  y    device fp16 [m, ldy], first N columns written (ldy >= N)
 * Dequantization happens inside the kernel; products accumulate in fp32 and
 * are rounded once to fp16 (nearest even).  Any M >= 1 is accepted; small M
 * is served by the weight-streaming kernel of qgemv_decode. */
qg_status qgemm_prefill(const qg_weight *w, const void *x, int64_t m, int64_t ldx,
                        void *y, int64_t ldy, void *stream);

/* The same projection written in the direct-head layout [H, M, D]: output
 * element (m, h D + d) goes to y[(h M + m) D + d], so per-head Q, K or V
 * tiles come out ready for attention with no transposition pass (comparison
 * page, section 4, and releases page, v0.2.1: "Direct-Head Multi-Head
 * Layout").
 *  head_dim  D: a multiple of 8 that divides N (else QG_ERR_SHAPE)
 *  y         device fp16, M * N contiguous elements, 16-byte aligned
 * Other arguments and errors as for qgemm_prefill. */
qg_status qgemm_prefill_heads(const qg_weight *w, const void *x, int64_t m, int64_t ldx,
                              void *y, int64_t head_dim, void *stream);

/* Fused gate/up projection with the SwiGLU epilogue (comparison page, section
 * 2.2): out[m, n] = SiLU(g) * u with g = (X Wg^T)[m, n], u = (X Wu^T)[m, n],
 * SiLU(g) = g / (1 + exp(-g)), evaluated in fp32 on the accumulators and
 * rounded once to fp16.  Gate and up never reach device memory.
 *  wg, wu  host descriptors with equal codec, N and K (else QG_ERR_MISMATCH)
 *  x       device fp16 [m, ldx];  out  device fp16 [m, ldo] */
qg_status qgemm_swiglu(const qg_weight *wg, const qg_weight *wu, const void *x,
                       int64_t m, int64_t ldx, void *out, int64_t ldo, void *stream);

/* Fused gate/up projection with the GeGLU epilogue: the SwiGLU entry point
 * with GELU in place of SiLU (releases page, v0.3.0, TransformerBlock: SwiGLU /
 * GeGLU activations).  GELU is the tanh form used by the Gemma family that
 * page names: GELU(g) = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))),
 * evaluated in fp32 on the accumulators and rounded once to fp16.  Arguments,
 * layouts and errors as for qgemm_swiglu. */
qg_status qgemm_geglu(const qg_weight *wg, const qg_weight *wu, const void *x,
                      int64_t m, int64_t ldx, void *out, int64_t ldo, void *stream);

/* Weight-streaming small-M projection (decode, M = 1, and speculative
 * verification of up to 64 candidate rows): Y = X W^T as for qgemm_prefill,
 * for 1 <= m <= 64 (else QG_ERR_SHAPE).  Each weight byte is read from device
 * memory once per call.  (Releases page v0.3.0: the quantized linear layer
 * takes a GEMV path for M = 1; comparison page section 2.4 and project index
 * Pillar 4: up to 64 draft tokens verified in one pass over the weights, whose
 * time is the weight bytes over the memory bandwidth.) */
qg_status qgemv_decode(const qg_weight *w, const void *x, int64_t m, int64_t ldx,
                       void *y, int64_t ldy, void *stream);

/* Byte sizes of the two planar planes of an [n, k] matrix of `codec` (N is
 * padded to 32 rows and K to 64 weights inside the planes; the padding decodes
 * to zero).  Either out-pointer may be NULL.  (The planar split of codes and
 * scales into separate 16-byte aligned arrays: comparison page, section 4.)
 * Errors: QG_ERR_CODEC, QG_ERR_SHAPE (K not a multiple of the block). */
qg_status qg_packed_sizes(int32_t codec, int64_t n, int64_t k, size_t *qs_bytes,
                          size_t *scales_bytes);

/* Size of the canonical encoding of an [n, k] matrix (see qg_codec). */
qg_status qg_canonical_size(int32_t codec, int64_t n, int64_t k, size_t *bytes);

/* Host-side repack of canonical codec bytes into the planar device format
 * (comparison page, section 4: codes split from scales into 16-byte aligned
 * planes).  Bit moves only; every code, scale and bias keeps its value.
 *  canonical   host, canonical_bytes long (checked: QG_ERR_SIZE); ternary
 *              code bytes are range-checked first (QG_ERR_CODE, nothing written)
 *  qs, scales  host outputs of the sizes from qg_packed_sizes; fully written
 * Padding rows and columns get zero scales so that they decode to zero. */
qg_status qg_pack_host(int32_t codec, int64_t n, int64_t k, const void *canonical,
                       size_t canonical_bytes, void *qs, void *scales);

/* Dequantize W into fp16 w_fp16 [n, ldw] (device) with the same per-codec
 * unpack routines the GEMM kernels feed to the matrix cores; each weight is the
 * binary16 value nearest its exact codec value.  For verification: the pages
 * check every codec's unpack bit for bit before and after each kernel change
 * (releases page v0.2.3, bit-exact parity suite; the shared unpack contract
 * TCodec::unpack_column).
 *  w_fp16  device fp16 [n, ldw], ldw >= K, a multiple of 8; 16-byte aligned
 * Errors as for qgemm_prefill. */
qg_status qg_dequant(const qg_weight *w, void *w_fp16, int64_t ldw, void *stream);

/* Name of the kernel instantiation a call would launch, as a kernel trace
 * prints it (host only; launches nothing).  entry: 0 qgemm_prefill,
 * 1 qgemm_prefill_heads, 2 qgemm_swiglu, 3 qgemm_geglu, 4 qgemv_decode.  The
 * launchers take their choice from the same function, so tests can show which
 * instantiations a set of shapes reaches (releases page v0.2.3: every codec
 * is checked at each boundary token count the dispatch distinguishes).
 *  name  host buffer of cap bytes, NUL-terminated on success
 * Errors: QG_ERR_NULL, QG_ERR_CODEC, QG_ERR_SHAPE (the entry point would reject
 * these sizes), QG_ERR_SIZE (cap too small). */
qg_status qg_kernel_for(int32_t entry, int32_t codec, int64_t m, int64_t n, int64_t k, char *name,
                        size_t cap);

/* Streaming-read calibration (not part of the GEMM path): reads every byte of
 * src once, with the same 128-bit non-temporal loads the GEMV uses.  It
 * measures the sustained HBM read rate one kernel achieves for a given byte
 * count on the device at hand -- the practical ceiling against which the
 * weight-streaming GEMV is compared (project index Pillar 4: decode time is
 * bytes streamed over bandwidth).  Each of QG_STREAM_READ_SLOTS waves XORs the
 * XOR of the 32-bit words it read into its own slot of out, so with out
 * zeroed beforehand the XOR over all slots is the XOR of all words of src.
 *  src    device, 16-byte aligned, bytes a positive multiple of 16, < 2 GiB
 *  out    device uint32 [QG_STREAM_READ_SLOTS], 16-byte aligned, read and written
 * Errors: QG_ERR_NULL, QG_ERR_SHAPE, QG_ERR_ALIGN, QG_ERR_LAUNCH. */
#define QG_STREAM_READ_SLOTS 4096
qg_status qg_stream_read(const void *src, size_t bytes, uint32_t *out, void *stream);

/* Attention over a Q8_0-compressed KV cache, prefill (comparison page section
 * 2.3 and project index Brick 4: a FlashAttention core with online softmax
 * whose K and V are dequantized from the Q8_0 cache as they are read; releases
 * page v0.2.3: D in {64, 128}; releases page v0.3.0: grouped-query attention
 * and causal masking).  For each query head h with KV head g = h / (heads /
 * kv_heads):
 *     O[h, i] = sum_t softmax_t(scale * Q[h, i] . K[g, t]) V[g, t]
 * over the keys t < s, and with causal != 0 only t <= (s - m) + i (the m
 * queries are the last m of the s positions).  K and V elements are the
 * binary16 values nearest q * d (the Q8_0 rule of QG_CODEC_Q8_0); scores,
 * softmax and sums are fp32, P is rounded to fp16 for the second product.
 *  q         device fp16 [heads, m, head_dim] (the direct-head layout of
 *            qgemm_prefill_heads), 16-byte aligned
 *  o         device fp16 [heads, m, head_dim], written; 16-byte aligned
 *  k_codes   device uint8 [kv_heads * s, head_dim], q + 128 for the Q8_0 code q
 *            (as qg_pack_kv_host writes them)
 *  k_scales  device fp16 [kv_heads * s, head_dim / 32] (d of each 32 codes)
 *  v_codes, v_scales  the same for V; all four 16-byte aligned
 *  head_dim  64 or 128;  1 <= heads <= 65535, heads % kv_heads == 0;
 *  1 <= m <= s;  causal 0 or 1;  scale > 0 and finite (usually 1/sqrt(D))
 * Buffers must stay below 2 GiB.  Errors: QG_ERR_NULL, QG_ERR_SHAPE,
 * QG_ERR_ALIGN, QG_ERR_LAUNCH; nothing is launched on an argument error. */
qg_status qattn_prefill_q8kv(const void *q, void *o, int64_t heads, int64_t m, int64_t head_dim,
                             const void *k_codes, const void *k_scales, const void *v_codes,
                             const void *v_scales, int64_t kv_heads, int64_t s, int32_t causal,
                             float scale, void *stream);

/* Host-side split of canonical Q8_0 rows (GGUF block_q8_0: fp16 d then 32
 * int8 codes, per 32 elements of a row) into the planar KV cache format of
 * qattn_prefill_q8kv: codes [rows, head_dim] as the unsigned bytes q + 128
 * (the sign bit flipped, so the kernel places them under a binary16 exponent
 * without a further operation) and scales [rows,
 * head_dim / 32] fp16.  Byte moves only.  head_dim a multiple of 32 (<= 4096);
 * canonical_bytes >= rows * head_dim / 32 * 34 (else QG_ERR_SIZE). */
qg_status qg_pack_kv_host(const void *canonical, size_t canonical_bytes, int64_t rows, int64_t head_dim,
                          void *codes, void *scales);

/* Static text for a status code. */
const char *qg_status_str(qg_status s);

/* ABI version of this header (major * 100 + minor). */
int32_t qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
