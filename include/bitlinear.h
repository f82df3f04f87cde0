/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear path:
 * ternary weights {-1, 0, +1} x int8 activations ("W1.58A8"), integer
 * accumulation, fp32 dequantisation, and the ReLU² feed-forward block.
 *
 * Pages the operations follow (by title and section):
 *  [P1] youngju.dev "BitNet論文分析：1-Bit LLMの時代": "1-Bit重みとSign関数"
 *       (binary weights, mean |W| scale), "Absmean量子化関数" (ternary
 *       weights), "BitNet b1.58" (BitLinear_b158: RMSNorm, per-token absmax
 *       activation quant, F.linear, rescale), "アーキテクチャ概要" (I2_S:
 *       2-bit codes 00/01/10, 16 weights per 32-bit word).
 *  [P2] ai-heartland.com "BitNet — 1-bit Transformersの実装ライブラリ":
 *       "BitLinearの仕組み" (flow; symmetric activation codes; float only in
 *       normalisation and rescale), "BitLinear層の基本実装" (drop-in Linear).
 *  [P3] dashen-tech.com "BitNet.cpp 深度解析": §2.3 (2-bit I2_S storage),
 *       §3.1 (Y = sum_pos - sum_neg, no multiplies).
 *  [P5] reinforz.co.jp, BitNet b1.58 2B4T news: W1.58A8, ReLU², no bias.
 *
 * Conventions
 *  - W is [N][K] row-major (N = out features, K = in features) as in the
 *    listings' nn.Parameter(out_features, in_features); X is [M][K];
 *    Y = X W^T is [M][N].
 *  - Kp = bl_padded_k(K) = K rounded up to a multiple of 64.
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees, synchronises, or keeps a pointer after return.
 *    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; results are valid after the caller
 *    synchronises that stream.  Calls on different streams that share no
 *    output buffer or workspace may run concurrently; the library keeps no
 *    state between calls (beyond one-time kernel attributes).
 *  - Only kernel launches are enqueued (no memset, copy or event), so a
 *    sequence of calls can be captured in a HIP graph and replayed; the
 *    pointers passed at capture time, workspaces included, stay baked into
 *    the graph.
 *  - Validation is host-only and happens before anything is enqueued; on
 *    any error nothing is launched and no memory is touched.  Device
 *    pointers are never dereferenced on the host.
 *  - Inputs containing NaN or Inf give unspecified (but memory-safe) results.
 *
 * Numeric contract (one IEEE binary32 rounding per operation, round to
 * nearest even, no fused multiply-add, correctly rounded / and sqrt):
 *  - eps = binary32(1e-5), Q = 127.
 *  - weight scale  g_w = binary32( binary64( exact sum |w| ) / (N*K) )
 *  - ternary code  t = clamp(rne(w / (g_w + eps)), -1, 1); binary t = w >= 0 ? +1 : -1
 *  - activation    g_m = max_k |x[m][k]|;  q = clamp(rne((x * 127) / (g_m + eps)), -127, 127)
 *  - accumulator   acc[m][n] = sum_k q[m][k] * t[n][k]   (exact int32)
 *  - output        y = ((float)acc * (g_w * g_m)) / 127
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    BL_OK = 0,
    BL_EINVAL = 1,     /* NULL where a pointer is required, or an unknown enum value   */
    BL_ESHAPE = 2,     /* a size <= 0, or above the documented limit                    */
    BL_EALIGN = 3,     /* a pointer not aligned as documented                           */
    BL_EWORKSPACE = 4, /* workspace pointer NULL or smaller than the size helper says   */
    BL_EHIP = 5        /* the HIP runtime reported an error when enqueuing the kernels */
};

/* Weight quantiser ([P1] "Absmean量子化関数" / "1-Bit重みとSign関数").
 * BL_BINARY_1BIT: the binary quantiser packed one bit per weight. */
enum { BL_TERNARY = 0, BL_BINARY = 1, BL_BINARY_1BIT = 2 };

/* Element type of float activations / hidden states (bf16 is widened exactly). */
enum { BL_F32 = 0, BL_BF16 = 1 };

/* Size limits (checked): 1 <= M <= BL_MAX_M, 1 <= N, K <= BL_MAX_DIM. */
#define BL_MAX_M 65536
#define BL_MAX_DIM 65536

/* Kp: K rounded up to a multiple of 64 (row stride of Xq in bytes, of Wp in
 * weights).  Returns 0 for K <= 0. */
int64_t bl_padded_k(int64_t K);

/* Bytes of a packed weight matrix: N * Kp / 4.  0 for invalid sizes. */
size_t bl_packed_bytes(int64_t N, int64_t K);

/* Kb: K rounded up to a multiple of 128 (weights per row of the 1-bit
 * layout).  Returns 0 for K <= 0. */
int64_t bl_padded_k_1bit(int64_t K);

/* Bytes of a 1-bit packed binary matrix: N * Kb / 8.  0 for invalid sizes. */
size_t bl_packed_bytes_1bit(int64_t N, int64_t K);

/* Workspace bytes bitlinear_pack needs (256 64-bit exponent bins). */
size_t bl_pack_workspace_bytes(int64_t N, int64_t K);

/* Static, human-readable text for a status code (host memory, never NULL). */
const char *bl_status_str(int status);

/*
 * bitlinear_pack -- quantise and pack one weight matrix (done once per
 * weight, as the I2_S conversion of [P1] "BitNet b1.58 2B4T" and [P3] §2.3).
 *
 *  W        [N][K] float32, device.  Any alignment (4 bytes).
 *  mode     BL_TERNARY: absmean ternarisation ([P1] "Absmean量子化関数").
 *           BL_BINARY : sign binarisation, +1 for w >= 0 including -0.0
 *                       ([P1] "1-Bit重みとSign関数"); same scale g_w.
 *           BL_BINARY_1BIT: the same binarisation in the 1-bit layout
 *                       below (for bitlinear_forward_1bit).
 *  Wp       [N][Kp/16] uint32 words, device, 16-byte aligned, written.
 *           Layout: word j of row n covers weights 16j..16j+15; weight
 *           16j + 4s + b is stored in byte b at bits 2s..2s+1 with code
 *           t + 1 (00 = -1, 01 = 0, 10 = +1; 11 never written).  Padding
 *           weights k >= K hold code 01.
 *           BL_BINARY_1BIT: [N][Kb/32] words (bl_packed_bytes_1bit bytes);
 *           word j of row n covers weights 32j..32j+31; weight 32j + 4s + b
 *           is bit 8b + s (s = 0..7, b = 0..3), 1 for +1 and 0 for -1;
 *           padding weights k >= K are bit 0.
 *  w_scale  1 float, device, written with g_w (the scale itself, not its
 *           reciprocal).
 *  ws       device workspace, 16-byte aligned, >= bl_pack_workspace_bytes;
 *           contents on entry are ignored and on exit are unspecified.
 *  Errors: BL_EINVAL (NULL pointer, bad mode), BL_ESHAPE, BL_EALIGN,
 *          BL_EWORKSPACE, BL_EHIP.
 */
int bitlinear_pack(const float *W, int64_t N, int64_t K, int mode, uint32_t *Wp,
                   float *w_scale, void *ws, size_t ws_bytes, void *stream);

/*
 * bitlinear_quant_act -- per-token absmax int8 quantisation ([P1] "BitNet
 * b1.58" activation_quant; range [-127, 127], [P2] "BitLinearの仕組み").
 *
 *  X        [M][K] float32 (dtype BL_F32) or bfloat16 (BL_BF16), device,
 *           element-aligned.
 *  Xq       [M][Kp] int8, device, 16-byte aligned, written; columns K..Kp-1
 *           are written as 0.
 *  x_scale  [M] float, device, written with g_m = max_k |x[m][k]|.
 *  x_rowsum [M] int32, device, written with sum_k q[m][k] (required: the
 *           product kernels of bitlinear_forward take it as an input).
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EHIP.
 */
int bitlinear_quant_act(const void *X, int dtype, int64_t M, int64_t K, int8_t *Xq,
                        float *x_scale, int32_t *x_rowsum, void *stream);

/*
 * bitlinear_forward -- Y = dequant(Xq . T^T) for packed ternary/binary
 * weights ([P1] "BitNet b1.58": F.linear then output * (w_scale * x_scale)
 * / Q; [P3] §3.1: the integer product is sum_pos - sum_neg).  No bias
 * ([P5]).
 *
 *  Xq       [M][Kp] int8 from bitlinear_quant_act (padding columns zero),
 *           device, 16-byte aligned.
 *  x_scale  [M] float g_m, device.
 *  x_rowsum [M] int32 row sums of Xq, device (required: the kernels use
 *           sum_k q*(t+1) - rowsum).
 *  Wp       [N][Kp/16] packed words from bitlinear_pack, 16-byte aligned.
 *  w_scale  1 float g_w, device.
 *  Y        [M][N] float32, device, 4-byte aligned, written.
 *  acc_out  [M][N] int32, device, or NULL; when given, the exact integer
 *           accumulators are written too (for inspection).
 *  The kernel is chosen by the shape (1 token: GEMV; up to 64 tokens: the
 *  skinny MFMA kernels; up to 192 tokens (384 with K >= 4096) on layers of
 *  2048..16384 outputs: the MFMA kernel that splits K over the waves of a
 *  block; else the tiled MFMA GEMM); all give identical bits.
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EHIP.
 */
int bitlinear_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                      int64_t M, int64_t K, const uint32_t *Wp, const float *w_scale,
                      int64_t N, float *Y, int32_t *acc_out, void *stream);

/*
 * bitlinear_forward_1bit -- bitlinear_forward for binary weights packed by
 * bitlinear_pack(..., BL_BINARY_1BIT, ...) ([P1] "1-Bit重みとSign関数":
 * t = +1 / -1 in one bit; the integer product is again sum_pos - sum_neg,
 * [P3] §3.1).  Same arguments, except
 *  Wb       [N][Kb/32] words of the 1-bit layout (Kb = bl_padded_k_1bit(K)),
 *           16-byte aligned.
 *  The kernel is chosen by M (1: the bit GEMV; otherwise the 1-bit MFMA
 *  kernel in slices of up to 64 tokens); the results equal those of the
 *  2-bit layout of the same weights bit for bit.
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EHIP.
 */
int bitlinear_forward_1bit(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                           int64_t M, int64_t K, const uint32_t *Wb, const float *w_scale,
                           int64_t N, float *Y, int32_t *acc_out, void *stream);

/*
 * bitlinear_quant_act_a48 -- BitNet a4.8 split activations ([P1] "BitNet
 * a4.8": the top fraction of the values is split off at 8 bits, the rest is
 * quantised to 4 bits).  Per token row m:
 *   outliers: the n_out entries of largest |x| (ties to the lower index);
 *   g8 = max |x| over them, q8 = clamp(rne(x * 127 / (g8 + 1e-5)), +-127);
 *   g4 = max |x| over the rest, q4 = clamp(rne(x * 7 / (g4 + 1e-5)), +-7);
 * each code vector is 0 where the other holds the entry (and past K).
 *  X        [M][K] float32 / bfloat16 (dtype), device.  n_out >= 0 (values
 *           above K mean every entry).
 *  Xq4, Xq8 [M][Kp] int8, device, 16-byte aligned, written.
 *  x4_scale, x8_scale [M] float (g4, g8); x4_rowsum, x8_rowsum [M] int32
 *           (row sums of q4, q8); all written.
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EHIP.
 */
int bitlinear_quant_act_a48(const void *X, int dtype, int64_t M, int64_t K, int64_t n_out,
                            int8_t *Xq4, float *x4_scale, int32_t *x4_rowsum, int8_t *Xq8,
                            float *x8_scale, int32_t *x8_rowsum, void *stream);

/* Workspace bytes of bitlinear_forward_a48: 8 * M * N. */
size_t bitlinear_a48_workspace_bytes(int64_t M, int64_t N);

/*
 * bitlinear_forward_a48 -- BitLinear on a4.8 activations and packed
 * ternary/binary weights: acc4 = q4 . t, acc8 = q8 . t (exact int32) and
 *   Y = (acc4 * (g_w * g4)) / 7 + (acc8 * (g_w * g8)) / 127,
 * each part dequantised in the order of [P1]'s listing, then added.
 *  Xq4..x8_rowsum from bitlinear_quant_act_a48; Wp, w_scale, Y as for
 *  bitlinear_forward.
 *  ws       >= bitlinear_a48_workspace_bytes(M, N) bytes, 16-byte aligned;
 *           after the call it holds acc4 [M][N] then acc8 [M][N] int32.
 *  Layout hint: when the two parts are stacked -- Xq8 == Xq4 + M * Kp,
 *  x8_scale == x4_scale + M and x8_rowsum == x4_rowsum + M -- and M <= 8,
 *  one product over the 2M code rows reads the weights once instead of
 *  twice.  Results are identical either way.
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EWORKSPACE, BL_EHIP.
 */
int bitlinear_forward_a48(const int8_t *Xq4, const float *x4_scale, const int32_t *x4_rowsum,
                          const int8_t *Xq8, const float *x8_scale, const int32_t *x8_rowsum,
                          int64_t M, int64_t K, const uint32_t *Wp, const float *w_scale,
                          int64_t N, float *Y, void *ws, size_t ws_bytes, void *stream);

/* bitlinear_forward with the kernel chosen by the caller (for cross-checks
 * and timing): BL_KERNEL_AUTO as bitlinear_forward; BL_KERNEL_GEMV needs
 * M == 1; BL_KERNEL_SKINNY needs M <= 64 (one MFMA tile row of 16/32/64
 * tokens, any of the skinny kernels); BL_KERNEL_TILED is the 128 x 256
 * tiled MFMA GEMM for any M.
 * Errors as bitlinear_forward, plus BL_ESHAPE when M does not fit the
 * chosen kernel and BL_EINVAL for an unknown kernel id. */
enum { BL_KERNEL_AUTO = 0, BL_KERNEL_GEMV = 1, BL_KERNEL_SKINNY = 2, BL_KERNEL_TILED = 3 };
int bitlinear_forward_kernel(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                             int64_t M, int64_t K, const uint32_t *Wp, const float *w_scale,
                             int64_t N, float *Y, int32_t *acc_out, int kernel, void *stream);

/*
 * bitlinear_forward_fused -- one BitLinear straight from float activations:
 * per-token quantisation ([P1] "BitNet b1.58" activation_quant) and the
 * product with fused dequant in one call.  For one token with Kp <= 7168,
 * or Kp <= 8192 when the packed matrix has 16 MiB or more, it is a single
 * kernel (every block quantises the token into LDS; identical bits);
 * otherwise bitlinear_quant_act into the workspace, then bitlinear_forward.
 * Results are bit-identical to that two-call sequence.
 *
 *  X        [M][K] float32 (BL_F32) or bfloat16 (BL_BF16), device.
 *  Wp, w_scale, N, Y   as bitlinear_forward.
 *  ws       >= bitlinear_fused_workspace_bytes(M, K) bytes, 16-byte aligned.
 *           On return it holds Xq [M][Kp] int8 at offset 0, x_scale [M] float
 *           at offset bitlinear_fused_workspace_offset(M, K, 1) and x_rowsum
 *           [M] int32 at offset bitlinear_fused_workspace_offset(M, K, 2).
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EWORKSPACE, BL_EHIP.
 */
size_t bitlinear_fused_workspace_bytes(int64_t M, int64_t K);
size_t bitlinear_fused_workspace_offset(int64_t M, int64_t K, int which);
int bitlinear_forward_fused(const void *X, int dtype, int64_t M, int64_t K, const uint32_t *Wp,
                            const float *w_scale, int64_t N, float *Y, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * bitlinear_forward_fused_norm -- the same with the layer's own RMSNorm in
 * front of the quantiser: y = BitLinear(RMSNorm(x)), the order of the
 * BitLinear_b158 forward in [P1] "BitNet b1.58" (normalise, quantise,
 * multiply, rescale).  Per token r = 1 / sqrt(ms + norm_eps) with
 * ms = binary32(binary64(exact sum x^2) / K), and xn = (x * r) * norm_w
 * (norm_w NULL: xn = x * r); the codes, scale and row sum are those of
 * bitlinear_quant_act on xn.  One float32 token with Kp <= 8192 runs as a
 * single kernel (every block normalises and quantises the token; identical
 * bits); otherwise the RMSNorm + quantiser kernel, then bitlinear_forward.
 *
 *  X, dtype, M, K, Wp, w_scale, N, Y   as bitlinear_forward_fused.
 *  norm_w   [K] float32, device, or NULL for ones.  norm_eps: the epsilon
 *           added to the mean square (torch.nn.RMSNorm's default for float32
 *           is 2^-23).
 *  ws       >= bitlinear_fused_norm_workspace_bytes(M, K) bytes, 16-byte
 *           aligned.  On return it holds what bitlinear_forward_fused leaves
 *           there (codes, scales, row sums at the same offsets) and xn
 *           [M][K] float32 at offset bitlinear_fused_workspace_bytes(M, K).
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN (norm_w too), BL_EWORKSPACE, BL_EHIP.
 */
size_t bitlinear_fused_norm_workspace_bytes(int64_t M, int64_t K);
int bitlinear_forward_fused_norm(const void *X, int dtype, int64_t M, int64_t K,
                                 const float *norm_w, float norm_eps, const uint32_t *Wp,
                                 const float *w_scale, int64_t N, float *Y, void *ws,
                                 size_t ws_bytes, void *stream);

/* Workspace layout of bitnet_ffn_forward.  bitnet_ffn_workspace_layout fills
 * off[BL_FFN_WS_COUNT] with byte offsets (each 256-byte aligned) and returns
 * the total size.  After a call the workspace holds the block's internals:
 *   XN  float [M][D]   RMSNorm output
 *   QX  int8  [M][Dp]  its int8 codes;   GX float [M] scales;  RSX int32 [M] row sums
 *   H   float [M][F]   relu(gate)^2 * up
 *   HN  float [M][F]   RMSNorm(h) (written only with SubLN)
 *   GH  float [M]      max |h| per token (stored as float bits)
 *   QH  int8  [M][Fp]  int8 codes of h;  RSH int32 [M] row sums
 *   GHP float [P][M]   per-block partial maxima of |h| (scratch)          */
enum {
    BL_FFN_WS_XN = 0, BL_FFN_WS_QX, BL_FFN_WS_GX, BL_FFN_WS_RSX, BL_FFN_WS_H, BL_FFN_WS_HN,
    BL_FFN_WS_GH, BL_FFN_WS_QH, BL_FFN_WS_RSH, BL_FFN_WS_GHP, BL_FFN_WS_COUNT
};
size_t bitnet_ffn_workspace_layout(int64_t M, int64_t D, int64_t F, size_t *off);
size_t bitnet_ffn_workspace_bytes(int64_t M, int64_t D, int64_t F);

/*
 * bitnet_ffn_forward -- the feed-forward block
 *   xn = RMSNorm(H) ([P1] "BitNet b1.58": normalise before quantising);
 *   g  = BitLinear_gate(xn), u = BitLinear_up(xn)   (D -> F, shared quant);
 *   h  = relu(g)^2 * u                               ([P5] ReLU², gated);
 *   hn = RMSNorm(h) over F, only with SubLN (subln_w != NULL): the norm
 *        every BitLinear of [P1] "BitNet b1.58" applies before quantising,
 *        the sub-layer norm of [P4] "正規化で分散を安定させる" and [P5];
 *   Y  = BitLinear_down(hn or h)                      (F -> D, requantised).
 * RMSNorm: ms = binary32(binary64(exact sum x^2) / D); r = 1 / sqrt(ms + eps);
 * xn = (x * r) * norm_w.  No residual is added (the caller owns it).
 *
 *  H        [M][D] float32 or bfloat16 (dtype), device.
 *  norm_w   [D] float, device, or NULL for ones.  norm_eps: RMSNorm epsilon
 *           (PyTorch's default for float32 is 2^-23).
 *  subln_w  [F] float, device: SubLN weight; NULL = no SubLN (the block as
 *           the 2B-class FFN workload states it).  subln_eps: its epsilon.
 *  Wg, Wu   [F][Dp/16] packed (16-byte aligned), sg, su their scales.
 *  Wd       [D][Fp/16] packed, sd its scale.
 *  Y        [M][D] float32, device, 4-byte aligned, written.
 *  ws       >= bitnet_ffn_workspace_bytes(M, D, F) bytes, 256-byte aligned.
 *  Errors: BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EWORKSPACE, BL_EHIP.
 */
int bitnet_ffn_forward(const void *H, int dtype, int64_t M, int64_t D, int64_t F,
                       const float *norm_w, float norm_eps, const float *subln_w,
                       float subln_eps, const uint32_t *Wg,
                       const float *sg, const uint32_t *Wu, const float *su,
                       const uint32_t *Wd, const float *sd, float *Y, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * bitnet_ffn_forward_static -- bitnet_ffn_forward for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid device allocation): the same block, bit for bit, with the workspace
 * taken from a scratch array of BL_FFN_STATIC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends.  It calls no
 * allocator.  The caller still passes every input and output.
 *
 *  Arguments as bitnet_ffn_forward, without ws / ws_bytes.
 *  Limit: bitnet_ffn_workspace_bytes(M, D, F) <= BL_FFN_STATIC_SCRATCH_BYTES,
 *         else BL_ESHAPE (e.g. D = 2560, F = 6912 fits up to 64 tokens).
 *  Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *  that overlap on one GPU (different streams, or a graph replay running
 *  beside another call) race; serialise them.  The scratch keeps the last
 *  call's contents; nothing in it needs to start at zero.
 *  Errors: as bitnet_ffn_forward, plus BL_ESHAPE for the limit above and
 *          BL_EHIP if the scratch address cannot be looked up.
 */
#define BL_FFN_STATIC_SCRATCH_BYTES (16 << 20)
int bitnet_ffn_forward_static(const void *H, int dtype, int64_t M, int64_t D, int64_t F,
                              const float *norm_w, float norm_eps, const float *subln_w,
                              float subln_eps, const uint32_t *Wg, const float *sg,
                              const uint32_t *Wu, const float *su, const uint32_t *Wd,
                              const float *sd, float *Y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
