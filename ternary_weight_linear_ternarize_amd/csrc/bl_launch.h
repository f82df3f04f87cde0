// Internal launchers of the gfx950 kernels (host side).  All enqueue on the
// given stream and return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// bitlinear_pack: zero bins, exponent-binned exact |w| sum, finalize g_w,
// ternarise/binarise + pack.  mode 0: ternary, 1: binary (2-bit codes),
// 2: binary in the 1-bit layout.
hipError_t launch_pack(const float* W, int64_t N, int64_t K, int mode, uint32_t* Wp,
                       float* w_scale, uint64_t* bins, hipStream_t s);

// BitNet a4.8 split activations (a48.hip): per row the n_out largest |x|
// as int8 codes (q8, scale g8), the rest as 4-bit codes in int8 storage (q4,
// scale g4); both [M][Kp], each zero where the other holds the entry.
hipError_t launch_act_quant_a48(const void* X, bool bf16, int64_t M, int64_t K, int64_t n_out,
                                int8_t* q4, float* g4, int32_t* rs4, int8_t* q8, float* g8,
                                int32_t* rs8, hipStream_t s);
// Y = (acc4 (g_w g4)) / 7 + (acc8 (g_w g8)) / 127.  acc ([2][M][N] int32:
// acc4 then acc8) is optional for one token with Kp <= 16384 and required
// otherwise (the accumulators of the two products are kept there).
hipError_t launch_forward_a48(const int8_t* x4, const float* g4, const int32_t* rs4,
                              const int8_t* x8, const float* g8, const int32_t* rs8, int64_t M,
                              int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N,
                              float* Y, int32_t* acc, hipStream_t s);

// The streaming skinny MFMA kernel on 1-bit binary weights (M <= 16 while
// the activations fit its LDS, or on layers of at least 1600 tiles of 16
// rows with the activations staged in phases: stream_1bit_ok).
bool stream_1bit_ok(int64_t M, int64_t K, int64_t N);
hipError_t launch_stream_1bit(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                              int64_t M, int64_t K, const uint32_t* Wb, const float* w_scale,
                              int64_t N, float* Y, int32_t* acc_out, hipStream_t s);

// Y = dequant(Xq . T^T) for binary weights in the 1-bit layout (rows of
// Kb = K rounded up to 128 weights; Xq rows of Kp = K rounded up to 64):
// the bit GEMV for one token, the 1-bit MFMA kernel otherwise (bin1.hip).
hipError_t launch_forward_1bit(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                               int64_t M, int64_t K, const uint32_t* Wb, const float* w_scale,
                               int64_t N, float* Y, int32_t* acc_out, hipStream_t s);

// Per-token absmax int8 quantisation.  When gamma_parts is non-null the
// scale of row m is max over p < nparts of gamma_parts[p * M + m] (partial
// maxima written by another kernel) instead of being computed from X.
hipError_t launch_act_quant(const void* X, bool bf16, int64_t M, int64_t K, int8_t* Xq,
                            float* x_scale, int32_t* rowsum, const float* gamma_parts,
                            int nparts, hipStream_t s);

// RMSNorm + per-token quantisation of the normalised rows.
hipError_t launch_rmsnorm_quant(const void* H, bool bf16, int64_t M, int64_t D,
                                const float* norm_w, float eps, float* xn, int8_t* Xq,
                                float* x_scale, int32_t* rowsum, hipStream_t s);

// Y = dequant(Xq . T^T) for one token (M == 1): the dot4 GEMV.
hipError_t launch_gemv(const int8_t* Xq, const float* x_scale, const int32_t* rowsum, int64_t K,
                       const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                       int32_t* acc_out, hipStream_t s);

// One token from float activations: quantise inside the GEMV (every block
// redoes the row into LDS) -- one launch.  Needs bl_padded_k(K) <= 7168, or a
// packed matrix of at least 16 MiB with bl_padded_k(K) <= 8192 (the streaming
// form; gemv_fused_ok).  xq_out/xs_out/rs_out (optional) receive the codes.
bool gemv_fused_ok(int64_t K, int64_t N);
hipError_t launch_gemv_fused(const void* X, bool bf16, int64_t K, const uint32_t* Wp,
                             const float* w_scale, int64_t N, float* Y, int32_t* acc_out,
                             int8_t* xq_out, float* xs_out, int32_t* rs_out, hipStream_t s);
// As launch_gemv_fused for a float32 row whose scale is the maximum of
// gparts[0..nparts) (partial maxima from launch_gemv_gateup).
hipError_t launch_gemv_parts(const float* X, const float* gparts, int nparts, int64_t K,
                             const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                             int8_t* xq_out, float* xs_out, int32_t* rs_out, hipStream_t s);

// One token of a float32 row RMS-normalised (norm_w, eps; the exact mean
// square), quantised and multiplied in one kernel (every block redoes the
// norm; block 0 writes xn, the codes, the scale and the row sum): the SubLN
// block's down projection.  Needs gemv_norm_ok(K) (padded K <= 8192).
bool gemv_norm_ok(int64_t K);
hipError_t launch_gemv_norm(const float* X, int64_t K, const float* norm_w, float eps,
                            const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                            float* xn_out, int8_t* xq_out, float* xs_out, int32_t* rs_out,
                            hipStream_t s);

// Y = dequant(Xq . T^T) on MFMA.  tiled == true: the 128 x 256 tiled
// kernel; false: the kernel the shape measured fastest on (the skinny
// kernels up to 64 tokens, the K-split kernel where ksplit_ok, else tiled).
hipError_t launch_mfma(const int8_t* Xq, const float* x_scale, const int32_t* rowsum, int64_t M,
                       int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                       int32_t* acc_out, bool tiled, hipStream_t s);

// FFN gate/up: h = relu(deq(gate))^2 * deq(up) for both weights at once, plus
// per-block partial maxima of |h| (gh_parts[p * M + m], p < *nparts).  The
// one-token GEMV form covers padded K up to 16384 (gemv_gateup_ok).
bool gemv_gateup_ok(int64_t K);
hipError_t launch_gemv_gateup(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                              int64_t K, const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                              const float* su, int64_t N, float* H, float* gh_parts, int* nparts,
                              hipStream_t s);
// The same for one token of float hidden state H: RMSNorm (exact mean
// square), quantisation and the gate/up product in one kernel (every block
// redoes the norm; block 0 writes xn, the codes, the scale and the row sum).
// Needs gemv_gateup_norm_ok(K) (padded K <= 4096).
bool gemv_gateup_norm_ok(int64_t K);
hipError_t launch_gemv_gateup_norm(const void* H, bool bf16, int64_t K, const float* norm_w,
                                   float eps, const uint32_t* Wg, const float* sg,
                                   const uint32_t* Wu, const float* su, int64_t N, float* Hout,
                                   float* gh_parts, int* nparts, float* xn_out, int8_t* xq_out,
                                   float* xs_out, int32_t* rs_out, hipStream_t s);
hipError_t launch_mfma_gateup(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                              int64_t M, int64_t K, const uint32_t* Wg, const float* sg,
                              const uint32_t* Wu, const float* su, int64_t N, float* H,
                              float* gh_parts, int* nparts, hipStream_t s);

// Up to 16 tokens with the weights loaded straight into MFMA operands
// (skinny.hip); direct_ok says whether the shape is covered (LDS, registers).
bool direct_ok(int64_t M, int64_t K, int64_t N, int nb);
// a4.8 codes stacked as 2 Mh rows (int4 rows, then the int8 rows of the same
// tokens, scales and row sums stacked alike): where the product runs on the
// streaming kernel, one launch writes both accumulators (acc4 then acc8 rows)
// and y of the Mh tokens (gemm.hip).
bool stream_a48_ok(int64_t M2, int64_t K, int64_t N);
hipError_t launch_stream_a48(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M2,
                             int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                             int32_t* acc, hipStream_t s);
hipError_t launch_direct(const int8_t* Xq, const float* x_scale, const int32_t* rowsum, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s);
hipError_t launch_direct_gateup(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                                int64_t M, int64_t K, const uint32_t* Wg, const float* sg,
                                const uint32_t* Wu, const float* su, int64_t N, float* H,
                                float* gh_parts, int* nparts, hipStream_t s);

// 2..64 tokens with K split over the 8 waves of a block and every load of a
// wave in flight at once (ksplit.hip); ksplit_ok says whether K fits the
// register budget of the tile the shape would take (nb: 1 plain, 2 gate/up).
bool ksplit_ok(int64_t M, int64_t K, int64_t N, int nb);
hipError_t launch_ksplit(const int8_t* Xq, const float* x_scale, const int32_t* rowsum, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s);
hipError_t launch_ksplit_gateup(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                                int64_t M, int64_t K, const uint32_t* Wg, const float* sg,
                                const uint32_t* Wu, const float* su, int64_t N, float* H,
                                float* gh_parts, int* nparts, hipStream_t s);
// Upper bounds of the partial-maximum slots per row the gate/up kernels write.
int64_t gemv_gateup_parts(int64_t N);
int64_t mfma_gateup_parts(int64_t M, int64_t N);

}  // namespace bl
