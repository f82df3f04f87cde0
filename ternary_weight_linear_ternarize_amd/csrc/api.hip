// C ABI of the BitLinear library: host-side validation, workspace layout and
// kernel dispatch.  Nothing here touches device memory on the host, allocates
// or synchronises; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "bitlinear.h"
#include "bl_launch.h"

// Scratch of bitnet_ffn_forward_static: one copy per GPU (a file-scope device
// array lives in the code object loaded on each device), held until the
// process ends.  In host code this name is only a host-side stand-in: the
// device address is looked up once per device (static_scratch_address) and
// only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[BL_FFN_STATIC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool dim_ok(int64_t v) { return v >= 1 && v <= BL_MAX_DIM; }
bool m_ok(int64_t v) { return v >= 1 && v <= BL_MAX_M; }
int64_t padk(int64_t K) { return (K + 63) / 64 * 64; }
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_EHIP; }

int check_forward(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                  int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N, float* Y) {
  if (!Xq || !x_scale || !x_rowsum || !Wp || !w_scale || !Y) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(K) || !dim_ok(N)) return BL_ESHAPE;
  if (!aligned(Xq, 16) || !aligned(Wp, 16) || !aligned(Y, 4) || !aligned(x_scale, 4) ||
      !aligned(x_rowsum, 4) || !aligned(w_scale, 4))
    return BL_EALIGN;
  return BL_OK;
}

// Argument checks shared by the two FFN entry points (everything but the
// workspace).
int ffn_check(const void* H, int dtype, int64_t M, int64_t D, int64_t F, const float* norm_w,
              const float* subln_w, const uint32_t* Wg, const float* sg, const uint32_t* Wu,
              const float* su, const uint32_t* Wd, const float* sd, const float* Y) {
  if (!H || !Wg || !sg || !Wu || !su || !Wd || !sd || !Y) return BL_EINVAL;
  if (dtype != BL_F32 && dtype != BL_BF16) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(D) || !dim_ok(F)) return BL_ESHAPE;
  if (!aligned(H, dtype == BL_F32 ? 4 : 2) || !aligned(Wg, 16) || !aligned(Wu, 16) ||
      !aligned(Wd, 16) || !aligned(Y, 4) || !aligned(sg, 4) || !aligned(su, 4) ||
      !aligned(sd, 4) || (norm_w && !aligned(norm_w, 4)) || (subln_w && !aligned(subln_w, 4)))
    return BL_EALIGN;
  return BL_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = reinterpret_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int64_t bl_padded_k(int64_t K) { return K <= 0 ? 0 : padk(K); }

size_t bl_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)N * (size_t)padk(K) / 4;
}

int64_t bl_padded_k_1bit(int64_t K) { return K <= 0 ? 0 : (K + 127) / 128 * 128; }

size_t bl_packed_bytes_1bit(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)N * (size_t)bl_padded_k_1bit(K) / 8;
}

size_t bl_pack_workspace_bytes(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return 256 * sizeof(uint64_t);
}

const char* bl_status_str(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument (null pointer or unknown enum value)";
    case BL_ESHAPE: return "invalid shape (size <= 0, above the limit, or not fitting the kernel)";
    case BL_EALIGN: return "misaligned pointer";
    case BL_EWORKSPACE: return "workspace missing or too small";
    case BL_EHIP: return "HIP runtime error while enqueuing kernels";
    default: return "unknown status";
  }
}

int bitlinear_pack(const float* W, int64_t N, int64_t K, int mode, uint32_t* Wp, float* w_scale,
                   void* ws, size_t ws_bytes, void* stream) {
  if (!W || !Wp || !w_scale) return BL_EINVAL;
  if (mode != BL_TERNARY && mode != BL_BINARY && mode != BL_BINARY_1BIT) return BL_EINVAL;
  if (!dim_ok(N) || !dim_ok(K)) return BL_ESHAPE;
  if (!ws || ws_bytes < bl_pack_workspace_bytes(N, K)) return BL_EWORKSPACE;
  if (!aligned(W, 4) || !aligned(Wp, 16) || !aligned(w_scale, 4) || !aligned(ws, 16))
    return BL_EALIGN;
  const int kind = mode == BL_TERNARY ? 0 : (mode == BL_BINARY ? 1 : 2);
  return hip_status(bl::launch_pack(W, N, K, kind, Wp, w_scale, reinterpret_cast<uint64_t*>(ws),
                                    as_stream(stream)));
}

int bitlinear_quant_act(const void* X, int dtype, int64_t M, int64_t K, int8_t* Xq,
                        float* x_scale, int32_t* x_rowsum, void* stream) {
  if (!X || !Xq || !x_scale || !x_rowsum) return BL_EINVAL;
  if (dtype != BL_F32 && dtype != BL_BF16) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(K)) return BL_ESHAPE;
  if (!aligned(X, dtype == BL_F32 ? 4 : 2) || !aligned(Xq, 16) || !aligned(x_scale, 4) ||
      !aligned(x_rowsum, 4))
    return BL_EALIGN;
  return hip_status(bl::launch_act_quant(X, dtype == BL_BF16, M, K, Xq, x_scale, x_rowsum,
                                         nullptr, 0, as_stream(stream)));
}

int bitlinear_forward_kernel(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                             int64_t M, int64_t K, const uint32_t* Wp, const float* w_scale,
                             int64_t N, float* Y, int32_t* acc_out, int kernel, void* stream) {
  int st = check_forward(Xq, x_scale, x_rowsum, M, K, Wp, w_scale, N, Y);
  if (st != BL_OK) return st;
  if (acc_out && !aligned(acc_out, 4)) return BL_EALIGN;
  hipStream_t s = as_stream(stream);
  if (kernel == BL_KERNEL_AUTO) {
    if (M == 1) return hip_status(bl::launch_gemv(Xq, x_scale, x_rowsum, K, Wp, w_scale, N, Y, acc_out, s));
    return hip_status(
        bl::launch_mfma(Xq, x_scale, x_rowsum, M, K, Wp, w_scale, N, Y, acc_out, false, s));
  }
  switch (kernel) {
    case BL_KERNEL_GEMV:
      if (M != 1) return BL_ESHAPE;
      return hip_status(bl::launch_gemv(Xq, x_scale, x_rowsum, K, Wp, w_scale, N, Y, acc_out, s));
    case BL_KERNEL_SKINNY:
      if (M > 64) return BL_ESHAPE;
      return hip_status(
          bl::launch_mfma(Xq, x_scale, x_rowsum, M, K, Wp, w_scale, N, Y, acc_out, false, s));
    case BL_KERNEL_TILED:
      return hip_status(
          bl::launch_mfma(Xq, x_scale, x_rowsum, M, K, Wp, w_scale, N, Y, acc_out, true, s));
    default:
      return BL_EINVAL;
  }
}

int bitlinear_forward(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                      int64_t K, const uint32_t* Wp, const float* w_scale, int64_t N, float* Y,
                      int32_t* acc_out, void* stream) {
  return bitlinear_forward_kernel(Xq, x_scale, x_rowsum, M, K, Wp, w_scale, N, Y, acc_out,
                                  BL_KERNEL_AUTO, stream);
}

int bitlinear_forward_1bit(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                           int64_t M, int64_t K, const uint32_t* Wb, const float* w_scale,
                           int64_t N, float* Y, int32_t* acc_out, void* stream) {
  int st = check_forward(Xq, x_scale, x_rowsum, M, K, Wb, w_scale, N, Y);
  if (st != BL_OK) return st;
  if (acc_out && !aligned(acc_out, 4)) return BL_EALIGN;
  return hip_status(bl::launch_forward_1bit(Xq, x_scale, x_rowsum, M, K, Wb, w_scale, N, Y,
                                            acc_out, as_stream(stream)));
}

int bitlinear_quant_act_a48(const void* X, int dtype, int64_t M, int64_t K, int64_t n_out,
                            int8_t* Xq4, float* x4_scale, int32_t* x4_rowsum, int8_t* Xq8,
                            float* x8_scale, int32_t* x8_rowsum, void* stream) {
  if (!X || !Xq4 || !x4_scale || !x4_rowsum || !Xq8 || !x8_scale || !x8_rowsum) return BL_EINVAL;
  if (dtype != BL_F32 && dtype != BL_BF16) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(K) || n_out < 0) return BL_ESHAPE;
  if (!aligned(X, dtype == BL_F32 ? 4 : 2) || !aligned(Xq4, 16) || !aligned(Xq8, 16) ||
      !aligned(x4_scale, 4) || !aligned(x4_rowsum, 4) || !aligned(x8_scale, 4) ||
      !aligned(x8_rowsum, 4))
    return BL_EALIGN;
  return hip_status(bl::launch_act_quant_a48(X, dtype == BL_BF16, M, K, n_out, Xq4, x4_scale,
                                             x4_rowsum, Xq8, x8_scale, x8_rowsum,
                                             as_stream(stream)));
}

size_t bitlinear_a48_workspace_bytes(int64_t M, int64_t N) {
  if (!m_ok(M) || !dim_ok(N)) return 0;
  return (size_t)M * (size_t)N * 8;
}

int bitlinear_forward_a48(const int8_t* Xq4, const float* x4_scale, const int32_t* x4_rowsum,
                          const int8_t* Xq8, const float* x8_scale, const int32_t* x8_rowsum,
                          int64_t M, int64_t K, const uint32_t* Wp, const float* w_scale,
                          int64_t N, float* Y, void* ws, size_t ws_bytes, void* stream) {
  int st = check_forward(Xq4, x4_scale, x4_rowsum, M, K, Wp, w_scale, N, Y);
  if (st != BL_OK) return st;
  if (!Xq8 || !x8_scale || !x8_rowsum) return BL_EINVAL;
  if (!aligned(Xq8, 16) || !aligned(x8_scale, 4) || !aligned(x8_rowsum, 4)) return BL_EALIGN;
  if (!ws || ws_bytes < bitlinear_a48_workspace_bytes(M, N)) return BL_EWORKSPACE;
  if (!aligned(ws, 16)) return BL_EALIGN;
  return hip_status(bl::launch_forward_a48(Xq4, x4_scale, x4_rowsum, Xq8, x8_scale, x8_rowsum, M,
                                           K, Wp, w_scale, N, Y, reinterpret_cast<int32_t*>(ws),
                                           as_stream(stream)));
}

size_t bitlinear_fused_workspace_offset(int64_t M, int64_t K, int which) {
  if (!m_ok(M) || !dim_ok(K)) return 0;
  const size_t q = up256((size_t)M * (size_t)padk(K));
  const size_t sc = up256((size_t)M * 4);
  switch (which) {
    case 0: return 0;
    case 1: return q;
    case 2: return q + sc;
    default: return q + 2 * sc;
  }
}

size_t bitlinear_fused_workspace_bytes(int64_t M, int64_t K) {
  return bitlinear_fused_workspace_offset(M, K, 3);
}

int bitlinear_forward_fused(const void* X, int dtype, int64_t M, int64_t K, const uint32_t* Wp,
                            const float* w_scale, int64_t N, float* Y, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!X || !Wp || !w_scale || !Y) return BL_EINVAL;
  if (dtype != BL_F32 && dtype != BL_BF16) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(K) || !dim_ok(N)) return BL_ESHAPE;
  if (!ws || ws_bytes < bitlinear_fused_workspace_bytes(M, K)) return BL_EWORKSPACE;
  if (!aligned(X, dtype == BL_F32 ? 4 : 2) || !aligned(Wp, 16) || !aligned(w_scale, 4) ||
      !aligned(Y, 4) || !aligned(ws, 16))
    return BL_EALIGN;
  char* base = reinterpret_cast<char*>(ws);
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* xs = reinterpret_cast<float*>(base + bitlinear_fused_workspace_offset(M, K, 1));
  int32_t* rs = reinterpret_cast<int32_t*>(base + bitlinear_fused_workspace_offset(M, K, 2));
  hipStream_t s = as_stream(stream);
  const bool bf16 = dtype == BL_BF16;
  if (M == 1 && bl::gemv_fused_ok(K, N))
    return hip_status(bl::launch_gemv_fused(X, bf16, K, Wp, w_scale, N, Y, nullptr, xq, xs, rs, s));
  hipError_t e = bl::launch_act_quant(X, bf16, M, K, xq, xs, rs, nullptr, 0, s);
  if (e != hipSuccess) return BL_EHIP;
  if (M == 1) return hip_status(bl::launch_gemv(xq, xs, rs, K, Wp, w_scale, N, Y, nullptr, s));
  return hip_status(bl::launch_mfma(xq, xs, rs, M, K, Wp, w_scale, N, Y, nullptr, false, s));
}

size_t bitlinear_fused_norm_workspace_bytes(int64_t M, int64_t K) {
  if (!m_ok(M) || !dim_ok(K)) return 0;
  return bitlinear_fused_workspace_bytes(M, K) + up256((size_t)M * (size_t)K * 4);
}

int bitlinear_forward_fused_norm(const void* X, int dtype, int64_t M, int64_t K,
                                 const float* norm_w, float norm_eps, const uint32_t* Wp,
                                 const float* w_scale, int64_t N, float* Y, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!X || !Wp || !w_scale || !Y) return BL_EINVAL;
  if (dtype != BL_F32 && dtype != BL_BF16) return BL_EINVAL;
  if (!m_ok(M) || !dim_ok(K) || !dim_ok(N)) return BL_ESHAPE;
  if (!ws || ws_bytes < bitlinear_fused_norm_workspace_bytes(M, K)) return BL_EWORKSPACE;
  if (!aligned(X, dtype == BL_F32 ? 4 : 2) || !aligned(Wp, 16) || !aligned(w_scale, 4) ||
      !aligned(Y, 4) || !aligned(ws, 16) || (norm_w && !aligned(norm_w, 4)))
    return BL_EALIGN;
  char* base = reinterpret_cast<char*>(ws);
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* xs = reinterpret_cast<float*>(base + bitlinear_fused_workspace_offset(M, K, 1));
  int32_t* rs = reinterpret_cast<int32_t*>(base + bitlinear_fused_workspace_offset(M, K, 2));
  float* xn = reinterpret_cast<float*>(base + bitlinear_fused_workspace_bytes(M, K));
  hipStream_t s = as_stream(stream);
  const bool bf16 = dtype == BL_BF16;
  // one float32 token: RMSNorm, quantisation and the product in one kernel
  if (M == 1 && !bf16 && bl::gemv_norm_ok(K))
    return hip_status(bl::launch_gemv_norm(reinterpret_cast<const float*>(X), K, norm_w, norm_eps,
                                           Wp, w_scale, N, Y, xn, xq, xs, rs, s));
  hipError_t e = bl::launch_rmsnorm_quant(X, bf16, M, K, norm_w, norm_eps, xn, xq, xs, rs, s);
  if (e != hipSuccess) return BL_EHIP;
  if (M == 1) return hip_status(bl::launch_gemv(xq, xs, rs, K, Wp, w_scale, N, Y, nullptr, s));
  return hip_status(bl::launch_mfma(xq, xs, rs, M, K, Wp, w_scale, N, Y, nullptr, false, s));
}

size_t bitnet_ffn_workspace_layout(int64_t M, int64_t D, int64_t F, size_t* off) {
  if (!m_ok(M) || !dim_ok(D) || !dim_ok(F)) return 0;
  const size_t m = (size_t)M;
  int64_t parts = bl::gemv_gateup_parts(F);
  const int64_t p2 = bl::mfma_gateup_parts(M, F);
  if (p2 > parts) parts = p2;
  const size_t sizes[BL_FFN_WS_COUNT] = {
      m * (size_t)D * 4,       // XN
      m * (size_t)padk(D),     // QX
      m * 4,                   // GX
      m * 4,                   // RSX
      m * (size_t)F * 4,       // H
      m * (size_t)F * 4,       // HN
      m * 4,                   // GH
      m * (size_t)padk(F),     // QH
      m * 4,                   // RSH
      m * (size_t)parts * 4,   // GHP
  };
  size_t o = 0;
  for (int i = 0; i < BL_FFN_WS_COUNT; ++i) {
    if (off) off[i] = o;
    o += up256(sizes[i]);
  }
  return o;
}

size_t bitnet_ffn_workspace_bytes(int64_t M, int64_t D, int64_t F) {
  return bitnet_ffn_workspace_layout(M, D, F, nullptr);
}

// The block once its arguments are checked; base is a workspace of at least
// bitnet_ffn_workspace_bytes(M, D, F) bytes, 256-byte aligned.
static int ffn_run(const void* H, int dtype, int64_t M, int64_t D, int64_t F,
                   const float* norm_w, float norm_eps, const float* subln_w, float subln_eps,
                   const uint32_t* Wg, const float* sg, const uint32_t* Wu, const float* su,
                   const uint32_t* Wd, const float* sd, float* Y, char* base, hipStream_t s) {
  size_t off[BL_FFN_WS_COUNT];
  bitnet_ffn_workspace_layout(M, D, F, off);
  float* xn = reinterpret_cast<float*>(base + off[BL_FFN_WS_XN]);
  int8_t* qx = reinterpret_cast<int8_t*>(base + off[BL_FFN_WS_QX]);
  float* gx = reinterpret_cast<float*>(base + off[BL_FFN_WS_GX]);
  int32_t* rsx = reinterpret_cast<int32_t*>(base + off[BL_FFN_WS_RSX]);
  float* h = reinterpret_cast<float*>(base + off[BL_FFN_WS_H]);
  float* hn = reinterpret_cast<float*>(base + off[BL_FFN_WS_HN]);
  float* gh = reinterpret_cast<float*>(base + off[BL_FFN_WS_GH]);
  int8_t* qh = reinterpret_cast<int8_t*>(base + off[BL_FFN_WS_QH]);
  int32_t* rsh = reinterpret_cast<int32_t*>(base + off[BL_FFN_WS_RSH]);
  float* ghp = reinterpret_cast<float*>(base + off[BL_FFN_WS_GHP]);
  const bool bf16 = dtype == BL_BF16;

  hipError_t e;
  int nparts = 0;
  if (M == 1 && bl::gemv_gateup_norm_ok(D)) {
    // one token: RMSNorm, quantisation and the gate/up GEMV in one kernel
    e = bl::launch_gemv_gateup_norm(H, bf16, D, norm_w, norm_eps, Wg, sg, Wu, su, F, h, ghp,
                                    &nparts, xn, qx, gx, rsx, s);
  } else {
    e = bl::launch_rmsnorm_quant(H, bf16, M, D, norm_w, norm_eps, xn, qx, gx, rsx, s);
    if (e != hipSuccess) return BL_EHIP;
    // one token: the gate/up GEMV while the row fits its K range, else the
    // MFMA gate/up kernels (which take any K)
    if (M == 1 && bl::gemv_gateup_ok(D))
      e = bl::launch_gemv_gateup(qx, gx, rsx, D, Wg, sg, Wu, su, F, h, ghp, &nparts, s);
    else
      e = bl::launch_mfma_gateup(qx, gx, rsx, M, D, Wg, sg, Wu, su, F, h, ghp, &nparts, s);
  }
  if (e != hipSuccess) return BL_EHIP;
  if (subln_w) {
    // SubLN: RMSNorm of h, then its int8 codes; one token: both inside the
    // down GEMV
    if (M == 1 && bl::gemv_norm_ok(F))
      return hip_status(
          bl::launch_gemv_norm(h, F, subln_w, subln_eps, Wd, sd, D, Y, hn, qh, gh, rsh, s));
    e = bl::launch_rmsnorm_quant(h, false, M, F, subln_w, subln_eps, hn, qh, gh, rsh, s);
  } else if (M == 1 && bl::gemv_fused_ok(F, 0)) {
    // requantise h inside the down GEMV (scale from the partial maxima)
    e = bl::launch_gemv_parts(h, ghp, nparts, F, Wd, sd, D, Y, qh, gh, rsh, s);
    return hip_status(e);
  } else {
    e = bl::launch_act_quant(h, false, M, F, qh, gh, rsh, ghp, nparts, s);
  }
  if (e != hipSuccess) return BL_EHIP;
  if (M == 1)
    e = bl::launch_gemv(qh, gh, rsh, F, Wd, sd, D, Y, nullptr, s);
  else
    e = bl::launch_mfma(qh, gh, rsh, M, F, Wd, sd, D, Y, nullptr, false, s);
  return hip_status(e);
}


int bitnet_ffn_forward(const void* H, int dtype, int64_t M, int64_t D, int64_t F,
                       const float* norm_w, float norm_eps, const float* subln_w,
                       float subln_eps, const uint32_t* Wg, const float* sg,
                       const uint32_t* Wu, const float* su, const uint32_t* Wd, const float* sd,
                       float* Y, void* ws, size_t ws_bytes, void* stream) {
  const int st = ffn_check(H, dtype, M, D, F, norm_w, subln_w, Wg, sg, Wu, su, Wd, sd, Y);
  if (st != BL_OK) return st;
  if (!ws || ws_bytes < bitnet_ffn_workspace_bytes(M, D, F)) return BL_EWORKSPACE;
  if (!aligned(ws, 256)) return BL_EALIGN;
  return ffn_run(H, dtype, M, D, F, norm_w, norm_eps, subln_w, subln_eps, Wg, sg, Wu, su, Wd, sd,
                 Y, reinterpret_cast<char*>(ws), as_stream(stream));
}

int bitnet_ffn_forward_static(const void* H, int dtype, int64_t M, int64_t D, int64_t F,
                              const float* norm_w, float norm_eps, const float* subln_w,
                              float subln_eps, const uint32_t* Wg, const float* sg,
                              const uint32_t* Wu, const float* su, const uint32_t* Wd,
                              const float* sd, float* Y, void* stream) {
  const int st = ffn_check(H, dtype, M, D, F, norm_w, subln_w, Wg, sg, Wu, su, Wd, sd, Y);
  if (st != BL_OK) return st;
  if (bitnet_ffn_workspace_bytes(M, D, F) > (size_t)BL_FFN_STATIC_SCRATCH_BYTES) return BL_ESHAPE;
  char* base = nullptr;
  if (static_scratch_address(&base) != hipSuccess) return BL_EHIP;
  return ffn_run(H, dtype, M, D, F, norm_w, norm_eps, subln_w, subln_eps, Wg, sg, Wu, su, Wd, sd,
                 Y, base, as_stream(stream));
}

}  // extern "C"
