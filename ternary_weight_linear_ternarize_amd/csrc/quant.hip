// Activation quantisation kernels on gfx950.
//
// youngju.dev "BitNet論文分析", section "BitNet b1.58" (activation_quant of
// BitLinear_b158): per token, scale = max |x| over the row, codes =
// clamp(round(x * Q / (scale + 1e-5))); Q = 127 and the symmetric range
// [-127, 127] (ai-heartland "BitLinearの仕組み": codes in {-Qb..Qb}).
// The same listing normalises with nn.RMSNorm before quantising; the
// RMSNorm kernel below makes the mean square exact and order-free (integer
// exponent bins of m^2, rounded once to binary64).
//
// One block per token row (256 threads, 1024 for few rows).  Codes are written four per 32-bit
// store into rows of Kp bytes; the padding columns get code 0.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

// Block-wide max (of non-negative values) / sum; blockDim.x a multiple of 64,
// at most 1024; red holds 16 entries.  Wave level on DPP moves, then every
// wave combines the per-wave values itself (no serial loop).
__device__ __forceinline__ float block_max(float v, float* red) {
  v = dpp::max_nonneg_f32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwv = blockDim.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = dpp::max_nonneg_f32(lane < nwv ? red[lane] : 0.0f);
  __syncthreads();
  return v;
}

__device__ __forceinline__ int block_sum(int v, int* red) {
  v = dpp::sum_i32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nwv = blockDim.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = dpp::sum_i32(lane < nwv ? red[lane] : 0);
  __syncthreads();
  return v;
}

// Writes the int8 codes of row values f(k) (k < K; 0 beyond) into q[0..Kp)
// and returns this thread's share of their sum.
template <typename F>
__device__ __forceinline__ int write_codes(F f, int64_t K, int64_t Kp, const QuantDiv& d,
                                           int8_t* q) {
  int rs = 0;
  uint32_t* q32 = reinterpret_cast<uint32_t*>(q);
  for (int64_t w = threadIdx.x; w < Kp / 4; w += blockDim.x) {
    uint32_t packed = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t k = 4 * w + b;
      int c = 0;
      if (k < K) c = quant_code_any(f(k), d);
      rs += c;
      packed |= ((uint32_t)(c & 0xff)) << (8 * b);
    }
    q32[w] = packed;
  }
  return rs;
}

// Loads words tid, tid+NT, ... (four consecutive elements each) of a row
// into registers; elements past K read as 0.
template <bool BF16, int NWT, int NT>
__device__ __forceinline__ void load_row_words(const char* base, int64_t K, int64_t nw,
                                               float (&xv)[NWT][4]) {
  const int tid = threadIdx.x;
  const bool vec = !BF16 && (K & 3) == 0;
#pragma unroll
  for (int j = 0; j < NWT; ++j) {
    const int64_t wd = tid + NT * j;
    if (vec && 4 * wd + 3 < K) {
      const float4 v = *reinterpret_cast<const float4*>(base + 16 * wd);
      xv[j][0] = v.x; xv[j][1] = v.y; xv[j][2] = v.z; xv[j][3] = v.w;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t k = 4 * wd + b;
        xv[j][b] = (wd < nw && k < K) ? load_act<BF16>(base, k) : 0.0f;
      }
    }
  }
}

// Writes the codes of the register-held row words and returns this thread's
// share of their sum.
template <int NWT, int NT>
__device__ __forceinline__ int store_row_codes(const float (&xv)[NWT][4], int64_t nw,
                                               const QuantDiv& d, int8_t* q) {
  int rs = 0;
#pragma unroll
  for (int j = 0; j < NWT; ++j) {
    const int64_t wd = threadIdx.x + NT * j;
    if (wd < nw) {
      uint32_t pk = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c = quant_code_any(xv[j][b], d);
        rs += c;
        pk |= ((uint32_t)(c & 0xff)) << (8 * b);
      }
      reinterpret_cast<uint32_t*>(q)[wd] = pk;
    }
  }
  return rs;
}

// NT threads per row.  NWT > 0: the row (Kp <= 4 NT NWT) is held in
// registers and read once; NWT == 0: any length, the row is read twice.
// Few rows take NT = 1024: these kernels are latency-bound, and a wave's
// time is its instruction count, so the row is spread over more waves.
template <bool BF16, int NWT, int NT>
__global__ __launch_bounds__(NT) void act_quant_kernel(const void* __restrict__ X, int64_t K,
                                                        int64_t Kp, int8_t* __restrict__ Xq,
                                                        float* __restrict__ x_scale,
                                                        int32_t* __restrict__ rowsum,
                                                        const float* __restrict__ gamma_parts,
                                                        int nparts, int64_t M) {
  __shared__ float redf[16];
  __shared__ int redi[16];
  const int64_t m = blockIdx.x;
  const char* base = reinterpret_cast<const char*>(X) + m * K * (BF16 ? 2 : 4);
  float g = 0.0f;
  // partial maxima: the first kAqParts per thread as branch-free loads issued
  // with the row's loads (both in flight at once), any beyond in a loop
  constexpr int kAqParts = 2;
  uint32_t gp[kAqParts] = {};
  if (gamma_parts) {
    const buf_rsrc rg = make_buf_rsrc(gamma_parts, (uint32_t)(4 * nparts * M));
#pragma unroll
    for (int i = 0; i < kAqParts; ++i) {
      const int p = threadIdx.x + NT * i;
      gp[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rg, p < nparts ? (uint32_t)(4 * ((int64_t)p * M + m)) : 0x80000000u, 0, 0);
    }
  }
  int rs;
  if constexpr (NWT > 0) {
    float xv[NWT][4];
    load_row_words<BF16, NWT, NT>(base, K, Kp / 4, xv);
    if (!gamma_parts) {
#pragma unroll
      for (int j = 0; j < NWT; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) g = fmaxf(g, fabsf(xv[j][b]));
    } else {
#pragma unroll
      for (int i = 0; i < kAqParts; ++i) g = fmaxf(g, __uint_as_float(gp[i]));
      for (int p = threadIdx.x + NT * kAqParts; p < nparts; p += NT)
        g = fmaxf(g, gamma_parts[(int64_t)p * M + m]);
    }
    g = block_max(g, redf);
    rs = store_row_codes<NWT, NT>(xv, Kp / 4, make_qdiv(g), Xq + m * Kp);
  } else {
    if (!gamma_parts) {
      for (int64_t k = threadIdx.x; k < K; k += blockDim.x) g = fmaxf(g, fabsf(load_act<BF16>(base, k)));
    } else {
#pragma unroll
      for (int i = 0; i < kAqParts; ++i) g = fmaxf(g, __uint_as_float(gp[i]));
      for (int p = threadIdx.x + NT * kAqParts; p < nparts; p += NT)
        g = fmaxf(g, gamma_parts[(int64_t)p * M + m]);
    }
    g = block_max(g, redf);
    rs = write_codes([&](int64_t k) { return load_act<BF16>(base, k); }, K, Kp, make_qdiv(g),
                     Xq + m * Kp);
  }
  rs = block_sum(rs, redi);
  if (threadIdx.x == 0) {
    x_scale[m] = g;
    if (rowsum) rowsum[m] = rs;
  }
}

// RMSNorm(D) of one row, then its int8 codes.  xn = (x * r) * w with
// r = 1 / sqrt(ms + eps), ms = binary32(binary64(exact sum x^2) / D).
// NWT > 0: the row (Dp <= 1024 * NWT) is held in registers; NWT == 0: any
// length, the row is re-read from memory for each pass.
template <bool BF16, int NWT, int NT>
__global__ __launch_bounds__(NT) void rmsnorm_quant_kernel(
    const void* __restrict__ H, int64_t D, int64_t Dp, const float* __restrict__ norm_w,
    float eps, float* __restrict__ xn, int8_t* __restrict__ Xq, float* __restrict__ x_scale,
    int32_t* __restrict__ rowsum) {
  constexpr int NR = NWT > 0 ? NWT : 1;
  __shared__ float redf[16];
  __shared__ int redi[16];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t m = blockIdx.x;
  const char* base = reinterpret_cast<const char*>(H) + m * D * (BF16 ? 2 : 4);
  const int64_t nw = Dp / 4;
  float xv[NR][4];
  float ms;
  if constexpr (NWT > 0) {
    load_row_words<BF16, NWT, NT>(base, D, nw, xv);
    __shared__ SumsqScratch sh;
    ms = block_meansq<NWT, NT>(xv, D, sh);
  } else {
    // rows longer than 16384: exponent bins over reloaded values
    __shared__ unsigned long long bins[4][kBins];
    __shared__ uint64_t tot[kBins];
    __shared__ unsigned long long limbs[kLimbs];
    __shared__ double res;
    for (int i = tid; i < 4 * kBins; i += NT) (&bins[0][0])[i] = 0ull;
    __syncthreads();
    for (int64_t k = tid; k < D; k += NT) {
      int bb;
      uint32_t mm;
      bin_of(load_act<BF16>(base, k), bb, mm);
      if (mm) atomicAdd(&bins[wave & 3][bb], (unsigned long long)mm * (unsigned long long)mm);
    }
    __syncthreads();
    for (int b = tid; b < kBins; b += NT) tot[b] = bins[0][b] + bins[1][b] + bins[2][b] + bins[3][b];
    __syncthreads();
    const double s = finalize_bins<2>(tot, limbs, &res);
    ms = (float)(s / (double)D);
  }
  // __builtin_sqrtf is correctly rounded under -fhip-fp32-correctly-rounded-divide-sqrt
  // (the __fsqrt_rn intrinsic maps to a native approximation on this toolchain).
  const float r = __fdiv_rn(1.0f, __builtin_sqrtf(__fadd_rn(ms, eps)));
  auto norm = [&](float x, int64_t k) {
    const float v = __fmul_rn(x, r);
    return norm_w ? __fmul_rn(v, norm_w[k]) : v;
  };
  float g = 0.0f;
  int rs;
  if constexpr (NWT > 0) {
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
      const int64_t wd = tid + NT * j;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t k = 4 * wd + b;
        const bool in = wd < nw && k < D;
        const float v = in ? norm(xv[j][b], k) : 0.0f;
        xv[j][b] = v;
        if (in) xn[m * D + k] = v;
        g = fmaxf(g, fabsf(v));
      }
    }
    g = block_max(g, redf);
    rs = store_row_codes<NWT, NT>(xv, nw, make_qdiv(g), Xq + m * Dp);
  } else {
    for (int64_t k = tid; k < D; k += NT) {
      const float v = norm(load_act<BF16>(base, k), k);
      xn[m * D + k] = v;
      g = fmaxf(g, fabsf(v));
    }
    g = block_max(g, redf);
    rs = write_codes([&](int64_t k) { return norm(load_act<BF16>(base, k), k); }, D, Dp,
                     make_qdiv(g), Xq + m * Dp);
  }
  rs = block_sum(rs, redi);
  if (tid == 0) {
    x_scale[m] = g;
    rowsum[m] = rs;
  }
}

template <int NWT, int NT>
static void act_quant_go(const void* X, bool bf16, int64_t M, int64_t K, int64_t Kp, int8_t* Xq,
                         float* x_scale, int32_t* rowsum, const float* gamma_parts, int nparts,
                         hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((act_quant_kernel<true, NWT, NT>), dim3((unsigned)M), dim3(NT), 0, s, X, K,
                       Kp, Xq, x_scale, rowsum, gamma_parts, nparts, M);
  else
    hipLaunchKernelGGL((act_quant_kernel<false, NWT, NT>), dim3((unsigned)M), dim3(NT), 0, s, X, K,
                       Kp, Xq, x_scale, rowsum, gamma_parts, nparts, M);
}

// Rows of up to 64 tokens run 1024 threads per row (see act_quant_kernel).
constexpr int64_t kWideRows = 64;

hipError_t launch_act_quant(const void* X, bool bf16, int64_t M, int64_t K, int8_t* Xq,
                            float* x_scale, int32_t* rowsum, const float* gamma_parts,
                            int nparts, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
#define BL_AQ(NWT, NT) act_quant_go<NWT, NT>(X, bf16, M, K, Kp, Xq, x_scale, rowsum, gamma_parts, nparts, s)
  if (M <= kWideRows) {
    if (Kp <= 4096) BL_AQ(1, 1024);
    else if (Kp <= 8192) BL_AQ(2, 1024);
    else if (Kp <= 16384) BL_AQ(4, 1024);
    else BL_AQ(0, 1024);
  } else {
    if (Kp <= 1024) BL_AQ(1, 256);
    else if (Kp <= 3072) BL_AQ(3, 256);
    else if (Kp <= 8192) BL_AQ(8, 256);
    else if (Kp <= 16384) BL_AQ(16, 256);
    else BL_AQ(0, 256);
  }
#undef BL_AQ
  return hipGetLastError();
}

template <int NWT, int NT>
static void rmsnorm_go(const void* H, bool bf16, int64_t M, int64_t D, int64_t Dp,
                       const float* norm_w, float eps, float* xn, int8_t* Xq, float* x_scale,
                       int32_t* rowsum, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((rmsnorm_quant_kernel<true, NWT, NT>), dim3((unsigned)M), dim3(NT), 0, s, H,
                       D, Dp, norm_w, eps, xn, Xq, x_scale, rowsum);
  else
    hipLaunchKernelGGL((rmsnorm_quant_kernel<false, NWT, NT>), dim3((unsigned)M), dim3(NT), 0, s, H,
                       D, Dp, norm_w, eps, xn, Xq, x_scale, rowsum);
}

hipError_t launch_rmsnorm_quant(const void* H, bool bf16, int64_t M, int64_t D,
                                const float* norm_w, float eps, float* xn, int8_t* Xq,
                                float* x_scale, int32_t* rowsum, hipStream_t s) {
  const int64_t Dp = (D + 63) / 64 * 64;
#define BL_RN(NWT, NT) rmsnorm_go<NWT, NT>(H, bf16, M, D, Dp, norm_w, eps, xn, Xq, x_scale, rowsum, s)
  // longer rows re-read the input rather than hold it (register pressure of
  // the exact sum of squares)
  if (M <= kWideRows) {
    if (Dp <= 4096) BL_RN(1, 1024);
    else if (Dp <= 8192) BL_RN(2, 1024);
    else BL_RN(0, 1024);
  } else {
    if (Dp <= 1024) BL_RN(1, 256);
    else if (Dp <= 3072) BL_RN(3, 256);
    else if (Dp <= 8192) BL_RN(8, 256);
    else BL_RN(0, 256);
  }
#undef BL_RN
  return hipGetLastError();
}

}  // namespace bl
