// Weight quantisation and packing (2-bit codes; 1-bit for binary weights) on
// gfx950.
//
// youngju.dev "BitNet論文分析", section "Absmean量子化関数": the ternary
// weight scale is the mean of |W| over the whole tensor; codes are
// clamp(round(W / (scale + 1e-5)), -1, 1).  Section "1-Bit重みとSign関数":
// binary codes are +1 where W >= 0, else -1, with the same mean-|W| scale.
// Section "アーキテクチャ概要" and dashen-tech "BitNet.cpp 深度解析" §2.3: two
// bits per weight, 00 = -1, 01 = 0, 10 = +1, sixteen weights per word.
//
// The mean is made exact and order-free: |w| = m * 2^(b-150) is binned by
// exponent b into unsigned 64-bit integer sums of m, combined exactly and
// rounded once to binary64, then divided by N*K in binary64 and rounded to
// binary32.  Three kernels: bins, finalize (one block), pack.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

__global__ void zero_bins_kernel(uint64_t* bins) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kBins) bins[i] = 0ull;
}

// Grid-stride over all n weights; per-wave LDS bins, then one global atomic
// add per non-empty bin per block.  Integer adds: the result does not depend
// on the order.
__global__ __launch_bounds__(256) void absmean_bins_kernel(const float* __restrict__ W,
                                                           int64_t n, uint64_t* bins) {
  __shared__ unsigned long long lbins[4][kBins];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * kBins; i += 256) (&lbins[0][0])[i] = 0ull;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n; i += stride) {
    int b;
    uint32_t m;
    bin_of(W[i], b, m);
    if (m) atomicAdd(&lbins[wave][b], (unsigned long long)m);
  }
  __syncthreads();
  for (int b = tid; b < kBins; b += 256) {
    unsigned long long v = lbins[0][b] + lbins[1][b] + lbins[2][b] + lbins[3][b];
    if (v) atomicAdd(reinterpret_cast<unsigned long long*>(&bins[b]), v);
  }
}

__global__ __launch_bounds__(64) void absmean_finalize_kernel(const uint64_t* __restrict__ bins,
                                                              int64_t n, float* w_scale) {
  __shared__ uint64_t lb[kBins];
  __shared__ unsigned long long limbs[kLimbs];
  __shared__ double res;
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) lb[i] = bins[i];
  __syncthreads();
  double s = finalize_bins<1>(lb, limbs, &res);
  if (threadIdx.x == 0) w_scale[0] = (float)(s / (double)n);
}

// One thread per packed word.  Row n, word j covers weights 16j..16j+15;
// weight 16j + 4s + b goes to byte b, bits 2s..2s+1, as code t + 1; weights
// past K are code 01.
template <bool BINARY>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ W, int64_t N,
                                                   int64_t K, int64_t words_per_row,
                                                   const float* __restrict__ w_scale,
                                                   uint32_t* __restrict__ Wp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * words_per_row) return;
  const int64_t n = idx / words_per_row, j = idx - n * words_per_row;
  const float d = __fadd_rn(w_scale[0], kEps);
  const float* row = W + n * K;
  uint32_t word = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t k = 16 * j + r;
    uint32_t code = 1u;
    if (k < K) {
      const float w = row[k];
      if constexpr (BINARY) {
        code = (w >= 0.0f) ? 2u : 0u;
      } else {
        float q = __builtin_rintf(__fdiv_rn(w, d));
        q = fminf(fmaxf(q, -1.0f), 1.0f);
        code = (uint32_t)((int)q + 1);
      }
    }
    const int s = r >> 2, b = r & 3;
    word |= code << (8 * b + 2 * s);
  }
  Wp[idx] = word;
}

// 1-bit layout of binary weights, one thread per word: row n, word j covers
// weights 32j..32j+31; weight 32j + 4s + b is bit 8b + s, 1 for w >= 0 (+1)
// and 0 for w < 0 (-1); weights past K (rows padded to 128) are bit 0.
__global__ __launch_bounds__(256) void pack1_kernel(const float* __restrict__ W, int64_t N,
                                                    int64_t K, int64_t words_per_row,
                                                    uint32_t* __restrict__ Wp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * words_per_row) return;
  const int64_t n = idx / words_per_row, j = idx - n * words_per_row;
  const float* row = W + n * K;
  uint32_t word = 0u;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int64_t k = 32 * j + r;
    const uint32_t bit = (k < K && row[k] >= 0.0f) ? 1u : 0u;
    word |= bit << (8 * (r & 3) + (r >> 2));
  }
  Wp[idx] = word;
}

hipError_t launch_pack(const float* W, int64_t N, int64_t K, int mode, uint32_t* Wp,
                       float* w_scale, uint64_t* bins, hipStream_t s) {
  const int64_t n = N * K;
  const int64_t kp = (K + 63) / 64 * 64;
  const int64_t wpr = kp / 16;
  hipLaunchKernelGGL(zero_bins_kernel, dim3(1), dim3(kBins), 0, s, bins);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(absmean_bins_kernel, dim3((unsigned)blocks), dim3(256), 0, s, W, n, bins);
  hipLaunchKernelGGL(absmean_finalize_kernel, dim3(1), dim3(64), 0, s, bins, n, w_scale);
  if (mode == 2) {
    const int64_t wpr1 = (K + 127) / 128 * 4;
    const unsigned b1 = (unsigned)((N * wpr1 + 255) / 256);
    hipLaunchKernelGGL(pack1_kernel, dim3(b1), dim3(256), 0, s, W, N, K, wpr1, Wp);
    return hipGetLastError();
  }
  const int64_t total = N * wpr;
  const unsigned pblocks = (unsigned)((total + 255) / 256);
  if (mode == 1)
    hipLaunchKernelGGL(pack_kernel<true>, dim3(pblocks), dim3(256), 0, s, W, N, K, wpr, w_scale, Wp);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3(pblocks), dim3(256), 0, s, W, N, K, wpr, w_scale, Wp);
  return hipGetLastError();
}

}  // namespace bl
