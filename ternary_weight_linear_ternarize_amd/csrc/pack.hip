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

// Each block reads one contiguous range of 4-weight units, kAbsUnits x 256
// at a time (float4 loads when W is 16-byte aligned).  Each lane sums exactly
// in a 96-bit integer A (three 32-bit limbs) at a fixed scale: with window
// base lo, a weight of bin b in [lo, lo + kAbsWin) adds m * 2^(b - lo) < 2^63,
// so A * 2^(lo - 150) is the lane's sum.  lo is set from the largest finite
// bin among the lane's first loads holding a non-zero weight (kAbsBelow bins
// below it, so the window reaches 2^9 above that weight); subnormal weights
// and weights outside the window go straight into the block's LDS bins
// (zeros, Inf and NaN add nothing).  At the end limb j of A is added to bin
// lo + 32 j (same value, bin form), and the block adds its non-empty bins to
// the global ones.  Bounds: a lane adds at most 2^13 + 16 weights (n <= 2^32
// over 2^19 lanes, ranges rounded up to 1024 units), so A < 2^77; lo is kept
// in [1, 190] so that lo + 64 is a bin.  Integer adds throughout: the result
// does not depend on the order.
constexpr int kAbsWin = 40;
constexpr int kAbsBelow = 30;
constexpr int kAbsUnits = 4;

__device__ __forceinline__ void absmean_add(uint32_t bits, int lo, uint32_t (&a)[3],
                                            unsigned long long* lbins) {
  // in the window e >= lo >= 1 and e < lo + kAbsWin <= 229: a normal finite
  // weight, m = mantissa with its implicit bit
  const int sh = (int)((bits >> 23) & 0xffu) - lo;
  if ((unsigned)sh < (unsigned)kAbsWin) {
    const uint64_t p = (uint64_t)((bits & 0x7fffffu) | 0x800000u) << sh;
    uint32_t c;
    a[0] = __builtin_addc(a[0], (uint32_t)p, 0u, &c);
    a[1] = __builtin_addc(a[1], (uint32_t)(p >> 32), c, &c);
    a[2] += c;
  } else if (bits & 0x7fffffffu) {
    // outside the window, subnormal, Inf or NaN (the last two add nothing)
    int b;
    uint32_t mb;
    bin_of(__uint_as_float(bits), b, mb);
    if (mb) atomicAdd(&lbins[b], (unsigned long long)mb);
  }
}

__global__ __launch_bounds__(256) void absmean_bins_kernel(const float* __restrict__ W,
                                                           int64_t n, bool vec, uint64_t* bins) {
  __shared__ unsigned long long lbins[kBins];
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += 256) lbins[i] = 0ull;
  __syncthreads();
  // block b reads units [b * per, (b + 1) * per), 16 KiB contiguous per step
  const int64_t units = (n + 3) / 4;
  const int64_t per = ((units + gridDim.x - 1) / gridDim.x + 1023) / 1024 * 1024;
  const int64_t ub = (int64_t)blockIdx.x * per;
  const int64_t ue = ub + per < units ? ub + per : units;
  int lo = 0;
  uint32_t a[3] = {0u, 0u, 0u};
  for (int64_t u0 = ub + tid; u0 < ue; u0 += kAbsUnits * 256) {
    uint32_t x[kAbsUnits][4];
#pragma unroll
    for (int h = 0; h < kAbsUnits; ++h) {
      const int64_t u = u0 + h * 256;
      if (vec && u < ue && 4 * u + 3 < n) {
        const uint4 f = reinterpret_cast<const uint4*>(W)[u];
        x[h][0] = f.x; x[h][1] = f.y; x[h][2] = f.z; x[h][3] = f.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[h][i] = u < ue && 4 * u + i < n ? __float_as_uint(W[4 * u + i]) : 0u;
      }
    }
    if (lo == 0) {
      // the window: from the largest finite non-zero bin of these loads
      int bm = 0;
#pragma unroll
      for (int h = 0; h < kAbsUnits; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = x[h][i] & 0x7fffffffu;
          if (u != 0u && u < 0x7f800000u) bm = max(bm, max((int)(u >> 23), 1));
        }
      if (bm) lo = min(max(bm - kAbsBelow, 1), 190);
    }
#pragma unroll
    for (int h = 0; h < kAbsUnits; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) absmean_add(x[h][i], lo, a, lbins);
  }
  if (lo != 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (a[j]) atomicAdd(&lbins[lo + 32 * j], (unsigned long long)a[j]);
  }
  __syncthreads();
  for (int b = tid; b < kBins; b += 256)
    if (lbins[b]) atomicAdd(reinterpret_cast<unsigned long long*>(&bins[b]), lbins[b]);
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

// Packing, one lane per four consecutive weights of a row (a float4 load when
// rows are 16-byte aligned, so a wave reads 1 KiB of contiguous weights), the
// lanes that share an output word combining their parts with shuffles.
//   MODE 0/1 (ternary / binary, 2-bit codes): word j of a row covers weights
//     16j..16j+15; weight 16j + 4s + b goes to byte b, bits 2s..2s+1, as code
//     t + 1; weights past K are code 01.  Four lanes per word.
//   MODE 2 (binary, 1-bit layout): word j covers weights 32j..32j+31; weight
//     32j + 4s + b is bit 8b + s, 1 for w >= 0 (+1) and 0 for w < 0 (-1);
//     weights past K (rows padded to 128) are bit 0.  Eight lanes per word.
// Block b covers row b / bpr, 4-weight units [1024 (b % bpr), +1024) of it;
// upr (units per padded row) is a multiple of the lanes per word.
template <int MODE>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ W, int64_t K,
                                                   int64_t upr, int bpr, bool vec,
                                                   const float* __restrict__ w_scale,
                                                   uint32_t* __restrict__ Wp) {
  constexpr int L = MODE == 2 ? 8 : 4;  // lanes per word
  constexpr int U = 4;                  // units per lane
  const int blk = (int)blockIdx.x;
  const int n = blk / bpr, seg = blk - n * bpr;
  const float* row = W + (int64_t)n * K;
  uint32_t* out = Wp + (int64_t)n * (upr / L);
  const float d = MODE == 0 ? __fadd_rn(w_scale[0], kEps) : 1.0f;
  // d >= 1e-5: d / 2 is exact; non-finite scales and weights take the division
  const bool dfin = __builtin_isfinite(d);
  const float hd = __fmul_rn(d, 0.5f);
  float w[U][4];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t k0 = 4 * ((int64_t)(seg * U + i) * 256 + threadIdx.x);
    if (vec && k0 + 3 < K) {
      const float4 f = *reinterpret_cast<const float4*>(row + k0);
      w[i][0] = f.x; w[i][1] = f.y; w[i][2] = f.z; w[i][3] = f.w;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) w[i][b] = k0 + b < K ? row[k0 + b] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t v = (int64_t)(seg * U + i) * 256 + threadIdx.x;  // unit within the row
    const int s = (int)(v % L);
    uint32_t part = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool in = 4 * v + b < K;
      if constexpr (MODE == 2) {
        part |= (in && w[i][b] >= 0.0f ? 1u : 0u) << (8 * b + s);
      } else {
        uint32_t code = 1u;
        if (in) {
          if constexpr (MODE == 1) {
            code = w[i][b] >= 0.0f ? 2u : 0u;
          } else if (dfin && __builtin_isfinite(w[i][b])) {
            // rne(fl(w / d)) is non-zero exactly when |w| > d / 2: at or
            // below it the quotient is at most 1/2 and rounds to 0; the next
            // float above d / 2 = m 2^(e-1) (1 <= m < 2) is d / 2 + 2^(e-24),
            // whose quotient exceeds 1/2 + 2^-25 and so rounds above 1/2
            code = fabsf(w[i][b]) > hd ? (w[i][b] > 0.0f ? 2u : 0u) : 1u;
          } else {
            float q = __builtin_rintf(__fdiv_rn(w[i][b], d));
            q = fminf(fmaxf(q, -1.0f), 1.0f);
            code = (uint32_t)((int)q + 1);
          }
        }
        part |= code << (8 * b + 2 * s);
      }
    }
    part |= __shfl_xor(part, 1);
    part |= __shfl_xor(part, 2);
    if constexpr (L == 8) part |= __shfl_xor(part, 4);
    if (s == 0 && v < upr) out[v / L] = part;
  }
}

hipError_t launch_pack(const float* W, int64_t N, int64_t K, int mode, uint32_t* Wp,
                       float* w_scale, uint64_t* bins, hipStream_t s) {
  const int64_t n = N * K;
  const int64_t kp = (K + 63) / 64 * 64;
  hipLaunchKernelGGL(zero_bins_kernel, dim3(1), dim3(kBins), 0, s, bins);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(W) & 15) == 0;
  const bool vec = aligned16 && K % 4 == 0;
  int64_t blocks = (n + 1023) / 1024;  // one 4-weight unit per thread at least
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(absmean_bins_kernel, dim3((unsigned)blocks), dim3(256), 0, s, W, n,
                     aligned16, bins);
  hipLaunchKernelGGL(absmean_finalize_kernel, dim3(1), dim3(64), 0, s, bins, n, w_scale);
  const int64_t kpad = mode == 2 ? (K + 127) / 128 * 128 : kp;
  const int64_t upr = kpad / 4;
  const int bpr = (int)((upr + 1023) / 1024);
  const unsigned pb = (unsigned)(N * bpr);
  if (mode == 2)
    hipLaunchKernelGGL(pack_kernel<2>, dim3(pb), dim3(256), 0, s, W, K, upr, bpr, vec, w_scale, Wp);
  else if (mode == 1)
    hipLaunchKernelGGL(pack_kernel<1>, dim3(pb), dim3(256), 0, s, W, K, upr, bpr, vec, w_scale, Wp);
  else
    hipLaunchKernelGGL(pack_kernel<0>, dim3(pb), dim3(256), 0, s, W, K, upr, bpr, vec, w_scale, Wp);
  return hipGetLastError();
}

}  // namespace bl
