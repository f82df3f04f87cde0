// Device helpers shared by the gfx950 kernels of the BitLinear path.
//
// Numeric rules (compile with -ffp-contract=off and correctly rounded
// binary32 divide/sqrt): every float operation below rounds once, in the
// order written, to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Scale offset added before dividing (youngju.dev "Absmean量子化関数" and
// "BitNet b1.58" activation_quant both add 1e-5 to the scale) and the
// activation code bound (symmetric range, ai-heartland "BitLinearの仕組み").
constexpr float kEps = 1e-5f;
constexpr float kQ = 127.0f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Load element i of a float32 or bfloat16 row.
template <bool BF16>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// int8 code of x given d = gamma + eps: clamp(rne((x * 127) / d), -127, 127).
__device__ __forceinline__ int quant_code(float x, float d) {
  float v = __fmul_rn(x, kQ);
  v = __fdiv_rn(v, d);
  v = __builtin_rintf(v);
  v = fminf(fmaxf(v, -kQ), kQ);
  return (int)v;
}

// Dequantised output: ((float)acc * (g_w * g_m)) / 127.
__device__ __forceinline__ float dequant(int acc, float s) {
  return __fdiv_rn(__fmul_rn((float)acc, s), kQ);
}

// ---------------------------------------------------------------------------
// Exact sums of binary32 magnitudes (or squares) through exponent bins.
//
// A finite |x| has bits u = (E << 23) | F.  With b = max(E, 1) and mantissa
// m = (E ? F | 2^23 : F), |x| = m * 2^(b - 150) and x^2 = m^2 * 2^(2(b - 150)).
// bin[b] accumulates m (SH = 1) or m^2 (SH = 2) as an unsigned 64-bit integer:
// the accumulation is integer, hence independent of order.  The total is
//   X * 2^(-149 * SH),  X = sum_b bin[b] << (SH * (b - 1)),
// which finalize_bins() forms exactly in 32-bit limbs and rounds once to
// binary64 (round to nearest, ties to even).

constexpr int kBins = 256;
constexpr int kLimbs = 20;  // 640 bits: enough for SH = 2 (506 + 64 bits)

__device__ __forceinline__ void bin_of(float x, int& b, uint32_t& m) {
  uint32_t u = __float_as_uint(x) & 0x7fffffffu;
  uint32_t e = u >> 23;
  uint32_t f = u & 0x7fffffu;
  b = e ? (int)e : 1;
  m = e ? (f | 0x800000u) : f;
  if (e == 255u) { b = 254; m = 0; }  // Inf/NaN: unspecified, keep in range
}

// Called by all threads of a block (blockDim.x >= 64).  `bins` (LDS, kBins
// entries) must be complete and visible (barrier before the call);
// `limbs` is LDS scratch of kLimbs uint64.  Returns the rounded sum in every
// thread.  Contains two __syncthreads().
template <int SH>
__device__ double finalize_bins(const uint64_t* bins, unsigned long long* limbs,
                                double* result) {
  const int tid = threadIdx.x;
  if (tid < kLimbs) limbs[tid] = 0ull;
  __syncthreads();
  for (int b = tid; b < kBins; b += blockDim.x) {
    uint64_t v = bins[b];
    if (v == 0ull || b == 0) continue;
    int s = SH * (b - 1);
    int L = s >> 5, o = s & 31;
    uint32_t p0 = (uint32_t)(v << o);
    uint32_t p1 = (uint32_t)(o ? (v >> (32 - o)) : (v >> 32));
    uint32_t p2 = (uint32_t)(o ? (v >> (64 - o)) : 0ull);
    atomicAdd(&limbs[L], (unsigned long long)p0);
    atomicAdd(&limbs[L + 1], (unsigned long long)p1);
    if (p2) atomicAdd(&limbs[L + 2], (unsigned long long)p2);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t w[kLimbs];
    unsigned long long carry = 0ull;
    for (int i = 0; i < kLimbs; ++i) {
      unsigned long long t = limbs[i] + carry;
      w[i] = (uint32_t)t;
      carry = t >> 32;
    }
    int top = -1;
    for (int i = kLimbs - 1; i >= 0; --i) {
      if (w[i]) { top = i; break; }
    }
    double r = 0.0;
    if (top >= 0) {
      int p = 32 * top + (31 - __clz((int)w[top]));  // index of the leading bit
      // bit k of X
      auto bit = [&](int k) -> uint32_t { return (w[k >> 5] >> (k & 31)) & 1u; };
      uint64_t mant = 0ull;
      int lo = p - 52;  // lowest bit kept
      if (lo <= 0) {
        for (int k = p; k >= 0; --k) mant = (mant << 1) | bit(k);
        r = ldexp((double)mant, -149 * SH);
      } else {
        for (int k = p; k >= lo; --k) mant = (mant << 1) | bit(k);
        uint32_t rnd = bit(lo - 1);
        bool sticky = false;
        int rb = lo - 1;  // bits strictly below rb
        for (int i = 0; i < (rb >> 5); ++i) sticky |= (w[i] != 0u);
        if (rb & 31) sticky |= (w[rb >> 5] & ((1u << (rb & 31)) - 1u)) != 0u;
        if (rnd && (sticky || (mant & 1ull))) {
          mant += 1ull;
          if (mant == (1ull << 53)) { mant >>= 1; lo += 1; }
        }
        r = ldexp((double)mant, lo - 149 * SH);
      }
    }
    *result = r;
  }
  __syncthreads();
  return *result;
}

// ---------------------------------------------------------------------------
// 2-bit weight words.  Word j of a row covers weights 16j..16j+15; weight
// 16j + 4s + b is stored in byte b at bits 2s (code t + 1).  Hence
//   (w >> 2s) & 0x03030303
// holds, in bytes 0..3, the codes of weights 16j+4s .. 16j+4s+3 -- four
// consecutive weights in natural order, ready for a 4-wide int8 dot product
// or an MFMA operand.

__device__ __forceinline__ void unpack_word(uint32_t w, int& c0, int& c1, int& c2, int& c3) {
  c0 = (int)(w & 0x03030303u);
  c1 = (int)((w >> 2) & 0x03030303u);
  c2 = (int)((w >> 4) & 0x03030303u);
  c3 = (int)((w >> 6) & 0x03030303u);
}

// sum over the 16 weights of one word of code * x, x given as 4 words of 4
// int8 in natural order.  Three of the four fields are used in place (scaled
// by 4 and 16) and rescaled exactly afterwards; all values stay < 2^7 per
// byte so the signed 8-bit dot product is exact.
struct Dot16 {
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  __device__ __forceinline__ void add(uint32_t w, int x0, int x1, int x2, int x3) {
    a0 = __builtin_amdgcn_sdot4((int)(w & 0x03030303u), x0, a0, false);
    a1 = __builtin_amdgcn_sdot4((int)(w & 0x0c0c0c0cu), x1, a1, false);
    a2 = __builtin_amdgcn_sdot4((int)(w & 0x30303030u), x2, a2, false);
    a3 = __builtin_amdgcn_sdot4((int)((w >> 6) & 0x03030303u), x3, a3, false);
  }
  __device__ __forceinline__ int total() const { return a0 + (a1 >> 2) + (a2 >> 4) + a3; }
};

}  // namespace bl
