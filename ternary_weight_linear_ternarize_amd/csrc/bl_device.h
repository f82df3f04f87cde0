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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of streamed data that is read once (non-temporal hint).
__device__ __forceinline__ uint4 load_stream_u4(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

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

// int8 code of x given d = gamma + eps: clamp(rne((x * 127) / d), -127, 127),
// with the quotient correctly rounded (IEEE division).
__device__ __forceinline__ int quant_code(float x, float d) {
  float v = __fmul_rn(x, kQ);
  v = __fdiv_rn(v, d);
  v = __builtin_rintf(v);
  v = fminf(fmaxf(v, -kQ), kQ);
  return (int)v;
}

// Per-row divisor for quant_code_fast: d = gamma + eps and y = 1/d correctly
// rounded.  `fast` is false when d is so large that 1/d would leave the normal
// range; such rows use quant_code.
struct QuantDiv {
  float d, y;
  bool fast;
};
__device__ __forceinline__ QuantDiv make_qdiv(float gamma) {
  QuantDiv q;
  q.d = __fadd_rn(gamma, kEps);
  q.y = __fdiv_rn(1.0f, q.d);
  q.fast = q.d < 0x1p100f;
  return q;
}

// Same code as quant_code, with the division done by Markstein's correction
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", 1990): with y = RN(1/d) and q0 = RN(a*y), the
// residual r = a - q0*d is exact through one fused multiply-add and
// RN(q0 + r*y) is the correctly rounded a/d.  Valid while d, 1/d and a stay
// in the normal range (guaranteed for QuantDiv::fast rows, d >= 1e-5).
__device__ __forceinline__ int quant_code_fast(float x, const QuantDiv& q) {
  const float a = __fmul_rn(x, kQ);
  const float q0 = __fmul_rn(a, q.y);
  const float r = __builtin_fmaf(-q0, q.d, a);
  float v = __builtin_fmaf(r, q.y, q0);
  v = __builtin_rintf(v);
  v = fminf(fmaxf(v, -kQ), kQ);
  return (int)v;
}

__device__ __forceinline__ int quant_code_any(float x, const QuantDiv& q) {
  return q.fast ? quant_code_fast(x, q) : quant_code(x, q.d);
}

// Dequantised output: ((float)acc * (g_w * g_m)) / 127, s = g_w * g_m.
__device__ __forceinline__ float dequant(int acc, float s) {
  return __fdiv_rn(__fmul_rn((float)acc, s), kQ);
}

// The same value with the division by 127 done by Markstein's correction
// from the correctly rounded reciprocal (exact while p / 127 stays normal;
// smaller products take the IEEE division).
constexpr float kInvQ = 1.0f / 127.0f;  // RN(1/127), folded at compile time
__device__ __forceinline__ float dequant_fast(int acc, float s) {
  const float p = __fmul_rn((float)acc, s);
  const float q0 = __fmul_rn(p, kInvQ);
  const float r = __builtin_fmaf(-q0, kQ, p);
  float q = __builtin_fmaf(r, kInvQ, q0);
  if (__builtin_expect(fabsf(p) < 0x1p-100f, 0)) q = __fdiv_rn(p, kQ);
  return q;
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
    // carry-propagate into 32-bit words (kept in limbs[], low halves)
    unsigned long long carry = 0ull;
    int top = -1;
    for (int i = 0; i < kLimbs; ++i) {
      const unsigned long long t = limbs[i] + carry;
      limbs[i] = t & 0xffffffffull;
      carry = t >> 32;
      if (t & 0xffffffffull) top = i;
    }
    double r = 0.0;
    if (top >= 0) {
      const uint32_t wt = (uint32_t)limbs[top];
      const int p = 32 * top + (31 - __clz((int)wt));  // leading bit of X
      if (p < 53) {
        const uint64_t x = limbs[0] | (top >= 1 ? (limbs[1] << 32) : 0ull);
        r = ldexp((double)x, -149 * SH);  // exact
      } else {
        // 64-bit window whose top bit is bit p of X, plus a sticky bit for
        // everything below the window
        const int lo = p - 63;
        uint64_t win;
        bool below = false;
        if (lo >= 0) {
          const int i = lo >> 5, o = lo & 31;
          const uint64_t t = limbs[i] | (limbs[i + 1] << 32);
          const uint64_t h = (i + 2 < kLimbs) ? limbs[i + 2] : 0ull;
          win = o ? ((t >> o) | (h << (64 - o))) : t;
          for (int j = 0; j < i; ++j) below |= (limbs[j] != 0ull);
          if (o) below |= (limbs[i] & ((1ull << o) - 1ull)) != 0ull;
        } else {
          win = (limbs[0] | (limbs[1] << 32)) << (-lo);
        }
        uint64_t mant = win >> 11;                     // 53 bits
        const bool rnd = (win >> 10) & 1ull;
        const bool sticky = below || (win & 0x3ffull) != 0ull;
        int e = p - 52;
        if (rnd && (sticky || (mant & 1ull))) {
          mant += 1ull;
          if (mant == (1ull << 53)) { mant >>= 1; e += 1; }
        }
        r = ldexp((double)mant, e - 149 * SH);
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
