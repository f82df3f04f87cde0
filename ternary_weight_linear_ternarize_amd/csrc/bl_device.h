// Device helpers shared by the gfx950 kernels of the BitLinear path.
//
// Numeric rules (compile with -ffp-contract=off and correctly rounded
// binary32 divide/sqrt): every float operation below rounds once, in the
// order written, to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

typedef __amdgpu_buffer_rsrc_t buf_rsrc;

// Raw buffer resource over [base, base + nbytes): loads past nbytes return 0.
__device__ __forceinline__ buf_rsrc make_buf_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// The per-token operands of an MFMA epilogue: x_scale and rowsum of the
// tokens a lane's result registers hold (token mbase + 16 tm + 4 (lane / 16)
// + r of 16-row tile tm, register r).  Loaded at a kernel's start as
// branch-free buffer loads (tokens past M read 0), so their round trip
// passes while the main loop runs instead of after it (as per-register loads
// in the epilogue, each behind its own bounds check, they were issued and
// waited for one at a time).
template <int TM>
struct TokenOperands {
  float xs[TM][4];
  int rs[TM][4];
  __device__ __forceinline__ void load(const float* x_scale, const int32_t* rowsum, int64_t M,
                                      int64_t mbase) {
    const buf_rsrc rx = make_buf_rsrc(x_scale, (uint32_t)(4 * M));
    const buf_rsrc rr = make_buf_rsrc(rowsum, (uint32_t)(4 * M));
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mbase + 16 * tm + 4 * g + r;
        const uint32_t off = m < M ? (uint32_t)(4 * m) : 0x80000000u;
        xs[tm][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
        rs[tm][r] = (int)__builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, 0);
      }
  }
};

// s_waitcnt operand that waits until at most n (< 64) vector memory
// operations of this wave are outstanding and leaves the other counters
// alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).
__host__ __device__ constexpr int vmcnt_only(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// LDS bytes stage_rows_lds writes for M rows of the given pitch.
__host__ __device__ constexpr int64_t staged_rows_bytes(int64_t M, int64_t pitch) {
  return (M * pitch + 1023) / 1024 * 1024;
}

// Copies bytes [k0, k0 + klen) of rows 0 .. M-1 of an int8 matrix (row stride
// Kp) into LDS rows of `pitch` bytes (pitch >= klen, multiples of 16; the
// bytes of a row past klen read as zero) with direct-to-LDS buffer loads:
// each load moves 64 lanes x 16 bytes into 1 KB of LDS in lane order, so all
// of the block's loads are in flight at once and no register holds the data.
// dst spans staged_rows_bytes(M, pitch).  The data is in LDS once this
// thread's loads have completed (s_waitcnt vmcnt(0)) and the block has
// synchronised.  Requires M * Kp < 2^30.
template <int NT>
__device__ __forceinline__ void stage_rows_lds(const int8_t* X, int64_t Kp, int M, int64_t k0,
                                               int klen, int pitch, int8_t* dst) {
  const buf_rsrc r = make_buf_rsrc(X, (uint32_t)(M * Kp));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int units = (int)(staged_rows_bytes(M, pitch) / 1024);
  for (int u = wave; u < units; u += NT / 64) {
    const int o = 1024 * u + 16 * lane;
    const int row = o / pitch, col = o - row * pitch;
    const int voff = (row < M && col < klen) ? (int)(row * Kp + k0) + col : 0x40000000;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + 1024 * u, 16, voff, 0, 0, 0);
  }
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

// The rounded, clamped code of x as a float (the same value as quant_code_any).
__device__ __forceinline__ float quant_value(float x, const QuantDiv& q) {
  const float a = __fmul_rn(x, kQ);
  float v;
  if (q.fast) {
    const float q0 = __fmul_rn(a, q.y);
    const float r = __builtin_fmaf(-q0, q.d, a);
    v = __builtin_fmaf(r, q.y, q0);
  } else {
    v = __fdiv_rn(a, q.d);
  }
  return __builtin_amdgcn_fmed3f(__builtin_rintf(v), -kQ, kQ);
}

// Codes of four consecutive values packed as signed bytes (value b in byte b).
// Each code c in [-127, 127] goes through the unsigned byte c + 128 (exact:
// an integral float in [1, 255]) and the top bit is flipped back.
__device__ __forceinline__ uint32_t quant_pack4(float x0, float x1, float x2, float x3,
                                                const QuantDiv& q) {
  uint32_t p = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(quant_value(x0, q), 128.0f), 0, 0u);
  p = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(quant_value(x1, q), 128.0f), 1, p);
  p = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(quant_value(x2, q), 128.0f), 2, p);
  p = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(quant_value(x3, q), 128.0f), 3, p);
  return p ^ 0x80808080u;
}

// Sum of the four signed bytes of a packed code word, added to acc.
__device__ __forceinline__ int add_bytes(uint32_t p, int acc) {
  return __builtin_amdgcn_sdot4((int)p, 0x01010101, acc, false);
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

// The four shifted-code byte vectors of one packed word: element s holds the
// codes of weights 16j+4s .. 16j+4s+3 (one MFMA operand dword each).
__device__ __forceinline__ v4i codes_operand(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)((w >> 2) & 0x03030303u);
  r[2] = (int)((w >> 4) & 0x03030303u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

// ---------------------------------------------------------------------------
// Exact sum of squares, fast path.
//
// With bmax the largest exponent bin of the row (bin_of), every square is
// x^2 = m^2 * 2^(2(b - 150)) = (m^2 << s) * 2^L, s = 2 (b - bmax) + 62,
// L = 2 (bmax - 150) - 62.  Terms with s >= 0 are added exactly into a
// 128-bit integer A (m^2 < 2^48, so a term is < 2^110 and 2^16 of them stay
// below 2^126); terms with s < 0 keep their bits from position -s up and set
// a flag if anything below was cut.  The true sum is T = (A + R) * 2^L with
// 0 <= R < 2^16 (at most 2^16 terms, each losing less than one unit), and
// R > 0 exactly when the flag is set.  All terms are non-negative, so R can
// change the binary64 rounding of T only through a carry into the rounding
// position; round128() reports that case (bits 16 .. rp-1 of A all ones) as
// undecided and the caller falls back to the exponent-bin sum.  Truncation
// happens only when the largest element is normal (m >= 2^23), and then
// A >= 2^108, so the rounding bit sits at position 55 or above.
struct Sum128 {
  uint64_t lo = 0, hi = 0;
  bool cut = false;
};

__device__ __forceinline__ void sq_add(float x, int bmax, Sum128& a) {
  int b;
  uint32_t m;
  bin_of(x, b, m);
  const uint64_t sq = (uint64_t)m * (uint64_t)m;  // < 2^48 (0 for a zero)
  const int s = 2 * (b - bmax) + 62;              // <= 62 for every nonzero x
  // straight-line selects: this runs once per element in latency-bound kernels
  const int sl = s > 0 ? s : 0;
  const int sr = s < 0 ? (-s < 63 ? -s : 63) : 0;
  const uint64_t add_lo = s >= 0 ? (sq << sl) : (sq >> sr);
  const uint64_t add_hi = sl > 16 ? (sq >> (64 - (sl > 16 ? sl : 17))) : 0ull;
  a.cut |= (sq & ((1ull << sr) - 1ull)) != 0ull;
  a.lo += add_lo;
  a.hi += add_hi + (a.lo < add_lo ? 1ull : 0ull);
}

__device__ __forceinline__ void sum128_merge(Sum128& a, uint64_t lo, uint64_t hi, bool cut) {
  a.lo += lo;
  a.hi += hi + (a.lo < lo ? 1ull : 0ull);
  a.cut |= cut;
}

// Low 64 bits of (hi:lo) >> k, 0 <= k < 128.
__device__ __forceinline__ uint64_t shr128(uint64_t lo, uint64_t hi, int k) {
  if (k == 0) return lo;
  if (k < 64) return (lo >> k) | (hi << (64 - k));
  return hi >> (k - 64);
}

// Binary64 rounding (to nearest, ties to even) of (A + R) * 2^L as described
// above; false when R could carry into the rounding position.
__device__ inline bool round128(const Sum128& a, int L, double* out) {
  if (a.hi == 0ull && a.lo == 0ull) {
    *out = 0.0;
    return !a.cut;
  }
  const int P = a.hi ? 127 - __clzll((long long)a.hi) : 63 - __clzll((long long)a.lo);
  if (P <= 52) {  // A < 2^53 is exact (no term was cut: the largest is subnormal)
    *out = ldexp((double)a.lo, L);
    return !a.cut;
  }
  const int rp = P - 53;  // position of the rounding bit
  if (a.cut) {
    if (rp <= 16) return false;
    const uint64_t mid = shr128(a.lo, a.hi, 16) & ((1ull << (rp - 16)) - 1ull);
    if (mid == (1ull << (rp - 16)) - 1ull) return false;
  }
  uint64_t mant = shr128(a.lo, a.hi, rp + 1) & ((1ull << 53) - 1ull);
  const bool rnd = (shr128(a.lo, a.hi, rp) & 1ull) != 0ull;
  bool below = a.cut;
  if (rp >= 64)
    below |= a.lo != 0ull || (a.hi & ((1ull << (rp - 64)) - 1ull)) != 0ull;
  else if (rp > 0)
    below |= (a.lo & ((1ull << rp) - 1ull)) != 0ull;
  int e = rp + 1 + L;
  if (rnd && (below || (mant & 1ull))) {
    mant += 1ull;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      e += 1;
    }
  }
  *out = ldexp((double)mant, e);
  return true;
}

// ---------------------------------------------------------------------------
// Wave-wide reductions on DPP lane moves (VALU latency, a few cycles per
// step) rather than ds_bpermute shuffles (LDS-pipe latency): quad
// exchanges, the half-row and row mirrors, then row broadcasts 15 and 31.
// Every lane of the wave must be active; the result is read from lane 63
// and returned (wave-uniform) to all lanes.
namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kBcast15 = 0x142;
constexpr int kBcast31 = 0x143;

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ int mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xF, false);
}

template <typename Op>
__device__ __forceinline__ int reduce_i32(int v, int ident, Op op) {
  v = op(v, mov<kXor1>(ident, v));
  v = op(v, mov<kXor2>(ident, v));
  v = op(v, mov<kHalfMirror>(ident, v));
  v = op(v, mov<kMirror>(ident, v));
  v = op(v, mov<kBcast15, 0xA>(ident, v));
  v = op(v, mov<kBcast31, 0xC>(ident, v));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int sum_i32(int v) {
  return reduce_i32(v, 0, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ int max_i32(int v) {
  return reduce_i32(v, INT32_MIN, [](int a, int b) { return a > b ? a : b; });
}
// Value of lane (lane ^ O) for O = 1 .. 32: quad permutes, row rotations
// (row_ror:n moves lane i - n to lane i within a row of 16) and the gfx950
// row/half swaps, all VALU ops.
template <int O>
__device__ __forceinline__ int xchg(int v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "stride");
  if constexpr (O == 1) {
    return mov<kXor1>(0, v);
  } else if constexpr (O == 2) {
    return mov<kXor2>(0, v);
  } else if constexpr (O == 4) {
    // banks 0, 2 take lane i + 4 (row_ror:12), banks 1, 3 take lane i - 4 (row_ror:4)
    const int r = __builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0x5, false);
    return __builtin_amdgcn_update_dpp(r, v, 0x124, 0xF, 0xA, false);
  } else if constexpr (O == 8) {
    return mov<0x128>(0, v);  // row_ror:8
  } else if constexpr (O == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 16) ? p[0] : p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 32) ? p[0] : p[1]);
  }
}

// max of non-negative floats (their bit patterns order as integers)
__device__ __forceinline__ float max_nonneg_f32(float v) {
  return __int_as_float(max_i32(__float_as_int(v)));
}

// 128-bit sum with a sticky flag (Sum128 above), same pattern.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ void merge_from(Sum128& a) {
  const uint32_t l0 = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)a.lo);
  const uint32_t l1 = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)(a.lo >> 32));
  const uint32_t h0 = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)a.hi);
  const uint32_t h1 = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)(a.hi >> 32));
  const int c = mov<CTRL, ROWMASK>(0, (int)a.cut);
  sum128_merge(a, (uint64_t)l0 | ((uint64_t)l1 << 32), (uint64_t)h0 | ((uint64_t)h1 << 32), c != 0);
}
__device__ __forceinline__ Sum128 sum128(Sum128 a) {
  merge_from<kXor1>(a);
  merge_from<kXor2>(a);
  merge_from<kHalfMirror>(a);
  merge_from<kMirror>(a);
  merge_from<kBcast15, 0xA>(a);
  merge_from<kBcast31, 0xC>(a);
  Sum128 r;
  r.lo = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a.lo, 63) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a.lo >> 32), 63) << 32);
  r.hi = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a.hi, 63) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a.hi >> 32), 63) << 32);
  r.cut = __builtin_amdgcn_readlane((int)a.cut, 63) != 0;
  return r;
}
// sum of doubles, same pattern
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ double movd(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)u);
  const uint32_t hi = (uint32_t)mov<CTRL, ROWMASK>(0, (int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)((uint64_t)lo | ((uint64_t)hi << 32)));
}
__device__ __forceinline__ double sum_f64(double v) {
  v += movd<kXor1>(v);
  v += movd<kXor2>(v);
  v += movd<kHalfMirror>(v);
  v += movd<kMirror>(v);
  v += movd<kBcast15, 0xA>(v);
  v += movd<kBcast31, 0xC>(v);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)((uint64_t)lo | ((uint64_t)hi << 32)));
}
}  // namespace dpp

// Exact binary64 rounding of the sum of squares of a block's row (NT
// threads), values held in registers, NWT words of 4 per thread.  Fast path
// as above; the exponent-bin sum when the rounding is undecided.
struct SumsqScratch {
  unsigned long long bins[4][kBins];
  uint64_t tot[kBins];
  unsigned long long limbs[kLimbs];
  uint64_t part[16][2];
  double res;
  int pcut[16];
  int bmax[16];
};

template <int NWT, int NT>
__device__ double block_sumsq_exact(const float (&xv)[NWT][4], SumsqScratch& sh) {
  constexpr int NWV = NT / 64;
  static_assert(NWV >= 1 && NWV <= 16, "block size");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int bmax = 0;
#pragma unroll
  for (int j = 0; j < NWT; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int bb;
      uint32_t mm;
      bin_of(xv[j][b], bb, mm);
      bmax = mm ? max(bmax, bb) : bmax;
    }
  bmax = dpp::max_i32(bmax);
  if (lane == 0) sh.bmax[wave] = bmax;
  __syncthreads();
  // second level: every wave combines the per-wave values itself
  bmax = dpp::max_i32(lane < NWV ? sh.bmax[lane] : 0);
  Sum128 acc;
#pragma unroll
  for (int j = 0; j < NWT; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) sq_add(xv[j][b], bmax, acc);
  acc = dpp::sum128(acc);
  if (lane == 0) {
    sh.part[wave][0] = acc.lo;
    sh.part[wave][1] = acc.hi;
    sh.pcut[wave] = acc.cut;
  }
  __syncthreads();
  Sum128 t;
  if (lane < NWV) {
    t.lo = sh.part[lane][0];
    t.hi = sh.part[lane][1];
    t.cut = sh.pcut[lane] != 0;
  }
  t = dpp::sum128(t);
  double s = 0.0;
  const bool ok = round128(t, 2 * (bmax - 150) - 62, &s);  // same in every thread
  if (!ok) {  // block-uniform
    for (int i = tid; i < 4 * kBins; i += NT) (&sh.bins[0][0])[i] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NWT; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int bb;
        uint32_t mm;
        bin_of(xv[j][b], bb, mm);
        if (mm) atomicAdd(&sh.bins[wave & 3][bb], (unsigned long long)mm * (unsigned long long)mm);
      }
    __syncthreads();
    for (int b = tid; b < kBins; b += NT)
      sh.tot[b] = sh.bins[0][b] + sh.bins[1][b] + sh.bins[2][b] + sh.bins[3][b];
    __syncthreads();
    s = finalize_bins<2>(sh.tot, sh.limbs, &sh.res);
  }
  return s;
}

// Mean square of a block's row for RMSNorm: ms = binary32(binary64(S) / D)
// with S the exact sum of squares (NT threads, values in registers).
//
// Fast path: S_a = the binary64 sum of the squares (each square is exact in
// binary64) in any order, |S_a - S| <= (n - 1) 2^-53 S <= 2^-37 S for
// n <= 2^16 non-negative terms, and q_a = RN64(S_a * RN64(1 / D)), within
// 2^-37 + 2^-51 of S / D relatively (the reciprocal is taken before the
// reduction, off its critical path).  If q_a is farther than 2^-35 q_a from
// both binary32 rounding midpoints around c = RN32(q_a), then S / D and every
// value within 2^-36 of it (the exact route's intermediate binary64 roundings
// included) round to c, so ms = c.  Otherwise (rows within ~2^-35 of a
// midpoint, all zero, or at the top of the range) the exact sum decides.
template <int NWT, int NT>
__device__ float block_meansq(const float (&xv)[NWT][4], int64_t D, SumsqScratch& sh) {
  constexpr int NWV = NT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double rD = 1.0 / (double)D;  // off the reduction's critical path
  double a0 = 0.0, a1 = 0.0;
#pragma unroll
  for (int j = 0; j < NWT; ++j)
#pragma unroll
    for (int b = 0; b < 4; b += 2) {
      const double x0 = (double)xv[j][b], x1 = (double)xv[j][b + 1];
      a0 += x0 * x0;
      a1 += x1 * x1;
    }
  double a = dpp::sum_f64(a0 + a1);
  double* dpart = reinterpret_cast<double*>(&sh.part[0][0]);
  if (lane == 0) dpart[wave] = a;
  __syncthreads();
  a = dpp::sum_f64(lane < NWV ? dpart[lane] : 0.0);
  const double qa = a * rD;
  const float c = (float)qa;
  // neighbours of c >= 0 (c = 0 gives a NaN below, hence the exact path)
  const uint32_t cb = __float_as_uint(c);
  const double lo = 0.5 * ((double)c + (double)__uint_as_float(cb - 1u));
  const double hi = 0.5 * ((double)c + (double)__uint_as_float(cb + 1u));
  const double tol = qa * 0x1p-35;
  if (cb < 0x7f7fffffu && qa - lo > tol && hi - qa > tol) return c;  // block-uniform
  __syncthreads();  // dpart (sh.part) is reused below
  const double s = block_sumsq_exact<NWT, NT>(xv, sh);
  return (float)(s / (double)D);
}

// sum over the 16 weights of one word of code * x, x given as 4 words of 4
// int8 in natural order.  Three of the four fields are used in place (scaled
// by 4 and 16) and rescaled exactly afterwards; all values stay < 2^7 per
// byte so the signed 8-bit dot product is exact.
// BitNet a4.8 output from the two accumulators of a token:
// y = (acc4 (g_w g4)) / 7 + (acc8 (g_w g8)) / 127, one rounding per operation
// (s4 = g_w g4 and s8 = g_w g8 already rounded).
__device__ __forceinline__ float a48_dequant(int acc4, float s4, int acc8, float s8) {
  const float y4 = __fdiv_rn(__fmul_rn((float)acc4, s4), 7.0f);
  const float y8 = __fdiv_rn(__fmul_rn((float)acc8, s8), kQ);
  return __fadd_rn(y4, y8);
}

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

// Dot16 against two code vectors at once (x and z, e.g. the 4-bit and the
// 8-bit parts of split activations): the masked weight fields are shared.
struct Dot16x2 {
  Dot16 x, z;
  __device__ __forceinline__ void add(uint32_t w, const int4& xv, const int4& zv) {
    const int m0 = (int)(w & 0x03030303u), m1 = (int)(w & 0x0c0c0c0cu);
    const int m2 = (int)(w & 0x30303030u), m3 = (int)((w >> 6) & 0x03030303u);
    x.a0 = __builtin_amdgcn_sdot4(m0, xv.x, x.a0, false);
    x.a1 = __builtin_amdgcn_sdot4(m1, xv.y, x.a1, false);
    x.a2 = __builtin_amdgcn_sdot4(m2, xv.z, x.a2, false);
    x.a3 = __builtin_amdgcn_sdot4(m3, xv.w, x.a3, false);
    z.a0 = __builtin_amdgcn_sdot4(m0, zv.x, z.a0, false);
    z.a1 = __builtin_amdgcn_sdot4(m1, zv.y, z.a1, false);
    z.a2 = __builtin_amdgcn_sdot4(m2, zv.z, z.a2, false);
    z.a3 = __builtin_amdgcn_sdot4(m3, zv.w, z.a3, false);
  }
};

// LDS byte offset of 16-byte piece p of the activation codes.  The four
// pieces of 64-weight chunk c are rotated by (c / 2) % 4, so the eight lanes
// of a ds_read_b128 phase (consecutive chunks, same piece) hit eight
// different 16-byte bank groups.
__device__ __forceinline__ int xslot(int p) {
  const int c = p >> 2;
  return 16 * (4 * c + ((p & 3) ^ ((c >> 1) & 3)));
}

// Sum of q over the set bits of 1-bit packed words (binary weights): word w
// holds 32 weights, weight 4s + b at bit 8b + s, against the activation codes
// x[0..7] (dword s = the codes of weights 4s .. 4s+3).  Bit s of every byte
// is masked in place, so group s enters its dot product scaled by 2^(s % 4)
// (groups 4..7 after one shift by 4); the four scaled sums are rescaled
// exactly at the end.  Bytes stay <= 8, so the signed dot product is exact.
struct DotBits32 {
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  __device__ __forceinline__ void add(uint32_t w, const int4& lo, const int4& hi) {
    a0 = __builtin_amdgcn_sdot4((int)(w & 0x01010101u), lo.x, a0, false);
    a1 = __builtin_amdgcn_sdot4((int)(w & 0x02020202u), lo.y, a1, false);
    a2 = __builtin_amdgcn_sdot4((int)(w & 0x04040404u), lo.z, a2, false);
    a3 = __builtin_amdgcn_sdot4((int)(w & 0x08080808u), lo.w, a3, false);
    const uint32_t w4 = w >> 4;
    a0 = __builtin_amdgcn_sdot4((int)(w4 & 0x01010101u), hi.x, a0, false);
    a1 = __builtin_amdgcn_sdot4((int)(w4 & 0x02020202u), hi.y, a1, false);
    a2 = __builtin_amdgcn_sdot4((int)(w4 & 0x04040404u), hi.z, a2, false);
    a3 = __builtin_amdgcn_sdot4((int)(w4 & 0x08080808u), hi.w, a3, false);
  }
  __device__ __forceinline__ int total() const { return a0 + (a1 >> 1) + (a2 >> 2) + (a3 >> 3); }
};

// MFMA operand of weights 16h .. 16h+15 of a 1-bit word: dword d holds group
// s = 4h + d (weights 4s .. 4s+3, bit s of each byte) as the bytes 2 * bit.
template <int H>
__device__ __forceinline__ v4i bits_operand(uint32_t w) {
  v4i r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int s = 4 * H + d;
    r[d] = (int)((s == 0 ? (w << 1) : (w >> (s - 1))) & 0x02020202u);
  }
  return r;
}

// Reduce v[0..R) (per-lane partials of R rows) across the 64 lanes with a
// transposing butterfly on DPP / lane-swap moves, small strides first: the
// first log2 R steps exchange halves of the row set, the rest add.  On return
// every lane l holds the full sum of row gemv_row<R>(l) in v[0] (the low
// log2 R bits of l, bit-reversed).
template <int R>
__device__ __forceinline__ int wave_transpose_reduce(int (&v)[R]) {
  const int lane = threadIdx.x & 63;
  int cnt = R;
  auto step = [&](auto o_tag) {
    constexpr int O = decltype(o_tag)::value;
    if (cnt > 1) {
      const int half = cnt >> 1;
      const bool hi = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < R / 2; ++i) {
        if (i < half) {
          const int keep = hi ? v[half + i] : v[i];
          const int send = hi ? v[i] : v[half + i];
          v[i] = keep + dpp::xchg<O>(send);
        }
      }
      cnt = half;
    } else {
      v[0] += dpp::xchg<O>(v[0]);
    }
  };
  step(std::integral_constant<int, 1>());
  step(std::integral_constant<int, 2>());
  step(std::integral_constant<int, 4>());
  step(std::integral_constant<int, 8>());
  step(std::integral_constant<int, 16>());
  step(std::integral_constant<int, 32>());
  return v[0];
}

// Row whose total lane l holds after wave_transpose_reduce<R>.
template <int R>
__device__ __forceinline__ int gemv_row(int lane) {
  constexpr int LOGR = (R == 1) ? 0 : (R == 2) ? 1 : (R == 4) ? 2 : (R == 8) ? 3 : 4;
  int r = 0;
#pragma unroll
  for (int b = 0; b < LOGR; ++b) r |= ((lane >> b) & 1) << (LOGR - 1 - b);
  return r;
}

}  // namespace bl
